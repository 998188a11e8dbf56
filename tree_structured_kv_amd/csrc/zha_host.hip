// zha_host.hip -- the C ABI of libzha: argument checks, sizing, launches.
//
// Nothing here allocates, frees or synchronises device memory; every launch
// goes to the caller's stream.  A call that fails its checks returns before
// enqueueing anything.
#include <math.h>
#include <string.h>

#include "zha_internal.h"

#include <algorithm>
#include <mutex>

using namespace zha;

// Scratch of zha_sparse_attn_noalloc: one fixed array per GPU, allocated
// with the code object when the library loads on a device and held until
// the process ends.  Host code never passes this name to a kernel (on the
// host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ZHA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_n(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

int64_t level_count(int64_t n, int c, int l) {
    for (int i = 0; i < l; ++i) n /= c;
    return n;
}

// Bytes of one stored node-key element.
uint64_t summary_bytes(const zha_geometry *g) { return g->summary_dtype == ZHA_BF16 ? 2 : 4; }

zha_status check_geometry(const zha_geometry *g) {
    if (!g) return ZHA_ERR_ARG;
    if (g->batch < 1 || g->num_kv_heads < 1 || g->group_size < 1) return ZHA_ERR_ARG;
    if (g->head_dim != 64 && g->head_dim != 128) return ZHA_ERR_UNSUPPORTED;
    if (g->chunk < 2 || g->chunk > 64 || (g->chunk & (g->chunk - 1))) return ZHA_ERR_UNSUPPORTED;
    if (g->num_refs != 1 && g->num_refs != 2 && g->num_refs != 4 && g->num_refs != 8 &&
        g->num_refs != 16)
        return ZHA_ERR_UNSUPPORTED;
    if (g->levels < 1 || g->levels > ZHA_MAX_LEVELS) return ZHA_ERR_UNSUPPORTED;
    if (g->dtype != ZHA_F32 && g->dtype != ZHA_BF16) return ZHA_ERR_UNSUPPORTED;
    if (g->summary_dtype != ZHA_F32 && g->summary_dtype != ZHA_BF16) return ZHA_ERR_UNSUPPORTED;
    if (g->max_tokens < 1 || g->max_tokens >= (int64_t(1) << 31)) return ZHA_ERR_ARG;
    if (g->max_tokens / g->chunk >= (int64_t(1) << kLevelShift)) return ZHA_ERR_UNSUPPORTED;
    if (!isfinite(g->sharpness)) return ZHA_ERR_ARG;
    if (int64_t(g->batch) * g->num_kv_heads > 65535) return ZHA_ERR_UNSUPPORTED;
    const int64_t walks = int64_t(g->batch) * g->num_kv_heads * g->group_size;
    if (walks > (int64_t(1) << 24)) return ZHA_ERR_UNSUPPORTED;
    return ZHA_OK;
}

zha_status check_tree(const zha_tree *t) {
    if (!t) return ZHA_ERR_ARG;
    zha_status s = check_geometry(&t->geom);
    if (s != ZHA_OK) return s;
    if (!t->tree_mem || !t->refs) return ZHA_ERR_ARG;
    if (t->n_tokens < 0 || t->n_tokens > t->geom.max_tokens) return ZHA_ERR_SHAPE;
    if (t->tree_bytes < zha_tree_bytes(&t->geom)) return ZHA_ERR_CAPACITY;
    return ZHA_OK;
}

int64_t total_nodes(const zha_geometry *g) {
    int64_t tot = 0;
    for (int l = 1; l <= g->levels; ++l) tot += level_count(g->max_tokens, g->chunk, l);
    return tot;
}

int32_t cand_capacity(const zha_tree *t, const zha_select *sel) {
    int64_t cap = sel->max_candidates > 0 ? sel->max_candidates : total_nodes(&t->geom);
    if (cap < 1) cap = 1;
    if (cap > (int64_t(1) << 24)) cap = int64_t(1) << 24;
    return static_cast<int32_t>(cap);
}

zha_status check_select(const zha_select *sel) {
    if (!sel) return ZHA_ERR_ARG;
    if (sel->mode != ZHA_TOPP && sel->mode != ZHA_TOPK) return ZHA_ERR_ARG;
    if (!isfinite(sel->p)) return ZHA_ERR_ARG;
    if (sel->mode == ZHA_TOPK) {
        if (sel->num_k < 1 || sel->num_k > ZHA_MAX_STEPS) return ZHA_ERR_ARG;
        for (int i = 0; i < sel->num_k; ++i)
            if (sel->k[i] < 1) return ZHA_ERR_ARG;
    }
    if (sel->max_blocks_per_walk < 1) return ZHA_ERR_ARG;
    if (sel->max_candidates < 0) return ZHA_ERR_ARG;
    if (sel->engine < ZHA_ENGINE_AUTO || sel->engine > ZHA_ENGINE_FUSED) return ZHA_ERR_ARG;
    if (sel->attn_engine < ZHA_ATTN_AUTO || sel->attn_engine > ZHA_ATTN_UNION) return ZHA_ERR_ARG;
    return ZHA_OK;
}

int64_t walks_of(const zha_geometry *g, int32_t qph) {
    return int64_t(g->batch) * g->num_kv_heads * g->group_size * qph;
}

struct SearchWs {
    uint64_t cand, score, state, tile_count, tile_map, u_ids, u_omask, u_n, u_next, h_score, u_rank,
        u_par, u_open, u_flat, u_score, b_roots, b_cnt, b_fill, b_first, b_inv, b_units, flat_cap, nbins,
        pcap, total;
};
// Workspace of zha_search; the union engine's arrays only where it can run
// (decode, at most 16 query heads per KV head).
SearchWs search_ws_layout(const zha_tree *t, const zha_select *sel, int32_t qph) {
    const uint64_t cap = static_cast<uint64_t>(cand_capacity(t, sel));
    const uint64_t walks = static_cast<uint64_t>(walks_of(&t->geom, qph));
    const bool uni = qph == 1 && t->geom.group_size <= 16;
    const uint64_t pairs = uni ? uint64_t(t->geom.batch) * t->geom.num_kv_heads : 0;
    const uint64_t uw = uni ? walks : 0;
    SearchWs l;
    l.cand = 0;
    l.score = align_up(walks * 2 * cap * sizeof(uint32_t));
    l.state = l.score + align_up(walks * cap * sizeof(float));
    l.tile_count = l.state + align_up(walks * sizeof(WalkState));
    l.tile_map = l.tile_count + align_up((ZHA_MAX_STEPS + 1) * sizeof(int32_t));
    l.u_ids = l.tile_map + align_up(walks * ((cap + kTile - 1) / kTile) * sizeof(int2));
    l.u_omask = l.u_ids + align_up(pairs * 2 * cap * sizeof(uint32_t));
    l.u_n = l.u_omask + align_up(pairs * 2 * cap * sizeof(uint32_t));
    l.u_next = l.u_n + align_up(pairs * 2 * sizeof(int32_t));
    l.h_score = l.u_next + align_up(uw * sizeof(int32_t));
    l.u_rank = l.h_score + align_up(uw * cap * sizeof(float));
    l.u_par = l.u_rank + align_up(pairs * cap * sizeof(int32_t));
    l.u_open = l.u_par + align_up(pairs * cap * sizeof(uint32_t));
    l.u_flat = l.u_open + align_up(uw * cap * sizeof(int32_t));
    l.flat_cap = pairs * (cap + kExpSlices * kFlatPad);
    l.u_score = l.u_flat + align_up(2 * l.flat_cap * 16);
    // block engine: parents are the nodes of levels >= 2; a walk keeps at
    // most cap/c + 1 of them per step
    const uint64_t all_pairs = uint64_t(t->geom.batch) * t->geom.num_kv_heads;
    l.nbins = 0;
    for (int lv = 2; lv <= t->geom.levels; ++lv) l.nbins += static_cast<uint64_t>(t->level_cap[lv]);
    l.pcap = cap / static_cast<uint64_t>(t->geom.chunk) + 1;
    const uint64_t gp = (uint64_t(t->geom.group_size) + 3) / 4 * 4;
    l.b_roots = l.u_score + align_up(pairs * cap * gp * sizeof(float));
    l.b_cnt = l.b_roots + align_up(cap * sizeof(uint32_t));
    l.b_fill = l.b_cnt + align_up(all_pairs * l.nbins * sizeof(int32_t));
    l.b_first = l.b_fill + align_up(all_pairs * l.nbins * sizeof(int32_t));
    l.b_inv = l.b_first + align_up(all_pairs * l.nbins * sizeof(int32_t));
    l.b_units = l.b_inv + align_up(walks * l.pcap * sizeof(int2));
    l.total = l.b_units + align_up(walks * l.pcap * sizeof(int4));
    return l;
}

// Attention work items of a call: each walk's keys (at most keys_bound)
// cut into chunks of at least kChunkMin keys, at least one item per walk.
int64_t attn_max_items(int64_t keys_bound, int64_t walks) {
    int64_t per = (keys_bound + kChunkMin - 1) / kChunkMin;
    if (per < 1) per = 1;
    return walks * (per + 1);     // + the block-keys item of a prefill walk
}

int64_t tree_keys_bound(const zha_tree *t, const zha_select *sel, int32_t qph) {
    return int64_t(sel->max_blocks_per_walk) * t->geom.chunk + t->geom.chunk - 1 + (qph > 1 ? qph : 0);
}

// The union attention path: bf16 caches; decode with at most 16 query heads
// per KV head (one matrix-core column per head), or a prefill block (groups
// of 16 walks of a (sequence, KV head) pair, taken in the order of their
// selection sketches).
struct UnionGeom {
    int64_t ugroups, n1cap, nchunks, cwords, wpg_max, gpp;
};
UnionGeom union_geom(const zha_tree *t, int32_t qph) {
    const zha_geometry &g = t->geom;
    UnionGeom u;
    const int64_t pairs = int64_t(g.batch) * g.num_kv_heads;
    u.gpp = qph > 1 ? (int64_t(g.group_size) * qph + 15) / 16 : 1;
    u.ugroups = pairs * u.gpp;
    u.n1cap = (g.max_tokens / g.chunk + 1) / 2 * 2;
    u.nchunks = (u.n1cap + kUaBlocks - 1) / kUaBlocks;
    u.cwords = (u.nchunks + 31) / 32;
    u.wpg_max = qph > 1 ? 1 : std::max<int64_t>(1, std::min<int64_t>(2048 / pairs, u.nchunks));
    return u;
}

bool union_attn_ok(const zha_tree *t, int32_t qph) {
    if (t->geom.dtype != ZHA_BF16) return false;
    if (t->geom.chunk < 4) return false;           // a lane's four keys must share a block
    if (qph == 1 && t->geom.group_size > 16) return false;
    const UnionGeom u = union_geom(t, qph);
    return u.wpg_max <= kUaMaxItems && u.ugroups * u.wpg_max < (int64_t(1) << 31);
}

// ZHA_ATTN_* a call runs (ZHA_ATTN_UNION only where union_attn_ok).
int resolve_attn(const zha_tree *t, const zha_select *sel, int32_t qph) {
    if (sel->attn_engine != ZHA_ATTN_AUTO) return sel->attn_engine;
    if (!union_attn_ok(t, qph)) return ZHA_ATTN_PER_WALK;
    return (qph > 1 || t->geom.group_size == 16) ? ZHA_ATTN_UNION : ZHA_ATTN_PER_WALK;
}

struct AttnWs {
    uint64_t part, item_off, item_walk, umask, uchunk, ic, upart, bpart, ukey, uperm, uinv, total;
    UnionGeom u;
};
// Per-walk items; with `t` (a call that may take the union path) also the
// union arrays.
AttnWs attn_ws_layout(int head_dim, int64_t keys_bound, int64_t walks, const zha_tree *t = nullptr,
                      int32_t qph = 1) {
    const uint64_t items = static_cast<uint64_t>(attn_max_items(keys_bound, walks));
    AttnWs l;
    l.part = 0;
    l.item_off = align_up(items * (head_dim + 2) * sizeof(float));
    l.item_walk = l.item_off + align_up(uint64_t(walks + 2) * sizeof(int32_t));
    l.umask = l.item_walk + align_up(items * sizeof(int32_t));
    const bool uni = t && union_attn_ok(t, qph);
    l.u = uni ? union_geom(t, qph) : UnionGeom{0, 0, 0, 0, 0, 1};
    const uint64_t ng = uint64_t(l.u.ugroups);
    l.uchunk = l.umask + align_up(ng * uint64_t(l.u.n1cap) * sizeof(uint16_t));
    l.ic = l.uchunk + align_up(ng * uint64_t(l.u.cwords) * sizeof(uint32_t));
    l.upart = l.ic + align_up(ng * uint64_t(l.u.wpg_max) * sizeof(int32_t));
    l.bpart = l.upart + align_up(ng * uint64_t(l.u.wpg_max) * 16 * (head_dim + 2) * sizeof(float));
    const uint64_t pw = uni && qph > 1 ? uint64_t(walks) : 0;   // prefill-only arrays
    l.ukey = l.bpart + align_up(pw * (head_dim + 2) * sizeof(float));
    l.uperm = l.ukey + align_up(pw * sizeof(unsigned long long));
    l.uinv = l.uperm + align_up(pw * sizeof(int32_t));
    l.total = l.uinv + align_up(pw * sizeof(int32_t));
    return l;
}

uint64_t attn_ws_bytes(const zha_tree *t, const zha_select *sel, int32_t qph) {
    return attn_ws_layout(t->geom.head_dim, tree_keys_bound(t, sel, qph), walks_of(&t->geom, qph), t, qph).total;
}

struct ForwardWs {
    uint64_t sel_blocks, sel_count, search, attn, total;
};
ForwardWs forward_ws_layout(const zha_tree *t, const zha_select *sel, int32_t qph) {
    const int64_t walks = walks_of(&t->geom, qph);
    ForwardWs l;
    l.sel_blocks = 0;
    l.sel_count = align_up(uint64_t(walks) * sel->max_blocks_per_walk * sizeof(int32_t));
    l.search = l.sel_count + align_up(uint64_t(walks) * sizeof(int32_t));
    l.attn = l.search + search_ws_layout(t, sel, qph).total;
    l.total = l.attn + attn_ws_bytes(t, sel, qph);
    return l;
}

zha_status hip_status(hipError_t e) { return e == hipSuccess ? ZHA_OK : ZHA_ERR_HIP; }

// The one-launch decode step keeps the records of the nodes an append makes
// (at most one per level) in LDS next to the leaf scratch: 64 KB at most.
bool fused_fits(const zha_tree *t) {
    const zha_geometry &g = t->geom;
    return fused_lds_bytes(g.head_dim, g.num_refs, g.chunk, static_cast<int>(summary_bytes(&g)), g.levels) <= 65536;
}

zha_status run_levels(zha_tree *t, const void *k_cache, int64_t n_old, int64_t n_new, hipStream_t st) {
    const zha_geometry &g = t->geom;
    char *mem = static_cast<char *>(t->tree_mem);
    for (int l = 1; l <= g.levels; ++l) {
        const int64_t a = level_count(n_old, g.chunk, l);
        const int64_t b = level_count(n_new, g.chunk, l);
        if (b <= a) break;   // nothing new here, hence nothing above either
        LevelArgs la;
        memset(&la, 0, sizeof(la));
        la.keys = k_cache;
        if (l > 1) {
            la.child_k = mem + t->key_off[l - 1];
            la.child_b = reinterpret_cast<const float *>(mem + t->bias_off[l - 1]);
            la.child_cap = t->level_cap[l - 1];
        }
        la.out_k = mem + t->key_off[l];
        la.out_b = reinterpret_cast<float *>(mem + t->bias_off[l]);
        la.refs = t->refs;
        la.max_tokens = g.max_tokens;
        la.out_cap = t->level_cap[l];
        la.j0 = a;
        la.count = b - a;
        la.kv_heads = g.num_kv_heads;
        la.pairs = g.batch * g.num_kv_heads;
        la.chunk = g.chunk;
        la.refs_n = g.num_refs;
        la.sharpness = g.sharpness;
        hipError_t e = launch_level(la, g.head_dim, g.dtype, g.summary_dtype, l == 1, st);
        if (e != hipSuccess) return ZHA_ERR_HIP;
    }
    return ZHA_OK;
}

int64_t visited_words_per_pair(const zha_tree *t) {
    int64_t bits = 0;
    for (int l = 1; l <= t->geom.levels; ++l) bits += t->level_cap[l];
    return (bits + 31) / 32;
}

// The engine a search runs on: the caller's choice, or for AUTO the one
// that measured fastest for the shape (block for prefill blocks, union when
// 16 query heads share a KV head in decode, level-synchronous -- with its
// dense top table -- for other wide top-p batches, else persistent).
int resolve_engine(const zha_tree *t, const zha_select *sel, int32_t qph) {
    if (sel->engine != ZHA_ENGINE_AUTO) return sel->engine;
    const int64_t walks = walks_of(&t->geom, qph);
    if (qph > 1) return ZHA_ENGINE_BLOCK;
    if (qph == 1 && t->geom.group_size == 16 && walks >= 64) return ZHA_ENGINE_UNION;
    if (sel->mode == ZHA_TOPP && walks >= 64) return ZHA_ENGINE_LEVEL_SYNC;
    return ZHA_ENGINE_PERSISTENT;
}

// Search arguments for the tree as it stands with n_tok tokens summarised;
// returns the number of roots (clamped to the candidate capacity).
int64_t fill_search(const zha_tree *t, int64_t n_tok, const void *q, int32_t qph, const zha_select *sel,
                    int32_t *sel_blocks, int32_t *sel_count, zha_walk_stats *stats, uint32_t *status,
                    uint32_t *visited, void *ws, int engine, SearchArgs &a) {
    const zha_geometry &g = t->geom;
    const int64_t walks = walks_of(&g, qph);
    SearchWs lay = search_ws_layout(t, sel, qph);
    const char *mem = static_cast<const char *>(t->tree_mem);
    memset(&a, 0, sizeof(a));
    for (int l = 1; l <= g.levels; ++l) {
        a.kap[l] = reinterpret_cast<const float *>(mem + t->key_off[l]);
        a.bet[l] = reinterpret_cast<const float *>(mem + t->bias_off[l]);
        a.cap[l] = t->level_cap[l];
        a.nl[l] = level_count(n_tok, g.chunk, l);
    }
    a.nl[0] = n_tok;
    a.nl[g.levels + 1] = 0;
    a.q = q;
    a.sel_blocks = sel_blocks;
    a.sel_count = sel_count;
    a.stats = stats;
    a.status = status;
    a.visited = visited;
    a.vis_words = visited_words_per_pair(t);
    {
        int64_t off = 0;
        for (int l = 1; l <= g.levels; ++l) {
            a.node_off[l] = off;
            off += t->level_cap[l];
        }
    }
    a.cand = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.cand);
    a.score = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.score);
    a.state = reinterpret_cast<WalkState *>(static_cast<char *>(ws) + lay.state);
    a.tile_count = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.tile_count);
    a.tile_map = reinterpret_cast<int2 *>(static_cast<char *>(ws) + lay.tile_map);
    a.u_ids = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.u_ids);
    a.u_omask = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.u_omask);
    a.u_n = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.u_n);
    a.u_next = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.u_next);
    a.h_score = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.h_score);
    a.u_rank = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.u_rank);
    a.u_par = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.u_par);
    a.u_open = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.u_open);
    a.u_flat = reinterpret_cast<int4 *>(static_cast<char *>(ws) + lay.u_flat);
    a.flat_cap = static_cast<int64_t>(lay.flat_cap);
    a.u_score = reinterpret_cast<float *>(static_cast<char *>(ws) + lay.u_score);
    a.b_roots = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + lay.b_roots);
    a.b_cnt = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.b_cnt);
    a.b_fill = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.b_fill);
    a.b_first = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + lay.b_first);
    a.b_inv = reinterpret_cast<int2 *>(static_cast<char *>(ws) + lay.b_inv);
    a.b_units = reinterpret_cast<int4 *>(static_cast<char *>(ws) + lay.b_units);
    a.nbins = static_cast<int64_t>(lay.nbins);
    a.pcap = static_cast<int32_t>(lay.pcap);
    {
        int64_t off = 0;
        for (int l = 0; l <= ZHA_MAX_LEVELS + 1; ++l) a.bin_lvl[l] = 0;
        for (int l = 2; l <= g.levels; ++l) {
            a.bin_lvl[l] = off;
            off += t->level_cap[l];
        }
        a.bin_lvl[g.levels + 1] = off;
    }
    a.pairs = g.batch * g.num_kv_heads;
    a.score_grid = 1024;
    a.n_tokens = n_tok;
    a.walks = static_cast<int32_t>(walks);
    a.qph = qph;
    a.heads = g.num_kv_heads * g.group_size;
    a.group = g.group_size;
    a.kv_heads = g.num_kv_heads;
    a.chunk = g.chunk;
    a.log2c = ilog2(g.chunk);
    a.levels = g.levels;
    a.mode = sel->mode;
    a.p = sel->p;
    for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
        if (sel->mode == ZHA_TOPK)
            a.k[i] = sel->k[i < sel->num_k ? i : sel->num_k - 1];
        else
            a.k[i] = 1;
    }
    a.sel_cap = sel->max_blocks_per_walk;
    a.cand_cap = cand_capacity(t, sel);
    a.sharpness = g.sharpness;
    // roots: all level-L nodes plus the parentless nodes of lower levels
    int64_t n0 = a.nl[g.levels];
    for (int l = 1; l < g.levels; ++l) n0 += a.nl[l] - int64_t(g.chunk) * a.nl[l + 1];
    a.n_roots = n0;
    if (n0 > a.cand_cap) n0 = a.cand_cap;
    // union engine: the first steps whose pair lists cannot exceed
    // kSmallList nodes run in one launch; a root at level l adds at most
    // c^s nodes to the list of step s < l
    a.small_steps = 0;
    if (engine == ZHA_ENGINE_UNION) {
        double all = 0.0;                          // nodes of the fused steps together
        for (int s = 0; s < g.levels && s < ZHA_MAX_STEPS; ++s) {
            double bound = 0.0, cs = 1.0;
            for (int i = 0; i < s; ++i) cs *= g.chunk;
            for (int l = s + 1; l <= g.levels; ++l) {
                const int64_t roots = (l == g.levels) ? a.nl[l] : a.nl[l] - int64_t(g.chunk) * a.nl[l + 1];
                bound += static_cast<double>(roots) * cs;
            }
            all += bound;
            if (bound > kSmallList || all > kTopNodes || all > a.cand_cap) break;
            a.small_steps = s + 1;
        }
    }
    // level-synchronous decode engine: its first steps run from one dense
    // score table of the top levels (all their nodes, every head of the
    // pair) when those levels are small -- at most kTopRowsMax nodes per pair
    // -- and a step's candidates cover most of its level (always under
    // top-p; under top-K when K_t * c reaches half the level below)
    a.top_steps = 0;
    a.top_lo = g.levels + 1;
    a.top_rows = 0;
    a.top_lds = 0;
    if (engine == ZHA_ENGINE_LEVEL_SYNC && qph == 1 && g.group_size <= 16) {
        int64_t rows = 0;
        for (int s = 0; s < g.levels && s < ZHA_MAX_STEPS; ++s) {
            const int l = g.levels - s;
            if (rows + t->level_cap[l] > kTopRowsMax || rows + t->level_cap[l] > a.cand_cap) break;
            if (sel->mode == ZHA_TOPK && s > 0 && 2 * int64_t(a.k[s - 1]) * g.chunk < t->level_cap[l]) break;
            rows += t->level_cap[l];
            a.top_steps = s + 1;
            a.top_lo = l;
        }
        if (a.top_steps > 0) {
            int64_t off = 0;
            for (int l = 0; l <= ZHA_MAX_LEVELS + 1; ++l) a.top_off[l] = 0;
            for (int l = a.top_lo; l <= g.levels; ++l) {
                a.top_off[l] = off;
                off += t->level_cap[l];
            }
            a.top_rows = off;
            // the top steps' lists (and the one they hand over) fit in LDS
            // when none can exceed kTopList candidates: step s meets at most
            // the level L - s of the top chain plus, for the parentless roots
            // of each lower level l, their level-(l - s) descendants
            a.top_lds = 1;
            for (int st = 0; st <= a.top_steps; ++st) {
                int64_t cs = 1;
                for (int i = 0; i < st; ++i) cs *= g.chunk;
                int64_t bound = g.levels - st >= 1 ? a.nl[g.levels - st] : 0;
                for (int l = 1; l < g.levels; ++l) {
                    if (l - st < 1) continue;
                    const int64_t par = a.nl[l] - int64_t(g.chunk) * a.nl[l + 1];
                    bound += std::min(a.nl[l - st], par * cs);
                }
                if (bound > kTopList) a.top_lds = 0;
            }
        }
    }
    // union engine with fewer than 16 heads per KV head: the heads' lists
    // overlap less, and on the last two steps (the widest) the
    // level-synchronous engine's per-walk scoring is faster; hand over there
    a.ls_from = 0;
    if (engine == ZHA_ENGINE_UNION && g.group_size < 16) {
        const int from = std::max(a.small_steps + 1, g.levels - 2);
        if (from < g.levels && from < ZHA_MAX_STEPS) a.ls_from = from;
    }
    return n0;
}

zha_status do_search(const zha_tree *t, const void *q, int32_t qph, const zha_select *sel,
                     int32_t *sel_blocks, int32_t *sel_count, zha_walk_stats *stats, uint32_t *status,
                     uint32_t *visited, void *ws, hipStream_t st) {
    const zha_geometry &g = t->geom;
    const int engine = resolve_engine(t, sel, qph);
    SearchArgs a;
    const int64_t n0 = fill_search(t, t->n_tokens, q, qph, sel, sel_blocks, sel_count, stats, status, visited,
                                   ws, engine, a);
    if (engine == ZHA_ENGINE_BLOCK)
        return hip_status(launch_block(a, g.head_dim, g.num_refs, g.dtype, g.summary_dtype, static_cast<int>(n0), st));
    if (engine == ZHA_ENGINE_LEVEL_SYNC && a.top_steps > 0)
        return hip_status(launch_top(a, g.head_dim, g.num_refs, g.dtype, g.summary_dtype, st));
    if (engine == ZHA_ENGINE_UNION)
        return hip_status(launch_union(a, g.head_dim, g.num_refs, g.dtype, g.summary_dtype, static_cast<int>(n0), st));
    return hip_status(launch_search(a, g.head_dim, g.num_refs, g.dtype, g.summary_dtype, engine, static_cast<int>(n0), st));
}

// Attention over block lists (tokens == nullptr) or token lists.
zha_status do_attn(const zha_tree *t, const void *q, int32_t qph, const void *k_cache,
                   const void *v_cache, const int32_t *sel_blocks, const int32_t *tokens,
                   const int32_t *sel_count, int32_t list_cap, int64_t keys_bound, void *out, void *ws,
                   hipStream_t st, int attn_engine = ZHA_ATTN_PER_WALK) {
    const zha_geometry &g = t->geom;
    const int64_t walks = walks_of(&g, qph);
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.sel_blocks = sel_blocks;
    a.tokens = tokens;
    a.sel_count = sel_count;
    const bool uni = attn_engine == ZHA_ATTN_UNION && tokens == nullptr;
    AttnWs lay = attn_ws_layout(g.head_dim, keys_bound, walks, uni ? t : nullptr, qph);
    char *wb = static_cast<char *>(ws);
    a.part = reinterpret_cast<float *>(wb + lay.part);
    a.item_off = reinterpret_cast<int32_t *>(wb + lay.item_off);
    a.item_walk = reinterpret_cast<int32_t *>(wb + lay.item_walk);
    a.max_tokens = g.max_tokens;
    a.n_tokens = t->n_tokens;
    a.n1 = level_count(t->n_tokens, g.chunk, 1);
    a.walks = static_cast<int32_t>(walks);
    a.qph = qph;
    a.heads = g.num_kv_heads * g.group_size;
    a.group = g.group_size;
    a.kv_heads = g.num_kv_heads;
    a.chunk = g.chunk;
    a.sel_cap = list_cap;
    const int64_t items = attn_max_items(keys_bound, walks);
    a.grid = static_cast<int32_t>(items < 2048 ? items : 2048);
    a.block_mfma = (qph > 1 && tokens == nullptr && g.dtype == ZHA_BF16) ? 1 : 0;
    a.sharpness = g.sharpness;
    a.pairs = g.batch * g.num_kv_heads;
    a.log2c = ilog2(g.chunk);
    if (uni) {
        a.umask = reinterpret_cast<uint16_t *>(wb + lay.umask);
        a.uchunk = reinterpret_cast<uint32_t *>(wb + lay.uchunk);
        a.ic = reinterpret_cast<int32_t *>(wb + lay.ic);
        a.part = reinterpret_cast<float *>(wb + lay.upart);
        a.bpart = qph > 1 ? reinterpret_cast<float *>(wb + lay.bpart) : nullptr;
        a.ukey = qph > 1 ? reinterpret_cast<unsigned long long *>(wb + lay.ukey) : nullptr;
        a.uperm = qph > 1 ? reinterpret_cast<int32_t *>(wb + lay.uperm) : nullptr;
        a.uinv = qph > 1 ? reinterpret_cast<int32_t *>(wb + lay.uinv) : nullptr;
        a.n1cap = lay.u.n1cap;
        a.ugroups = lay.u.ugroups;
        a.cwords = static_cast<int32_t>(lay.u.cwords);
        a.gpp = static_cast<int32_t>(lay.u.gpp);
        // decode: about 2048 workgroups in all, each over a contiguous range
        // of chunks; prefill: one workgroup per group, over all chunks
        const int64_t nchunks = (a.n1 + kUaBlocks - 1) / kUaBlocks;
        int64_t wpg = std::min<int64_t>(lay.u.wpg_max, std::max<int64_t>(1, nchunks));
        const int64_t cpw = nchunks > 0 ? (nchunks + wpg - 1) / wpg : 0;
        if (cpw > 0) wpg = (nchunks + cpw - 1) / cpw;
        a.items_pp = static_cast<int32_t>(wpg);
        a.ua_cpw = static_cast<int32_t>(cpw);
        return hip_status(launch_attn_union(a, g.head_dim, st));
    }
    return hip_status(launch_attn(a, g.head_dim, g.dtype, st));
}

// Logits row stride of the dense baseline: a multiple of 4 floats, so a lane
// stores 4 consecutive logits as one 16-byte write.
uint64_t dense_row_pad(const zha_geometry &g) { return (uint64_t(g.max_tokens) + 3) / 4 * 4; }

struct DenseWs {
    uint64_t logits, sel, sel_n, budget, attn, total;
};
DenseWs dense_ws_layout(const zha_tree *t, int32_t max_budget) {
    const zha_geometry &g = t->geom;
    const uint64_t walks = static_cast<uint64_t>(walks_of(&g, 1));
    DenseWs l;
    l.logits = 0;
    l.sel = align_up(walks * dense_row_pad(g) * sizeof(float));
    l.sel_n = l.sel + align_up(walks * uint64_t(max_budget) * sizeof(int32_t));
    l.budget = l.sel_n + align_up(walks * sizeof(int32_t));
    l.attn = l.budget + align_up(walks * sizeof(int32_t));
    l.total = l.attn + attn_ws_layout(g.head_dim, max_budget, walks).total;
    return l;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept; nullptr on a HIP error.
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

uint64_t zha_tree_bytes(const zha_geometry *g) {
    if (check_geometry(g) != ZHA_OK) return 0;
    const uint64_t pairs = uint64_t(g->batch) * g->num_kv_heads;
    uint64_t off = 0;
    for (int l = 1; l <= g->levels; ++l) {
        const uint64_t cap = static_cast<uint64_t>(level_count(g->max_tokens, g->chunk, l));
        off += align_up(pairs * cap * g->num_refs * g->head_dim * summary_bytes(g));
        off += align_up(pairs * cap * g->num_refs * sizeof(float));
    }
    return off;
}

int32_t zha_depth_for(int64_t n_tokens, int32_t chunk, int64_t max_top) {
    if (n_tokens < 0 || chunk < 2 || chunk > 64 || (chunk & (chunk - 1)) || max_top < 1) return -1;
    int32_t L = 1;
    while (L < ZHA_MAX_LEVELS && level_count(n_tokens, chunk, L) > max_top) ++L;
    return L;
}

zha_status zha_tree_init(zha_tree *t, const zha_geometry *g, void *tree_mem, uint64_t tree_bytes,
                         const float *refs) {
    if (!t) return ZHA_ERR_ARG;
    zha_status s = check_geometry(g);
    if (s != ZHA_OK) return s;
    if (!tree_mem || !refs) return ZHA_ERR_ARG;
    if (!aligned16(tree_mem) || !aligned16(refs)) return ZHA_ERR_ALIGN;
    const uint64_t need = zha_tree_bytes(g);
    if (tree_bytes < need) return ZHA_ERR_CAPACITY;
    memset(t, 0, sizeof(*t));
    t->geom = *g;
    t->n_tokens = 0;
    t->tree_mem = tree_mem;
    t->tree_bytes = tree_bytes;
    t->refs = refs;
    const uint64_t pairs = uint64_t(g->batch) * g->num_kv_heads;
    uint64_t off = 0;
    for (int l = 1; l <= g->levels; ++l) {
        const int64_t cap = level_count(g->max_tokens, g->chunk, l);
        t->level_cap[l] = cap;
        t->key_off[l] = off;
        off += align_up(pairs * uint64_t(cap) * g->num_refs * g->head_dim * summary_bytes(g));
        t->bias_off[l] = off;
        off += align_up(pairs * uint64_t(cap) * g->num_refs * sizeof(float));
    }
    return ZHA_OK;
}

zha_status zha_build(zha_tree *t, const void *k_cache, int64_t n_tokens, void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if (!k_cache) return ZHA_ERR_ARG;
    if (!aligned16(k_cache)) return ZHA_ERR_ALIGN;
    if (n_tokens < 0 || n_tokens > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    s = run_levels(t, k_cache, 0, n_tokens, static_cast<hipStream_t>(stream));
    if (s == ZHA_OK) t->n_tokens = n_tokens;
    return s;
}

zha_status zha_append(zha_tree *t, const void *k_cache, int64_t n_new, void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if (!k_cache) return ZHA_ERR_ARG;
    if (!aligned16(k_cache)) return ZHA_ERR_ALIGN;
    if (n_new < 0) return ZHA_ERR_ARG;
    if (t->n_tokens + n_new > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    s = run_levels(t, k_cache, t->n_tokens, t->n_tokens + n_new, static_cast<hipStream_t>(stream));
    if (s == ZHA_OK) t->n_tokens += n_new;
    return s;
}

uint64_t zha_search_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head) {
    if (check_tree(t) != ZHA_OK || check_select(sel) != ZHA_OK || q_per_head < 1) return 0;
    return search_ws_layout(t, sel, q_per_head).total;
}

int32_t zha_search_engine(const zha_tree *t, const zha_select *sel, int32_t q_per_head) {
    if (check_tree(t) != ZHA_OK || check_select(sel) != ZHA_OK || q_per_head < 1) return -1;
    const int e = resolve_engine(t, sel, q_per_head);
    if (e == ZHA_ENGINE_UNION && (q_per_head != 1 || t->geom.group_size > 16)) return -1;
    if (e == ZHA_ENGINE_FUSED) return -1;             // zha_forward only: zha_search never runs it
    return e;
}

int32_t zha_attn_engine(const zha_tree *t, const zha_select *sel, int32_t q_per_head) {
    if (check_tree(t) != ZHA_OK || check_select(sel) != ZHA_OK || q_per_head < 1) return -1;
    const int e = resolve_attn(t, sel, q_per_head);
    if (e == ZHA_ATTN_UNION && !union_attn_ok(t, q_per_head)) return -1;
    return e;
}

uint64_t zha_visited_words(const zha_tree *t) {
    if (check_tree(t) != ZHA_OK) return 0;
    return static_cast<uint64_t>(visited_words_per_pair(t)) * t->geom.batch * t->geom.num_kv_heads;
}

zha_status zha_search(const zha_tree *t, const void *q, int32_t q_per_head, const zha_select *sel,
                      int32_t *sel_blocks, int32_t *sel_count, zha_walk_stats *stats,
                      uint32_t *status, uint32_t *visited, void *ws, uint64_t ws_bytes, void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if ((s = check_select(sel)) != ZHA_OK) return s;
    if (q_per_head < 1) return ZHA_ERR_ARG;
    if (walks_of(&t->geom, q_per_head) > (int64_t(1) << 24)) return ZHA_ERR_UNSUPPORTED;
    if (!q || !sel_blocks || !sel_count || !status || !ws) return ZHA_ERR_ARG;
    if (!aligned16(q) || !aligned16(ws) || !aligned_n(sel_blocks, 4) || !aligned_n(sel_count, 4) ||
        !aligned_n(status, 4) || (stats && !aligned_n(stats, 8)) || (visited && !aligned_n(visited, 4)))
        return ZHA_ERR_ALIGN;
    if (sel->engine == ZHA_ENGINE_UNION && (q_per_head != 1 || t->geom.group_size > 16))
        return ZHA_ERR_UNSUPPORTED;
    if (sel->engine == ZHA_ENGINE_FUSED) return ZHA_ERR_UNSUPPORTED;     // zha_forward only
    if (ws_bytes < zha_search_workspace_bytes(t, sel, q_per_head)) return ZHA_ERR_WORKSPACE;
    return do_search(t, q, q_per_head, sel, sel_blocks, sel_count, stats, status, visited, ws,
                     static_cast<hipStream_t>(stream));
}

uint64_t zha_attn_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head) {
    if (check_tree(t) != ZHA_OK || check_select(sel) != ZHA_OK || q_per_head < 1) return 0;
    return attn_ws_bytes(t, sel, q_per_head);
}

zha_status zha_sparse_attn(const zha_tree *t, const void *q, int32_t q_per_head, const void *k_cache,
                           const void *v_cache, const zha_select *sel, const int32_t *sel_blocks,
                           const int32_t *sel_count, void *out, void *ws, uint64_t ws_bytes,
                           void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if ((s = check_select(sel)) != ZHA_OK) return s;
    if (q_per_head < 1) return ZHA_ERR_ARG;
    if (walks_of(&t->geom, q_per_head) > (int64_t(1) << 24)) return ZHA_ERR_UNSUPPORTED;
    if (q_per_head > 1 && t->n_tokens + q_per_head > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    if (!q || !k_cache || !v_cache || !sel_blocks || !sel_count || !out || !ws) return ZHA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(ws) || !aligned_n(sel_blocks, 4) || !aligned_n(sel_count, 4))
        return ZHA_ERR_ALIGN;
    if (ws_bytes < zha_attn_workspace_bytes(t, sel, q_per_head)) return ZHA_ERR_WORKSPACE;
    const int ae = resolve_attn(t, sel, q_per_head);
    if (ae == ZHA_ATTN_UNION && !union_attn_ok(t, q_per_head)) return ZHA_ERR_UNSUPPORTED;
    return do_attn(t, q, q_per_head, k_cache, v_cache, sel_blocks, nullptr, sel_count,
                   sel->max_blocks_per_walk, tree_keys_bound(t, sel, q_per_head), out, ws,
                   static_cast<hipStream_t>(stream), ae);
}

zha_status zha_sparse_attn_noalloc(const zha_tree *t, const void *q, int32_t q_per_head,
                                   const void *k_cache, const void *v_cache, const zha_select *sel,
                                   const int32_t *sel_blocks, const int32_t *sel_count, void *out,
                                   void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if ((s = check_select(sel)) != ZHA_OK) return s;
    if (q_per_head < 1) return ZHA_ERR_ARG;
    if (walks_of(&t->geom, q_per_head) > (int64_t(1) << 24)) return ZHA_ERR_UNSUPPORTED;
    if (q_per_head > 1 && t->n_tokens + q_per_head > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    if (!q || !k_cache || !v_cache || !sel_blocks || !sel_count || !out) return ZHA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned_n(sel_blocks, 4) || !aligned_n(sel_count, 4))
        return ZHA_ERR_ALIGN;
    if (sel->attn_engine == ZHA_ATTN_UNION) return ZHA_ERR_UNSUPPORTED;
    const int64_t keys_bound = tree_keys_bound(t, sel, q_per_head);
    const uint64_t need = attn_ws_layout(t->geom.head_dim, keys_bound, walks_of(&t->geom, q_per_head)).total;
    if (need > ZHA_NOALLOC_SCRATCH_BYTES) return ZHA_ERR_WORKSPACE;
    void *ws = scratch_ptr();
    if (!ws) return ZHA_ERR_HIP;
    return do_attn(t, q, q_per_head, k_cache, v_cache, sel_blocks, nullptr, sel_count,
                   sel->max_blocks_per_walk, keys_bound, out, ws, static_cast<hipStream_t>(stream),
                   ZHA_ATTN_PER_WALK);
}

uint64_t zha_forward_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head) {
    if (check_tree(t) != ZHA_OK || check_select(sel) != ZHA_OK || q_per_head < 1) return 0;
    return forward_ws_layout(t, sel, q_per_head).total;
}

zha_status zha_forward(zha_tree *t, int64_t n_new, const void *q, int32_t q_per_head,
                       const void *k_cache, const void *v_cache, const zha_select *sel, void *out,
                       zha_walk_stats *stats, uint32_t *status, void *ws, uint64_t ws_bytes,
                       void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if ((s = check_select(sel)) != ZHA_OK) return s;
    if (q_per_head < 1 || n_new < 0) return ZHA_ERR_ARG;
    if (walks_of(&t->geom, q_per_head) > (int64_t(1) << 24)) return ZHA_ERR_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !out || !status || !ws) return ZHA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(ws) || !aligned_n(status, 4) || (stats && !aligned_n(stats, 8)))
        return ZHA_ERR_ALIGN;
    if (t->n_tokens + n_new > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    if (q_per_head > 1 && t->n_tokens + q_per_head > t->geom.max_tokens) return ZHA_ERR_CAPACITY;
    if (sel->engine == ZHA_ENGINE_UNION && (q_per_head != 1 || t->geom.group_size > 16))
        return ZHA_ERR_UNSUPPORTED;
    if (sel->engine == ZHA_ENGINE_FUSED && (q_per_head != 1 || n_new > 1 || !fused_fits(t)))
        return ZHA_ERR_UNSUPPORTED;
    const int ae = resolve_attn(t, sel, q_per_head);
    if (ae == ZHA_ATTN_UNION && !union_attn_ok(t, q_per_head) && sel->engine != ZHA_ENGINE_FUSED)
        return ZHA_ERR_UNSUPPORTED;
    if (ws_bytes < zha_forward_workspace_bytes(t, sel, q_per_head)) return ZHA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sel->engine == ZHA_ENGINE_FUSED) {
        // the append, the walk and the attention in one launch
        const zha_geometry &g = t->geom;
        const int64_t n_tok = t->n_tokens + n_new;
        ForwardWs lay = forward_ws_layout(t, sel, q_per_head);
        char *wsb = static_cast<char *>(ws);
        FusedArgs f;
        memset(&f, 0, sizeof(f));
        (void)fill_search(t, n_tok, q, 1, sel, reinterpret_cast<int32_t *>(wsb + lay.sel_blocks),
                          reinterpret_cast<int32_t *>(wsb + lay.sel_count), stats, status, nullptr,
                          wsb + lay.search, ZHA_ENGINE_PERSISTENT, f.s);
        f.k = k_cache;
        f.v = v_cache;
        f.out = out;
        f.refs = t->refs;
        f.max_tokens = g.max_tokens;
        f.fresh_m = 0;
        for (int l = 1; l <= g.levels; ++l) {
            if (level_count(n_tok, g.chunk, l) > level_count(t->n_tokens, g.chunk, l)) f.fresh_m = l;
            f.tree_k[l] = static_cast<char *>(t->tree_mem) + t->key_off[l];
            f.tree_b[l] = reinterpret_cast<float *>(static_cast<char *>(t->tree_mem) + t->bias_off[l]);
        }
        s = hip_status(launch_fused(f, g.head_dim, g.num_refs, g.dtype, g.summary_dtype, st));
        if (s == ZHA_OK) t->n_tokens = n_tok;
        return s;
    }
    // decode: the new rows join the tree first, so the query sees them
    if (q_per_head == 1 && n_new > 0) {
        s = run_levels(t, k_cache, t->n_tokens, t->n_tokens + n_new, st);
        if (s != ZHA_OK) return s;
        t->n_tokens += n_new;
    }
    ForwardWs lay = forward_ws_layout(t, sel, q_per_head);
    char *w = static_cast<char *>(ws);
    int32_t *sb = reinterpret_cast<int32_t *>(w + lay.sel_blocks);
    int32_t *sc = reinterpret_cast<int32_t *>(w + lay.sel_count);
    s = do_search(t, q, q_per_head, sel, sb, sc, stats, status, nullptr, w + lay.search, st);
    if (s != ZHA_OK) return s;
    s = do_attn(t, q, q_per_head, k_cache, v_cache, sb, nullptr, sc, sel->max_blocks_per_walk,
                tree_keys_bound(t, sel, q_per_head), out, w + lay.attn, st, ae);
    if (s != ZHA_OK) return s;
    // prefill: the block joins the tree after its own queries have searched it
    if (q_per_head > 1 && n_new > 0) {
        s = run_levels(t, k_cache, t->n_tokens, t->n_tokens + n_new, st);
        if (s != ZHA_OK) return s;
        t->n_tokens += n_new;
    }
    return ZHA_OK;
}

uint64_t zha_dense_workspace_bytes(const zha_tree *t, int32_t max_budget) {
    if (check_tree(t) != ZHA_OK || max_budget < 1) return 0;
    return dense_ws_layout(t, max_budget).total;
}

// Both dense baselines: logits, the selection (budget per walk given, or
// from top-p over keys when budget is null), then attention.
zha_status dense_attn(const zha_tree *t, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *budget, float p, int32_t max_budget, void *out, int32_t *sel_tokens,
                      int32_t *sel_count, uint32_t *status, void *ws, uint64_t ws_bytes, void *stream) {
    zha_status s = check_tree(t);
    if (s != ZHA_OK) return s;
    if (max_budget < 1) return ZHA_ERR_ARG;
    if (!q || !k_cache || !v_cache || !out || !ws) return ZHA_ERR_ARG;
    if (!budget && !isfinite(p)) return ZHA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(ws) || (budget && !aligned_n(budget, 4)) || (sel_tokens && !aligned_n(sel_tokens, 4)) ||
        (sel_count && !aligned_n(sel_count, 4)) || (status && !aligned_n(status, 4)))
        return ZHA_ERR_ALIGN;
    if (ws_bytes < zha_dense_workspace_bytes(t, max_budget)) return ZHA_ERR_WORKSPACE;
    const zha_geometry &g = t->geom;
    hipStream_t st = static_cast<hipStream_t>(stream);
    DenseWs lay = dense_ws_layout(t, max_budget);
    char *wb = static_cast<char *>(ws);
    DenseArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k_cache;
    a.budget_out = budget ? nullptr : reinterpret_cast<int32_t *>(wb + lay.budget);
    a.budget = budget ? budget : a.budget_out;
    a.status = status;
    a.p = p;
    a.logits = reinterpret_cast<float *>(wb + lay.logits);
    a.sel = sel_tokens ? sel_tokens : reinterpret_cast<int32_t *>(wb + lay.sel);
    a.sel_n = sel_count ? sel_count : reinterpret_cast<int32_t *>(wb + lay.sel_n);
    a.max_tokens = g.max_tokens;
    a.n_tokens = t->n_tokens;
    a.row_pad = static_cast<int64_t>(dense_row_pad(g));
    a.walks = static_cast<int32_t>(walks_of(&g, 1));
    a.heads = g.num_kv_heads * g.group_size;
    a.group = g.group_size;
    a.kv_heads = g.num_kv_heads;
    a.max_budget = max_budget;
    a.sharpness = g.sharpness;
    s = hip_status(launch_dense(a, g.head_dim, g.dtype, st));
    if (s != ZHA_OK) return s;
    return do_attn(t, q, 1, k_cache, v_cache, nullptr, a.sel, a.sel_n, max_budget, max_budget, out,
                   wb + lay.attn, st);
}

zha_status zha_dense_topk_attn(const zha_tree *t, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *budget, int32_t max_budget,
                               void *out, int32_t *sel_tokens, void *ws, uint64_t ws_bytes,
                               void *stream) {
    if (!budget) return ZHA_ERR_ARG;
    return dense_attn(t, q, k_cache, v_cache, budget, 0.f, max_budget, out, sel_tokens, nullptr, nullptr, ws,
                      ws_bytes, stream);
}

zha_status zha_dense_topp_attn(const zha_tree *t, const void *q, const void *k_cache,
                               const void *v_cache, float p, int32_t max_budget, void *out,
                               int32_t *sel_tokens, int32_t *sel_count, uint32_t *status, void *ws,
                               uint64_t ws_bytes, void *stream) {
    return dense_attn(t, q, k_cache, v_cache, nullptr, p, max_budget, out, sel_tokens, sel_count, status, ws,
                      ws_bytes, stream);
}

zha_status zha_bw_probe(const void *buf, uint64_t bytes, float *sink, void *stream) {
    if (!buf || !sink) return ZHA_ERR_ARG;
    if (!aligned16(buf) || !aligned_n(sink, 4)) return ZHA_ERR_ALIGN;
    return hip_status(launch_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

const char *zha_status_string(zha_status s) {
    switch (s) {
        case ZHA_OK: return "ok";
        case ZHA_ERR_ARG: return "invalid argument";
        case ZHA_ERR_SHAPE: return "inconsistent shape";
        case ZHA_ERR_ALIGN: return "device pointer not aligned";
        case ZHA_ERR_CAPACITY: return "capacity exceeded";
        case ZHA_ERR_WORKSPACE: return "workspace too small";
        case ZHA_ERR_UNSUPPORTED: return "unsupported geometry or mode";
        case ZHA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
