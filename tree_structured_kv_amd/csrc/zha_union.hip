// zha_union.hip -- the union search engine: one candidate list per
// (sequence, KV head) pair, shared by the pair's query heads.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "Common misunderstandings": each attention head walks the tree
// on its own -- here every head still gets its own scores and its own cut
// ("How does top-p differ from top-K?") over exactly its own candidates
// ("Run a small tree yourself").  What the heads of a group share is the
// tree, so they share the reads: at step t the pair's list holds the union
// of the heads' candidate sets (the children of every node any head opened,
// in list order), and every node of it is scored for all heads at once.
//
// Per step:
//   k_un_score  grid-wide over a flat list of (pair, list position, node)
//               entries: a node record is read once and scored for all
//               heads of the group with fp32 16x16x4 matrix-core tiles
//               (heads x (node, ref)), then s * dot + bias and the max over
//               references;
//   k_un_cut    one workgroup per walk (head h of pair p): its candidates are
//               the children of the nodes it opened at the previous step,
//               found through the parents' ranks in the union list; the
//               head's exact radix-select cut, its level-1 selections in
//               span order, the higher nodes it opens (list positions, in
//               order) and head bit h on them;
//   k_un_expand up to kExpSlices workgroups per pair, each over a slice of
//               its list: ranks of the opened nodes (in list order), the
//               next union list (their children, written coalesced) and
//               its flat scoring entries.
// A head's candidates keep the list order, so selections, statistics and
// the cut are those of a walk of that head alone.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// Four bf16 values (two packed 32-bit words) as a matrix-core operand.
__device__ __forceinline__ short4_t pack4(uint32_t lo, uint32_t hi) {
    short4_t r;
    r[0] = static_cast<short>(lo & 0xffffu);
    r[1] = static_cast<short>(lo >> 16);
    r[2] = static_cast<short>(hi & 0xffffu);
    r[3] = static_cast<short>(hi >> 16);
    return r;
}

constexpr int kScoreThreads = 256;
constexpr int kUG = 2;                // matrix tiles in flight per wavefront
constexpr int kLdsCand = 14848;       // candidate scores a cut stages in LDS (58 KB)
constexpr int kLdsPar = 2048;         // parents whose ranks and node ids a cut stages in LDS (16 KB)
constexpr int kExpMin = 256;          // list entries per expand workgroup (at least)
static_assert(kSmallList <= 64, "a fused step's candidates fit one wavefront, one per lane");

__device__ __forceinline__ int head_walk(const SearchArgs &a, int pair, int h) {
    const int b = pair / a.kv_heads, g = pair % a.kv_heads;
    return b * a.heads + g * a.group + h;
}

__device__ __forceinline__ int round_flat(int n) { return (n + kFlatPad - 1) / kFlatPad * kFlatPad; }

// A head's candidate ids by index: child x & (c - 1) of its opened parent
// x >> log2c when the parents' node ids are staged in LDS, else the pair's
// list entry at the candidate's list position.
template <typename Pos>
struct CandIds {
    const uint32_t *ids;
    Pos pos;
    const uint32_t *pid;              // parents' node ids in LDS, or null
    int log2c;
    __device__ __forceinline__ uint32_t operator[](int x) const {
        if (!pid) return ids[pos(x)];
        const uint32_t p = pid[x >> log2c];
        const uint32_t c = 1u << log2c;
        return (((p >> kLevelShift) - 1u) << kLevelShift) | ((p & kIndexMask) * c + (static_cast<uint32_t>(x) & (c - 1u)));
    }
};

struct ExpandShared {
    uint32_t seg_cnt[kWaves];
    uint32_t pre_cnt[kWaves];
    int32_t flat_base;
    int32_t need;
};

// Block-wide sum of a uint32 per thread (kThreads threads).
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, SelectShared &sh) {
    unsigned long long tot;
    (void)block_exscan64(v, sh.scan64, &tot);
    return static_cast<uint32_t>(tot);
}

}  // namespace

template <int R>
__global__ __launch_bounds__(512) void k_un_init(SearchArgs a) {
    const int tid = threadIdx.x;
    const int p = blockIdx.x;
    const int cap = a.cand_cap;
    if (p == 0 && tid <= ZHA_MAX_STEPS) a.tile_count[tid] = 0;
    __shared__ uint32_t s_flags;
    if (tid == 0) s_flags = 0;
    __syncthreads();
    uint32_t flags = 0;
    uint32_t *ids = a.u_ids + static_cast<int64_t>(p) * 2 * cap;
    const int n = write_roots(a, ids, flags);
    uint32_t *om = a.u_omask + static_cast<int64_t>(p) * 2 * cap;     // step 0's masks
    for (int i = tid; i < n; i += blockDim.x) om[i] = 0;
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid == 0) {
        a.u_n[2 * p] = n;
        a.u_n[2 * p + 1] = 0;
    }
    if (tid < a.group) {
        const int w = head_walk(a, p, tid);
        WalkState *st = a.state + w;
        st->n = n;
        st->buf = 0;
        st->sel_n = 0;
        st->unforced = 0;
        st->flags = s_flags;
        st->steps = 0;
        for (int i = 0; i < ZHA_MAX_STEPS; ++i) { st->scored[i] = 0; st->opened[i] = 0; }
        a.u_next[w] = 0;
        if (n == 0) finish_walk<R>(a, w, 0, st->scored, st->opened, 0, 0, s_flags);
    }
}

// Level bases of the node records, staged in LDS: a block may mix levels.
struct LevelTables {
    const float *kap[ZHA_MAX_LEVELS + 1];
    const float *bet[ZHA_MAX_LEVELS + 1];
    int64_t cap[ZHA_MAX_LEVELS + 1];
};

__device__ __forceinline__ void load_tables(const SearchArgs &a, LevelTables &tb) {
    if (threadIdx.x <= ZHA_MAX_LEVELS) {
        tb.kap[threadIdx.x] = a.kap[threadIdx.x];
        tb.bet[threadIdx.x] = a.bet[threadIdx.x];
        tb.cap[threadIdx.x] = a.cap[threadIdx.x];
    }
}

// Step t scoring.  The flat list holds, pair after pair, one entry per node
// of the pair's union list, each pair's run padded to a multiple of
// kFlatPad (pad entries repeat a real node and store nothing); at t = 0 the
// entries are the roots, the same count n0 for every pair, and are computed.
// A wavefront takes NPG = 16/R nodes per matrix tile (the 16 columns are
// (node, ref), the rows the group's heads), kUG tiles per block, and walks
// one contiguous run of blocks, fetching the next block's entries while the
// current block's records load; a block never straddles two pairs.  Matrix
// step k of lane group q = lane/16 multiplies element d = 16*(k/4) + 4*q +
// k%4 of the query and of the reference row (one permutation of D for both
// operands), so one 16-byte load of the four lanes of a column reads 64
// contiguous bytes of its row.
//
// score_run: one wavefront scores blocks b0 .. b1-1 (WB = NPG*kUG entries
// each) of a list whose entry e is entry(e) = {pair, list position (-1:
// pad), node id}; out(pair, position, id, grp, v) takes the scores v[0..3]
// of heads 4*grp .. 4*grp+3 of each real entry (one lane per entry and
// grp).
template <int D, int R, typename QT, typename ST, typename Entry, typename Out>
__device__ __forceinline__ void score_run(const SearchArgs &a, const LevelTables &tb, Entry entry, int b0, int b1,
                                          Out out) {
    constexpr int NPG = 16 / R;           // nodes per matrix tile
    constexpr int KS = D / 4;             // 16x16x4 steps
    constexpr int WB = NPG * kUG;         // nodes per block
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;
    const float *const *s_kap = tb.kap;
    const float *const *s_bet = tb.bet;
    const int64_t *s_cap = tb.cap;
    if (b0 >= b1) return;
    const float s = a.sharpness;

    int4 nxt[kUG];
#pragma unroll
    for (int u = 0; u < kUG; ++u) nxt[u] = entry(b0 * WB + u * NPG + col / R);
    int cur_pair = -1;
    // query operand: fp32 values, or for bf16 queries the raw 16-bit pairs
    // (half the registers; widened per matrix step)
    constexpr bool kPacked = sizeof(QT) == 2;
    float qa[kPacked ? 1 : KS];
    uint32_t qpk[kPacked ? KS / 2 : 1];
    auto qval = [&](int k) -> float {
        if constexpr (kPacked)
            return __uint_as_float((k & 1) ? (qpk[k >> 1] & 0xffff0000u) : (qpk[k >> 1] << 16));
        else
            return qa[k];
    };
    // bf16 keys and queries go to bf16 matrix products instead
    constexpr bool kBf16Mma = sizeof(ST) == 2 && sizeof(QT) == 2;
    constexpr int KS2 = D / 16;           // 16x16x16 steps
    short4_t qh[kBf16Mma ? KS2 : 1];
    // query operand: row = head `col` of the pair's group (zero past G)
    auto load_query = [&](int p) {
        if (p == cur_pair) return;
        cur_pair = p;
        const bool ok = col < a.group;
        const int w = head_walk(a, p, ok ? col : 0);
        const QT *qrow = static_cast<const QT *>(a.q) + static_cast<int64_t>(w) * D;
        if constexpr (kBf16Mma) {
#pragma unroll
            for (int m = 0; m < KS2 / 2; ++m) {
                uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * m + 8 * grp);
                if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
                qh[2 * m] = pack4(v.x, v.y);
                qh[2 * m + 1] = pack4(v.z, v.w);
            }
        } else if constexpr (kPacked) {
            const QT *qp = qrow + 4 * grp;
#pragma unroll
            for (int j = 0; j < KS / 4; ++j) {
                const uint2 v = *reinterpret_cast<const uint2 *>(qp + 16 * j);
                qpk[2 * j] = ok ? v.x : 0u;
                qpk[2 * j + 1] = ok ? v.y : 0u;
            }
        } else {
            const QT *qp = qrow + 4 * grp;
#pragma unroll
            for (int j = 0; j < KS / 4; ++j) Vec4<QT>::load(qp + 16 * j, qa + 4 * j);
#pragma unroll
            for (int k = 0; k < KS; ++k) qa[k] = ok ? qa[k] : 0.f;
        }
    };
    for (int b = b0; b < b1; ++b) {
        int4 ent[kUG];
#pragma unroll
        for (int u = 0; u < kUG; ++u) ent[u] = nxt[u];
        if (b + 1 < b1) {
#pragma unroll
            for (int u = 0; u < kUG; ++u) nxt[u] = entry((b + 1) * WB + u * NPG + col / R);
        }
        const int p = __builtin_amdgcn_readfirstlane(ent[0].x);
        float bias[kUG];
        float4_t acc[kUG];
#pragma unroll
        for (int u = 0; u < kUG; ++u) acc[u] = float4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf16Mma) {
            // bf16 keys and queries: 16x16x16 bf16 products, exact products
            // summed in fp32.  Step k of lane group q takes elements
            // 32*(k/2) + 8*q + 4*(k%2) .. +3 of both rows, so one 16-byte
            // load serves two steps.
            short4_t kh[kUG][KS2];
#pragma unroll
            for (int u = 0; u < kUG; ++u) {
                const uint32_t id = static_cast<uint32_t>(ent[u].z);
                const int lvl = static_cast<int>(id >> kLevelShift);
                const int64_t node = static_cast<int64_t>(p) * s_cap[lvl] + (id & kIndexMask);
                const bf16_t *kp = reinterpret_cast<const bf16_t *>(s_kap[lvl]) + node * (R * D) + (col % R) * D + 8 * grp;
#pragma unroll
                for (int m = 0; m < KS2 / 2; ++m) {
                    const gu4_t v = gload_u4(kp + 32 * m);
                    kh[u][2 * m] = pack4(v.x, v.y);
                    kh[u][2 * m + 1] = pack4(v.z, v.w);
                }
                bias[u] = gload_f(s_bet[lvl] + node * R + (col % R));
            }
            load_query(p);
#pragma unroll
            for (int k = 0; k < KS2; ++k)
#pragma unroll
                for (int u = 0; u < kUG; ++u)
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qh[k], kh[u][k], acc[u], 0, 0, 0);
        } else {
        float kb[kUG][KS];
#pragma unroll
        for (int u = 0; u < kUG; ++u) {
            const uint32_t id = static_cast<uint32_t>(ent[u].z);
            const int lvl = static_cast<int>(id >> kLevelShift);
            const int64_t node = static_cast<int64_t>(p) * s_cap[lvl] + (id & kIndexMask);
            const ST *kp = reinterpret_cast<const ST *>(s_kap[lvl]) + node * (R * D) + (col % R) * D + 4 * grp;
#pragma unroll
            for (int k = 0; k < KS; k += 4) {
                GVec4<ST>::load(kp + 4 * k, &kb[u][k]);
            }
            bias[u] = gload_f(s_bet[lvl] + node * R + (col % R));
        }
        load_query(p);
        // the kUG products interleaved, so consecutive matrix ops are independent
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int u = 0; u < kUG; ++u)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(qval(k), kb[u][k], acc[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUG; ++u) {
            const int pos = ent[u].y;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = fmaf(s, acc[u][e], bias[u]);
                x = group_max<R>(x);
                if (x != x) x = -INFINITY;
                v[e] = (x == 0.f) ? 0.f : x;
            }
            if ((col % R) == 0 && pos >= 0) out(p, pos, static_cast<uint32_t>(ent[u].z), grp, v);
        }
    }
}

// Scores of heads 4*grp .. 4*grp+3 of list entry `pos` of pair p to
// u_score (one 16-byte store), and the node marked in the visited bitmap.
struct UScoreOut {
    const SearchArgs &a;
    __device__ __forceinline__ void operator()(int p, int pos, uint32_t id, int grp, const float (&v)[4]) const {
        const int gp = (a.group + 3) & ~3;
        if (4 * grp < a.group)
            *reinterpret_cast<float4 *>(a.u_score + (static_cast<int64_t>(p) * a.cand_cap + pos) * gp + 4 * grp) =
                make_float4(v[0], v[1], v[2], v[3]);
        if (a.visited && grp == 0) {
            const int64_t bitn = a.node_off[id >> kLevelShift] + (id & kIndexMask);
            atomicOr(a.visited + p * a.vis_words + (bitn >> 5), 1u << (bitn & 31));
        }
    }
};

template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kScoreThreads) void k_un_score(SearchArgs a, int t, int n0) {
    constexpr int WB = (16 / R) * kUG;    // nodes per block
    constexpr int kSW = kScoreThreads / 64;
    static_assert(kFlatPad % WB == 0, "a block must not straddle two pairs");
    const int wave = threadIdx.x >> 6;
    __shared__ LevelTables tb;
    load_tables(a, tb);
    __syncthreads();
    const int n0p = round_flat(n0);
    const int n_flat = (t == 0) ? a.pairs * n0p : a.tile_count[t];
    const int nb = n_flat / WB;
    const int nw = gridDim.x * kSW;
    const int per = (nb + nw - 1) / nw;
    const int b0 = (blockIdx.x * kSW + wave) * per;
    const int b1 = min(nb, b0 + per);
    const int4 *flat = a.u_flat + (t & 1) * a.flat_cap;
    // entry of flat position e: at t = 0 the roots of every pair, each
    // pair's run padded to a multiple of kFlatPad
    auto entry = [&](int e) -> int4 {
        if (t == 0) {
            const int p = e / n0p, pos = e - p * n0p;
            const uint32_t *ids = a.u_ids + static_cast<int64_t>(p) * 2 * a.cand_cap;
            const uint32_t id = ids[pos < n0 ? pos : n0 - 1];
            return make_int4(p, pos < n0 ? pos : -1, static_cast<int>(id), 0);
        }
        return flat[e];
    };
    score_run<D, R, QT, ST>(a, tb, entry, b0, b1, UScoreOut{a});
}

// Step t, one workgroup per walk (head h of pair p).  The head's candidates
// are, in order, the children of the list entries it opened at step t-1 (at
// t = 0: every root); child e of the entry of rank k among all opened
// entries sits at list position k*c + e, and those positions increase with
// the candidate index, so the ones inside a truncated list form a prefix.
// The parents' ranks are staged in LDS, the candidates' scores too when they
// fit (every pass of the cut then reads LDS), their ids in the walk's global
// array.  After the exact cut, level-1 nodes go to the selection in span
// order, higher nodes are recorded (list positions, in order) for the next
// step and get head bit h in the pair's open masks.
template <int R>
__device__ __forceinline__ void cut_head(const SearchArgs &a, int t, int w, SelectShared &sh, uint32_t *s_one,
                                         uint32_t *s_high, float *lds_sc, int32_t *lds_par, uint32_t *lds_pid) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = w / a.group, h = w % a.group;
    const uint32_t bit = 1u << h;
    const int cap = a.cand_cap, log2c = a.log2c, c = a.chunk;
    const int buf = t & 1;                         // list, masks and lengths alternate by step
    const int n_u = a.u_n[2 * p + buf];
    const int n_open_prev = (t == 0) ? 0 : a.u_next[w];
    if (t > 0 && n_open_prev == 0) return;         // this head opened nothing more
    WalkState *st = a.state + w;
    const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + buf) * cap;
    const uint32_t *prev_ids = a.u_ids + (static_cast<int64_t>(p) * 2 + (buf ^ 1)) * cap;   // step t-1's list
    const int gp = (a.group + 3) & ~3;
    const float *sc = a.u_score + static_cast<int64_t>(p) * cap * gp + h;   // score of position i: sc[i * gp]
    const int32_t *rank = a.u_rank + static_cast<int64_t>(p) * cap;
    uint32_t *om = a.u_omask + (static_cast<int64_t>(p) * 2 + buf) * cap;
    int32_t *opened_pos = a.u_open + static_cast<int64_t>(w) * cap;
    // the head's candidates' list positions when the parents' ranks do not
    // fit in LDS (the second of the walk's two candidate buffers)
    uint32_t *cux = a.cand + static_cast<int64_t>(w) * 2 * cap + cap;
    float *csc = a.h_score + static_cast<int64_t>(w) * cap;         // their scores (fallback)
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    const int64_t raw64 = (t == 0) ? n_u : static_cast<int64_t>(n_open_prev) * c;
    const int raw = static_cast<int>(raw64 < cap ? raw64 : cap);
    const bool par_lds = n_open_prev <= kLdsPar;
    if (t > 0) {
        if (par_lds) {
            for (int j0 = tid; j0 < n_open_prev; j0 += kScanU * kThreads) {
                int i[kScanU];
#pragma unroll
                for (int u = 0; u < kScanU; ++u) {
                    const int j = j0 + u * kThreads;
                    i[u] = j < n_open_prev ? opened_pos[j] : 0;
                }
#pragma unroll
                for (int u = 0; u < kScanU; ++u) {
                    const int j = j0 + u * kThreads;
                    if (j < n_open_prev) {
                        lds_par[j] = rank[i[u]];
                        if (t > a.small_steps) lds_pid[j] = prev_ids[i[u]];
                    }
                }
            }
        } else {
            for (int x0 = tid; x0 < raw; x0 += kScanU * kThreads) {
                int i[kScanU];
#pragma unroll
                for (int u = 0; u < kScanU; ++u) {
                    const int x = x0 + u * kThreads;
                    i[u] = x < raw ? opened_pos[x >> log2c] : 0;
                }
#pragma unroll
                for (int u = 0; u < kScanU; ++u) {
                    const int x = x0 + u * kThreads;
                    if (x < raw) cux[x] = static_cast<uint32_t>(rank[i[u]] * c + (x & (c - 1)));
                }
            }
        }
    }
    __syncthreads();
    auto position = [&](int x) -> int {
        if (t == 0) return x;
        if (par_lds) return lds_par[x >> log2c] * c + (x & (c - 1));
        return static_cast<int>(cux[x]);
    };
    // the candidates inside the list: a prefix of length cnt
    uint32_t valid = 0;
    for (int x = tid; x < raw; x += kThreads) valid += position(x) < n_u;
    const int cnt = static_cast<int>(block_sum_u32(valid, sh));   // also a barrier
    if (cnt == 0) {
        if (tid == 0) a.u_next[w] = 0;
        return;
    }
    const bool forced = step_forced(a, t, cnt);
    const bool sc_lds = cnt <= kLdsCand;
    float *vs = sc_lds ? lds_sc : csc;
    // the candidates' scores only: a node id is fetched where it is needed
    // (the few candidates tied at the cut's score, and the opened ones)
    float m = -INFINITY;
    if (!forced) {
        constexpr int GU = 2 * kScanU;             // score loads in flight per thread
        for (int x0 = tid; x0 < cnt; x0 += GU * kThreads) {
            float v[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int x = x0 + u * kThreads;
                v[u] = x < cnt ? sc[static_cast<int64_t>(position(x)) * gp] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int x = x0 + u * kThreads;
                if (x < cnt) {
                    vs[x] = v[u];
                    m = fmaxf(m, v[u]);
                }
            }
        }
    }
    __syncthreads();
    // the parents' node ids come from step t-1's list, which is in memory
    // only when a grid-wide step built it (not k_un_small's last step)
    const bool pid_lds = t > a.small_steps && par_lds;
    const CandIds<decltype(position)> cand{ids, position, pid_lds ? lds_pid : nullptr, log2c};
    unsigned long long tau = 0;
    uint32_t path = (sc_lds || forced) ? 0u : kPathLdsSpill;
    if (!forced) {
        const float mx = block_max(m, sh);
        // a list too long for LDS is cut from global memory: twice the
        // loads in flight per thread
        tau = sc_lds ? cut_tau_win(a, cnt, cand, lds_sc, mx, a.k[t], sh, &path)
                     : cut_tau_win<2 * kScanU>(a, cnt, cand, csc, mx, a.k[t], sh, &path);
    }

    // open, in candidate order: wavefront v owns segment v (64*kScanU a round)
    const int seg = ((cnt + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int c0 = wave * seg, c1 = min(cnt, c0 + seg);
    // the score decides unless it equals the cut's: then the span start does
    const uint32_t tau_hi = static_cast<uint32_t>(tau >> 32);
    auto opens = [&](int k, uint32_t &id) -> bool {
        if (!forced) {
            const float v = vs[k];
            const uint32_t hi = ordered_bits(v);
            if (hi < tau_hi) { id = 0; return false; }
            id = cand[k];
            return hi > tau_hi || rank_key(v, id, log2c) >= tau;
        }
        id = cand[k];
        return true;
    };
    uint32_t n1 = 0, nopen = 0, nhigh = 0;
    for (int b0 = c0; b0 < c1; b0 += 64 * kScanU) {
        bool op[kScanU];
        uint32_t id[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int k = b0 + 64 * u + lane;
            id[u] = 0;
            op[u] = k < c1 && opens(k, id[u]);
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            n1 += __popcll(__ballot(op[u] && (id[u] >> kLevelShift) == 1u));
            nopen += __popcll(__ballot(op[u]));
            nhigh += __popcll(__ballot(op[u] && (id[u] >> kLevelShift) > 1u));
        }
    }
    if (lane == 0) {
        s_one[wave] = n1;
        s_high[wave] = nhigh;
    }
    const uint32_t tot_open = block_sum_u32(lane == 0 ? nopen : 0u, sh);   // also a barrier
    const int64_t sel0 = st->sel_n;
    uint32_t pre1 = 0, tot1 = 0, preh = 0, toth = 0;
    for (int v = 0; v < kWaves; ++v) {
        if (v < wave) { pre1 += s_one[v]; preh += s_high[v]; }
        tot1 += s_one[v];
        toth += s_high[v];
    }
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;
    for (int b0 = c0; b0 < c1; b0 += 64 * kScanU) {
        bool op[kScanU];
        uint32_t id[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int k = b0 + 64 * u + lane;
            id[u] = 0;
            op[u] = k < c1 && opens(k, id[u]);
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int k = b0 + 64 * u + lane;
            const bool l1 = op[u] && (id[u] >> kLevelShift) == 1u;
            const bool hi = op[u] && (id[u] >> kLevelShift) > 1u;
            const unsigned long long m1 = __ballot(l1);
            const unsigned long long mh = __ballot(hi);
            if (l1) {
                const int64_t pos = sel0 + pre1 + __popcll(m1 & below);
                if (pos < a.sel_cap) selw[pos] = static_cast<int32_t>(id[u] & kIndexMask);
            }
            if (hi) {
                const int i = position(k);
                opened_pos[preh + __popcll(mh & below)] = i;
                atomicOr(&om[i], bit);
            }
            pre1 += __popcll(m1);
            preh += __popcll(mh);
        }
    }
    if (tid == 0) {
        st->scored[t] = cnt;
        st->opened[t] = static_cast<int32_t>(tot_open);
        st->flags |= path;
        if (!forced) st->unforced += cnt;
        st->sel_n = static_cast<int32_t>(sel0 + tot1);
        st->steps = t + 1;
        a.u_next[w] = static_cast<int32_t>(toth);
    }
}


// An open mask: set by atomics, so read past L1 (a kernel that cuts and
// expands in one workgroup may hold a stale line of it there).
__device__ __forceinline__ uint32_t load_mask(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups that build one pair's next list: one per kExpMin entries of
// its current list, at most kExpSlices.
__device__ __forceinline__ int expand_slices(int n_u) {
    const int ns = n_u / kExpMin;
    return ns < 1 ? 1 : (ns > kExpSlices ? kExpSlices : ns);
}

// Step t, workgroup s of pair p, after every head's cut: the list entries
// any head opened get their rank (in list order) and the next list is their
// children, rank by rank.  Workgroup s takes one slice of the list: it
// counts the opened entries before its slice (its first rank), ranks its
// own, writes their children and, when some head's next cut needs scores,
// appends them to the flat scoring list of step t+1; it also clears the
// next step's open masks at those positions (the masks alternate between
// two buffers, as the list lengths do, so no slice reads what another
// clears).  The last slice sees the whole list: it records the next length
// and finishes the walks after the last step.
template <int R>
__device__ __forceinline__ void expand_slice(const SearchArgs &a, int t, int p, int s, ExpandShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cap = a.cand_cap, c = a.chunk, log2c = a.log2c;
    const int cur = t & 1, nxt = cur ^ 1;
    const int n_u = a.u_n[2 * p + cur];
    // at the last level every candidate is a level-1 node: nothing was
    // marked for opening, only the walks are finished
    const bool final_step = (t + 1 >= a.levels) || (t + 1 >= ZHA_MAX_STEPS);
    const int ns = final_step ? 1 : expand_slices(n_u);
    if (s >= ns) return;
    const bool keeper = s == ns - 1;
    if (n_u <= 0) {                                // finished at an earlier step
        if (keeper && tid == 0) a.u_n[2 * p + nxt] = 0;
        return;
    }
    const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + cur) * cap;
    uint32_t *nids = a.u_ids + (static_cast<int64_t>(p) * 2 + nxt) * cap;
    const uint32_t *om = a.u_omask + (static_cast<int64_t>(p) * 2 + cur) * cap;
    uint32_t *om_next = a.u_omask + (static_cast<int64_t>(p) * 2 + nxt) * cap;
    int32_t *rank = a.u_rank + static_cast<int64_t>(p) * cap;
    uint32_t *par = a.u_par + static_cast<int64_t>(p) * cap;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    const int per = ((n_u + ns - 1) / ns + 63) / 64 * 64;
    const int i0 = final_step ? 0 : min(n_u, s * per);
    const int i1 = final_step ? 0 : min(n_u, i0 + per);
    // opened entries before the slice
    uint32_t cb = 0;
    for (int j0 = tid; j0 < i0; j0 += kScanU * kThreads) {
        uint32_t mv[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int i = j0 + u * kThreads;
            mv[u] = i < i0 ? load_mask(om + i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) cb += mv[u] != 0u;
    }
    // ... and in each wavefront's segment of it
    const int seg = ((i1 - i0 + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int s0 = min(i1, i0 + wave * seg), s1 = min(i1, s0 + seg);
    uint32_t mine = 0;
    for (int base = s0; base < s1; base += 64 * kScanU) {
        uint32_t mv[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int i = base + 64 * u + lane;
            mv[u] = i < s1 ? load_mask(om + i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) mine += __popcll(__ballot(mv[u] != 0u));
    }
    cb = wave_total_u32(cb);
    if (lane == 0) {
        sh.seg_cnt[wave] = mine;
        sh.pre_cnt[wave] = cb;
    }
    __syncthreads();
    uint32_t k0 = 0, before = 0, km = 0;
    for (int v = 0; v < kWaves; ++v) {
        k0 += sh.pre_cnt[v];
        if (v < wave) before += sh.seg_cnt[v];
        km += sh.seg_cnt[v];
    }
    before += k0;
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const bool emit = i < s1 && load_mask(om + i) != 0u;
        const unsigned long long bal = __ballot(emit);
        if (emit) {
            const uint32_t k = before + __popcll(bal & below);
            rank[i] = static_cast<int32_t>(k);
            par[k] = ids[i];
        }
        before += __popcll(bal);
    }
    // this slice's children: ranks k0 .. k0+km-1, positions (k0 + r) * c + e
    const int64_t total = static_cast<int64_t>(k0) + km;   // the whole list's (last slice only)
    const int64_t x0 = static_cast<int64_t>(k0) * c;
    const int64_t x1 = min(static_cast<int64_t>(k0 + km) * c, static_cast<int64_t>(cap));
    const int cnt = x1 > x0 ? static_cast<int>(x1 - x0) : 0;
    if (tid == 0) {
        bool need = false;
        for (int hh = 0; hh < a.group && !final_step && cnt > 0; ++hh) {
            const int64_t nh = static_cast<int64_t>(a.u_next[head_walk(a, p, hh)]) * c;
            if (nh > 0 && !step_forced(a, t + 1, static_cast<int>(nh < cap ? nh : cap))) need = true;
        }
        sh.need = need ? 1 : 0;
        sh.flat_base = need ? atomicAdd(&a.tile_count[t + 1], round_flat(cnt)) : 0;
    }
    __syncthreads();                               // par[] and the flat base are ready
    if (!final_step && cnt > 0) {
        const bool need = sh.need != 0;
        const int fbase = sh.flat_base;
        int4 *flat = a.u_flat + ((t + 1) & 1) * a.flat_cap;
        const int padded = need ? round_flat(cnt) : cnt;
        for (int x = tid; x < padded; x += kThreads) {
            const int64_t xr = x0 + (x < cnt ? x : 0);
            const uint32_t pid = par[xr >> log2c];
            const uint32_t lvl = pid >> kLevelShift, j = pid & kIndexMask;
            const uint32_t child = ((lvl - 1u) << kLevelShift) | (j * static_cast<uint32_t>(c) + (xr & (c - 1)));
            if (x < cnt) {
                nids[xr] = child;
                om_next[xr] = 0u;
            }
            if (need) flat[fbase + x] = make_int4(p, x < cnt ? static_cast<int>(xr) : -1, static_cast<int>(child), 0);
        }
    }
    if (!keeper) return;
    int64_t n_next = total * c;
    const bool overflow = n_next > cap;
    if (overflow) n_next = cap;
    const bool last = (n_next == 0) || final_step;
    if (tid == 0) a.u_n[2 * p + nxt] = last ? 0 : static_cast<int32_t>(n_next);
    if (tid < a.group) {
        const int w = head_walk(a, p, tid);
        WalkState *st = a.state + w;
        if (overflow) st->flags |= ZHA_FLAG_CAND_OVERFLOW;
        if (last) {
            st->n = 0;                             // finished: later level-synchronous steps skip it
            finish_walk<R>(a, w, st->steps, st->scored, st->opened, st->sel_n, st->unforced, st->flags);
        }
    }
}

// Step t, one workgroup per walk: the head's cut (cut_head), and, when the
// level-synchronous engine takes the next step, the hand-over (to_ls_walk:
// it needs only what this walk's cut wrote).
template <int R>
__global__ __launch_bounds__(kThreads) void k_un_cut(SearchArgs a, int t, int handover) {
    __shared__ SelectShared sh;
    __shared__ uint32_t s_one[kWaves], s_high[kWaves];
    __shared__ float s_sc[kLdsCand];
    __shared__ int32_t s_par[kLdsPar];
    __shared__ uint32_t s_pid[kLdsPar];
    // a pair's heads on one XCD: they read the same rows of the pair's score
    // table, which that XCD's L2 then fetches once
    const int w = static_cast<int>(xcd_item(blockIdx.x, static_cast<int64_t>(a.pairs) * a.group));
    if (w < 0) return;
    if (a.u_n[2 * (w / a.group) + (t & 1)] <= 0) return;   // the pair has finished (all its heads)
    cut_head<R>(a, t, w, sh, s_one, s_high, s_sc, s_par, s_pid);
    if (handover) {
        __syncthreads();                           // this walk's opened positions and count are written
        to_ls_walk<R>(a, t, w);
    }
}

// Step t, kExpSlices workgroups per pair, after every head's cut (a kernel
// boundary: a device-wide fence inside one kernel costs far more on this
// GPU, whose L2 caches are per XCD): the pair's next list (expand_slice).
template <int R>
__global__ __launch_bounds__(kThreads) void k_un_expand(SearchArgs a, int t) {
    __shared__ ExpandShared sh;
    expand_slice<R>(a, t, blockIdx.x / kExpSlices, blockIdx.x % kExpSlices, sh);
}

// The first `steps` steps of every pair in one launch, one workgroup per
// pair, in LDS.  The host bounds the candidates of each of these steps to
// kSmallList per pair: every node a walk of the pair could meet at step s is
// a depth-s descendant of a root (D_s), and D_0 .. D_{steps-1} are few.  The
// workgroup enumerates them, scores them all for every head in one pass of
// record loads (matrix tiles, as the grid-wide scorer), then runs each step's
// cut per head on one wavefront (the candidates are the children of the
// entries the head opened, in order; lane_tau's cut key)
// from LDS, and builds no list in memory until the last step: there it
// writes what the grid-wide kernels take over -- the next union list (the
// children of the entries any head opened, in order), its cleared open masks
// and flat scoring entries, the ranks of the opened entries, each head's
// opened positions and count, and the walk states.  Entries of D_s that no
// head reaches are scored but never read.
struct TopShared {
    uint32_t id[kTopNodes];               // D_0, D_1, .. concatenated
    int16_t cbase[kTopNodes];             // index in D_{s+1} of an entry's first child (-1: level 1)
    float sc[kTopNodes][16];              // scores, [entry][head]
    int32_t doff[ZHA_MAX_STEPS + 2];      // D_s = entries doff[s] .. doff[s+1]-1
    uint8_t open[2][16][kSmallList];      // a head's opened entries (index in D_s), by step parity
    int32_t nopen[16];
    uint32_t mask[kSmallList];            // heads that opened each entry of D_s
    uint8_t ord[kSmallList];              // the entry of each rank among the opened ones
    int32_t scored[16][ZHA_MAX_STEPS], opened[16][ZHA_MAX_STEPS];
    int32_t unforced[16], sel_n[16], steps[16];
    uint32_t flags[16];
    int32_t active[16];
    int32_t need;
};

template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kThreads) void k_un_small(SearchArgs a, int steps) {
    constexpr int WB = (16 / R) * kUG;    // nodes per scoring block
    const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cap = a.cand_cap, c = a.chunk, log2c = a.log2c, G = a.group;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    __shared__ LevelTables tb;
    __shared__ TopShared T;
    load_tables(a, tb);
    const int n0 = a.u_n[2 * p];                   // the roots (k_un_init)
    if (n0 <= 0) return;                           // empty tree: k_un_init finished the walks (uniform)
    const uint32_t *ids0 = a.u_ids + static_cast<int64_t>(p) * 2 * cap;
    for (int i = tid; i < n0; i += kThreads) T.id[i] = ids0[i];
    if (tid == 0) {
        T.doff[0] = 0;
        T.doff[1] = n0;
    }
    if (tid < G) {
        const WalkState &st = a.state[head_walk(a, p, tid)];
        for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
            T.scored[tid][i] = st.scored[i];
            T.opened[tid][i] = st.opened[i];
        }
        T.unforced[tid] = st.unforced;
        T.sel_n[tid] = st.sel_n;
        T.steps[tid] = st.steps;
        T.flags[tid] = st.flags;
        T.active[tid] = 1;
        T.nopen[tid] = 0;
    }
    __syncthreads();
    // D_{s+1}: the children of D_s's entries above level 1, in order (one
    // wavefront; D_s holds at most 64 entries, one per lane)
    for (int s = 0; s + 1 < steps; ++s) {
        if (wave == 0) {
            const int b = T.doff[s], e = T.doff[s + 1];
            const int i = b + lane;
            uint32_t id = 0;
            bool par = false;
            if (i < e) {
                id = T.id[i];
                par = (id >> kLevelShift) > 1u;
            }
            const unsigned long long bal = __ballot(par);
            const int k = __popcll(bal & below);
            if (i < e) T.cbase[i] = static_cast<int16_t>(par ? k * c : -1);
            if (par) {
                const uint32_t lvl = id >> kLevelShift, j = id & kIndexMask;
                for (int ch = 0; ch < c; ++ch)
                    T.id[e + k * c + ch] = ((lvl - 1u) << kLevelShift) | (j * static_cast<uint32_t>(c) + ch);
            }
            if (lane == 0) T.doff[s + 2] = e + __popcll(bal) * c;
        }
        __syncthreads();
    }
    // every entry of D_0 .. D_{steps-1}, scored for every head
    {
        const int ntot = T.doff[steps];
        const int nb = (ntot + WB - 1) / WB;
        const int per = (nb + kWaves - 1) / kWaves;
        const int b0 = wave * per, b1 = min(nb, b0 + per);
        auto entry = [&](int e) -> int4 {
            const int pos = e < ntot ? e : ntot - 1;
            return make_int4(p, e < ntot ? e : -1, static_cast<int>(T.id[pos]), 0);
        };
        auto out = [&](int, int pos, uint32_t, int grp, const float (&v)[4]) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * grp + e < G) T.sc[pos][4 * grp + e] = v[e];
        };
        score_run<D, R, QT, ST>(a, tb, entry, b0, b1, out);
    }
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int b = T.doff[s], cur = s & 1;
        // some head's cut needs scores (the nodes of the step are then
        // marked visited, as the grid-wide scorer marks its lists)
        if (tid == 0) T.need = 0;
        for (int i = tid; i < kSmallList; i += kThreads) T.mask[i] = 0u;
        __syncthreads();
        if (tid < G && T.active[tid]) {
            const int cnt = (s == 0) ? n0 : T.nopen[tid] * c;
            if (!step_forced(a, s, cnt)) T.need = 1;
        }
        __syncthreads();
        for (int h = wave; h < G; h += kWaves) {
            if (!T.active[h]) continue;            // opened nothing at an earlier step
            const int w = head_walk(a, p, h);
            const int cnt = (s == 0) ? n0 : T.nopen[h] * c;
            // candidate x: entry `pos` of D_s
            int pos = 0;
            if (lane < cnt)
                pos = (s == 0) ? lane : T.cbase[T.doff[s - 1] + T.open[cur ^ 1][h][lane >> log2c]] + (lane & (c - 1));
            const bool in = lane < cnt;
            const uint32_t id = in ? T.id[b + pos] : 0u;
            const float v = in ? T.sc[b + pos][h] : -INFINITY;
            if (a.visited && T.need && in) {
                const int64_t bitn = a.node_off[id >> kLevelShift] + (id & kIndexMask);
                atomicOr(a.visited + static_cast<int64_t>(p) * a.vis_words + (bitn >> 5), 1u << (bitn & 31));
            }
            const bool forced = step_forced(a, s, cnt);
            unsigned long long tau = 0;
            if (!forced) tau = lane_tau(a, in, v, id, wave_max(in ? v : -INFINITY, 1, 64), cnt, a.k[s]);
            // open, in candidate order
            const bool op = in && (forced || rank_key(v, id, log2c) >= tau);
            const bool l1 = op && (id >> kLevelShift) == 1u;
            const bool hi = op && (id >> kLevelShift) > 1u;
            const unsigned long long m1 = __ballot(l1), mh = __ballot(hi);
            const int sel0 = T.sel_n[h];
            if (l1) {
                const int64_t at = static_cast<int64_t>(sel0) + __popcll(m1 & below);
                if (at < a.sel_cap) a.sel_blocks[static_cast<int64_t>(w) * a.sel_cap + at] = static_cast<int32_t>(id & kIndexMask);
            }
            if (hi) {
                T.open[cur][h][__popcll(mh & below)] = static_cast<uint8_t>(pos);
                atomicOr(&T.mask[pos], 1u << h);
            }
            const int nopen = __popcll(__ballot(op));
            if (lane == 0) {
                T.scored[h][s] = cnt;
                T.opened[h][s] = nopen;
                if (!forced) T.unforced[h] += cnt;
                T.sel_n[h] = sel0 + __popcll(m1);
                T.steps[h] = s + 1;
                T.nopen[h] = __popcll(mh);
                T.active[h] = __popcll(mh) > 0;
            }
        }
        __syncthreads();
        // the union of the opened entries, ranked in order (one wavefront)
        const int nd = T.doff[s + 1] - b;
        __shared__ int32_t s_total;
        if (wave == 0) {
            const bool o = lane < nd && T.mask[lane] != 0u;
            const unsigned long long bal = __ballot(o);
            if (s + 1 == steps && o) {
                const int k = __popcll(bal & below);
                a.u_rank[static_cast<int64_t>(p) * cap + lane] = k;
                a.u_par[static_cast<int64_t>(p) * cap + k] = T.id[b + lane];
                T.ord[k] = static_cast<uint8_t>(lane);
            }
            if (lane == 0) s_total = __popcll(bal);
        }
        __syncthreads();
        const int total = s_total;
        int64_t n_next = static_cast<int64_t>(total) * c;
        const bool overflow = n_next > cap;
        if (overflow) n_next = cap;
        const bool last = (n_next == 0) || (s + 1 >= a.levels) || (s + 1 >= ZHA_MAX_STEPS);
        if (!last && s + 1 < steps) continue;      // uniform: the next step runs from LDS
        // hand-over (or the end of the pair's walks)
        const int nxt = (s + 1) & 1;
        if (!last) {
            uint32_t *nids = a.u_ids + (static_cast<int64_t>(p) * 2 + nxt) * cap;
            uint32_t *om_next = a.u_omask + (static_cast<int64_t>(p) * 2 + nxt) * cap;
            __shared__ int32_t s_need, s_base;
            if (tid == 0) {
                bool need = false;
                for (int h = 0; h < G; ++h) {
                    const int64_t nh = static_cast<int64_t>(T.nopen[h]) * c;
                    if (nh > 0 && !step_forced(a, s + 1, static_cast<int>(nh < cap ? nh : cap))) need = true;
                }
                s_need = need ? 1 : 0;
                s_base = need ? atomicAdd(&a.tile_count[s + 1], round_flat(static_cast<int>(n_next))) : 0;
            }
            __syncthreads();
            const int cnt = static_cast<int>(n_next);
            const int padded = s_need ? round_flat(cnt) : cnt;
            int4 *flat = a.u_flat + static_cast<int64_t>((s + 1) & 1) * a.flat_cap;
            // ranked entry k is the k-th set entry of the mask
            for (int x = tid; x < padded; x += kThreads) {
                const int xr = x < cnt ? x : 0;
                const uint32_t pid = T.id[b + T.ord[xr >> log2c]];   // the opened entry of rank xr / c
                const uint32_t lvl = pid >> kLevelShift, j = pid & kIndexMask;
                const uint32_t child = ((lvl - 1u) << kLevelShift) | (j * static_cast<uint32_t>(c) + (xr & (c - 1)));
                if (x < cnt) {
                    nids[x] = child;
                    om_next[x] = 0u;
                }
                if (s_need) flat[s_base + x] = make_int4(p, x < cnt ? x : -1, static_cast<int>(child), 0);
            }
        }
        if (tid == 0) {
            a.u_n[2 * p + nxt] = last ? 0 : static_cast<int32_t>(n_next);
            a.u_n[2 * p + (nxt ^ 1)] = last ? 0 : nd;
        }
        if (tid < G) {
            const int h = tid, w = head_walk(a, p, h);
            WalkState *st = a.state + w;
            for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
                st->scored[i] = T.scored[h][i];
                st->opened[i] = T.opened[h][i];
            }
            const uint32_t fl = T.flags[h] | (overflow ? ZHA_FLAG_CAND_OVERFLOW : 0u);
            st->unforced = T.unforced[h];
            st->sel_n = T.sel_n[h];
            st->steps = T.steps[h];
            st->flags = fl;
            a.u_next[w] = T.nopen[h];
            if (last) {
                st->n = 0;
                finish_walk<R>(a, w, T.steps[h], T.scored[h], T.opened[h], T.sel_n[h], T.unforced[h], fl);
            }
        }
        // each head's opened entries of D_s, as list positions for the next cut
        for (int i = tid; i < G * kSmallList; i += kThreads) {
            const int h = i / kSmallList, k = i - h * kSmallList;
            if (!last && k < T.nopen[h])
                a.u_open[static_cast<int64_t>(head_walk(a, p, h)) * cap + k] = T.open[s & 1][h][k];
        }
        return;
    }
}

// Hand-over to the level-synchronous engine after the union cut of step t,
// run by walk w's cut workgroup once its cut is done: the walk's candidates
// of step t+1 -- the children of the list entries it opened, in order,
// exactly the list that engine's own cut would have written -- become that
// engine's candidate list; the walk state is set (finished if nothing
// remains) and the scoring tiles registered.
template <int R>
__device__ __forceinline__ void to_ls_walk(const SearchArgs &a, int t, int w) {
    const int tid = threadIdx.x;
    const int p = w / a.group;
    const int cap = a.cand_cap, c = a.chunk, log2c = a.log2c;
    if (a.u_n[2 * p + (t & 1)] <= 0) return;      // the pair finished earlier; so did its walks
    __shared__ WalkState st;
    __shared__ int s_base;
    if (tid == 0) st = a.state[w];
    const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + (t & 1)) * cap;
    const int32_t *opened_pos = a.u_open + static_cast<int64_t>(w) * cap;
    int64_t nn = static_cast<int64_t>(a.u_next[w]) * c;
    const bool overflow = nn > cap;
    if (overflow) nn = cap;
    uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * cap;     // buffer 0
    for (int64_t x = tid; x < nn; x += kThreads) {
        const uint32_t pid = ids[opened_pos[x >> log2c]];
        const uint32_t lvl = pid >> kLevelShift, j = pid & kIndexMask;
        cur[x] = ((lvl - 1u) << kLevelShift) | (j * static_cast<uint32_t>(c) + static_cast<uint32_t>(x & (c - 1)));
    }
    __syncthreads();
    if (tid == 0) {
        if (overflow) st.flags |= ZHA_FLAG_CAND_OVERFLOW;
        st.buf = 0;
        st.n = static_cast<int32_t>(nn);
        if (st.n == 0 || t + 1 >= a.levels || t + 1 >= ZHA_MAX_STEPS) {
            st.n = 0;
            finish_walk<R>(a, w, st.steps, st.scored, st.opened, st.sel_n, st.unforced, st.flags);
        }
        a.state[w] = st;
        s_base = 0;
        if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t + 1, st.n))
            s_base = atomicAdd(&a.tile_count[t + 1], (st.n + kTile - 1) / kTile);
    }
    __syncthreads();
    if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t + 1, st.n)) {
        const int ntile = (st.n + kTile - 1) / kTile;
        for (int k = tid; k < ntile; k += kThreads) a.tile_map[s_base + k] = make_int2(w, k * kTile);
    }
}

// Workgroups of the scorer that fit on the device at once (its wavefronts
// take equal runs of blocks, so all of them should be resident), per device.
template <typename K>
static int resident_grid(K kernel, int threads) {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cache[dev] = cus * per_cu;
    }
    return cache[dev];
}

template <int D, int R, typename QT, typename ST>
static hipError_t launch_union_t(const SearchArgs &a, int n0, hipStream_t st) {
    hipLaunchKernelGGL((k_un_init<R>), dim3(a.pairs), dim3(512), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int score_grid = resident_grid(k_un_score<D, R, QT, ST>, kScoreThreads);
    const int t0 = a.small_steps;
    if (t0 > 0) {
        hipLaunchKernelGGL((k_un_small<D, R, QT, ST>), dim3(a.pairs), dim3(kThreads), 0, st, a, t0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int t1 = a.ls_from > 0 ? a.ls_from : a.levels;   // union steps: t0 .. t1-1
    for (int t = t0; t < t1 && t < ZHA_MAX_STEPS; ++t) {
        const bool skip = (t == 0) && (n0 <= 1 || (a.mode == ZHA_TOPK && a.k[0] >= n0) ||
                                       (a.mode == ZHA_TOPP && a.p >= 1.0f));
        if (!skip) {
            hipLaunchKernelGGL((k_un_score<D, R, QT, ST>), dim3(score_grid), dim3(kScoreThreads), 0, st, a, t,
                               n0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const int handover = (t + 1 == a.ls_from) ? 1 : 0;
        hipLaunchKernelGGL((k_un_cut<R>), dim3(static_cast<unsigned>(xcd_grid(int64_t(a.pairs) * a.group))),
                           dim3(kThreads), 0, st, a, t, handover);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (!handover) {
            hipLaunchKernelGGL((k_un_expand<R>), dim3(a.pairs * kExpSlices), dim3(kThreads), 0, st, a, t);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (a.ls_from > 0)
        return launch_ls_from(a, D, R, sizeof(QT) == 2 ? ZHA_BF16 : ZHA_F32, sizeof(ST) == 2 ? ZHA_BF16 : ZHA_F32,
                              a.ls_from, st);
    return hipSuccess;
}

template <int D, typename QT, typename ST>
static hipError_t launch_union_d(const SearchArgs &a, int R, int n0, hipStream_t st) {
    switch (R) {
        case 1: return launch_union_t<D, 1, QT, ST>(a, n0, st);
        case 2: return launch_union_t<D, 2, QT, ST>(a, n0, st);
        case 4: return launch_union_t<D, 4, QT, ST>(a, n0, st);
        case 8: return launch_union_t<D, 8, QT, ST>(a, n0, st);
        case 16: return launch_union_t<D, 16, QT, ST>(a, n0, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, typename QT>
static hipError_t launch_union_s(const SearchArgs &a, int R, int sdtype, int n0, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_union_d<D, QT, bf16_t>(a, R, n0, st) : launch_union_d<D, QT, float>(a, R, n0, st);
}

hipError_t launch_union(const SearchArgs &a, int D, int R, int dtype, int sdtype, int n0, hipStream_t st) {
    if (a.pairs <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_union_s<64, bf16_t>(a, R, sdtype, n0, st)
                                 : launch_union_s<64, float>(a, R, sdtype, n0, st);
    return dtype == ZHA_BF16 ? launch_union_s<128, bf16_t>(a, R, sdtype, n0, st)
                             : launch_union_s<128, float>(a, R, sdtype, n0, st);
}

}  // namespace zha
