// zha_union.hip -- the union search engine: one candidate list per
// (sequence, KV head) pair, shared by the pair's query heads.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "Common misunderstandings": each attention head walks the tree
// on its own -- here every head still gets its own scores and its own cut
// ("How does top-p differ from top-K?") over exactly its own candidates
// ("Run a small tree yourself").  What the heads of a group share is the
// tree, so they share the reads: at step t the pair's list holds the union
// of the heads' candidate sets, each node tagged with the mask of heads it
// is a candidate for.  Children of an opened node inherit the mask of the
// heads that opened it, which is exactly the set of heads whose next
// candidates they are.
//
// Per step:
//   k_un_score  grid-wide over 32-node tiles of every pair's list: a node
//               record is read once and scored for all heads of the group
//               with fp32 16x16x4 matrix-core tiles (heads x (node, ref)),
//               then s * dot + bias and the max over references;
//   k_un_cut    one workgroup per walk: the head's exact radix-select cut
//               over the list entries carrying its bit, its level-1
//               selections in span order, its bit on the higher nodes it opens;
//   k_un_expand one workgroup per pair: the next union list (children of the
//               nodes any head opened, tagged with those heads).
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kCutThreads = 1024;     // workgroup of the expand kernel
constexpr int kCutWaves = kCutThreads / 64;
constexpr int kScoreThreads = 256;
constexpr int kUG = 2;                // node groups in flight per wavefront

__device__ __forceinline__ int head_walk(const SearchArgs &a, int pair, int h) {
    const int b = pair / a.kv_heads, g = pair % a.kv_heads;
    return b * a.heads + g * a.group + h;
}

struct ExpandShared {
    uint32_t seg_cnt[kCutWaves];
    int32_t tile_base, tile_n;
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
    uint32_t *mask = a.u_mask + static_cast<int64_t>(p) * 2 * cap;
    const int n = write_roots(a, ids, flags);
    const uint32_t all = (a.group >= 32) ? 0xffffffffu : ((1u << a.group) - 1u);
    uint32_t *om = a.u_omask + static_cast<int64_t>(p) * cap;
    for (int i = tid; i < n; i += blockDim.x) {
        mask[i] = all;
        om[i] = 0;
    }
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
        if (n == 0) finish_walk<R>(a, w, 0, st->scored, st->opened, 0, 0, s_flags);
    }
}

// Step t scoring of every pair's union list: a wavefront takes NPG = 16/R
// nodes at a time (the 16 columns of a matrix-core tile are (node, ref)),
// the rows are the group's heads.  Matrix step k of lane group q = lane/16
// multiplies element d = 16*(k/4) + 4*q + k%4 of the query and of the
// reference row (one permutation of D for both operands), so one 16-byte
// load of the four lanes of a column reads 64 contiguous bytes of its row.
template <int D, int R, typename QT>
__global__ __launch_bounds__(kScoreThreads) void k_un_score(SearchArgs a, int t, int tiles0) {
    constexpr int NPG = 16 / R;           // nodes per tile
    constexpr int KS = D / 4;             // 16x16x4 steps
    constexpr int kSW = kScoreThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int n_tiles = (t == 0) ? a.pairs * tiles0 : a.tile_count[t];
    const float s = a.sharpness;
    // each workgroup takes one contiguous run of tiles, so consecutive tiles
    // mostly belong to the same pair and keep the query operand
    const int per = (n_tiles + gridDim.x - 1) / gridDim.x;
    const int tile0 = blockIdx.x * per;
    const int tile1 = min(n_tiles, tile0 + per);
    int cur_pair = -1;
    float qa[KS];
    for (int tile = tile0; tile < tile1; ++tile) {
        int p, start;
        if (t == 0) {
            p = tile / tiles0;
            start = (tile % tiles0) * kTile;
        } else {
            const int2 e = a.tile_map[tile];
            p = e.x;
            start = e.y;
        }
        const int n_u = a.u_n[2 * p];
        const int buf = a.u_n[2 * p + 1];
        const int end = min(n_u, start + kTile);
        const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + buf) * a.cand_cap;
        // query operand: row = head `col` of the pair's group (zero past G)
        if (p != cur_pair) {
            cur_pair = p;
            const bool ok = col < a.group;
            const int w = head_walk(a, p, ok ? col : 0);
            const QT *qp = static_cast<const QT *>(a.q) + static_cast<int64_t>(w) * D + 4 * grp;
#pragma unroll
            for (int k = 0; k < KS; ++k) qa[k] = ok ? Elem<QT>::load(qp, 16 * (k / 4) + (k % 4)) : 0.f;
        }
        for (int g0 = start + wave * NPG; g0 < end; g0 += kSW * NPG * kUG) {
            float kb[kUG][KS];
            float bias[kUG];
            int node_i[kUG];
#pragma unroll
            for (int u = 0; u < kUG; ++u) {
                const int i = g0 + u * kSW * NPG + col / R;
                node_i[u] = i;
                const int ic = i < end ? i : end - 1;
                const uint32_t id = ids[ic];
                const int lvl = static_cast<int>(id >> kLevelShift);
                const int64_t node = static_cast<int64_t>(p) * a.cap[lvl] + (id & kIndexMask);
                const float *kp = a.kap[lvl] + node * (R * D) + (col % R) * D + 4 * grp;
#pragma unroll
                for (int k = 0; k < KS; k += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(kp + 4 * k);
                    kb[u][k] = v.x; kb[u][k + 1] = v.y; kb[u][k + 2] = v.z; kb[u][k + 3] = v.w;
                }
                bias[u] = a.bet[lvl][node * R + (col % R)];
            }
#pragma unroll
            for (int u = 0; u < kUG; ++u) {
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KS; ++k)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[k], kb[u][k], acc, 0, 0, 0);
                const int i = node_i[u];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = fmaf(s, acc[e], bias[u]);
                    v = group_max<R>(v);
                    if (v != v) v = -INFINITY;
                    if (v == 0.f) v = 0.f;
                    const int h = 4 * grp + e;
                    if ((col % R) == 0 && i < end && h < a.group)
                        a.u_score[(static_cast<int64_t>(p) * a.group + h) * a.cand_cap + i] = v;
                }
                if (a.visited && (col % R) == 0 && grp == 0 && i < end) {
                    const uint32_t id = ids[i];
                    const int64_t bitn = a.node_off[id >> kLevelShift] + (id & kIndexMask);
                    atomicOr(a.visited + p * a.vis_words + (bitn >> 5), 1u << (bitn & 31));
                }
            }
        }
    }
}

// Step t, one workgroup per walk (head h of pair p): the entries of the
// pair's list that carry bit h are compacted (in list order) into the
// walk's own (id, score, list index) arrays; the head's exact cut then runs
// over those alone, its level-1 selections go out in span order, and bit h
// is set on every higher node it opens.
template <int R>
__global__ __launch_bounds__(kThreads) void k_un_cut(SearchArgs a, int t) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x;
    const int p = w / a.group, h = w % a.group;
    const uint32_t bit = 1u << h;
    const int cap = a.cand_cap, log2c = a.log2c;
    __shared__ SelectShared sh;
    __shared__ uint32_t s_seg[kWaves];
    const int n_u = a.u_n[2 * p];
    const int buf = a.u_n[2 * p + 1];
    if (n_u <= 0) return;                          // the pair has finished (uniform)
    const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + buf) * cap;
    const uint32_t *mask = a.u_mask + (static_cast<int64_t>(p) * 2 + buf) * cap;
    const float *sc = a.u_score + (static_cast<int64_t>(p) * a.group + h) * cap;
    uint32_t *om = a.u_omask + static_cast<int64_t>(p) * cap;
    uint32_t *cid = a.cand + static_cast<int64_t>(w) * 2 * cap;     // this head's candidates
    uint32_t *cux = cid + cap;                                       // their list positions
    float *csc = a.h_score + static_cast<int64_t>(w) * cap;         // their scores
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // compaction: wavefront v owns list segment v, 64*kScanU entries a round
    const int seg = ((n_u + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int s0 = wave * seg, s1 = min(n_u, s0 + seg);
    uint32_t mine = 0;
    for (int b0 = s0; b0 < s1; b0 += 64 * kScanU) {
        uint32_t mv[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int i = b0 + 64 * u + lane;
            mv[u] = i < s1 ? mask[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) mine += __popcll(__ballot((mv[u] & bit) != 0u));
    }
    if (lane == 0) s_seg[wave] = mine;
    __syncthreads();
    uint32_t before = 0, cnt_u = 0;
    for (int v = 0; v < kWaves; ++v) {
        if (v < wave) before += s_seg[v];
        cnt_u += s_seg[v];
    }
    const int cnt = static_cast<int>(cnt_u);
    const bool forced = step_forced(a, t, cnt);
    float m = -INFINITY;
    for (int b0 = s0; b0 < s1; b0 += 64 * kScanU) {
        uint32_t mv[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int i = b0 + 64 * u + lane;
            mv[u] = i < s1 ? mask[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int i = b0 + 64 * u + lane;
            const bool in = (mv[u] & bit) != 0u;
            const unsigned long long bal = __ballot(in);
            if (in) {
                const uint32_t k = before + __popcll(bal & below);
                cid[k] = ids[i];
                cux[k] = static_cast<uint32_t>(i);
                if (!forced) {
                    const float v = sc[i];
                    csc[k] = v;
                    m = fmaxf(m, v);
                }
            }
            before += __popcll(bal);
        }
    }
    __syncthreads();
    if (cnt == 0) {
        if (tid == 0) a.u_next[w] = 0;
        return;
    }
    unsigned long long tau = 0;
    if (!forced) {
        const float mx = block_max(m, sh);
        tau = cut_tau(a, cnt, cid, csc, mx, a.k[t], sh);
    }

    // open, in list order over the compact arrays
    const int seg2 = ((cnt + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int c0 = wave * seg2, c1 = min(cnt, c0 + seg2);
    uint32_t n1 = 0, nopen = 0, nhigh = 0;
    for (int base = c0; base < c1; base += 64) {
        const int k = base + lane;
        bool open = false;
        uint32_t id = 0;
        if (k < c1) {
            id = cid[k];
            open = forced || rank_key(csc[k], id, log2c) >= tau;
        }
        n1 += __popcll(__ballot(open && (id >> kLevelShift) == 1u));
        nopen += __popcll(__ballot(open));
        nhigh += __popcll(__ballot(open && (id >> kLevelShift) > 1u));
    }
    if (lane == 0) s_seg[wave] = n1;
    const uint32_t tot_open = block_sum_u32(lane == 0 ? nopen : 0u, sh);
    const uint32_t tot_high = block_sum_u32(lane == 0 ? nhigh : 0u, sh);
    WalkState *st = a.state + w;
    const int64_t sel0 = st->sel_n;
    uint32_t pre = 0, tot1 = 0;
    for (int v = 0; v < kWaves; ++v) {
        if (v < wave) pre += s_seg[v];
        tot1 += s_seg[v];
    }
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;
    for (int base = c0; base < c1; base += 64) {
        const int k = base + lane;
        bool open = false;
        uint32_t id = 0;
        if (k < c1) {
            id = cid[k];
            open = forced || rank_key(csc[k], id, log2c) >= tau;
        }
        const bool l1 = open && (id >> kLevelShift) == 1u;
        const unsigned long long m1 = __ballot(l1);
        if (l1) {
            const int64_t pos = sel0 + pre + __popcll(m1 & below);
            if (pos < a.sel_cap) selw[pos] = static_cast<int32_t>(id & kIndexMask);
        }
        if (open && (id >> kLevelShift) > 1u) atomicOr(&om[cux[k]], bit);
        pre += __popcll(m1);
    }
    if (tid == 0) {
        st->scored[t] = cnt;
        st->opened[t] = static_cast<int32_t>(tot_open);
        if (!forced) st->unforced += cnt;
        st->sel_n = static_cast<int32_t>(sel0 + tot1);
        st->steps = t + 1;
        a.u_next[w] = static_cast<int32_t>(tot_high) * a.chunk;
    }
}

// Step t, one workgroup per pair: the next list holds the children of every
// node some head opened, in span order, each child tagged with the heads
// that opened its parent.
template <int R>
__global__ __launch_bounds__(kCutThreads) void k_un_expand(SearchArgs a, int t) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x;
    const int cap = a.cand_cap, c = a.chunk;
    __shared__ ExpandShared sh;
    const int n_u = a.u_n[2 * p];
    const int buf = a.u_n[2 * p + 1];
    if (n_u <= 0) return;
    const uint32_t *ids = a.u_ids + (static_cast<int64_t>(p) * 2 + buf) * cap;
    uint32_t *nids = a.u_ids + (static_cast<int64_t>(p) * 2 + (buf ^ 1)) * cap;
    uint32_t *nmask = a.u_mask + (static_cast<int64_t>(p) * 2 + (buf ^ 1)) * cap;
    uint32_t *om = a.u_omask + static_cast<int64_t>(p) * cap;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    const int seg = ((n_u + kCutWaves - 1) / kCutWaves + 63) / 64 * 64;
    const int s0 = wave * seg, s1 = min(n_u, s0 + seg);
    uint32_t mine = 0;
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        mine += __popcll(__ballot(i < s1 && om[i] != 0u));
    }
    if (lane == 0) sh.seg_cnt[wave] = mine;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int v = 0; v < kCutWaves; ++v) {
        if (v < wave) before += sh.seg_cnt[v];
        total += sh.seg_cnt[v];
    }
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const uint32_t m = (i < s1) ? om[i] : 0u;
        const bool emit = m != 0u;
        const unsigned long long bal = __ballot(emit);
        if (emit) {
            const int64_t k = before + __popcll(bal & below);
            const uint32_t id = ids[i];
            const uint32_t lvl = id >> kLevelShift, j = id & kIndexMask;
            const uint32_t cid = (lvl - 1u) << kLevelShift;
            for (int e = 0; e < c; ++e) {
                const int64_t pos = k * c + e;
                if (pos < cap) {
                    nids[pos] = cid | (j * static_cast<uint32_t>(c) + e);
                    nmask[pos] = m;
                }
            }
        }
        before += __popcll(bal);
    }
    int64_t n_next = static_cast<int64_t>(total) * c;
    const bool overflow = n_next > cap;
    if (overflow) n_next = cap;
    const bool last = (n_next == 0) || (t + 1 >= a.levels) || (t + 1 >= ZHA_MAX_STEPS);
    __syncthreads();
    // clear the open masks for the next step
    const int64_t clear = (n_next > n_u) ? n_next : n_u;
    for (int64_t i = tid; i < clear; i += kCutThreads) om[i] = 0;
    if (tid == 0) {
        a.u_n[2 * p] = last ? 0 : static_cast<int32_t>(n_next);
        a.u_n[2 * p + 1] = buf ^ 1;
        bool need_scores = false;
        for (int hh = 0; hh < a.group && !last; ++hh) {
            const int nh = a.u_next[p * a.group + hh];
            if (nh > 0 && !step_forced(a, t + 1, nh)) need_scores = true;
        }
        sh.tile_n = 0;
        if (need_scores) {
            sh.tile_n = static_cast<int>((n_next + kTile - 1) / kTile);
            sh.tile_base = atomicAdd(&a.tile_count[t + 1], sh.tile_n);
        }
    }
    __syncthreads();
    for (int k = tid; k < sh.tile_n; k += kCutThreads) a.tile_map[sh.tile_base + k] = make_int2(p, k * kTile);
    if (tid < a.group) {
        const int w = head_walk(a, p, tid);
        WalkState *st = a.state + w;
        if (overflow) st->flags |= ZHA_FLAG_CAND_OVERFLOW;
        if (last) finish_walk<R>(a, w, st->steps, st->scored, st->opened, st->sel_n, st->unforced, st->flags);
    }
}

template <int D, int R, typename QT>
static hipError_t launch_union_t(const SearchArgs &a, int n0, hipStream_t st) {
    hipLaunchKernelGGL((k_un_init<R>), dim3(a.pairs), dim3(512), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles0 = (n0 + kTile - 1) / kTile;
    for (int t = 0; t < a.levels && t < ZHA_MAX_STEPS; ++t) {
        const bool skip = (t == 0) && (n0 <= 1 || (a.mode == ZHA_TOPK && a.k[0] >= n0) ||
                                       (a.mode == ZHA_TOPP && a.p >= 1.0f));
        if (!skip) {
            hipLaunchKernelGGL((k_un_score<D, R, QT>), dim3(a.score_grid), dim3(kScoreThreads), 0, st, a,
                               t, tiles0 > 0 ? tiles0 : 1);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((k_un_cut<R>), dim3(a.pairs * a.group), dim3(kThreads), 0, st, a, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_un_expand<R>), dim3(a.pairs), dim3(kCutThreads), 0, st, a, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, typename QT>
static hipError_t launch_union_d(const SearchArgs &a, int R, int n0, hipStream_t st) {
    switch (R) {
        case 1: return launch_union_t<D, 1, QT>(a, n0, st);
        case 2: return launch_union_t<D, 2, QT>(a, n0, st);
        case 4: return launch_union_t<D, 4, QT>(a, n0, st);
        case 8: return launch_union_t<D, 8, QT>(a, n0, st);
        case 16: return launch_union_t<D, 16, QT>(a, n0, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_union(const SearchArgs &a, int D, int R, int dtype, int n0, hipStream_t st) {
    if (a.pairs <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_union_d<64, bf16_t>(a, R, n0, st)
                                 : launch_union_d<64, float>(a, R, n0, st);
    return dtype == ZHA_BF16 ? launch_union_d<128, bf16_t>(a, R, n0, st)
                             : launch_union_d<128, float>(a, R, n0, st);
}

}  // namespace zha
