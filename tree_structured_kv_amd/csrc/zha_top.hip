// zha_top.hip -- the first steps of decode walks over a densely scored top
// of the tree, handing over to the level-synchronous engine.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "What does a node summarize?": a node's score for query q is
// the largest over references r of s <key_r, q> + bias_r.  "Run a small tree
// yourself": each step scores the candidates, normalises them with one
// softmax over the step's list and opens a prefix ("How does top-p differ
// from top-K?").
//
// GPU design.  The top levels of a tree are small (at 256K keys, chunk 8:
// 1 + 8 + 64 + 512 nodes per (sequence, KV head)) and under top-p almost
// every one of their nodes becomes a candidate of some query head of the
// pair.  So instead of a chain of small dependent launches (score the few
// candidates of a step, cut, expand, repeat), k_top_score scores every node
// of those levels for every query head of its pair in one launch that uses
// the whole GPU (a record is read once for all heads of the group), and
// k_top_cut then runs each walk's first steps -- cut, open, next candidates
// -- from that table without touching a node record, and leaves the walk's
// state, candidate list and scoring tiles for the level-synchronous steps
// below.  A candidate outside the table (a node whose parent chunk has not
// filled yet, and its children) is scored by the cut workgroup itself.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_score.h"
#include "zha_walk.h"

namespace zha {

namespace {

constexpr int kTopThreads = 256;      // k_top_score workgroup
constexpr int kTopU = 4;              // nodes in flight per wavefront

// Score of one candidate for one query, by one wavefront (all lanes get it).
template <int D, int R, typename ST>
__device__ __forceinline__ float score_one(const SearchArgs &a, int64_t pair, const float (&qv)[row_epl<D, ST>()],
                                           uint32_t id, uint32_t &flags) {
    constexpr int EPL = row_epl<D, ST>();
    constexpr int LPR = D / EPL;
    constexpr int RPL = 64 / LPR;
    constexpr int NL = (R + RPL - 1) / RPL;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rsub = lane / LPR;
    const int lvl = static_cast<int>(id >> kLevelShift);
    const int64_t node = pair * a.cap[lvl] + static_cast<int64_t>(id & kIndexMask);
    const ST *kp = reinterpret_cast<const ST *>(a.kap[lvl]) + node * (R * D);
    float best = -INFINITY;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int r = l * RPL + rsub;
        float kv[EPL];
        float b = -INFINITY;
        if (r < R) {
            if constexpr (EPL == 8)
                Vec16<ST>::load(kp + r * D + EPL * sub, kv);
            else
                Vec4<ST>::load(kp + r * D + EPL * sub, kv);
            b = a.bet[lvl][node * R + r];
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) kv[e] = 0.f;
        }
        float d = kv[0] * qv[0];
#pragma unroll
        for (int e = 1; e < EPL; ++e) d = fmaf(kv[e], qv[e], d);
        d = group_sum<LPR>(d);
        best = fmaxf(best, fmaf(a.sharpness, d, b));
    }
    float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 0));
#pragma unroll
    for (int gq = 1; gq < RPL; ++gq)
        m = fmaxf(m, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), gq * LPR)));
    if (m != m) { m = -INFINITY; flags |= ZHA_FLAG_NONFINITE; }
    if (m == 0.f) m = 0.f;
    return m;
}

}  // namespace

// Lane exchange with lane ^ O inside 32-lane groups.
template <int O>
__device__ __forceinline__ float xchg(float v) {
    if constexpr (O == 1)
        return dpp<kDppXor1>(v);
    else if constexpr (O == 2)
        return dpp<kDppXor2>(v);
    else
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (O << 10) | 0x1F));
}

// One level of a transposed sum: slots [0, M/2) keep their value plus the
// partner's slot j + M/2 (which holds the same head there); a single slot
// is summed plainly.
template <int O, int M, int GP>
__device__ __forceinline__ void sum_level(float (&v)[GP]) {
    if constexpr (M >= 2) {
#pragma unroll
        for (int j = 0; j < M / 2; ++j) v[j] += xchg<O>(v[j + M / 2]);
    } else {
        v[0] += xchg<O>(v[0]);
    }
}

// GP per-head partial dot products per lane summed over aligned groups of
// LPR lanes, the groups paired as in group_sum (1, 2, 4, 8, 16 lanes apart,
// so every head's sum is the same tree of additions, bit for bit), but
// with each level moving only half the slots still held: slot j of lane l
// holds head j ^ lane_head(l), and at the end slot 0 holds head lane_head(l).
template <int LPR, int GP>
__device__ __forceinline__ float transposed_sum(float (&v)[GP]) {
    static_assert(GP <= LPR && LPR <= 32, "the heads fit the lanes of a row");
    sum_level<1, GP>(v);
    sum_level<2, (GP >= 2 ? GP / 2 : 1)>(v);
    if constexpr (LPR >= 8) sum_level<4, (GP >= 4 ? GP / 4 : 1)>(v);
    if constexpr (LPR >= 16) sum_level<8, (GP >= 8 ? GP / 8 : 1)>(v);
    if constexpr (LPR >= 32) sum_level<16, (GP >= 16 ? GP / 16 : 1)>(v);
    return v[0];
}

// The head whose sum a lane ends with: lane bit k selects the upper half at
// level k.
template <int GP>
__device__ __forceinline__ int lane_head(int lane) {
    int h = 0;
#pragma unroll
    for (int k = 0, m = GP / 2; m >= 1; ++k, m >>= 1)
        if (lane & (1 << k)) h += m;
    return h;
}

// Every live node of levels top_lo .. L, every query head of its pair:
// grid (workgroups per pair, pairs); a wavefront takes kTopU nodes at a
// time, reads each record once (16-byte loads) and scores it for the GP
// query heads held in registers (slot j of a lane holds the query of head
// j ^ lane_head, as transposed_sum expects).  The lanes ending with head h
// in the first reference group write its score.
template <int D, int R, typename QT, typename ST, int GP>
__global__ __launch_bounds__(kTopThreads) void k_top_score(SearchArgs a) {
    constexpr int EPL = row_epl<D, ST>();
    constexpr int LPR = D / EPL;
    constexpr int RPL = 64 / LPR;
    constexpr int NL = (R + RPL - 1) / RPL;
    constexpr int kW = kTopThreads / 64;
    // the wavefront index as a uniform value: the node loop below and its
    // per-level table lookups then run on scalar registers and scalar loads
    // (with a per-lane index they would be vector loads of the argument
    // buffer, one dependent round trip per lookup)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane % LPR, rsub = lane / LPR;
    const int64_t pair = blockIdx.y;
    const int G = a.group;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x <= ZHA_MAX_STEPS) a.tile_count[threadIdx.x] = 0;
    const int my_head = lane_head<GP>(sub);
    // the pair's query heads: walks pair*G .. pair*G + G - 1 (decode)
    float qv[GP][EPL];
#pragma unroll
    for (int j = 0; j < GP; ++j) {
        const int h = j ^ my_head;
        const int hh = h < G ? h : 0;
        const QT *qp = static_cast<const QT *>(a.q) + (pair * G + hh) * D + EPL * sub;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[j][e] = Elem<QT>::load(qp, e);
    }
    // live nodes of the table, level by level from the top
    int64_t live = 0;
    for (int l = a.top_lo; l <= a.levels; ++l) live += a.nl[l];
    const int gp = (G + 3) & ~3;
    float *tab = a.u_score + pair * a.top_rows * gp;
    const float s = a.sharpness;
    const bool writer = rsub == 0 && sub < GP && my_head < G;
    for (int64_t x0 = (static_cast<int64_t>(blockIdx.x) * kW + wave) * kTopU; x0 < live;
         x0 += static_cast<int64_t>(gridDim.x) * kW * kTopU) {
        float kv[kTopU][NL][EPL];
        float bv[kTopU][NL];
        int64_t row[kTopU];
#pragma unroll
        for (int u = 0; u < kTopU; ++u) {
            // the u-th node: its level and index (levels from the top)
            int64_t x = x0 + u;
            const bool ok = x < live;
            if (!ok) x = live - 1;
            int l = a.levels;
            while (l > a.top_lo && x >= a.nl[l]) { x -= a.nl[l]; --l; }
            row[u] = ok ? a.top_off[l] + x : -1;
            const int64_t node = pair * a.cap[l] + x;
            const ST *kp = reinterpret_cast<const ST *>(a.kap[l]) + node * (R * D);
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int r = i * RPL + rsub;
                if (r < R) {
                    // each record is read once for all heads of the pair:
                    // streaming loads
                    if constexpr (EPL == 8)
                        Vec16<ST>::load_nt(kp + r * D + EPL * sub, kv[u][i]);
                    else
                        Vec4<ST>::load_nt(kp + r * D + EPL * sub, kv[u][i]);
                    bv[u][i] = a.bet[l][node * R + r];
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) kv[u][i][e] = 0.f;
                    bv[u][i] = -INFINITY;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kTopU; ++u) {
            float best = -INFINITY;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                float pd[GP];
#pragma unroll
                for (int j = 0; j < GP; ++j) {
                    float d = kv[u][i][0] * qv[j][0];
#pragma unroll
                    for (int e = 1; e < EPL; ++e) d = fmaf(kv[u][i][e], qv[j][e], d);
                    pd[j] = d;
                }
                const float d = transposed_sum<LPR, GP>(pd);
                best = fmaxf(best, fmaf(s, d, bv[u][i]));
            }
            // max over the RPL reference groups (lanes LPR apart)
            if constexpr (RPL >= 4)
                best = fmaxf(best, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(best), 0x401F)));
            if constexpr (RPL >= 2) best = fmaxf(best, xor_lane_f(best, 32));
            float m = best;
            if (m != m) m = -INFINITY;
            if (m == 0.f) m = 0.f;
            if (row[u] >= 0 && writer) tab[row[u] * gp + my_head] = m;
        }
    }
}

// Steps 0 .. top_steps-1 of every walk from the table, one workgroup per
// walk (as the persistent engine's step loop), then the hand-over to the
// level-synchronous steps: the walk state, the candidate list of step
// top_steps and its scoring tiles.
template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kThreads) void k_top_cut(SearchArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // a pair's heads on one XCD: they read the same rows of the pair's table
    const int w = static_cast<int>(xcd_item(blockIdx.x, a.walks));
    if (w < 0) return;
    const int64_t pair = walk_pair(w, 1, a.heads, a.group, a.kv_heads);
    const int h = w % a.group;
    const int cap = a.cand_cap, gp = (a.group + 3) & ~3;

    __shared__ SelectShared sh;
    __shared__ WalkState st;
    __shared__ int s_rest, s_base;
    __shared__ int32_t s_scored[ZHA_MAX_STEPS], s_opened[ZHA_MAX_STEPS];
    __shared__ float s_tab[kTopRowsMax];             // this head's column of the table
    __shared__ int32_t s_toff[ZHA_MAX_LEVELS + 2];   // first table row of each level (looked up per lane)
    __shared__ uint32_t s_list[2 * kTopList];        // two candidate lists (when a.top_lds)
    __shared__ float s_sc[kTopList];
    if (tid == 0) sh.flags = 0;
    if (tid < ZHA_MAX_LEVELS + 2) s_toff[tid] = static_cast<int32_t>(a.top_off[tid]);
    {
        const float *tab = a.u_score + pair * a.top_rows * gp + h;
        for (int64_t r = tid; r < a.top_rows; r += kThreads) s_tab[r] = tab[r * gp];
    }

    float qv[row_epl<D, ST>()];
    load_q<D, QT, ST>(a, w, qv);
    uint32_t *gbufs = a.cand + static_cast<int64_t>(w) * 2 * cap;
    const bool in_lds = a.top_lds != 0;
    uint32_t *lists = in_lds ? s_list : gbufs;
    // lists are clamped to the candidate capacity in either mode: the list
    // handed over must fit the walk's global buffers and tile map
    const int lcap = in_lds ? min(kTopList, cap) : cap;
    int buf = 0;
    float *sc = in_lds ? s_sc : a.score + static_cast<int64_t>(w) * cap;
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;
    uint32_t flags = 0;
    int n = write_roots(a, lists, flags);
    __syncthreads();
    int64_t sel_n = 0;
    int32_t unforced = 0;
    int t = 0;
    for (; t < a.top_steps && n > 0; ++t) {
        const uint32_t *cur = lists + static_cast<int64_t>(buf) * lcap;
        uint32_t *nxt = lists + static_cast<int64_t>(buf ^ 1) * lcap;
        const bool forced = step_forced(a, t, n);
        unsigned long long tau = 0;
        if (!forced) {
            // table scores; candidates below the table are counted
            if (tid == 0) s_rest = 0;
            __syncthreads();
            float m = -INFINITY;
            int rest = 0;
            for (int i = tid; i < n; i += kThreads) {
                const uint32_t id = cur[i];
                const int lvl = static_cast<int>(id >> kLevelShift);
                if (lvl >= a.top_lo) {
                    const float v = s_tab[s_toff[lvl] + (id & kIndexMask)];
                    sc[i] = v;
                    m = fmaxf(m, v);
                } else {
                    ++rest;
                }
                if (a.visited) {
                    const int64_t bit = a.node_off[lvl] + (id & kIndexMask);
                    atomicOr(a.visited + pair * a.vis_words + (bit >> 5), 1u << (bit & 31));
                }
            }
            if (rest) atomicAdd(&s_rest, rest);
            __syncthreads();
            if (s_rest > 0) {
                // the few below the table: one wavefront each
                for (int i = wave; i < n; i += kWaves) {
                    const uint32_t id = __builtin_amdgcn_readfirstlane(cur[i]);
                    if (static_cast<int>(id >> kLevelShift) >= a.top_lo) continue;
                    const float v = score_one<D, R, ST>(a, pair, qv, id, flags);
                    if (lane == 0) sc[i] = v;
                    m = fmaxf(m, v);
                }
            }
            if (n <= 64) {
                // one candidate per lane of wavefront 0: the sort-based cut
                __syncthreads();                     // sc[] is complete
                if (wave == 0) {
                    const bool in = lane < n;
                    const float v = in ? sc[lane] : -INFINITY;
                    const uint32_t id = in ? cur[lane] : 0u;
                    const unsigned long long k = lane_tau(a, in, v, id, wave_max(v, 1, 64), n, a.k[t]);
                    if (lane == 0) sh.tau = k;
                }
                __syncthreads();
                tau = sh.tau;
            } else {
                const float mx = block_max(m, sh);     // also a barrier: sc[] is complete
                tau = cut_tau_win(a, n, cur, sc, mx, a.k[t], sh, &flags);
            }
            unforced += n;
        }
        uint32_t ta, tb;
        open_cut(a, n, cur, sc, forced, tau, nxt, selw, sel_n, ta, tb, sh, lcap);
        if (tid == 0) {
            s_scored[t] = n;
            s_opened[t] = static_cast<int32_t>(ta + tb);
        }
        sel_n += ta;
        int64_t nn = static_cast<int64_t>(tb) * a.chunk;
        if (nn > lcap) { flags |= ZHA_FLAG_CAND_OVERFLOW; nn = lcap; }
        buf ^= 1;
        n = static_cast<int>(nn);
        __syncthreads();
    }
    // the list the level-synchronous steps take over, in the walk's buffer 0
    if (in_lds) {
        const uint32_t *fin = lists + static_cast<int64_t>(buf) * lcap;
        for (int i = tid; i < n; i += kThreads) gbufs[i] = fin[i];
        buf = 0;
    }
    if (flags) atomicOr(&sh.flags, flags);
    __syncthreads();
    if (tid == 0) {
        st.n = n;
        st.buf = buf;
        st.sel_n = static_cast<int32_t>(sel_n);
        st.unforced = unforced;
        st.flags = sh.flags;
        st.steps = t;
        for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
            st.scored[i] = i < t ? s_scored[i] : 0;
            st.opened[i] = i < t ? s_opened[i] : 0;
        }
        if (st.n == 0 || t >= a.levels || t >= ZHA_MAX_STEPS) {
            st.n = 0;
            finish_walk<R>(a, w, t, st.scored, st.opened, st.sel_n, st.unforced, st.flags);
        }
        a.state[w] = st;
        s_base = 0;
        if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t, st.n))
            s_base = atomicAdd(&a.tile_count[t], (st.n + kTile - 1) / kTile);
    }
    __syncthreads();
    if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t, st.n)) {
        const int ntile = (st.n + kTile - 1) / kTile;
        for (int k = tid; k < ntile; k += kThreads) a.tile_map[s_base + k] = make_int2(w, k * kTile);
    }
}

// ---- launchers ---------------------------------------------------------------------

template <int D, int R, typename QT, typename ST>
static hipError_t launch_top_t(const SearchArgs &a, hipStream_t st) {
    int64_t live = 0;
    for (int l = a.top_lo; l <= a.levels; ++l) live += a.nl[l];
    const int64_t per_wg = (kTopThreads / 64) * kTopU;
    int gx = static_cast<int>((live + per_wg - 1) / per_wg);
    if (gx < 1) gx = 1;
    dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(a.pairs));
    if (a.group <= 4)
        hipLaunchKernelGGL((k_top_score<D, R, QT, ST, 4>), grid, dim3(kTopThreads), 0, st, a);
    else if (a.group <= 8)
        hipLaunchKernelGGL((k_top_score<D, R, QT, ST, 8>), grid, dim3(kTopThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_top_score<D, R, QT, ST, 16>), grid, dim3(kTopThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_top_cut<D, R, QT, ST>), dim3(static_cast<unsigned>(xcd_grid(a.walks))), dim3(kThreads), 0,
                       st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.top_steps < a.levels)
        return launch_ls_from(a, D, R, sizeof(QT) == 2 ? ZHA_BF16 : ZHA_F32, sizeof(ST) == 2 ? ZHA_BF16 : ZHA_F32,
                              a.top_steps, st);
    return hipSuccess;
}

template <int D, typename QT, typename ST>
static hipError_t launch_top_r(const SearchArgs &a, int R, hipStream_t st) {
    switch (R) {
        case 1: return launch_top_t<D, 1, QT, ST>(a, st);
        case 2: return launch_top_t<D, 2, QT, ST>(a, st);
        case 4: return launch_top_t<D, 4, QT, ST>(a, st);
        case 8: return launch_top_t<D, 8, QT, ST>(a, st);
        case 16: return launch_top_t<D, 16, QT, ST>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, typename QT>
static hipError_t launch_top_s(const SearchArgs &a, int R, int sdtype, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_top_r<D, QT, bf16_t>(a, R, st) : launch_top_r<D, QT, float>(a, R, st);
}

hipError_t launch_top(const SearchArgs &a, int D, int R, int dtype, int sdtype, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_top_s<64, bf16_t>(a, R, sdtype, st) : launch_top_s<64, float>(a, R, sdtype, st);
    return dtype == ZHA_BF16 ? launch_top_s<128, bf16_t>(a, R, sdtype, st) : launch_top_s<128, float>(a, R, sdtype, st);
}

}  // namespace zha
