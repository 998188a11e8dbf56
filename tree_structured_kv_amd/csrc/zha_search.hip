// zha_search.hip -- top-down tree walks for decode queries.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".
//   "What does a node summarize?": a node's score for query q is the largest
//     over references r of s <key_r, q> + bias_r.
//   "Run a small tree yourself": per step the walk scores every candidate,
//     normalises the scores with one softmax over the whole candidate list,
//     opens a prefix of the list ordered by mass, reads the keys of opened
//     bottom-level nodes and makes the children of the other opened nodes
//     the next candidates, until no candidates remain.
//   "How does top-p differ from top-K?": top-p opens the smallest prefix
//     whose mass reaches p (the node that crosses p included); top-K opens
//     exactly K.
//   "Common misunderstandings": every query head walks on its own.
//
// Two engines share the scoring, cut and opening code below.
//
// * Persistent (k_search_decode): one workgroup (8 wavefronts) per walk, the
//   step loop inside the kernel, no host round trip.  Best when every walk
//   does the same work (top-K).
// * Level-synchronous (k_ls_*): per step, one grid-wide scoring launch over
//   a flat list of 32-candidate tiles of all walks, then one cut launch with
//   a workgroup per walk.  Kernel boundaries are the only synchronisation.
//   Under top-p a few walks can score ten times the median; spreading their
//   candidates over the whole GPU keeps every CU streaming.
//
// Scoring: a candidate's R keys are one contiguous R*D*4-byte record; a
// wavefront reads it with 16-byte loads (D/4 lanes per reference), sums the
// dot products with DPP/swizzle cross-lane adds and takes the max over
// references.  The cut is an exact radix select over 64-bit rank keys
// (ordered score bits, then the complement of the span start, so equal
// scores open in span order).  For top-p the softmax masses are integers
// (exp(score - max) scaled by 2^31 and rounded), so every sum is exact and
// the cut is bit-reproducible.  Opened nodes are compacted in candidate
// order, which keeps every candidate list in span order without a sort.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

namespace {

constexpr int kScoreThreads = 256;     // workgroup of the level-synchronous scorer
constexpr int kU = 4;                  // candidates in flight per wavefront

// Elements of a node-key row per lane: 16 bytes of keys (4 fp32, or 8 bf16
// while that still leaves at least 16 lanes per row).
template <int D, typename ST>
constexpr int row_epl() { return (sizeof(ST) == 2 && D >= 128) ? 8 : 4; }

template <int D, typename QT, typename ST>
__device__ __forceinline__ void load_q(const SearchArgs &a, int w, float (&qv)[row_epl<D, ST>()]) {
    constexpr int EPL = row_epl<D, ST>();
    constexpr int LPR = D / EPL;
    const int sub = (threadIdx.x & 63) % LPR;
    const QT *qp = static_cast<const QT *>(a.q) + static_cast<int64_t>(w) * D + EPL * sub;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = Elem<QT>::load(qp, e);
}

// One wavefront scores candidates first, first + stride, ... below `end`, kU
// at a time, and writes sc[i]; returns the largest score it wrote.  The
// candidate's R biases sit at a wavefront-uniform address and come in
// through scalar loads (no search writes node records).  With kScalarList
// the candidate ids do too: only where the list was written by an earlier
// launch, since the scalar cache does not see this kernel's own stores.
template <int D, int R, typename ST, bool kScalarList>
__device__ __forceinline__ float score_wave(const SearchArgs &a, int64_t pair,
                                            const float (&qv)[row_epl<D, ST>()],
                                            const uint32_t *cur, float *sc, int first, int end,
                                            int stride, uint32_t &flags) {
    constexpr int EPL = row_epl<D, ST>();  // key elements per lane (one 16-byte load)
    constexpr int LPR = D / EPL;          // lanes per reference row
    constexpr int RPL = 64 / LPR;         // references per 64-lane load
    constexpr int NL = (R + RPL - 1) / RPL;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rsub = lane / LPR;
    const float s = a.sharpness;
    float wmax = -INFINITY;
    if (first >= end) return wmax;

    first = __builtin_amdgcn_readfirstlane(first);
    end = __builtin_amdgcn_readfirstlane(end);
    uint32_t ids[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int i = first + u;
        ids[u] = kScalarList ? cload_u32(cur + (i < end ? i : end - 1)) : cur[i < end ? i : end - 1];
    }
    for (int base = first; base < end; base += stride) {
        float kv[kU][NL][EPL];
        float bv[kU][NL];
        uint32_t cid[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t id = __builtin_amdgcn_readfirstlane(ids[u]);   // the same for every lane
            cid[u] = id;
            const int lvl = static_cast<int>(id >> kLevelShift);
            const int64_t node = pair * a.cap[lvl] + static_cast<int64_t>(id & kIndexMask);
            const ST *kp = reinterpret_cast<const ST *>(a.kap[lvl]) + node * (R * D);
            float bsr[R];
#pragma unroll
            for (int r = 0; r < R; ++r) bsr[r] = cload_f(a.bet[lvl] + node * R + r);
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const int r = l * RPL + rsub;
                if (r < R) {
                    if constexpr (EPL == 8)
                        Vec16<ST>::load(kp + r * D + EPL * sub, kv[u][l]);
                    else
                        Vec4<ST>::load(kp + r * D + EPL * sub, kv[u][l]);
                    // this lane's reference r = l*RPL + rsub, chosen among SGPRs
                    float b = bsr[l * RPL];
#pragma unroll
                    for (int g = 1; g < RPL; ++g)
                        if (rsub == g && l * RPL + g < R) b = bsr[l * RPL + g];
                    bv[u][l] = b;
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) kv[u][l][e] = 0.f;
                    bv[u][l] = -INFINITY;
                }
            }
        }
        // ids of the next round, fetched while this round's records stream in
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = base + stride + u;
            ids[u] = kScalarList ? cload_u32(cur + (i < end ? i : end - 1)) : cur[i < end ? i : end - 1];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float best = -INFINITY;
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                float d = kv[u][l][0] * qv[0];
#pragma unroll
                for (int e = 1; e < EPL; ++e) d = fmaf(kv[u][l][e], qv[e], d);
                d = group_sum<LPR>(d);
                best = fmaxf(best, fmaf(s, d, bv[u][l]));
            }
            // max over the RPL reference groups of the wavefront
            float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 0));
#pragma unroll
            for (int gq = 1; gq < RPL; ++gq)
                m = fmaxf(m, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), gq * LPR)));
            if (m != m) { m = -INFINITY; flags |= ZHA_FLAG_NONFINITE; }
            if (m == 0.f) m = 0.f;          // one zero
            const int i = base + u;
            if (i < end) {
                if (lane == 0) {
                    sc[i] = m;
                    if (a.visited) {
                        const uint32_t id = cid[u];
                        const int64_t bit = a.node_off[id >> kLevelShift] + (id & kIndexMask);
                        atomicOr(a.visited + pair * a.vis_words + (bit >> 5), 1u << (bit & 31));
                    }
                }
                wmax = fmaxf(wmax, m);
            }
        }
    }
    return wmax;
}

// Workgroup (kThreads): open every candidate with a rank key >= tau (all if
// forced), in candidate order: level-1 nodes append their block id to the
// selection, others append their c children to nxt.  Returns the number of
// level-1 and of higher nodes opened.
__device__ void open_cut(const SearchArgs &a, int n, const uint32_t *cur, const float *sc,
                         bool forced, unsigned long long tau, uint32_t *nxt, int32_t *selw,
                         int64_t sel_n, uint32_t &ta, uint32_t &tb, SelectShared &sh) {
    const int tid = threadIdx.x;
    const int c = a.chunk, log2c = a.log2c, cap = a.cand_cap;
    const int per = (n + kThreads - 1) / kThreads;
    const int i0 = tid * per;
    const int i1 = min(n, i0 + per);
    uint32_t ca = 0, cb = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t id = cur[i];
        const bool open = forced || rank_key(sc[i], id, log2c) >= tau;
        if (open) { if ((id >> kLevelShift) == 1u) ++ca; else ++cb; }
    }
    unsigned long long tot;
    const unsigned long long off =
        block_exscan64((static_cast<unsigned long long>(ca) << 32) | cb, sh.scan64, &tot);
    uint32_t oa = static_cast<uint32_t>(off >> 32), ob = static_cast<uint32_t>(off);
    ta = static_cast<uint32_t>(tot >> 32);
    tb = static_cast<uint32_t>(tot);
    for (int i = i0; i < i1; ++i) {
        const uint32_t id = cur[i];
        const bool open = forced || rank_key(sc[i], id, log2c) >= tau;
        if (!open) continue;
        const uint32_t lvl = id >> kLevelShift, j = id & kIndexMask;
        if (lvl == 1u) {
            const int64_t pos = sel_n + oa++;
            if (pos < a.sel_cap) selw[pos] = static_cast<int32_t>(j);
        } else {
            const int64_t base = static_cast<int64_t>(ob++) * c;
            const uint32_t cid = ((lvl - 1u) << kLevelShift);
            for (int e = 0; e < c; ++e) {
                if (base + e < cap) nxt[base + e] = cid | (j * static_cast<uint32_t>(c) + e);
            }
        }
    }
}

}  // namespace

// ---- persistent engine --------------------------------------------------------

template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kThreads) void k_search_decode(SearchArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    if (w >= a.walks) return;
    const int64_t pair = walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
    const int cap = a.cand_cap;

    __shared__ SelectShared sh;
    __shared__ int32_t s_scored[ZHA_MAX_STEPS], s_opened[ZHA_MAX_STEPS];
    if (tid == 0) sh.flags = 0;

    float qv[row_epl<D, ST>()];
    load_q<D, QT, ST>(a, w, qv);

    uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * cap;
    uint32_t *nxt = cur + cap;
    float *sc = a.score + static_cast<int64_t>(w) * cap;
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;

    uint32_t flags = 0;
    int n = write_roots(a, cur, flags);
    __syncthreads();

    int64_t sel_n = 0;
    int32_t unforced = 0;
    int t = 0;
    for (; t < ZHA_MAX_STEPS && n > 0; ++t) {
        const bool forced = step_forced(a, t, n);
        unsigned long long tau = 0;
        if (!forced) {
            float wmax = score_wave<D, R, ST, false>(a, pair, qv, cur, sc, wave * kU, n, kWaves * kU, flags);
            if (lane == 0) sh.red[wave] = wmax;
            __syncthreads();
            float mx = sh.red[0];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) mx = fmaxf(mx, sh.red[i]);
            tau = cut_tau_win(a, n, cur, sc, mx, a.k[t], sh, &flags);
            unforced += n;
        }
        uint32_t ta, tb;
        open_cut(a, n, cur, sc, forced, tau, nxt, selw, sel_n, ta, tb, sh);
        if (tid == 0) {
            s_scored[t] = n;
            s_opened[t] = static_cast<int32_t>(ta + tb);
        }
        sel_n += ta;
        int64_t nn = static_cast<int64_t>(tb) * a.chunk;
        if (nn > cap) { flags |= ZHA_FLAG_CAND_OVERFLOW; nn = cap; }
        uint32_t *tmp = cur; cur = nxt; nxt = tmp;
        n = static_cast<int>(nn);
        __syncthreads();
    }
    if (flags) atomicOr(&sh.flags, flags);
    __syncthreads();
    if (tid == 0) finish_walk<R>(a, w, t, s_scored, s_opened, sel_n, unforced, sh.flags);
}

// ---- level-synchronous engine ---------------------------------------------------

template <int R>
__global__ __launch_bounds__(kThreads) void k_ls_init(SearchArgs a) {
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    const int cap = a.cand_cap;
    if (w == 0 && tid <= ZHA_MAX_STEPS) a.tile_count[tid] = 0;
    __shared__ uint32_t s_flags;
    if (tid == 0) s_flags = 0;
    __syncthreads();
    uint32_t flags = 0;
    uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * cap;
    const int n = write_roots(a, cur, flags);
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid == 0) {
        WalkState st;
        st.n = n;
        st.buf = 0;
        st.sel_n = 0;
        st.unforced = 0;
        st.flags = s_flags;
        st.steps = 0;
        for (int i = 0; i < ZHA_MAX_STEPS; ++i) { st.scored[i] = 0; st.opened[i] = 0; }
        a.state[w] = st;
        if (n == 0) finish_walk<R>(a, w, 0, st.scored, st.opened, 0, 0, st.flags);
    }
}

// Step t scoring over a flat tile list: at step 0 every walk has the same
// roots, so its tiles are laid out arithmetically; later steps use the tiles
// the cut kernel of the step before registered.
template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kScoreThreads) void k_ls_score(SearchArgs a, int t, int tiles0) {
    constexpr int kSW = kScoreThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_tiles = (t == 0) ? a.walks * tiles0 : a.tile_count[t];
    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        int w, start;
        if (t == 0) {
            w = tile / tiles0;
            start = (tile % tiles0) * kTile;
        } else {
            const int2 e = a.tile_map[tile];
            w = __builtin_amdgcn_readfirstlane(e.x);
            start = __builtin_amdgcn_readfirstlane(e.y);
        }
        const int n = a.state[w].n;
        const int buf = a.state[w].buf;
        const int end = min(n, start + kTile);
        const int64_t pair = walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
        const uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * a.cand_cap +
                              static_cast<int64_t>(buf) * a.cand_cap;
        float *sc = a.score + static_cast<int64_t>(w) * a.cand_cap;
        float qv[row_epl<D, ST>()];
        load_q<D, QT, ST>(a, w, qv);
        uint32_t flags = 0;
        (void)score_wave<D, R, ST, true>(a, pair, qv, cur, sc, start + wave * kU, end, kSW * kU, flags);
        if (flags && lane == 0) atomicOr(a.status, flags);
    }
}

// Step t cut: one workgroup per walk.
constexpr int kLsStage = 6144;         // candidates a level-synchronous cut stages in LDS (48 KB)
constexpr int kStageU = 12;            // staging loads in flight per thread

template <int R>
__global__ __launch_bounds__(kThreads) void k_ls_cut(SearchArgs a, int t) {
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    __shared__ SelectShared sh;
    __shared__ uint32_t s_id[kLsStage];
    __shared__ float s_sc[kLsStage];
    __shared__ WalkState st;
    __shared__ int s_base;
    if (tid == 0) st = a.state[w];
    __syncthreads();
    const int n = st.n;
    if (n <= 0) return;                    // finished earlier (uniform)
    const int cap = a.cand_cap;
    uint32_t *bufs = a.cand + static_cast<int64_t>(w) * 2 * cap;
    const uint32_t *cur = bufs + static_cast<int64_t>(st.buf) * cap;
    uint32_t *nxt = bufs + static_cast<int64_t>(st.buf ^ 1) * cap;
    const float *sc = a.score + static_cast<int64_t>(w) * cap;
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;

    const bool forced = step_forced(a, t, n);
    // the walk's candidate ids and scores, staged in LDS once (kLsStage
    // entries at most; all loads of a lane in flight together), so that the
    // cut's passes and the opening read no global memory
    const bool staged = n <= kLsStage;
    float m = -INFINITY;
    if (staged) {
        for (int i0 = tid; i0 < n; i0 += kStageU * kThreads) {
            uint32_t id[kStageU];
            float v[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kThreads;
                id[u] = i < n ? cur[i] : 0u;
                v[u] = (i < n && !forced) ? sc[i] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kThreads;
                if (i < n) {
                    s_id[i] = id[u];
                    s_sc[i] = v[u];
                    m = fmaxf(m, v[u]);
                }
            }
        }
    } else if (!forced) {
        for (int i = tid; i < n; i += kThreads) m = fmaxf(m, sc[i]);
    }
    const uint32_t *cid = staged ? s_id : cur;
    const float *csc = staged ? s_sc : sc;
    unsigned long long tau = 0;
    uint32_t path = (staged || forced) ? 0u : kPathLdsSpill;
    if (!forced) {
        const float mx = block_max(m, sh);        // also a barrier: the staged entries are complete
        tau = cut_tau_win(a, n, cid, csc, mx, a.k[t], sh, &path);
    } else {
        __syncthreads();
    }
    uint32_t ta, tb;
    open_cut(a, n, cid, csc, forced, tau, nxt, selw, st.sel_n, ta, tb, sh);
    __syncthreads();
    if (tid == 0) {
        int64_t nn = static_cast<int64_t>(tb) * a.chunk;
        if (nn > cap) { st.flags |= ZHA_FLAG_CAND_OVERFLOW; nn = cap; }
        st.flags |= path;
        st.scored[t] = n;
        st.opened[t] = static_cast<int32_t>(ta + tb);
        if (!forced) st.unforced += n;
        st.sel_n += static_cast<int32_t>(ta);
        st.steps = t + 1;
        st.buf ^= 1;
        st.n = static_cast<int32_t>(nn);
        if (st.n == 0 || t + 1 >= a.levels || t + 1 >= ZHA_MAX_STEPS) {
            st.n = 0;
            finish_walk<R>(a, w, t + 1, st.scored, st.opened, st.sel_n, st.unforced, st.flags);
        }
        a.state[w] = st;
        s_base = 0;
        if (st.n > 0 && !step_forced(a, t + 1, st.n))
            s_base = atomicAdd(&a.tile_count[t + 1], (st.n + kTile - 1) / kTile);
    }
    __syncthreads();
    // register the next step's tiles unless its cut needs no scores
    if (st.n > 0 && !step_forced(a, t + 1, st.n)) {
        const int ntile = (st.n + kTile - 1) / kTile;
        for (int k = tid; k < ntile; k += kThreads) a.tile_map[s_base + k] = make_int2(w, k * kTile);
    }
}

// ---- launchers ---------------------------------------------------------------------

template <int D, int R, typename QT, typename ST>
static hipError_t launch_t(const SearchArgs &a, int engine, int n0, hipStream_t st) {
    if (engine != ZHA_ENGINE_LEVEL_SYNC) {
        hipLaunchKernelGGL((k_search_decode<D, R, QT, ST>), dim3(a.walks), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_ls_init<R>), dim3(a.walks), dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles0 = (n0 + kTile - 1) / kTile;
    for (int t = 0; t < a.levels && t < ZHA_MAX_STEPS; ++t) {
        // step 0's forcing is the same for every walk (same roots)
        const bool skip = (t == 0) && (n0 <= 1 || (a.mode == ZHA_TOPK && a.k[0] >= n0) ||
                                       (a.mode == ZHA_TOPP && a.p >= 1.0f));
        if (!skip) {
            hipLaunchKernelGGL((k_ls_score<D, R, QT, ST>), dim3(a.score_grid), dim3(kScoreThreads), 0, st,
                               a, t, tiles0 > 0 ? tiles0 : 1);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((k_ls_cut<R>), dim3(a.walks), dim3(kThreads), 0, st, a, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// Steps t0 .. of the level-synchronous engine, after another engine wrote
// the walks' state, candidate lists and scoring tiles of step t0.
template <int D, int R, typename QT, typename ST>
static hipError_t launch_ls_from_t(const SearchArgs &a, int t0, hipStream_t st) {
    hipError_t e;
    for (int t = t0; t < a.levels && t < ZHA_MAX_STEPS; ++t) {
        hipLaunchKernelGGL((k_ls_score<D, R, QT, ST>), dim3(a.score_grid), dim3(kScoreThreads), 0, st, a, t, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_ls_cut<R>), dim3(a.walks), dim3(kThreads), 0, st, a, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, typename QT, typename ST>
static hipError_t launch_ls_from_d(const SearchArgs &a, int R, int t0, hipStream_t st) {
    switch (R) {
        case 1: return launch_ls_from_t<D, 1, QT, ST>(a, t0, st);
        case 2: return launch_ls_from_t<D, 2, QT, ST>(a, t0, st);
        case 4: return launch_ls_from_t<D, 4, QT, ST>(a, t0, st);
        case 8: return launch_ls_from_t<D, 8, QT, ST>(a, t0, st);
        case 16: return launch_ls_from_t<D, 16, QT, ST>(a, t0, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ls_from(const SearchArgs &a, int D, int R, int dtype, int sdtype, int t0, hipStream_t st) {
    if (D == 64) {
        if (dtype == ZHA_BF16)
            return sdtype == ZHA_BF16 ? launch_ls_from_d<64, bf16_t, bf16_t>(a, R, t0, st)
                                      : launch_ls_from_d<64, bf16_t, float>(a, R, t0, st);
        return sdtype == ZHA_BF16 ? launch_ls_from_d<64, float, bf16_t>(a, R, t0, st)
                                  : launch_ls_from_d<64, float, float>(a, R, t0, st);
    }
    if (dtype == ZHA_BF16)
        return sdtype == ZHA_BF16 ? launch_ls_from_d<128, bf16_t, bf16_t>(a, R, t0, st)
                                  : launch_ls_from_d<128, bf16_t, float>(a, R, t0, st);
    return sdtype == ZHA_BF16 ? launch_ls_from_d<128, float, bf16_t>(a, R, t0, st)
                              : launch_ls_from_d<128, float, float>(a, R, t0, st);
}

template <int D, typename QT, typename ST>
static hipError_t launch_search_d(const SearchArgs &a, int R, int engine, int n0, hipStream_t st) {
    switch (R) {
        case 1: return launch_t<D, 1, QT, ST>(a, engine, n0, st);
        case 2: return launch_t<D, 2, QT, ST>(a, engine, n0, st);
        case 4: return launch_t<D, 4, QT, ST>(a, engine, n0, st);
        case 8: return launch_t<D, 8, QT, ST>(a, engine, n0, st);
        case 16: return launch_t<D, 16, QT, ST>(a, engine, n0, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, typename QT>
static hipError_t launch_search_s(const SearchArgs &a, int R, int sdtype, int engine, int n0, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_search_d<D, QT, bf16_t>(a, R, engine, n0, st)
                              : launch_search_d<D, QT, float>(a, R, engine, n0, st);
}

hipError_t launch_search(const SearchArgs &a, int D, int R, int dtype, int sdtype, int engine, int n0,
                         hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_search_s<64, bf16_t>(a, R, sdtype, engine, n0, st)
                                 : launch_search_s<64, float>(a, R, sdtype, engine, n0, st);
    return dtype == ZHA_BF16 ? launch_search_s<128, bf16_t>(a, R, sdtype, engine, n0, st)
                             : launch_search_s<128, float>(a, R, sdtype, engine, n0, st);
}

}  // namespace zha
