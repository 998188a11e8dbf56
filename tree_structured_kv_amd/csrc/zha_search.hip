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
#include "zha_score.h"

namespace zha {

namespace {

constexpr int kScoreThreads = 256;     // workgroup of the level-synchronous scorer

}  // namespace

// ---- persistent engine --------------------------------------------------------

// At most 128 VGPRs (four wavefronts per SIMD: two workgroups per CU); the
// two scoring variants together would take 136 and leave one.
template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kThreads, 4) void k_search_decode(SearchArgs a) {
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
            // streaming record loads when the group's heads, each with a list
            // as long as this one, cover less than half of the step's level
            // (the rule of the level-synchronous scorer, from this walk's
            // count: under top-K every head's list has the same length)
            const bool stream = static_cast<int64_t>(n) * a.group * 2 < a.nl[max(1, a.levels - t)];
            const float wmax =
                stream ? score_wave<D, R, ST, false, false, true>(a, pair, qv, cur, sc, wave * kU, n, kWaves * kU, flags)
                       : score_wave<D, R, ST, false>(a, pair, qv, cur, sc, wave * kU, n, kWaves * kU, flags);
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

// Step t scoring over tiles of kTile candidates of one walk.  The tiles are
// taken in walk order -- a pair's heads are consecutive walks whose lists,
// all in span order, overlap -- and XCD x takes the x-th eighth of that
// order with its workgroups side by side, so the heads of a pair read the
// node records they share through one L2 at about the same time.  Step 0's
// tiles are arithmetic (every walk has the same roots).  Later steps count
// each walk's tiles from its state (the walks whose cut at step t needs
// scores) in LDS when there are at most kPlanWalks walks, else take the
// tiles the cut kernels registered.
//
// Records come in through streaming (nontemporal) loads when the step's
// candidates over all walks are fewer than half the pairs' nodes of the
// step's level: the heads of a pair then rarely read the same record, and a
// streaming read moves a whole-line-per-instruction access faster.  Where the
// heads' lists cover most of a level they overlap, and ordinary loads leave
// the shared records in L2 for the next head (measured: 256K clustered keys,
// 8 heads per pair, 22% of level 1 per step, 137 -> 133 us per launch;
// 64K AR(1) keys, 4 heads, more than the whole level, 10% slower streamed).
template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kScoreThreads) void k_ls_score(SearchArgs a, int t, int tiles0) {
    constexpr int kSW = kScoreThreads / 64;
    __shared__ int s_first[kPlanWalks + 1];    // each walk's first tile, then the total
    __shared__ int s_part[kSW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool plan = t > 0 && ls_tile_plan(a);
    int n_tiles;
    if (t == 0) {
        n_tiles = a.walks * tiles0;
    } else if (!plan) {
        n_tiles = a.tile_count[t];
    } else {
        for (int w = threadIdx.x; w < a.walks; w += kScoreThreads) {
            const int n = a.state[w].n;
            s_first[w] = (n > 0 && !step_forced(a, t, n)) ? (n + kTile - 1) / kTile : 0;
        }
        __syncthreads();
        // exclusive scan: each thread a run of consecutive walks
        const int per = (a.walks + kScoreThreads - 1) / kScoreThreads;
        const int w0 = min(a.walks, static_cast<int>(threadIdx.x) * per);
        const int w1 = min(a.walks, w0 + per);
        int sum = 0;
        for (int w = w0; w < w1; ++w) sum += s_first[w];
        const int incl = static_cast<int>(wave_scan_u32(static_cast<uint32_t>(sum)));
        if (lane == 63) s_part[wave] = incl;
        __syncthreads();
        int run = incl - sum, total = 0;
#pragma unroll
        for (int k = 0; k < kSW; ++k) {
            const int v = s_part[k];
            if (k < wave) run += v;
            total += v;
        }
        for (int w = w0; w < w1; ++w) {
            const int v = s_first[w];
            s_first[w] = run;
            run += v;
        }
        if (threadIdx.x == 0) s_first[a.walks] = total;
        __syncthreads();
        n_tiles = total;
    }
    // workgroups go to the XCDs in turn; the host makes the grid a multiple
    // of kXcds
    const int x = blockIdx.x % kXcds, per_x = max(1, static_cast<int>(gridDim.x) / kXcds);
    const int first = static_cast<int>(static_cast<int64_t>(n_tiles) * x / kXcds) + static_cast<int>(blockIdx.x) / kXcds;
    const int end = static_cast<int>(static_cast<int64_t>(n_tiles) * (x + 1) / kXcds);
    int pw = 0;                                // walk of the current tile (plan)
    if (plan && first < end) {
        int hi = a.walks;                      // s_first[pw] <= first < s_first[hi]
        while (hi - pw > 1) {
            const int mid = (pw + hi) >> 1;
            if (s_first[mid] <= first) pw = mid; else hi = mid;
        }
    }
    const int lvl = max(1, a.levels - t);       // the level of the step's candidates
    const bool stream = plan && static_cast<int64_t>(n_tiles) * kTile * 2 < a.nl[lvl] * a.pairs;
    auto tiles = [&](auto kstream) {
    for (int tile = first; tile < end; tile += per_x) {
        int w, start;
        if (t == 0) {
            w = tile / tiles0;
            start = (tile % tiles0) * kTile;
        } else if (plan) {
            while (s_first[pw + 1] <= tile) ++pw;
            w = __builtin_amdgcn_readfirstlane(pw);
            start = __builtin_amdgcn_readfirstlane((tile - s_first[pw]) * kTile);
        } else {
            const int2 e = a.tile_map[tile];
            w = __builtin_amdgcn_readfirstlane(e.x);
            start = __builtin_amdgcn_readfirstlane(e.y);
        }
        const int n = a.state[w].n;
        const int buf = a.state[w].buf;
        const int end_w = min(n, start + kTile);
        const int64_t pair = walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
        const uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * a.cand_cap +
                              static_cast<int64_t>(buf) * a.cand_cap;
        float *sc = a.score + static_cast<int64_t>(w) * a.cand_cap;
        float qv[row_epl<D, ST>()];
        load_q<D, QT, ST>(a, w, qv);
        uint32_t flags = 0;
        (void)score_wave<D, R, ST, true, false, decltype(kstream)::value>(a, pair, qv, cur, sc, start + wave * kU,
                                                                            end_w, kSW * kU, flags);
        if (flags && lane == 0) atomicOr(a.status, flags);
    }
    };
    if (stream)
        tiles(std::true_type{});
    else
        tiles(std::false_type{});
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
        if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t + 1, st.n))
            s_base = atomicAdd(&a.tile_count[t + 1], (st.n + kTile - 1) / kTile);
    }
    __syncthreads();
    // register the next step's tiles unless its cut needs no scores (or the
    // scorer counts them itself)
    if (!ls_tile_plan(a) && st.n > 0 && !step_forced(a, t + 1, st.n)) {
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
