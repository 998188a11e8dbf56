// zha_walk.h -- walk helpers shared by the search engines of libzha.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works"; the walk itself is described in its section "Run a small tree
// yourself", the cut in "How does top-p differ from top-K?".
#pragma once

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

constexpr float kMassScale = 2147483648.0f;  // 2^31: integer softmax masses

// e^x for the integer masses of a cut (x = score - max <= 0): one hardware
// exp2 of x*log2(e).  Every cut takes its masses from this one function, so
// equal scores give equal masses everywhere; it is not the libm expf.
__device__ __forceinline__ float mass_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// 64-bit rank key of a candidate: ordered score bits, then the complement of
// its span start, so that equal scores rank in span order.
__device__ __forceinline__ uint64_t rank_key(float score, uint32_t id, int log2c) {
    const uint32_t lvl = id >> kLevelShift;
    const uint32_t j = id & kIndexMask;
    const uint32_t start = j << (log2c * lvl);
    return (static_cast<uint64_t>(ordered_bits(score)) << 32) |
           static_cast<uint64_t>(0xffffffffu - start);
}

// A step whose cut needs no scores: one candidate, K at least the list, or
// p >= 1 (every candidate opens).
__device__ __forceinline__ bool step_forced(const SearchArgs &a, int t, int n) {
    return (n <= 1) || (a.mode == ZHA_TOPK && a.k[t] >= n) || (a.mode == ZHA_TOPP && a.p >= 1.0f);
}

// Whether the level-synchronous scorer counts each walk's tiles itself from
// the walk states (else the kernel that sets a walk's next list registers
// its tiles in tile_map).
__device__ __forceinline__ bool ls_tile_plan(const SearchArgs &a) { return a.walks <= kPlanWalks; }

// Workgroup: the roots -- every level-L node, then the nodes of lower levels
// whose parent chunk is not full yet, in span order.  Returns their number
// (clamped to the candidate capacity).
__device__ __forceinline__ int write_roots(const SearchArgs &a, uint32_t *cur, uint32_t &flags) {
    const int tid = threadIdx.x, c = a.chunk, L = a.levels, cap = a.cand_cap;
    int64_t n_roots = 0;
    for (int l = L; l >= 1; --l) {
        const int64_t first = (l == L) ? 0 : static_cast<int64_t>(c) * a.nl[l + 1];
        const int64_t cnt = a.nl[l] - first;
        for (int64_t i = tid; i < cnt; i += blockDim.x) {
            const int64_t pos = n_roots + i;
            if (pos < cap) cur[pos] = (static_cast<uint32_t>(l) << kLevelShift) | static_cast<uint32_t>(first + i);
        }
        n_roots += cnt;
    }
    if (n_roots > cap) { flags |= ZHA_FLAG_CAND_OVERFLOW; n_roots = cap; }
    return static_cast<int>(n_roots);
}

// One thread: sel_count, status and the per-walk statistics.
template <int R>
__device__ __forceinline__ void finish_walk(const SearchArgs &a, int w, int steps, const int32_t *scored,
                            const int32_t *opened, int64_t sel_n, int32_t unforced, uint32_t fl) {
    if (sel_n > a.sel_cap) fl |= ZHA_FLAG_SEL_OVERFLOW;
    a.sel_count[w] = static_cast<int32_t>(sel_n < a.sel_cap ? sel_n : a.sel_cap);
    if (fl & kFlagBits) atomicOr(a.status, fl & kFlagBits);
    if (a.stats) {
        zha_walk_stats st;
        int64_t tot_scored = 0;
        for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
            st.scored[i] = i < steps ? scored[i] : 0;
            st.opened[i] = i < steps ? opened[i] : 0;
            if (i < steps) tot_scored += scored[i];
        }
        const int64_t tail = a.n_tokens - static_cast<int64_t>(a.chunk) * a.nl[1];
        st.steps = steps;
        st.keys_read = static_cast<int32_t>(sel_n * a.chunk + tail);
        st.blocks = static_cast<int32_t>(sel_n);
        st.unforced_scored = unforced;
        st.comparisons = tot_scored * R + st.keys_read;
        st.flags = fl & kFlagBits;
        st.paths = fl >> kPathShift;
        a.stats[w] = st;
    }
}

constexpr int kThreads = 512;          // workgroup of the cut kernels
constexpr int kWaves = kThreads / 64;
constexpr int kScanU = 4;              // list entries in flight per thread in a scan

constexpr int kWinPasses = 4;          // value-window passes of the fast cut
constexpr int kWinFinal = 64;          // candidates ranked one by one at its end

struct SelectShared {
    uint32_t hcnt[256];
    unsigned long long hw[256];
    unsigned long long scan64[kWaves];
    unsigned long long tau;
    unsigned long long above;
    uint32_t dig;
    uint32_t cnt;
    float red[kWaves];
    uint32_t flags;
    // fast cut: the last window's candidates (key, weight), then in key order
    unsigned long long fkey[kWinFinal];
    unsigned long long fw[kWinFinal];
    unsigned long long skey[kWinFinal];
    unsigned long long sw[kWinFinal];
    uint32_t nf;
};

// Block-wide exclusive scan of a uint64 per thread (kThreads threads);
// returns the prefix and writes the total to *total.
__device__ __forceinline__ unsigned long long block_exscan64(unsigned long long v,
                                                             unsigned long long *scratch,
                                                             unsigned long long *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long incl = wave_scan_u64(v);
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    unsigned long long base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        unsigned long long x = scratch[w];
        if (w < wave) base += x;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// Workgroup (kThreads): the rank key of the candidate at the cut of a step
// that is not forced; every candidate with a key >= it opens.
// With `mask` non-null only entries i with (mask[i] & bit) are candidates
// (the union engine's per-head view of a pair's list); `n` is then the
// length of the list and `cnt` the number of candidates.  `cur` gives the
// candidates' node ids by index: an array, or an accessor that finds them
// (cur[i]).
template <int U = kScanU, typename Ids>
__device__ __forceinline__ unsigned long long cut_tau(const SearchArgs &a, int n, Ids cur,
                                                      const float *sc, float mx, int kt, SelectShared &sh,
                                                      const uint32_t *mask = nullptr, uint32_t bit = 0,
                                                      int cnt = -1) {
    if (cnt < 0) cnt = n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int log2c = a.log2c;
    const bool by_mass = (a.mode == ZHA_TOPP) && (a.p > 0.f);
    const bool flat = !(mx > -INFINITY);   // every score -inf: equal masses
    unsigned long long target;
    if (by_mass) {
        unsigned long long zpart = 0;
        for (int i0 = tid; i0 < n; i0 += U * kThreads) {
            bool in[U];
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                in[u] = i < n && (!mask || (mask[i] & bit));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = in[u] ? sc[i0 + u * kThreads] : 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!in[u]) continue;
                const float e = flat ? 1.f : mass_exp(v[u] - mx);
                zpart += static_cast<unsigned long long>(__float2uint_rn(e * kMassScale));
            }
        }
        unsigned long long z;
        (void)block_exscan64(zpart, sh.scan64, &z);
        const double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
        target = static_cast<unsigned long long>(tq);
        if (target < 1) target = 1;
        if (target > z) target = z;
    } else {
        const int m = (a.mode == ZHA_TOPK) ? (kt < cnt ? kt : cnt) : 1;
        target = static_cast<unsigned long long>(m < 1 ? 1 : m);
    }

    unsigned long long prefix = 0, need = target, tau = 0;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 256; i += kThreads) { sh.hcnt[i] = 0; sh.hw[i] = 0; }
        __syncthreads();
        for (int i0 = tid; i0 < n; i0 += U * kThreads) {
            bool in[U];
            float v[U];
            uint32_t idv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                in[u] = i < n && (!mask || (mask[i] & bit));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                v[u] = in[u] ? sc[i] : 0.f;
                idv[u] = in[u] ? cur[i] : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!in[u]) continue;
                const unsigned long long key = rank_key(v[u], idv[u], log2c);
                if (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8))) {
                    const uint32_t dg = static_cast<uint32_t>(key >> shift) & 255u;
                    unsigned long long wgt = 1;
                    if (by_mass) {
                        const float e = flat ? 1.f : mass_exp(v[u] - mx);
                        wgt = static_cast<unsigned long long>(__float2uint_rn(e * kMassScale));
                    }
                    atomicAdd(&sh.hcnt[dg], 1u);
                    if (wgt) atomicAdd(&sh.hw[dg], wgt);
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane covers digits 255-4*lane .. 252-4*lane (descending)
            unsigned long long lw[4], lsum = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { lw[e] = sh.hw[255 - 4 * lane - e]; lsum += lw[e]; }
            unsigned long long incl = wave_scan_u64(lsum);
            const unsigned long long excl = incl - lsum;
            const unsigned long long mask = __ballot(incl >= need);
            const int first = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : 63;
            if (lane == first) {
                unsigned long long run = excl;
                int pick = 3;
                for (int e = 0; e < 4; ++e) {
                    if (run + lw[e] >= need) { pick = e; break; }
                    run += lw[e];
                }
                if (!mask) { pick = 3; run = excl + lw[0] + lw[1] + lw[2]; }
                const uint32_t dg = 255u - 4u * lane - pick;
                sh.dig = dg;
                sh.above = run;
                sh.cnt = sh.hcnt[dg];
            }
        }
        __syncthreads();
        prefix |= static_cast<unsigned long long>(sh.dig) << shift;
        need -= sh.above;
        const uint32_t cnt = sh.cnt;
        if (pass == 7) {
            tau = prefix;
            break;
        }
        if (cnt <= 1) {
            // at most one key carries this prefix: fetch it
            for (int i = tid; i < n; i += kThreads) {
                if (mask && !(mask[i] & bit)) continue;
                const unsigned long long key = rank_key(sc[i], cur[i], log2c);
                if ((key >> shift) == (prefix >> shift)) sh.tau = key;
            }
            __syncthreads();
            tau = (cnt == 0) ? 0ull : sh.tau;
            __syncthreads();
            break;
        }
        __syncthreads();
    }
    return tau;
}

// Wavefront, at most 64 candidates, one per lane (key 0 and weight 0 on the
// other lanes): the cut key of cut_tau -- the rank key of the candidate at
// which the weight summed in decreasing key order first reaches what the
// step needs (weights and need exactly as there) -- by a bitonic sort of the
// (key, weight) pairs across the lanes (keys are distinct: they hold the
// span start), an inclusive scan of the weights and a ballot.
__device__ __forceinline__ unsigned long long lane_tau(const SearchArgs &a, bool in, float v, uint32_t id, float mx, int n, int kt) {
    const int lane = threadIdx.x & 63;
    const bool by_mass = (a.mode == ZHA_TOPP) && (a.p > 0.f);
    const bool flat = !(mx > -INFINITY);   // every score -inf: equal masses
    uint32_t wt = 0u;
    if (in) wt = by_mass ? __float2uint_rn((flat ? 1.f : mass_exp(v - mx)) * kMassScale) : 1u;
    unsigned long long key = in ? rank_key(v, id, a.log2c) : 0ull;
    unsigned long long need;
    if (by_mass) {
        const unsigned long long z = wave_total_u64(wt);
        const double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
        need = static_cast<unsigned long long>(tq);
        if (need < 1) need = 1;
        if (need > z) need = z;
    } else {
        const int m = (a.mode == ZHA_TOPK) ? (kt < n ? kt : n) : 1;
        need = static_cast<unsigned long long>(m < 1 ? 1 : m);
    }
    // descending bitonic sort over the 64 lanes
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const unsigned long long ok = xor_lane64_n(key, j);
            const uint32_t ow = xor_lane_n(wt, j);
            const bool lower = (lane & j) == 0, desc = (lane & k) == 0;
            const bool take = (lower == desc) ? (ok > key) : (ok < key);
            if (take) {
                key = ok;
                wt = ow;
            }
        }
    }
    unsigned long long incl = wave_scan_u64(wt);
    const unsigned long long hit = __ballot(lane < n && incl >= need);
    const int first = hit ? (__ffsll(static_cast<long long>(hit)) - 1) : (n - 1);
    return read_lane64(key, first);
}

// Bin of score v in a window of 256 bins counted down from `top` (bin 0
// holds the highest scores; values below the window fall in bin 255).
// Monotone: a higher score never lands in a higher bin.
__device__ __forceinline__ int win_bin(float v, float top, float scale) {
    float d = (top - v) * scale;
    d = fminf(fmaxf(d, 0.f), 255.f);
    return static_cast<int>(d);
}

// Workgroup (kThreads): the same key as cut_tau, found by narrowing a
// window of score values instead of key digits.  Each pass bins the
// candidates still in the window (bin membership of every earlier pass is
// re-tested exactly, so no float boundary is ever recomputed), takes the
// bin where the running weight from the top crosses what is still needed,
// and stops once that bin holds at most kWinFinal candidates; those are then
// ranked by their full keys.  Weights are the integer masses of cut_tau (or
// counts), so the crossing is the same candidate.  Scores spread over the
// bins, so the shared-memory histogram sees little contention.  Falls back
// to cut_tau when every score is -inf or a window cannot be split (ties);
// that fallback ORs kPathTieSelect into *path (every thread's copy).
template <int U = kScanU, typename Ids>
__device__ __forceinline__ unsigned long long cut_tau_win(const SearchArgs &a, int n, Ids cur,
                                                          const float *sc, float mx, int kt, SelectShared &sh,
                                                          uint32_t *path = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int log2c = a.log2c;
    if (!(mx > -INFINITY)) {
        if (path) *path |= kPathTieSelect;
        return cut_tau<U>(a, n, cur, sc, mx, kt, sh);
    }
    if (n <= 64) {
        // one candidate per lane of wavefront 0: the sort-based cut
        if (wave == 0) {
            const bool in = lane < n;
            const float v = in ? sc[lane] : -INFINITY;
            const uint32_t id = in ? cur[lane] : 0u;
            const unsigned long long k = lane_tau(a, in, v, id, mx, n, kt);
            if (lane == 0) sh.tau = k;
        }
        __syncthreads();
        const unsigned long long tau = sh.tau;
        __syncthreads();
        return tau;
    }
    const bool by_mass = (a.mode == ZHA_TOPP) && (a.p > 0.f);
    // total weight and the lowest finite score
    unsigned long long zpart = 0;
    float mn = mx;
    for (int i0 = tid; i0 < n; i0 += U * kThreads) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kThreads;
            v[u] = i < n ? sc[i] : mx;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v[u] > -INFINITY) mn = fminf(mn, v[u]);
            if (by_mass && i0 + u * kThreads < n)
                zpart += static_cast<unsigned long long>(__float2uint_rn(mass_exp(v[u] - mx) * kMassScale));
        }
    }
    mn = -wave_max(-mn, 1, 64);
    if (lane == 0) sh.red[wave] = mn;
    unsigned long long z;
    (void)block_exscan64(zpart, sh.scan64, &z);    // barriers: sh.red is complete
#pragma unroll
    for (int i = 0; i < kWaves; ++i) mn = fminf(mn, sh.red[i]);
    __syncthreads();
    unsigned long long need;
    if (by_mass) {
        const double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
        need = static_cast<unsigned long long>(tq);
        if (need < 1) need = 1;
        if (need > z) need = z;
    } else {
        const int m = (a.mode == ZHA_TOPK) ? (kt < n ? kt : n) : 1;
        need = static_cast<unsigned long long>(m < 1 ? 1 : m);
    }
    // scores more than 23 below the top carry integer mass 0 and can never
    // be the crossing candidate of a mass cut
    float top = mx, bot = by_mass ? fmaxf(mn, mx - 23.f) : mn;
    float w_top[kWinPasses], w_scale[kWinPasses];
    int w_bin[kWinPasses];
    int depth = 0;
    bool done = false;
    for (; depth < kWinPasses; ++depth) {
        if (!(top > bot)) break;                   // the window is a single value: ties
        const float scale = 256.f / (top - bot);
        w_top[depth] = top;
        w_scale[depth] = scale;
        for (int i = tid; i < 256; i += kThreads) { sh.hcnt[i] = 0; sh.hw[i] = 0; }
        __syncthreads();
        for (int i0 = tid; i0 < n; i0 += U * kThreads) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                v[u] = i < n ? sc[i] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i0 + u * kThreads >= n) continue;
                bool in = true;
                for (int q = 0; q < depth; ++q) in = in && win_bin(v[u], w_top[q], w_scale[q]) == w_bin[q];
                if (!in) continue;
                const int b = win_bin(v[u], top, scale);
                unsigned long long wgt = 1;
                if (by_mass) wgt = static_cast<unsigned long long>(__float2uint_rn(mass_exp(v[u] - mx) * kMassScale));
                atomicAdd(&sh.hcnt[b], 1u);
                if (wgt) atomicAdd(&sh.hw[b], wgt);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane covers bins 4*lane .. 4*lane+3 (ascending = scores descending)
            unsigned long long lw[4], lsum = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { lw[e] = by_mass ? sh.hw[4 * lane + e] : sh.hcnt[4 * lane + e]; lsum += lw[e]; }
            unsigned long long incl = wave_scan_u64(lsum);
            const unsigned long long excl = incl - lsum;
            const unsigned long long mask = __ballot(incl >= need);
            const int first = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : 63;
            if (lane == first) {
                unsigned long long run = excl;
                int pick = 3;
                for (int e = 0; e < 4; ++e) {
                    if (run + lw[e] >= need) { pick = e; break; }
                    run += lw[e];
                }
                if (!mask) { pick = 3; run = excl + lw[0] + lw[1] + lw[2]; }
                sh.dig = 4u * lane + pick;
                sh.above = run;
                sh.cnt = sh.hcnt[4 * lane + pick];
            }
        }
        __syncthreads();
        const int b = static_cast<int>(sh.dig);
        need -= sh.above;
        w_bin[depth] = b;
        const uint32_t cb = sh.cnt;
        __syncthreads();
        if (cb <= static_cast<uint32_t>(kWinFinal)) { ++depth; done = true; break; }
        // the next window spans bin b (membership is still decided by the
        // exact bin tests above; these bounds only spread the next pass)
        const float nt = top - static_cast<float>(b) / scale;
        const float nb = top - static_cast<float>(b + 1) / scale;
        top = fminf(nt, top);
        bot = fmaxf(nb, bot);
    }
    if (!done) {
        if (path) *path |= kPathTieSelect;
        return cut_tau<U>(a, n, cur, sc, mx, kt, sh);
    }

    // the final bin's candidates, ranked by key
    if (tid == 0) sh.nf = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const float v = sc[i];
        bool in = true;
        for (int q = 0; q < depth; ++q) in = in && win_bin(v, w_top[q], w_scale[q]) == w_bin[q];
        if (!in) continue;
        const uint32_t slot = atomicAdd(&sh.nf, 1u);
        if (slot < static_cast<uint32_t>(kWinFinal)) {
            sh.fkey[slot] = rank_key(v, cur[i], log2c);
            sh.fw[slot] = by_mass ? static_cast<unsigned long long>(__float2uint_rn(mass_exp(v - mx) * kMassScale)) : 1ull;
        }
    }
    __syncthreads();
    const int nf = static_cast<int>(sh.nf < static_cast<uint32_t>(kWinFinal) ? sh.nf : kWinFinal);
    if (tid < nf) {
        const unsigned long long k = sh.fkey[tid];
        int r = 0;
        for (int j = 0; j < nf; ++j) r += sh.fkey[j] > k;
        sh.skey[r] = k;
        sh.sw[r] = sh.fw[tid];
    }
    __syncthreads();
    if (wave == 0) {
        // the first rank whose running weight reaches what is still needed
        // (kWinFinal = one per lane): a scan and a ballot
        const unsigned long long wv = lane < nf ? sh.sw[lane] : 0ull;
        unsigned long long incl = wave_scan_u64(wv);
        const unsigned long long hit = __ballot(lane < nf && incl >= need);
        const int r = hit ? (__ffsll(static_cast<long long>(hit)) - 1) : nf - 1;
        if (lane == 0) sh.tau = nf > 0 ? sh.skey[r] : 0ull;
    }
    __syncthreads();
    const unsigned long long tau = sh.tau;
    __syncthreads();
    return tau;
}

__device__ __forceinline__ float block_max(float v, SelectShared &sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v, 1, 64);
    if (lane == 0) sh.red[wave] = v;
    __syncthreads();
    float m = sh.red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = fmaxf(m, sh.red[i]);
    __syncthreads();
    return m;
}

}  // namespace zha
