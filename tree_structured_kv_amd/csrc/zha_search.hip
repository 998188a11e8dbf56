// zha_search.hip -- top-down tree walk for decode queries.
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
// GPU design: one workgroup (4 wavefronts) per walk, the level loop inside
// the kernel, no host round trip.  A candidate's R keys are one contiguous
// R*D*4-byte record; a wavefront reads it with 16-byte loads (D/4 lanes per
// reference), reduces the dot products across lanes and takes the max over
// references.  The cut is an exact radix select over 64-bit rank keys
// (ordered score bits, then the complement of the span start, so equal
// scores open in span order).  For top-p the softmax masses are integers
// (exp(score - max) scaled by 2^31 and rounded), so every sum is exact and
// the cut is bit-reproducible.  Opened nodes are compacted in candidate
// order, which keeps every candidate list in span order without a sort.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

constexpr int kWaves = kBlock / 64;
constexpr float kMassScale = 2147483648.0f;  // 2^31

__device__ __forceinline__ uint64_t rank_key(float score, uint32_t id, int log2c) {
    const uint32_t lvl = id >> kLevelShift;
    const uint32_t j = id & kIndexMask;
    const uint32_t start = j << (log2c * lvl);
    return (static_cast<uint64_t>(ordered_bits(score)) << 32) |
           static_cast<uint64_t>(0xffffffffu - start);
}

struct SelectShared {
    uint32_t hcnt[256];
    unsigned long long hw[256];
    unsigned long long scan64[kWaves];
    unsigned long long tau;
    unsigned long long need;
    unsigned long long above;
    uint32_t dig;
    uint32_t cnt;
    float red[kWaves];
    uint32_t flags;
};

// Block-wide exclusive scan of a uint64 per thread; returns the prefix and
// writes the total to *total.
__device__ __forceinline__ unsigned long long block_exscan64(unsigned long long v,
                                                             unsigned long long *scratch,
                                                             unsigned long long *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        unsigned long long o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
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

}  // namespace

template <int D, int R, typename QT>
__global__ __launch_bounds__(kBlock) void k_search_decode(SearchArgs a) {
    constexpr int LPR = D / 4;            // lanes per reference row (float4 each)
    constexpr int RPL = 64 / LPR;         // references per 64-lane load
    constexpr int NL = (R + RPL - 1) / RPL;
    constexpr int U = 2;                  // candidates in flight per wavefront

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    if (w >= a.walks) return;
    const int b = w / a.heads, h = w % a.heads, g = h / a.group;
    const int64_t pair = static_cast<int64_t>(b) * a.kv_heads + g;
    const int c = a.chunk, log2c = a.log2c, L = a.levels;
    const float s = a.sharpness;
    const int cap = a.cand_cap;

    __shared__ SelectShared sh;
    __shared__ int32_t s_scored[ZHA_MAX_STEPS], s_opened[ZHA_MAX_STEPS];
    if (tid == 0) sh.flags = 0;

    // this lane's 4 query elements
    const int sub = lane % LPR, rsub = lane / LPR;
    float qv[4];
    {
        const QT *qp = static_cast<const QT *>(a.q) + static_cast<int64_t>(w) * D + 4 * sub;
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[e] = Elem<QT>::load(qp, e);
    }

    uint32_t *cur = a.cand + static_cast<int64_t>(w) * 2 * cap;
    uint32_t *nxt = cur + cap;
    float *sc = a.score + static_cast<int64_t>(w) * cap;
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;

    // Roots: every level-L node, then the nodes of lower levels whose parent
    // chunk is not full yet, in span order.
    uint32_t flags = 0;
    int64_t n_roots = 0;
    for (int l = L; l >= 1; --l) {
        const int64_t first = (l == L) ? 0 : static_cast<int64_t>(c) * a.nl[l + 1];
        const int64_t cnt = a.nl[l] - first;
        for (int64_t i = tid; i < cnt; i += kBlock) {
            const int64_t pos = n_roots + i;
            if (pos < cap) cur[pos] = (static_cast<uint32_t>(l) << kLevelShift) | static_cast<uint32_t>(first + i);
        }
        n_roots += cnt;
    }
    if (n_roots > cap) { flags |= ZHA_FLAG_CAND_OVERFLOW; n_roots = cap; }
    int n = static_cast<int>(n_roots);
    __syncthreads();

    int64_t sel_n = 0;
    int32_t unforced = 0;
    int t = 0;
    for (; t < ZHA_MAX_STEPS && n > 0; ++t) {
        const int kt = a.k[t];
        const bool forced = (n == 1) || (a.mode == ZHA_TOPK && kt >= n) ||
                            (a.mode == ZHA_TOPP && a.p >= 1.0f);
        unsigned long long tau = 0;
        if (!forced) {
            // ---- score every candidate ----------------------------------
            float wmax = -INFINITY;
            for (int base = wave * U; base < n; base += kWaves * U) {
                float4 kv[U][NL];
                float bv[U][NL];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = base + u;
                    const uint32_t id = (i < n) ? cur[i] : cur[base];
                    const int lvl = static_cast<int>(id >> kLevelShift);
                    const int64_t node = pair * a.cap[lvl] + static_cast<int64_t>(id & kIndexMask);
                    const float *kp = a.kap[lvl] + node * (R * D);
                    const float *bp = a.bet[lvl] + node * R;
#pragma unroll
                    for (int l = 0; l < NL; ++l) {
                        const int r = l * RPL + rsub;
                        if (r < R) {
                            kv[u][l] = *reinterpret_cast<const float4 *>(kp + r * D + 4 * sub);
                            bv[u][l] = bp[r];
                        } else {
                            kv[u][l] = make_float4(0.f, 0.f, 0.f, 0.f);
                            bv[u][l] = -INFINITY;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float best = -INFINITY;
#pragma unroll
                    for (int l = 0; l < NL; ++l) {
                        float d = kv[u][l].x * qv[0];
                        d = fmaf(kv[u][l].y, qv[1], d);
                        d = fmaf(kv[u][l].z, qv[2], d);
                        d = fmaf(kv[u][l].w, qv[3], d);
                        d = wave_sum(d, LPR);
                        const float v = fmaf(s, d, bv[u][l]);
                        best = fmaxf(best, v);
                    }
                    best = wave_max(best, LPR, 64);
                    if (best != best) { best = -INFINITY; flags |= ZHA_FLAG_NONFINITE; }
                    if (best == 0.f) best = 0.f;          // one zero
                    const int i = base + u;
                    if (i < n) {
                        if (lane == 0) sc[i] = best;
                        wmax = fmaxf(wmax, best);
                    }
                }
            }
            if (lane == 0) sh.red[wave] = wmax;
            __syncthreads();
            float mx = sh.red[0];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) mx = fmaxf(mx, sh.red[i]);

            // ---- cut target ----------------------------------------------
            const bool by_mass = (a.mode == ZHA_TOPP) && (a.p > 0.f);
            const bool flat = !(mx > -INFINITY);   // every score -inf: equal masses
            unsigned long long target;
            if (by_mass) {
                unsigned long long zpart = 0;
                for (int i = tid; i < n; i += kBlock) {
                    const float e = flat ? 1.f : expf(sc[i] - mx);
                    zpart += static_cast<unsigned long long>(__float2uint_rn(e * kMassScale));
                }
                unsigned long long z;
                (void)block_exscan64(zpart, sh.scan64, &z);
                double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
                target = static_cast<unsigned long long>(tq);
                if (target < 1) target = 1;
                if (target > z) target = z;
            } else {
                const int m = (a.mode == ZHA_TOPK) ? (kt < n ? kt : n) : 1;
                target = static_cast<unsigned long long>(m < 1 ? 1 : m);
            }

            // ---- radix select of the crossing rank key ---------------------
            unsigned long long prefix = 0, need = target;
            bool found = false;
            for (int pass = 0; pass < 8 && !found; ++pass) {
                const int shift = 56 - 8 * pass;
                for (int i = tid; i < 256; i += kBlock) { sh.hcnt[i] = 0; sh.hw[i] = 0; }
                __syncthreads();
                for (int i = tid; i < n; i += kBlock) {
                    const float scv = sc[i];
                    const unsigned long long key = rank_key(scv, cur[i], log2c);
                    if (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8))) {
                        const uint32_t dg = static_cast<uint32_t>(key >> shift) & 255u;
                        unsigned long long wgt = 1;
                        if (by_mass) {
                            const float e = flat ? 1.f : expf(scv - mx);
                            wgt = static_cast<unsigned long long>(__float2uint_rn(e * kMassScale));
                        }
                        atomicAdd(&sh.hcnt[dg], 1u);
                        if (wgt) atomicAdd(&sh.hw[dg], wgt);
                    }
                }
                __syncthreads();
                if (wave == 0) {
                    // lane covers digits 255-4*lane .. 252-4*lane (descending)
                    unsigned long long lw[4], lsum = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { lw[e] = sh.hw[255 - 4 * lane - e]; lsum += lw[e]; }
                    unsigned long long incl = lsum;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        unsigned long long o = __shfl_up(incl, off, 64);
                        if (lane >= off) incl += o;
                    }
                    const unsigned long long excl = incl - lsum;
                    unsigned long long mask = __ballot(incl >= need);
                    int first = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : 63;
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
                if (sh.cnt <= 1 || pass == 7) {
                    if (pass == 7) {
                        tau = prefix;
                    } else {
                        // exactly one key carries this prefix: fetch it
                        for (int i = tid; i < n; i += kBlock) {
                            const unsigned long long key = rank_key(sc[i], cur[i], log2c);
                            if ((key >> shift) == (prefix >> shift)) sh.tau = key;
                        }
                        __syncthreads();
                        tau = (sh.cnt == 0) ? 0ull : sh.tau;
                    }
                    found = true;
                }
                __syncthreads();
            }
            unforced += n;
        }

        // ---- open: compact in candidate (span) order ------------------------
        const int per = (n + kBlock - 1) / kBlock;
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
        const uint32_t ta = static_cast<uint32_t>(tot >> 32), tb = static_cast<uint32_t>(tot);
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
        if (tid == 0) {
            s_scored[t] = n;
            s_opened[t] = static_cast<int32_t>(ta + tb);
        }
        sel_n += ta;
        int64_t nn = static_cast<int64_t>(tb) * c;
        if (nn > cap) { flags |= ZHA_FLAG_CAND_OVERFLOW; nn = cap; }
        uint32_t *tmp = cur; cur = nxt; nxt = tmp;
        n = static_cast<int>(nn);
        __syncthreads();
    }
    if (sel_n > a.sel_cap) flags |= ZHA_FLAG_SEL_OVERFLOW;

    // ---- outputs ------------------------------------------------------------
    if (flags) atomicOr(&sh.flags, flags);
    __syncthreads();
    if (tid == 0) {
        const uint32_t fl = sh.flags;
        a.sel_count[w] = static_cast<int32_t>(sel_n < a.sel_cap ? sel_n : a.sel_cap);
        if (fl) atomicOr(a.status, fl);
        if (a.stats) {
            zha_walk_stats st;
            int64_t tot_scored = 0;
            for (int i = 0; i < ZHA_MAX_STEPS; ++i) {
                st.scored[i] = i < t ? s_scored[i] : 0;
                st.opened[i] = i < t ? s_opened[i] : 0;
                if (i < t) tot_scored += s_scored[i];
            }
            const int64_t tail = a.n_tokens - static_cast<int64_t>(c) * a.nl[1];
            st.steps = t;
            st.keys_read = static_cast<int32_t>(sel_n * c + tail);
            st.blocks = static_cast<int32_t>(sel_n);
            st.unforced_scored = unforced;
            st.comparisons = tot_scored * R + st.keys_read;
            st.flags = fl;
            st.reserved = 0;
            a.stats[w] = st;
        }
    }
}

template <int D, typename QT>
static hipError_t launch_search_d(const SearchArgs &a, int R, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(a.walks));
    switch (R) {
        case 1: hipLaunchKernelGGL((k_search_decode<D, 1, QT>), grid, dim3(kBlock), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_search_decode<D, 2, QT>), grid, dim3(kBlock), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_search_decode<D, 4, QT>), grid, dim3(kBlock), 0, st, a); break;
        case 8: hipLaunchKernelGGL((k_search_decode<D, 8, QT>), grid, dim3(kBlock), 0, st, a); break;
        case 16: hipLaunchKernelGGL((k_search_decode<D, 16, QT>), grid, dim3(kBlock), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_search(const SearchArgs &a, int D, int R, int dtype, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_search_d<64, bf16_t>(a, R, st)
                                 : launch_search_d<64, float>(a, R, st);
    return dtype == ZHA_BF16 ? launch_search_d<128, bf16_t>(a, R, st)
                             : launch_search_d<128, float>(a, R, st);
}

}  // namespace zha
