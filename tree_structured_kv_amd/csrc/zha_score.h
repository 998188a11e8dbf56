// zha_score.h -- node scoring and the ordered opening of a cut, shared by
// the per-walk search engines (zha_search.hip) and the one-launch decode
// step (zha_fused.hip).
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "What does a node summarize?": a node's score for query q is
// the largest over references r of s <key_r, q> + bias_r.  "Run a small tree
// yourself": opened bottom-level nodes give their keys, other opened nodes
// give their children as the next candidates.
#pragma once

#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

// Nodes a launch itself has just made (the one-launch decode step appends
// before it searches): level l in 1..m has its new node j[l], whose record
// the workgroup keeps in LDS (k[l]: [R][D] of the summary type, b[l]: [R]).
struct FreshNodes {
    int m;
    int64_t j[ZHA_MAX_LEVELS + 1];
    const void *k[ZHA_MAX_LEVELS + 1];
    const float *b[ZHA_MAX_LEVELS + 1];
};

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
// With kStream the records come in through nontemporal (streaming) loads:
// for steps whose records the group's other heads are unlikely to read too.
template <int D, int R, typename ST, bool kScalarList, bool kFresh = false, bool kStream = false>
__device__ __forceinline__ float score_wave(const SearchArgs &a, int64_t pair,
                                            const float (&qv)[row_epl<D, ST>()],
                                            const uint32_t *cur, float *sc, int first, int end,
                                            int stride, uint32_t &flags,
                                            const FreshNodes *fresh = nullptr) {
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
            // the R biases: up to 8 come in through scalar loads (one set
            // per candidate in flight); with more, each lane loads its own
            // reference's (kU x 16 scalar values would not fit the SGPRs)
            constexpr bool kScalarBias = R <= 8;
            float bsr[kScalarBias ? R : 1];
            const float *bp = a.bet[lvl] + node * R;
            if (kFresh && lvl <= fresh->m && static_cast<int64_t>(id & kIndexMask) == fresh->j[lvl]) {
                // made by this launch: the workgroup's own copy in LDS
                kp = reinterpret_cast<const ST *>(fresh->k[lvl]);
                bp = fresh->b[lvl];
                if constexpr (kScalarBias) {
#pragma unroll
                    for (int r = 0; r < R; ++r) bsr[r] = bp[r];
                }
            } else if constexpr (kScalarBias) {
#pragma unroll
                for (int r = 0; r < R; ++r) bsr[r] = cload_f(bp + r);
            }
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const int r = l * RPL + rsub;
                if (r < R) {
                    if constexpr (EPL == 8 && kStream)
                        Vec16<ST>::load_nt(kp + r * D + EPL * sub, kv[u][l]);
                    else if constexpr (EPL == 8)
                        Vec16<ST>::load(kp + r * D + EPL * sub, kv[u][l]);
                    else if constexpr (kStream)
                        Vec4<ST>::load_nt(kp + r * D + EPL * sub, kv[u][l]);
                    else
                        Vec4<ST>::load(kp + r * D + EPL * sub, kv[u][l]);
                    if constexpr (kScalarBias) {
                        // this lane's reference r = l*RPL + rsub, chosen among SGPRs
                        float b = bsr[l * RPL];
#pragma unroll
                        for (int g = 1; g < RPL; ++g)
                            if (rsub == g && l * RPL + g < R) b = bsr[l * RPL + g];
                        bv[u][l] = b;
                    } else {
                        bv[u][l] = bp[r];
                    }
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
__device__ inline void open_cut(const SearchArgs &a, int n, const uint32_t *cur, const float *sc,
                         bool forced, unsigned long long tau, uint32_t *nxt, int32_t *selw,
                         int64_t sel_n, uint32_t &ta, uint32_t &tb, SelectShared &sh, int nxt_cap = -1) {
    const int tid = threadIdx.x;
    const int c = a.chunk, log2c = a.log2c, cap = nxt_cap >= 0 ? nxt_cap : a.cand_cap;
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

}  // namespace zha
