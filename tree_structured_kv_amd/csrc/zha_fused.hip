// zha_fused.hip -- one decode step in one launch: the append of the new
// token, the walk, and attention over the walk's selection.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".
//   "How is the tree built?": a node is made only when its chunk fills, so a
//     one-token append makes at most one node per level (levels 1..m where
//     c^m divides the new length), each from c children of which the last
//     is the node made just below it.
//   "Run a small tree yourself", "How does top-p differ from top-K?": the
//     walk (the persistent engine's step loop: score, one softmax over the
//     step's candidates, cut, open).
//   "Common misunderstandings": every query head walks on its own and then
//     attends exactly the original keys it chose.
//
// GPU design.  One workgroup (8 wavefronts) per walk and no cooperation
// between workgroups, so nothing waits on another workgroup and any number
// of them may be resident.  The nodes the append makes are computed by every
// workgroup of the pair into its own LDS, with the very code the build
// kernels use (leaf_node, upper_node: the same bits), and the pair's first
// walk also writes them to the tree; the walk scores a node made by this
// launch from its LDS copy, every other node from HBM.  The attention then
// streams the walk's selected blocks and the raw tail: a key row is read by
// D*e/16 lanes with 16-byte loads, every lane group keeps its own online
// softmax (max, sum, weighted V slice) and the groups and wavefronts are
// merged at the end.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_score.h"
#include "zha_summary.h"
#include "zha_walk.h"

namespace zha {

namespace {

constexpr int kFU = 2;   // key rows in flight per lane group (attention)

__device__ __forceinline__ float lane_group_sum(float v, int width) {
#pragma unroll
    for (int off = 1; off < width; off <<= 1) v += xor_lane_f(v, off);
    return v;
}

// Merge the online-softmax state (m, l, acc) with the one `off` lanes away.
template <int EPL>
__device__ __forceinline__ void merge_shfl(float &m, float &l, float (&acc)[EPL], int off) {
    const float m2 = xor_lane_f(m, off);
    const float l2 = xor_lane_f(l, off);
    const float mm = fmaxf(m, m2);
    const float c1 = (m > -INFINITY) ? expf(m - mm) : 0.f;
    const float c2 = (m2 > -INFINITY) ? expf(m2 - mm) : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float a2 = xor_lane_f(acc[e], off);
        acc[e] = acc[e] * c1 + a2 * c2;
    }
    l = l * c1 + l2 * c2;
    m = mm;
}

}  // namespace

template <int D, int R, typename KT, typename ST>
__global__ __launch_bounds__(kThreads) void k_step_fused(FusedArgs f) {
    const SearchArgs &a = f.s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x;
    if (w >= a.walks) return;
    const int64_t pair = walk_pair(w, 1, a.heads, a.group, a.kv_heads);
    const int g = static_cast<int>(pair % a.kv_heads);
    const int c = a.chunk, cap = a.cand_cap;
    const float s = a.sharpness;
    const bool leader = (w % a.group) == 0;   // the pair's first query head

    extern __shared__ float lds[];
    __shared__ SelectShared sh;
    __shared__ int32_t s_scored[ZHA_MAX_STEPS], s_opened[ZHA_MAX_STEPS];
    __shared__ float s_sig[64];
    if (tid == 0) sh.flags = 0;

    // ---- 1. the nodes this append makes (levels 1..m), into LDS ----------------
    constexpr int P = D + 4;
    constexpr int RECF = (R * D * static_cast<int>(sizeof(ST)) + 15) / 16 * 4;   // key record, floats
    constexpr int RECS = (RECF + R + 3) & ~3;                                     // + biases, 16-byte aligned
    float *rho = lds;                         // [R][P]   references (leaf_node)
    float *kk = rho + R * P;                  // [c][P]   the chunk's keys
    float *wt = kk + c * P;                   // [R][c]
    float *mx_s = wt + c * R;                 // [R]
    float *z_s = mx_s + R;                    // [R]
    float *recs = lds + ((R * P + c * P + c * R + 2 * R + 3) & ~3);   // per level: key record, then R biases
    __shared__ FreshNodes fr;                 // read at uniform addresses (LDS broadcast)
    if (tid <= ZHA_MAX_LEVELS) {
        const int l = tid;
        const bool made = l >= 1 && l <= f.fresh_m;
        if (l == 0) fr.m = f.fresh_m;
        fr.j[l] = made ? a.nl[l] - 1 : -1;
        fr.k[l] = made ? recs + (l - 1) * RECS : nullptr;
        fr.b[l] = made ? recs + (l - 1) * RECS + RECF : nullptr;
    }
    __syncthreads();
    const float *refs = f.refs + static_cast<int64_t>(g) * R * D;
    if (f.fresh_m > 0) {
        for (int idx = tid; idx < R * (D / 4); idx += kThreads) {
            const int r = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
            *reinterpret_cast<float4 *>(rho + r * P + d4) = *reinterpret_cast<const float4 *>(refs + r * D + d4);
        }
        __syncthreads();
        for (int l = 1; l <= f.fresh_m; ++l) {
            ST *ok = reinterpret_cast<ST *>(const_cast<void *>(fr.k[l]));
            float *ob = const_cast<float *>(fr.b[l]);
            const int64_t j = fr.j[l];
            if (wave == 0) {
                if (l == 1) {
                    const KT *keys = static_cast<const KT *>(f.k) + (pair * f.max_tokens + j * c) * D;
                    leaf_node<D, KT, ST>(rho, kk, wt, mx_s, z_s, keys, ok, ob, R, c, s);
                } else {
                    const ST *ck = reinterpret_cast<const ST *>(a.kap[l - 1]) + pair * a.cap[l - 1] * (R * D);
                    const float *cb = a.bet[l - 1] + pair * a.cap[l - 1] * R;
                    const ST *last_k = reinterpret_cast<const ST *>(fr.k[l - 1]);
                    const float *last_b = fr.b[l - 1];
                    upper_node<D, ST>(
                        refs, s_sig,
                        [&](int i) { return i == c - 1 ? last_k : ck + (j * c + i) * (R * D); },
                        [&](int i) { return i == c - 1 ? last_b : cb + (j * c + i) * R; }, ok, ob, R, c, s);
                }
            }
            __syncthreads();
        }
        // the pair's first walk writes them to the tree (no walk of this
        // launch reads them from there)
        if (leader) {
            for (int l = 1; l <= f.fresh_m; ++l) {
                const int64_t node = pair * a.cap[l] + fr.j[l];
                const float *src = static_cast<const float *>(fr.k[l]);
                float *dk = reinterpret_cast<float *>(static_cast<char *>(f.tree_k[l]) + node * (R * D * sizeof(ST)));
                for (int i = tid; i < R * D * static_cast<int>(sizeof(ST)) / 4; i += kThreads) dk[i] = src[i];
                for (int r = tid; r < R; r += kThreads) f.tree_b[l][node * R + r] = fr.b[l][r];
            }
        }
    }

    // ---- 2. the walk (the persistent engine's step loop) ------------------------
    float qv[row_epl<D, ST>()];
    load_q<D, KT, ST>(a, w, qv);
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
            float wmax = score_wave<D, R, ST, false, true>(a, pair, qv, cur, sc, wave * kU, n, kWaves * kU, flags,
                                                           &fr);
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

    // ---- 3. attention over the selected blocks and the raw tail -----------------
    constexpr int EPL = 16 / static_cast<int>(sizeof(KT));   // elements of a row per lane
    constexpr int LPR = D / EPL;                             // lanes per row
    constexpr int RPW = 64 / LPR;                            // rows per wavefront load
    const int grp = lane / LPR, sub = lane % LPR;
    const int64_t nb = sel_n < a.sel_cap ? sel_n : a.sel_cap;
    const int64_t n1 = a.nl[1];
    const int64_t body = nb * c;
    const int64_t total = body + (a.n_tokens - static_cast<int64_t>(c) * n1);
    const KT *kb = static_cast<const KT *>(f.k) + pair * f.max_tokens * D + sub * EPL;
    const KT *vb = static_cast<const KT *>(f.v) + pair * f.max_tokens * D + sub * EPL;
    float qa[EPL];
    {
        const KT *qp = static_cast<const KT *>(a.q) + static_cast<int64_t>(w) * D + sub * EPL;
        Vec16<KT>::load(qp, qa);
    }
    float m = -INFINITY, lsum = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    const int64_t stride = static_cast<int64_t>(kWaves) * RPW * kFU;
    for (int64_t t0 = (static_cast<int64_t>(wave) * RPW + grp) * kFU; t0 < total; t0 += stride) {
        float kv[kFU][EPL], vv[kFU][EPL];
        bool live[kFU];
#pragma unroll
        for (int u = 0; u < kFU; ++u) {
            const int64_t i = t0 + u;
            live[u] = i < total;
            int64_t tok = 0;
            if (live[u]) tok = i < body ? static_cast<int64_t>(selw[i / c]) * c + (i % c) : c * n1 + (i - body);
            Vec16<KT>::load(kb + tok * D, kv[u]);
            Vec16<KT>::load(vb + tok * D, vv[u]);
        }
#pragma unroll
        for (int u = 0; u < kFU; ++u) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qa[e], kv[u][e], d);
            d = lane_group_sum(d, LPR);
            const float lg = live[u] ? s * d : -INFINITY;
            const float mn = fmaxf(m, lg);
            if (mn > -INFINITY) {
                const float cs = (m > -INFINITY) ? expf(m - mn) : 0.f;
                const float p = live[u] ? expf(lg - mn) : 0.f;
                lsum = lsum * cs + p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vv[u][e], acc[e] * cs);
                m = mn;
            }
        }
    }
    // lane groups of the wavefront, then the wavefronts
    for (int off = LPR; off < 64; off <<= 1) merge_shfl<EPL>(m, lsum, acc, off);
    __syncthreads();
    float *part = lds;                        // [kWaves][D + 2] (LDS of the append is free again)
    if (grp == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) part[wave * (D + 2) + sub * EPL + e] = acc[e];
        if (sub == 0) {
            part[wave * (D + 2) + D] = m;
            part[wave * (D + 2) + D + 1] = lsum;
        }
    }
    __syncthreads();
    for (int d = tid; d < D; d += kThreads) {
        float mm = -INFINITY;
        for (int v = 0; v < kWaves; ++v) mm = fmaxf(mm, part[v * (D + 2) + D]);
        float L = 0.f, o = 0.f;
        if (mm > -INFINITY) {
            for (int v = 0; v < kWaves; ++v) {
                const float mv = part[v * (D + 2) + D];
                const float cv = (mv > -INFINITY) ? expf(mv - mm) : 0.f;
                L += part[v * (D + 2) + D + 1] * cv;
                o += part[v * (D + 2) + d] * cv;
            }
        }
        const float r = L > 0.f ? o / L : 0.f;
        Elem<KT>::store(static_cast<KT *>(f.out), static_cast<int64_t>(w) * D + d, r);
    }
}

// LDS bytes of k_step_fused (the append's scratch and records; at least the
// attention merge).
size_t fused_lds_bytes(int D, int R, int c, int sbytes, int m) {
    const int P = D + 4;
    const size_t fixed = static_cast<size_t>((R * P + c * P + c * R + 2 * R + 3) & ~3);
    const size_t recf = static_cast<size_t>((R * D * sbytes + 15) / 16 * 4);
    const size_t recs = (recf + R + 3) & ~static_cast<size_t>(3);
    size_t fl = (m > 0 ? fixed + static_cast<size_t>(m) * recs : 0);
    const size_t merge = static_cast<size_t>(kWaves) * (D + 2);
    if (fl < merge) fl = merge;
    return fl * sizeof(float);
}

template <int D, int R, typename KT, typename ST>
static hipError_t launch_fused_t(const FusedArgs &f, hipStream_t st) {
    const size_t lds = fused_lds_bytes(D, R, f.s.chunk, static_cast<int>(sizeof(ST)), f.fresh_m);
    hipLaunchKernelGGL((k_step_fused<D, R, KT, ST>), dim3(f.s.walks), dim3(kThreads), lds, st, f);
    return hipGetLastError();
}

template <int D, typename KT, typename ST>
static hipError_t launch_fused_r(const FusedArgs &f, int R, hipStream_t st) {
    switch (R) {
        case 1: return launch_fused_t<D, 1, KT, ST>(f, st);
        case 2: return launch_fused_t<D, 2, KT, ST>(f, st);
        case 4: return launch_fused_t<D, 4, KT, ST>(f, st);
        case 8: return launch_fused_t<D, 8, KT, ST>(f, st);
        case 16: return launch_fused_t<D, 16, KT, ST>(f, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, typename KT>
static hipError_t launch_fused_s(const FusedArgs &f, int R, int sdtype, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_fused_r<D, KT, bf16_t>(f, R, st) : launch_fused_r<D, KT, float>(f, R, st);
}

hipError_t launch_fused(const FusedArgs &f, int D, int R, int dtype, int sdtype, hipStream_t st) {
    if (f.s.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_fused_s<64, bf16_t>(f, R, sdtype, st)
                                 : launch_fused_s<64, float>(f, R, sdtype, st);
    return dtype == ZHA_BF16 ? launch_fused_s<128, bf16_t>(f, R, sdtype, st)
                             : launch_fused_s<128, float>(f, R, sdtype, st);
}

}  // namespace zha
