// zha_attn.hip -- split-K decode attention over the selected original keys.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  Sections "How is the tree built?" and "Common
// misunderstandings": the summaries only find the way; ordinary softmax
// attention then runs on exactly the original keys and values chosen, with
// the full cache kept.  A walk's key set is the c keys of every listed
// level-1 block plus the raw tail past the last whole chunk.
//
// GPU design: grid = walks x splits.  Each workgroup streams a contiguous
// range of the walk's selected keys; a key row is D*e bytes, read as 16-byte
// pieces by D*e/16 lanes, so one 64-lane load covers 64*16/(D*e) keys.  The
// online softmax state (max, sum, weighted V) lives per key slot and is merged
// across slots, wavefronts and finally splits (k_attn_combine), all in fp32.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

constexpr int kWaves = kBlock / 64;

struct Online {
    float m, l;
};

__device__ __forceinline__ void merge_state(float &m, float &l, float *acc, float m2, float l2,
                                            const float *acc2, int n) {
    const float mm = fmaxf(m, m2);
    if (!(mm > -INFINITY)) return;   // both empty
    const float c1 = (m > -INFINITY) ? expf(m - mm) : 0.f;
    const float c2 = (m2 > -INFINITY) ? expf(m2 - mm) : 0.f;
    l = l * c1 + l2 * c2;
    for (int e = 0; e < n; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    m = mm;
}

}  // namespace

template <int D, typename KT>
__global__ __launch_bounds__(kBlock) void k_attn_partial(AttnArgs a) {
    constexpr int EPL = Vec16<KT>::N;     // elements per lane per row
    constexpr int LPK = D / EPL;          // lanes per key row
    constexpr int KPW = 64 / LPK;         // keys per 64-lane load
    constexpr int U = 2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x / a.splits;
    const int split = blockIdx.x % a.splits;
    if (w >= a.walks) return;
    const int b = w / a.heads, h = w % a.heads, g = h / a.group;
    const int64_t pair = static_cast<int64_t>(b) * a.kv_heads + g;
    const int c = a.chunk;
    const float s = a.sharpness;

    int64_t nb = a.sel_count[w];
    if (nb > a.sel_cap) nb = a.sel_cap;
    if (nb < 0) nb = 0;
    const int64_t body = nb * c;
    const int64_t total = body + (a.n_tokens - static_cast<int64_t>(c) * a.n1);
    const int64_t k0 = total * split / a.splits;
    const int64_t k1 = total * (split + 1) / a.splits;

    const int slot = lane / LPK, sub = lane % LPK;
    float qv[EPL];
    {
        const KT *qp = static_cast<const KT *>(a.q) + static_cast<int64_t>(w) * D;
        for (int e = 0; e < EPL; ++e) qv[e] = Elem<KT>::load(qp, sub * EPL + e);
    }
    const KT *kb = static_cast<const KT *>(a.k) + pair * a.max_tokens * D;
    const KT *vb = static_cast<const KT *>(a.v) + pair * a.max_tokens * D;
    const int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;
    const int64_t tail0 = static_cast<int64_t>(c) * a.n1;

    float m = -INFINITY, l = 0.f, acc[EPL];
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    const int64_t stride = static_cast<int64_t>(kWaves) * KPW;
    for (int64_t kk = k0 + wave * KPW + slot; kk < k1; kk += stride * U) {
        float kr[U][EPL], vr[U][EPL];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t ki = kk + u * stride;
            ok[u] = ki < k1;
            int64_t tok = 0;
            if (ok[u]) {
                if (ki < body) {
                    const int64_t blk = selw[ki / c];
                    ok[u] = blk >= 0 && blk < a.n1;    // ids outside the live level are skipped
                    tok = ok[u] ? blk * c + (ki % c) : 0;
                } else {
                    tok = tail0 + (ki - body);
                }
            }
            Vec16<KT>::load(kb + tok * D + sub * EPL, kr[u]);
            Vec16<KT>::load(vb + tok * D + sub * EPL, vr[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(kr[u][e], qv[e], d);
            d = wave_sum(d, LPK);
            if (!ok[u]) continue;
            const float lg = s * d;
            const float mn = fmaxf(m, lg);
            const float corr = (m > -INFINITY) ? expf(m - mn) : 0.f;
            const float pe = expf(lg - mn);
            l = l * corr + pe;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pe, vr[u][e], acc[e] * corr);
            m = mn;
        }
    }

    // merge key slots inside the wavefront (lanes with equal `sub`)
    for (int off = LPK; off < 64; off <<= 1) {
        float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64), acc2[EPL];
        for (int e = 0; e < EPL; ++e) acc2[e] = __shfl_xor(acc[e], off, 64);
        merge_state(m, l, acc, m2, l2, acc2, EPL);
    }
    __shared__ float sm[kWaves], sl[kWaves], sacc[kWaves][D];
    if (slot == 0) {
        for (int e = 0; e < EPL; ++e) sacc[wave][sub * EPL + e] = acc[e];
        if (sub == 0) { sm[wave] = m; sl[wave] = l; }
    }
    __syncthreads();
    if (tid < D) {
        float mm = sm[0], ll = sl[0], av = sacc[0][tid];
        for (int wv = 1; wv < kWaves; ++wv) merge_state(mm, ll, &av, sm[wv], sl[wv], &sacc[wv][tid], 1);
        float *part = a.part + (static_cast<int64_t>(w) * a.splits + split) * (D + 2);
        part[2 + tid] = av;
        if (tid == 0) { part[0] = mm; part[1] = ll; }
    }
}

template <int D, typename KT>
__global__ __launch_bounds__(D) void k_attn_combine(const float *part, void *out, int splits) {
    const int w = blockIdx.x, e = threadIdx.x;
    const float *pw = part + static_cast<int64_t>(w) * splits * (D + 2);
    float mm = -INFINITY;
    for (int sp = 0; sp < splits; ++sp) mm = fmaxf(mm, pw[sp * (D + 2)]);
    float ll = 0.f, av = 0.f;
    if (mm > -INFINITY) {
        for (int sp = 0; sp < splits; ++sp) {
            const float ms = pw[sp * (D + 2)];
            if (!(ms > -INFINITY)) continue;
            const float cf = expf(ms - mm);
            ll = fmaf(pw[sp * (D + 2) + 1], cf, ll);
            av = fmaf(pw[sp * (D + 2) + 2 + e], cf, av);
        }
    }
    const float o = (ll > 0.f) ? av / ll : 0.f;
    Elem<KT>::store(static_cast<KT *>(out), static_cast<int64_t>(w) * D + e, o);
}

template <int D, typename KT>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(a.walks * a.splits));
    hipLaunchKernelGGL((k_attn_partial<D, KT>), grid, dim3(kBlock), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_combine<D, KT>), dim3(a.walks), dim3(D), 0, st,
                       static_cast<const float *>(a.part), a.out, a.splits);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int D, int dtype, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_attn_t<64, bf16_t>(a, st) : launch_attn_t<64, float>(a, st);
    return dtype == ZHA_BF16 ? launch_attn_t<128, bf16_t>(a, st) : launch_attn_t<128, float>(a, st);
}

}  // namespace zha
