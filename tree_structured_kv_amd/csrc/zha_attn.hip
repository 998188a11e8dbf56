// zha_attn.hip -- split-K decode attention over the selected original keys.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  Sections "How is the tree built?" and "Common
// misunderstandings": the summaries only find the way; ordinary softmax
// attention then runs on exactly the original keys and values chosen, with
// the full cache kept.  A walk's key set is the c keys of every listed
// level-1 block plus the raw tail past the last whole chunk.
//
// GPU design.  Walks select very different numbers of keys under top-p, so
// the work is planned on the device: k_attn_plan cuts every walk's key list
// into chunks of kChunkKeys and lays the (walk, chunk) items out flat;
// k_attn_partial is a grid-stride loop over the items, so every workgroup
// streams about the same number of bytes whatever the spread between walks.
// A key row is D*e bytes read as 16-byte pieces by D*e/16 lanes.  The online
// softmax state (max, sum, weighted V) lives per key slot and is merged
// across slots, wavefronts and finally items (k_attn_combine), all in fp32.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

constexpr int kWaves = kBlock / 64;

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

__device__ __forceinline__ int64_t walk_entries(const AttnArgs &a, int w) {
    int64_t nb = a.sel_count[w];
    if (nb > a.sel_cap) nb = a.sel_cap;
    if (nb < 0) nb = 0;
    return nb;
}

// Keys of a walk: the c keys of every listed block plus the raw tail (or
// the listed tokens), then, for query t of a prefill block, the block's own
// keys n_tokens .. n_tokens + t.
__device__ __forceinline__ int64_t walk_keys(const AttnArgs &a, int w) {
    const int64_t nb = walk_entries(a, w);
    const int64_t causal = (a.qph > 1) ? (w % a.qph) + 1 : 0;
    if (a.tokens) return nb + causal;
    return nb * a.chunk + (a.n_tokens - static_cast<int64_t>(a.chunk) * a.n1) + causal;
}

}  // namespace

// One workgroup: item offsets = exclusive scan of max(1, ceil(keys / chunk))
// over walks, and the walk id of every item.
__global__ __launch_bounds__(1024) void k_attn_plan(AttnArgs a) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < a.walks; base += 1024) {
        const int w = base + tid;
        int32_t cnt = 0;
        if (w < a.walks) {
            const int64_t keys = walk_keys(a, w);
            cnt = static_cast<int32_t>((keys + kChunkKeys - 1) / kChunkKeys);
            if (cnt < 1) cnt = 1;
        }
        int32_t incl = cnt;
        for (int off = 1; off < 64; off <<= 1) {
            int32_t o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int32_t before = carry;
        for (int i = 0; i < wave; ++i) before += wsum[i];
        const int32_t start = before + incl - cnt;
        if (w < a.walks) {
            a.item_off[w] = start;
            for (int32_t i = 0; i < cnt; ++i) a.item_walk[start + i] = w;
        }
        __syncthreads();
        if (tid == 1023) carry = start + cnt;
        __syncthreads();
    }
    if (tid == 0) a.item_off[a.walks] = carry;
}

template <int D, typename KT>
__global__ __launch_bounds__(kBlock) void k_attn_partial(AttnArgs a) {
    constexpr int EPL = Vec16<KT>::N;     // elements per lane per row
    constexpr int LPK = D / EPL;          // lanes per key row
    constexpr int KPW = 64 / LPK;         // keys per 64-lane load
    constexpr int U = 8;                  // key rows in flight per lane group

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane / LPK, sub = lane % LPK;
    const int c = a.chunk;
    const float s = a.sharpness;
    const int32_t n_items = a.item_off[a.walks];
    __shared__ float sm[kWaves], sl[kWaves], sacc[kWaves][D];

    for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int w = a.item_walk[item];
        const int64_t chunk = item - a.item_off[w];
        const int64_t pair = walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
        const int64_t nb = walk_entries(a, w);
        const int64_t body = a.tokens ? nb : nb * c;
        const int64_t tree_keys = a.tokens ? nb : body + (a.n_tokens - static_cast<int64_t>(c) * a.n1);
        const int64_t total = walk_keys(a, w);
        const int64_t k0 = chunk * kChunkKeys;
        const int64_t k1 = (k0 + kChunkKeys < total) ? k0 + kChunkKeys : total;

        float qv[EPL];
        {
            const KT *qp = static_cast<const KT *>(a.q) + static_cast<int64_t>(w) * D;
            for (int e = 0; e < EPL; ++e) qv[e] = Elem<KT>::load(qp, sub * EPL + e);
        }
        const KT *kb = static_cast<const KT *>(a.k) + pair * a.max_tokens * D;
        const KT *vb = static_cast<const KT *>(a.v) + pair * a.max_tokens * D;
        const int32_t *selw = (a.tokens ? a.tokens : a.sel_blocks) + static_cast<int64_t>(w) * a.sel_cap;
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
                    if (ki >= tree_keys) {
                        tok = a.n_tokens + (ki - tree_keys);   // the block's own keys (causal)
                    } else if (a.tokens) {
                        const int64_t tk = selw[ki];
                        ok[u] = tk >= 0 && tk < a.n_tokens;   // ids outside the cache are skipped
                        tok = ok[u] ? tk : 0;
                    } else if (ki < body) {
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
        if (slot == 0) {
            for (int e = 0; e < EPL; ++e) sacc[wave][sub * EPL + e] = acc[e];
            if (sub == 0) { sm[wave] = m; sl[wave] = l; }
        }
        __syncthreads();
        if (tid < D) {
            float mm = sm[0], ll = sl[0], av = sacc[0][tid];
            for (int wv = 1; wv < kWaves; ++wv) merge_state(mm, ll, &av, sm[wv], sl[wv], &sacc[wv][tid], 1);
            float *part = a.part + static_cast<int64_t>(item) * (D + 2);
            part[2 + tid] = av;
            if (tid == 0) { part[0] = mm; part[1] = ll; }
        }
        __syncthreads();
    }
}

template <int D, typename KT>
__global__ __launch_bounds__(D) void k_attn_combine(AttnArgs a) {
    const int w = blockIdx.x, e = threadIdx.x;
    const int32_t i0 = a.item_off[w], i1 = a.item_off[w + 1];
    float mm = -INFINITY;
    for (int32_t i = i0; i < i1; ++i) mm = fmaxf(mm, a.part[static_cast<int64_t>(i) * (D + 2)]);
    float ll = 0.f, av = 0.f;
    if (mm > -INFINITY) {
        for (int32_t i = i0; i < i1; ++i) {
            const float *p = a.part + static_cast<int64_t>(i) * (D + 2);
            if (!(p[0] > -INFINITY)) continue;
            const float cf = expf(p[0] - mm);
            ll = fmaf(p[1], cf, ll);
            av = fmaf(p[2 + e], cf, av);
        }
    }
    const float o = (ll > 0.f) ? av / ll : 0.f;
    Elem<KT>::store(static_cast<KT *>(a.out), static_cast<int64_t>(w) * D + e, o);
}

template <int D, typename KT>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_attn_plan, dim3(1), dim3(1024), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_partial<D, KT>), dim3(static_cast<unsigned>(a.grid)), dim3(kBlock), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_combine<D, KT>), dim3(a.walks), dim3(D), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int D, int dtype, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_attn_t<64, bf16_t>(a, st) : launch_attn_t<64, float>(a, st);
    return dtype == ZHA_BF16 ? launch_attn_t<128, bf16_t>(a, st) : launch_attn_t<128, float>(a, st);
}

}  // namespace zha
