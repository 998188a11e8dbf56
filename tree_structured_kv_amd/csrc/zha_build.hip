// zha_build.hip -- summarise one tree level (build and append).
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  Section "What does a node summarize?": for every reference
// query rho_r a node stores one tangent (key_r, bias_r) of the subtree's
// log-sum-exp; from c children it is
//     sigma_i = s <child key_{i,r}, rho_r> + child bias_{i,r}
//     key_r   = sum_i softmax(sigma)_i child key_{i,r}
//     bias_r  = logsumexp(sigma) - s <key_r, rho_r>.
// Section "How is the tree built?": level 1 summarises each whole chunk of c
// raw keys (a raw key is its own tangent for every reference, bias 0) and
// level l summarises each whole chunk of c level-(l-1) nodes.
//
// One wavefront per node; a lane holds D/64 consecutive elements of every
// row, so every row read and every key write is one coalesced 64-lane access.
// The arithmetic of a node depends only on its children, so a node computed
// by an append is bit-identical to the same node computed by a full build.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

template <int D, typename KT, bool LEAF, typename ST>
__global__ __launch_bounds__(kBlock) void k_summarize(LevelArgs a) {
    constexpr int EPL = D / 64;                 // elements per lane
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t jn = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + wave;
    if (jn >= a.count) return;                  // whole wavefront leaves; no barriers below
    const int64_t j = a.j0 + jn;
    const int pair = blockIdx.y;
    const int g = pair % a.kv_heads;
    const int R = a.refs_n;
    const int c = a.chunk;
    const float s = a.sharpness;

    __shared__ float sig_lds[kBlock / 64][64];
    float *sig = sig_lds[wave];

    const KT *keys = static_cast<const KT *>(a.keys) + static_cast<int64_t>(pair) * a.max_tokens * D;
    const ST *ck = static_cast<const ST *>(a.child_k) + static_cast<int64_t>(pair) * a.child_cap * R * D;
    const float *cb = a.child_b + static_cast<int64_t>(pair) * a.child_cap * R;
    ST *ok = static_cast<ST *>(a.out_k) + (static_cast<int64_t>(pair) * a.out_cap + j) * R * D;
    float *ob = a.out_b + (static_cast<int64_t>(pair) * a.out_cap + j) * R;
    const float *refs = a.refs + static_cast<int64_t>(g) * R * D;

    for (int r = 0; r < R; ++r) {
        float rho[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) rho[e] = refs[r * D + lane * EPL + e];

        // scores of the c children under rho_r
        float mx = -INFINITY;
        for (int i = 0; i < c; ++i) {
            const int64_t child = j * c + i;
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float x = LEAF ? Elem<KT>::load(keys, child * D + lane * EPL + e)
                               : Elem<ST>::load(ck, (child * R + r) * D + lane * EPL + e);
                part = fmaf(x, rho[e], part);
            }
            float dotv = wave_sum(part, 64);
            float sg = s * dotv + (LEAF ? 0.f : cb[child * R + r]);
            if (lane == 0) sig[i] = sg;
            mx = fmaxf(mx, sg);
        }
        __builtin_amdgcn_wave_barrier();
        float z = 0.f;
        for (int i = 0; i < c; ++i) z += expf(sig[i] - mx);
        const float inv_z = 1.f / z;

        // weighted sum of the child keys
        float acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
        for (int i = 0; i < c; ++i) {
            const int64_t child = j * c + i;
            const float w = expf(sig[i] - mx) * inv_z;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float x = LEAF ? Elem<KT>::load(keys, child * D + lane * EPL + e)
                               : Elem<ST>::load(ck, (child * R + r) * D + lane * EPL + e);
                acc[e] = fmaf(w, x, acc[e]);
            }
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            Elem<ST>::store(ok, r * D + lane * EPL + e, acc[e]);
            // the bias uses the key as stored (bf16: rounded)
            const float kept = (sizeof(ST) == 2) ? bf16_to_f32(f32_to_bf16(acc[e])) : acc[e];
            part = fmaf(kept, rho[e], part);
        }
        const float kr = wave_sum(part, 64);
        if (lane == 0) ob[r] = (mx + logf(z)) - s * kr;
        __builtin_amdgcn_wave_barrier();   // sig[] is rewritten for the next r
    }
}

// Level 1, one wavefront per node, the chunk's c keys staged once in LDS
// (fp32) next to the group's R references (one copy per workgroup):
//   1. lane pair p = r*c + i: sigma = s <K_i, rho_r>; max and sum of
//      exp(sigma - max) over the c lanes of reference r; w = softmax;
//   2. lane item (r, 16 elements): key_r = sum_i w_i K_i, written as
//      coalesced 16-float runs; bias_r = max + log(sum) - s <key_r, rho_r>
//      summed over the D/16 lanes of r.
// Every key is read from HBM once; the passes over it run from LDS.
template <int D, typename KT, typename ST>
__global__ __launch_bounds__(kBlock) void k_leaf(LevelArgs a, int waves) {
    constexpr int P = D + 4;                    // LDS row pitch (floats)
    constexpr int NS = D / 16;                  // 16-element slices of a row
    extern __shared__ float lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int R = a.refs_n, c = a.chunk;
    const int pair = blockIdx.y;
    const int g = pair % a.kv_heads;
    const float s = a.sharpness;
    float *rho = lds;                                          // [R][P]
    const int per_wave = (c * P + c * R + 2 * R + 3) & ~3;     // 16-byte aligned regions
    float *kk = lds + R * P + wave * per_wave;                 // [c][P]
    float *wt = kk + c * P;                                    // [R][c]
    float *mx_s = wt + c * R;                                  // [R]
    float *z_s = mx_s + R;                                     // [R]
    const float *refs = a.refs + static_cast<int64_t>(g) * R * D;
    for (int idx = threadIdx.x; idx < R * (D / 4); idx += blockDim.x) {
        const int r = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
        *reinterpret_cast<float4 *>(rho + r * P + d4) = *reinterpret_cast<const float4 *>(refs + r * D + d4);
    }
    __syncthreads();
    const int64_t jn = static_cast<int64_t>(blockIdx.x) * waves + wave;
    if (wave >= waves || jn >= a.count) return;  // no workgroup barrier below
    const int64_t j = a.j0 + jn;
    const KT *keys = static_cast<const KT *>(a.keys) + (static_cast<int64_t>(pair) * a.max_tokens + j * c) * D;
    ST *ok = static_cast<ST *>(a.out_k) + (static_cast<int64_t>(pair) * a.out_cap + j) * R * D;
    float *ob = a.out_b + (static_cast<int64_t>(pair) * a.out_cap + j) * R;

    // the chunk's keys, 16 bytes per lane per round
    constexpr int EV = 16 / static_cast<int>(sizeof(KT));       // elements per 16 bytes
    for (int idx = lane; idx < c * (D / EV); idx += 64) {
        const int i = idx / (D / EV), d0 = (idx % (D / EV)) * EV;
        float v[EV];
        if constexpr (sizeof(KT) == 2) {
            Vec16<KT>::load(keys + i * D + d0, v);
        } else {
            const float4 x = *reinterpret_cast<const float4 *>(keys + i * D + d0);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        }
#pragma unroll
        for (int e = 0; e < EV; e += 4)
            *reinterpret_cast<float4 *>(kk + i * P + d0 + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    // 1. scores and softmax weights, one (r, i) pair per lane and round
    for (int p0 = 0; p0 < c * R; p0 += 64) {
        const int pi = p0 + lane;
        const bool live = pi < c * R;
        const int r = live ? pi / c : 0, i = live ? pi % c : 0;
        const float *kr = kk + i * P;
        const float *qr = rho + r * P;
        float d = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; e += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(kr + e);
            const float4 y = *reinterpret_cast<const float4 *>(qr + e);
            d = fmaf(x.x, y.x, d);
            d = fmaf(x.y, y.y, d);
            d = fmaf(x.z, y.z, d);
            d = fmaf(x.w, y.w, d);
        }
        const float sg = live ? s * d : -INFINITY;
        float m = sg;
        for (int off = 1; off < c; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const float ex = live ? expf(sg - m) : 0.f;
        float z = ex;
        for (int off = 1; off < c; off <<= 1) z += __shfl_xor(z, off, 64);
        if (live) {
            wt[r * c + i] = ex / z;
            if (i == 0) { mx_s[r] = m; z_s[r] = z; }
        }
    }
    __builtin_amdgcn_wave_barrier();
    // 2. keys and biases, one (r, 16-element slice) per lane and round
    for (int t0 = 0; t0 < R * NS; t0 += 64) {
        const int ti = t0 + lane;
        const bool live = ti < R * NS;
        const int r = live ? ti / NS : 0, d0 = live ? (ti % NS) * 16 : 0;
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        for (int i = 0; i < c; ++i) {
            const float w = wt[r * c + i];
            const float *kr = kk + i * P + d0;
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(kr + e);
                acc[e] = fmaf(w, x.x, acc[e]);
                acc[e + 1] = fmaf(w, x.y, acc[e + 1]);
                acc[e + 2] = fmaf(w, x.z, acc[e + 2]);
                acc[e + 3] = fmaf(w, x.w, acc[e + 3]);
            }
        }
        if constexpr (sizeof(ST) == 2) {
            // the stored key is the bf16 rounding; the bias uses it
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = bf16_to_f32(f32_to_bf16(acc[e]));
        }
        float part = 0.f;
        const float *qr = rho + r * P + d0;
#pragma unroll
        for (int e = 0; e < 16; ++e) part = fmaf(acc[e], qr[e], part);
        for (int off = 1; off < NS; off <<= 1) part += __shfl_xor(part, off, 64);
        if (live) {
            if constexpr (sizeof(ST) == 2) {
                uint32_t wv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wv[e] = static_cast<uint32_t>(f32_to_bf16(acc[2 * e])) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[2 * e + 1])) << 16);
                *reinterpret_cast<uint4 *>(ok + r * D + d0) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                *reinterpret_cast<uint4 *>(ok + r * D + d0 + 8) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
            } else {
#pragma unroll
                for (int e = 0; e < 16; e += 4)
                    *reinterpret_cast<float4 *>(ok + r * D + d0 + e) =
                        make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            }
            if (d0 == 0) ob[r] = (mx_s[r] + logf(z_s[r])) - s * part;
        }
    }
}

// Workgroup shape of k_leaf: as many node wavefronts as fit in 64 KB of LDS.
static int leaf_waves(const LevelArgs &a, int D, size_t &lds_bytes) {
    const int P = D + 4;
    const size_t per_wave = (static_cast<size_t>(a.chunk) * P + static_cast<size_t>(a.chunk) * a.refs_n +
                             2 * static_cast<size_t>(a.refs_n) + 3) / 4 * 4;
    const size_t fixed = static_cast<size_t>(a.refs_n) * P;
    int waves = kBlock / 64;
    while (waves > 1 && (fixed + waves * per_wave) * sizeof(float) > 65536) --waves;
    lds_bytes = (fixed + waves * per_wave) * sizeof(float);
    return waves;
}

template <int D, typename KT, typename ST>
static hipError_t launch_level_t(const LevelArgs &a, bool leaf, hipStream_t st) {
    if (leaf) {
        size_t lds = 0;
        const int waves = leaf_waves(a, D, lds);
        dim3 grid(static_cast<unsigned>((a.count + waves - 1) / waves), static_cast<unsigned>(a.pairs));
        hipLaunchKernelGGL((k_leaf<D, KT, ST>), grid, dim3(kBlock), lds, st, a, waves);
        return hipGetLastError();
    }
    dim3 grid(static_cast<unsigned>((a.count + (kBlock / 64) - 1) / (kBlock / 64)),
              static_cast<unsigned>(a.pairs));
    hipLaunchKernelGGL((k_summarize<D, KT, false, ST>), grid, dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <int D, typename KT>
static hipError_t launch_level_s(const LevelArgs &a, int sdtype, bool leaf, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_level_t<D, KT, bf16_t>(a, leaf, st) : launch_level_t<D, KT, float>(a, leaf, st);
}

hipError_t launch_level(const LevelArgs &a, int D, int dtype, int sdtype, bool leaf, hipStream_t st) {
    if (a.count <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_level_s<64, bf16_t>(a, sdtype, leaf, st)
                                 : launch_level_s<64, float>(a, sdtype, leaf, st);
    return dtype == ZHA_BF16 ? launch_level_s<128, bf16_t>(a, sdtype, leaf, st)
                             : launch_level_s<128, float>(a, sdtype, leaf, st);
}

}  // namespace zha
