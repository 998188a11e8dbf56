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

template <int D, typename KT, bool LEAF>
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
    const float *ck = a.child_k + static_cast<int64_t>(pair) * a.child_cap * R * D;
    const float *cb = a.child_b + static_cast<int64_t>(pair) * a.child_cap * R;
    float *ok = a.out_k + (static_cast<int64_t>(pair) * a.out_cap + j) * R * D;
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
                               : ck[(child * R + r) * D + lane * EPL + e];
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
                               : ck[(child * R + r) * D + lane * EPL + e];
                acc[e] = fmaf(w, x, acc[e]);
            }
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            ok[r * D + lane * EPL + e] = acc[e];
            part = fmaf(acc[e], rho[e], part);
        }
        const float kr = wave_sum(part, 64);
        if (lane == 0) ob[r] = (mx + logf(z)) - s * kr;
        __builtin_amdgcn_wave_barrier();   // sig[] is rewritten for the next r
    }
}

template <int D, typename KT>
static hipError_t launch_level_t(const LevelArgs &a, bool leaf, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((a.count + (kBlock / 64) - 1) / (kBlock / 64)),
              static_cast<unsigned>(a.pairs));
    if (leaf)
        hipLaunchKernelGGL((k_summarize<D, KT, true>), grid, dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_summarize<D, KT, false>), grid, dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_level(const LevelArgs &a, int D, int dtype, bool leaf, hipStream_t st) {
    if (a.count <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_level_t<64, bf16_t>(a, leaf, st)
                                 : launch_level_t<64, float>(a, leaf, st);
    return dtype == ZHA_BF16 ? launch_level_t<128, bf16_t>(a, leaf, st)
                             : launch_level_t<128, float>(a, leaf, st);
}

}  // namespace zha
