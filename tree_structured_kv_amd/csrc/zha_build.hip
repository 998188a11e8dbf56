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
#include "zha_summary.h"

#include <algorithm>

namespace zha {

// Level >= 2: one wavefront per node (upper_node), the rows of up to CBT
// children in flight together (8 for chunks of up to 8: fewer registers,
// more wavefronts; 16 above).
template <int D, typename ST, int CBT>
__global__ __launch_bounds__(kBlock) void k_summarize(LevelArgs a) {
    const int wave = threadIdx.x >> 6;
    const int64_t jn = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + wave;
    if (jn >= a.count) return;                  // whole wavefront leaves; no barriers below
    const int64_t j = a.j0 + jn;
    const int pair = blockIdx.y;
    const int g = pair % a.kv_heads;
    const int R = a.refs_n;
    const int c = a.chunk;

    __shared__ float sig_lds[kBlock / 64][64];

    const ST *ck = static_cast<const ST *>(a.child_k) + static_cast<int64_t>(pair) * a.child_cap * R * D;
    const float *cb = a.child_b + static_cast<int64_t>(pair) * a.child_cap * R;
    ST *ok = static_cast<ST *>(a.out_k) + (static_cast<int64_t>(pair) * a.out_cap + j) * R * D;
    float *ob = a.out_b + (static_cast<int64_t>(pair) * a.out_cap + j) * R;
    const float *refs = a.refs + static_cast<int64_t>(g) * R * D;
    auto child_k = [&](int i) { return ck + (j * c + i) * R * D; };
    auto child_b = [&](int i) { return cb + (j * c + i) * R; };
    upper_node<D, ST, decltype(child_k), decltype(child_b), CBT>(refs, sig_lds[wave], child_k, child_b, ok, ob, R, c,
                                                                 a.sharpness);
}

// Level 1, one wavefront per node at a time (leaf_node), the chunk's c keys
// staged once in LDS (fp32) next to the group's R references (one copy per
// workgroup, which loops over nodes).
// Every key is read from HBM once; the passes over it run from LDS.
template <int D, typename KT, typename ST>
__global__ __launch_bounds__(kBlock) void k_leaf(LevelArgs a, int waves) {
    constexpr int P = D + 4;                    // LDS row pitch (floats)
    extern __shared__ float lds[];
    const int wave = threadIdx.x >> 6;
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
    if (wave >= waves) return;                   // no workgroup barrier below
    // each node wavefront takes nodes gridDim.x * waves apart
    const int64_t stride = static_cast<int64_t>(gridDim.x) * waves;
    for (int64_t jn = static_cast<int64_t>(blockIdx.x) * waves + wave; jn < a.count; jn += stride) {
        const int64_t j = a.j0 + jn;
        const KT *keys = static_cast<const KT *>(a.keys) + (static_cast<int64_t>(pair) * a.max_tokens + j * c) * D;
        ST *ok = static_cast<ST *>(a.out_k) + (static_cast<int64_t>(pair) * a.out_cap + j) * R * D;
        float *ob = a.out_b + (static_cast<int64_t>(pair) * a.out_cap + j) * R;
        __builtin_amdgcn_wave_barrier();         // the previous node's LDS reads come first
        leaf_node<D, KT, ST>(rho, kk, wt, mx_s, z_s, keys, ok, ob, R, c, s);
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
        int64_t gx = (a.count + waves - 1) / waves;
        // about 8192 workgroups in all, each node wavefront looping over nodes
        // (one reference staging per workgroup; 4-5% faster than a
        // workgroup per node group at 256K and 1M)
        gx = std::min<int64_t>(gx, std::max<int64_t>(1, 8192 / a.pairs));
        dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(a.pairs));
        hipLaunchKernelGGL((k_leaf<D, KT, ST>), grid, dim3(kBlock), lds, st, a, waves);
        return hipGetLastError();
    }
    dim3 grid(static_cast<unsigned>((a.count + (kBlock / 64) - 1) / (kBlock / 64)),
              static_cast<unsigned>(a.pairs));
    if (a.chunk <= 8)
        hipLaunchKernelGGL((k_summarize<D, ST, 8>), grid, dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_summarize<D, ST, 16>), grid, dim3(kBlock), 0, st, a);
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
