// zha_summary.h -- one tree node from its children, one wavefront per node.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  Section "What does a node summarize?": for every reference
// query rho_r a node keeps one tangent (key_r, bias_r) of its subtree's
// log-sum-exp, made from its c children as
//     sigma_i = s <child key_{i,r}, rho_r> + child bias_{i,r}
//     key_r   = sum_i softmax(sigma)_i child key_{i,r}
//     bias_r  = logsumexp(sigma) - s <key_r, rho_r>
// (a raw key is its own tangent for every reference, with bias 0).  The build
// and append kernels and the one-launch decode step all summarise through
// these two functions, so a node has the same bits whichever made it.
#pragma once

#include "zha_device.h"

namespace zha {

// Level-1 node from a chunk of c raw keys, one wavefront.  rho: the R
// references staged in LDS at row pitch D + 4 floats; kk [c][D + 4], wt
// [R][c], mx_s [R], z_s [R]: this wavefront's LDS scratch; keys: the chunk's
// c rows; ok [R][D], ob [R]: the node's record (global or LDS).
//   1. sigma = s <K_i, rho_r> for every key i and reference r as 16x16x4
//      fp32 matrix products (keys as rows, references as columns), into
//      wt; then lane pair p = r*c + i: max and sum of exp(sigma - max) over
//      the c lanes of reference r; w = softmax;
//   2. lane item (r, 16 elements): key_r = sum_i w_i K_i, written as
//      coalesced 16-float runs; bias_r = max + log(sum) - s <key_r, rho_r>
//      summed over the D/16 lanes of r.
template <int D, typename KT, typename ST>
__device__ __forceinline__ void leaf_node(const float *rho, float *kk, float *wt, float *mx_s, float *z_s,
                                          const KT *keys, ST *ok, float *ob, int R, int c, float s) {
    constexpr int P = D + 4;                    // LDS row pitch (floats)
    constexpr int NS = D / 16;                  // 16-element slices of a row
    const int lane = threadIdx.x & 63;
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
    // 1a. the scores on the matrix cores: in product step m, lane group
    //     q = lane/16 multiplies element q*D/4 + m of key row i (the tile's
    //     row lane%16) and of reference r (column lane%16): one order of the
    //     dot product's terms for every (i, r).  The product's lane holds
    //     keys 4q .. 4q+3 of the tile for reference lane%16.
    {
        constexpr int QD = D / 4;
        const int col = lane & 15, q = lane >> 4;
        const bool rok = col < R;
        const float *qr = rho + (rok ? col : 0) * P + q * QD;
        for (int i0 = 0; i0 < c; i0 += 16) {
            const bool kok = i0 + col < c;
            const float *kr = kk + (kok ? i0 + col : 0) * P + q * QD;
            gf4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < QD; m += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(kr + m);
                const float4 y = *reinterpret_cast<const float4 *>(qr + m);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kok ? x.x : 0.f, rok ? y.x : 0.f, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kok ? x.y : 0.f, rok ? y.y : 0.f, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kok ? x.z : 0.f, rok ? y.z : 0.f, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kok ? x.w : 0.f, rok ? y.w : 0.f, acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + 4 * q + e;
                if (i < c && rok) wt[col * c + i] = s * acc[e];
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    // 1b. softmax weights, one (r, i) pair per lane and round
    for (int p0 = 0; p0 < c * R; p0 += 64) {
        const int pi = p0 + lane;
        const bool live = pi < c * R;
        const int r = live ? pi / c : 0, i = live ? pi % c : 0;
        const float sg = live ? wt[r * c + i] : -INFINITY;
        float m = sg;
        for (int off = 1; off < c; off <<= 1) m = fmaxf(m, xor_lane_f(m, off));
        const float ex = live ? expf(sg - m) : 0.f;
        float z = ex;
        for (int off = 1; off < c; off <<= 1) z += xor_lane_f(z, off);
        if (live) {
            wt[r * c + i] = ex / z;
            if (i == 0) { mx_s[r] = m; z_s[r] = z; }
        }
    }
    __builtin_amdgcn_wave_barrier();
    // 2. keys and biases, one (r, 16 elements) per lane and round.  A lane's
    //    16 elements are 16/G groups of G = 16 bytes / sizeof(ST) consecutive
    //    elements, group e at G*s + NS*G*e for slice s = lane's index among
    //    the NS lanes of reference r: one 16-byte store per group, and the NS
    //    lanes of a reference write NS*G consecutive elements (a 128-byte
    //    line at D = 128) per store instruction.
    constexpr int G = 16 / static_cast<int>(sizeof(ST));
    for (int t0 = 0; t0 < R * NS; t0 += 64) {
        const int ti = t0 + lane;
        const bool live = ti < R * NS;
        const int r = live ? ti / NS : 0, sl = live ? ti % NS : 0;
        auto dim = [&](int k) { return G * sl + NS * G * (k / G) + (k % G); };   // element k's dimension
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        for (int i = 0; i < c; ++i) {
            const float w = wt[r * c + i];
            const float *kr = kk + i * P;
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(kr + dim(e));
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
        const float *qr = rho + r * P;
#pragma unroll
        for (int e = 0; e < 16; ++e) part = fmaf(acc[e], qr[dim(e)], part);
        for (int off = 1; off < NS; off <<= 1) part += xor_lane_f(part, off);
        if (live) {
            if constexpr (sizeof(ST) == 2) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    uint32_t wv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wv[e] = static_cast<uint32_t>(f32_to_bf16(acc[8 * g + 2 * e])) |
                                (static_cast<uint32_t>(f32_to_bf16(acc[8 * g + 2 * e + 1])) << 16);
                    *reinterpret_cast<uint4 *>(ok + r * D + dim(8 * g)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; e += 4)
                    *reinterpret_cast<float4 *>(ok + r * D + dim(e)) =
                        make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            }
            if (sl == 0) ob[r] = (mx_s[r] + logf(z_s[r])) - s * part;
        }
    }
}

// Node of level >= 2 from its c children, one wavefront: child_k(i) is the
// i-th child's key record [R][D], child_b(i) its biases [R] (each in global
// memory or LDS); refs [R][D] the references; sig: 64 floats of LDS for this
// wavefront; ok [R][D], ob [R]: the node's record.  A lane holds D/64
// consecutive elements of every row.
template <int D, typename ST, typename CK, typename CB, int CBT = 16>
__device__ __forceinline__ void upper_node(const float *refs, float *sig, CK child_k, CB child_b, ST *ok,
                                           float *ob, int R, int c, float s) {
    constexpr int EPL = D / 64;                 // elements per lane
    const int lane = threadIdx.x & 63;
    for (int r = 0; r < R; ++r) {
        float rho[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) rho[e] = refs[r * D + lane * EPL + e];
        // scores of the c children under rho_r; the rows of up to CBT
        // children (and their biases) are loaded before any is used, so
        // their loads are in flight together
        float xs[CBT][EPL];
        float bs[CBT];
        float mx = -INFINITY;
        for (int i0 = 0; i0 < c; i0 += CBT) {
#pragma unroll
            for (int u = 0; u < CBT; ++u) {
                if (i0 + u < c) {
                    const ST *ck = child_k(i0 + u);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) xs[u][e] = Elem<ST>::load(ck, r * D + lane * EPL + e);
                    bs[u] = child_b(i0 + u)[r];
                }
            }
#pragma unroll
            for (int u = 0; u < CBT; ++u) {
                if (i0 + u < c) {
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) part = fmaf(xs[u][e], rho[e], part);
                    float dotv = wave_sum(part, 64);
                    float sg = s * dotv + bs[u];
                    if (lane == 0) sig[i0 + u] = sg;
                    mx = fmaxf(mx, sg);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        float z = 0.f;
        for (int i = 0; i < c; ++i) z += expf(sig[i] - mx);
        const float inv_z = 1.f / z;
        // weighted sum of the child keys (rows still in registers when
        // c <= CBT)
        float acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
        if (c <= CBT) {
#pragma unroll
            for (int u = 0; u < CBT; ++u) {
                if (u < c) {
                    const float w = expf(sig[u] - mx) * inv_z;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, xs[u][e], acc[e]);
                }
            }
        } else {
            for (int i = 0; i < c; ++i) {
                const ST *ck = child_k(i);
                const float w = expf(sig[i] - mx) * inv_z;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    float x = Elem<ST>::load(ck, r * D + lane * EPL + e);
                    acc[e] = fmaf(w, x, acc[e]);
                }
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
}  // namespace zha
