// zha_dense.hip -- the dense full-scan indexer the tree search is measured
// against: exact logits s<q, K_i> for every key, the `budget` highest per
// walk, then attention over exactly those keys.  This is the indexer that
// scores every key before choosing ([ZHA lesson] = the page "How does a tree
// of summaries search a context? How ZHA works", and the news page "Zyphra AI
// Introduces ZHA, a Path to True Subquadratic Attention" on indexers that
// scan the whole context), written from its plain definition.
//
// GPU design.  k_dense_logits reads every K row once per (sequence, KV head)
// and scores it for all query heads of the group: for bf16 caches that is a
// [heads x D] x [D x keys] contraction done with 16x16x16 bf16 MFMA tiles
// (heads padded to 16), so the pass stays bound by HBM, not by VALU.
// k_dense_select then finds each walk's budget-th largest logit exactly with
// an 11 + 11 + 10-bit radix select over order-preserving keys (one read of
// the walk's logits per level; eight copies of the LDS histogram so that
// lanes whose logits share a bin rarely collide on one address) and compacts
// the selected indices in ascending order; among equal logits the lower
// index wins.  Attention reuses the planned split-K kernels with token lists.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t logit_key(float f) {
    if (f != f) f = -INFINITY;
    if (f == 0.f) f = 0.f;
    return ordered_bits(f);
}

}  // namespace

// bf16 logits: one wavefront per 16-key group, all heads of the pair (16 per
// MFMA tile).  The D dimension is split as lane group g = lane/16 owning
// elements [D/4 * g, D/4 * (g+1)) in both operands, so every lane reads one
// contiguous piece of its key row and of each query row.
template <int D>
__global__ __launch_bounds__(kBlock) void k_dense_logits_mfma(DenseArgs a) {
    constexpr int KS = D / 16;            // MFMA steps (16 elements each)
    constexpr int PER = D / 4;            // elements per lane group
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.y;
    const int grp = lane >> 4, col = lane & 15;
    const int g_kv = pair % a.kv_heads;
    const int b = pair / a.kv_heads;
    const int64_t n = a.n_tokens;
    const bf16_t *kb = static_cast<const bf16_t *>(a.k) + static_cast<int64_t>(pair) * a.max_tokens * D;
    const int n_groups = static_cast<int>((n + 15) / 16);

    for (int hb = 0; hb < a.group; hb += 16) {
        // query operand: row = head hb + col of this pair's group
        short4_t qa[KS];
        {
            const int h = hb + col;
            const bool ok = h < a.group;
            const int w = b * a.heads + g_kv * a.group + (ok ? h : 0);
            const bf16_t *qp = static_cast<const bf16_t *>(a.q) + static_cast<int64_t>(w) * D + grp * PER;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                short4_t v;
                v.x = ok ? static_cast<short>(qp[4 * kk + 0]) : 0;
                v.y = ok ? static_cast<short>(qp[4 * kk + 1]) : 0;
                v.z = ok ? static_cast<short>(qp[4 * kk + 2]) : 0;
                v.w = ok ? static_cast<short>(qp[4 * kk + 3]) : 0;
                qa[kk] = v;
            }
        }
        constexpr int UG = 4;                 // 16-key groups in flight per wavefront
        const int gstride = gridDim.x * (kBlock / 64);
        for (int kg0 = blockIdx.x * (kBlock / 64) + wave; kg0 < n_groups; kg0 += gstride * UG) {
            short4_t kbv[UG][KS];
#pragma unroll
            for (int u = 0; u < UG; ++u) {
                const int64_t key = static_cast<int64_t>(kg0 + u * gstride) * 16 + col;
                const int64_t row = key < n ? key : n - 1;
                const bf16_t *kp = kb + row * D + grp * PER;
#pragma unroll
                for (int kk = 0; kk < KS; kk += 2) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(kp + 4 * kk);
                    kbv[u][kk] = short4_t{static_cast<short>(v.x & 0xffff), static_cast<short>(v.x >> 16),
                                          static_cast<short>(v.y & 0xffff), static_cast<short>(v.y >> 16)};
                    kbv[u][kk + 1] = short4_t{static_cast<short>(v.z & 0xffff), static_cast<short>(v.z >> 16),
                                              static_cast<short>(v.w & 0xffff), static_cast<short>(v.w >> 16)};
                }
            }
#pragma unroll
            for (int u = 0; u < UG; ++u) {
                const int64_t key = static_cast<int64_t>(kg0 + u * gstride) * 16 + col;
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qa[kk], kbv[u][kk], acc, 0, 0, 0);
                if (key < n) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int h = hb + 4 * grp + i;
                        if (h < a.group) {
                            const int64_t w = static_cast<int64_t>(b) * a.heads + g_kv * a.group + h;
                            a.logits[w * a.row_pad + key] = a.sharpness * acc[i];
                        }
                    }
                }
            }
        }
    }
}

// fp32 logits (VALU): a wavefront per key row slice, all heads of the pair.
template <int D>
__global__ __launch_bounds__(kBlock) void k_dense_logits_f32(DenseArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.y;
    const int g_kv = pair % a.kv_heads;
    const int b = pair / a.kv_heads;
    const int64_t n = a.n_tokens;
    const float *kb = static_cast<const float *>(a.k) + static_cast<int64_t>(pair) * a.max_tokens * D;
    constexpr int EPL = D / 64;
    for (int64_t key = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + wave; key < n;
         key += static_cast<int64_t>(gridDim.x) * (kBlock / 64)) {
        float kv[EPL];
        for (int e = 0; e < EPL; ++e) kv[e] = kb[key * D + lane * EPL + e];
        for (int h = 0; h < a.group; ++h) {
            const int64_t w = static_cast<int64_t>(b) * a.heads + g_kv * a.group + h;
            const float *qp = static_cast<const float *>(a.q) + w * D;
            float d = 0.f;
            for (int e = 0; e < EPL; ++e) d = fmaf(kv[e], qp[lane * EPL + e], d);
            d = wave_sum(d, 64);
            if (lane == 0) a.logits[w * a.row_pad + key] = a.sharpness * d;
        }
    }
}

// One workgroup per walk: exact top-budget selection over the walk's logits.
__global__ __launch_bounds__(kSelThreads) void k_dense_select(DenseArgs a) {
    const int w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = a.n_tokens;
    const float *lg = a.logits + static_cast<int64_t>(w) * a.row_pad;
    int32_t *out = a.sel + static_cast<int64_t>(w) * a.max_budget;
    constexpr int kCopies = 8;            // histogram copies: lanes l and l+8 share one
    __shared__ uint32_t hist[kCopies][2048];
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ uint32_t s_bin, s_above;
    __shared__ unsigned long long scan[kSelWaves];

    int64_t k = a.budget[w];
    if (k > n) k = n;
    if (k > a.max_budget) k = a.max_budget;
    if (k < 1 || n < 1) {
        if (tid == 0) a.sel_n[w] = 0;
        return;
    }

    // three radix levels over the 32-bit key: bits [31:21], [20:10], [9:0]
    uint32_t prefix = 0;     // decided high bits of the threshold key
    uint32_t need = static_cast<uint32_t>(k);
    const int copy = lane & (kCopies - 1);
#pragma unroll
    for (int lev = 0; lev < 3; ++lev) {
        const int sh = (lev == 0) ? 21 : (lev == 1) ? 10 : 0;
        const int wd = (lev == 2) ? 10 : 11;
        const int nb = 1 << wd;
        for (int i = tid; i < kCopies * 2048; i += kSelThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        const uint32_t want = (lev == 0) ? 0u : (prefix >> (sh + wd));
        for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * kSelThreads;
                v[u] = (i < n) ? lg[i] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * kSelThreads;
                const uint32_t key = logit_key(v[u]);
                const bool match = (i < n) && ((lev == 0) || ((key >> (sh + wd)) == want));
                if (match) atomicAdd(&hist[copy][(key >> sh) & (nb - 1)], 1u);
            }
        }
        __syncthreads();
        // scan bins from the top: thread t holds bins nb-1-2t, nb-2-2t
        uint32_t c2[2], tsum = 0;
        for (int e = 0; e < 2; ++e) {
            const int bin = nb - 1 - 2 * tid - e;
            uint32_t cnt = 0;
            if (bin >= 0)
                for (int cp = 0; cp < kCopies; ++cp) cnt += hist[cp][bin];
            c2[e] = cnt;
            tsum += cnt;
        }
        uint32_t incl = tsum;
        for (int off = 1; off < 64; off <<= 1) {
            uint32_t o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
        for (int i = 0; i < wave; ++i) before += wsum[i];
        const uint32_t excl = before + incl - tsum;
        if (excl < need && excl + tsum >= need) {
            uint32_t run = excl;
            for (int e = 0; e < 2; ++e) {
                if (run + c2[e] >= need) {
                    s_bin = static_cast<uint32_t>(nb - 1 - 2 * tid - e);
                    s_above = run;
                    break;
                }
                run += c2[e];
            }
        }
        __syncthreads();
        prefix |= s_bin << sh;
        need -= s_above;
        __syncthreads();
    }
    const uint32_t tau = prefix;   // keys > tau open; `need` of the keys == tau open, lowest index first

    // ordered compaction: wavefront v owns the contiguous segment
    // [v*seg, (v+1)*seg) and walks it 64 consecutive logits at a time
    // (coalesced); ballots give each lane its rank inside the step.
    const int64_t seg = (((n + kSelWaves - 1) / kSelWaves) + 63) / 64 * 64;
    const int64_t s0 = wave * seg;
    const int64_t s1 = (s0 + seg < n) ? s0 + seg : n;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    constexpr int UC = 8;                 // 64-logit steps in flight per wavefront
    uint32_t ca = 0, ct = 0;
    for (int64_t base0 = s0; base0 < s1; base0 += 64 * UC) {
        uint32_t kv[UC];
#pragma unroll
        for (int u = 0; u < UC; ++u) {
            const int64_t i = base0 + 64 * u + lane;
            kv[u] = (i < s1) ? logit_key(lg[i]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < UC; ++u) {
            const int64_t i = base0 + 64 * u + lane;
            ca += __popcll(__ballot(i < s1 && kv[u] > tau));
            ct += __popcll(__ballot(i < s1 && kv[u] == tau));
        }
    }
    if (lane == 0) scan[wave] = (static_cast<unsigned long long>(ca) << 32) | ct;
    __syncthreads();
    unsigned long long ex = 0;
    for (int i = 0; i < wave; ++i) ex += scan[i];
    uint32_t oa = static_cast<uint32_t>(ex >> 32), ot = static_cast<uint32_t>(ex);
    for (int64_t base0 = s0; base0 < s1; base0 += 64 * UC) {
      uint32_t kv[UC];
#pragma unroll
      for (int u = 0; u < UC; ++u) {
          const int64_t i = base0 + 64 * u + lane;
          kv[u] = (i < s1) ? logit_key(lg[i]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int64_t i = base0 + 64 * u + lane;
        const uint32_t key = kv[u];
        const bool above = i < s1 && key > tau;
        const bool tie = i < s1 && key == tau;
        const unsigned long long ma = __ballot(above), mt = __ballot(tie);
        const uint32_t my_tie = ot + __popcll(mt & below);       // tie rank of this lane
        const bool take_tie = tie && my_tie < need;
        const unsigned long long mtake = __ballot(take_tie);
        const uint32_t ties_before = (ot < need) ? ot : need;    // ties taken before this step
        const uint32_t pos = oa + ties_before + __popcll(ma & below) + __popcll(mtake & below);
        if (above || take_tie) out[pos] = static_cast<int32_t>(i);
        oa += __popcll(ma);
        ot += __popcll(mt);
      }
    }
    if (tid == 0) a.sel_n[w] = static_cast<int32_t>(k);
}

hipError_t launch_dense(const DenseArgs &a, int D, int dtype, hipStream_t st) {
    if (a.walks <= 0 || a.n_tokens <= 0) return hipSuccess;
    const int pairs = a.walks / a.heads * a.kv_heads;
    const int64_t groups = (a.n_tokens + 15) / 16;
    int gx = static_cast<int>((groups + 3) / 4);
    const int per_pair = (2048 + pairs - 1) / pairs;   // about 2048 workgroups in all
    if (gx > per_pair) gx = per_pair;
    if (gx < 1) gx = 1;
    dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(pairs));
    if (dtype == ZHA_BF16) {
        if (D == 64)
            hipLaunchKernelGGL(k_dense_logits_mfma<64>, grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(k_dense_logits_mfma<128>, grid, dim3(kBlock), 0, st, a);
    } else {
        if (D == 64)
            hipLaunchKernelGGL(k_dense_logits_f32<64>, grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(k_dense_logits_f32<128>, grid, dim3(kBlock), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_dense_select, dim3(a.walks), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace zha
