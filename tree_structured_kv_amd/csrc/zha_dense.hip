// zha_dense.hip -- the dense full-scan indexer the tree search is measured
// against: exact logits s<q, K_i> for every key, the `budget` highest per
// walk, then attention over exactly those keys.  This is the indexer that
// scores every key before choosing ([ZHA lesson] = the page "How does a tree
// of summaries search a context? How ZHA works", and the news page "Zyphra AI
// Introduces ZHA, a Path to True Subquadratic Attention" on indexers that
// scan the whole context), written from its plain definition.
//
// GPU design.  k_dense_kpass reads every K row once per (sequence, KV head)
// and scores it for all query heads of the group: for bf16 caches that is a
// [keys x D] x [D x heads] contraction done with gfx950's 16x16x32 bf16
// matrix products (heads padded to 16), so the pass stays bound by HBM, not
// by VALU, and each head's fp32 logits leave in 64-byte runs.
// k_dense_select then finds each walk's budget-th largest logit exactly (a
// 12-bit histogram pass, the crossing bin gathered into LDS and narrowed
// there by two 10-bit levels) and compacts the selected indices in ascending
// order: three reads of the walk's logits; among equal logits the lower
// index wins.  Attention reuses the planned split-K kernels with token lists.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t logit_key(float f) {
    if (f != f) f = -INFINITY;
    if (f == 0.f) f = 0.f;
    return ordered_bits(f);
}

}  // namespace

// bf16 logits, keys as the rows of S^T = K Q^T: one wavefront per 128-key
// run (eight 16-key tiles in flight; four were 3% slower), every head of
// the pair as a column
// (16 per tile), gfx950's 16x16x32 bf16 matrix product.  Lane group kb =
// lane/16 owns the D/4 contiguous dims [kb*D/4, (kb+1)*D/4) of both operands
// (a dot product may take its terms in any order, so the k index need only
// agree between the operands), which it reads as 16-byte pieces of its key
// row.  The product's lane holds 4 consecutive keys of one head, stored as
// one float4: each head's logits are written in 64-byte runs, through
// streaming stores (the select reads them back from HBM anyway).
template <int D>
__global__ __launch_bounds__(kBlock) void k_dense_kpass(DenseArgs a) {
    constexpr int PER = D / 4;            // dims per lane group
    constexpr int KS = PER / 8;           // 16x16x32 steps (8 dims a lane each)
    constexpr int UT = 8;                 // 16-key tiles in flight
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.y;
    const int kb = lane >> 4, col = lane & 15;
    const int g_kv = pair % a.kv_heads;
    const int b = pair / a.kv_heads;
    const int64_t n = a.n_tokens;
    const bf16_t *kbase = static_cast<const bf16_t *>(a.k) + static_cast<int64_t>(pair) * a.max_tokens * D + kb * PER;
    const int64_t runs = (n + 16 * UT - 1) / (16 * UT);
    const int64_t rstride = static_cast<int64_t>(gridDim.x) * (kBlock / 64);

    for (int hb = 0; hb < a.group; hb += 16) {
        // query operand: column = head hb + col
        bf16x8_t qb[KS];
        const int h = hb + col;
        const bool hok = h < a.group;
        const int64_t w = static_cast<int64_t>(b) * a.heads + g_kv * a.group + (hok ? h : 0);
        {
            const bf16_t *qp = static_cast<const bf16_t *>(a.q) + w * D + kb * PER;
#pragma unroll
            for (int s = 0; s < KS; ++s) qb[s] = hok ? *reinterpret_cast<const bf16x8_t *>(qp + 8 * s) : bf16x8_t{};
        }
        float *lrow = a.logits + w * a.row_pad;
        for (int64_t run = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + wave; run < runs; run += rstride) {
            const int64_t key0 = run * (16 * UT);
            bf16x8_t kv[UT][KS];
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                int64_t row = key0 + 16 * u + col;
                row = row < n ? row : n - 1;
#pragma unroll
                for (int s = 0; s < KS; ++s) kv[u][s] = *reinterpret_cast<const bf16x8_t *>(kbase + row * D + 8 * s);
            }
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[u][s], qb[s], acc, 0, 0, 0);
                if (!hok) continue;
                const int64_t k4 = key0 + 16 * u + 4 * kb;     // this lane's 4 keys
                const float4 v = make_float4(a.sharpness * acc[0], a.sharpness * acc[1], a.sharpness * acc[2],
                                             a.sharpness * acc[3]);
                if (k4 + 3 < n) {
                    __builtin_nontemporal_store(gf4_t{v.x, v.y, v.z, v.w},
                                                (__attribute__((address_space(1))) gf4_t *)(lrow + k4));
                } else {
                    if (k4 < n) lrow[k4] = v.x;
                    if (k4 + 1 < n) lrow[k4 + 1] = v.y;
                    if (k4 + 2 < n) lrow[k4 + 2] = v.z;
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

// Workgroup (kSelThreads): the bin, among nb bins counted in `copies`
// interleaved copies of a histogram (bin x of copy c at h[c * nb + x]), where
// the count from the top reaches `need`; *above = the count in the bins
// above it.  Bins are scanned from the highest.
__device__ __forceinline__ void top_bin(const uint32_t *h, int copies, int nb, uint32_t need, uint32_t *s_wsum,
                                        uint32_t *s_bin, uint32_t *s_above) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = nb / kSelThreads;     // bins per thread (1 or 4), highest first
    uint32_t cnt[4] = {0, 0, 0, 0}, tsum = 0;
    for (int e = 0; e < per; ++e) {
        const int bin = nb - 1 - per * tid - e;
        uint32_t c = 0;
        for (int cp = 0; cp < copies; ++cp) c += h[cp * nb + bin];
        cnt[e] = c;
        tsum += c;
    }
    const uint32_t incl = wave_scan_u32(tsum);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < wave; ++i) before += s_wsum[i];
    const uint32_t excl = before + incl - tsum;
    if (excl < need && excl + tsum >= need) {
        uint32_t run = excl;
        for (int e = 0; e < per; ++e) {
            if (run + cnt[e] >= need) {
                *s_bin = static_cast<uint32_t>(nb - 1 - per * tid - e);
                *s_above = run;
                break;
            }
            run += cnt[e];
        }
    }
    __syncthreads();
}

// One workgroup per walk: exact top-budget selection over the walk's logits
// (order-preserving 32-bit keys; among equal logits the lower index wins).
//   pass 1: histogram of the top 12 key bits -> the bin holding the
//           budget-th largest key;
//   pass 2: that bin's keys and indices gathered into LDS (at most kSelBuf
//           of them; a larger bin is narrowed by two more passes over the
//           logits and one counting pass instead), where two 10-bit radix
//           levels give the exact key tau, while every wavefront segment of
//           the compaction counts its keys above the bin;
//   pass 3: ordered compaction of the keys above tau and of the first ties,
//           each segment starting at the prefix of those counts.
constexpr int kSelBuf = 8192;
__global__ __launch_bounds__(kSelThreads) void k_dense_select(DenseArgs a) {
    const int w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = a.n_tokens;
    const float *lg = a.logits + static_cast<int64_t>(w) * a.row_pad;
    int32_t *out = a.sel + static_cast<int64_t>(w) * a.max_budget;
    constexpr int kCopies = 4;            // histogram copies: lanes l and l+4 share one
    __shared__ uint32_t buf[2 * kSelBuf]; // pass 1: kCopies x 4096 bins; pass 2: the bin's keys, then indices
    __shared__ uint32_t h2[1024];
    __shared__ uint32_t s_above_seg[kSelWaves], s_tie_seg[kSelWaves];
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ uint32_t s_bin, s_above, s_n;
    __shared__ unsigned long long scan[kSelWaves];

    int64_t k = a.budget[w];
    if (k > n) k = n;
    if (k > a.max_budget) k = a.max_budget;
    if (k < 1 || n < 1) {
        if (tid == 0) a.sel_n[w] = 0;
        return;
    }
    const int copy = lane & (kCopies - 1);
    uint32_t need = static_cast<uint32_t>(k);

    // pass 1: bits [31:20]
    for (int i = tid; i < kCopies * 4096; i += kSelThreads) buf[i] = 0;
    __syncthreads();
    for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * kSelThreads;
            v[u] = (i < n) ? lg[i] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * kSelThreads < n) atomicAdd(&buf[copy * 4096 + (logit_key(v[u]) >> 20)], 1u);
    }
    __syncthreads();
    top_bin(buf, kCopies, 4096, need, wsum, &s_bin, &s_above);
    const uint32_t b1 = s_bin;
    need -= s_above;
    uint32_t in_bin = 0;
    for (int cp = 0; cp < kCopies; ++cp) in_bin += buf[cp * 4096 + b1];
    __syncthreads();

    // compaction segments: wavefront v owns [v*seg, (v+1)*seg), seg a multiple of 64
    const int64_t seg = (((n + kSelWaves - 1) / kSelWaves) + 63) / 64 * 64;
    uint32_t prefix = b1 << 20;
    const bool gathered = in_bin <= static_cast<uint32_t>(kSelBuf);
    uint32_t *bkey = buf, *bidx = buf + kSelBuf;
    if (gathered) {
        // pass 2: gather the bin's keys and indices, count each segment's
        // keys above the bin, then two 10-bit levels in LDS
        if (tid == 0) s_n = 0;
        if (tid < kSelWaves) { s_above_seg[tid] = 0; s_tie_seg[tid] = 0; }
        __syncthreads();
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
                const bool live = i < n;
                if (live && (key >> 20) == b1) {
                    const uint32_t slot = atomicAdd(&s_n, 1u);
                    bkey[slot] = key;
                    bidx[slot] = static_cast<uint32_t>(i);
                }
                // the wavefront's 64 indices lie in one segment
                const uint32_t up = static_cast<uint32_t>(__popcll(__ballot(live && (key >> 20) > b1)));
                if (lane == 0 && up) atomicAdd(&s_above_seg[(i - lane) / seg], up);
            }
        }
        __syncthreads();
        const int nb = static_cast<int>(s_n);
#pragma unroll
        for (int lev = 0; lev < 2; ++lev) {
            const int sh = lev == 0 ? 10 : 0;
            for (int i = tid; i < 1024; i += kSelThreads) h2[i] = 0;
            __syncthreads();
            for (int i = tid; i < nb; i += kSelThreads) {
                const uint32_t key = buf[i];
                if (lev == 0 || (key >> 10) == (prefix >> 10)) atomicAdd(&h2[(key >> sh) & 1023u], 1u);
            }
            __syncthreads();
            top_bin(h2, 1, 1024, need, wsum, &s_bin, &s_above);
            prefix |= s_bin << sh;
            need -= s_above;
            __syncthreads();
        }
        // the gathered keys above tau and equal to it, per segment
        for (int i = tid; i < nb; i += kSelThreads) {
            const uint32_t key = bkey[i];
            const int sg = static_cast<int>(bidx[i] / seg);
            if (key > prefix) atomicAdd(&s_above_seg[sg], 1u);
            else if (key == prefix) atomicAdd(&s_tie_seg[sg], 1u);
        }
        __syncthreads();
    } else {
        // the bin is too large for LDS: two more passes over the logits
        uint32_t *hist = buf;
#pragma unroll
        for (int lev = 0; lev < 2; ++lev) {
            const int sh = lev == 0 ? 10 : 0;
            for (int i = tid; i < 4 * 1024; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t i = i0 + u * kSelThreads;
                    v[u] = (i < n) ? lg[i] : -INFINITY;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t key = logit_key(v[u]);
                    if (i0 + u * kSelThreads < n && (key >> (sh + 10)) == (prefix >> (sh + 10)))
                        atomicAdd(&hist[copy * 1024 + ((key >> sh) & 1023u)], 1u);
                }
            }
            __syncthreads();
            top_bin(hist, kCopies, 1024, need, wsum, &s_bin, &s_above);
            prefix |= s_bin << sh;
            need -= s_above;
            __syncthreads();
        }
    }
    const uint32_t tau = prefix;   // keys > tau open; `need` of the keys == tau open, lowest index first

    // ordered compaction: wavefront v owns the contiguous segment
    // [v*seg, (v+1)*seg) and walks it 64 consecutive logits at a time
    // (coalesced); ballots give each lane its rank inside the step.
    const int64_t s0 = wave * seg;
    const int64_t s1 = (s0 + seg < n) ? s0 + seg : n;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    constexpr int UC = 8;                 // 64-logit steps in flight per wavefront
    uint32_t ca = 0, ct = 0;
    if (gathered) {
        ca = s_above_seg[wave];
        ct = s_tie_seg[wave];
    } else
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

// The bin, among nb bins (counts hc, integer masses hm), where the mass
// summed from the highest bin down first reaches `need`; *s_mab / *s_cab =
// the mass and the count in the bins above it.
__device__ __forceinline__ void top_bin_mass(const uint32_t *hc, const unsigned long long *hm, int nb,
                                             unsigned long long need, unsigned long long *s_wsum, uint32_t *s_bin,
                                             unsigned long long *s_mab, uint32_t *s_cab) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = nb / kSelThreads;     // bins per thread (1 or 4), highest first
    unsigned long long ms[4] = {0, 0, 0, 0}, tsum = 0;
    uint32_t cs[4] = {0, 0, 0, 0}, csum = 0;
    for (int e = 0; e < per; ++e) {
        const int bin = nb - 1 - per * tid - e;
        ms[e] = hm[bin];
        cs[e] = hc[bin];
        tsum += ms[e];
        csum += cs[e];
    }
    // inclusive scans of mass and count over the threads (highest bins first)
    const unsigned long long im = wave_scan_u64(tsum), ic = wave_scan_u64(csum);
    if (lane == 63) { s_wsum[wave] = im; s_wsum[kSelWaves + wave] = ic; }
    __syncthreads();
    unsigned long long bm = 0, bc = 0;
    for (int i = 0; i < wave; ++i) { bm += s_wsum[i]; bc += s_wsum[kSelWaves + i]; }
    const unsigned long long em = bm + im - tsum, ec = bc + ic - csum;
    if (em < need && em + tsum >= need) {
        unsigned long long run = em, rc = ec;
        for (int e = 0; e < per; ++e) {
            if (run + ms[e] >= need) {
                *s_bin = static_cast<uint32_t>(nb - 1 - per * tid - e);
                *s_mab = run;
                *s_cab = static_cast<uint32_t>(rc);
                break;
            }
            run += ms[e];
            rc += cs[e];
        }
    }
    __syncthreads();
}

// Top-p over keys, one workgroup per walk: the length of the smallest prefix
// of the keys ordered by (logit descending, index ascending) whose softmax
// mass reaches p -- the integer masses of the tree's cuts, exp(l - max)*2^31
// rounded, so the sums are exact -- written as the walk's budget for
// k_dense_select, which then selects exactly that prefix.  Four reads of the
// walk's logits: the maximum; a 12-bit histogram of the order-preserving key
// bits with counts and masses (and the total mass); two 10-bit levels on the
// keys of the crossing bin.  The keys equal to the crossing key all carry
// the same mass, so the number of them to take is a division.  p >= 1
// takes every key, p <= 0 the first one.
__global__ __launch_bounds__(kSelThreads) void k_dense_topp_budget(DenseArgs a) {
    const int w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = a.n_tokens;
    const float *lg = a.logits + static_cast<int64_t>(w) * a.row_pad;
    __shared__ uint32_t hc[4096];
    __shared__ unsigned long long hm[4096];
    __shared__ unsigned long long s_wsum[2 * kSelWaves];
    __shared__ float s_red[kSelWaves];
    __shared__ uint32_t s_bin, s_cab;
    __shared__ unsigned long long s_mab;
    int64_t k;
    if (n < 1) {
        k = 0;
    } else if (a.p >= 1.f) {
        k = n;
    } else if (!(a.p > 0.f)) {
        k = 1;
    } else {
        // pass 1: the largest logit
        float m = -INFINITY;
        for (int64_t i = tid; i < n; i += kSelThreads) m = fmaxf(m, lg[i]);
        m = wave_max(m, 1, 64);
        if (lane == 0) s_red[wave] = m;
        __syncthreads();
        float M = s_red[0];
        for (int i = 1; i < kSelWaves; ++i) M = fmaxf(M, s_red[i]);
        auto mass = [&](float v) -> unsigned long long {
            return static_cast<unsigned long long>(__float2uint_rn(mass_exp(v - M) * kMassScale));
        };
        // pass 2: top 12 key bits, counts and masses; the total mass
        for (int i = tid; i < 4096; i += kSelThreads) { hc[i] = 0; hm[i] = 0; }
        __syncthreads();
        unsigned long long z = 0;
        for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * kSelThreads;
                v[u] = (i < n) ? lg[i] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (i0 + u * kSelThreads >= n) continue;
                const uint32_t b = logit_key(v[u]) >> 20;
                const unsigned long long wt = mass(v[u]);
                atomicAdd(&hc[b], 1u);
                if (wt) atomicAdd(&hm[b], wt);
                z += wt;
            }
        }
        z = wave_total_u64(z);
        if (lane == 0) s_wsum[wave] = z;
        __syncthreads();
        unsigned long long Z = 0;
        for (int i = 0; i < kSelWaves; ++i) Z += s_wsum[i];
        __syncthreads();
        unsigned long long need = static_cast<unsigned long long>(ceil(static_cast<double>(a.p) * static_cast<double>(Z)));
        if (need < 1) need = 1;
        if (need > Z) need = Z;
        top_bin_mass(hc, hm, 4096, need, s_wsum, &s_bin, &s_mab, &s_cab);
        uint32_t prefix = s_bin << 20;
        need -= s_mab;
        int64_t above = s_cab;
        // passes 3 and 4: the next 10 bits, then the last 10, of the keys
        // that share the prefix so far
        uint32_t tie_cnt = 0;
        unsigned long long tie_mass = 0;
        for (int lev = 0; lev < 2; ++lev) {
            const int sh = lev == 0 ? 10 : 0;
            __syncthreads();
            for (int i = tid; i < 1024; i += kSelThreads) { hc[i] = 0; hm[i] = 0; }
            __syncthreads();
            for (int64_t i0 = tid; i0 < n; i0 += 4 * kSelThreads) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t i = i0 + u * kSelThreads;
                    v[u] = (i < n) ? lg[i] : -INFINITY;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (i0 + u * kSelThreads >= n) continue;
                    const uint32_t key = logit_key(v[u]);
                    if ((key >> (sh + 10)) != (prefix >> (sh + 10))) continue;
                    const uint32_t b = (key >> sh) & 1023u;
                    const unsigned long long wt = mass(v[u]);
                    atomicAdd(&hc[b], 1u);
                    if (wt) atomicAdd(&hm[b], wt);
                }
            }
            __syncthreads();
            top_bin_mass(hc, hm, 1024, need, s_wsum, &s_bin, &s_mab, &s_cab);
            prefix |= s_bin << sh;
            need -= s_mab;
            above += s_cab;
            tie_cnt = hc[s_bin];
            tie_mass = hm[s_bin];
        }
        // keys equal to the crossing key: equal masses; take as many as the
        // remaining need asks for, lowest index first (k_dense_select)
        const unsigned long long wt = tie_cnt ? tie_mass / tie_cnt : 0ull;
        int64_t take = wt ? static_cast<int64_t>((need + wt - 1) / wt) : static_cast<int64_t>(tie_cnt);
        if (take > tie_cnt) take = tie_cnt;
        if (take < 1) take = 1;
        k = above + take;
    }
    if (tid == 0) {
        int64_t kk = k;
        if (kk > a.max_budget) {
            kk = a.max_budget;
            if (a.status) atomicOr(a.status, ZHA_FLAG_SEL_OVERFLOW);
        }
        a.budget_out[w] = static_cast<int32_t>(kk);
    }
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
        // 128-key runs, about 2048 workgroups of 4 wavefronts in all
        const int64_t runs = (a.n_tokens + 127) / 128;
        int rx = static_cast<int>((runs + 3) / 4);
        if (rx > per_pair) rx = per_pair;
        if (rx < 1) rx = 1;
        dim3 rgrid(static_cast<unsigned>(rx), static_cast<unsigned>(pairs));
        if (D == 64)
            hipLaunchKernelGGL(k_dense_kpass<64>, rgrid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(k_dense_kpass<128>, rgrid, dim3(kBlock), 0, st, a);
    } else {
        if (D == 64)
            hipLaunchKernelGGL(k_dense_logits_f32<64>, grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(k_dense_logits_f32<128>, grid, dim3(kBlock), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.budget_out) {
        // top-p over keys: each walk's prefix length first
        hipLaunchKernelGGL(k_dense_topp_budget, dim3(a.walks), dim3(kSelThreads), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_dense_select, dim3(a.walks), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace zha
