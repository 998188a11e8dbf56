// zha_attn_union.hip -- attention over the union of the selected blocks of a
// group of walks that share a KV cache, one matrix-core column per walk.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "Common misunderstandings": every query head walks on its own
// and attends exactly the original keys it selected.  Walks that share a KV
// cache often select the same blocks; here such a block is read once and
// used for every walk of the group that selected it, with a walk mask per
// block.  A group is
//   decode (q_per_head = 1): the G query heads of a (sequence, KV head) pair;
//   prefill blocks: 16 walks of one pair (any of its G x q_per_head query
//                rows), consecutive in the order of a sketch of their
//                selections, so that the walks of a group select alike.
//
//   k_ua_sig     prefill: each walk's sketch, two minhashes of the blocks it
//                selected (for each of two fixed hash functions, the
//                smallest hash over its blocks): walks whose block sets
//                overlap much agree on them often;
//   k_ua_order   prefill: per pair (up to kUaSortMax walks at a time), a
//                bitonic sort in LDS of the (sketch, index) keys; the sorted
//                order, and its inverse, define the groups;
//   k_ua_build   the groups' block masks (16 bits per level-1 block, one per
//                column: the walks that selected it) and chunk bits (one per
//                kUaBlocks blocks), built in LDS one slice of blocks at a time;
//   k_ua_attn    workgroup r of group g takes a range of chunks (the group's
//                last workgroup also the raw tail, which every walk attends);
//                a marked chunk's blocks are compacted in LDS; each wavefront
//                takes 16-key tiles, computes the logits of all columns at
//                once with bf16 16x16x32 matrix products S^T = K Q^T (rows =
//                keys, columns = walks), masks the columns that did not
//                select a key's block, keeps an online softmax per column in
//                fp32 and accumulates O^T += V^T P^T with bf16 products (V
//                exact, P as the sum of two bf16 parts, fp32 sums), its state
//                carried across the chunks; the wavefronts' states are merged
//                in LDS into one partial per (workgroup, column);
//   k_ua_combine one workgroup per decode walk merges its group's partials;
//   k_ua_combine_pf one wavefront per prefill walk merges its group's
//                partials with the block's own keys (k_attn_block).
// A walk's result is the same softmax over the same key set as the per-walk
// kernels of zha_attn.hip, summed in another order.
#include "zha_device.h"
#include "zha_internal.h"

#include <algorithm>

namespace zha {

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kUaWaves = 4;
constexpr int kUaBatch = 1024;         // selected blocks gathered in LDS before their tiles run

// Elements q of four 32-bit words w0..w3 (each two bf16: q = 0 low half, 1
// high half) packed in order as a 16x16x16 operand (two v_perm_b32).
__device__ __forceinline__ short4_t pick4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int q) {
    const uint32_t sel = q ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, sel), hi = __builtin_amdgcn_perm(w3, w2, sel);
    return __builtin_bit_cast(short4_t, make_uint2(lo, hi));
}

__device__ __forceinline__ bf16x8_t as_bf8(gu4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// The running maximum of a column moves only when the column's logits rise
// more than this far above it (base-2 units): weights stay below 2^kLazy and
// the running sums are rescaled rarely (exact: every sum and the final
// normalisation use the same reference).
constexpr float kLazy = 8.f;


// The walks of a pair are consecutive: its G query heads, each with its
// q_per_head query rows.
__device__ __forceinline__ int64_t ua_wpp(const AttnArgs &a) {
    return static_cast<int64_t>(a.group) * a.qph;
}

// The KV pair of group g.
__device__ __forceinline__ int64_t ua_pair(const AttnArgs &a, int64_t g) {
    return a.qph == 1 ? g : g / a.gpp;
}

// The walk of column col of group g, or -1 past the group's walks.
__device__ __forceinline__ int64_t ua_walk(const AttnArgs &a, int64_t g, int col) {
    if (a.qph == 1) return col < a.group ? g * a.group + col : -1;
    const int64_t p = g / a.gpp, wpp = ua_wpp(a);
    const int64_t s = (g - p * a.gpp) * 16 + col;   // sorted position within the pair
    return s < wpp ? p * wpp + a.uperm[p * wpp + s] : -1;
}

// Group and column of walk w.
__device__ __forceinline__ void ua_slot(const AttnArgs &a, int64_t w, int64_t &g, int &col) {
    if (a.qph == 1) {
        g = w / a.group;
        col = static_cast<int>(w - g * a.group);
        return;
    }
    const int64_t wpp = ua_wpp(a);
    const int64_t s = a.uinv[w];
    g = (w / wpp) * a.gpp + s / 16;
    col = static_cast<int>(s % 16);
}

// MurmurHash3's 32-bit finalizer (an invertible mix), over x and a seed.
__device__ __forceinline__ uint32_t ua_mix(uint32_t x, uint32_t seed) {
    x ^= seed;
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

}  // namespace

// Prefill: the sort key of every walk, 16 lanes a walk: the smallest value of
// each of two hash functions over the blocks it selected (ids outside the
// level are ignored; a walk without blocks gets the largest values), then its
// index within its pair's sort segment.  Low bits of the second minhash are
// dropped to make room for the index, which makes every key distinct.
__global__ __launch_bounds__(256) void k_ua_sig(AttnArgs a) {
    constexpr int U = 4;
    const int tid = threadIdx.x, sub = tid & 15;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 16 + (tid >> 4);
    uint32_t m1 = 0xffffffffu, m2 = 0xffffffffu;
    if (w < a.walks) {
        int64_t nb = a.sel_count[w];
        nb = nb < 0 ? 0 : (nb > a.sel_cap ? a.sel_cap : nb);
        const int32_t *sel = a.sel_blocks + w * a.sel_cap;
        for (int64_t i0 = sub; i0 < nb; i0 += 16 * U) {
            int32_t b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = i0 + 16 * u < nb ? sel[i0 + 16 * u] : -1;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (b[u] < 0 || b[u] >= a.n1) continue;
                m1 = min(m1, ua_mix(static_cast<uint32_t>(b[u]), 0x9e3779b9u));
                m2 = min(m2, ua_mix(static_cast<uint32_t>(b[u]), 0x7f4a7c15u));
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        m1 = min(m1, xor_lane_n(m1, off));
        m2 = min(m2, xor_lane_n(m2, off));
    }
    if (w < a.walks && sub == 0) {
        const uint64_t loc = static_cast<uint64_t>((w % ua_wpp(a)) % kUaSortMax);
        a.ukey[w] = (static_cast<uint64_t>(m1) << 32) | (static_cast<uint64_t>(m2 >> 15) << 14) | loc;
    }
}

// Prefill: one workgroup per (pair, segment of kUaSortMax walks) sorts the
// segment's keys ascending in LDS (a bitonic network over the next power of
// two, padded with keys above every real one) and writes the pair-local walk
// at each sorted position (uperm) and the sorted position of each walk
// (uinv).  Keys are distinct, so the order is the same on every run.
__global__ __launch_bounds__(1024) void k_ua_order(AttnArgs a) {
    static_assert(kUaSortMax == 16384, "the key keeps 14 bits of segment index");
    __shared__ unsigned long long s[kUaSortMax];
    const int tid = threadIdx.x;
    const int64_t wpp = ua_wpp(a);
    const int nseg = static_cast<int>((wpp + kUaSortMax - 1) / kUaSortMax);
    const int64_t p = blockIdx.x / nseg;
    const int64_t l0 = static_cast<int64_t>(blockIdx.x - p * nseg) * kUaSortMax;
    const int n = static_cast<int>(min<int64_t>(kUaSortMax, wpp - l0));
    int N = 1;
    while (N < n) N <<= 1;
    const int64_t base = p * wpp + l0;             // first walk of the segment
    for (int i = tid; i < N; i += 1024) s[i] = i < n ? a.ukey[base + i] : ~0ull;
    __syncthreads();
    // each stage as N/2 compare-exchange pairs (i, i + j), i with bit j clear
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int q = tid; q < N / 2; q += 1024) {
                const int i = ((q & ~(j - 1)) << 1) | (q & (j - 1));
                const int ij = i + j;
                const unsigned long long x = s[i], y = s[ij];
                if (((i & k) == 0) ? (x > y) : (x < y)) {
                    s[i] = y;
                    s[ij] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < n; i += 1024) {
        const int loc = static_cast<int>(s[i] & (kUaSortMax - 1));
        a.uperm[base + i] = static_cast<int32_t>(l0 + loc);
        a.uinv[base + loc] = static_cast<int32_t>(l0 + i);
    }
}

// One workgroup (T lanes: 1,024 for decode pairs, whose lists are long; 256
// for prefill groups, which are many and short) per (group, slice of
// kUaSlice level-1 blocks):
// the group's walks' lists, taken as one run of entries, set each walk's
// column bit on the blocks it selected in the slice, in LDS (eight list loads
// in flight per lane); then the slice's masks (zeros included, so nothing
// needs clearing first) and chunk bits go out with plain coalesced stores.
constexpr int kUbLoads = 8;

template <int T>
__global__ __launch_bounds__(T) void k_ua_build(AttnArgs a) {
    static_assert(kUaBlocks == 128 && kUaSlice == 128 * kUaBlocks, "chunk-bit layout");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nsl = static_cast<int>((a.n1 + kUaSlice - 1) / kUaSlice);
    const int64_t g = blockIdx.x / nsl;
    const int sl = static_cast<int>(blockIdx.x - g * nsl);
    const int64_t b0 = static_cast<int64_t>(sl) * kUaSlice;
    const int64_t b1 = min(a.n1, b0 + kUaSlice);
    const int nw = static_cast<int>((b1 - b0 + 1) / 2);      // mask words of the slice
    __shared__ uint32_t sm[kUaSlice / 2];
    __shared__ int64_t s_off[17], s_row[16];      // entry prefix per column; list row start
    __shared__ int32_t s_cbit[kUaSlice / kUaBlocks];
    for (int k = tid; k < kUaSlice / 2; k += T) sm[k] = 0u;
    if (tid == 0) {
        const int ncols = a.qph == 1 ? a.group : 16;
        int64_t off = 0;
        int c = 0;
        for (; c < ncols; ++c) {
            const int64_t w = ua_walk(a, g, c);
            if (w < 0) break;                      // past the group's walks
            int64_t nb = a.sel_count[w];
            nb = nb < 0 ? 0 : (nb > a.sel_cap ? a.sel_cap : nb);
            s_off[c] = off;
            s_row[c] = w * a.sel_cap;
            off += nb;
        }
        for (; c <= 16; ++c) s_off[c] = off;       // empty columns past the walks
    }
    __syncthreads();
    const int64_t total = s_off[16];
    int c = 0;                                     // column of this lane's next entry
    for (int64_t base = 0; base < total; base += T * kUbLoads) {
        int32_t blk[kUbLoads];
        int col[kUbLoads];
#pragma unroll
        for (int u = 0; u < kUbLoads; ++u) {
            const int64_t i = base + u * T + tid;
            blk[u] = -1;
            col[u] = 0;
            if (i < total) {
                while (i >= s_off[c + 1]) ++c;     // entries rise with u, so c only moves up
                col[u] = c;
                blk[u] = a.sel_blocks[s_row[c] + (i - s_off[c])];
            }
        }
#pragma unroll
        for (int u = 0; u < kUbLoads; ++u)
            if (blk[u] >= b0 && blk[u] < b1)
                atomicOr(&sm[(blk[u] - b0) >> 1], (1u << col[u]) << (16 * (blk[u] & 1)));
    }
    __syncthreads();
    uint32_t *mask = reinterpret_cast<uint32_t *>(a.umask) + g * (a.n1cap / 2) + (b0 >> 1);
    for (int k = tid; k < nw; k += T) mask[k] = sm[k];
    // chunk bits: a chunk of kUaBlocks blocks is 64 mask words, one per lane;
    // each wavefront tests CW chunks, then four lanes pack 32 chunks a word
    constexpr int CW = (kUaSlice / kUaBlocks) / (T / 64);
    for (int j = 0; j < CW; ++j) {
        const int ch = wave * CW + j;
        const int k = ch * 64 + lane;
        const uint32_t v = k < nw ? sm[k] : 0u;
        const bool any = __ballot(v != 0u) != 0ull;
        if (lane == 0) s_cbit[ch] = any ? 1 : 0;
    }
    __syncthreads();
    if (tid < 4) {
        uint32_t bits = 0u;
        for (int j = 0; j < 32; ++j) bits |= static_cast<uint32_t>(s_cbit[tid * 32 + j]) << j;
        const int64_t word = b0 / (32 * kUaBlocks) + tid;
        if (word < a.cwords) a.uchunk[g * a.cwords + word] = bits;
    }
}

// NT: key and value rows through streaming (nontemporal) loads.
template <int D, bool NT>
__global__ __launch_bounds__(256) void k_ua_attn(AttnArgs a) {
    constexpr int DS = D / 32;            // bf16 16x16x32 steps of a logit
    constexpr int DT = D / 16;            // row tiles of O^T: row i of tile q is d = DT*i + q
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int c = a.chunk, log2c = a.log2c, wpg = a.items_pp;
    // prefill: neighbouring groups (sorted by sketch) select alike, so runs
    // of them go to one XCD, whose L2 then serves their shared blocks
    const int64_t item = a.qph == 1 ? static_cast<int64_t>(blockIdx.x) : xcd_item(blockIdx.x, a.ugroups * wpg);
    if (item < 0) return;
    const int64_t g = item / wpg;
    const int r = static_cast<int>(item - g * wpg);
    const int64_t p = ua_pair(a, g);
    const int nchunks = static_cast<int>((a.n1 + kUaBlocks - 1) / kUaBlocks);
    const int j0 = r * a.ua_cpw, j1 = min(nchunks, j0 + a.ua_cpw);
    // logits in base-2 units (s * log2(e) * <q, k>), so each weight is one
    // hardware exp2; the partials leave in natural units
    const float s = a.sharpness * 1.4426950408889634f;
    const int64_t tail0 = static_cast<int64_t>(c) * a.n1;
    const int tail_keys = static_cast<int>(a.n_tokens - tail0);
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint16_t *gmask = a.umask + g * a.n1cap;
    const uint32_t *gchunks = a.uchunk + g * a.cwords;
    __shared__ int32_t s_blk[kUaBatch];
    __shared__ uint32_t s_msk[kUaBatch];
    __shared__ int32_t s_cnt[kUaWaves];
    __shared__ float s_m[kUaWaves][16], s_l[kUaWaves][16];
    __shared__ float s_o[kUaWaves][D * 16];
    const bf16_t *kc = static_cast<const bf16_t *>(a.k) + p * a.max_tokens * D;
    const bf16_t *vc = static_cast<const bf16_t *>(a.v) + p * a.max_tokens * D;
    // B operand of S^T: lane (column col, group grp) holds the query of
    // column col at elements 32*st + 8*grp .. +7 (zero past the group's
    // walks); the key rows of the A operand take the same elements (a dot
    // product may sum its terms in any order, so lane group grp may own any
    // slice of the head dimension as long as both operands agree)
    const int64_t qw = ua_walk(a, g, col);
    const bool hv = qw >= 0;
    bf16x8_t qb[DS];
    {
        const bf16_t *qr = static_cast<const bf16_t *>(a.q) + (hv ? qw : 0) * D + 8 * grp;
#pragma unroll
        for (int st = 0; st < DS; ++st) {
            gu4_t v = gload_u4(qr + 32 * st);
            if (!hv) v = gu4_t{0u, 0u, 0u, 0u};
            qb[st] = as_bf8(v);
        }
    }
    // online softmax state of column col, kept across the workgroup's chunks
    float m_run = -INFINITY, l_run = 0.f;
    float4_t acc[DT];
#pragma unroll
    for (int q = 0; q < DT; ++q) acc[q] = float4_t{0.f, 0.f, 0.f, 0.f};
    bool any = false;

    // The workgroup's selected blocks are gathered into an LDS batch (two
    // chunks per round, one wavefront per half chunk) and the batch's keys
    // run as one stream of 16-key tiles, so the tile loop is long and the
    // barriers few even when each chunk holds only a handful of blocks; the
    // raw tail (last workgroup of the group) runs as a pass of its own.
    auto process = [&](const int nkeys, const bool tail_item) {
        auto token_of = [&](int kk) -> int64_t {
            if (tail_item) return tail0 + kk;
            return (static_cast<int64_t>(s_blk[kk >> log2c]) << log2c) + (kk & (c - 1));
        };
        const int ntiles = (nkeys + 15) / 16;
        struct Tile {
            bf16x8_t kb[DS];                  // A operand of S^T
            uint32_t vw[4][DT / 2];           // V rows for O^T += V^T P^T
        };
        // key rows of tile t: for S^T, key kbase + col (same elements as
        // qb); for the second product at step e, key kbase + 4*grp + e,
        // elements DT*col .. DT*col + DT - 1
        auto load_tile = [&](int t, Tile &T) {
            const int kbase = t * 16;
            const int ka = kbase + col;
            const bf16_t *kr = kc + token_of(ka < nkeys ? ka : kbase) * D + 8 * grp;
#pragma unroll
            for (int st = 0; st < DS; ++st) T.kb[st] = as_bf8(NT ? gload_u4_nt(kr + 32 * st) : gload_u4(kr + 32 * st));
            // the lane group's four keys kq .. kq+3 are consecutive rows of
            // one block (blocks hold at least four keys) or of the tail, so
            // one lookup serves all four (keys past the end reuse the first
            // row; their weights are zero)
            const int kq = kbase + 4 * grp;
            const bf16_t *vq = vc + token_of(kq < nkeys ? kq : kbase) * D + DT * col;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16_t *vr = vq + (kq + e < nkeys ? e * D : 0);
                if constexpr (DT == 8) {
                    const gu4_t v = NT ? gload_u4_nt(vr) : gload_u4(vr);
                    T.vw[e][0] = v.x; T.vw[e][1] = v.y; T.vw[e][2] = v.z; T.vw[e][3] = v.w;
                } else {
                    const gu2_t v = NT ? gload_u2_nt(vr) : gload_u2(vr);
                    T.vw[e][0] = v.x; T.vw[e][1] = v.y;
                }
            }
        };
        auto run_tile = [&](int t, const Tile &T) {
            const int kbase = t * 16;
            float4_t sa = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < DS; ++st) sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.kb[st], qb[st], sa, 0, 0, 0);
            // logits of column col for keys kbase + 4*grp + e; masked: -inf
            float x[4], tmax = -INFINITY;
            const int kq = kbase + 4 * grp;
            // the four keys share one block, so one mask
            const bool qok = hv && kq < nkeys && (tail_item || ((s_msk[kq >> log2c] >> col) & 1u));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (qok && kq + e < nkeys) ? s * sa[e] : -INFINITY;
                tmax = fmaxf(tmax, x[e]);
            }
            tmax = fmaxf(tmax, xor_lane_f(tmax, 16));
            tmax = fmaxf(tmax, xor_lane_f(tmax, 32));
            const float mt = fmaxf(m_run, tmax);
            const bool move = mt > m_run + kLazy;
            if (__ballot(move) != 0ull) {
                const float corr = move ? ((m_run > -INFINITY) ? __builtin_amdgcn_exp2f(m_run - mt) : 0.f) : 1.f;
                if (move) m_run = mt;
                l_run *= corr;
#pragma unroll
                for (int q = 0; q < DT; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[q][e] *= corr;
            }
            float pe[4], psum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pe[e] = (x[e] > -INFINITY) ? __builtin_amdgcn_exp2f(x[e] - m_run) : 0.f;
                psum += pe[e];
            }
            psum += xor_lane_f(psum, 16);
            psum += xor_lane_f(psum, 32);
            l_run += psum;
            // O^T += V^T P^T as bf16 16x16x16 products: the probabilities of
            // keys 4*grp .. 4*grp+3 are already this lane's B operand; each is
            // split into two bf16 parts, hi (p truncated) and lo (the exact
            // remainder, rounded: within 2^-16 of p relative), so the fp32
            // sums keep fp32 accuracy while V stays exact
            short4_t ph, pl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t u = __float_as_uint(pe[e]);
                ph[e] = static_cast<short>(u >> 16);
                pl[e] = __builtin_bit_cast(short, static_cast<__bf16>(pe[e] - __uint_as_float(u & 0xffff0000u)));
            }
#pragma unroll
            for (int q = 0; q < DT; ++q) {
                // A operand: element DT*col + q of keys 4*grp + e
                const short4_t va = pick4(T.vw[0][q >> 1], T.vw[1][q >> 1], T.vw[2][q >> 1], T.vw[3][q >> 1], q & 1);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, acc[q], 0, 0, 0);
            }
        };
        // one tile in flight per wavefront (two cost occupancy and were slower)
        for (int t = wave; t < ntiles; t += kUaWaves) {
            Tile T;
            load_tile(t, T);
            run_tile(t, T);
        }
    };
    // the next chunk at or after x in [j0, j1) holding a selected block (j1: none)
    auto next_set = [&](int x) -> int {
        while (x < j1) {
            const uint32_t wd = gchunks[x >> 5] >> (x & 31);
            if (wd != 0u) return x + __ffs(wd) - 1;
            x = (x | 31) + 1;
        }
        return j1;
    };
    int nb = 0;                                    // blocks in the batch
    int ja = next_set(j0);
    while (ja < j1) {
        const int jb = next_set(ja + 1);
        const int jm = (wave < 2) ? ja : jb;
        const int blk = jm * kUaBlocks + (wave & 1) * 64 + lane;
        const uint32_t mk = (jm < j1 && blk < a.n1) ? gmask[blk] : 0u;
        const unsigned long long bal = __ballot(mk != 0u);
        if (lane == 0) s_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = nb, total = nb;
#pragma unroll
        for (int v = 0; v < kUaWaves; ++v) {
            if (v < wave) before += s_cnt[v];
            total += s_cnt[v];
        }
        if (mk != 0u) {
            const int at = before + __popcll(bal & below);
            s_blk[at] = blk;
            s_msk[at] = mk;
        }
        nb = total;
        ja = (jb < j1) ? next_set(jb + 1) : j1;
        __syncthreads();                           // s_cnt is read; the batch entries are written
        if (nb > 0 && (ja >= j1 || nb + 2 * kUaBlocks > kUaBatch)) {
            any = true;
            process(nb * c, false);
            __syncthreads();                       // the tiles read s_blk / s_msk
            nb = 0;
        }
    }
    if (r == wpg - 1 && tail_keys > 0) {
        any = true;
        process(tail_keys, true);
    }
    if (!any) {                                    // uniform: no keys in this workgroup's range
        if (tid == 0) a.ic[item] = 0;
        return;
    }
    // merge the wavefronts' states per column
    if (grp == 0) {
        s_m[wave][col] = m_run * 0.6931471805599453f;   // natural units from here on
        s_l[wave][col] = l_run;
    }
#pragma unroll
    for (int q = 0; q < DT; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_o[wave][(DT * (4 * grp + e) + q) * 16 + col] = acc[q][e];
    __syncthreads();
    for (int i = tid; i < D * 16; i += 256) {
        const int d = i >> 4, h = i & 15;
        float mm = -INFINITY;
#pragma unroll
        for (int v = 0; v < kUaWaves; ++v) mm = fmaxf(mm, s_m[v][h]);
        float ll = 0.f, oo = 0.f;
        if (mm > -INFINITY) {
#pragma unroll
            for (int v = 0; v < kUaWaves; ++v) {
                if (!(s_m[v][h] > -INFINITY)) continue;
                const float f = expf(s_m[v][h] - mm);
                ll = fmaf(s_l[v][h], f, ll);
                oo = fmaf(s_o[v][d * 16 + h], f, oo);
            }
        }
        float *part = a.part + (item * 16 + h) * (D + 2);
        part[2 + d] = oo;
        if (d == 0) {
            part[0] = mm;
            part[1] = ll;
        }
    }
    if (tid == 0) a.ic[item] = 1;
}

// Decode: one workgroup per walk: its group's workgroup flags staged in LDS,
// then each wavefront merges every fourth partial (online, one pass), then
// the four states are merged.
template <int D>
__global__ __launch_bounds__(256) void k_ua_combine(AttnArgs a) {
    constexpr int EPL = D / 64;           // output elements per lane
    const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t g;
    int col;
    ua_slot(a, w, g, col);
    const int wpg = a.items_pp;
    const int64_t i0 = g * wpg;
    __shared__ int32_t s_items[kUaMaxItems];
    __shared__ int32_t s_n;
    __shared__ float s_m[kUaWaves], s_l[kUaWaves], s_acc[kUaWaves][D];
    if (tid == 0) s_n = 0;
    __syncthreads();
    for (int j = tid; j < wpg; j += 256)
        if (a.ic[i0 + j] != 0) s_items[atomicAdd(&s_n, 1)] = j;
    __syncthreads();
    const int n = s_n;
    float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[k] = 0.f;
    for (int x = wave; x < n; x += kUaWaves) {
        const float *pp = a.part + ((i0 + s_items[x]) * 16 + col) * (D + 2);
        const float pm = pp[0], pls = pp[1];
        float v[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[k] = pp[2 + lane * EPL + k];
        if (!(pm > -INFINITY)) continue;
        const float mn = fmaxf(m, pm);
        const float c1 = (m > -INFINITY) ? expf(m - mn) : 0.f, c2 = expf(pm - mn);
        l = l * c1 + pls * c2;
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[k] = acc[k] * c1 + v[k] * c2;
        m = mn;
    }
    if (lane == 0) {
        s_m[wave] = m;
        s_l[wave] = l;
    }
#pragma unroll
    for (int k = 0; k < EPL; ++k) s_acc[wave][lane * EPL + k] = acc[k];
    __syncthreads();
    if (tid < D) {
        float mm = -INFINITY;
#pragma unroll
        for (int v = 0; v < kUaWaves; ++v) mm = fmaxf(mm, s_m[v]);
        float ll = 0.f, av = 0.f;
        if (mm > -INFINITY) {
#pragma unroll
            for (int v = 0; v < kUaWaves; ++v) {
                if (!(s_m[v] > -INFINITY)) continue;
                const float f = expf(s_m[v] - mm);
                ll = fmaf(s_l[v], f, ll);
                av = fmaf(s_acc[v][tid], f, av);
            }
        }
        const float o = (ll > 0.f) ? av / ll : 0.f;
        Elem<bf16_t>::store(static_cast<bf16_t *>(a.out), static_cast<int64_t>(w) * D + tid, o);
    }
}

// Prefill: one wavefront per walk merges its group's partials (in order)
// and the partial of the block's own keys (bpart, from k_attn_block).
template <int D>
__global__ __launch_bounds__(256) void k_ua_combine_pf(AttnArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= a.walks) return;
    int64_t g;
    int col;
    ua_slot(a, w, g, col);
    const int wpg = a.items_pp;
    float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[k] = 0.f;
    auto merge = [&](const float *pp) {
        const float pm = pp[0], pls = pp[1];
        float v[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[k] = pp[2 + lane * EPL + k];
        if (!(pm > -INFINITY)) return;
        const float mn = fmaxf(m, pm);
        const float c1 = (m > -INFINITY) ? expf(m - mn) : 0.f, c2 = expf(pm - mn);
        l = l * c1 + pls * c2;
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[k] = acc[k] * c1 + v[k] * c2;
        m = mn;
    };
    for (int r = 0; r < wpg; ++r)
        if (a.ic[g * wpg + r] != 0) merge(a.part + ((g * wpg + r) * 16 + col) * (D + 2));
    merge(a.bpart + w * (D + 2));
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const float o = (l > 0.f) ? acc[k] / l : 0.f;
        Elem<bf16_t>::store(static_cast<bf16_t *>(a.out), w * D + lane * EPL + k, o);
    }
}

template <int D>
static hipError_t launch_ua_t(const AttnArgs &a, hipStream_t st) {
    const int64_t nsl = std::max<int64_t>(1, (a.n1 + kUaSlice - 1) / kUaSlice);
    const int64_t wg4 = (a.walks + 3) / 4;
    hipError_t e;
    if (a.qph > 1) {
        hipLaunchKernelGGL(k_ua_sig, dim3(static_cast<unsigned>((a.walks + 15) / 16)), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t wpp = static_cast<int64_t>(a.group) * a.qph;
        const int64_t nseg = (wpp + kUaSortMax - 1) / kUaSortMax;
        hipLaunchKernelGGL(k_ua_order, dim3(static_cast<unsigned>(a.pairs * nseg)), dim3(1024), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.n1 > 0) {
        if (a.qph == 1)
            hipLaunchKernelGGL(k_ua_build<1024>, dim3(static_cast<unsigned>(a.ugroups * nsl)), dim3(1024), 0, st, a);
        else
            hipLaunchKernelGGL(k_ua_build<256>, dim3(static_cast<unsigned>(a.ugroups * nsl)), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t items = a.ugroups * a.items_pp;
    // decode reads each selected block once per pair: streaming loads;
    // prefill groups on one XCD share blocks through its L2: ordinary loads
    if (a.qph == 1)
        hipLaunchKernelGGL((k_ua_attn<D, true>), dim3(static_cast<unsigned>(items)), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_ua_attn<D, false>), dim3(static_cast<unsigned>(xcd_grid(items))), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.qph == 1) {
        hipLaunchKernelGGL((k_ua_combine<D>), dim3(a.walks), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if ((e = launch_attn_block(a, D, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_ua_combine_pf<D>), dim3(static_cast<unsigned>(wg4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn_union(const AttnArgs &a, int D, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    return D == 64 ? launch_ua_t<64>(a, st) : launch_ua_t<128>(a, st);
}

}  // namespace zha
