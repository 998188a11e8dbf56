// zha_attn.hip -- split-K decode attention over the selected original keys.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  Sections "How is the tree built?" and "Common
// misunderstandings": the summaries only steer the walk; plain softmax
// attention is then computed over the original keys and values the walk
// picked, and the cache itself is never reduced.  A walk's key set is the c keys of every listed
// level-1 block plus the raw tail past the last whole chunk.
//
// GPU design.  Walks select very different numbers of keys under top-p, so
// the work is planned on the device: k_attn_plan cuts every walk's key list
// into chunks and lays the (walk, chunk) items out flat (512 keys per item
// when the call reads under 2M keys in all, so that long walks spread over
// more workgroups, 2048 from 8M on, where fewer, longer items stream
// better, else 1024);
// k_attn_partial is a grid-stride loop over the items, so every workgroup
// streams about the same number of bytes whatever the spread between walks.
// When the walks together select fewer keys than half of all the pairs'
// cache keys, the heads of a pair rarely share a key and the key and value
// rows come in through streaming (nontemporal) loads; otherwise ordinary
// loads leave the shared rows in L2 for the next head (measured: 256K
// clustered keys, 5% of the keys selected over a pair's heads, 100 -> 92 us;
// 64K AR(1) keys, 80%, 3% slower streamed).  The plan decides it.
// A key row is D*e bytes read as 16-byte pieces by D*e/16 lanes.  The online
// softmax state (max, sum, weighted V) lives per key slot and is merged
// across slots, wavefronts and finally items (k_attn_combine), all in fp32.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Elements q of four 32-bit words w0..w3 (each two bf16: q = 0 low half, 1
// high half) packed in order as a 16x16x16 operand (two v_perm_b32).
__device__ __forceinline__ short4_t pick4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int q) {
    const uint32_t sel = q ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, sel), hi = __builtin_amdgcn_perm(w3, w2, sel);
    return __builtin_bit_cast(short4_t, make_uint2(lo, hi));
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Elements q of eight 32-bit words w[0..7] (each two bf16: q = 0 low half,
// 1 high half) packed in order as a 16x16x32 operand (four v_perm_b32).
__device__ __forceinline__ bf16x8_t pick8(const uint32_t (&w)[8], int q) {
    const uint32_t sel = q ? 0x07060302u : 0x05040100u;
    uint4 r;
    r.x = __builtin_amdgcn_perm(w[1], w[0], sel);
    r.y = __builtin_amdgcn_perm(w[3], w[2], sel);
    r.z = __builtin_amdgcn_perm(w[5], w[4], sel);
    r.w = __builtin_amdgcn_perm(w[7], w[6], sel);
    return __builtin_bit_cast(bf16x8_t, r);
}

// A query's running maximum moves only when its logits rise more than this
// far above it (base-2 units): weights stay below 2^kLazy and the running
// sums are rescaled rarely (exact: every sum and the final normalisation use
// the same reference).
constexpr float kLazy = 8.f;

constexpr int kWaves = kBlock / 64;

// Two online-softmax states with maxima in base-2 units.
__device__ __forceinline__ void merge_state(float &m, float &l, float *acc, float m2, float l2,
                                            const float *acc2, int n) {
    const float mm = fmaxf(m, m2);
    if (!(mm > -INFINITY)) return;   // both empty
    const float c1 = (m > -INFINITY) ? __builtin_amdgcn_exp2f(m - mm) : 0.f;
    const float c2 = (m2 > -INFINITY) ? __builtin_amdgcn_exp2f(m2 - mm) : 0.f;
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
// keys n_tokens .. n_tokens + t (unless k_attn_block takes those).
__device__ __forceinline__ int64_t walk_keys(const AttnArgs &a, int w) {
    const int64_t nb = walk_entries(a, w);
    const int64_t causal = (a.qph > 1 && !a.block_mfma) ? (w % a.qph) + 1 : 0;
    if (a.tokens) return nb + causal;
    return nb * a.chunk + (a.n_tokens - static_cast<int64_t>(a.chunk) * a.n1) + causal;
}

}  // namespace

// One workgroup: the keys per item (from the call's total), item offsets =
// exclusive scan of max(1, ceil(keys / item keys)) over walks, and the walk
// id of every item.
__global__ __launch_bounds__(1024) void k_attn_plan(AttnArgs a) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t carry;
    __shared__ unsigned long long ksum[16];
    __shared__ int32_t s_ck;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long mine = 0;
    for (int w = tid; w < a.walks; w += 1024) mine += static_cast<unsigned long long>(walk_keys(a, w));
    mine = wave_total_u64(mine);
    if (lane == 0) ksum[wave] = mine;
    if (tid == 0) carry = 0;
    __syncthreads();
    if (tid == 0) {
        unsigned long long tot = 0;
        for (int i = 0; i < 16; ++i) tot += ksum[i];
        s_ck = tot < (2ull << 20) ? kChunkMin : (tot < (8ull << 20) ? 1024 : kChunkMax);
        const unsigned long long pairs = static_cast<unsigned long long>(a.walks) / (a.group * a.qph);
        const bool stream = 2 * tot < pairs * static_cast<unsigned long long>(a.n_tokens);
        a.item_off[a.walks + 1] = s_ck | (stream ? kStreamBit : 0);
    }
    __syncthreads();
    const int ck = s_ck;
    for (int base = 0; base < a.walks; base += 1024) {
        const int w = base + tid;
        int32_t cnt = 0;
        if (w < a.walks) {
            const int64_t keys = walk_keys(a, w);
            cnt = static_cast<int32_t>((keys + ck - 1) / ck);
            if (a.block_mfma) ++cnt;                 // the last item: the block's own keys
            if (cnt < 1) cnt = 1;
        }
        const int32_t incl = static_cast<int32_t>(wave_scan_u32(static_cast<uint32_t>(cnt)));
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
    constexpr int U = 4;                  // key rows in flight per lane group (2, 6, 8, 16: slower)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane / LPK, sub = lane % LPK;
    const int c = a.chunk;
    const float s = a.sharpness * 1.4426950408889634f;   // base-2 logits: one hardware exp2 per weight
    const int32_t n_items = a.item_off[a.walks];
    const int32_t plan = a.item_off[a.walks + 1];
    const int ck = plan & ~kStreamBit;          // keys per item (at most kChunkMax)
    __shared__ float sm[kWaves], sl[kWaves], sacc[kWaves][D];
    __shared__ int32_t s_ids[kChunkMax + 1];    // the item's block (or token) ids

    auto items = [&](auto kstream) {
    constexpr bool kStream = decltype(kstream)::value;
    for (int32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int w = a.item_walk[item];
        const int64_t chunk = item - a.item_off[w];
        if (a.block_mfma && item == a.item_off[w + 1] - 1) continue;   // k_attn_block's item
        const int64_t pair = walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
        const int64_t nb = walk_entries(a, w);
        const int64_t body = a.tokens ? nb : nb * c;
        const int64_t tree_keys = a.tokens ? nb : body + (a.n_tokens - static_cast<int64_t>(c) * a.n1);
        const int64_t total = walk_keys(a, w);
        const int64_t k0 = chunk * ck;
        const int64_t k1 = (k0 + ck < total) ? k0 + ck : total;

        float qv[EPL];
        {
            const KT *qp = static_cast<const KT *>(a.q) + static_cast<int64_t>(w) * D;
            for (int e = 0; e < EPL; ++e) qv[e] = Elem<KT>::load(qp, sub * EPL + e);
        }
        const KT *kb = static_cast<const KT *>(a.k) + pair * a.max_tokens * D;
        const KT *vb = static_cast<const KT *>(a.v) + pair * a.max_tokens * D;
        const int32_t *selw = (a.tokens ? a.tokens : a.sel_blocks) + static_cast<int64_t>(w) * a.sel_cap;
        const int64_t tail0 = static_cast<int64_t>(c) * a.n1;
        // the ids this item reads, staged once (the key loop then needs no
        // dependent global load): entries e0 .. e1-1 of the walk's list
        const int64_t kb1 = (k1 < body) ? k1 : body;
        const int64_t e0 = a.tokens ? k0 : k0 / c;
        const int64_t e1 = (kb1 <= k0) ? e0 : (a.tokens ? kb1 : (kb1 + c - 1) / c);
        for (int64_t i = tid; i < e1 - e0; i += kBlock) s_ids[i] = selw[e0 + i];
        __syncthreads();

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
                        const int64_t tk = s_ids[ki - e0];
                        ok[u] = tk >= 0 && tk < a.n_tokens;   // ids outside the cache are skipped
                        tok = ok[u] ? tk : 0;
                    } else if (ki < body) {
                        const int64_t blk = s_ids[ki / c - e0];
                        ok[u] = blk >= 0 && blk < a.n1;    // ids outside the live level are skipped
                        tok = ok[u] ? blk * c + (ki % c) : 0;
                    } else {
                        tok = tail0 + (ki - body);
                    }
                }
                if constexpr (kStream) {
                    Vec16<KT>::load_nt(kb + tok * D + sub * EPL, kr[u]);
                    Vec16<KT>::load_nt(vb + tok * D + sub * EPL, vr[u]);
                } else {
                    Vec16<KT>::load(kb + tok * D + sub * EPL, kr[u]);
                    Vec16<KT>::load(vb + tok * D + sub * EPL, vr[u]);
                }
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
                const float corr = (m > -INFINITY) ? __builtin_amdgcn_exp2f(m - mn) : 0.f;
                const float pe = __builtin_amdgcn_exp2f(lg - mn);
                l = l * corr + pe;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pe, vr[u][e], acc[e] * corr);
                m = mn;
            }
        }

        // merge key slots inside the wavefront (lanes with equal `sub`)
#pragma unroll
        for (int off = LPK; off < 64; off <<= 1) {
            float m2 = xor_lane_f(m, off), l2 = xor_lane_f(l, off), acc2[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc2[e] = xor_lane_f(acc[e], off);
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
            if (tid == 0) { part[0] = mm * 0.6931471805599453f; part[1] = ll; }   // natural units
        }
        __syncthreads();
    }
    };
    if (plan & kStreamBit)
        items(std::true_type{});
    else
        items(std::false_type{});
}

// Prefill: attention of every query of the block over the block's own keys
// (query t sees keys 0..t of the block, at positions n_tokens + 0..t), as a
// partial state in the walk's last work item; k_attn_combine merges it with
// the tree keys' items.  One workgroup per (pair, head, 64-query tile), one
// wavefront per 16 queries; key tiles of 64 go through LDS (K and V
// row-major).  Logits come from bf16 16x16x16 matrix products computed as
// S^T = K Q^T (rows = keys, columns = queries), so the probabilities already
// sit in the B-operand layout of the products O^T += V^T P^T: lane group g
// holds keys 4g .. 4g+3 of a 16-key slice.  Those are bf16 16x16x16 products
// too, with each probability split into two bf16 parts (hi: p truncated, lo:
// the exact remainder rounded; within 2^-16 relative), so the fp32 sums keep
// fp32 accuracy while V stays exact
// (fp32 16x16x4 products would take 16 times the matrix-core time).  Row i of
// output tile q is element d = DT*i + q, so a lane reads the DT consecutive
// elements DT*col .. of each of its keys' V rows once for all tiles.
// Online softmax in fp32.
template <int D>
__global__ __launch_bounds__(256, 3) void k_attn_block(AttnArgs a) {
    constexpr int KT = 64;                 // keys per tile
    constexpr int KP = D + 8;              // sK / sV row pitch (elements)
    constexpr int DS = D / 32;             // bf16 16x16x32 steps of a logit
    constexpr int DT = D / 16;             // output row tiles of O^T
    constexpr int VW = DT / 2;             // 32-bit words of a lane's V slice
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int T = a.qph;
    const int qtiles = (T + 63) / 64;
    // longest query tiles first (causal work grows with the tile)
    const int qt = qtiles - 1 - static_cast<int>(blockIdx.x % qtiles);
    const int hq = static_cast<int>(blockIdx.x / qtiles);      // query head over all pairs
    const int pair = hq / a.group;
    __shared__ bf16_t sK[KT * KP];
    __shared__ bf16_t sV[KT * KP];
    const bf16_t *kbase = static_cast<const bf16_t *>(a.k) + (static_cast<int64_t>(pair) * a.max_tokens + a.n_tokens) * D;
    const bf16_t *vbase = static_cast<const bf16_t *>(a.v) + (static_cast<int64_t>(pair) * a.max_tokens + a.n_tokens) * D;
    const int q0 = qt * 64 + wave * 16;                    // this wavefront's first query
    const int myq = q0 + col;                              // this lane's query (column)
    const int64_t walk = static_cast<int64_t>(hq) * T + (myq < T ? myq : T - 1);
    // B operand of S^T: Q^T, lane (query col, group grp) holds d = 32*k +
    // 8*grp .. +7 (the key rows of the A operand take the same elements: a
    // dot product may sum its terms in any order)
    bf16x8_t qb[DS];
    {
        const bf16_t *qp = static_cast<const bf16_t *>(a.q) + walk * D + 8 * grp;
#pragma unroll
        for (int k = 0; k < DS; ++k) qb[k] = *reinterpret_cast<const bf16x8_t *>(qp + 32 * k);
    }
    // logits in base-2 units (one hardware exp2 per weight); the partial
    // leaves in natural units
    const float s = a.sharpness * 1.4426950408889634f;
    float m = -INFINITY, l = 0.f;
    float4_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    const int last_key = min(T, qt * 64 + 64);             // keys this tile of queries can see
    for (int k0 = 0; k0 < last_key; k0 += KT) {
        __syncthreads();
        // stage keys k0 .. k0+63 (rows past the block are zero)
        for (int idx = tid; idx < KT * (D / 8); idx += 256) {
            const int key = idx / (D / 8), d8 = (idx % (D / 8)) * 8;
            uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
            if (k0 + key < T) {
                kv = *reinterpret_cast<const uint4 *>(kbase + static_cast<int64_t>(k0 + key) * D + d8);
                vv = *reinterpret_cast<const uint4 *>(vbase + static_cast<int64_t>(k0 + key) * D + d8);
            }
            *reinterpret_cast<uint4 *>(sK + key * KP + d8) = kv;
            *reinterpret_cast<uint4 *>(sV + key * KP + d8) = vv;
        }
        __syncthreads();
        if (k0 > q0 + 15) continue;                        // every key of the tile is in this wave's future
        // S^T for 4 slices of 16 keys: lane holds keys 16*sub + 4*grp + e, query col
        float p[4][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            float4_t st = {0.f, 0.f, 0.f, 0.f};
            const bf16_t *kr = sK + (16 * sub + col) * KP + 8 * grp;
#pragma unroll
            for (int k = 0; k < DS; ++k) {
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(kr + 32 * k);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[k], st, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = k0 + 16 * sub + 4 * grp + e;
                const float lg = (key <= myq && key < T) ? s * st[e] : -INFINITY;
                p[sub][e] = lg;
                tmax = fmaxf(tmax, lg);
            }
        }
        // row (query) max over the 4 lane groups holding this column
        tmax = fmaxf(tmax, xor_lane_f(tmax, 16));
        tmax = fmaxf(tmax, xor_lane_f(tmax, 32));
        const float mt = fmaxf(m, tmax);
        const bool move = mt > m + kLazy;
        if (__ballot(move) != 0ull) {
            const float corr = move ? ((m > -INFINITY) ? __builtin_amdgcn_exp2f(m - mt) : 0.f) : 1.f;
            if (move) m = mt;
            l *= corr;
#pragma unroll
            for (int i = 0; i < DT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] *= corr;
        }
        float psum = 0.f;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pe = (p[sub][e] > -INFINITY) ? __builtin_amdgcn_exp2f(p[sub][e] - m) : 0.f;
                p[sub][e] = pe;
                psum += pe;
            }
        psum += xor_lane_f(psum, 16);
        psum += xor_lane_f(psum, 32);
        l += psum;
        // O^T += V^T P^T as bf16 16x16x32 products over 32 keys at a time:
        // the lane's eight K slots are its own keys 16*sub + 4*grp + e of
        // slices sub = 2h, 2h + 1 (any assignment of keys to slots sums the
        // same terms), so its probabilities are already its B operand; each
        // is split into two bf16 parts, hi (p truncated) and lo (the exact
        // remainder, rounded), so the fp32 sums keep fp32 accuracy
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8_t ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = p[2 * h + (e >> 2)][e & 3];
                const uint32_t u = __float_as_uint(pv);
                ph[e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(u >> 16));
                pl[e] = static_cast<__bf16>(pv - __uint_as_float(u & 0xffff0000u));
            }
            uint32_t vw[VW][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = 16 * (2 * h + (e >> 2)) + 4 * grp + (e & 3);
                const uint32_t *vr = reinterpret_cast<const uint32_t *>(sV + key * KP + DT * col);
#pragma unroll
                for (int j = 0; j < VW; ++j) vw[j][e] = vr[j];
            }
#pragma unroll
            for (int q = 0; q < DT; ++q) {
                const bf16x8_t va = pick8(vw[q >> 1], q & 1);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, acc[q], 0, 0, 0);
            }
        }
    }
    if (myq >= T) return;
    // the walk's last item: {m, l, unnormalised sum of p * v}
    float *part = a.bpart ? a.bpart + walk * (D + 2)
                          : a.part + static_cast<int64_t>(a.item_off[walk + 1] - 1) * (D + 2);
#pragma unroll
    for (int q = 0; q < DT; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[2 + DT * (4 * grp + e) + q] = acc[q][e];
    if (grp == 0) {
        part[0] = m * 0.6931471805599453f;         // natural units
        part[1] = l;
    }
}

// One workgroup per walk, lane e = output element e: the items' maxima are
// read spread over the lanes, then the items are merged in order, U at a
// time with their loads issued together.
template <int D, typename KT>
__global__ __launch_bounds__(D) void k_attn_combine(AttnArgs a) {
    constexpr int U = 4;
    const int w = blockIdx.x, e = threadIdx.x;
    const int32_t i0 = a.item_off[w], n = a.item_off[w + 1] - i0;
    const float *part = a.part + static_cast<int64_t>(i0) * (D + 2);
    __shared__ float s_max[D / 64];
    float mm = -INFINITY;
    for (int j = e; j < n; j += D) mm = fmaxf(mm, part[static_cast<int64_t>(j) * (D + 2)]);
    mm = wave_max(mm, 1, 64);
    if ((e & 63) == 0) s_max[e >> 6] = mm;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < D / 64; ++i) mm = fmaxf(mm, s_max[i]);
    float ll = 0.f, av = 0.f;
    if (mm > -INFINITY) {
        for (int j0 = 0; j0 < n; j0 += U) {
            float pm[U], pl[U], pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pm[u] = -INFINITY;
                pl[u] = pv[u] = 0.f;
                if (j0 + u < n) {
                    const float *p = part + static_cast<int64_t>(j0 + u) * (D + 2);
                    pm[u] = p[0];
                    pl[u] = p[1];
                    pv[u] = p[2 + e];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!(pm[u] > -INFINITY)) continue;
                const float cf = expf(pm[u] - mm);
                ll = fmaf(pl[u], cf, ll);
                av = fmaf(pv[u], cf, av);
            }
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
    if constexpr (sizeof(KT) == 2) {
        if (a.block_mfma) {
            const int qtiles = (a.qph + 63) / 64;
            hipLaunchKernelGGL((k_attn_block<D>), dim3(static_cast<unsigned>(a.walks / a.qph * qtiles)), dim3(256),
                               0, st, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL((k_attn_combine<D, KT>), dim3(a.walks), dim3(D), 0, st, a);
    return hipGetLastError();
}

// The block's own keys of a bf16 prefill block alone (the union path
// merges them itself).
hipError_t launch_attn_block(const AttnArgs &a, int D, hipStream_t st) {
    const int qtiles = (a.qph + 63) / 64;
    const dim3 grid(static_cast<unsigned>(a.walks / a.qph * qtiles));
    if (D == 64)
        hipLaunchKernelGGL((k_attn_block<64>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_attn_block<128>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, int D, int dtype, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_attn_t<64, bf16_t>(a, st) : launch_attn_t<64, float>(a, st);
    return dtype == ZHA_BF16 ? launch_attn_t<128, bf16_t>(a, st) : launch_attn_t<128, float>(a, st);
}

}  // namespace zha
