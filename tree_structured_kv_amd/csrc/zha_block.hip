// zha_block.hip -- the block search engine: the walks of a prefill query
// block, scored node-major on matrix cores.
//
// [ZHA lesson] = the page "How does a tree of summaries search a context? How
// ZHA works".  "Common misunderstandings": every head walks the tree on its
// own for every query, so a block of T queries is G*T independent walks per
// (sequence, KV head) pair -- with the same score, cut and opening rules as
// a decode walk ("Run a small tree yourself", "How does top-p differ from
// top-K?").  What the walks share is the tree: thousands of them open the
// same few upper nodes, so the engine scores node-major.  Nothing here
// changes a result: each score is still s<key_r, q> + bias_r maxed over r
// for one (walk, node), and each walk's cut sees only its own candidates.
//
// Per step t:
//   k_bk_score  t = 0: the roots (the same list for every walk) against all
//               the pair's walks, 64 walks x 16 (node, ref) columns per
//               matrix tile group; t > 0: one unit per (parent node, up to
//               64 walks that opened it) scores the parent's c children
//               for those walks.  fp32 16x16x4 matrix products, the node
//               record loaded once per unit and reused by every row tile;
//   k_bk_cut    one wavefront per walk: the exact value-window cut over its
//               candidates (children of the parents it opened, in order),
//               level-1 selections in span order and the higher nodes it
//               opens (its next parents);
//   k_bk_bins   per run of 64 walks of a pair: the walks opening each
//               parent, counted in LDS, then added to the parent's count;
//   k_bk_group  one workgroup: offsets of every parent's walk list (a scan
//               over the counts) and the unit list;
//   k_bk_bins   (fill) per run again: each run reserves its range of every
//               parent's list, then writes its (walk, slot) entries.
// A walk's candidate x is child x % c of its parent x / c (at t = 0: root
// x), so candidate ids are never stored, only each walk's parent list.
#include "zha_device.h"
#include "zha_internal.h"
#include "zha_walk.h"

namespace zha {

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));

// An fp32 value as the exact sum of three bf16 values: hi and mid keep the
// top 8 significant bits of x and of x - hi (truncation leaves an exact
// remainder), and the remaining at most 8 bits fit lo exactly.
__device__ __forceinline__ void split3(float x, short &hi, short &mid, short &lo) {
    const uint32_t u = __float_as_uint(x);
    const float h = __uint_as_float(u & 0xffff0000u);
    const float r = x - h;
    const uint32_t ur = __float_as_uint(r);
    const float m = __uint_as_float(ur & 0xffff0000u);
    const float l = r - m;
    hi = static_cast<short>(u >> 16);
    mid = static_cast<short>(ur >> 16);
    lo = static_cast<short>(__float_as_uint(l) >> 16);
}

constexpr int kBkThreads = 256;        // scorer workgroup
constexpr int kBkRows = 64;            // walks per unit (four row tiles of 16)
constexpr int kGroupThreads = 1024;    // k_bk_group workgroup
constexpr int kBkRun = 64;             // walks per counting / list-filling workgroup
constexpr int kBkHist = 8192;          // parents per pair counted in LDS (32 KB)
constexpr int kBkCutRegs = 16;         // candidates per lane a cut keeps in registers

__device__ __forceinline__ int64_t pair_of(const SearchArgs &a, int w) {
    return walk_pair(w, a.qph, a.heads, a.group, a.kv_heads);
}

// Bin of a parent node (level >= 2) within its pair.
__device__ __forceinline__ int64_t parent_bin(const SearchArgs &a, uint32_t id) {
    return a.bin_lvl[id >> kLevelShift] + (id & kIndexMask);
}

__device__ __forceinline__ uint32_t child_id(uint32_t parent, int e, int c) {
    const uint32_t lvl = parent >> kLevelShift, j = parent & kIndexMask;
    return ((lvl - 1u) << kLevelShift) | (j * static_cast<uint32_t>(c) + static_cast<uint32_t>(e));
}

// Per-wavefront shared state of the cut (one wavefront per workgroup).
struct WaveCut {
    uint32_t hcnt[256];
    unsigned long long hw[256];
    unsigned long long fkey[kWinFinal];
    unsigned long long fw[kWinFinal];
    unsigned long long skey[kWinFinal];
    unsigned long long sw[kWinFinal];
    uint32_t nf;
    uint32_t dig, cnt;
    unsigned long long above;
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) { return wave_total_u64(v); }

}  // namespace

// Roots of the tree (every pair has the same level sizes), and every walk's
// state.
template <int R>
__global__ __launch_bounds__(kBkThreads) void k_bk_init(SearchArgs a, int n0) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        if (tid <= ZHA_MAX_STEPS) a.tile_count[tid] = 0;
        uint32_t flags = 0;
        (void)write_roots(a, a.b_roots, flags);
    }
    // parent counts start at zero (k_bk_group clears them after each use)
    const int64_t nb = static_cast<int64_t>(a.pairs) * a.nbins;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kBkThreads + tid; b < nb;
         b += static_cast<int64_t>(gridDim.x) * kBkThreads)
        a.b_cnt[b] = 0;
    const int w = blockIdx.x * kBkThreads + tid;
    if (w >= a.walks) return;
    WalkState st;
    st.n = n0;
    st.buf = 0;
    st.sel_n = 0;
    st.unforced = 0;
    st.flags = (a.n_roots > a.cand_cap) ? ZHA_FLAG_CAND_OVERFLOW : 0u;
    st.steps = 0;
    for (int i = 0; i < ZHA_MAX_STEPS; ++i) { st.scored[i] = 0; st.opened[i] = 0; }
    a.state[w] = st;
    if (n0 == 0) finish_walk<R>(a, w, 0, st.scored, st.opened, 0, 0, st.flags);
}

// Step t scoring.  A unit is (pair, parent, rows): at t = 0 the parent is
// the root list and the rows are 64 consecutive walks of the pair; later the
// rows are the walks (and their slots) of one opened parent, whose c
// children are the columns.  A wavefront owns column tiles wave, wave+4, ..
// (NPG = 16/R nodes x R references each); it loads a column tile's records
// once and runs every row tile of the unit against them.  bf16 queries: each
// fp32 key element is split into three bf16 parts whose sum is exact
// (split3; one part when the keys are stored in bf16) and every 32-element
// slice of the dot product is three bf16 16x16x32 products (exact bf16
// products summed in fp32, as with fp32 products, in far fewer matrix-core
// cycles); fp32 queries take fp32 16x16x4 products.
template <int D, int R, typename QT, typename ST>
__global__ __launch_bounds__(kBkThreads) void k_bk_score(SearchArgs a, int t, int n0) {
    constexpr int NPG = 16 / R;
    constexpr int KS = D / 4;
    constexpr int kSW = kBkThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    __shared__ const float *s_kap[ZHA_MAX_LEVELS + 1];
    __shared__ const float *s_bet[ZHA_MAX_LEVELS + 1];
    __shared__ int64_t s_cap[ZHA_MAX_LEVELS + 1];
    if (threadIdx.x <= ZHA_MAX_LEVELS) {
        s_kap[threadIdx.x] = a.kap[threadIdx.x];
        s_bet[threadIdx.x] = a.bet[threadIdx.x];
        s_cap[threadIdx.x] = a.cap[threadIdx.x];
    }
    __syncthreads();
    const int c = a.chunk;
    const int pw = a.group * a.qph;                       // walks per pair
    const int upp = (pw + kBkRows - 1) / kBkRows;         // root units per pair
    const int n_units = (t == 0) ? a.pairs * upp : a.tile_count[t];
    const int per = (n_units + gridDim.x - 1) / gridDim.x;
    const int u0 = blockIdx.x * per, u1 = min(n_units, u0 + per);
    const float s = a.sharpness;
    const int cap = a.cand_cap;
    const bool mark = a.visited != nullptr;
    // the unit's rows: walk, candidate slot base and query, staged in LDS
    // once per unit (the row loop then has no dependent global load)
    constexpr int QP = D + 16 / static_cast<int>(sizeof(QT));   // s_q row pitch (elements)
    constexpr int PPR = D * static_cast<int>(sizeof(QT)) / 16;  // 16-byte pieces per query row
    __shared__ int32_t s_walk[kBkRows], s_slot[kBkRows];
    __shared__ __align__(16) QT s_q[kBkRows * QP];

    for (int unit = u0; unit < u1; ++unit) {
        int pair, rows, first;
        uint32_t parent = 0;
        int nchild;
        if (t == 0) {
            pair = unit / upp;
            first = pair * pw + (unit % upp) * kBkRows;   // first walk
            rows = min(kBkRows, (pair + 1) * pw - first);
            nchild = n0;
        } else {
            const int4 u = a.b_units[unit];
            pair = u.x;
            parent = static_cast<uint32_t>(u.y);
            first = u.z;                                  // first entry of b_inv
            rows = u.w;
            nchild = c;
        }
        const int n_ct = (nchild + NPG - 1) / NPG;
        const int n_rt = (rows + 15) / 16;
        // walk and candidate slot base of output row r of row tile rt
        auto row_of = [&](int r, int &walk, int &slot0) {
            if (t == 0) {
                walk = first + r;
                slot0 = 0;
            } else {
                const int2 e = a.b_inv[first + r];
                walk = e.x;
                slot0 = e.y * c;
            }
        };
        __syncthreads();                                  // the previous unit is done with s_*
        for (int idx = threadIdx.x; idx < kBkRows * PPR; idx += kBkThreads) {
            const int r = idx / PPR, pc = idx - r * PPR;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r < rows) {
                int walk, slot0;
                row_of(r, walk, slot0);
                v = *reinterpret_cast<const uint4 *>(static_cast<const QT *>(a.q) + static_cast<int64_t>(walk) * D +
                                                     pc * (16 / static_cast<int>(sizeof(QT))));
                if (pc == 0) {
                    s_walk[r] = walk;
                    s_slot[r] = slot0;
                }
            }
            *reinterpret_cast<uint4 *>(s_q + r * QP + pc * (16 / static_cast<int>(sizeof(QT)))) = v;
        }
        __syncthreads();
        for (int ct = wave; ct < n_ct; ct += kSW) {
            // this lane's column: node ct*NPG + col/R, reference col%R
            const int ci = min(ct * NPG + col / R, nchild - 1);
            const uint32_t id = (t == 0) ? a.b_roots[ci] : child_id(parent, ci, c);
            const int lvl = static_cast<int>(id >> kLevelShift);
            const int64_t node = static_cast<int64_t>(pair) * s_cap[lvl] + (id & kIndexMask);
            // bf16 queries: each 32-element slice j of the dot product is
            // NP bf16 16x16x32 products (the key as three exact bf16 parts;
            // one when the keys are stored in bf16), lane group grp taking
            // elements 32*j + 8*grp .. +7 of the query row and of the
            // reference row; fp32 queries: fp32 16x16x4 products, lane group
            // grp taking elements 16*j + 4*grp .. +3
            constexpr int NJ = D / 32;
            constexpr int NP = (sizeof(ST) == 2) ? 1 : 3;     // bf16 keys are their own hi part
            const ST *krow = reinterpret_cast<const ST *>(s_kap[lvl]) + node * (R * D) + (col % R) * D;
            float kb[KS];
            short8_t kbf[NP][NJ];
            if constexpr (sizeof(QT) == 2) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    GVec4<ST>::load(krow + 32 * j + 8 * grp, &kb[8 * j]);
                    GVec4<ST>::load(krow + 32 * j + 8 * grp + 4, &kb[8 * j + 4]);
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        short hi, mid, lo;
                        split3(kb[8 * j + i], hi, mid, lo);
                        kbf[0][j][i] = hi;
                        if constexpr (NP == 3) {
                            kbf[1][j][i] = mid;
                            kbf[2][j][i] = lo;
                        }
                    }
            } else {
#pragma unroll
                for (int k = 0; k < KS; k += 4) GVec4<ST>::load(krow + 4 * grp + 4 * k, &kb[k]);
            }
            const float bias = gload_f(s_bet[lvl] + node * R + (col % R));
            if (mark && (col % R) == 0 && grp == 0 && ct * NPG + col / R < nchild) {
                const int64_t bitn = a.node_off[lvl] + (id & kIndexMask);
                atomicOr(a.visited + static_cast<int64_t>(pair) * a.vis_words + (bitn >> 5), 1u << (bitn & 31));
            }
            for (int rt = 0; rt < n_rt; ++rt) {
                // query operand: row `col` of this tile (zero past the unit)
                const QT *qr = s_q + (rt * 16 + col) * QP + 4 * grp;
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (sizeof(QT) == 2) {
                    const QT *qr8 = s_q + (rt * 16 + col) * QP + 8 * grp;
                    bf16x8_t qa[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) qa[j] = *reinterpret_cast<const bf16x8_t *>(qr8 + 32 * j);
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                qa[j], __builtin_bit_cast(bf16x8_t, kbf[pp][j]), acc, 0, 0, 0);
                } else {
#pragma unroll
                    for (int j = 0; j < KS / 4; ++j) {
                        const float4_t qv = *reinterpret_cast<const float4_t *>(qr + 16 * j);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[i], kb[4 * j + i], acc, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = fmaf(s, acc[e], bias);
                    v = group_max<R>(v);
                    if (v != v) v = -INFINITY;
                    if (v == 0.f) v = 0.f;
                    const int r = rt * 16 + 4 * grp + e;
                    const int child = ct * NPG + col / R;
                    if ((col % R) == 0 && r < rows && child < nchild) {
                        const int slot = s_slot[r] + child;
                        if (slot < cap) a.score[static_cast<int64_t>(s_walk[r]) * cap + slot] = v;
                    }
                }
            }
        }
    }
}

// Step t cut, one wavefront (workgroup) per walk.  Its scores and candidate
// ids are loaded into registers once, all loads in flight, when there are at
// most 64 * kBkCutRegs candidates (the passes then read no memory); longer
// lists are read kBkCutRegs a lane at a time in every pass.
template <int R>
__global__ __launch_bounds__(64) void k_bk_cut(SearchArgs a, int t) {
    constexpr int KR = kBkCutRegs;
    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    __shared__ WaveCut sh;
    // the walk state's scalar fields only: a copy of the whole record (with
    // its per-step arrays written at a runtime step) would live in scratch
    WalkState *gst = a.state + w;
    const int n = gst->n;
    if (n <= 0) return;                                   // finished earlier
    const int buf = gst->buf;
    const int32_t sel_n0 = gst->sel_n, unforced0 = gst->unforced;
    uint32_t st_flags = gst->flags;
    const int cap = a.cand_cap, c = a.chunk, log2c = a.log2c;
    uint32_t *parents = a.cand + static_cast<int64_t>(w) * 2 * cap;
    const uint32_t *par_cur = parents + static_cast<int64_t>(buf) * cap;
    uint32_t *par_nxt = parents + static_cast<int64_t>(buf ^ 1) * cap;
    const float *sc = a.score + static_cast<int64_t>(w) * cap;
    int32_t *selw = a.sel_blocks + static_cast<int64_t>(w) * a.sel_cap;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    auto cand_id = [&](int x) -> uint32_t {
        if (t == 0) return a.b_roots[x];
        return child_id(par_cur[x >> log2c], x & (c - 1), c);
    };
    const bool staged = n <= 64 * KR;
    float vr[KR];
    uint32_t ir[KR];
    if (staged) {
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int x = lane + 64 * i;
            vr[i] = x < n ? sc[x] : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int x = lane + 64 * i;
            ir[i] = x < n ? cand_id(x) : 0u;
        }
    }
    // f(score, x, id, x < n) for x = lane, lane + 64, ... (every lane takes
    // part in every round of 64 candidates; rounds in increasing x); ids are
    // read only when asked for
    auto rounds = [&](bool want_id, auto &&f) {
        if (staged) {
            const int nr = (n + 63) >> 6;
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                if (i >= nr) break;
                const int x = lane + 64 * i;
                f(vr[i], x, ir[i], x < n);
            }
            return;
        }
        for (int x0 = 0; x0 < n; x0 += 64 * KR) {
            float v[KR];
            uint32_t id[KR];
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                const int x = x0 + lane + 64 * i;
                v[i] = x < n ? sc[x] : -INFINITY;
                id[i] = 0u;
            }
            if (want_id) {
#pragma unroll
                for (int i = 0; i < KR; ++i) {
                    const int x = x0 + lane + 64 * i;
                    id[i] = x < n ? cand_id(x) : 0u;
                }
            }
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                if (x0 + 64 * i >= n) break;
                const int x = x0 + lane + 64 * i;
                f(v[i], x, id[i], x < n);
            }
        }
    };

    const bool forced = step_forced(a, t, n);
    unsigned long long tau = 0;
    uint32_t path = staged ? 0u : kPathLongList;
    if (!forced && n <= 64) {
        // one candidate per lane (staged: vr[0], ir[0]): the sort-based cut
        const bool in = lane < n;
        tau = lane_tau(a, in, vr[0], ir[0], wave_max(vr[0], 1, 64), n, a.k[t]);
    } else if (!forced) {
        const bool by_mass = (a.mode == ZHA_TOPP) && (a.p > 0.f);
        float mx = -INFINITY;
        rounds(false, [&](float v, int, uint32_t, bool in) {
            if (in) mx = fmaxf(mx, v);
        });
        mx = wave_max(mx, 1, 64);
        bool exact_done = false;
        if (mx > -INFINITY) {
            float mn = mx;
            unsigned long long z = 0;
            rounds(false, [&](float v, int, uint32_t, bool in) {
                if (!in) return;
                if (v > -INFINITY) mn = fminf(mn, v);
                if (by_mass) z += static_cast<unsigned long long>(__float2uint_rn(mass_exp(v - mx) * kMassScale));
            });
            mn = -wave_max(-mn, 1, 64);
            z = wave_sum_u64(z);
            unsigned long long need;
            if (by_mass) {
                const double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
                need = static_cast<unsigned long long>(tq);
                if (need < 1) need = 1;
                if (need > z) need = z;
            } else {
                const int m = (a.mode == ZHA_TOPK) ? (a.k[t] < n ? a.k[t] : n) : 1;
                need = static_cast<unsigned long long>(m < 1 ? 1 : m);
            }
            // value-window passes (as cut_tau_win, one wavefront)
            float top = mx, bot = by_mass ? fmaxf(mn, mx - 23.f) : mn;
            float w_top[kWinPasses], w_scale[kWinPasses];
            int w_bin[kWinPasses];
            int depth = 0;
            bool found = false;
            // the windows live in registers: every index below is a
            // compile-time constant (a runtime index would put the arrays in
            // scratch memory)
#pragma unroll
            for (int q = 0; q < kWinPasses; ++q) { w_top[q] = 0.f; w_scale[q] = 0.f; w_bin[q] = 0; }
            auto in_window = [&](float v) -> bool {
                bool inw = true;
#pragma unroll
                for (int q = 0; q < kWinPasses; ++q)
                    if (q < depth) inw = inw && win_bin(v, w_top[q], w_scale[q]) == w_bin[q];
                return inw;
            };
            for (; depth < kWinPasses; ++depth) {
                if (!(top > bot)) break;
                const float scale = 256.f / (top - bot);
#pragma unroll
                for (int q = 0; q < kWinPasses; ++q) {
                    if (q == depth) {
                        w_top[q] = top;
                        w_scale[q] = scale;
                    }
                }
                for (int i = lane; i < 256; i += 64) { sh.hcnt[i] = 0; sh.hw[i] = 0; }
                __syncthreads();
                rounds(false, [&](float v, int, uint32_t, bool in) {
                    if (!in) return;
                    if (!in_window(v)) return;
                    const int b = win_bin(v, top, scale);
                    unsigned long long wgt = 1;
                    if (by_mass) wgt = static_cast<unsigned long long>(__float2uint_rn(mass_exp(v - mx) * kMassScale));
                    atomicAdd(&sh.hcnt[b], 1u);
                    if (wgt) atomicAdd(&sh.hw[b], wgt);
                });
                __syncthreads();
                {
                    unsigned long long lw[4], lsum = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lw[e] = by_mass ? sh.hw[4 * lane + e] : sh.hcnt[4 * lane + e];
                        lsum += lw[e];
                    }
                    unsigned long long incl = wave_scan_u64(lsum);
                    const unsigned long long excl = incl - lsum;
                    const unsigned long long mask = __ballot(incl >= need);
                    const int firstl = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : 63;
                    if (lane == firstl) {
                        unsigned long long run = excl;
                        int pick = 3;
                        for (int e = 0; e < 4; ++e) {
                            if (run + lw[e] >= need) { pick = e; break; }
                            run += lw[e];
                        }
                        if (!mask) { pick = 3; run = excl + lw[0] + lw[1] + lw[2]; }
                        sh.dig = 4u * lane + pick;
                        sh.above = run;
                        sh.cnt = sh.hcnt[4 * lane + pick];
                    }
                }
                __syncthreads();
                const int b = static_cast<int>(sh.dig);
                need -= sh.above;
#pragma unroll
                for (int q = 0; q < kWinPasses; ++q)
                    if (q == depth) w_bin[q] = b;
                const uint32_t cb = sh.cnt;
                __syncthreads();
                if (cb <= static_cast<uint32_t>(kWinFinal)) { ++depth; found = true; break; }
                const float nt = top - static_cast<float>(b) / scale;
                const float nb = top - static_cast<float>(b + 1) / scale;
                top = fminf(nt, top);
                bot = fmaxf(nb, bot);
            }
            if (found) {
                if (lane == 0) sh.nf = 0;
                __syncthreads();
                rounds(true, [&](float v, int, uint32_t id, bool in) {
                    if (!in) return;
                    if (!in_window(v)) return;
                    const uint32_t slot = atomicAdd(&sh.nf, 1u);
                    if (slot < static_cast<uint32_t>(kWinFinal)) {
                        sh.fkey[slot] = rank_key(v, id, log2c);
                        sh.fw[slot] = by_mass ? static_cast<unsigned long long>(
                                                    __float2uint_rn(mass_exp(v - mx) * kMassScale))
                                              : 1ull;
                    }
                });
                __syncthreads();
                const int nf = static_cast<int>(sh.nf < static_cast<uint32_t>(kWinFinal) ? sh.nf : kWinFinal);
                if (lane < nf) {
                    const unsigned long long k = sh.fkey[lane];
                    int r = 0;
                    for (int j = 0; j < nf; ++j) r += sh.fkey[j] > k;
                    sh.skey[r] = k;
                    sh.sw[r] = sh.fw[lane];
                }
                __syncthreads();
                unsigned long long wv = lane < nf ? sh.sw[lane] : 0ull;
                unsigned long long incl = wave_scan_u64(wv);
                const unsigned long long hit = __ballot(lane < nf && incl >= need);
                const int r = hit ? (__ffsll(static_cast<long long>(hit)) - 1) : (nf - 1);
                tau = (nf > 0) ? sh.skey[r] : 0ull;
                __syncthreads();
                exact_done = true;
            }
        }
        if (!exact_done) {
            // every score -inf, or a window that cannot be split: sort-free
            // fallback over full keys, one candidate at a time (rare)
            path |= kPathTieSelect;
            unsigned long long need = 1;
            const bool by_mass2 = (a.mode == ZHA_TOPP) && (a.p > 0.f) && (mx > -INFINITY);
            unsigned long long z = 0;
            for (int x = lane; x < n; x += 64)
                z += by_mass2 ? static_cast<unsigned long long>(__float2uint_rn(mass_exp(sc[x] - mx) * kMassScale)) : 1ull;
            z = wave_sum_u64(z);
            if (a.mode == ZHA_TOPK) {
                need = static_cast<unsigned long long>(a.k[t] < n ? a.k[t] : n);
            } else if (a.p > 0.f) {
                const double tq = ceil(static_cast<double>(a.p) * static_cast<double>(z));
                need = static_cast<unsigned long long>(tq);
                if (need < 1) need = 1;
                if (need > z) need = z;
            }
            // tau = the largest key whose weight at or above it reaches need
            unsigned long long best = 0;
            for (int x = lane; x < n; x += 64) {
                const unsigned long long kx = rank_key(sc[x], cand_id(x), log2c);
                unsigned long long above = 0;
                for (int y = 0; y < n; ++y) {
                    const unsigned long long ky = rank_key(sc[y], cand_id(y), log2c);
                    if (ky >= kx)
                        above += by_mass2 ? static_cast<unsigned long long>(__float2uint_rn(mass_exp(sc[y] - mx) * kMassScale))
                                          : 1ull;
                }
                if (above >= need && kx > best) best = kx;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned long long o = xor_lane64_n(best, off);
                best = o > best ? o : best;
            }
            tau = best;
        }
    }

    // open, in candidate order
    const int pcap = a.pcap;
    uint32_t n1 = 0, nh = 0, nopen = 0;
    rounds(true, [&](float v, int, uint32_t idx, bool in) {
        bool open = false;
        uint32_t id = 0;
        if (in) {
            id = idx;
            open = forced || rank_key(v, id, log2c) >= tau;
        }
        const bool l1 = open && (id >> kLevelShift) == 1u;
        const bool hi = open && (id >> kLevelShift) > 1u;
        const unsigned long long m1 = __ballot(l1), mh = __ballot(hi);
        if (l1) {
            const int64_t pos = static_cast<int64_t>(sel_n0) + n1 + __popcll(m1 & below);
            if (pos < a.sel_cap) selw[pos] = static_cast<int32_t>(id & kIndexMask);
        }
        if (hi) {
            const uint32_t j = nh + __popcll(mh & below);
            if (static_cast<int>(j) < pcap) par_nxt[j] = id;
        }
        n1 += __popcll(m1);
        nh += __popcll(mh);
        nopen += __popcll(__ballot(open));
    });
    int64_t nn = static_cast<int64_t>(nh) * c;
    if (nn > cap) { st_flags |= ZHA_FLAG_CAND_OVERFLOW; nn = cap; }
    st_flags |= path;
    const int32_t unforced = forced ? unforced0 : unforced0 + n;
    const int32_t sel_n = sel_n0 + static_cast<int32_t>(n1);
    const bool done = nn == 0 || t + 1 >= a.levels || t + 1 >= ZHA_MAX_STEPS;
    if (lane == 0) {
        gst->scored[t] = n;
        gst->opened[t] = static_cast<int32_t>(nopen);
        gst->flags = st_flags;
        gst->unforced = unforced;
        gst->sel_n = sel_n;
        gst->steps = t + 1;
        gst->buf = buf ^ 1;
        gst->n = done ? 0 : static_cast<int32_t>(nn);
        if (done) finish_walk<R>(a, w, t + 1, gst->scored, gst->opened, sel_n, unforced, st_flags);
    }
}

// Offsets of every parent's walk list (exclusive scan of the counts, pair
// after pair) and the unit list; clears the counts for the next step.
__global__ __launch_bounds__(kGroupThreads) void k_bk_group(SearchArgs a, int t) {
    __shared__ unsigned long long scan[kGroupThreads / 64];
    __shared__ unsigned long long carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t total = static_cast<int64_t>(a.pairs) * a.nbins;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int64_t b0 = 0; b0 < total; b0 += kGroupThreads) {
        const int64_t b = b0 + tid;
        int cnt = 0;
        if (b < total) {
            cnt = a.b_cnt[b];
            a.b_cnt[b] = 0;
            a.b_fill[b] = 0;
        }
        const unsigned long long units = static_cast<unsigned long long>((cnt + kBkRows - 1) / kBkRows);
        // entries in the low 40 bits, units in the high 24
        const unsigned long long v = static_cast<unsigned long long>(cnt) | (units << 40);
        unsigned long long incl = wave_scan_u64(v);
        if (lane == 63) scan[wave] = incl;
        __syncthreads();
        unsigned long long before = carry;
        for (int i = 0; i < wave; ++i) before += scan[i];
        const unsigned long long excl = before + incl - v;
        if (b < total) {
            const int first = static_cast<int>(excl & ((1ull << 40) - 1));
            const int ufirst = static_cast<int>(excl >> 40);
            a.b_first[b] = first;
            if (cnt > 0) {
                const int pair = static_cast<int>(b / a.nbins);
                const int64_t local = b - static_cast<int64_t>(pair) * a.nbins;
                int lvl = 2;
                while (lvl < a.levels && local >= a.bin_lvl[lvl + 1]) ++lvl;
                const uint32_t parent = (static_cast<uint32_t>(lvl) << kLevelShift) |
                                        static_cast<uint32_t>(local - a.bin_lvl[lvl]);
                for (int k = 0; k < static_cast<int>(units); ++k)
                    a.b_units[ufirst + k] = make_int4(pair, static_cast<int>(parent), first + k * kBkRows,
                                                      min(kBkRows, cnt - k * kBkRows));
            }
        }
        __syncthreads();
        if (tid == kGroupThreads - 1) carry = excl + v;
        __syncthreads();
    }
    if (tid == 0) a.tile_count[t] = static_cast<int32_t>(carry >> 40);
}

// The parents walk w's next cut scores the children of (its current parent
// list, after its cut), or 0 when that cut needs no scores.
__device__ __forceinline__ int bk_parents(const SearchArgs &a, int w, const uint32_t *&par) {
    const int n = a.state[w].n;
    const int t1 = a.state[w].steps;                      // the step about to be cut
    if (n <= 0 || step_forced(a, t1, n)) return 0;
    par = a.cand + static_cast<int64_t>(w) * 2 * a.cand_cap + static_cast<int64_t>(a.state[w].buf) * a.cand_cap;
    return (n + a.chunk - 1) / a.chunk;
}

// One workgroup per run of kBkRun walks of one pair (four wavefronts, a walk
// each at a time).  !FILL: every walk counts under each parent it opened
// (b_cnt, before k_bk_group); FILL: its (walk, slot) entries go into those
// parents' lists (b_inv, after k_bk_group).  Thousands of walks open the
// same upper parents, so the run first counts in LDS and then touches each
// parent's global counter once: one atomic per (run, parent) instead of one
// per (walk, parent).  The order of a parent's entries is whatever the
// atomics give; a score does not depend on its row in a tile, so results do
// not.  With more than kBkHist parents per pair the entries take one global
// atomic each.
template <bool FILL>
__global__ __launch_bounds__(kBkThreads) void k_bk_bins(SearchArgs a) {
    __shared__ int32_t h[kBkHist];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t wpp = static_cast<int64_t>(a.group) * a.qph;
    const int64_t runs = (wpp + kBkRun - 1) / kBkRun;
    const int64_t p = blockIdx.x / runs;
    const int64_t w0 = p * wpp + (blockIdx.x - p * runs) * kBkRun;
    const int64_t w1 = min(w0 + kBkRun, (p + 1) * wpp);
    const int64_t nb = a.nbins;
    const bool lds = nb <= kBkHist;
    int32_t *cnt = a.b_cnt + p * nb;
    int32_t *fill = a.b_fill + p * nb;
    const int32_t *first = a.b_first + p * nb;
    if (lds) {
        for (int k = tid; k < nb; k += kBkThreads) h[k] = 0;
        __syncthreads();
    }
    for (int64_t w = w0 + wave; w < w1; w += kBkThreads / 64) {
        const uint32_t *par = nullptr;
        const int np = bk_parents(a, static_cast<int>(w), par);
        for (int j = lane; j < np; j += 64) {
            const int64_t b = parent_bin(a, par[j]);
            if (lds) {
                atomicAdd(&h[b], 1);
            } else if (!FILL) {
                atomicAdd(&cnt[b], 1);
            } else {
                const int pos = first[b] + atomicAdd(&fill[b], 1);
                a.b_inv[pos] = make_int2(static_cast<int>(w), j);
            }
        }
    }
    if (!lds) return;                              // uniform
    __syncthreads();
    for (int k = tid; k < nb; k += kBkThreads) {
        const int v = h[k];
        if (v == 0) continue;
        if (FILL)
            h[k] = first[k] + atomicAdd(&fill[k], v);   // this run's first entry of parent k
        else
            atomicAdd(&cnt[k], v);
    }
    if (!FILL) return;
    __syncthreads();
    for (int64_t w = w0 + wave; w < w1; w += kBkThreads / 64) {
        const uint32_t *par = nullptr;
        const int np = bk_parents(a, static_cast<int>(w), par);
        for (int j = lane; j < np; j += 64) {
            const int pos = atomicAdd(&h[parent_bin(a, par[j])], 1);
            a.b_inv[pos] = make_int2(static_cast<int>(w), j);
        }
    }
}

template <int D, int R, typename QT, typename ST>
static hipError_t launch_block_t(const SearchArgs &a, int n0, hipStream_t st) {
    const int init_grid = (a.walks + kBkThreads - 1) / kBkThreads;
    hipLaunchKernelGGL((k_bk_init<R>), dim3(init_grid > 0 ? init_grid : 1), dim3(kBkThreads), 0, st, a, n0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int score_grid = 2048;
    const int64_t wpp = static_cast<int64_t>(a.group) * a.qph;
    const unsigned runs_grid = static_cast<unsigned>(a.pairs * ((wpp + kBkRun - 1) / kBkRun));
    const bool skip0 = n0 <= 1 || (a.mode == ZHA_TOPK && a.k[0] >= n0) || (a.mode == ZHA_TOPP && a.p >= 1.0f);
    for (int t = 0; t < a.levels && t < ZHA_MAX_STEPS; ++t) {
        if (t > 0 || !skip0) {
            hipLaunchKernelGGL((k_bk_score<D, R, QT, ST>), dim3(score_grid), dim3(kBkThreads), 0, st, a, t, n0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((k_bk_cut<R>), dim3(a.walks), dim3(64), 0, st, a, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (t + 1 < a.levels && t + 1 < ZHA_MAX_STEPS) {
            hipLaunchKernelGGL(k_bk_bins<false>, dim3(runs_grid), dim3(kBkThreads), 0, st, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_bk_group, dim3(1), dim3(kGroupThreads), 0, st, a, t + 1);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_bk_bins<true>, dim3(runs_grid), dim3(kBkThreads), 0, st, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <int D, typename QT, typename ST>
static hipError_t launch_block_d(const SearchArgs &a, int R, int n0, hipStream_t st) {
    switch (R) {
        case 1: return launch_block_t<D, 1, QT, ST>(a, n0, st);
        case 2: return launch_block_t<D, 2, QT, ST>(a, n0, st);
        case 4: return launch_block_t<D, 4, QT, ST>(a, n0, st);
        case 8: return launch_block_t<D, 8, QT, ST>(a, n0, st);
        case 16: return launch_block_t<D, 16, QT, ST>(a, n0, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, typename QT>
static hipError_t launch_block_s(const SearchArgs &a, int R, int sdtype, int n0, hipStream_t st) {
    return sdtype == ZHA_BF16 ? launch_block_d<D, QT, bf16_t>(a, R, n0, st) : launch_block_d<D, QT, float>(a, R, n0, st);
}

hipError_t launch_block(const SearchArgs &a, int D, int R, int dtype, int sdtype, int n0, hipStream_t st) {
    if (a.walks <= 0) return hipSuccess;
    if (D == 64)
        return dtype == ZHA_BF16 ? launch_block_s<64, bf16_t>(a, R, sdtype, n0, st)
                                 : launch_block_s<64, float>(a, R, sdtype, n0, st);
    return dtype == ZHA_BF16 ? launch_block_s<128, bf16_t>(a, R, sdtype, n0, st)
                             : launch_block_s<128, float>(a, R, sdtype, n0, st);
}

}  // namespace zha
