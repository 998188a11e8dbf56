// zha_internal.h -- argument blocks shared by the host layer and the HIP
// kernels of libzha.  Not part of the public ABI (see include/zha.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zha.h"

namespace zha {

// Candidate ids inside a walk: level in the top 4 bits, index in the rest.
constexpr int kLevelShift = 28;
constexpr uint32_t kIndexMask = (1u << kLevelShift) - 1u;
constexpr int kBlock = 256;          // threads per workgroup of most kernels
constexpr int kChunkMin = 512;       // keys per attention work item: the planner picks 512 .. 2048
constexpr int kChunkMax = 2048;      // (more, smaller items when a call reads few keys)
constexpr int32_t kStreamBit = 1 << 30;  // in the attention plan's keys-per-item word: streaming loads
constexpr int kTile = 32;            // candidates per tile of the level-synchronous scorer
constexpr int kPlanWalks = 4096;     // walks up to which that scorer orders its tiles itself (in LDS)
constexpr int kFlatPad = 32;         // union engine: each run of scoring entries is padded to this
constexpr int kExpSlices = 8;        // union engine: workgroups (runs) per pair building the next list
constexpr int kSmallList = 64;       // union engine: list bound of the steps fused into one launch
constexpr int kTopNodes = 256;       // union engine: nodes the fused first steps may meet, all steps
constexpr int kUaBlocks = 128;       // union attention: level-1 blocks per work item
constexpr int kUaMaxItems = 4096;    // union attention: work items per pair (at most)
constexpr int kUaSlice = 16384;      // union attention: level-1 blocks per mask-building workgroup
constexpr int kUaSortMax = 16384;    // union attention, prefill: walks sorted together (one workgroup)
constexpr int kXcds = 8;             // MI355X: accelerator dies (XCDs), each with its own L2

constexpr int kTopRowsMax = 2048;   // level-synchronous engine: nodes per pair of the dense top table
constexpr int kTopList = 4096;      // candidates a top step keeps in LDS

// Which slower or rarer code paths a walk took (bits 16.. of the flags a walk
// carries through the engines; finish_walk moves them to zha_walk_stats.paths
// as ZHA_PATH_*, and only the low bits reach the status word).
constexpr uint32_t kPathShift = 16;
constexpr uint32_t kPathTieSelect = 1u << kPathShift;   // ZHA_PATH_TIE_SELECT
constexpr uint32_t kPathLongList = 2u << kPathShift;    // ZHA_PATH_LONG_LIST
constexpr uint32_t kPathLdsSpill = 4u << kPathShift;    // ZHA_PATH_LDS_SPILL
constexpr uint32_t kFlagBits = (1u << kPathShift) - 1u;

// Workgroups go to the XCDs in turn (workgroup i to XCD i mod kXcds).  With
// a grid of xcd_grid(n) workgroups, workgroup i takes item xcd_item(i, n)
// (nothing when that is -1): runs of consecutive items share one XCD and its
// L2.
__host__ __device__ constexpr int64_t xcd_grid(int64_t n) { return (n + kXcds - 1) / kXcds * kXcds; }
__device__ __forceinline__ int64_t xcd_item(int64_t i, int64_t n) {
    const int64_t v = (i % kXcds) * ((n + kXcds - 1) / kXcds) + i / kXcds;
    return v < n ? v : -1;
}

// Per-walk state of the level-synchronous search engine (workspace).
struct WalkState {
    int32_t n;                       // candidates of the current step (0 = finished)
    int32_t buf;                     // current candidate buffer (0 or 1)
    int32_t sel_n;                   // level-1 blocks found so far (before clamp)
    int32_t unforced;                // candidates scored so far
    uint32_t flags;
    int32_t steps;
    int32_t scored[ZHA_MAX_STEPS];
    int32_t opened[ZHA_MAX_STEPS];
};

// One level of summaries for a node range, every (sequence, KV head) pair.
struct LevelArgs {
    const void *keys;          // level 1: K cache (pair stride max_tokens * D elements)
    const void *child_k;       // level >= 2: keys of level l-1   (pair stride child_cap*R*D)
    const float *child_b;      // level >= 2: biases of level l-1 (pair stride child_cap*R)
    void *out_k;               // level l keys   (pair stride out_cap*R*D; fp32 or bf16)
    float *out_b;              // level l biases (pair stride out_cap*R)
    const float *refs;         // [kv_heads][R][D]
    int64_t max_tokens;
    int64_t child_cap;
    int64_t out_cap;
    int64_t j0;                // first node to summarise
    int64_t count;             // nodes to summarise per pair
    int32_t kv_heads;
    int32_t pairs;
    int32_t chunk;
    int32_t refs_n;
    float sharpness;
};

struct SearchArgs {
    const float *kap[ZHA_MAX_LEVELS + 1];  // level-l keys, pair 0 (bf16 data when the summaries are bf16)
    const float *bet[ZHA_MAX_LEVELS + 1];  // level-l biases, pair 0
    int64_t cap[ZHA_MAX_LEVELS + 1];       // nodes per pair at level l (stride)
    int64_t nl[ZHA_MAX_LEVELS + 2];        // live nodes at level l; nl[L+1] = 0
    const void *q;                         // [walks][D]
    int32_t *sel_blocks;                   // [walks][sel_cap]
    int32_t *sel_count;                    // [walks]
    zha_walk_stats *stats;                 // [walks] or null
    uint32_t *status;
    uint32_t *visited;                     // [pairs][vis_words] or null
    int64_t node_off[ZHA_MAX_LEVELS + 1];  // bit of node (l, 0) in a pair's bitmap
    int64_t vis_words;                     // bitmap words per pair
    uint32_t *cand;                        // ws [walks][2][cand_cap]
    float *score;                          // ws [walks][cand_cap]
    WalkState *state;                      // ws [walks]          (level-synchronous)
    int32_t *tile_count;                   // ws [ZHA_MAX_STEPS+1] tiles (level-synchronous) or
                                           // flat entries (union) per step
    int2 *tile_map;                        // ws [walks * ceil(cand_cap / kTile)]
    // union engine: one candidate list per (sequence, KV head) pair, the
    // union over its query heads, with a head mask per node
    uint32_t *u_ids;                       // ws [pairs][2][cand_cap]
    uint32_t *u_omask;                     // ws [pairs][2][cand_cap]  heads that opened the node (by step parity)
    int32_t *u_n;                          // ws [pairs][2]  list size (by step parity)
    int32_t *u_next;                       // ws [walks]  entries a head opened (levels > 1)
    float *u_score;                        // ws [pairs][cand_cap][round_up(group, 4)]
    float *h_score;                        // ws [walks][cand_cap]  a head's gathered scores
    int32_t *u_rank;                       // ws [pairs][cand_cap]  rank of an opened entry
    uint32_t *u_par;                       // ws [pairs][cand_cap]  opened entry of each rank
    int32_t *u_open;                       // ws [walks][cand_cap]  list positions a head opened
    int4 *u_flat;                          // ws [2][flat_cap]  {pair, position, node id, 0}
    int64_t flat_cap;                      // entries per flat buffer
    // block engine (prefill query blocks): walks grouped by the parent they opened
    uint32_t *b_roots;                     // ws [cand_cap]  the roots (the same for every pair)
    int32_t *b_cnt;                        // ws [pairs][nbins]  walks that opened each parent
    int32_t *b_fill;                       // ws [pairs][nbins]
    int32_t *b_first;                      // ws [pairs][nbins]  first entry of each parent
    int2 *b_inv;                           // ws [walks * pcap]  {walk, slot of the parent}
    int4 *b_units;                         // ws [walks * pcap]  {pair, parent id, first entry, rows}
    int64_t nbins;                         // parents (nodes of levels >= 2) per pair
    int64_t bin_lvl[ZHA_MAX_LEVELS + 2];   // first bin of level l within a pair
    int32_t pcap;                          // parents a walk keeps per step
    int64_t n_roots;                       // roots before clamping to cand_cap
    int32_t top_steps;                     // level-synchronous engine: first steps cut from a dense
                                           // score table of the top levels (0: none)
    int32_t top_lo;                        // lowest level of that table (levels top_lo .. L)
    int64_t top_off[ZHA_MAX_LEVELS + 2];   // row of node (l, 0) in a pair's table
    int64_t top_rows;                      // table rows per pair (scores at [pair][row][gp], in u_score)
    int32_t top_lds;                       // 1: the top steps' lists fit in LDS (kTopList entries)
    int32_t small_steps;                   // union engine: first steps done by one workgroup per pair
    int32_t ls_from;                       // union engine: steps from here run level-synchronously (0: none)
    int32_t pairs;
    int64_t n_tokens;
    int32_t walks;
    int32_t qph;                           // queries per head (1 = decode)
    int32_t heads;                         // query heads per sequence
    int32_t group;
    int32_t kv_heads;
    int32_t chunk;
    int32_t log2c;
    int32_t levels;
    int32_t mode;
    float p;
    int32_t k[ZHA_MAX_STEPS];
    int32_t sel_cap;
    int32_t cand_cap;
    int32_t score_grid;                    // workgroups of the level-synchronous scorer
    float sharpness;
};

struct AttnArgs {
    const void *q;                 // [walks][D]
    const void *k;                 // cache
    const void *v;                 // cache
    void *out;                     // [walks][D]
    const int32_t *sel_blocks;     // [walks][sel_cap] level-1 blocks, or
    const int32_t *tokens;         // [walks][sel_cap] token ids (then no blocks, no tail)
    const int32_t *sel_count;      // [walks] entries of sel_blocks / tokens
    float *part;                   // ws [max_items][D + 2]
    int32_t *item_off;             // ws [walks + 2]: first item of each walk; [walks + 1]: keys per item
    int32_t *item_walk;            // ws [max_items]: walk of each item
    int64_t max_tokens;
    int64_t n_tokens;
    int64_t n1;                    // whole level-1 chunks
    int32_t walks;
    int32_t qph;                   // queries per head; > 1: a prefill block at
                                   // positions [n_tokens, n_tokens + qph)
    int32_t heads;
    int32_t group;
    int32_t kv_heads;
    int32_t chunk;
    int32_t sel_cap;
    int32_t grid;                  // workgroups of the item loop
    int32_t block_mfma;            // prefill: the block's own keys go to k_attn_block
                                   // (one extra item per walk, the last one)
    float sharpness;
    // union path: per group of walks sharing a KV cache (decode: a pair's
    // heads; prefill: 16 walks of a pair, consecutive in the order of their
    // selection sketches), the union of their selected blocks, one column
    // per walk
    uint16_t *umask;               // ws [ugroups][n1cap]  columns that selected each level-1 block
    uint32_t *uchunk;              // ws [ugroups][cwords]  chunks of kUaBlocks blocks holding one
    int32_t *ic;                   // ws [ugroups][items_pp]  1: the workgroup wrote partials
    float *bpart;                  // ws [walks][D + 2]  prefill: the block's own keys (k_attn_block)
    unsigned long long *ukey;      // ws [walks]  prefill: sketch key of each walk (sort key)
    int32_t *uperm;                // ws [walks]  prefill: pair-local walk at each sorted position
    int32_t *uinv;                 // ws [walks]  prefill: sorted position of each walk within its pair
    int64_t n1cap;                 // level-1 blocks per group (stride of umask, even)
    int64_t ugroups;
    int32_t cwords;
    int32_t gpp;                   // prefill: groups per pair (16 sorted walks each)
    int32_t items_pp;              // workgroups (partials) per group
    int32_t ua_cpw;                // kUaBlocks-block chunks per workgroup
    int32_t pairs;
    int32_t log2c;
};

struct DenseArgs {
    const void *q;                 // [walks][D]
    const void *k;                 // cache
    const int32_t *budget;         // [walks]
    int32_t *budget_out;           // top-p over keys: ws [walks], written by k_dense_topp_budget
    uint32_t *status;              // top-p over keys: flags (nullable)
    float p;                       // top-p over keys: the mass to reach
    float *logits;                 // ws [walks][row_pad]
    int32_t *sel;                  // [walks][max_budget] selected token ids, ascending
    int32_t *sel_n;                // [walks]
    int64_t max_tokens;
    int64_t n_tokens;
    int64_t row_pad;               // logits row stride
    int32_t walks;
    int32_t heads;
    int32_t group;
    int32_t kv_heads;
    int32_t max_budget;
    float sharpness;
};

// One decode step in one launch (zha_forward with ZHA_ENGINE_FUSED): the
// search arguments describe the tree after the append.
struct FusedArgs {
    SearchArgs s;
    const void *k;                          // K cache
    const void *v;                          // V cache
    void *out;                              // [walks][D]
    const float *refs;                      // [kv_heads][R][D]
    int64_t max_tokens;
    int32_t fresh_m;                        // levels 1..fresh_m gain their last node in this append
    void *tree_k[ZHA_MAX_LEVELS + 1];       // level-l keys, pair 0 (written by the pairs' first walks)
    float *tree_b[ZHA_MAX_LEVELS + 1];      // level-l biases, pair 0
};

hipError_t launch_level(const LevelArgs &a, int D, int dtype, int sdtype, bool leaf, hipStream_t st);
hipError_t launch_search(const SearchArgs &a, int D, int R, int dtype, int sdtype, int engine, int n0,
                         hipStream_t st);
hipError_t launch_union(const SearchArgs &a, int D, int R, int dtype, int sdtype, int n0, hipStream_t st);
hipError_t launch_ls_from(const SearchArgs &a, int D, int R, int dtype, int sdtype, int t0, hipStream_t st);
hipError_t launch_top(const SearchArgs &a, int D, int R, int dtype, int sdtype, hipStream_t st);
hipError_t launch_block(const SearchArgs &a, int D, int R, int dtype, int sdtype, int n0, hipStream_t st);
hipError_t launch_attn(const AttnArgs &a, int D, int dtype, hipStream_t st);
hipError_t launch_attn_union(const AttnArgs &a, int D, hipStream_t st);
hipError_t launch_attn_block(const AttnArgs &a, int D, hipStream_t st);
hipError_t launch_dense(const DenseArgs &a, int D, int dtype, hipStream_t st);
hipError_t launch_fused(const FusedArgs &f, int D, int R, int dtype, int sdtype, hipStream_t st);
size_t fused_lds_bytes(int D, int R, int c, int sbytes, int m);
hipError_t launch_probe(const void *buf, uint64_t bytes, float *sink, hipStream_t st);

}  // namespace zha
