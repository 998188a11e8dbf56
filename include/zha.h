/*
 * zha.h -- C ABI of the MI355X (gfx950) library for tree-structured KV search.
 *
 * The method is Zyphra Hierarchical Attention (ZHA) as described on the page
 * "How does a tree of summaries search a context? How ZHA works"
 * (learn.chabulab.com), cited below as [ZHA lesson] with a section name, and
 * on the arXiv abstract "Subquadratic Attention with a Hierarchical
 * Tree-Structured Indexer" (2610.42112), cited as [ZHA abstract].
 *
 * Three operations make up the hot path:
 *   1. build / append the tree of compressed key summaries over a KV cache
 *      that stays intact ([ZHA lesson] "How is the tree built?",
 *      "What does a node summarize?");
 *   2. walk the tree top-down for a batch of queries, one walk per query head,
 *      opening nodes by top-p or top-K at every step ([ZHA lesson] "How does
 *      top-p differ from top-K?", "Run a small tree yourself", "Common
 *      misunderstandings");
 *   3. softmax attention over exactly the original keys and values the walk
 *      chose ([ZHA lesson] "How is the tree built?").
 *
 * Conventions shared by every call:
 *   - All device memory is owned by the caller.  The library never
 *     allocates, frees or synchronises; work is enqueued on the caller's HIP
 *     stream (hipStream_t passed as void*; NULL = the null stream).
 *   - Every call validates its arguments on the host first.  A call that
 *     returns anything but ZHA_OK has enqueued nothing.
 *   - Device-side conditions (capacity overflow, non-finite scores) set bits
 *     in a caller-provided uint32 status word (ZHA_FLAG_*), readable after the
 *     stream is synchronised; the results stay deterministic.
 *   - Device pointers must be 16-byte aligned (ZHA_ERR_ALIGN otherwise).
 *   - Layouts (row-major, last index fastest):
 *       K, V cache   [batch][kv_heads][max_tokens][head_dim]   dtype
 *       Q, out       [batch][kv_heads*group][q_per_head][head_dim] dtype
 *       refs         [kv_heads][num_refs][head_dim]            float32
 *     Query head h uses KV head h / group.  One tree per (sequence, KV head);
 *     every query head of the group walks it separately.
 *   - Supported: head_dim 64 or 128; chunk a power of two in [2, 64];
 *     levels 1..12; num_refs in {1, 2, 4, 8, 16}; dtype float32 or bfloat16.
 *     Anything else returns ZHA_ERR_UNSUPPORTED.
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZHA_MAX_LEVELS 12
#define ZHA_MAX_STEPS 12

typedef enum {
    ZHA_OK = 0,
    ZHA_ERR_ARG = 1,         /* null pointer or out-of-range scalar           */
    ZHA_ERR_SHAPE = 2,       /* token counts / sizes inconsistent             */
    ZHA_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned       */
    ZHA_ERR_CAPACITY = 4,    /* append past max_tokens, tree memory too small */
    ZHA_ERR_WORKSPACE = 5,   /* workspace smaller than the sizing call says   */
    ZHA_ERR_UNSUPPORTED = 6, /* geometry outside the supported set            */
    ZHA_ERR_HIP = 7          /* a HIP launch failed                           */
} zha_status;

typedef enum { ZHA_F32 = 0, ZHA_BF16 = 1 } zha_dtype;

enum { ZHA_TOPP = 0, ZHA_TOPK = 1 };

/* Search engines (zha_select.engine).  All give the same selections (the
 * persistent and level-synchronous engines bit-identical results; the union
 * engine sums dot products in another order, so a score may differ in the
 * last fp32 bits, which matters only at cuts closer than that).
 *   ZHA_ENGINE_PERSISTENT: one workgroup per walk runs all steps in one
 *     launch; best when every walk does the same work.
 *   ZHA_ENGINE_LEVEL_SYNC: per step, one launch scores the candidates of all
 *     walks as one flat list and one launch cuts each walk; balances walks
 *     of very different sizes.
 *   ZHA_ENGINE_UNION: per step, each (sequence, KV head) pair keeps one list,
 *     the union of its query heads' candidates with a head mask per node;
 *     every node record is read once and scored for all heads of the group
 *     (fp32 matrix-core tiles), then each head cuts its own candidates.
 *     With fewer than 16 heads per KV head the last two steps (the widest,
 *     where the heads' lists overlap least) run level-synchronously.
 *     Decode only (q_per_head = 1), group_size <= 16.
 *   ZHA_ENGINE_BLOCK: for prefill blocks (any q_per_head): the walks are
 *     grouped by the parent node they opened and each parent's children are
 *     scored for all of its walks at once (fp32 matrix-core tiles); the root
 *     list is scored against every walk the same way.  One wavefront cuts
 *     each walk.
 *   ZHA_ENGINE_FUSED: zha_forward only, decode (q_per_head = 1) with
 *     n_new <= 1: the append, the walk and the attention of a decode step
 *     in one launch, one workgroup per walk (the walk is the persistent
 *     engine's, so selections and stats equal it bit for bit; attention is
 *     summed in another order than zha_sparse_attn's).  Nodes the append
 *     makes are computed by each of the pair's workgroups for itself and
 *     written to the tree by the pair's first query head; no workgroup waits
 *     on another.  AUTO never picks it.
 *   ZHA_ENGINE_AUTO: block for prefill (q_per_head > 1), else union for
 *     decode with at least 64 walks and 16 query heads per KV head, or 8 to
 *     16 under top-p, else level-synchronous for top-p with at least 64
 *     walks, else persistent. */
enum {
    ZHA_ENGINE_AUTO = 0,
    ZHA_ENGINE_PERSISTENT = 1,
    ZHA_ENGINE_LEVEL_SYNC = 2,
    ZHA_ENGINE_UNION = 3,
    ZHA_ENGINE_BLOCK = 4,
    ZHA_ENGINE_FUSED = 5
};

/* Attention paths (zha_select.attn_engine).  Both attend exactly the keys
 * each walk selected and give the same result up to the order of fp32 sums.
 *   ZHA_ATTN_PER_WALK: every walk reads its own selected blocks (split-K
 *     work items per walk).
 *   ZHA_ATTN_UNION: per group of walks that share a KV cache, every block
 *     any of them selected is read once and attended by each walk that
 *     selected it (bf16 matrix-core logits for the whole group, a walk mask
 *     per block).  bf16 caches, chunk >= 4.  Decode (q_per_head = 1): the
 *     group is a (sequence, KV head) pair's query heads, group_size <= 16.
 *     Prefill blocks (q_per_head > 1): groups of 16 walks of a pair, taken
 *     in the order of a sketch of their selections.  A walk's list is taken
 *     as a set: a block listed twice counts once (zha_search never lists a
 *     block twice).
 *   ZHA_ATTN_AUTO: union for bf16 prefill blocks and for bf16 decode with 16
 *     query heads per KV head (where it applies), else per-walk. */
enum { ZHA_ATTN_AUTO = 0, ZHA_ATTN_PER_WALK = 1, ZHA_ATTN_UNION = 2 };

/* Device status bits. */
#define ZHA_FLAG_CAND_OVERFLOW 1u  /* a step had more candidates than max_candidates;
                                      the excess (in span order) was dropped      */
#define ZHA_FLAG_SEL_OVERFLOW 2u   /* more level-1 blocks opened than
                                      max_blocks_per_walk; the excess was dropped */
#define ZHA_FLAG_NONFINITE 4u      /* a node score was NaN; it ranked last        */

/* Shape of the cache and of the tree over it.
 * sharpness: the scale s in every score s*<key, query> + bias, which is also
 * the attention logit scale (usually 1/sqrt(head_dim)).  levels = number of
 * summary levels above the raw keys ([ZHA lesson] "How is the tree built?":
 * one level summarises `chunk` keys, two levels chunk^2, ...). */
typedef struct {
    int32_t batch;
    int32_t num_kv_heads;
    int32_t group_size;      /* query heads per KV head                       */
    int32_t head_dim;
    int32_t chunk;           /* children per node                             */
    int32_t num_refs;        /* reference queries R (tangents per node)       */
    int32_t levels;
    int32_t dtype;           /* zha_dtype of K, V, Q and out                  */
    int64_t max_tokens;      /* cache capacity per (sequence, KV head)        */
    float sharpness;
    int32_t summary_dtype;   /* zha_dtype of the stored node keys: ZHA_F32
                                (default), or ZHA_BF16 -- each key rounded to
                                bf16 (nearest, ties to even) after it is
                                computed in fp32, and its bias computed from
                                the rounded key, so a node's score at its own
                                reference query is still the subtree's
                                log-sum-exp.  Biases are always fp32.        */
} zha_geometry;

/* How a walk opens nodes at each step ([ZHA lesson] "How does top-p differ
 * from top-K?").
 *   ZHA_TOPP: open the smallest prefix of the candidates ordered by score
 *     (descending; equal scores by span start, ascending) whose softmax mass
 *     reaches p.  p >= 1 opens every candidate, p <= 0 opens one.
 *   ZHA_TOPK: open min(k[t], candidates) at step t; k[t] = k[num_k-1] for
 *     t >= num_k.
 * The softmax runs jointly over the step's whole candidate list.
 * max_blocks_per_walk bounds the stored level-1 selections of a walk;
 * max_candidates bounds a step's candidate list (0 = the largest level). */
typedef struct {
    int32_t mode;
    float p;
    int32_t k[ZHA_MAX_STEPS];
    int32_t num_k;
    int32_t max_blocks_per_walk;
    int32_t max_candidates;
    int32_t engine;          /* ZHA_ENGINE_* (search)                         */
    int32_t attn_engine;     /* ZHA_ATTN_* (sparse attention)                 */
} zha_select;

/* Host handle of one tree set (all sequences and KV heads).  Plain data: the
 * caller keeps it; zha_build / zha_append update n_tokens.  Fill it with
 * zha_tree_init only. */
typedef struct {
    zha_geometry geom;
    int64_t n_tokens;                            /* tokens summarised so far  */
    void *tree_mem;                              /* device, caller-owned      */
    uint64_t tree_bytes;
    const float *refs;                           /* device, caller-owned      */
    int64_t level_cap[ZHA_MAX_LEVELS + 1];       /* nodes per pair, level l   */
    uint64_t key_off[ZHA_MAX_LEVELS + 1];        /* byte offset of level-l keys   */
    uint64_t bias_off[ZHA_MAX_LEVELS + 1];       /* byte offset of level-l biases */
} zha_tree;

/* Per-walk accounting ([ZHA lesson] "Run a small tree yourself": a walk's
 * work is R per scored node plus one per key read). */
typedef struct {
    int32_t scored[ZHA_MAX_STEPS];   /* candidates at step t                  */
    int32_t opened[ZHA_MAX_STEPS];   /* candidates opened at step t           */
    int32_t steps;
    int32_t keys_read;               /* selected keys incl. the raw tail      */
    int32_t blocks;                  /* level-1 blocks opened (before clamp)  */
    int32_t unforced_scored;         /* candidates whose scores were computed */
    int64_t comparisons;             /* R * sum(scored) + keys_read           */
    uint32_t flags;                  /* ZHA_FLAG_* raised by this walk        */
    uint32_t paths;                  /* ZHA_PATH_*: slower code paths taken   */
} zha_walk_stats;

/* zha_walk_stats.paths: code paths a walk's cuts took that are rare or
 * slower, reported so that tests and profiles can tell which ran.  They
 * never change a result.
 *   ZHA_PATH_TIE_SELECT: a cut's value window could not be split (more than
 *     64 candidates with equal scores around the cut, or every score -inf),
 *     so the cut key was found by the tie-exact select over full rank keys
 *     (score, then span start).
 *   ZHA_PATH_LONG_LIST: a prefill-block cut (ZHA_ENGINE_BLOCK) read a list
 *     longer than the 1,024 candidates it keeps in registers.
 *   ZHA_PATH_LDS_SPILL: a decode cut had more candidates than it stages in
 *     LDS and ran its passes over global memory. */
#define ZHA_PATH_TIE_SELECT 1u
#define ZHA_PATH_LONG_LIST 2u
#define ZHA_PATH_LDS_SPILL 4u

/* ---- sizing and set-up (host only, no device work) -------------------- */

/* Bytes of tree memory for `g`: for every level l = 1..levels, keys
 * (summary_dtype: float32 or bf16)
 * [batch][kv_heads][floor(max_tokens/chunk^l)][num_refs][head_dim]
 * then biases float32 [batch][kv_heads][floor(max_tokens/chunk^l)][num_refs],
 * each array 256-byte aligned.  Returns 0 if `g` is invalid. */
uint64_t zha_tree_bytes(const zha_geometry *g);

/* Depth rule of the demo program ([ZHA lesson] "Run a small tree yourself":
 * summary levels are added until the top level holds at most 64 nodes): the
 * fewest levels L >= 1 with floor(n_tokens / chunk^L) <= max_top, at most
 * ZHA_MAX_LEVELS.  Host only.  -1 if n_tokens < 0, chunk is not a power of
 * two in [2, 64] or max_top < 1. */
int32_t zha_depth_for(int64_t n_tokens, int32_t chunk, int64_t max_top);

/* Fill `t` for tree memory `tree_mem` (device, >= zha_tree_bytes) and the
 * reference queries `refs` (device float32 [kv_heads][num_refs][head_dim],
 * [ZHA lesson] "What does a node summarize?": fixed sample questions).
 * Sets n_tokens = 0.  No device work. */
zha_status zha_tree_init(zha_tree *t, const zha_geometry *g, void *tree_mem,
                         uint64_t tree_bytes, const float *refs);

/* ---- 1. build and append ------------------------------------------------ */

/* Summarise the first n_tokens rows of k_cache into levels 1..levels from
 * scratch and set t->n_tokens = n_tokens.  Level 1 summarises each whole
 * chunk of keys (a key is its own tangent for every reference, bias 0);
 * level l >= 2 summarises each whole chunk of level-(l-1) nodes.  Per
 * reference r: weights softmax(s*<child key_r, rho_r> + child bias_r), the new
 * key the weighted sum of child keys, the new bias the log-sum-exp of those
 * scores minus s*<new key, rho_r> ([ZHA lesson] "What does a node
 * summarize?").  Partial chunks are not summarised. */
zha_status zha_build(zha_tree *t, const void *k_cache, int64_t n_tokens, void *stream);

/* The caller has written rows [n, n + n_new) of every (sequence, KV head) of
 * k_cache, n = t->n_tokens.  Summarise every chunk that these rows complete,
 * at every level, and set t->n_tokens = n + n_new ([ZHA lesson] "How is the
 * tree built?": a new node appears whenever a chunk has filled).  The result is
 * bit-identical to zha_build over n + n_new tokens.  ZHA_ERR_CAPACITY if
 * n + n_new > max_tokens. */
zha_status zha_append(zha_tree *t, const void *k_cache, int64_t n_new, void *stream);

/* ---- 2. search ------------------------------------------------------------ */

/* Workspace bytes of zha_search for q_per_head queries per head. */
uint64_t zha_search_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head);

/* The engine (ZHA_ENGINE_PERSISTENT, _LEVEL_SYNC, _UNION or _BLOCK) zha_search runs
 * for these arguments: sel->engine itself, or what ZHA_ENGINE_AUTO resolves
 * to.  Host only, enqueues nothing.  -1 if the tree or selection is invalid
 * or the engine does not support the shape.  All engines give identical
 * selections wherever the cut's score gap exceeds rounding. */
int32_t zha_search_engine(const zha_tree *t, const zha_select *sel, int32_t q_per_head);

/* One walk per (sequence, query head, query).  Candidates start as the
 * roots: every top-level node plus every node whose parent chunk has not
 * filled; per step they are scored (max over r of s*<key_r, q> + bias_r),
 * normalised with a softmax over the whole step and cut by `sel`; opened
 * level-1 nodes select their `chunk` keys, other opened nodes give their
 * children as the next candidates ([ZHA lesson] "Run a small tree
 * yourself", "Common misunderstandings": each head walks on its own).  Raw
 * keys past the last whole chunk are always selected (not listed).
 *   q_per_head  1: decode, one query per head seeing the tree's tokens
 *               [0, n_tokens).  > 1: a prefill block whose queries sit at
 *               positions n_tokens .. n_tokens + q_per_head - 1; every query
 *               walks the tree as it stands (the tokens before the block).
 *   sel_blocks  device int32 [walks][max_blocks_per_walk]: level-1 block ids
 *               j (keys j*chunk .. j*chunk+chunk-1), in the order found
 *               (steps in order, each step in span order)
 *   sel_count   device int32 [walks]: blocks stored (<= max_blocks_per_walk)
 *   stats       device zha_walk_stats [walks], may be NULL
 *   status      device uint32, OR-ed with ZHA_FLAG_* (not cleared)
 *   visited     device uint32 [batch*kv_heads][zha_visited_words/pairs], may be
 *               NULL (see zha_visited_words)
 * walks = batch * kv_heads * group_size * q_per_head, in Q's order. */
zha_status zha_search(const zha_tree *t, const void *q, int32_t q_per_head,
                      const zha_select *sel, int32_t *sel_blocks, int32_t *sel_count,
                      zha_walk_stats *stats, uint32_t *status, uint32_t *visited,
                      void *ws, uint64_t ws_bytes, void *stream);

/* 32-bit words of the optional `visited` bitmap of zha_search: per (sequence,
 * KV head) pair, one bit per node of every level (levels 1..L one after the
 * other, each max_tokens/chunk^l nodes long), rounded up to whole words.
 * When `visited` is given, every node whose score an unforced cut needed
 * sets its bit (OR; the caller clears it).  The set bits are the records a
 * search has to read at least once per pair, whatever the number of query
 * heads that scored them. */
uint64_t zha_visited_words(const zha_tree *t);

/* ---- 3. sparse attention --------------------------------------------------- */

/* Workspace bytes of zha_sparse_attn. */
uint64_t zha_attn_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head);

/* The attention path (ZHA_ATTN_PER_WALK or ZHA_ATTN_UNION) zha_sparse_attn
 * runs for these arguments: sel->attn_engine itself, or what ZHA_ATTN_AUTO
 * resolves to.  Host only, enqueues nothing.  -1 if the tree or selection is
 * invalid or the path does not support the shape. */
int32_t zha_attn_engine(const zha_tree *t, const zha_select *sel, int32_t q_per_head);

/* out = softmax over the selected keys of s*<q, K_i>, applied to V_i, for
 * every walk: exactly the original keys of the listed level-1 blocks plus
 * the raw tail [chunk*floor(n_tokens/chunk), n_tokens) ([ZHA lesson] "How is
 * the tree built?", "Common misunderstandings").  For a prefill block
 * (q_per_head > 1) query t also attends the block's own keys n_tokens ..
 * n_tokens + t (causal; rows the caller has written, n_tokens + q_per_head <=
 * max_tokens or ZHA_ERR_CAPACITY).  fp32 accumulation; a bf16 output is
 * rounded to nearest-even once.  Block ids outside [0, floor(n_tokens/chunk))
 * are skipped; entries past sel_count are ignored. */
zha_status zha_sparse_attn(const zha_tree *t, const void *q, int32_t q_per_head,
                           const void *k_cache, const void *v_cache,
                           const zha_select *sel, const int32_t *sel_blocks,
                           const int32_t *sel_count, void *out,
                           void *ws, uint64_t ws_bytes, void *stream);

/* ---- attention without any allocation ---------------------------------------- */

/* Bytes of the fixed device scratch of zha_sparse_attn_noalloc (64 MiB per
 * GPU, part of the library's code object: each GPU the library runs on holds
 * it from the library's first use there until the process ends). */
#define ZHA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * zha_sparse_attn with the per-walk attention path (ZHA_ATTN_PER_WALK; the
 * same kernels, so the same result bit for bit) and no workspace argument.
 * Its work items and partial states live in the fixed scratch instead.  The
 * call allocates and frees nothing, on the device or the host.
 *   Arguments, layouts and errors as zha_sparse_attn, plus:
 *   ZHA_ERR_WORKSPACE   the call needs more than ZHA_NOALLOC_SCRATCH_BYTES
 *                       (it needs zha_attn_workspace_bytes of the same
 *                       arguments with attn_engine = ZHA_ATTN_PER_WALK; a
 *                       smaller max_blocks_per_walk lowers it);
 *   ZHA_ERR_UNSUPPORTED sel->attn_engine is ZHA_ATTN_UNION (AUTO runs the
 *                       per-walk path here);
 *   ZHA_ERR_HIP         the scratch's device address could not be found.
 * Every call on a GPU uses that GPU's one scratch, whose contents after a
 * call are that call's: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs clearing between calls (every word a call reads it has
 * written first). */
zha_status zha_sparse_attn_noalloc(const zha_tree *t, const void *q, int32_t q_per_head,
                                   const void *k_cache, const void *v_cache,
                                   const zha_select *sel, const int32_t *sel_blocks,
                                   const int32_t *sel_count, void *out, void *stream);

/* ---- one decode step ------------------------------------------------------- */

/* Workspace bytes of zha_forward (search + attention + selection lists). */
uint64_t zha_forward_workspace_bytes(const zha_tree *t, const zha_select *sel, int32_t q_per_head);

/* One step of a layer with the selection lists kept in the workspace: the
 * upkeep of the tree as the cache grows ([ZHA lesson] "How is the tree
 * built?": a node is summarised once its chunk of children is complete), the
 * top-down walk of every query head ("Run a small tree yourself") and
 * ordinary attention over the original keys the walk chose ("Common
 * misunderstandings": summaries only steer the search).
 * Decode (q_per_head = 1): zha_append(n_new) first (the new token's key is
 * then visible to its own query), then zha_search and zha_sparse_attn; with
 * sel->engine = ZHA_ENGINE_FUSED (n_new = 1) the three run in one launch.
 * Prefill block (q_per_head > 1): zha_search and zha_sparse_attn for the
 * block at positions [n_tokens, n_tokens + q_per_head), then
 * zha_append(n_new) (normally n_new = q_per_head).
 * Arguments: q, k_cache, v_cache, out, stats and status as for zha_search
 * and zha_sparse_attn (device pointers, caller-owned, stats may be null);
 * ws: caller-owned device workspace of at least
 * zha_forward_workspace_bytes(t, sel, q_per_head) bytes, ws_bytes its size;
 * stream: the hipStream_t every launch goes to (null: the default stream).
 * Errors: the argument checks of the three calls (ZHA_ERR_ARG, _ALIGN,
 * _CAPACITY, _UNSUPPORTED) and ZHA_ERR_WORKSPACE for a short workspace
 * return before anything is enqueued; a failed launch returns ZHA_ERR_HIP. */
zha_status zha_forward(zha_tree *t, int64_t n_new, const void *q, int32_t q_per_head,
                       const void *k_cache, const void *v_cache, const zha_select *sel,
                       void *out, zha_walk_stats *stats, uint32_t *status,
                       void *ws, uint64_t ws_bytes, void *stream);

/* ---- measurement helpers (same-GPU baselines) ------------------------------ */

/* Workspace bytes of zha_dense_topk_attn for budgets up to max_budget. */
uint64_t zha_dense_workspace_bytes(const zha_tree *t, int32_t max_budget);

/* Dense full-scan indexer, the baseline the tree search is measured against:
 * exact logits s*<q, K_i> for every key i < t->n_tokens (one pass over K per
 * (sequence, KV head) serving all its query heads), the budget[w] highest
 * logits of each walk (ties: lower index first), then attention over exactly
 * those keys into out.  Decode only (one query per head); uses the tree
 * handle for its shapes and n_tokens only.  This is the indexer that scores
 * every key before choosing, written from its plain definition ([ZHA lesson]
 * "How does a tree of summaries search a context?"; news page "Zyphra AI
 * Introduces ZHA, a Path to True Subquadratic Attention").
 *   budget      device int32 [walks], clamped to [1, min(n_tokens, max_budget)]
 *   sel_tokens  device int32 [walks][max_budget] or NULL: the chosen token
 *               ids of each walk in ascending order (first budget[w] entries) */
zha_status zha_dense_topk_attn(const zha_tree *t, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *budget, int32_t max_budget,
                               void *out, int32_t *sel_tokens, void *ws, uint64_t ws_bytes,
                               void *stream);

/* Dense top-p over keys, the baseline's other selection rule: the same
 * exact logits, then for each walk the smallest prefix of its keys ordered
 * by (logit descending, index ascending) whose softmax mass over all keys
 * reaches p (masses are exp(logit - max) * 2^31 rounded to integers, as in
 * the tree's cuts, so the sums are exact), then attention over exactly
 * those keys.  p >= 1 takes every key, p <= 0 the first one ([ZHA lesson]
 * "How does top-p differ from top-K?" for the prefix rule, applied here to
 * keys instead of nodes).  Workspace: zha_dense_workspace_bytes(t,
 * max_budget).
 *   sel_tokens  device int32 [walks][max_budget] or NULL (as above)
 *   sel_count   device int32 [walks] or NULL: the prefix length of each walk
 *               (clamped to max_budget)
 *   status      device uint32 or NULL: ZHA_FLAG_SEL_OVERFLOW is ORed in
 *               when a prefix is longer than max_budget
 * Returns ZHA_ERR_ARG for a non-finite p. */
zha_status zha_dense_topp_attn(const zha_tree *t, const void *q, const void *k_cache,
                               const void *v_cache, float p, int32_t max_budget, void *out,
                               int32_t *sel_tokens, int32_t *sel_count, uint32_t *status, void *ws,
                               uint64_t ws_bytes, void *stream);

/* Streaming read of `bytes` from device buffer `buf` (sum into *sink, a
 * device float); gives the achievable HBM read bandwidth on this GPU. */
zha_status zha_bw_probe(const void *buf, uint64_t bytes, float *sink, void *stream);

/* Static text for a status code. */
const char *zha_status_string(zha_status s);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
