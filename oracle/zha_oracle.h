/*
 * zha_oracle.h -- plain fp64 CPU oracle for tree-structured KV search (ZHA).
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no source, header, table or helper with the GPU library.
 *
 * Source of every definition: the web page "How does a tree of summaries
 * search a context? How ZHA works" (learn.chabulab.com), abbreviated below as
 * [ZHA lesson], and its sections:
 *   "How is the tree built?"             -- levels of chunks, originals kept
 *   "What does a node summarize?"        -- summarize(), node score, tangents
 *   "How does top-p differ from top-K?"  -- the top-p cut
 *   "Run a small tree yourself"          -- level construction, the walk,
 *                                           comparison accounting
 *   "Common misunderstandings"           -- per-head walks, attention on
 *                                           originals
 * Readings where the page is silent are marked READING and listed in the
 * repository's design notes.
 */
#ifndef ZHA_ORACLE_H
#define ZHA_ORACLE_H
#include <stdint.h>

#define ORA_MAX_LEVELS 12

#define ORA_TOPP 0
#define ORA_TOPK 1

typedef struct {
    int32_t scored[ORA_MAX_LEVELS];  /* |C_t|: candidates scored at step t       */
    int32_t opened[ORA_MAX_LEVELS];  /* m_t: candidates opened at step t          */
    int32_t steps;                   /* number of steps taken                     */
    int32_t forced[ORA_MAX_LEVELS];  /* 1 if step t's cut needed no scores        */
    int64_t keys_read;               /* |Sigma| including the raw tail            */
    int64_t comparisons;             /* R * sum_t |C_t| + |Sigma|                 */
    int64_t unforced_scored;         /* sum of |C_t| over unforced steps          */
    double  gap;                     /* min cut gap over unforced steps (+inf)    */
} ora_walk_stats;

/* Number of nodes at level l (1..L) for n tokens: floor(n / c^l). */
int64_t ora_level_nodes(int64_t n, int c, int l);

/* x rounded to the nearest bfloat16 value (8 significant bits), ties to
 * even. */
double ora_round_bf16(double x);

/* One node from its c children, each holding R (key, bias) tangents.  With
 * key_bf16 != 0 the node's keys are stored rounded to bfloat16 and its
 * biases are computed from the rounded keys. */
void ora_summarize(int c, int R, int d, double s,
                   const double *child_k,   /* [c][R][d] */
                   const double *child_b,   /* [c][R]    */
                   const double *refs,      /* [R][d]    */
                   double *node_k,          /* [R][d]    */
                   double *node_b,          /* [R]       */
                   int key_bf16);

/* Node score for a query: max over r of s<key_r, q> + bias_r. */
double ora_node_score(int R, int d, double s, const double *node_k,
                      const double *node_b, const double *q);

/* Build levels 1..L over the first n keys.  Level l's nodes are stored at
 * node offset off_l = sum_{l' < l} ora_level_nodes(n, c, l') (level 1 at 0)
 * of tree_k [nodes][R][d] and tree_b [nodes][R]. */
void ora_build(int64_t n, int d, int c, int R, int L, double s,
               const double *keys,   /* [n][d] */
               const double *refs,   /* [R][d] */
               double *tree_k, double *tree_b,
               int key_bf16);        /* node keys stored as bfloat16 */

/* One walk for one query.  sel receives the selected token indices in
 * ascending order (capacity n).  Returns 0 on success, -1 on bad input. */
int ora_walk(int64_t n, int d, int c, int R, int L, double s,
             const double *tree_k, const double *tree_b,
             const double *q, int mode, double p,
             const int32_t *ksched, int nk,
             int64_t *sel, int64_t *n_sel, ora_walk_stats *st);

/* Attention of q over the listed original keys: out = sum_i w_i V_i with
 * w = softmax over the list of s<q, K_i>.  *lse gets log sum_i exp(s<q,K_i>). */
void ora_attend(int64_t n_sel, const int64_t *sel, int d, double s,
                const double *q, const double *K, const double *V,
                double *out, double *lse);

/* Dense attention mass that the listed keys hold: sum over the list of
 * softmax over all n keys of s<q, K_i>. */
double ora_mass_kept(int64_t n, int64_t n_sel, const int64_t *sel, int d,
                     double s, const double *q, const double *K);

#endif
