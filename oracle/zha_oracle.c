/*
 * zha_oracle.c -- plain fp64 CPU oracle for tree-structured KV search (ZHA).
 *
 * TEST INFRASTRUCTURE ONLY (see zha_oracle.h).  Plain loops in double
 * precision, no blocking, no SIMD, no fusion.  A library sort (qsort) is the
 * only primitive used.  Citations name the page "How does a tree of summaries
 * search a context? How ZHA works" as [ZHA lesson] and one of its sections.
 */
#include "zha_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int64_t ora_level_nodes(int64_t n, int c, int l)
{
    /* [ZHA lesson] "Run a small tree yourself": a level is built from whole
     * chunks of the level below only, so level l holds floor(n / c^l) nodes. */
    int64_t m = n;
    for (int i = 0; i < l; ++i) m /= c;
    return m;
}

static int64_t ipow(int64_t b, int e)
{
    int64_t r = 1;
    for (int i = 0; i < e; ++i) r *= b;
    return r;
}

static double dot(int d, const double *a, const double *b)
{
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += a[i] * b[i];
    return acc;
}

double ora_round_bf16(double x)
{
    /* bfloat16 keeps 8 significant bits: scale the significand to [128, 256),
     * round to the nearest integer (ties to even: the default rounding mode
     * of nearbyint) and scale back. */
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);            /* x = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

void ora_summarize(int c, int R, int d, double s,
                   const double *child_k, const double *child_b,
                   const double *refs, double *node_k, double *node_b,
                   int key_bf16)
{
    /* [ZHA lesson] "What does a node summarize?": for each reference query
     * rho_r, score every child tangent as s<key, rho_r> + bias, take the
     * softmax of those scores as weights, the new key is the weighted sum of
     * the child keys, and the new bias is the log-sum-exp of the scores minus
     * s<new key, rho_r>.  The softmax and log-sum-exp are max-shifted.
     * With key_bf16 the key is stored rounded to bfloat16 and the bias is
     * taken against the stored key, so the score at rho_r stays the
     * log-sum-exp. */
    double *sig = (double *)malloc(sizeof(double) * (size_t)c);
    for (int r = 0; r < R; ++r) {
        const double *rho = refs + (size_t)r * d;
        double mx = -INFINITY;
        for (int i = 0; i < c; ++i) {
            const double *k = child_k + ((size_t)i * R + r) * d;
            sig[i] = s * dot(d, k, rho) + child_b[(size_t)i * R + r];
            if (sig[i] > mx) mx = sig[i];
        }
        double z = 0.0;
        for (int i = 0; i < c; ++i) z += exp(sig[i] - mx);
        double *out = node_k + (size_t)r * d;
        for (int e = 0; e < d; ++e) out[e] = 0.0;
        for (int i = 0; i < c; ++i) {
            double w = exp(sig[i] - mx) / z;
            const double *k = child_k + ((size_t)i * R + r) * d;
            for (int e = 0; e < d; ++e) out[e] += w * k[e];
        }
        if (key_bf16)
            for (int e = 0; e < d; ++e) out[e] = ora_round_bf16(out[e]);
        double lse = mx + log(z);
        node_b[r] = lse - s * dot(d, out, rho);
    }
    free(sig);
}

double ora_node_score(int R, int d, double s, const double *node_k,
                      const double *node_b, const double *q)
{
    /* [ZHA lesson] "What does a node summarize?": score = the largest over
     * reference queries of (s * dot(key_r, q) + bias_r). */
    double best = -INFINITY;
    for (int r = 0; r < R; ++r) {
        double v = s * dot(d, node_k + (size_t)r * d, q) + node_b[r];
        if (v > best) best = v;
    }
    return best;
}

void ora_build(int64_t n, int d, int c, int R, int L, double s,
               const double *keys, const double *refs,
               double *tree_k, double *tree_b, int key_bf16)
{
    /* [ZHA lesson] "How is the tree built?" and "Run a small tree yourself":
     * level 1 summarises each whole chunk of c neighbouring keys, a leaf
     * being the raw key for every reference with bias 0; level l >= 2
     * summarises each whole chunk of c level-(l-1) nodes. */
    double *ck = (double *)malloc(sizeof(double) * (size_t)c * R * d);
    double *cb = (double *)malloc(sizeof(double) * (size_t)c * R);
    int64_t off_prev = 0, off = 0;
    for (int l = 1; l <= L; ++l) {
        int64_t nl = ora_level_nodes(n, c, l);
        for (int64_t j = 0; j < nl; ++j) {
            for (int i = 0; i < c; ++i) {
                for (int r = 0; r < R; ++r) {
                    double *dst = ck + ((size_t)i * R + r) * d;
                    if (l == 1) {
                        const double *src = keys + (size_t)(j * c + i) * d;
                        memcpy(dst, src, sizeof(double) * (size_t)d);
                        cb[(size_t)i * R + r] = 0.0;
                    } else {
                        int64_t child = off_prev + j * c + i;
                        memcpy(dst, tree_k + ((size_t)child * R + r) * d,
                               sizeof(double) * (size_t)d);
                        cb[(size_t)i * R + r] = tree_b[(size_t)child * R + r];
                    }
                }
            }
            ora_summarize(c, R, d, s, ck, cb, refs,
                          tree_k + (size_t)(off + j) * R * d,
                          tree_b + (size_t)(off + j) * R, key_bf16);
        }
        off_prev = off;
        off += nl;
    }
    free(ck);
    free(cb);
}

/* ---- the walk --------------------------------------------------------- */

typedef struct {
    int level;
    int64_t j;       /* index within its level             */
    int64_t start;   /* first token of its span: j * c^level */
    double score;
} cand;

static int by_score_then_start(const void *a, const void *b)
{
    /* READING: order by score descending, then by span start ascending.  The
     * page sorts by mass; mass is monotone in score within a step. */
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    if (x->start < y->start) return -1;
    if (x->start > y->start) return 1;
    return 0;
}

static int by_start(const void *a, const void *b)
{
    const cand *x = (const cand *)a, *y = (const cand *)b;
    return (x->start > y->start) - (x->start < y->start);
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

int ora_walk(int64_t n, int d, int c, int R, int L, double s,
             const double *tree_k, const double *tree_b,
             const double *q, int mode, double p,
             const int32_t *ksched, int nk,
             int64_t *sel, int64_t *n_sel, ora_walk_stats *st)
{
    if (L < 1 || L > ORA_MAX_LEVELS || c < 2 || n < 0) return -1;
    if (mode == ORA_TOPK && (nk < 1 || ksched == NULL)) return -1;

    int64_t nl[ORA_MAX_LEVELS + 2], off[ORA_MAX_LEVELS + 2];
    nl[0] = n;
    off[1] = 0;
    for (int l = 1; l <= L; ++l) {
        nl[l] = ora_level_nodes(n, c, l);
        off[l + 1] = off[l] + nl[l];
    }
    nl[L + 1] = 0;

    memset(st, 0, sizeof(*st));
    st->gap = INFINITY;

    /* READING: the roots are all level-L nodes plus every node at a lower
     * level whose chunk above has not filled yet (no parent), in span order;
     * raw keys past the last whole level-1 chunk are always read. */
    int64_t total_nodes = off[L + 1];
    cand *cur = (cand *)malloc(sizeof(cand) * (size_t)(total_nodes + 1));
    cand *nxt = (cand *)malloc(sizeof(cand) * (size_t)(total_nodes + 1));
    int64_t ncur = 0;
    for (int l = L; l >= 1; --l) {
        int64_t first = (l == L) ? 0 : (int64_t)c * nl[l + 1];
        for (int64_t j = first; j < nl[l]; ++j) {
            cur[ncur].level = l;
            cur[ncur].j = j;
            cur[ncur].start = j * ipow(c, l);
            cur[ncur].score = 0.0;
            ++ncur;
        }
    }

    int64_t ns = 0;
    int t = 0;
    /* [ZHA lesson] "Run a small tree yourself" (route): score every
     * candidate, normalise with a softmax, sort, open a prefix, opened
     * bottom-level nodes give their keys and the others give their children
     * as the next candidates; stop when no candidates remain. */
    while (ncur > 0) {
        if (t >= ORA_MAX_LEVELS) break; /* cannot happen: depth <= L */
        st->scored[t] = (int32_t)ncur;
        for (int64_t i = 0; i < ncur; ++i) {
            int64_t node = off[cur[i].level] + cur[i].j;
            cur[i].score = ora_node_score(R, d, s, tree_k + (size_t)node * R * d,
                                          tree_b + (size_t)node * R, q);
        }
        qsort(cur, (size_t)ncur, sizeof(cand), by_score_then_start);

        /* softmax over the whole candidate list of this step */
        double mx = cur[0].score;
        double z = 0.0;
        for (int64_t i = 0; i < ncur; ++i) z += exp(cur[i].score - mx);

        int64_t m;
        int forced = 0;
        double gap = INFINITY;
        if (mode == ORA_TOPK) {
            /* [ZHA lesson] "How does top-p differ from top-K?": top-K opens
             * exactly K nodes.  READING: K may differ per step, and a step
             * with fewer than K candidates opens them all. */
            int32_t k = ksched[t < nk ? t : nk - 1];
            if (k < 1) k = 1;
            if ((int64_t)k >= ncur) {
                m = ncur;
                forced = 1;
            } else {
                m = k;
                gap = cur[m - 1].score - cur[m].score;
            }
        } else {
            /* [ZHA lesson] "How does top-p differ from top-K?": open the
             * smallest prefix of the mass-sorted list whose sum reaches p,
             * the element that crosses p included.  READING: p >= 1 opens
             * every candidate, p <= 0 opens one. */
            if (p >= 1.0) {
                m = ncur;
                forced = 1;
            } else if (p <= 0.0) {
                m = 1;
                if (ncur > 1) gap = cur[0].score - cur[1].score;
            } else {
                double cum = 0.0, prev = 0.0;
                m = ncur;
                for (int64_t i = 0; i < ncur; ++i) {
                    prev = cum;
                    cum += exp(cur[i].score - mx) / z;
                    if (cum >= p) {
                        m = i + 1;
                        break;
                    }
                }
                gap = p - prev;
                if (m < ncur) {
                    double g2 = cum - p;
                    double g3 = cur[m - 1].score - cur[m].score;
                    if (g2 < gap) gap = g2;
                    if (g3 < gap) gap = g3;
                }
            }
        }
        if (ncur == 1) {
            forced = 1;
            gap = INFINITY;
        }
        st->opened[t] = (int32_t)m;
        st->forced[t] = forced;
        if (!forced) {
            st->unforced_scored += ncur;
            if (gap < st->gap) st->gap = gap;
        }

        int64_t nn = 0;
        for (int64_t i = 0; i < m; ++i) {
            if (cur[i].level == 1) {
                for (int e = 0; e < c; ++e) sel[ns++] = cur[i].start + e;
            } else {
                int l = cur[i].level - 1;
                for (int e = 0; e < c; ++e) {
                    nxt[nn].level = l;
                    nxt[nn].j = cur[i].j * c + e;
                    nxt[nn].start = nxt[nn].j * ipow(c, l);
                    nxt[nn].score = 0.0;
                    ++nn;
                }
            }
        }
        qsort(nxt, (size_t)nn, sizeof(cand), by_start);
        cand *tmp = cur;
        cur = nxt;
        nxt = tmp;
        ncur = nn;
        ++t;
    }
    st->steps = t;

    for (int64_t i = (int64_t)c * nl[1]; i < n; ++i) sel[ns++] = i;
    qsort(sel, (size_t)ns, sizeof(int64_t), cmp_i64);
    *n_sel = ns;

    int64_t total_scored = 0;
    for (int i = 0; i < t; ++i) total_scored += st->scored[i];
    st->keys_read = ns;
    /* [ZHA lesson] "Run a small tree yourself": work = R per scored
     * candidate plus one per key read. */
    st->comparisons = (int64_t)R * total_scored + ns;

    free(cur);
    free(nxt);
    return 0;
}

void ora_attend(int64_t n_sel, const int64_t *sel, int d, double s,
                const double *q, const double *K, const double *V,
                double *out, double *lse)
{
    /* [ZHA lesson] "How is the tree built?" and "Common misunderstandings":
     * plain softmax attention over the original keys and values that the
     * walk picked (the summaries are used for routing only). */
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    if (n_sel <= 0) {
        *lse = -INFINITY;
        return;
    }
    double *lg = (double *)malloc(sizeof(double) * (size_t)n_sel);
    double mx = -INFINITY;
    for (int64_t i = 0; i < n_sel; ++i) {
        lg[i] = s * dot(d, K + (size_t)sel[i] * d, q);
        if (lg[i] > mx) mx = lg[i];
    }
    double z = 0.0;
    for (int64_t i = 0; i < n_sel; ++i) z += exp(lg[i] - mx);
    for (int64_t i = 0; i < n_sel; ++i) {
        double w = exp(lg[i] - mx) / z;
        const double *v = V + (size_t)sel[i] * d;
        for (int e = 0; e < d; ++e) out[e] += w * v[e];
    }
    *lse = mx + log(z);
    free(lg);
}

double ora_mass_kept(int64_t n, int64_t n_sel, const int64_t *sel, int d,
                     double s, const double *q, const double *K)
{
    /* [ZHA lesson] "Run a small tree yourself": the share of the true dense
     * softmax over all keys that falls on the keys read. */
    if (n <= 0) return 0.0;
    double *lg = (double *)malloc(sizeof(double) * (size_t)n);
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        lg[i] = s * dot(d, K + (size_t)i * d, q);
        if (lg[i] > mx) mx = lg[i];
    }
    double z = 0.0;
    for (int64_t i = 0; i < n; ++i) z += exp(lg[i] - mx);
    double kept = 0.0;
    for (int64_t i = 0; i < n_sel; ++i) kept += exp(lg[sel[i]] - mx) / z;
    free(lg);
    return kept;
}
