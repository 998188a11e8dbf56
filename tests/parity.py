"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding and the fp64 oracle on the same seeded inputs, and compare them under
one contract:

* tree records: row-wise |gpu - oracle|_inf <= 2e-5 * max(1, |oracle|_inf);
* selections: bit-exact (set of keys, per-step scored/opened counts,
  comparisons) on every walk whose oracle cut gap exceeds 1e-4 (score units
  for an ordering decision, mass units for the top-p threshold);
* outputs: against oracle attention over the GPU's own selection.  fp32:
  row-wise |gpu - oracle|_inf / |oracle|_inf <= 1e-5.  bf16 (fp32 arithmetic,
  one final round-to-nearest-even): every element within 2e-3 of the power
  of two at or above its exact value, plus 1e-5 of the row's max for the
  fp32 arithmetic before the rounding.  Correct rounding to 8 significant
  bits errs by at most 2^-9 (1.95e-3) of that power of two; measured against
  the element itself or the row's max the same rounding can reach 2^-8, so
  no such reading of 2e-3 holds for a correctly rounded bf16 output.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O
from tree_structured_kv_amd import synth as S

GAP = 1e-4
TOL_TREE = 2e-5
TOL_OUT = {"f32": 1e-5, "bf16": 2e-3}


def make_inputs(w: S.Workload, pairs=None, unstructured=False):
    """K, V [B][H][n][d], Q [B][Hq][d], refs [H][R][d] as float32 numpy (bf16-exact
    for bf16 workloads).  Pairs outside `pairs` are copies of the first listed."""
    B, H = w.batch, w.kv_heads
    K = np.empty((B, H, w.n, w.d), np.float32)
    V = np.empty_like(K)
    Q = np.empty((B, w.heads, w.d), np.float32)
    want = pairs if pairs is not None else [(b, g) for b in range(B) for g in range(H)]
    done = {}
    for (b, g) in want:
        ps = None if unstructured else S.structure(w, b, g)
        k, v = S.pair_kv(w, b, g, unstructured=unstructured, ps=ps)
        K[b, g], V[b, g] = k, v
        Q[b, g * w.group:(g + 1) * w.group] = S.pair_queries(
            w, b, g, ps=ps, unstructured_keys=k if unstructured else None)
        done[(b, g)] = True
    b0, g0 = want[0]
    for b in range(B):
        for g in range(H):
            if (b, g) not in done:
                K[b, g], V[b, g] = K[b0, g0], V[b0, g0]
                Q[b, g * w.group:(g + 1) * w.group] = Q[b0, g0 * w.group:(g0 + 1) * w.group]
    R = np.stack([S.refs(w, g) for g in range(H)])
    return K, V, Q, R


def oracle_tree(w: S.Workload, K, R, b, g, n, key_bf16=False):
    return O.build(K[b, g, :n].astype(np.float64), R[g].astype(np.float64), w.chunk, w.levels,
                   w.sharpness, key_bf16=key_bf16)


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def oracle_walk(tree, q, select):
    mode = O.TOPK if select["mode"] == "topk" else O.TOPP
    return O.walk(tree, q.astype(np.float64), mode, p=select.get("p", 0.9),
                  ksched=select.get("k", (1,)))


def gpu_tokens(blocks, count, c, n):
    """Selected tokens of one walk from the GPU's block list (+ the raw tail)."""
    bl = np.asarray(blocks[:count], dtype=np.int64)
    toks = (bl[:, None] * c + np.arange(c)[None, :]).reshape(-1)
    tail = np.arange(c * (n // c), n, dtype=np.int64)
    return np.sort(np.concatenate([toks, tail]))


def binade_top(x):
    """The power of two at or above |x| (2^-126 for zero)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.ceil(np.log2(ax)).astype(np.int64))


def out_ok(gpu, ref, dtype):
    """The output contract above; returns (ok, measured error)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if dtype == "f32":
        e = row_rel_err(gpu, ref)
        return e <= TOL_OUT["f32"], e
    slack = 1e-5 * max(np.max(np.abs(ref)), 1e-30)
    err = np.maximum(np.abs(gpu - ref) - slack, 0.0) / binade_top(ref)
    e = float(np.max(err))
    return e <= TOL_OUT["bf16"], e


def row_rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def select_struct(Z, select, max_blocks, max_candidates=0, engine="auto", attn="auto"):
    return Z.make_select(select["mode"], select.get("p", 0.9), select.get("k", (1,)),
                         max_blocks=max_blocks, max_candidates=max_candidates, engine=engine, attn=attn)


# ---- validity of a walk whose cut is not unique ---------------------------------
#
# Where the oracle's cut gap is at most GAP, several selections are correct.
# check_walk_valid replays the walk on the oracle's fp64 tree following the
# GPU's own choices and asks, at every step, that the set the GPU opened is a
# valid cut of that step's candidates under fp64 scores within VALID_TOL:
#   top-K: it holds min(K_t, |C_t|) candidates, and no candidate left closed
#          scores more than VALID_TOL above an opened one;
#   top-p: the same order condition; the opened softmax mass reaches
#          p - VALID_TOL; without its least-scoring member it stays below
#          p + VALID_TOL (p >= 1 opens all; p <= 0 opens one).
# The GPU reports only its level-1 blocks and per-step counts, so the opened
# set of a step is rebuilt: a level-1 candidate is open iff its block is
# selected; a higher candidate is open if a selected block lies below it; the
# rest of the step's opened count must come from the remaining higher
# candidates (opened, yet none of their descendants selected), taken in score
# order with every order of near-tied scores tried.  Every selected block must
# have been opened at some step, and the per-step scored/opened counts,
# steps, keys read and comparisons must match the replay.

VALID_TOL = 1e-4
_MAX_BRANCHES = 256


def _roots(n, c, L):
    nl = [n // c ** l for l in range(L + 2)]
    out = [(L, j) for j in range(nl[L])]
    for l in range(L - 1, 0, -1):
        out += [(l, j) for j in range(c * nl[l + 1], nl[l])]
    return sorted(out, key=lambda x: x[1] * c ** x[0])


def _scores(tree, cand, q):
    idx = np.array([tree.offsets[l] + j for (l, j) in cand], dtype=np.int64)
    k = tree.k[idx]
    b = tree.b[idx]
    return np.max(tree.s * np.einsum("nrd,d->nr", k, q) + b, axis=1)


def _cut_ok(select, t, S, P, opened_mask):
    n = len(S)
    m = int(opened_mask.sum())
    if m == 0:
        return False, "nothing opened"
    if n == 1:
        return (m == 1), "forced single"
    closed = ~opened_mask
    if closed.any() and S[opened_mask].min() < S[closed].max() - VALID_TOL:
        return False, f"order: opened {S[opened_mask].min():.6f} < closed {S[closed].max():.6f}"
    if select["mode"] == "topk":
        ks = select.get("k", (1,))
        k = ks[min(t, len(ks) - 1)]
        return (m == min(k, n)), f"top-K count {m} != {min(k, n)}"
    p = select.get("p", 0.9)
    if p >= 1.0:
        return (m == n), "p >= 1 opens all"
    if p <= 0.0:
        return (m == 1), "p <= 0 opens one"
    mass = float(P[opened_mask].sum())
    if mass < p - VALID_TOL:
        return False, f"mass {mass:.6f} < p"
    if mass - float(P[opened_mask].min()) >= p + VALID_TOL:
        return False, f"not minimal: {mass - float(P[opened_mask].min()):.6f} >= p"
    return True, ""


def check_walk_valid(tree, q, select, gpu_blocks, gpu_stats):
    """(ok, reason): the GPU's walk is a sequence of valid cuts (see above)."""
    import itertools
    q = np.asarray(q, np.float64)
    n, c, L = tree.n, tree.c, tree.L
    G1 = set(int(x) for x in gpu_blocks)
    if len(G1) != len(gpu_blocks):
        return False, "a block listed twice"
    anc = {l: set(j // c ** (l - 1) for j in G1) for l in range(2, L + 1)}
    scored, opened = list(gpu_stats["scored"]), list(gpu_stats["opened"])
    fail = []

    def rec(t, cand, seen1, sc_sum):
        if not cand:
            if t != gpu_stats["steps"]:
                fail.append(f"steps {t} != {gpu_stats['steps']}")
                return False
            if seen1 != G1:
                fail.append(f"{len(G1 - seen1)} selected blocks never opened")
                return False
            keys = len(G1) * c + (n - c * (n // c))
            if gpu_stats["keys_read"] != keys or gpu_stats["comparisons"] != tree.R * sc_sum + keys:
                fail.append("keys read / comparisons")
                return False
            return True
        if t >= len(scored) or scored[t] != len(cand):
            fail.append(f"step {t}: scored {scored[t] if t < len(scored) else None} != {len(cand)}")
            return False
        S = _scores(tree, cand, q)
        P = np.exp(S - S.max())
        P /= P.sum()
        known = np.array([(j in G1) if l == 1 else (j in anc[l]) for (l, j) in cand])
        maybe = [i for i, (l, j) in enumerate(cand) if l >= 2 and not known[i]]
        e = opened[t] - int(known.sum())
        if e < 0 or e > len(maybe):
            fail.append(f"step {t}: opened {opened[t]} vs {int(known.sum())} forced open, {len(maybe)} free")
            return False
        choices = [()]
        if e > 0:
            starts = np.array([cand[i][1] * c ** cand[i][0] for i in maybe])
            ms = np.array([S[i] for i in maybe])
            order = [maybe[i] for i in np.lexsort((starts, -ms))]
            edge = S[order[e - 1]]
            must = [i for i in order[:e] if e == len(order) or S[i] > S[order[e]] + VALID_TOL]
            free = [i for i in order if i not in must and S[i] >= edge - VALID_TOL]
            need = e - len(must)
            combos = itertools.combinations(free, need)
            choices = [tuple(must) + cmb for cmb in itertools.islice(combos, _MAX_BRANCHES)]
        for ch in choices:
            mask = known.copy()
            mask[list(ch)] = True
            ok, why = _cut_ok(select, t, S, P, mask)
            if not ok:
                fail.append(f"step {t}: {why}")
                continue
            nxt = []
            s1 = set(seen1)
            for i in np.nonzero(mask)[0]:
                l, j = cand[i]
                if l == 1:
                    s1.add(j)
                else:
                    nxt.extend((l - 1, j * c + x) for x in range(c))
            nxt.sort(key=lambda x: x[1] * c ** x[0])
            if rec(t + 1, nxt, s1, sc_sum + len(cand)):
                return True
        return False

    ok = rec(0, _roots(n, c, L), set(), 0)
    return ok, ("" if ok else "; ".join(fail[-3:]))
