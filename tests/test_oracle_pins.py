"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Page: "How does a tree of summaries search a context? How ZHA works"
([ZHA lesson]).  Each test names the statement it pins.  Nothing here calls
the GPU library; the independent quantities (true log-sum-exp of a subtree,
the direct one-level summary of a span, dense softmax attention, brute force
over subsets) are written from their definitions with numpy/scipy.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tree(O, n=256, d=16, c=4, R=3, L=3, s=0.7, seed=0, ref_scale=1.0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d))
    refs = ref_scale * rng.standard_normal((R, d))
    return K, refs, O.build(K, refs, c, L, s)


def _direct(keys_span, refs, s):
    """Summary of a span straight from its raw keys (no recursion)."""
    R, d = refs.shape
    kap = np.zeros((R, d))
    bet = np.zeros(R)
    for r in range(R):
        z = s * keys_span @ refs[r]
        w = np.exp(z - z.max())
        w /= w.sum()
        kap[r] = w @ keys_span
        bet[r] = logsumexp(z) - s * kap[r] @ refs[r]
    return kap, bet


def _spans(tree, l):
    span = tree.c ** l
    return [(j * span, (j + 1) * span) for j in range(tree.nodes_at(l))]


# P1 -- [ZHA lesson] "What does a node summarize?": at one of its own
# reference queries a node's estimate has no error, so its score at rho_r equals
# the true log-sum-exp of its subtree's keys under rho_r.
def test_exact_at_reference(oracle_mod):
    O = oracle_mod
    K, refs, tr = _tree(O)
    for l in range(1, tr.L + 1):
        kl, bl = tr.level(l)
        for j, (a, z) in enumerate(_spans(tr, l)):
            for r in range(tr.R):
                est = O.node_score(kl[j], bl[j], refs[r], tr.s)
                true = logsumexp(tr.s * K[a:z] @ refs[r])
                assert abs(est - true) <= 1e-12 * max(1.0, abs(true))


# P2 -- same section: the estimate is a lower bound of the true log-sum-exp
# for every query (tangents of a convex function lie below it).
def test_never_exceeds_true_value(oracle_mod):
    O = oracle_mod
    K, refs, tr = _tree(O, seed=1)
    rng = np.random.default_rng(7)
    queries = [np.zeros(tr.d), K[5], 10 * K[77], refs[0] + 1e-3]
    queries += [sc * rng.standard_normal(tr.d) for sc in (0.1, 1.0, 5.0) for _ in range(20)]
    worst = -np.inf
    for q in queries:
        for l in range(1, tr.L + 1):
            kl, bl = tr.level(l)
            for j, (a, z) in enumerate(_spans(tr, l)):
                est = O.node_score(kl[j], bl[j], q, tr.s)
                true = logsumexp(tr.s * K[a:z] @ q)
                worst = max(worst, est - true)
                assert est <= true + 1e-12 * max(1.0, abs(true))
    assert worst < 0.5  # the bound is tight somewhere, loose nowhere absurd


# P3 -- same section (the paper's footnote): summarising the children's
# summaries yields exactly the summary of the raw keys of the whole span.
def test_merge_equals_direct_summary(oracle_mod):
    O = oracle_mod
    K, refs, tr = _tree(O, n=4 ** 3 * 2 + 9, seed=2)
    for l in range(1, tr.L + 1):
        kl, bl = tr.level(l)
        for j, (a, z) in enumerate(_spans(tr, l)):
            kap, bet = _direct(K[a:z], refs, tr.s)
            assert np.max(np.abs(kl[j] - kap)) <= 1e-12 * max(1.0, np.max(np.abs(kap)))
            assert np.max(np.abs(bl[j] - bet)) <= 1e-12 * max(1.0, np.max(np.abs(bet)))


# P4 -- closed forms of the summary: a zero reference gives the plain mean key
# and bias ln|span|; a span of identical keys k gives key k, bias ln|span|,
# and the score is then exact for every query.
def test_closed_forms(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(3)
    n, d, c, L = 64, 8, 4, 3
    K = rng.standard_normal((n, d))
    refs = np.zeros((2, d))
    refs[1] = rng.standard_normal(d)
    tr = O.build(K, refs, c, L, 0.9)
    for l in range(1, L + 1):
        kl, bl = tr.level(l)
        for j, (a, z) in enumerate(_spans(tr, l)):
            assert np.allclose(kl[j][0], K[a:z].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(bl[j][0] - math.log(z - a)) < 1e-12
    k = rng.standard_normal(d)
    Ksame = np.tile(k, (n, 1))
    tr2 = O.build(Ksame, rng.standard_normal((3, d)), c, L, 1.3)
    for l in range(1, L + 1):
        kl, bl = tr2.level(l)
        for j in range(tr2.nodes_at(l)):
            assert np.allclose(kl[j], np.tile(k, (3, 1)), atol=1e-13)
            assert np.allclose(bl[j], math.log(c ** l), atol=1e-12)
            q = 3 * rng.standard_normal(d)
            est = O.node_score(kl[j], bl[j], q, 1.3)
            true = logsumexp(np.full(c ** l, 1.3 * k @ q))
            assert abs(est - true) < 1e-11


def _dense(q, K, V, s):
    z = s * K @ q
    w = np.exp(z - z.max())
    w /= w.sum()
    return w @ V


# P5 -- p = 1 (or K at least every candidate set) opens everything, so the
# output is plain dense attention; comparisons = R * (all nodes) + n.  Holds
# on ragged lengths too (the partial-chunk reading).
@pytest.mark.parametrize("n", [256, 256 + 3, 64 * 3 + 16 * 2 + 4 + 1, 3])
def test_open_all_is_dense_attention(oracle_mod, n):
    O = oracle_mod
    rng = np.random.default_rng(n)
    d, c, R, L, s = 12, 4, 3, 3, 0.5
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    refs = rng.standard_normal((R, d))
    tr = O.build(K, refs, c, L, s)
    q = 2 * rng.standard_normal(d)
    total_nodes = sum(n // c ** l for l in range(1, L + 1))
    for mode, kw in ((O.TOPP, dict(p=1.0)), (O.TOPK, dict(ksched=[10 ** 6]))):
        sel, st = O.walk(tr, q, mode, **kw)
        assert np.array_equal(sel, np.arange(n))
        assert st["comparisons"] == R * total_nodes + n
        out, lse = O.attend(sel, q, K, V, s)
        ref = _dense(q, K, V, s)
        assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        assert abs(lse - logsumexp(s * K @ q)) < 1e-12 * max(1.0, abs(lse))
        assert abs(O.mass_kept(sel, q, K, s) - 1.0) < 1e-12


def test_open_all_comparisons_demo_geometry(oracle_mod):
    O = oracle_mod
    g = json.load(open(os.path.join(GOLDEN, "widget_accounting.json")))
    rng = np.random.default_rng(11)
    n, c, R, L = (g["geometry"][k] for k in ("tokens", "chunk", "references", "levels"))
    K = rng.standard_normal((n, 16))
    tr = O.build(K, rng.standard_normal((R, 16)) / 4, c, L, 0.25)
    sel, st = O.walk(tr, rng.standard_normal(16), O.TOPP, p=1.0)
    assert st["comparisons"] == g["derived"]["open_all_comparisons"]
    assert st["keys_read"] == n


# P6 -- the widget's printed accounting ([ZHA lesson], "Try it"): 64 top
# nodes; opening 4, 9, 25 at the three steps reads 100 keys for 564
# comparisons on any data; top-K 6 reads 24 keys (472 comparisons).
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_widget_accounting(oracle_mod, seed):
    O = oracle_mod
    g = json.load(open(os.path.join(GOLDEN, "widget_accounting.json")))
    n, c, R, L = (g["geometry"][k] for k in ("tokens", "chunk", "references", "levels"))
    rng = np.random.default_rng(seed)
    d = 16
    if seed == 2:   # structured keys too
        cent = rng.standard_normal((64, d))
        K = np.repeat(cent, n // 64, axis=0) + 0.3 * rng.standard_normal((n, d))
    else:
        K = rng.standard_normal((n, d))
    tr = O.build(K, rng.standard_normal((R, d)) / 4, c, L, 0.25)
    assert tr.nodes_at(L) == g["geometry"]["top_nodes"]
    q = rng.standard_normal(d)
    trace = g["one_place_trace_scored_opened"]
    sel, st = O.walk(tr, q, O.TOPK, ksched=[o for _, o in trace])
    assert [[a, b] for a, b in zip(st["scored"], st["opened"])] == trace
    assert st["keys_read"] == g["one_place_keys_read"] == len(sel)
    assert st["comparisons"] == g["one_place_comparisons"]
    sel, st = O.walk(tr, q, O.TOPK, ksched=[6])
    assert st["keys_read"] == g["topk6_keys_read"]
    assert st["comparisons"] == g["derived"]["topk6_comparisons"]
    # comparisons - keys read is R per scored node (eight-place row: 604 nodes)
    e = g["eight_places_comparisons"] - g["eight_places_keys_read"]
    assert e % R == 0 and e // R == g["derived"]["eight_places_scored_nodes"]
    assert g["unstructured_comparisons"] % R == 0
    for p in (0.5, 0.9, 0.99):
        sel, st = O.walk(tr, q, O.TOPP, p=p)
        assert (st["comparisons"] - st["keys_read"]) % R == 0
        assert st["keys_read"] % c == 0


def _single_level(O, m, d=6, c=2, R=2, s=1.0, seed=0, scale=1.0):
    """A one-level tree: the m level-1 nodes are the whole first candidate set."""
    rng = np.random.default_rng(seed)
    K = scale * rng.standard_normal((m * c, d))
    refs = rng.standard_normal((R, d))
    tr = O.build(K, refs, c, 1, s)
    return K, refs, tr


def _direct_scores(K, refs, c, s, q, level=1):
    span = c ** level
    out = []
    for j in range(K.shape[0] // span):
        kap, bet = _direct(K[j * span:(j + 1) * span], refs, s)
        out.append(max(s * kap[r] @ q + bet[r] for r in range(refs.shape[0])))
    return np.array(out)


# P7 -- [ZHA lesson] "How does top-p differ from top-K?": top-p takes the
# fewest nodes whose estimated attention mass together reaches p; checked by
# brute force over all subsets of up to 12 candidates.
@pytest.mark.parametrize("seed", range(12))
def test_topp_is_smallest_set(oracle_mod, seed):
    O = oracle_mod
    m = 4 + seed % 9
    K, refs, tr = _single_level(O, m, seed=seed, scale=1.0 + seed % 3)
    rng = np.random.default_rng(100 + seed)
    q = 2 * rng.standard_normal(K.shape[1])
    S = _direct_scores(K, refs, 2, 1.0, q)
    P = np.exp(S - S.max())
    P /= P.sum()
    for p in (0.3, 0.6, 0.9, 0.97):
        sel, st = O.walk(tr, q, O.TOPP, p=p)
        opened = sorted(set((sel // 2).tolist()))
        best = None
        for size in range(1, m + 1):
            masses = [(sum(P[list(cmb)]), cmb) for cmb in itertools.combinations(range(m), size)
                      if sum(P[list(cmb)]) >= p - 1e-15]
            if masses:
                best = max(masses)
                break
        assert len(opened) == len(best[1])
        assert abs(sum(P[opened]) - best[0]) < 1e-12


# P9 -- greedy special case: top-K = 1 at every step is the argmax descent,
# found here by brute force over directly-summarised spans.
@pytest.mark.parametrize("seed", range(6))
def test_greedy_descent(oracle_mod, seed):
    O = oracle_mod
    rng = np.random.default_rng(seed)
    n, d, c, R, L, s = 3 * 4 ** 3, 8, 4, 3, 3, 0.8
    K = rng.standard_normal((n, d)) + np.repeat(rng.standard_normal((n // 16, d)), 16, axis=0)
    refs = rng.standard_normal((R, d))
    tr = O.build(K, refs, c, L, s)
    q = 2 * rng.standard_normal(d)
    sel, st = O.walk(tr, q, O.TOPK, ksched=[1])
    span = c ** L
    cand = list(range(n // span))
    level = L
    while True:
        sc = [max(s * kap @ q + bet for kap, bet in zip(*_direct(K[j * c ** level:(j + 1) * c ** level], refs, s)))
              for j in cand]
        best = cand[int(np.argmax(sc))]
        if level == 1:
            break
        cand = [best * c + e for e in range(c)]
        level -= 1
    assert np.array_equal(sel, np.arange(best * c, best * c + c))
    assert st["opened"] == [1] * L and st["scored"] == [n // span] + [c] * (L - 1)


# Gap of a top-K cut = score difference at the cut (the parity contract's
# stability measure), checked against independently computed scores.
def test_topk_gap_definition(oracle_mod):
    O = oracle_mod
    K, refs, tr = _single_level(O, 10, seed=5)
    q = np.random.default_rng(9).standard_normal(K.shape[1])
    S = np.sort(_direct_scores(K, refs, 2, 1.0, q))[::-1]
    for k in (1, 3, 7):
        _, st = O.walk(tr, q, O.TOPK, ksched=[k])
        assert abs(st["gap"] - (S[k - 1] - S[k])) < 1e-12
    _, st = O.walk(tr, q, O.TOPK, ksched=[10])
    assert st["gap"] == math.inf and st["unforced_scored"] == 0


# READING (ties): equal scores open in span order.  Two identical chunks give
# identical nodes; top-K = 1 must pick the earlier one.
def test_tie_break_by_span_start(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(4)
    d, c = 6, 2
    K = rng.standard_normal((8, d))
    K[6:8] = K[2:4]          # node 3 duplicates node 1
    K[0:2] *= 0.01           # nodes 0 and 2 weak
    K[4:6] *= 0.01
    refs = rng.standard_normal((2, d))
    tr = O.build(K, refs, c, 1, 1.0)
    q = 3 * (K[2] + K[3])
    k1, b1 = tr.level(1)
    assert np.array_equal(k1[1], k1[3]) and np.array_equal(b1[1], b1[3])
    s_all = [O.node_score(k1[j], b1[j], q, 1.0) for j in range(4)]
    assert s_all[1] == s_all[3] == max(s_all)
    sel, _ = O.walk(tr, q, O.TOPK, ksched=[1])
    assert np.array_equal(sel, [2, 3])
    sel, _ = O.walk(tr, q, O.TOPK, ksched=[2])
    assert np.array_equal(sel, [2, 3, 6, 7])


# READING (p outside (0, 1)): p >= 1 opens all, p <= 0 opens exactly one.
def test_p_edges(oracle_mod):
    O = oracle_mod
    K, refs, tr = _single_level(O, 9, seed=8)
    q = np.random.default_rng(1).standard_normal(K.shape[1])
    sel, st = O.walk(tr, q, O.TOPP, p=1.5)
    assert st["opened"] == [9] and st["forced"] == [1]
    sel, st = O.walk(tr, q, O.TOPP, p=0.0)
    assert st["opened"] == [1]
    S = _direct_scores(K, refs, 2, 1.0, q)
    assert np.array_equal(sel // 2, [int(np.argmax(S))] * 2)


# READING (partial chunks): the roots plus the raw tail partition [0, n), so
# every key can be reached; parentless nodes join the first candidate list.
def test_roots_and_tail_partition(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(6)
    c, L = 4, 3
    for n in (0, 1, 3, 4, 17, 64, 64 + 16 + 4 + 3, 2 * 64 + 3 * 16 + 2 * 4 + 1):
        K = rng.standard_normal((max(n, 1), 5))[:n]
        tr = O.build(K, rng.standard_normal((2, 5)), c, L, 1.0)
        sel, st = O.walk(tr, rng.standard_normal(5), O.TOPP, p=1.0)
        assert np.array_equal(sel, np.arange(n))
        nl = [n // c ** l for l in range(L + 2)]
        roots = nl[L] + sum(nl[l] - c * nl[l + 1] for l in range(1, L))
        assert (st["scored"][0] if st["steps"] else 0) == roots


# P11 -- max-shifted softmax / log-sum-exp stay finite for scores ~ +-1e4.
def test_overflow_safety(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(12)
    n, d = 64, 4
    K = 100 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    refs = 100 * rng.standard_normal((2, d))
    tr = O.build(K, refs, 4, 3, 1.0)
    assert np.all(np.isfinite(tr.k)) and np.all(np.isfinite(tr.b))
    q = 100 * rng.standard_normal(d)
    for p in (0.9, 1.0):
        sel, st = O.walk(tr, q, O.TOPP, p=p)
        out, lse = O.attend(sel, q, K, V, 1.0)
        assert np.all(np.isfinite(out)) and np.isfinite(lse)
        assert abs(lse) > 1e3


# The oracle's tree depends on each node's span only: building over a prefix
# gives a prefix of every level (so appending tokens never rewrites a node).
def test_prefix_property(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(13)
    K = rng.standard_normal((300, 6))
    refs = rng.standard_normal((3, 6))
    full = O.build(K, refs, 4, 3, 0.6)
    part = O.build(K[:173], refs, 4, 3, 0.6)
    for l in range(1, 4):
        a, b = part.level(l)
        A, B = full.level(l)
        assert np.array_equal(a, A[: a.shape[0]]) and np.array_equal(b, B[: b.shape[0]])


# P-bf16 -- bf16 node keys (a storage variant of "What does a node
# summarize?"): the rounding is round-to-nearest-even to 8 significant bits,
# checked on hand-computed ties and against torch's float32 -> bfloat16
# conversion; every stored key is a bf16 value within half a bf16 step of the
# fp64 summary; and because each bias is taken against the stored key, the
# node's tangent for rho_r is still exact at rho_r.
def test_round_bf16_definition(oracle_mod):
    O = oracle_mod
    cases = {1.0: 1.0, 1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, 1 + 2 ** -8 + 2 ** -20: 1 + 2 ** -7,
             -2.5: -2.5, 3.14159: 3.140625, 0.0: 0.0, 255.5: 256.0, 2 ** -100 * 1.00390625: 2 ** -100}
    for x, want in cases.items():
        assert O.round_bf16(x) == want, (x, O.round_bf16(x), want)
    import torch
    rng = np.random.default_rng(7)
    xs = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.round_bf16(float(x)) for x in xs])
    assert np.array_equal(got, ref)


def test_bf16_keys_tangent_exact_at_reference(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(3)
    n, d, c, R, L, s = 256, 16, 4, 3, 3, 0.7
    K = rng.standard_normal((n, d))
    refs = rng.standard_normal((R, d))
    tr = O.build(K, refs, c, L, s, key_bf16=True)
    exact = O.build(K, refs, c, L, s)
    for l in range(1, L + 1):
        kl, bl = tr.level(l)
        for j, (a, z) in enumerate(_spans(tr, l)):
            for r in range(R):
                assert all(O.round_bf16(x) == x for x in kl[j, r])
                tangent = s * kl[j, r] @ refs[r] + bl[j, r]
                true = logsumexp(s * K[a:z] @ refs[r])
                assert abs(tangent - true) <= 1e-12 * max(1.0, abs(true))
    k1, _ = tr.level(1)
    e1, _ = exact.level(1)
    assert np.all(np.abs(k1 - e1) <= np.ldexp(1.0, np.floor(np.log2(np.abs(e1) + 1e-300)).astype(int) - 8))


# ---- multi-level walks against a brute-force numpy walk --------------------
#
# The walk of [ZHA lesson] "Run a small tree yourself" (route) written again in
# numpy, from scratch, over node scores taken from the direct one-level
# summary of each node's span (pinned above to equal the recursive records):
# at every step the whole candidate list -- the children of every node opened
# at the step before, across all parents -- is normalised by one softmax, and
# the cut is taken on that joint list ([ZHA lesson] "How does top-p differ
# from top-K?": the smallest score-ordered group whose mass reaches p).

def _np_roots(n, c, L):
    nl = [n // c ** l for l in range(L + 2)]
    roots = [(L, j) for j in range(nl[L])]
    for l in range(L - 1, 0, -1):
        roots += [(l, j) for j in range(c * nl[l + 1], nl[l])]
    return sorted(roots, key=lambda x: x[1] * c ** x[0])


def _np_walk(K, refs, c, L, s, q, p=None, k=None):
    """Returns (selected tokens, per-step [scored, opened], per-step masses
    in cut order with the cut m and the sorted scores) of one walk."""
    n = K.shape[0]
    memo = {}

    def score(node):
        if node not in memo:
            l, j = node
            kap, bet = _direct(K[j * c ** l:(j + 1) * c ** l], refs, s)
            memo[node] = max(s * kap[r] @ q + bet[r] for r in range(refs.shape[0]))
        return memo[node]

    cand = _np_roots(n, c, L)
    sel, trace, steps = [], [], []
    t = 0
    while cand:
        S = np.array([score(x) for x in cand])
        starts = np.array([j * c ** l for (l, j) in cand])
        order = np.lexsort((starts, -S))             # score descending, then span start
        P = np.exp(S - S.max())
        P /= P.sum()
        if k is not None:
            m = min(k, len(cand))
        elif p >= 1.0:
            m = len(cand)
        else:
            cum = np.cumsum(P[order])
            hit = np.nonzero(cum >= p)[0]
            m = int(hit[0]) + 1 if hit.size else len(cand)
        opened = [cand[i] for i in order[:m]]
        trace.append([len(cand), m])
        steps.append((S[order], P[order], m))
        nxt = []
        for (l, j) in opened:
            if l == 1:
                sel.extend(range(j * c, j * c + c))
            else:
                nxt.extend((l - 1, j * c + e) for e in range(c))
        cand = sorted(nxt, key=lambda x: x[1] * c ** x[0])
        t += 1
    sel.extend(range(c * (n // c), n))
    return np.array(sorted(sel), dtype=np.int64), trace, steps


def _clustered(rng, n, d, seg, amp):
    cent = rng.standard_normal((n // seg + 1, d))
    cent /= np.linalg.norm(cent, axis=1, keepdims=True)
    return amp * np.repeat(cent, seg, axis=0)[:n] + rng.standard_normal((n, d))


# Top-p over three levels: the joint softmax across all opened parents.  A cut
# made per parent, or a softmax over one parent's children, opens other nodes
# at steps 2 and 3 on these walks.
@pytest.mark.parametrize("p", [0.5, 0.9])
@pytest.mark.parametrize("n", [4 ** 3 * 6, 4 ** 3 * 6 + 4 * 3 + 2])
def test_multilevel_topp_walk_brute_force(oracle_mod, p, n):
    O = oracle_mod
    rng = np.random.default_rng(int(p * 10) + n)
    d, c, R, L, s = 8, 4, 3, 3, 0.6
    K = _clustered(rng, n, d, 11, 2.5)
    refs = rng.standard_normal((R, d)) / 2
    tr = O.build(K, refs, c, L, s)
    multi = 0
    for i in range(50):
        q = 2.5 * K[rng.integers(0, n)] / max(np.linalg.norm(K[0]), 1e-9) + 0.5 * rng.standard_normal(d)
        sel, st = O.walk(tr, q, O.TOPP, p=p)
        want, trace, _ = _np_walk(K, refs, c, L, s, q, p=p)
        assert np.array_equal(sel, want), i
        assert [[a, b] for a, b in zip(st["scored"], st["opened"])] == trace, i
        assert st["keys_read"] == len(want)
        assert st["comparisons"] == R * sum(a for a, _ in trace) + len(want)
        multi += sum(1 for a, b in trace[1:] if b > 1 and a > c)
    assert multi > 20          # many steps cut a list spanning several parents


@pytest.mark.parametrize("ks", [(3,), (2, 5, 7), (1, 4)])
def test_multilevel_topk_walk_brute_force(oracle_mod, ks):
    O = oracle_mod
    rng = np.random.default_rng(sum(ks))
    n, d, c, R, L, s = 4 ** 3 * 5 + 9, 8, 4, 3, 3, 0.6
    K = _clustered(rng, n, d, 7, 2.0)
    refs = rng.standard_normal((R, d)) / 2
    tr = O.build(K, refs, c, L, s)
    for i in range(20):
        q = 2.0 * rng.standard_normal(d)
        sel, st = O.walk(tr, q, O.TOPK, ksched=list(ks))
        # K may change per step: the schedule's last entry repeats
        want, trace = _np_walk_sched(K, refs, c, L, s, q, ks)
        assert np.array_equal(sel, want), i
        assert [[a, b] for a, b in zip(st["scored"], st["opened"])] == trace, i


def _np_walk_sched(K, refs, c, L, s, q, ks):
    """Top-K walk with a per-step K (brute force, as _np_walk)."""
    n = K.shape[0]
    cand = _np_roots(n, c, L)
    sel, trace = [], []
    t = 0
    while cand:
        S = np.array([max(s * kap[r] @ q + bet[r] for r in range(refs.shape[0]))
                      for kap, bet in (_direct(K[j * c ** l:(j + 1) * c ** l], refs, s) for (l, j) in cand)])
        starts = np.array([j * c ** l for (l, j) in cand])
        order = np.lexsort((starts, -S))
        m = min(ks[min(t, len(ks) - 1)], len(cand))
        trace.append([len(cand), m])
        nxt = []
        for i in order[:m]:
            l, j = cand[i]
            if l == 1:
                sel.extend(range(j * c, j * c + c))
            else:
                nxt.extend((l - 1, j * c + e) for e in range(c))
        cand = sorted(nxt, key=lambda x: x[1] * c ** x[0])
        t += 1
    sel.extend(range(c * (n // c), n))
    return np.array(sorted(sel), dtype=np.int64), trace


# The top-p cut gap (the stability measure of the parity contract): over the
# unforced steps, the smallest of the score drop at the cut, the overshoot
# C_m - p and the room p - C_(m-1) before the last opened node, all from the
# brute-force walk's independently sorted masses.
@pytest.mark.parametrize("p", [0.3, 0.7, 0.9])
def test_topp_gap_from_sorted_masses(oracle_mod, p):
    O = oracle_mod
    rng = np.random.default_rng(int(100 * p))
    n, d, c, R, L, s = 4 ** 3 * 4 + 6, 8, 4, 3, 3, 0.6
    K = _clustered(rng, n, d, 9, 2.0)
    refs = rng.standard_normal((R, d)) / 2
    tr = O.build(K, refs, c, L, s)
    which = {"score": 0, "over": 0, "room": 0}
    for i in range(50):
        q = 2.0 * rng.standard_normal(d)
        _, st = O.walk(tr, q, O.TOPP, p=p)
        _, _, steps = _np_walk(K, refs, c, L, s, q, p=p)
        want, arg = math.inf, None
        for Ssorted, Psorted, m in steps:
            if len(Ssorted) == 1:
                continue                              # forced: one candidate
            cum = np.cumsum(Psorted)
            terms = {"room": p - (cum[m - 2] if m >= 2 else 0.0)}
            if m < len(Ssorted):
                terms["over"] = cum[m - 1] - p
                terms["score"] = Ssorted[m - 1] - Ssorted[m]
            k = min(terms, key=terms.get)
            if terms[k] < want:
                want, arg = terms[k], k
        assert abs(st["gap"] - want) <= 1e-12, (i, st["gap"], want)
        if arg:
            which[arg] += 1
    assert all(v > 0 for v in which.values()), which   # each term decides some walk


# Attention over a strict subset of the keys ([ZHA lesson] "How is the tree
# built?" and "Common misunderstandings": attention runs on the chosen
# original keys only): a softmax over exactly K[sel] applied to V[sel], and
# the dense mass those keys hold, from numpy, on random unsorted-in-memory
# subsets far from the identity.
def test_attend_and_mass_on_strict_subsets(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(21)
    n, d, s = 300, 10, 0.4
    K = 2 * rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    for i in range(30):
        q = 2 * rng.standard_normal(d)
        size = int(rng.integers(1, n // 2))
        sel = np.sort(rng.choice(np.arange(n // 3, n), size=min(size, n - n // 3), replace=False))
        out, lse = O.attend(sel, q, K, V, s)
        z = s * K[sel] @ q
        w = np.exp(z - z.max())
        w /= w.sum()
        assert np.max(np.abs(out - w @ V[sel])) <= 1e-12 * max(1.0, np.max(np.abs(out)))
        assert abs(lse - logsumexp(z)) <= 1e-12 * max(1.0, abs(lse))
        zall = s * K @ q
        pall = np.exp(zall - zall.max())
        pall /= pall.sum()
        assert abs(O.mass_kept(sel, q, K, s) - pall[sel].sum()) <= 1e-12
    assert O.mass_kept(np.array([], dtype=np.int64), q, K, s) == 0.0
    out, lse = O.attend(np.array([], dtype=np.int64), q, K, V, s)
    assert np.all(out == 0.0) and lse == -math.inf
