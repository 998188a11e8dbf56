"""The walk-validity check used by the GPU parity tests (tests/parity.py,
check_walk_valid), exercised on the CPU: the oracle's own walks are valid,
including those whose cut gap is under 1e-4; selections with a planted
mistake are not; where two candidates tie exactly, either choice is valid.
The rule it checks is [ZHA lesson] "How does top-p differ from top-K?": top-K
opens the K best candidates of a step, top-p the fewest best candidates whose
joint softmax mass reaches p."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import oracle as O
from tests import parity as P
from tree_structured_kv_amd import synth as S


def _blocks(sel, c, n):
    return O.blocks_of(sel, c, n)[0]


def _demo():
    w = replace(S.WORKLOADS[0], n=1024 + 7, segments=16)
    ps = S.structure(w, 0, 0)
    K, _ = S.pair_kv(w, 0, 0, ps=ps)
    Q = S.pair_queries(w, 0, 0, count=60, ps=ps)
    tr = O.build(K.astype(np.float64), S.refs(w, 0).astype(np.float64), w.chunk, w.levels, w.sharpness)
    return w, tr, Q


SELECTS = [dict(mode="topp", p=0.9), dict(mode="topp", p=0.5), dict(mode="topk", k=(3,)),
           dict(mode="topk", k=(2, 5, 7)), dict(mode="topp", p=1.0), dict(mode="topp", p=0.0)]


@pytest.mark.parametrize("si", range(len(SELECTS)))
def test_oracle_walks_are_valid(si):
    select = SELECTS[si]
    w, tr, Q = _demo()
    unstable = 0
    for q in Q:
        sel, st = P.oracle_walk(tr, q, select)
        unstable += st["gap"] <= P.GAP
        ok, why = P.check_walk_valid(tr, q, select, _blocks(sel, w.chunk, w.n), st)
        assert ok, why
    if select["mode"] == "topp" and 0 < select["p"] < 1:
        assert unstable > 0           # the checker is exercised where it matters


def test_planted_mistakes_are_invalid():
    w, tr, Q = _demo()
    c, n = w.chunk, w.n
    select = dict(mode="topp", p=0.9)
    caught = dict(dropped=0, extra=0, swapped=0, count=0)
    tried = swaps = 0
    for q in Q[:30]:
        sel, st = P.oracle_walk(tr, q, select)
        bl = list(_blocks(sel, c, n))
        if len(bl) < 2:
            continue
        tried += 1
        ok, _ = P.check_walk_valid(tr, q, select, bl[1:], st)
        caught["dropped"] += not ok
        never = next(j for j in range(n // c) if j not in bl and all(j // c != b // c for b in bl))
        ok, _ = P.check_walk_valid(tr, q, select, bl + [never], st)
        caught["extra"] += not ok
        st2 = dict(st, opened=list(st["opened"]))
        st2["opened"][-1] += 1
        ok, _ = P.check_walk_valid(tr, q, select, bl, st2)
        caught["count"] += not ok
        # swap the best opened level-1 block for the worst closed candidate of
        # the last step (a child of an opened parent): same step, same counts
        k1, b1 = tr.level(1)
        s_of = lambda j: max(tr.s * k1[j, r] @ q + b1[j, r] for r in range(tr.R))
        best = max(bl, key=s_of)
        closed = [p * c + x for p in set(j // c for j in bl) for x in range(c) if p * c + x not in bl]
        closed = [j for j in closed if s_of(best) - s_of(j) > 10 * P.VALID_TOL]
        if closed:
            worst = min(closed, key=s_of)
            ok, _ = P.check_walk_valid(tr, q, select, [j for j in bl if j != best] + [worst], st)
            caught["swapped"] += not ok
            swaps += 1
    assert tried >= 20
    assert caught["dropped"] == tried and caught["extra"] == tried and caught["count"] == tried
    assert swaps >= 10 and caught["swapped"] == swaps


def test_exact_tie_either_choice_is_valid():
    """Two identical chunks give identical nodes: top-K 1 may open either
    under the validity rule (the tie-break reading picks the earlier one, and
    the bit-exact check holds the GPU to that)."""
    rng = np.random.default_rng(4)
    d, c = 6, 2
    K = rng.standard_normal((8, d))
    K[6:8] = K[2:4]
    K[0:2] *= 0.01
    K[4:6] *= 0.01
    refs = rng.standard_normal((2, d))
    tr = O.build(K, refs, c, 1, 1.0)
    q = 3 * (K[2] + K[3])
    sel, st = O.walk(tr, q, O.TOPK, ksched=[1])
    assert np.array_equal(sel, [2, 3]) and st["gap"] == 0.0
    select = dict(mode="topk", k=(1,))
    assert P.check_walk_valid(tr, q, select, [1], st)[0]
    assert P.check_walk_valid(tr, q, select, [3], st)[0]
    assert not P.check_walk_valid(tr, q, select, [0], st)[0]
