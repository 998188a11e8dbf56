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
