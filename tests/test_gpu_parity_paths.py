"""GPU parity on the paths and sizes the main parity file does not reach:
exact score ties (the tie-exact select), cuts too wide for their LDS stage or
register stage, a late prefill block at full size, and the length sweep's
deep trees (7 to 9 levels).  Contract: tests/parity.py; every walk is checked
(bit-exact where the cut is unique, else a valid cut at every step)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tree_structured_kv_amd import synth as S
from tests import parity as P
from tests.test_gpu_parity import _check_walk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from tree_structured_kv_amd import zha
    return zha


def _device(Z, w, K, V, Q, R, n_build, summary="f32"):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(dt).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(dt).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(dt).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                           w.n, w.sharpness, summary=summary)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, n_build)
    return Kt, Vt, Qt, idx


def _run(Z, idx, Qt, Kt, Vt, select, engine, qph=1, max_blocks=None):
    g = idx.geom
    sel = P.select_struct(Z, select, max_blocks or g.max_tokens // g.chunk, engine=engine)
    bufs = idx.search(Qt, sel, qph=qph)
    out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"], qph=qph)
    torch.cuda.synchronize()
    from tree_structured_kv_amd.zha import stats_to_dicts
    return (bufs["sel_blocks"].cpu().numpy(), bufs["sel_count"].cpu().numpy(),
            stats_to_dicts(bufs["stats"].cpu()), out.float().cpu().numpy(), int(bufs["status"].cpu()[0]))


# ---- exact ties ----------------------------------------------------------------

def _tied_inputs():
    """One chunk of 4 keys repeated over the whole cache (synth.repeated_chunk_pair):
    every node of a level holds the same record, so every cut falls among
    equal scores and the reading "equal scores open in span order" decides
    it alone."""
    w = replace(S.WORKLOADS[1], n=16384 + 16 + 4 + 3, batch=1, kv_heads=2, group=8, chunk=4, refs=4,
                levels=3)
    K = np.empty((1, 2, w.n, w.d), np.float32)
    V = np.empty_like(K)
    Q = np.empty((1, w.heads, w.d), np.float32)
    for g in range(2):
        K[0, g], V[0, g], Q[0, g * w.group:(g + 1) * w.group] = S.repeated_chunk_pair(w, g)
    R = np.stack([S.refs(w, g) for g in range(2)])
    return w, K, V, Q, R


@pytest.mark.parametrize("engine", ["persistent", "level-sync", "union", "block"])
@pytest.mark.parametrize("select", [dict(mode="topk", k=(70,)), dict(mode="topp", p=0.45),
                                    dict(mode="topk", k=(1,)), dict(mode="topk", k=(3, 100, 7))])
def test_exact_ties_open_in_span_order(Z, engine, select):
    w, K, V, Q, R = _tied_inputs()
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, w.n)
    blocks, count, stats, outs, status = _run(Z, idx, Qt, Kt, Vt, select, engine)
    assert status == 0
    trees = {g: P.oracle_tree(w, K, R, 0, g, w.n) for g in range(2)}
    tie_select = 0
    for h in range(w.heads):
        g = h // w.group
        q = Q[0, h]
        sel_o, st_o = P.oracle_walk(trees[g], q, select)
        assert st_o["gap"] == 0.0
        toks = P.gpu_tokens(blocks[h], count[h], w.chunk, w.n)
        # all scores of a step are equal: the cut is unique, compare exactly
        assert np.array_equal(toks, sel_o), (h, engine)
        assert stats[h]["scored"] == st_o["scored"] and stats[h]["opened"] == st_o["opened"], h
        assert stats[h]["comparisons"] == st_o["comparisons"]
        tie_select += bool(stats[h]["paths"] & Z.PATH_TIE_SELECT)
        ref, _ = O.attend(toks, q.astype(np.float64), K[0, g].astype(np.float64), V[0, g].astype(np.float64),
                          w.sharpness)
        assert P.out_ok(outs[0, h], ref, w.dtype)[0], h
    # more than 64 equal scores straddle every cut: the tie-exact select ran
    assert tie_select == w.heads, (tie_select, engine)


# ---- wide cuts: LDS and register stages overflow ----------------------------------

def _flat_inputs():
    """512K random keys, chunk 16, 3 levels, and queries of tiny norm: the node
    scores are nearly flat, so top-p 0.9 opens most candidates and the last
    step cuts a list of about 26,000 (over the 14,336 scores a union cut and
    the 6,144 a level-synchronous cut stage in LDS, and the 1,024 a
    prefill-block cut keeps in registers)."""
    w = replace(S.WORKLOADS[2], n=1 << 19, batch=1, kv_heads=1, group=16, chunk=16, refs=8, levels=3)
    K, V = S.pair_kv(w, 0, 0, unstructured=True)
    Q = S.small_queries(w, w.heads, 0.05)[None]
    R = np.stack([S.refs(w, 0)])
    return w, K[None, None], V[None, None], Q, R


_flat = {}


@pytest.mark.parametrize("engine,bit", [("union", "PATH_LDS_SPILL"), ("level-sync", "PATH_LDS_SPILL"),
                                        ("block", "PATH_LONG_LIST")])
def test_wide_cuts_spill_their_stage(Z, engine, bit):
    if "in" not in _flat:
        w, K, V, Q, R = _flat_inputs()
        _flat["in"] = (w, K, V, Q, R, P.oracle_tree(w, K, R, 0, 0, w.n))
    w, K, V, Q, R, tree = _flat["in"]
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, w.n)
    select = dict(mode="topp", p=0.9)
    blocks, count, stats, outs, status = _run(Z, idx, Qt, Kt, Vt, select, engine)
    assert status == 0
    hit = 0
    stable = 0
    for h in range(w.heads):
        q = Q[0, h]
        sel_o, st_o = P.oracle_walk(tree, q, select)
        toks = P.gpu_tokens(blocks[h], count[h], w.chunk, w.n)
        stable += _check_walk(tree, q, select, blocks[h, :count[h]], toks, stats[h], sel_o, st_o, (h, engine))
        assert max(stats[h]["scored"]) > 14336, stats[h]["scored"]
        hit += bool(stats[h]["paths"] & getattr(Z, bit))
        ref, _ = O.attend(toks, q.astype(np.float64), K[0, 0].astype(np.float64), V[0, 0].astype(np.float64),
                          w.sharpness)
        assert P.out_ok(outs[0, h], ref, w.dtype)[0], h
    assert hit == w.heads, (hit, engine)


# ---- a late prefill block at full size --------------------------------------------

def test_full_size_late_prefill_block(Z):
    """The streaming workload's last block: 4,096 queries per head at
    positions 258,048 .. 262,143 walk the tree of the 258,048 tokens before
    them (64 top nodes, chunk 16, R 8, 8 KV heads x 4 query heads), in the
    launch configuration the bench runs (block engine, union attention).  KV
    heads 0 and 7 hold their own seeded data (the other six copy them); 16
    sampled queries of each of their heads are checked against the oracle
    walk and attention (selection plus the block's keys up to the query)."""
    w = S.WORKLOADS[3]
    T = w.block
    T0 = w.n - T
    B, H = w.batch, w.kv_heads
    picks = [0, H - 1]
    dt = torch.bfloat16
    dev = torch.device("cuda")
    Kt = torch.empty(B, H, w.n, w.d, dtype=dt, device=dev)
    Vt = torch.empty_like(Kt)
    Qt = torch.empty(B, w.heads, T, w.d, dtype=dt, device=dev)
    host = {}
    for g in picks:
        ps = S.structure(w, 0, g)
        k, v = S.pair_kv(w, 0, g, ps=ps)
        q = S.pair_queries(w, 0, g, count=w.group * T, ps=ps, block=T0 // T).reshape(w.group, T, w.d)
        host[g] = (k, v, q)
    for g in range(H):
        k, v, q = host[g if g in host else picks[g % 2]]
        Kt[0, g].copy_(torch.from_numpy(k).to(dt))
        Vt[0, g].copy_(torch.from_numpy(v).to(dt))
        Qt[0, g * w.group:(g + 1) * w.group].copy_(torch.from_numpy(q).to(dt))
    R = np.stack([S.refs(w, g) for g in range(H)])
    geom = Z.make_geometry(B, H, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype, w.n, w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, T0)
    assert idx.n_tokens // w.chunk ** w.levels == 63
    select = dict(mode="topp", p=0.9)
    sel = P.select_struct(Z, select, 8192)
    assert idx.engine(sel, T) == "block" and idx.attn_engine(sel, T) == "union"
    bufs = idx.search(Qt, sel, qph=T)
    out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    torch.cuda.synchronize()
    assert int(bufs["status"].cpu()[0]) == 0
    from tree_structured_kv_amd.zha import stats_to_dicts
    rows = [g * w.group * T + hh * T + t for g in picks for hh in range(w.group)
            for t in np.random.default_rng(g).choice(T, size=16, replace=False)]
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    stats = stats_to_dicts(bufs["stats"].cpu())
    outs = out.float().cpu().numpy().reshape(w.heads * T, w.d)
    stable = 0
    for g in picks:
        k, v, q = host[g]
        tree = O.build(k[:T0].astype(np.float64), R[g].astype(np.float64), w.chunk, w.levels, w.sharpness)
        kd, vd = k.astype(np.float64), v.astype(np.float64)
        for wi in [r for r in rows if r // (w.group * T) == g]:
            hh, t = divmod(wi - g * w.group * T, T)
            qq = q[hh, t]
            sel_o, st_o = P.oracle_walk(tree, qq, select)
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, T0)
            stable += _check_walk(tree, qq, select, blocks[wi, :count[wi]], toks, stats[wi], sel_o, st_o,
                                  (g, hh, t))
            keys = np.concatenate([toks, np.arange(T0, T0 + t + 1)])
            ref, _ = O.attend(keys, qq.astype(np.float64), kd, vd, w.sharpness)
            assert P.out_ok(outs[wi], ref, w.dtype)[0], (g, hh, t)
    assert stable >= 0.3 * len(rows), (stable, len(rows))


# ---- the length sweep's deep trees --------------------------------------------------

@pytest.mark.parametrize("n,levels", [(1 << 20, None), (1 << 20, 9), (1 << 22, None)])
def test_sweep_geometry_deep_trees(Z, n, levels):
    """Nested keys of the length sweep (head_dim 64, chunk 4, 4 references,
    sharpness 20, top-p 0.9) at 1M and 4M tokens, with the depth rule (7 and
    8 levels: at most 64 top nodes) and with 9 levels at 1M (4 top nodes): 8
    one-place queries against the oracle walk and attention, on the
    per-walk engines the sweep's batch of queries runs."""
    d, c, R, s = 64, 4, 4, 20.0
    L = levels or Z.zha_depth_for(n, c, 64)
    assert levels or n // c ** L <= 64 < n // c ** (L - 1)
    K = S.nested_keys(n, d)
    V = S.nested_values(n, d)
    Q = S.nested_queries(n, d, 8)
    refs = S.nested_refs(R, d)
    tree = O.build(K.astype(np.float64), refs.astype(np.float64), c, L, s)
    w = replace(S.WORKLOADS[0], n=n, d=d, batch=1, kv_heads=1, group=8, chunk=c, refs=R, levels=L)
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).view(1, 1, n, d)
    Vt = torch.from_numpy(V).to(dev).view(1, 1, n, d)
    Qt = torch.from_numpy(Q).to(dev).view(1, 8, d)
    geom = Z.make_geometry(1, 1, 8, d, c, R, L, "f32", n, s)
    idx = Z.Index(geom, torch.from_numpy(refs).view(1, R, d))
    idx.build(Kt, n)
    select = dict(mode="topp", p=0.9)
    Kd, Vd = K.astype(np.float64), V.astype(np.float64)
    for engine in ("persistent", "level-sync"):
        blocks, count, stats, outs, status = _run(Z, idx, Qt, Kt, Vt, select, engine)
        assert status == 0
        stable = 0
        for h in range(8):
            q = Q[h]
            sel_o, st_o = P.oracle_walk(tree, q, select)
            assert st_o["steps"] == L
            toks = P.gpu_tokens(blocks[h], count[h], c, n)
            stable += _check_walk(tree, q, select, blocks[h, :count[h]], toks, stats[h], sel_o, st_o, (h, engine))
            ref, _ = O.attend(toks, q.astype(np.float64), Kd, Vd, s)
            assert P.out_ok(outs[0, h], ref, "f32")[0], (h, engine)
        assert stable >= 4, stable
