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


# ---- a pair that finishes inside the union engine before the hand-over ----------

@pytest.mark.parametrize("n", [256 * 80 + 14, 256 * 20 + 14])
@pytest.mark.parametrize("select", [dict(mode="topk", k=(1,)), dict(mode="topp", p=0.9)])
def test_union_pair_done_before_handover(Z, n, select):
    """Chunk 4, 4 levels, 8 heads per KV head: the union engine runs the
    first steps and the level-synchronous engine the last two.  On pair 0 one
    parentless level-1 chunk points along the heads' mean query, so every
    head opens only that root at the first step and the pair's walks end
    there: with 83 roots inside the grid-wide union cut, with 23 inside the
    fused first step.  The level-synchronous steps must leave those walks as
    they are; pair 1 (plain keys) walks to the bottom.  Every walk against
    the oracle."""
    w = replace(S.WORKLOADS[1], n=n, batch=1, kv_heads=2, group=8, chunk=4, refs=4, levels=4)
    K, V, Q, R = P.make_inputs(w)
    hot = (n // 4 - 2) * 4                     # the middle one of the three parentless chunks
    u = Q[0, :8].astype(np.float64).mean(0)
    u *= 8.0 * np.linalg.norm(K[0, 0], axis=1).mean() / np.linalg.norm(u)
    K[0, 0, hot:hot + 4] = S.round_bf16(np.repeat(u[None, :].astype(np.float32), 4, 0))
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, n)
    trees = [P.oracle_tree(w, K, R, 0, g, n) for g in range(2)]
    blocks, count, stats, outs, status = _run(Z, idx, Qt, Kt, Vt, select, "union")
    assert status == 0
    done_early = 0
    for h in range(w.heads):
        g = h // w.group
        q = Q[0, h]
        sel_o, st_o = P.oracle_walk(trees[g], q, select)
        if g == 0:
            assert st_o["steps"] == 1 and st_o["gap"] > P.GAP, (h, st_o["steps"])   # the case holds
            done_early += 1
        toks = P.gpu_tokens(blocks[h], count[h], w.chunk, n)
        _check_walk(trees[g], q, select, blocks[h, :count[h]], toks, stats[h], sel_o, st_o, (h, n))
        ref, _ = O.attend(toks, q.astype(np.float64), K[0, g].astype(np.float64),
                          V[0, g].astype(np.float64), w.sharpness)
        assert P.out_ok(outs[0, h], ref, w.dtype)[0], h
    assert done_early == 8


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


# ---- the decode step in one launch (zha_forward, ZHA_ENGINE_FUSED) ----------------

def _fwd_lists(Z, idx, sel, ws):
    """The selection lists zha_forward keeps at the start of its workspace:
    sel_blocks [walks][max_blocks] int32, then sel_count [walks] at the next
    256-byte boundary."""
    W = idx.walks
    nb = W * sel.max_blocks_per_walk * 4
    blocks = ws[:nb].view(torch.int32).view(W, sel.max_blocks_per_walk)
    off = (nb + 255) // 256 * 256
    count = ws[off:off + 4 * W].view(torch.int32)
    return blocks.cpu().numpy(), count.cpu().numpy()


@pytest.mark.parametrize("name,n0", [("ar1-small", 8192 - 3), ("demo", 4096 - 70), ("clustered-small", 32768 - 2)])
def test_fused_decode_steps(Z, name, n0):
    """Decode steps of one token each through the one-launch path: after
    every step the selections and stats equal the persistent engine's on a
    tree built over the same tokens (bit for bit), every walk is checked
    against the oracle walk (bit-exact where its cut is unique, else valid),
    the output against oracle attention over the selection, and after the
    last step the appended tree equals a full build bit for bit (the steps
    cross whole level-1 chunks and, at n = 8,192 / 4,096 / 32,768, complete
    a node on every level at once)."""
    from tests.test_gpu_parity import _case
    w, _ = _case(name)
    K, V, Q, R = P.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, n0)
    steps = min(w.n - n0, 12)
    select = dict(mode="topp", p=0.9)
    sel_f = P.select_struct(Z, select, w.n // w.chunk, engine="fused")
    sel_p = P.select_struct(Z, select, w.n // w.chunk, engine="persistent", attn="per-walk")
    ws = idx.forward_workspace(sel_f)
    out = torch.empty_like(Qt)
    stats = torch.zeros(idx.walks, Z.STATS_WORDS, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    from tree_structured_kv_amd.zha import stats_to_dicts
    for k in range(steps):
        idx.forward(1, Qt, Kt, Vt, sel_f, out, stats, status, ws)
        n = n0 + k + 1
        assert idx.n_tokens == n
        ref = Z.Index(idx.geom, torch.from_numpy(R))
        ref.build(Kt, n)
        bufs = ref.search(Qt, sel_p)
        torch.cuda.synchronize()
        assert int(status.cpu()[0]) == 0
        fb, fc = _fwd_lists(Z, idx, sel_f, ws)
        pb, pc = bufs["sel_blocks"].cpu().numpy(), bufs["sel_count"].cpu().numpy()
        assert np.array_equal(fc, pc), (k, n)
        for wi in range(idx.walks):
            assert np.array_equal(fb[wi, :fc[wi]], pb[wi, :pc[wi]]), (k, wi)
        assert torch.equal(stats, bufs["stats"]), k
        if k in (0, steps - 1) or n % w.chunk == 0:
            st = stats_to_dicts(stats.cpu())
            outs = out.float().cpu().numpy()
            trees = {(b, g): P.oracle_tree(w, K, R, b, g, n) for b in range(w.batch) for g in range(w.kv_heads)}
            for b in range(w.batch):
                for h in range(w.heads):
                    g = h // w.group
                    wi = b * w.heads + h
                    sel_o, st_o = P.oracle_walk(trees[(b, g)], Q[b, h], select)
                    toks = P.gpu_tokens(fb[wi], fc[wi], w.chunk, n)
                    _check_walk(trees[(b, g)], Q[b, h], select, fb[wi, :fc[wi]], toks, st[wi], sel_o, st_o, (k, b, h))
                    o, _ = O.attend(toks, Q[b, h].astype(np.float64), K[b, g, :n].astype(np.float64),
                                    V[b, g, :n].astype(np.float64), w.sharpness)
                    assert P.out_ok(outs[b, h], o, w.dtype)[0], (k, b, h)
    full = Z.Index(idx.geom, torch.from_numpy(R))
    full.build(Kt, idx.n_tokens)
    torch.cuda.synchronize()
    for l in range(1, w.levels + 1):
        live = idx.n_tokens // w.chunk ** l
        assert torch.equal(idx.level(l)[0][:, :, :live], full.level(l)[0][:, :, :live]), l
        assert torch.equal(idx.level(l)[1][:, :, :live], full.level(l)[1][:, :, :live]), l


def test_fused_rejects_what_it_does_not_run(Z):
    w, _ = (replace(S.WORKLOADS[1].scaled(n=8197, batch=2), kv_heads=2, levels=4), None)
    K, V, Q, R = P.make_inputs(w)
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, 4000)
    sel = P.select_struct(Z, dict(mode="topp", p=0.9), w.n // w.chunk, engine="fused")
    ws = idx.forward_workspace(sel)
    out = torch.empty_like(Qt)
    stats = torch.zeros(idx.walks, Z.STATS_WORDS, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(Z.ZhaError) as e:
        idx.forward(2, Qt, Kt, Vt, sel, out, stats, status, ws)           # more than one token
    assert e.value.code == 6
    with pytest.raises(Z.ZhaError) as e:
        idx.search(Qt, sel)                                                # zha_forward only
    assert e.value.code == 6
    assert idx.n_tokens == 4000 and idx.engine(sel) is None


# ---- the dense baseline's select on heavy ties ------------------------------------

@pytest.mark.parametrize("chunk", [4, 2])
def test_dense_select_heavy_ties(Z, chunk):
    """The dense indexer's exact top-budget select when the cache repeats a
    pattern of `chunk` keys: every head's logits take `chunk` values, each
    about n/chunk times, so the crossing bin holds thousands of equal keys --
    gathered into LDS (chunk 4: ~4,100 per value) or too many for it (chunk
    2: ~8,200, narrowed over the logits instead).  Ties go to the lower
    index; the set must equal the fp64 order exactly."""
    w = replace(S.WORKLOADS[1], n=16384 + 16 + 4 + 3, batch=1, kv_heads=2, group=8, chunk=chunk, refs=4,
                levels=3)
    K = np.empty((1, 2, w.n, w.d), np.float32)
    V = np.empty_like(K)
    Q = np.empty((1, w.heads, w.d), np.float32)
    for g in range(2):
        K[0, g], V[0, g], Q[0, g * w.group:(g + 1) * w.group] = S.repeated_chunk_pair(w, g, seed=chunk)
    R = np.stack([S.refs(w, g) for g in range(2)])
    Kt, Vt, Qt, idx = _device(Z, w, K, V, Q, R, w.n)
    walks = w.heads
    budget = np.array([1, 3, w.n // chunk - 1, w.n // chunk, w.n // chunk + 5, 2 * (w.n // chunk) + 1,
                       w.n - 1, w.n, 100, 4000, 8191, 8193, 12000, 5, 17, 9000], np.int32)[:walks]
    maxb = int(budget.max())
    sel_t = torch.full((walks, maxb), -1, dtype=torch.int32, device="cuda")
    out = idx.dense_topk_attn(Qt, Kt, Vt, torch.from_numpy(budget).cuda(), maxb, sel_tokens=sel_t)
    torch.cuda.synchronize()
    got_all = sel_t.cpu().numpy()
    outs = out.float().cpu().numpy()
    for h in range(walks):
        g = h // w.group
        k = int(budget[h])
        lg = w.sharpness * (K[0, g].astype(np.float64) @ Q[0, h].astype(np.float64))
        vals = np.unique(lg)
        assert len(vals) == chunk and np.min(np.diff(vals)) > 1e-3      # well separated values
        order = np.lexsort((np.arange(w.n), -lg))
        want = np.sort(order[:k])
        got = got_all[h, :k].astype(np.int64)
        assert np.array_equal(got, want), (h, k)
        ref, _ = O.attend(got, Q[0, h].astype(np.float64), K[0, g].astype(np.float64), V[0, g].astype(np.float64),
                          w.sharpness)
        assert P.out_ok(outs[0, h], ref, w.dtype)[0], h
