"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that span several
workgroups, levels and a ragged tail.  Contract: see tests/parity.py."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tree_structured_kv_amd import synth as S
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from tree_structured_kv_amd import zha
    return zha


def _case(name):
    W = S.WORKLOADS
    if name == "demo":          # the fp32 demo geometry, 64 query heads on one tree
        return replace(W[0], group=64), None
    if name == "demo-unstructured":
        return replace(W[0], group=64), "unstructured"
    if name == "ar1-small":     # ragged: 8192 + 5 tokens, 4 levels
        return replace(W[1].scaled(n=8197, batch=2), kv_heads=2, levels=4), None
    if name == "clustered-small":
        return replace(W[2].scaled(n=32768 + 77, batch=2), kv_heads=2, levels=5), None
    if name == "mixed-small":
        return replace(W[4].scaled(n=65536 + 3, batch=2), levels=4), None
    if name.endswith("-b8"):    # the same shapes on eight sequences (each its own seeds)
        w, v = _case(name[:-3] + "-small")
        return replace(w, batch=8), v
    if name == "wide32":        # chunk 32: two 16-key score tiles per level-1 node, 32 children per parent
        return replace(W[2].scaled(n=32 * 32 * 4 + 45, batch=1), kv_heads=2, chunk=32, levels=2), None
    if name == "wide64":        # chunk 64, the largest the library takes
        return replace(W[2].scaled(n=64 * 64 * 2 + 99, batch=1), kv_heads=2, chunk=64, levels=2), None
    if name == "mha-small":     # one query head per KV head
        return replace(W[1].scaled(n=4096 + 7, batch=2), kv_heads=4, group=1, levels=3), None
    raise KeyError(name)


CASES = ["demo", "demo-unstructured", "ar1-small", "clustered-small", "mixed-small", "mha-small"]

_cache = {}


def _setup(Z, name, summary="f32"):
    if (name, summary) in _cache:
        return _cache[(name, summary)]
    w, variant = _case(name)
    K, V, Q, R = P.make_inputs(w, unstructured=(variant == "unstructured"))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(dt).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(dt).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(dt).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                           w.n, w.sharpness, summary=summary)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, w.n)
    trees = {(b, g): P.oracle_tree(w, K, R, b, g, w.n, key_bf16=(summary == "bf16"))
             for b in range(w.batch) for g in range(w.kv_heads)}
    _cache[(name, summary)] = (w, K, V, Q, R, Kt, Vt, Qt, idx, trees)
    return _cache[(name, summary)]


@pytest.mark.parametrize("name", CASES)
def test_tree_records(Z, name):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    torch.cuda.synchronize()
    worst = 0.0
    for l in range(1, w.levels + 1):
        gk, gb = idx.level(l)
        gk = gk.cpu().numpy()
        gb = gb.cpu().numpy()
        for (b, g), tr in trees.items():
            ok, ob = tr.level(l)
            if ok.shape[0] == 0:
                continue
            nk = gk[b, g, : ok.shape[0]]
            nb = gb[b, g, : ok.shape[0]]
            ek = np.max(np.abs(nk - ok), axis=(1, 2)) / np.maximum(1.0, np.max(np.abs(ok), axis=(1, 2)))
            eb = np.max(np.abs(nb - ob), axis=1) / np.maximum(1.0, np.max(np.abs(ob), axis=1))
            worst = max(worst, float(ek.max()), float(eb.max()))
    assert worst <= P.TOL_TREE, worst


@pytest.mark.parametrize("name", ["demo", "ar1-small", "clustered-small", "mixed-small"])
def test_tree_records_bf16_summaries(Z, name):
    """bf16 node keys: each stored key is the bf16 rounding of its summary, so
    it equals the oracle's (fp64 summary, rounded) or differs by one bf16
    step where the fp32 and fp64 summaries straddle a rounding boundary, or
    by the fp32 bar (2e-5 of the row's largest key) where the summary
    cancels to a tiny value.  Above level 1 a parent also inherits its
    children's one-step differences (a convex combination of them: at most
    one bf16 step of the row's largest key).  The bias follows the stored
    key (tolerance: the key differences' share of s<key, rho> plus the fp32
    bar).  Nearly every key must match exactly."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name, "bf16")
    torch.cuda.synchronize()
    n_keys = n_exact = 0
    for l in range(1, w.levels + 1):
        gk, gb = idx.level(l)
        assert gk.dtype == torch.bfloat16
        gk = gk.float().cpu().numpy().astype(np.float64)
        gb = gb.cpu().numpy().astype(np.float64)
        for (b, g), tr in trees.items():
            ok, ob = tr.level(l)
            if ok.shape[0] == 0:
                continue
            nk = gk[b, g, : ok.shape[0]]
            nb = gb[b, g, : ok.shape[0]]
            rowmax = np.max(np.abs(ok), axis=2, keepdims=True)
            ulp = P.bf16_ulp(ok) + P.TOL_TREE * np.maximum(1.0, rowmax)
            if l > 1:
                ulp = ulp + P.bf16_ulp(rowmax)
            assert np.all(np.abs(nk - ok) <= ulp), l
            n_keys += nk.size
            n_exact += int(np.sum(nk == ok))
            rho = R[g].astype(np.float64)                               # [R][d]
            slack = w.sharpness * np.sum(ulp * np.abs(rho)[None], axis=2)  # [nodes][R]
            tol = P.TOL_TREE * np.maximum(1.0, np.abs(ob)) + slack
            assert np.all(np.abs(nb - ob) <= tol), l
    assert n_exact >= 0.999 * n_keys, (n_exact, n_keys)


@pytest.mark.parametrize("engine", ["level-sync", "union", "block"])
@pytest.mark.parametrize("sname", ["topp90", "topk4"])
@pytest.mark.parametrize("name", ["clustered-small", "mixed-small"])
def test_search_and_attention_bf16_summaries(Z, name, sname, engine):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name, "bf16")
    select = SELECTS[sname]
    sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
    _compare(w, K, V, Q, trees, select, bufs, out, min_stable=0.3)


@pytest.mark.parametrize("name", ["demo", "ar1-small", "mixed-small"])
def test_build_equals_appends(Z, name):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    other = Z.Index(idx.geom, torch.from_numpy(R))
    other.tree_mem.fill_(0x7F)
    rng = np.random.default_rng(5)
    done = 0
    steps = [1, 1, 3, w.chunk - 1, w.chunk, 1000]
    while done < w.n:
        m = steps.pop(0) if steps else int(rng.integers(1, 5000))
        m = min(m, w.n - done)
        other.append(Kt, m)
        done += m
    assert other.n_tokens == w.n
    torch.cuda.synchronize()
    worst = 0.0
    for l in range(1, w.levels + 1):
        a_k, a_b = idx.level(l)
        b_k, b_b = other.level(l)
        live = w.n // w.chunk ** l
        assert torch.equal(a_k[:, :, :live], b_k[:, :, :live]), l
        assert torch.equal(a_b[:, :, :live], b_b[:, :, :live]), l
        # the appended tree against the oracle directly, not only the build
        nk, nb = b_k.cpu().numpy(), b_b.cpu().numpy()
        for (b, g), tr in trees.items():
            ok, ob = tr.level(l)
            if ok.shape[0] == 0:
                continue
            ek = np.max(np.abs(nk[b, g, :ok.shape[0]] - ok), axis=(1, 2)) / np.maximum(1.0, np.max(np.abs(ok), axis=(1, 2)))
            eb = np.max(np.abs(nb[b, g, :ok.shape[0]] - ob), axis=1) / np.maximum(1.0, np.max(np.abs(ob), axis=1))
            worst = max(worst, float(ek.max()), float(eb.max()))
    assert worst <= P.TOL_TREE, worst


@pytest.mark.parametrize("name", ["wide32", "wide64"])
def test_wide_chunks(Z, name):
    """Chunks above 16 keys: the level-1 summary takes its scores over
    several 16-key matrix tiles and an upper node reloads its children's rows
    for the weighted sum.  Records against the oracle, appends bit-identical
    to the build, and AUTO's search and attention against the oracle."""
    test_tree_records(Z, name)
    test_build_equals_appends(Z, name)
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    for select in (dict(mode="topp", p=0.9), dict(mode="topk", k=(2,))):
        sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select)
        _compare(w, K, V, Q, trees, select, bufs, out, min_stable=0.0)


SELECTS = {
    "topp90": dict(mode="topp", p=0.9),
    "topp50": dict(mode="topp", p=0.5),
    "topk4": dict(mode="topk", k=(4,)),
    "topk-sched": dict(mode="topk", k=(2, 6, 12)),
    "greedy": dict(mode="topk", k=(1,)),
    "p0": dict(mode="topp", p=0.0),
}


def _run(Z, idx, Qt, Kt, Vt, select, max_blocks=None, max_candidates=0, engine="auto"):
    g = idx.geom
    if max_blocks is None:
        max_blocks = g.max_tokens // g.chunk
    sel = P.select_struct(Z, select, max_blocks, max_candidates, engine)
    bufs = idx.search(Qt, sel)
    out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"])
    torch.cuda.synchronize()
    return sel, bufs, out


def _check_walk(tree, q, select, gpu_blocks, toks, st, sel_o, st_o, where, full_stats=True):
    """Every walk is checked.  Where the oracle's cut gap exceeds GAP the
    GPU's selection and counts must equal the oracle's bit-exactly (returns
    1); otherwise the GPU's walk must be a sequence of valid cuts under the
    fp64 scores within VALID_TOL (tests/parity.py, check_walk_valid;
    returns 0)."""
    if st_o["gap"] > P.GAP:
        assert np.array_equal(toks, sel_o), where
        assert st["scored"] == st_o["scored"] and st["opened"] == st_o["opened"], where
        assert st["comparisons"] == st_o["comparisons"], where
        assert st["keys_read"] == st_o["keys_read"], where
        if full_stats:
            assert st["unforced_scored"] == st_o["unforced_scored"], where
        return 1
    ok, why = P.check_walk_valid(tree, q, select, np.asarray(gpu_blocks), st)
    assert ok, (where, why)
    return 0


def _compare(w, K, V, Q, trees, select, bufs, out, min_stable=0.3):
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    from tree_structured_kv_amd.zha import stats_to_dicts
    stats = stats_to_dicts(bufs["stats"].cpu())
    outs = out.float().cpu().numpy()
    assert int(bufs["status"].cpu()[0]) == 0
    stable = 0
    walks = 0
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            g = h // w.group
            wi = b * w.heads + h
            q = Q[b, h]
            sel_o, st_o = P.oracle_walk(trees[(b, g)], q, select)
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, w.n)
            st = stats[wi]
            walks += 1
            stable += _check_walk(trees[(b, g)], q, select, blocks[wi, :count[wi]], toks, st, sel_o, st_o,
                                  (b, h))
            ref, _ = O.attend(toks, q.astype(np.float64), K[b, g].astype(np.float64),
                              V[b, g].astype(np.float64), w.sharpness)
            ok, e = P.out_ok(outs[b, h], ref, w.dtype)
            worst = max(worst, e)
            assert ok, (b, h, e)
    assert stable >= min_stable * walks, (stable, walks)
    return stable, walks, worst


@pytest.mark.parametrize("engine", ["persistent", "level-sync", "union", "block"])
@pytest.mark.parametrize("sname", list(SELECTS))
@pytest.mark.parametrize("name", CASES)
def test_search_and_attention(Z, name, sname, engine):
    if engine == "union" and name.startswith("demo"):
        pytest.skip("the union engine takes at most 16 query heads per KV head (demo case: 64)")
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    select = SELECTS[sname]
    sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
    min_stable = 0.15 if name.startswith("demo") and select["mode"] == "topp" else 0.3
    _compare(w, K, V, Q, trees, select, bufs, out, min_stable=min_stable)


@pytest.mark.parametrize("engine", ["persistent", "level-sync", "union", "block"])
@pytest.mark.parametrize("name", ["ar1-b8", "clustered-b8", "mixed-b8"])
def test_search_and_attention_more_sequences(Z, name, engine):
    """Top-p 0.9 on eight sequences per KV head: the keys, values and queries
    of each (sequence, KV head) come from seeds of their own, so this is the
    main parity check over four times as many independent inputs."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    select = SELECTS["topp90"]
    sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
    _compare(w, K, V, Q, trees, select, bufs, out, min_stable=0.3)


@pytest.mark.parametrize("sname", ["topp90", "topk4", "p0"])
@pytest.mark.parametrize("name", ["ar1-small", "clustered-small", "mixed-small", "mha-small"])
def test_union_attention(Z, name, sname):
    """The union attention path (each pair's selected blocks read once, all
    heads at once) against the fp64 oracle on the same selections, and
    against the per-walk path."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    select = SELECTS[sname]
    g = idx.geom
    sel_u = P.select_struct(Z, select, g.max_tokens // g.chunk, attn="union")
    sel_p = P.select_struct(Z, select, g.max_tokens // g.chunk, attn="per-walk")
    bufs = idx.search(Qt, sel_u)
    out_u = idx.sparse_attn(Qt, Kt, Vt, sel_u, bufs["sel_blocks"], bufs["sel_count"])
    out_p = idx.sparse_attn(Qt, Kt, Vt, sel_p, bufs["sel_blocks"], bufs["sel_count"])
    torch.cuda.synchronize()
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    ou, op = out_u.float().cpu().numpy(), out_p.float().cpu().numpy()
    for b in range(w.batch):
        for h in range(w.heads):
            gi = h // w.group
            wi = b * w.heads + h
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, w.n)
            ref, _ = O.attend(toks, Q[b, h].astype(np.float64), K[b, gi].astype(np.float64),
                              V[b, gi].astype(np.float64), w.sharpness)
            for o in (ou[b, h], op[b, h]):
                ok, e = P.out_ok(o, ref, w.dtype)
                assert ok, (b, h, e)


def test_union_attention_given_lists(Z):
    """Hand-made block lists: random sorted sets (some with a repeated id,
    which the union path takes once), ids outside the live level (skipped),
    entries past sel_count (ignored), empty lists (then only the 3-key raw
    tail, which every walk attends)."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "mixed-small")
    g = idx.geom
    n1 = w.n // w.chunk
    assert w.n % w.chunk == 3          # a 3-key raw tail every walk attends
    cap = 64
    rng = np.random.default_rng(5)
    walks = w.batch * w.heads
    blocks = np.full((walks, cap), -1, np.int32)
    count = np.zeros(walks, np.int32)
    for wi in range(walks):
        k = int(rng.integers(0, cap + 1))
        ids = np.sort(rng.choice(n1 + 40, size=k, replace=False)).astype(np.int32)   # some past n1
        if wi % 5 == 1 and k > 4:                     # repeat an id (runs of three on one mask word)
            ids[2] = ids[1] = ids[3] if ids[3] % 2 == 1 else ids[1]
            ids = np.sort(ids)
        blocks[wi, :k] = ids
        count[wi] = k if wi % 7 else 0
    tb = torch.from_numpy(blocks).cuda()
    tc = torch.from_numpy(count).cuda()
    outs = {}
    for attn in ("union", "per-walk"):
        sel = P.select_struct(Z, SELECTS["topp90"], cap, attn=attn)
        outs[attn] = idx.sparse_attn(Qt, Kt, Vt, sel, tb, tc).float().cpu().numpy()
    torch.cuda.synchronize()
    for wi in range(walks):
        b, h = divmod(wi, w.heads)
        gi = h // w.group
        ids = blocks[wi, : count[wi]]
        ids = ids[(ids >= 0) & (ids < n1)]
        repeated = len(np.unique(ids)) < len(ids)
        ids = np.unique(ids)
        toks = np.sort(np.concatenate([(ids[:, None] * w.chunk + np.arange(w.chunk)).reshape(-1),
                                       np.arange(n1 * w.chunk, w.n)])).astype(np.int64)
        ref, _ = O.attend(toks, Q[b, h].astype(np.float64), K[b, gi].astype(np.float64),
                          V[b, gi].astype(np.float64), w.sharpness)
        for attn, o in outs.items():
            if repeated and attn == "per-walk":
                continue                      # the per-walk path attends a repeated block twice
            ok, e = P.out_ok(o.reshape(walks, -1)[wi], ref, w.dtype)
            assert ok, (attn, wi, e)


def test_union_attention_rejects_unsupported(Z):
    """fp32 caches and more than 16 query heads per KV head take the per-walk
    path only: an explicit union request is an error."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "demo")       # fp32, 64 heads per KV head
    sel = P.select_struct(Z, SELECTS["topp90"], idx.geom.max_tokens // idx.geom.chunk, attn="union")
    bufs = idx.search(Qt, P.select_struct(Z, SELECTS["topp90"], idx.geom.max_tokens // idx.geom.chunk))
    with pytest.raises(Z.ZhaError) as ei:
        idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"])
    assert ei.value.code == 6


@pytest.mark.parametrize("name", CASES)
def test_open_all_is_dense(Z, name):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    for select in (dict(mode="topp", p=1.0), dict(mode="topk", k=(10 ** 6,))):
        sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select)
        count = bufs["sel_count"].cpu().numpy()
        assert np.all(count == w.n // w.chunk)
        outs = out.float().cpu().numpy()
        for b in range(w.batch):
            for h in range(w.heads):
                g = h // w.group
                ref, _ = O.attend(np.arange(w.n), Q[b, h].astype(np.float64),
                                  K[b, g].astype(np.float64), V[b, g].astype(np.float64), w.sharpness)
                assert P.out_ok(outs[b, h], ref, w.dtype)[0], (b, h)


def test_widget_accounting_on_gpu(Z):
    """The page's widget trace (64->4, 16->9, 36->25: 100 keys, 564
    comparisons) and top-K 6 (24 keys, 472 comparisons), on the GPU."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "demo")
    from tree_structured_kv_amd.zha import stats_to_dicts
    for select, want in ((dict(mode="topk", k=(4, 9, 25)), (564, 100, [64, 16, 36], [4, 9, 25])),
                         (dict(mode="topk", k=(6,)), (472, 24, [64, 24, 24], [6, 6, 6]))):
        sel, bufs, out = _run(Z, idx, Qt, Kt, Vt, select)
        for st in stats_to_dicts(bufs["stats"].cpu()):
            assert (st["comparisons"], st["keys_read"], st["scored"], st["opened"]) == want


@pytest.mark.parametrize("engine", ["persistent", "level-sync", "union", "block"])
def test_deterministic(Z, engine):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "clustered-small")
    select = SELECTS["topp90"]
    _, b1, o1 = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
    _, b2, o2 = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
    for k in ("sel_blocks", "sel_count", "stats"):
        c1 = b1["sel_count"]
        if k == "sel_blocks":
            for wi in range(c1.numel()):
                n = int(c1[wi])
                assert torch.equal(b1[k][wi, :n], b2[k][wi, :n])
        else:
            assert torch.equal(b1[k], b2[k])
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("engine", ["union", "block"])
def test_matrix_engines_agree_on_stable_walks(Z, engine):
    """The union and block engines score with matrix-core tiles (another
    summation order): their selections equal the persistent engine's wherever
    the cut gap is not tiny, and their stats count each walk's own candidates."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "mixed-small")
    for select in (SELECTS["topp90"], SELECTS["topk4"]):
        _, b1, o1 = _run(Z, idx, Qt, Kt, Vt, select, engine="persistent")
        _, b2, o2 = _run(Z, idx, Qt, Kt, Vt, select, engine=engine)
        c1, c2 = b1["sel_count"].cpu(), b2["sel_count"].cpu()
        same = 0
        for wi in range(c1.numel()):
            n1, n2 = int(c1[wi]), int(c2[wi])
            if n1 == n2 and torch.equal(b1["sel_blocks"][wi, :n1], b2["sel_blocks"][wi, :n2]):
                same += 1
        assert same >= 0.9 * c1.numel()


def test_union_rejects_unsupported(Z):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "demo")     # 64 heads per KV head
    sel = P.select_struct(Z, SELECTS["topp90"], 1024, engine="union")
    with pytest.raises(Z.ZhaError):
        idx.search(Qt, sel)


def test_engines_agree(Z):
    """Both search engines give bit-identical selections, stats and outputs."""
    for name in ("clustered-small", "mixed-small", "ar1-small"):
        w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
        for select in (SELECTS["topp90"], SELECTS["topk4"]):
            _, b1, o1 = _run(Z, idx, Qt, Kt, Vt, select, engine="persistent")
            _, b2, o2 = _run(Z, idx, Qt, Kt, Vt, select, engine="level-sync")
            assert torch.equal(b1["sel_count"], b2["sel_count"])
            assert torch.equal(b1["stats"], b2["stats"])
            for wi in range(b1["sel_count"].numel()):
                n = int(b1["sel_count"][wi])
                assert torch.equal(b1["sel_blocks"][wi, :n], b2["sel_blocks"][wi, :n])
            assert torch.equal(o1, o2)


@pytest.mark.parametrize("engine", ["persistent", "level-sync", "union", "block"])
def test_overflow_is_flagged_and_deterministic(Z, engine):
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "mixed-small")
    select = SELECTS["topp90"]
    for kw, flag in ((dict(max_blocks=2), Z.FLAG_SEL_OVERFLOW), (dict(max_candidates=20), Z.FLAG_CAND_OVERFLOW)):
        _, b1, o1 = _run(Z, idx, Qt, Kt, Vt, select, engine=engine, **kw)
        _, b2, o2 = _run(Z, idx, Qt, Kt, Vt, select, engine=engine, **kw)
        assert int(b1["status"].cpu()[0]) & flag
        assert torch.equal(o1, o2)
        assert torch.equal(b1["sel_count"], b2["sel_count"])
        assert torch.all(torch.isfinite(o1.float()))


def test_forward_equals_parts(Z):
    """zha_forward(n_new) = zha_append(n_new) + zha_search + zha_sparse_attn."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, "ar1-small")
    select = SELECTS["topp90"]
    g = idx.geom
    sel = P.select_struct(Z, select, g.max_tokens // g.chunk)
    n0 = w.n - 37
    a = Z.Index(g, torch.from_numpy(R))
    a.build(Kt, n0)
    out_f = torch.empty_like(Qt)
    stats = torch.zeros(a.walks, Z.STATS_WORDS, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    a.forward(37, Qt, Kt, Vt, sel, out_f, stats, status, a.forward_workspace(sel))
    _, bufs, out_p = _run(Z, idx, Qt, Kt, Vt, select)
    assert a.n_tokens == w.n
    assert torch.equal(out_f, out_p)
    assert torch.equal(stats, bufs["stats"])


@pytest.mark.parametrize("name", ["demo", "clustered-small", "mixed-small"])
def test_dense_topk_baseline(Z, name):
    """The dense full-scan baseline: exact top-budget keys by logit (ties to
    the lower index) and attention over them, against fp64 logits."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    rng = np.random.default_rng(3)
    walks = w.batch * w.heads
    budget = rng.integers(1, min(w.n, 3000), size=walks).astype(np.int32)
    budget[0] = w.n          # everything
    budget[-1] = 1
    maxb = int(budget.max())
    bt = torch.from_numpy(budget).cuda()
    sel_t = torch.full((walks, maxb), -1, dtype=torch.int32, device="cuda")
    out = idx.dense_topk_attn(Qt, Kt, Vt, bt, maxb, sel_tokens=sel_t)
    torch.cuda.synchronize()
    sel_np = sel_t.cpu().numpy()
    outs = out.float().cpu().numpy()
    stable = 0
    for b in range(w.batch):
        for h in range(w.heads):
            wi = b * w.heads + h
            g = h // w.group
            k = int(budget[wi])
            got = sel_np[wi, :k].astype(np.int64)
            assert np.all(np.diff(got) > 0)
            lg = w.sharpness * (K[b, g].astype(np.float64) @ Q[b, h].astype(np.float64))
            order = np.lexsort((np.arange(w.n), -lg))
            want = np.sort(order[:k])
            gap = np.inf if k >= w.n else lg[order[k - 1]] - lg[order[k]]
            if gap > P.GAP:
                stable += 1
                assert np.array_equal(got, want), (b, h)
            ref, _ = O.attend(got, Q[b, h].astype(np.float64), K[b, g].astype(np.float64),
                              V[b, g].astype(np.float64), w.sharpness)
            assert P.out_ok(outs[b, h], ref, w.dtype)[0], (b, h)
    assert stable >= 0.5 * walks


@pytest.mark.parametrize("name", ["demo", "clustered-small", "mixed-small"])
@pytest.mark.parametrize("p", [0.5, 0.9, 1.0, 0.0])
def test_dense_topp_baseline(Z, name, p):
    """The dense baseline with top-p over keys: the smallest prefix of the
    keys by (logit descending, index ascending) whose softmax mass over all
    keys reaches p, against fp64 logits and masses.  Where the prefix is
    decided with room to spare (its mass without the last key at least 2e-5
    below p, with it at least 2e-5 above, and the boundary logits more than
    1e-4 apart) the key set must be the fp64 one; elsewhere it must be a
    valid top-p prefix within 1e-4.  p = 1 takes every key, p = 0 one."""
    w, K, V, Q, R, Kt, Vt, Qt, idx, trees = _setup(Z, name)
    walks = w.batch * w.heads
    maxb = w.n
    sel_t = torch.full((walks, maxb), -1, dtype=torch.int32, device="cuda")
    cnt_t = torch.zeros(walks, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = idx.dense_topp_attn(Qt, Kt, Vt, p, maxb, sel_tokens=sel_t, sel_count=cnt_t, status=status)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == 0
    sel_np, cnt = sel_t.cpu().numpy(), cnt_t.cpu().numpy()
    outs = out.float().cpu().numpy()
    stable = 0
    for b in range(w.batch):
        for h in range(w.heads):
            wi = b * w.heads + h
            g = h // w.group
            k = int(cnt[wi])
            got = sel_np[wi, :k].astype(np.int64)
            assert k >= 1 and np.all(np.diff(got) > 0), (b, h)
            lg = w.sharpness * (K[b, g].astype(np.float64) @ Q[b, h].astype(np.float64))
            pm = np.exp(lg - lg.max())
            pm /= pm.sum()
            order = np.lexsort((np.arange(w.n), -lg))
            cum = np.cumsum(pm[order])
            if p >= 1.0:
                assert k == w.n, (b, h)
            elif p <= 0.0:
                assert k == 1 and got[0] == order[0], (b, h)
            else:
                kw = int(np.searchsorted(cum, p)) + 1          # first prefix with mass >= p
                kw = min(kw, w.n)
                lo = cum[kw - 2] if kw >= 2 else 0.0
                gap_mass = min(p - lo, cum[kw - 1] - p)
                gap_lg = np.inf if kw >= w.n else lg[order[kw - 1]] - lg[order[kw]]
                # the GPU's logits are fp32 sums (about 1e-5 off), which
                # moves a prefix mass by about as much: a margin of 2e-5 in
                # mass decides the prefix
                if gap_mass > 2e-5 and gap_lg > P.GAP:
                    stable += 1
                    assert np.array_equal(got, np.sort(order[:kw])), (b, h)
                else:
                    # a valid prefix: nothing outside outranks a member by more
                    # than the tolerance, and its mass crosses p within it
                    inside = np.zeros(w.n, bool)
                    inside[got] = True
                    lo_in = lg[inside].min()
                    assert (~inside).sum() == 0 or lg[~inside].max() <= lo_in + P.VALID_TOL, (b, h)
                    mass = pm[inside].sum()
                    least = got[np.argmin(lg[got])]
                    assert mass >= p - P.VALID_TOL and mass - pm[least] < p + P.VALID_TOL, (b, h)
            ref, _ = O.attend(got, Q[b, h].astype(np.float64), K[b, g].astype(np.float64),
                              V[b, g].astype(np.float64), w.sharpness)
            assert P.out_ok(outs[b, h], ref, w.dtype)[0], (b, h)
    if 0.0 < p < 1.0:
        # every walk was checked above; with thousands of keys the key at the
        # crossing often carries less than 2e-4 of the mass, so a prefix
        # decided with 1e-4 to spare on both sides is the minority
        assert stable >= max(1, 0.05 * walks), stable


# ---- prefill blocks ------------------------------------------------------------

_pcache = {}


def _prefill_setup(Z, T=128):
    """A streamed cache (chunk 16, R 8, 3 levels) with a ragged prefix of
    T0 = 2*4096 + 300 tokens already in the tree and a block of T (128)
    queries per head at positions T0 .. T0+T-1 whose K/V rows are written."""
    if ("p", T) in _pcache:
        return _pcache[("p", T)]
    T0 = 2 * 4096 + 300
    w = replace(S.WORKLOADS[3].scaled(n=T0 + T, batch=1), kv_heads=2)
    K, V, _, R = P.make_inputs(w)
    Q = np.zeros((w.batch, w.heads, T, w.d), np.float32)
    for g in range(w.kv_heads):
        q = S.pair_queries(w, 0, g, count=w.group * T, block=T0 // w.block)
        Q[0, g * w.group:(g + 1) * w.group] = q.reshape(w.group, T, w.d)
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(torch.bfloat16).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(torch.bfloat16).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(torch.bfloat16).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                           w.n, w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, T0)
    trees = {(0, g): P.oracle_tree(w, K, R, 0, g, T0) for g in range(w.kv_heads)}
    _pcache[("p", T)] = (w, T0, T, K, V, Q, R, Kt, Vt, Qt, idx, trees)
    return _pcache[("p", T)]


@pytest.mark.parametrize("engine,T", [("persistent", 128), ("level-sync", 128), ("block", 128),
                                      ("level-sync", 160)])
@pytest.mark.parametrize("sname", ["topp90", "topk4", "open-all"])
def test_prefill_block(Z, sname, engine, T):
    """Prefill: every query of the block walks the tree of the tokens before
    the block, then attends its selection plus the block's keys up to itself.
    The level-synchronous scorer orders its tiles itself up to 4,096 walks
    (32 heads x 128 queries) and takes the tiles the cut kernels register
    beyond (x 160)."""
    w, T0, T, K, V, Q, R, Kt, Vt, Qt, idx, trees = _prefill_setup(Z, T)
    select = dict(mode="topp", p=1.0) if sname == "open-all" else SELECTS[sname]
    sel = P.select_struct(Z, select, T0 // w.chunk, engine=engine)
    bufs = idx.search(Qt, sel, qph=T)
    out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    torch.cuda.synchronize()
    from tree_structured_kv_amd.zha import stats_to_dicts
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    stats = stats_to_dicts(bufs["stats"].cpu())
    outs = out.float().cpu().numpy()
    assert int(bufs["status"].cpu()[0]) == 0
    stable = walks = 0
    rng = np.random.default_rng(0)
    for h in range(w.heads):
        g = h // w.group
        for t in rng.choice(T, size=16, replace=False):
            wi = h * T + t
            q = Q[0, h, t]
            sel_o, st_o = P.oracle_walk(trees[(0, g)], q, select)
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, T0)
            walks += 1
            stable += _check_walk(trees[(0, g)], q, select, blocks[wi, :count[wi]], toks, stats[wi], sel_o,
                                  st_o, (h, t))
            keys = np.concatenate([toks, np.arange(T0, T0 + t + 1)])
            ref, _ = O.attend(keys, q.astype(np.float64), K[0, g].astype(np.float64),
                              V[0, g].astype(np.float64), w.sharpness)
            ok, e = P.out_ok(outs[0, h, t], ref, w.dtype)
            assert ok, (h, t, e)
            if sname == "open-all":   # dense causal attention
                dense, _ = O.attend(np.arange(T0 + t + 1), q.astype(np.float64),
                                    K[0, g].astype(np.float64), V[0, g].astype(np.float64), w.sharpness)
                assert P.out_ok(outs[0, h, t], dense, w.dtype)[0]
    assert stable >= 0.3 * walks


@pytest.mark.parametrize("sname", ["topp90", "topk4", "open-all"])
@pytest.mark.parametrize("T", [128, 99])
def test_prefill_attention_paths(Z, sname, T):
    """Prefill blocks: the union attention path (groups of 16 walks of a
    pair in the order of their selection sketches; with T = 99 the pair's
    4 x 99 walks leave a ragged last group) and the per-walk path, each
    against oracle attention over the same selection plus the block's keys
    up to the query on sampled queries, and against each other on every
    query."""
    w, T0, _, K, V, Q, R, Kt, Vt, Qt, idx, trees = _prefill_setup(Z)
    Qb = Qt[:, :, :T].contiguous()
    select = dict(mode="topp", p=1.0) if sname == "open-all" else SELECTS[sname]
    sel_u = P.select_struct(Z, select, T0 // w.chunk, attn="union")
    sel_p = P.select_struct(Z, select, T0 // w.chunk, attn="per-walk")
    assert idx.attn_engine(sel_u, T) == "union"
    bufs = idx.search(Qb, sel_u, qph=T)
    out_u = idx.sparse_attn(Qb, Kt, Vt, sel_u, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    out_p = idx.sparse_attn(Qb, Kt, Vt, sel_p, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    torch.cuda.synchronize()
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    ou, op = out_u.float().cpu().numpy(), out_p.float().cpu().numpy()
    assert np.all(np.abs(ou - op) <= 1e-2 * np.maximum(1.0, np.abs(op)))
    rng = np.random.default_rng(1)
    for h in range(w.heads):
        g = h // w.group
        for t in list(rng.choice(T, size=8, replace=False)) + [T - 1]:
            wi = h * T + t
            q = Q[0, h, t]
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, T0)
            keys = np.concatenate([toks, np.arange(T0, T0 + t + 1)])
            ref, _ = O.attend(keys, q.astype(np.float64), K[0, g].astype(np.float64),
                              V[0, g].astype(np.float64), w.sharpness)
            for o in (ou[0, h, t], op[0, h, t]):
                ok, e = P.out_ok(o, ref, w.dtype)
                assert ok, (h, t, e)


def test_prefill_union_sort_segments(Z):
    """A prefill block whose pair holds more walks than one sort segment
    (4 heads x 4,100 queries = 16,400 > 16,384): the union path (sorted
    groups, two segments) against the per-walk path on every query and
    against the oracle on sampled queries of both segments, the ragged
    last group included."""
    T0, T = 1024 + 40, 4100
    w = replace(S.WORKLOADS[3].scaled(n=T0 + T, batch=1), kv_heads=1)
    K, V, _, R = P.make_inputs(w)
    q = S.pair_queries(w, 0, 0, count=w.group * T)
    Q = q.reshape(1, w.group, T, w.d).astype(np.float32)
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(torch.bfloat16).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(torch.bfloat16).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(torch.bfloat16).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                           w.n, w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, T0)
    select = SELECTS["topp90"]
    sel_u = P.select_struct(Z, select, T0 // w.chunk, attn="union")
    sel_p = P.select_struct(Z, select, T0 // w.chunk, attn="per-walk")
    assert idx.attn_engine(sel_u, T) == "union"
    bufs = idx.search(Qt, sel_u, qph=T)
    out_u = idx.sparse_attn(Qt, Kt, Vt, sel_u, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    out_p = idx.sparse_attn(Qt, Kt, Vt, sel_p, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    torch.cuda.synchronize()
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    ou, op = out_u.float().cpu().numpy(), out_p.float().cpu().numpy()
    assert np.all(np.isfinite(ou))
    assert np.all(np.abs(ou - op) <= 1e-2 * np.maximum(1.0, np.abs(op)))
    rng = np.random.default_rng(3)
    # walks 16,384 .. 16,399 (head 3, queries 4,084 ..) form the second segment
    picks = [(3, T - 1), (3, T - 16), (3, 4084), (0, 0), (1, 2049)]
    picks += [(int(h), int(t)) for h, t in zip(rng.integers(0, w.group, 6), rng.integers(0, T, 6))]
    for h, t in picks:
        wi = h * T + t
        toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, T0)
        keys = np.concatenate([toks, np.arange(T0, T0 + t + 1)])
        ref, _ = O.attend(keys, Q[0, h, t].astype(np.float64), K[0, 0].astype(np.float64),
                          V[0, 0].astype(np.float64), w.sharpness)
        ok, e = P.out_ok(ou[0, h, t], ref, w.dtype)
        assert ok, (h, t, e)


def test_prefill_forward_appends_after_search(Z):
    """zha_forward on a prefill block: search + attention on the tree before
    the block, then the block is appended (the tree equals a full build)."""
    w, T0, T, K, V, Q, R, Kt, Vt, Qt, idx, trees = _prefill_setup(Z)
    select = SELECTS["topp90"]
    sel = P.select_struct(Z, select, T0 // w.chunk)
    a = Z.Index(idx.geom, torch.from_numpy(R))
    a.build(Kt, T0)
    out_f = torch.empty_like(Qt)
    stats = torch.zeros(a.walks * T, Z.STATS_WORDS, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    a.forward(T, Qt, Kt, Vt, sel, out_f, stats, status, a.forward_workspace(sel, T), qph=T)
    bufs = idx.search(Qt, sel, qph=T)
    out_p = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"], qph=T)
    full = Z.Index(idx.geom, torch.from_numpy(R))
    full.build(Kt, T0 + T)
    torch.cuda.synchronize()
    assert a.n_tokens == T0 + T
    assert torch.equal(out_f, out_p)
    assert torch.equal(stats, bufs["stats"])
    for l in range(1, w.levels + 1):
        live = (T0 + T) // w.chunk ** l
        assert torch.equal(a.level(l)[0][:, :, :live], full.level(l)[0][:, :, :live])
        assert torch.equal(a.level(l)[1][:, :, :live], full.level(l)[1][:, :, :live])


# ---- short caches: empty, shorter than a chunk, top levels still empty ------------

ENGINES = ["persistent", "level-sync", "union", "block"]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("n_tok", [0, 3, 60, 100, 256])
def test_short_caches(Z, n_tok, engine):
    """Caches of 0 tokens (empty selection, zero output), fewer tokens than a
    chunk (everything is raw tail), and lengths whose top levels are still
    empty (the roots are parentless lower nodes): selections, stats and
    outputs against the oracle on every walk (chunk 4, 3 levels, 256 slots)."""
    w = replace(S.WORKLOADS[1], n=256, batch=1, kv_heads=2, group=4, chunk=4, refs=4, levels=3)
    K, V, Q, R = P.make_inputs(w)
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(torch.bfloat16).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(torch.bfloat16).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(torch.bfloat16).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                           w.n, w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, n_tok)
    for select in (SELECTS["topp90"], SELECTS["topk4"]):
        sel = P.select_struct(Z, select, w.n // w.chunk, engine=engine)
        bufs = idx.search(Qt, sel)
        out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"])
        torch.cuda.synchronize()
        assert int(bufs["status"].cpu()[0]) == 0
        blocks = bufs["sel_blocks"].cpu().numpy()
        count = bufs["sel_count"].cpu().numpy()
        from tree_structured_kv_amd.zha import stats_to_dicts
        stats = stats_to_dicts(bufs["stats"].cpu())
        outs = out.float().cpu().numpy()
        for h in range(w.heads):
            g = h // w.group
            tr = P.oracle_tree(w, K, R, 0, g, n_tok)
            q = Q[0, h]
            sel_o, st_o = P.oracle_walk(tr, q, select)
            toks = P.gpu_tokens(blocks[h], count[h], w.chunk, n_tok)
            _check_walk(tr, q, select, blocks[h, :count[h]], toks, stats[h], sel_o, st_o, (h, n_tok))
            ref, _ = O.attend(toks, q.astype(np.float64), K[0, g].astype(np.float64),
                              V[0, g].astype(np.float64), w.sharpness)
            if n_tok == 0:
                assert len(toks) == 0 and np.all(outs[0, h] == 0.0)
            assert P.out_ok(outs[0, h], ref, w.dtype)[0], h


# ---- full sizes: the bench's geometries and launch configuration, sampled walks ----

@pytest.mark.parametrize("wid,select", [(1, dict(mode="topp", p=0.9)),
                                        (2, dict(mode="topp", p=0.9)), (2, dict(mode="topk", k=(64,))),
                                        (4, dict(mode="topp", p=0.9))])
def test_full_size_sampled(Z, wid, select):
    """The decode workloads at full size (65,536, 262,144 and 1,048,576 keys,
    every sequence and KV head, AUTO engine as the bench runs it): the walks of
    two sampled (sequence, KV head) pairs (four at 64K, whose pairs hold only 4
    query heads) against the oracle walk on that pair's fp64 tree, and their
    outputs against oracle attention.  Other pairs hold copies of the sampled
    pairs' data, so the launch shapes are the real ones."""
    w = S.WORKLOADS[wid]
    B, H = w.batch, w.kv_heads
    picks = [(0, 0), (B - 1, H - 1)] + ([(3, 2), (5, 6)] if wid == 1 else [])
    dt = torch.bfloat16
    dev = torch.device("cuda")
    Kt = torch.empty(B, H, w.n, w.d, dtype=dt, device=dev)
    Vt = torch.empty_like(Kt)
    Qt = torch.empty(B, w.heads, w.d, dtype=dt, device=dev)
    host = {}
    for (b, g) in picks:
        ps = S.structure(w, b, g)
        k, v = S.pair_kv(w, b, g, ps=ps)
        q = S.pair_queries(w, b, g, ps=ps)
        host[(b, g)] = (k, v, q)
    kt = {bg: torch.from_numpy(host[bg][0]).to(dev).to(dt) for bg in picks}
    vt = {bg: torch.from_numpy(host[bg][1]).to(dev).to(dt) for bg in picks}
    qt = {bg: torch.from_numpy(host[bg][2]).to(dev).to(dt) for bg in picks}
    for b in range(B):
        for g in range(H):
            src = (b, g) if (b, g) in host else picks[(b * H + g) % len(picks)]
            Kt[b, g].copy_(kt[src])
            Vt[b, g].copy_(vt[src])
            Qt[b, g * w.group:(g + 1) * w.group].copy_(qt[src])
    R = np.stack([S.refs(w, g) for g in range(H)])
    geom = Z.make_geometry(B, H, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype, w.n, w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, w.n)
    sel = P.select_struct(Z, select, w.n // w.chunk)
    bufs = idx.search(Qt, sel)
    out = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"])
    torch.cuda.synchronize()
    assert int(bufs["status"].cpu()[0]) == 0
    from tree_structured_kv_amd.zha import stats_to_dicts
    blocks = bufs["sel_blocks"].cpu().numpy()
    count = bufs["sel_count"].cpu().numpy()
    stats = stats_to_dicts(bufs["stats"].cpu())
    outs = out.float().cpu().numpy()
    stable = walks = 0
    for (b, g) in picks:
        k, v, q = host[(b, g)]
        tr = O.build(k.astype(np.float64), R[g].astype(np.float64), w.chunk, w.levels, w.sharpness)
        for hh in range(w.group):
            h = g * w.group + hh
            wi = b * w.heads + h
            sel_o, st_o = P.oracle_walk(tr, q[hh], select)
            toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, w.n)
            walks += 1
            stable += _check_walk(tr, q[hh], select, blocks[wi, :count[wi]], toks, stats[wi], sel_o, st_o,
                                  (b, h))
            ref, _ = O.attend(toks, q[hh].astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                              w.sharpness)
            assert P.out_ok(outs[b, h], ref, w.dtype)[0], (b, h)
    # at 1M a third of the heads target 1 segment; those targeting 8 or 64
    # segments see near-flat scores whose cut gaps fall under 1e-4; AR(1)
    # keys (64K) are smooth, so neighbouring nodes score alike and most cuts
    # are that close too.  Those walks are checked for validity instead.
    assert stable >= {1: 1, 4: 0.25 * walks}.get(wid, 0.5 * walks), (stable, walks)
