"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before any launch (no GPU needed: every call here
fails validation, so nothing reaches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(zha_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def Z():
    from tree_structured_kv_amd import zha
    return zha


def test_every_declared_symbol_is_exported(Z):
    names = _declared()
    assert "zha_build" in names and "zha_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(Z.lib, n), n
    assert sorted(Z.EXPORTS) == names


def test_struct_sizes_match_header(Z):
    # layouts the header fixes: 8 int32 + int64 + float + int32 = 48 bytes
    assert ctypes.sizeof(Z.Geometry) == 48
    assert ctypes.sizeof(Z.WalkStats) == 4 * (2 * 12 + 8)
    assert ctypes.sizeof(Z.Select) == 4 * (2 + 12 + 5)


def test_attention_workspace_and_engine_choice(Z):
    """The union attention arrays exist only where that path can run (bf16
    decode, at most 16 query heads per KV head); an unknown attention engine
    is rejected (workspace size 0)."""
    g = _geom(Z, group=16, max_tokens=8192)
    t = Z.TreeHandle()
    t.geom = g
    t.n_tokens = 0
    t.tree_mem = t.refs = 256          # never dereferenced by the sizing calls
    t.tree_bytes = Z.zha_tree_bytes(g)
    for lv in range(1, 4):
        t.level_cap[lv] = 8192 // 8 ** lv
    sel = Z.make_select("topp", 0.9, max_blocks=1024)
    dec = Z.lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), 1)
    pre = Z.lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), 4)
    assert dec > 0 and pre > 0
    # union arrays: 16-bit masks [pairs][n1cap], chunk bits, workgroup flags
    # and partials [pairs][workgroups][16][D+2]
    pairs, n1cap = 4, 8192 // 8
    nchunks = n1cap // 128
    wpg = min(4096 // pairs, nchunks)
    union = pairs * n1cap * 2 + pairs * 4 + pairs * wpg * 4 + pairs * wpg * 16 * 130 * 4
    g32 = _geom(Z, group=16, max_tokens=8192, dtype="f32")
    t.geom = g32
    t.tree_bytes = Z.zha_tree_bytes(g32)
    dec32 = Z.lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), 1)
    assert dec - dec32 >= union
    # prefill (4 query rows per head): groups of 16 of a pair's 16 x 4 walks,
    # one workgroup each, plus per walk the block's own partial, the sort key,
    # the sorted order and its inverse
    walks, ug = pairs * 16 * 4, pairs * (16 * 4 // 16)
    union_pf = (ug * n1cap * 2 + ug * 4 + ug * 4 + ug * 16 * 130 * 4
                + walks * 130 * 4 + walks * 8 + walks * 4 + walks * 4)
    pre32 = Z.lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), 4)
    assert pre - pre32 >= union_pf
    bad = Z.make_select("topp", 0.9, max_blocks=1024)
    bad.attn_engine = 7
    assert Z.lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(bad), 1) == 0
    assert Z.zha_attn_engine(t, bad, 1) is None
    # AUTO: union for bf16 decode with 16 heads per KV head, else per-walk
    t.geom = g
    t.tree_bytes = Z.zha_tree_bytes(g)
    assert Z.zha_attn_engine(t, sel, 1) == "union"
    assert Z.zha_attn_engine(t, sel, 4) == "union"          # bf16 prefill blocks: groups of 16 walks
    assert Z.zha_attn_engine(t, Z.make_select("topp", 0.9, max_blocks=1024, attn="per-walk"), 1) == "per-walk"
    g8 = _geom(Z, group=8, max_tokens=8192)
    t.geom = g8
    t.tree_bytes = Z.zha_tree_bytes(g8)
    assert Z.zha_attn_engine(t, sel, 1) == "per-walk"
    assert Z.zha_attn_engine(t, Z.make_select("topp", 0.9, max_blocks=1024, attn="union"), 1) == "union"
    t.geom = g32
    t.tree_bytes = Z.zha_tree_bytes(g32)
    assert Z.zha_attn_engine(t, Z.make_select("topp", 0.9, max_blocks=1024, attn="union"), 1) is None
    assert Z.zha_attn_engine(t, sel, 4) == "per-walk"       # fp32 prefill


def _geom(Z, **kw):
    base = dict(batch=2, kv_heads=2, group=2, head_dim=128, chunk=8, refs=4, levels=3,
                dtype="bf16", max_tokens=4096, sharpness=0.088)
    base.update(kw)
    return Z.make_geometry(**base)


def test_tree_bytes_formula(Z):
    g = _geom(Z)
    pairs = 4
    want = 0
    for l in (1, 2, 3):
        cap = 4096 // 8 ** l
        for nbytes in (pairs * cap * 4 * 128 * 4, pairs * cap * 4 * 4):
            want += (nbytes + 255) // 256 * 256
    assert Z.zha_tree_bytes(g) == want


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(chunk=3), dict(chunk=128), dict(refs=3),
                                dict(levels=0), dict(levels=13), dict(dtype=5),
                                dict(max_tokens=0), dict(batch=0), dict(sharpness=float("inf"))])
def test_bad_geometry_rejected(Z, kw):
    g = _geom(Z, **kw)
    if kw.get("dtype") == 5:
        g.dtype = 5
    assert Z.zha_tree_bytes(g) == 0
    t = Z.TreeHandle()
    rc = Z.lib.zha_tree_init(ctypes.byref(t), ctypes.byref(g), 1 << 20, 1 << 40, 1 << 20)
    assert rc in (1, 6)


def _handle(Z, **kw):
    g = _geom(Z, **kw)
    t = Z.TreeHandle()
    rc = Z.lib.zha_tree_init(ctypes.byref(t), ctypes.byref(g), 0x100000, Z.zha_tree_bytes(g), 0x200000)
    assert rc == 0
    return t


def test_tree_init_checks(Z):
    g = _geom(Z)
    t = Z.TreeHandle()
    need = Z.zha_tree_bytes(g)
    assert Z.lib.zha_tree_init(ctypes.byref(t), ctypes.byref(g), 0x100008, need, 0x200000) == 3
    assert Z.lib.zha_tree_init(ctypes.byref(t), ctypes.byref(g), 0x100000, need - 1, 0x200000) == 4
    assert Z.lib.zha_tree_init(ctypes.byref(t), ctypes.byref(g), None, need, 0x200000) == 1
    t = _handle(Z)
    assert t.n_tokens == 0
    assert list(t.level_cap)[1:4] == [512, 64, 8]


def test_build_append_argument_errors(Z):
    t = _handle(Z)
    assert Z.lib.zha_build(ctypes.byref(t), None, 16, None) == 1
    assert Z.lib.zha_build(ctypes.byref(t), 0x300004, 16, None) == 3
    assert Z.lib.zha_build(ctypes.byref(t), 0x300000, 4097, None) == 4
    assert Z.lib.zha_build(ctypes.byref(t), 0x300000, -1, None) == 4
    assert Z.lib.zha_append(ctypes.byref(t), 0x300000, -1, None) == 1
    assert Z.lib.zha_append(ctypes.byref(t), 0x300000, 4097, None) == 4
    assert t.n_tokens == 0


def test_search_argument_errors(Z):
    t = _handle(Z)
    sel = Z.make_select("topp", 0.9, max_blocks=64)
    ws = Z.zha_search_workspace_bytes(t, sel)
    assert ws > 0
    args = lambda **o: [ctypes.byref(t), o.get("q", 0x400000), o.get("qph", 1), ctypes.byref(o.get("sel", sel)),
                        o.get("blocks", 0x500000), o.get("count", 0x600000), None, o.get("status", 0x700000),
                        o.get("visited", None), o.get("ws", 0x800000), o.get("wsb", ws), None]
    assert Z.lib.zha_search(*args(q=None)) == 1
    assert Z.lib.zha_search(*args(q=0x400002)) == 3
    assert Z.lib.zha_search(*args(status=None)) == 1
    assert Z.lib.zha_search(*args(visited=0x900002)) == 3
    assert Z.lib.zha_search(*args(wsb=ws - 1)) == 5
    assert Z.lib.zha_search(*args(qph=0)) == 1
    assert Z.lib.zha_search(*args(qph=1 << 22)) == 6   # too many walks
    bad = Z.make_select("topk", k=(0,), max_blocks=64)
    assert Z.lib.zha_search(*args(sel=bad)) == 1
    bad = Z.make_select("topp", 0.9, max_blocks=0)
    assert Z.lib.zha_search(*args(sel=bad)) == 1
    bad = Z.make_select("topp", float("nan"), max_blocks=8)
    assert Z.lib.zha_search(*args(sel=bad)) == 1
    bad = Z.make_select("topp", 0.9, max_blocks=8, engine=7)
    assert Z.lib.zha_search(*args(sel=bad)) == 1


def test_visited_words(Z):
    t = _handle(Z)
    assert Z.zha_visited_words(t) == 4 * ((512 + 64 + 8 + 31) // 32)


def test_workspace_sizes_grow_with_capacity(Z):
    t = _handle(Z)
    s1 = Z.make_select("topp", 0.9, max_blocks=64, max_candidates=100)
    s2 = Z.make_select("topp", 0.9, max_blocks=64, max_candidates=1000)
    assert Z.zha_search_workspace_bytes(t, s2) > Z.zha_search_workspace_bytes(t, s1)
    f = Z.zha_forward_workspace_bytes(t, s1)
    assert f >= Z.zha_search_workspace_bytes(t, s1) + Z.zha_attn_workspace_bytes(t, s1)


def test_attn_forward_argument_errors(Z):
    t = _handle(Z)
    sel = Z.make_select("topp", 0.9, max_blocks=64)
    ws = Z.zha_attn_workspace_bytes(t, sel)
    base = [ctypes.byref(t), 0x400000, 1, 0x410000, 0x420000, ctypes.byref(sel), 0x430000, 0x440000,
            0x450000, 0x460000, ws, None]
    a = list(base); a[3] = None
    assert Z.lib.zha_sparse_attn(*a) == 1
    a = list(base); a[8] = 0x450008
    assert Z.lib.zha_sparse_attn(*a) == 3
    a = list(base); a[10] = ws - 1
    assert Z.lib.zha_sparse_attn(*a) == 5
    a = list(base); a[2] = 4097    # a prefill block past the cache capacity
    assert Z.lib.zha_sparse_attn(*a) == 4
    fw = Z.zha_forward_workspace_bytes(t, sel)
    assert Z.lib.zha_forward(ctypes.byref(t), 5000, 0x400000, 1, 0x410000, 0x420000, ctypes.byref(sel),
                             0x450000, None, 0x470000, 0x460000, fw, None) == 4
    assert Z.lib.zha_forward(ctypes.byref(t), 0, 0x400000, 1, 0x410000, 0x420000, ctypes.byref(sel),
                             0x450000, None, 0x470000, 0x460000, fw - 1, None) == 5


def test_dense_argument_errors(Z):
    t = _handle(Z)
    ws = Z.zha_dense_workspace_bytes(t, 128)
    assert ws > Z.zha_dense_workspace_bytes(t, 1) > 0
    assert Z.zha_dense_workspace_bytes(t, 0) == 0
    base = [ctypes.byref(t), 0x400000, 0x410000, 0x420000, 0x430000, 128, 0x440000, None, 0x450000, ws, None]
    a = list(base); a[4] = None
    assert Z.lib.zha_dense_topk_attn(*a) == 1
    a = list(base); a[5] = 0
    assert Z.lib.zha_dense_topk_attn(*a) == 1
    a = list(base); a[2] = 0x410004
    assert Z.lib.zha_dense_topk_attn(*a) == 3
    a = list(base); a[9] = ws - 1
    assert Z.lib.zha_dense_topk_attn(*a) == 5


def test_status_strings(Z):
    for code in range(8):
        assert Z.lib.zha_status_string(code)


def test_search_engine_resolution(Z):
    # explicit engines pass through; AUTO follows the shape; union needs decode and <= 16 heads
    small = _handle(Z)                                   # 2 x 2 x 2 heads: 8 walks
    topp = Z.make_select("topp", 0.9, max_blocks=64)
    topk = Z.make_select("topk", k=(4,), max_blocks=64)
    assert Z.zha_search_engine(small, topp) == "persistent"
    assert Z.zha_search_engine(small, topp, 16) == "block"           # 128 walks of a prefill block
    assert Z.zha_search_engine(small, topk, 16) == "block"
    for e in ("persistent", "level-sync", "union", "block"):
        s = Z.make_select("topp", 0.9, max_blocks=64, engine=e)
        assert Z.zha_search_engine(small, s) == e
    assert Z.zha_search_engine(small, Z.make_select("topp", 0.9, max_blocks=64, engine="union"), 4) is None
    wide = _handle(Z, batch=4, kv_heads=1, group=16)     # 64 decode walks, 16 heads per KV head
    assert Z.zha_search_engine(wide, topp) == "union"
    assert Z.zha_search_engine(wide, topk) == "union"
    assert Z.zha_search_engine(wide, topp, 2) == "block"
    big = _handle(Z, batch=4, kv_heads=1, group=32)
    assert Z.zha_search_engine(big, Z.make_select("topp", 0.9, max_blocks=64, engine="union")) is None
    eight = _handle(Z, batch=4, kv_heads=2, group=8)     # 64 decode walks, 8 heads per KV head
    assert Z.zha_search_engine(eight, topp) == "level-sync"          # with its dense top table
    assert Z.zha_search_engine(eight, topk) == "persistent"
    four = _handle(Z, batch=8, kv_heads=2, group=4)      # 64 walks, 4 heads per KV head
    assert Z.zha_search_engine(four, topp) == "level-sync"


def test_sweep_depth_policy_and_nested_inputs(Z):
    # the length sweep's depth rule (zha_depth_for): fewest levels leaving <= 64 top nodes (chunk 4)
    import sys
    sys.path.insert(0, ROOT)
    import bench
    import numpy as np
    from tree_structured_kv_amd import synth as S
    depth = [Z.zha_depth_for(n, 4, 64) for n in bench.SWEEP_NS]
    assert depth == [3, 4, 5, 6, 7, 8, 9]
    assert all(n // 4 ** L <= 64 < n // 4 ** (L - 1) for n, L in zip(bench.SWEEP_NS, depth))
    k1 = S.nested_keys(5000, 64)
    k2 = S.nested_keys(5000, 64)
    assert k1.dtype == np.float32 and k1.shape == (5000, 64) and np.array_equal(k1, k2)
    # keys of one 64-key segment are close, neighbouring segments less so
    seg = k1[:64]
    assert np.min(seg @ seg.mean(0)) > 0.9 * np.max(k1[64:128] @ seg.mean(0)) - 1.0
    assert S.nested_queries(5000, 64, 8).shape == (8, 64)


def test_binding_checks_tensors_before_any_call(Z):
    """The C ABI sees bare pointers only, so the binding checks every tensor
    it passes (device, contiguity, dtype, element count of the layout in
    zha.h) and raises ZhaError before the library is called.  No tensor here
    is on a GPU, so each call must stop at the first check it reaches."""
    import torch
    g = _geom(Z)
    t = Z.TreeHandle()
    t.geom = g
    sel = Z.make_select("topp", 0.9, max_blocks=64)
    walks = 2 * 2 * 2
    q = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(Z.ZhaError) as e:
        Z.zha_search(t, q, sel, None, None, None, None, None)
    assert "not on the GPU" in str(e.value)
    with pytest.raises(Z.ZhaError) as e:
        Z.zha_build(t, torch.zeros(1, dtype=torch.bfloat16), 16)
    assert e.value.code == 1
    with pytest.raises(Z.ZhaError):
        Z.zha_tree_init(g, torch.zeros(16, dtype=torch.uint8), torch.zeros(2, 4, 128))
    # the checks themselves, on host tensors taken for device ones
    Z_on_gpu = Z._on_gpu
    Z._on_gpu = lambda x: True
    try:
        Z._need_cache(t, torch.zeros(2, 2, 4096, 128, dtype=torch.bfloat16), "k_cache")
        for bad in (torch.zeros(2, 2, 4095, 128, dtype=torch.bfloat16),               # short cache
                    torch.zeros(2, 2, 4096, 128, dtype=torch.float32),                # wrong dtype
                    torch.zeros(2, 2, 128, 4096, dtype=torch.bfloat16).transpose(2, 3)):  # a view
            with pytest.raises(Z.ZhaError) as e:
                Z._need_cache(t, bad, "k_cache")
            assert e.value.code == 2
        Z._need_rows(t, torch.zeros(walks, 128, dtype=torch.bfloat16), "q", 1)
        with pytest.raises(Z.ZhaError):
            Z._need_rows(t, torch.zeros(walks, 128, dtype=torch.bfloat16), "q", 4)
        with pytest.raises(Z.ZhaError):
            Z._need_lists(t, sel, torch.zeros(walks * 63, dtype=torch.int32),
                          torch.zeros(walks, dtype=torch.int32), 1)
        with pytest.raises(Z.ZhaError):
            Z._need_lists(t, sel, torch.zeros(walks * 64, dtype=torch.int64),
                          torch.zeros(walks, dtype=torch.int32), 1)
        Z._need_lists(t, sel, torch.zeros(walks * 64, dtype=torch.int32), torch.zeros(walks, dtype=torch.int32), 1)
    finally:
        Z._on_gpu = Z_on_gpu


def test_depth_rule(Z):
    """[ZHA lesson] "Run a small tree yourself": levels are added until at most
    64 nodes remain on top (demo geometry: 4,096 keys, chunk 4, 3 levels, 64
    top nodes)."""
    assert Z.zha_depth_for(4096, 4, 64) == 3
    assert Z.zha_depth_for(4097, 4, 64) == 3
    assert Z.zha_depth_for(4096 * 4 + 3, 4, 64) == 4
    assert Z.zha_depth_for(1 << 20, 4, 64) == 7
    assert Z.zha_depth_for(1 << 22, 4, 64) == 8
    assert Z.zha_depth_for(1 << 24, 4, 64) == 9
    assert Z.zha_depth_for(65536, 16, 1) == 4
    assert Z.zha_depth_for(10, 4, 64) == 1
    assert Z.zha_depth_for(0, 4, 64) == 1
    assert Z.zha_depth_for(1 << 30, 2, 1) == 12         # capped at ZHA_MAX_LEVELS
    for bad in ((-1, 4, 64), (100, 3, 64), (100, 128, 64), (100, 4, 0)):
        assert Z.zha_depth_for(*bad) == -1
    for n in (1, 63, 64, 65, 4095, 300000, 5 << 20):
        L = Z.zha_depth_for(n, 4, 64)
        assert n // 4 ** L <= 64 and (L == 1 or n // 4 ** (L - 1) > 64)
