"""zha_sparse_attn_noalloc -- attention with no workspace argument, its work
items and partial states in the library's fixed per-GPU scratch -- against
zha_sparse_attn on the per-walk path (the same kernels, so bit for bit), on
two calls in a row, the second with a smaller input than the first (the
scratch keeps the first call's contents), and against oracle attention over
the same selections."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import parity as P
from tree_structured_kv_amd import synth as S

pytestmark = pytest.mark.gpu


def _one(Z, w, qph=1):
    K, V, Q, R = P.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    Kt = torch.from_numpy(K).to(dev).to(dt).contiguous()
    Vt = torch.from_numpy(V).to(dev).to(dt).contiguous()
    Qt = torch.from_numpy(Q).to(dev).to(dt).contiguous()
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype, w.n,
                           w.sharpness)
    idx = Z.Index(geom, torch.from_numpy(R))
    idx.build(Kt, w.n)
    sel = Z.make_select("topp", 0.9, max_blocks=w.n // w.chunk, attn="per-walk")
    bufs = idx.search(Qt, sel)
    ref = idx.sparse_attn(Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"])
    out = torch.full_like(ref, float("nan"))
    Z.zha_sparse_attn_noalloc(idx.handle, Qt, Kt, Vt, sel, bufs["sel_blocks"], bufs["sel_count"], out)
    torch.cuda.synchronize()
    return w, K, V, Q, bufs, ref, out


def test_noalloc_equals_workspace_path_twice():
    assert torch.cuda.is_available()
    from tree_structured_kv_amd import zha as Z
    big = replace(S.WORKLOADS[1].scaled(n=8197, batch=2), kv_heads=2, levels=4)     # bf16, 16 walks
    small = replace(S.WORKLOADS[0].scaled(n=1024 + 3), group=4)                       # fp32, 4 walks
    for w in (big, small):
        w, K, V, Q, bufs, ref, out = _one(Z, w)
        assert torch.equal(out, ref), w.name
        blocks = bufs["sel_blocks"].cpu().numpy()
        count = bufs["sel_count"].cpu().numpy()
        outs = out.float().cpu().numpy()
        for b in range(w.batch):
            for h in range(w.heads):
                wi = b * w.heads + h
                g = h // w.group
                toks = P.gpu_tokens(blocks[wi], count[wi], w.chunk, w.n)
                o, _ = O.attend(toks, Q[b, h].astype(np.float64), K[b, g].astype(np.float64),
                                V[b, g].astype(np.float64), w.sharpness)
                assert P.out_ok(outs[b, h], o, w.dtype)[0], (w.name, b, h)


def test_noalloc_rejects_before_running():
    from tree_structured_kv_amd import zha as Z
    w = replace(S.WORKLOADS[1].scaled(n=8197, batch=2), kv_heads=2, levels=4)
    geom = Z.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype, w.n,
                           w.sharpness)
    idx = Z.Index(geom, torch.zeros(w.kv_heads, w.refs, w.d))
    dev = torch.device("cuda")
    Kt = torch.zeros(w.batch, w.kv_heads, w.n, w.d, dtype=torch.bfloat16, device=dev)
    Qt = torch.zeros(w.batch, w.heads, w.d, dtype=torch.bfloat16, device=dev)
    o = torch.zeros_like(Qt)
    union = Z.make_select("topp", 0.9, max_blocks=64, attn="union")
    sb = torch.zeros(w.batch * w.heads, 64, dtype=torch.int32, device=dev)
    sc = torch.zeros(w.batch * w.heads, dtype=torch.int32, device=dev)
    with pytest.raises(Z.ZhaError) as e:
        Z.zha_sparse_attn_noalloc(idx.handle, Qt, Kt, Kt, union, sb, sc, o)
    assert e.value.code == 6
    # 16 walks x 1M blocks of 8 keys: far more work items than the scratch holds
    huge = Z.make_select("topp", 0.9, max_blocks=1 << 20)
    with pytest.raises(Z.ZhaError) as e:
        Z.zha_sparse_attn_noalloc(idx.handle, Qt, Kt, Kt, huge, 1 << 12, 1 << 12, o)
    assert e.value.code == 5
