"""Decode benchmark of tree-structured KV search on one MI355X.

One step = one decode token for every sequence of the batch through one
attention layer: zha_search (the tree walk of every query head) followed by
zha_sparse_attn (attention over the selected original keys), inputs resident
in HBM.  Prints one JSON line:

  value         queries/s = batch / step time (a query = one sequence's token,
                all its query heads)
  roofline      the search kernel (the dominant launch): algorithmic bytes per
                launch / its mean HIP-event duration, against 8 TB/s
  cpu_baseline  the fp64 oracle (search + attention) on a bounded sample of
                the same workload, on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/sec (search+sparse attn) at 256K/1M keys; % HBM roofline"
HBM_PEAK_GBS = 8000.0
ROTATIONS = 8

WORKLOADS = {
    # name: (workload id, selection)
    "decode-256K-topp": (2, dict(mode="topp", p=0.9)),
    "decode-256K-topk64": (2, dict(mode="topk", k=(64,))),
    "decode-1M-topp": (4, dict(mode="topp", p=0.9)),
    "decode-64K-topp": (1, dict(mode="topp", p=0.9)),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gen_inputs(w, threads):
    """Seeded inputs straight into device tensors, one pair at a time."""
    import torch
    from tree_structured_kv_amd import synth as S
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    K = torch.empty(w.batch, w.kv_heads, w.n, w.d, dtype=dt, device=dev)
    V = torch.empty_like(K)
    Q = torch.empty(ROTATIONS, w.batch, w.heads, w.d, dtype=dt, device=dev)

    def one(bg):
        b, g = bg
        ps = S.structure(w, b, g)
        k, v = S.pair_kv(w, b, g, ps=ps)
        qs = [S.pair_queries(w, b, g, rot=r, ps=ps) for r in range(ROTATIONS)]
        kt = torch.from_numpy(k).to(dt)
        vt = torch.from_numpy(v).to(dt)
        qt = torch.from_numpy(np.stack(qs)).to(dt)
        return b, g, kt, vt, qt

    pairs = [(b, g) for b in range(w.batch) for g in range(w.kv_heads)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for b, g, kt, vt, qt in ex.map(one, pairs):
            K[b, g].copy_(kt)
            V[b, g].copy_(vt)
            Q[:, b, g * w.group:(g + 1) * w.group].copy_(qt)
    R = torch.from_numpy(np.stack([S.refs(w, g) for g in range(w.kv_heads)]))
    torch.cuda.synchronize()
    return K, V, Q, R


def hbm_probe(Z, gib=4.0, reps=5):
    import torch
    buf = torch.empty(int(gib * (1 << 30)) // 16 * 16, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    Z.zha_bw_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(reps):
        e0.record()
        Z.zha_bw_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return best


def walk_bytes(w, stats_rows):
    """Algorithmic bytes of the walks: per unforced-scored candidate one node
    record R*(4d+4); per walk its query (read) ...; per selected key its K and
    V rows; per walk one output row."""
    e = 2 if w.dtype == "bf16" else 4
    nu = w.refs * (4 * w.d + 4)
    scored = sum(s["unforced_scored"] for s in stats_rows)
    keys = sum(s["keys_read"] for s in stats_rows)
    walks = len(stats_rows)
    search = nu * scored + walks * w.d * e
    attn = 2 * w.d * e * keys + walks * w.d * e * 2
    return search, attn, scored, keys


_PREPARED = {}


def prepare(w, threads):
    """Device inputs and the built tree of a workload (kept for reuse)."""
    import torch
    from tree_structured_kv_amd import zha as Zm
    if w.wid in _PREPARED:
        return _PREPARED[w.wid]
    t0 = time.time()
    K, V, Q, R = gen_inputs(w, threads)
    log(f"{w.name}: inputs generated in {time.time() - t0:.1f}s")
    geom = Zm.make_geometry(w.batch, w.kv_heads, w.group, w.d, w.chunk, w.refs, w.levels, w.dtype,
                            w.n, w.sharpness)
    idx = Zm.Index(geom, R)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    idx.build(K, w.n)            # first build also loads the kernels
    ev[0].record()
    idx.build(K, w.n)
    ev[1].record()
    torch.cuda.synchronize()
    _PREPARED[w.wid] = (K, V, Q, R, idx, ev[0].elapsed_time(ev[1]))
    return _PREPARED[w.wid]


def run_gpu(Z, w, select, steps, warmup, threads):
    import torch
    from tree_structured_kv_amd import zha as Zm
    K, V, Q, R, idx, build_ms = prepare(w, threads)
    sel = Zm.make_select(select["mode"], select.get("p", 0.9), select.get("k", (1,)),
                         max_blocks=w.n // w.chunk)
    bufs = idx.search_buffers(sel)
    out = torch.empty(w.batch, w.heads, w.d, dtype=K.dtype, device="cuda")
    aws = idx.attn_workspace(sel)

    def step(r, evs=None):
        q = Q[r % ROTATIONS]
        if evs:
            evs[0].record()
        idx.search(q, sel, bufs)
        if evs:
            evs[1].record()
        idx.sparse_attn(q, K, V, sel, bufs["sel_blocks"], bufs["sel_count"], out, aws)
        if evs:
            evs[2].record()

    # accounting pass (untimed): the walks of every query rotation
    per_rot = []
    for r in range(ROTATIONS):
        step(r)
        torch.cuda.synchronize()
        rows = Zm.stats_to_dicts(bufs["stats"].cpu())
        per_rot.append(rows)
        status = int(bufs["status"].cpu()[0])
    for r in range(warmup):
        step(r)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    search_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]

    # per-step bytes in the order the steps ran
    sb, ab, sc_, kr_ = [], [], [], []
    for i in range(steps):
        s, a, sc, kr = walk_bytes(w, per_rot[i % ROTATIONS])
        sb.append(s); ab.append(a); sc_.append(sc); kr_.append(kr)
    walks = w.batch * w.heads
    comps = [np.mean([s["comparisons"] for s in rows]) for rows in per_rot]
    keys = [np.mean([s["keys_read"] for s in rows]) for rows in per_rot]
    allw = [s for rows in per_rot for s in rows]
    dist = {}
    for k in ("unforced_scored", "keys_read"):
        v = np.array([s[k] for s in allw], dtype=np.float64)
        dist[k] = dict(mean=float(v.mean()), p50=float(np.percentile(v, 50)),
                       p90=float(np.percentile(v, 90)), max=float(v.max()))
    res = dict(
        workload=w, select=select, wall_s=wall, steps=steps,
        ms_per_step=wall / steps * 1e3,
        qps=w.batch * steps / wall,
        walks_per_s=walks * steps / wall,
        search_ms=float(np.mean(search_ms)), attn_ms=float(np.mean(attn_ms)),
        search_bytes=float(np.mean(sb)), attn_bytes=float(np.mean(ab)),
        build_ms=build_ms,
        comparisons_per_walk=float(np.mean(comps)),
        keys_read_per_walk=float(np.mean(keys)),
        status=status, dist=dist,
        idx=idx, K=K, V=V, Q=Q, R=R, per_rot=per_rot,
    )
    return res


def cpu_baseline(w, select, Q_host, seconds_budget=15.0):
    """The fp64 oracle (walk + attention) over the query heads of sampled
    sequences, threads over walks (ctypes drops the GIL)."""
    from oracle import oracle as O
    from tree_structured_kv_amd import synth as S
    cores = min(len(os.sched_getaffinity(0)), 16)
    t_build = time.time()
    b = 0
    trees, KV = {}, {}

    def build_pair(g):
        ps = S.structure(w, b, g)
        k, v = S.pair_kv(w, b, g, ps=ps)
        kd, vd = k.astype(np.float64), v.astype(np.float64)
        tr = O.build(kd, S.refs(w, g).astype(np.float64), w.chunk, w.levels, w.sharpness)
        return g, tr, kd, vd

    with ThreadPoolExecutor(max_workers=min(cores, w.kv_heads)) as ex:
        for g, tr, kd, vd in ex.map(build_pair, range(w.kv_heads)):
            trees[g], KV[g] = tr, (kd, vd)
    build_s = time.time() - t_build
    mode = O.TOPK if select["mode"] == "topk" else O.TOPP

    def one(h):
        g = h // w.group
        q = Q_host[h].astype(np.float64)
        sel, st = O.walk(trees[g], q, mode, p=select.get("p", 0.9), ksched=select.get("k", (1,)))
        O.attend(sel, q, KV[g][0], KV[g][1], w.sharpness)
        return st["comparisons"]

    # time whole queries (all heads of sequence 0) until the budget is spent
    reps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        while True:
            list(ex.map(one, range(w.heads)))
            reps += 1
            if time.perf_counter() - t0 > seconds_budget:
                break
    dt = time.perf_counter() - t0
    return dict(value=reps / dt, unit="queries/s", cores=cores, kind="oracle",
                sample=f"sequence 0 ({w.kv_heads} KV heads, {w.heads} query heads, rotation 0) "
                       f"of {w.name}, repeated {reps}x; oracle trees built untimed in {build_s:.1f}s",
                seconds=dt)


def summary(res, bw_ach):
    w = res["workload"]
    sel = res["select"]
    s_gbs = res["search_bytes"] / (res["search_ms"] * 1e-3) / 1e9
    step_bytes = res["search_bytes"] + res["attn_bytes"]
    step_gbs = step_bytes / (res["ms_per_step"] * 1e-3) / 1e9
    return dict(
        workload=w.name, select=sel,
        qps=res["qps"], walks_per_s=res["walks_per_s"], ms_per_step=res["ms_per_step"],
        search_ms=res["search_ms"], attn_ms=res["attn_ms"], build_ms=res["build_ms"],
        search_gbs=s_gbs, step_gbs=step_gbs,
        step_frac_of_peak=step_gbs / HBM_PEAK_GBS,
        step_frac_of_achievable=(step_gbs / bw_ach) if bw_ach else None,
        comparisons_per_walk=res["comparisons_per_walk"],
        keys_read_per_walk=res["keys_read_per_walk"], dense_keys=w.n,
        status=res["status"], per_walk=res["dist"],
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode-256K-topp", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default="decode-1M-topp,decode-256K-topk64",
                    help="comma-separated extra workloads reported under 'also'")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--threads", type=int, default=min(16, len(os.sched_getaffinity(0))))
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(each (sequence, KV head) pair is independent; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tree_structured_kv_amd import synth as S
    from tree_structured_kv_amd import zha as Zm
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    bw_ach = hbm_probe(Zm)
    log(f"achievable HBM read bandwidth {bw_ach:.0f} GB/s")

    wid, select = WORKLOADS[args.workload]
    w = S.WORKLOADS[wid]
    res = run_gpu(Zm, w, select, args.steps, args.warmup, args.threads)
    main_sum = summary(res, bw_ach)
    log(json.dumps(main_sum))
    Q0 = res["Q"][0, 0].float().cpu().numpy()

    also = []
    for name in [x for x in args.also.split(",") if x]:
        wid2, sel2 = WORKLOADS[name]
        r2 = run_gpu(Zm, S.WORKLOADS[wid2], sel2, max(5, args.steps // 3), 2, args.threads)
        s2 = summary(r2, bw_ach)
        log(json.dumps(s2))
        also.append(s2)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, select, Q0)
        log(f"cpu baseline {cpu}")

    ach = main_sum["search_gbs"]
    out = {
        "metric": METRIC,
        "value": main_sum["qps"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_sum["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} {args.workload}",
            "tokens": w.n, "batch": w.batch, "kv_heads": w.kv_heads, "group": w.group,
            "head_dim": w.d, "chunk": w.chunk, "refs": w.refs, "levels": w.levels,
            "kv_dtype": w.dtype, "select": select, "parallelism": "single-gpu",
        },
        "roofline": {
            "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "traffic": None,
            "kernel": "k_search_decode", "bytes_per_launch": res["search_bytes"],
            "launch_ms": main_sum["search_ms"], "achievable_gbs": bw_ach,
        },
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "step": {k: main_sum[k] for k in ("search_ms", "attn_ms", "build_ms", "step_gbs",
                                          "step_frac_of_peak", "step_frac_of_achievable",
                                          "comparisons_per_walk", "keys_read_per_walk",
                                          "dense_keys", "walks_per_s", "status")},
        "also": also,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
