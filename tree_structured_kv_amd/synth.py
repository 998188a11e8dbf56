"""Seeded synthetic workloads for tree-structured KV search.

This module only draws random inputs (keys, values, queries, reference
queries) with the shapes and structure of the five workloads below.  It holds
none of the search method's arithmetic, so both the GPU path and the fp64
oracle can take their inputs from it.

Every draw is a PCG64 stream keyed by (0x5A4A, workload, sequence, kv-head,
stream id[, rotation]), so any single (sequence, kv-head) pair can be
regenerated on its own, in any process, bit for bit.  Values are drawn in
float32; bf16 workloads round them once, to nearest-even, and keep them as
float32 arrays that hold exactly bf16-representable values.

Workloads (geometry: N keys, head_dim d, batch B, KV heads x group, chunk c,
references R, summary levels L):
  0  tiny fp32 demo geometry: 64 aligned segments of 64 keys,
     key = 3 * unit centroid + N(0, 0.3^2); query = 3 * centroid + noise.
     Variant "unstructured": keys N(0, 1), query = a key + N(0, 0.3^2).
  1  bf16 decode, smooth keys: AR(1) latent z_t = 0.99 z_{t-1} +
     sqrt(1 - 0.99^2) eta_t, key = z_t + N(0, 0.5^2); a query is the
     1/sqrt(m)-scaled sum of the mean latents of m ~ U{1..8} random aligned
     64-token segments.
  2  bf16 decode at 256K, clustered keys: 1024 segments cut at 1023 distinct
     uniform points, key = 16 * unit centroid + N(0, 1); a query targets one
     segment: 16 * centroid + N(0, 1).
  3  as 2, streamed in blocks of 4096 tokens (chunk 16, 3 levels); a query
     of block k targets a segment that starts before the block.
  4  bf16 decode at 1M: 4096 segments as in 2, then each key is replaced with
     probability 0.05 by N(0, 1) * sqrt((16^2 + d) / d); walk (b, h) targets
     m = (1, 8, 64)[(H_q * b + h) mod 3] distinct segments:
     16 * (sum of m centroids) / sqrt(m) + N(0, 1).
Reference queries are N(0, 1) / sqrt(d), one set per KV head.  Values are
N(0, 1).  The sharpness is fp32(1 / sqrt(d)).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

ROOT_SEED = 0x5A4A
S_KEYS, S_VALUES, S_QUERIES, S_REFS, S_STRUCT = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    n: int              # tokens per sequence
    d: int              # head_dim
    batch: int
    kv_heads: int
    group: int          # query heads per KV head
    chunk: int
    refs: int
    levels: int
    dtype: str          # "f32" or "bf16" for K, V, Q and the output
    structure: str      # "segments", "ar1", "mixed"
    segments: int = 0
    amp: float = 0.0
    noise: float = 1.0
    random_frac: float = 0.0
    block: int = 0      # streaming block length (workload 3)
    select: dict = field(default_factory=dict)

    @property
    def heads(self) -> int:
        return self.kv_heads * self.group

    @property
    def sharpness(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def scaled(self, n: int | None = None, batch: int | None = None) -> "Workload":
        """Same structure at a different length and/or batch (segment count
        scales with the length so segment sizes stay the same)."""
        w = self
        if n is not None and n != w.n:
            seg = max(1, round(w.segments * n / w.n)) if w.segments else 0
            w = replace(w, n=n, segments=seg)
        if batch is not None:
            w = replace(w, batch=batch)
        return w


WORKLOADS = {
    0: Workload(0, "demo-4K-fp32", 4096, 64, 1, 1, 1, 4, 4, 3, "f32", "segments",
                segments=64, amp=3.0, noise=0.3, select=dict(mode="topp", p=0.9)),
    1: Workload(1, "decode-64K-bf16-ar1", 65536, 128, 8, 8, 4, 8, 4, 5, "bf16", "ar1",
                noise=0.5, select=dict(mode="topp", p=0.9)),
    2: Workload(2, "decode-256K-bf16-clustered", 262144, 128, 16, 4, 8, 8, 8, 6, "bf16",
                "segments", segments=1024, amp=16.0, noise=1.0,
                select=dict(mode="topp", p=0.9)),
    3: Workload(3, "prefill-256K-bf16-stream", 262144, 128, 1, 8, 4, 16, 8, 3, "bf16",
                "segments", segments=1024, amp=16.0, noise=1.0, block=4096,
                select=dict(mode="topp", p=0.9)),
    4: Workload(4, "decode-1M-bf16-mixed", 1048576, 128, 32, 1, 16, 16, 8, 5, "bf16",
                "mixed", segments=4096, amp=16.0, noise=1.0, random_frac=0.05,
                select=dict(mode="topp", p=0.9)),
}


def _rng(w: Workload, b: int, g: int, stream: int, *extra: int) -> np.random.Generator:
    seq = np.random.SeedSequence([ROOT_SEED, w.wid, b, g, stream, *extra])
    return np.random.Generator(np.random.PCG64(seq))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _cast(w: Workload, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16(x) if w.dtype == "bf16" else x


def _unit(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / np.maximum(np.linalg.norm(v, axis=-1, keepdims=True), 1e-30)


@dataclass
class PairStructure:
    """The hidden structure of one (sequence, KV head) cache."""
    seg_start: np.ndarray | None = None   # [S] first token of each segment
    centroids: np.ndarray | None = None   # [S][d] unit directions
    latent: np.ndarray | None = None      # [n][d] AR(1) latent (workload 1)


def structure(w: Workload, b: int, g: int) -> PairStructure:
    rng = _rng(w, b, g, S_STRUCT)
    if w.structure == "ar1":
        from scipy.signal import lfilter
        rho = 0.99
        eta = rng.standard_normal((w.n, w.d), dtype=np.float32).astype(np.float64)
        x = eta.copy()
        x[1:] *= math.sqrt(1.0 - rho * rho)
        z = lfilter([1.0], [1.0, -rho], x, axis=0)
        return PairStructure(latent=z)
    nseg = w.segments
    if w.wid == 0:
        starts = np.arange(nseg, dtype=np.int64) * (w.n // nseg)
    else:
        cuts = rng.choice(np.arange(1, w.n), size=nseg - 1, replace=False) if nseg > 1 else []
        starts = np.concatenate([[0], np.sort(np.asarray(cuts, dtype=np.int64))])
    cent = _unit(rng.standard_normal((nseg, w.d)))
    return PairStructure(seg_start=starts, centroids=cent)


def segment_of(ps: PairStructure, n: int) -> np.ndarray:
    idx = np.zeros(n, dtype=np.int64)
    idx[ps.seg_start[1:]] = 1
    return np.cumsum(idx)


def pair_kv(w: Workload, b: int, g: int, unstructured: bool = False,
            ps: PairStructure | None = None):
    """Keys and values of one pair as float32 [n][d] (bf16-exact for bf16)."""
    rk = _rng(w, b, g, S_KEYS)
    rv = _rng(w, b, g, S_VALUES)
    eps = rk.standard_normal((w.n, w.d), dtype=np.float32)
    if unstructured:
        K = eps
    elif w.structure == "ar1":
        ps = ps or structure(w, b, g)
        K = (ps.latent + w.noise * eps).astype(np.float32)
    else:
        ps = ps or structure(w, b, g)
        seg = segment_of(ps, w.n)
        cen = (w.amp * ps.centroids).astype(np.float32)
        K = cen[seg] + np.float32(w.noise) * eps
        if w.random_frac > 0.0:
            flip = rk.random(w.n) < w.random_frac
            scale = np.float32(math.sqrt((w.amp ** 2 + w.d) / w.d))
            K[flip] = rk.standard_normal((int(flip.sum()), w.d), dtype=np.float32) * scale
    V = rv.standard_normal((w.n, w.d), dtype=np.float32)
    return _cast(w, K), _cast(w, V)


def refs(w: Workload, g: int) -> np.ndarray:
    """Reference queries of KV head g: N(0, 1) / sqrt(d), float32 [R][d]."""
    r = _rng(w, 0, g, S_REFS)
    return (r.standard_normal((w.refs, w.d)) / math.sqrt(w.d)).astype(np.float32)


def pair_queries(w: Workload, b: int, g: int, rot: int = 0, count: int | None = None,
                 unstructured_keys: np.ndarray | None = None,
                 ps: PairStructure | None = None, block: int | None = None) -> np.ndarray:
    """Queries of the G heads of group g in sequence b, float32 [count][d].

    ``count`` defaults to the group size (one decode query per head).  For the
    streaming workload, ``block`` is the index of the query block."""
    count = w.group if count is None else count
    rq = _rng(w, b, g, S_QUERIES, rot)
    if unstructured_keys is not None:
        pick = rq.integers(0, unstructured_keys.shape[0], size=count)
        q = unstructured_keys[pick].astype(np.float64) + 0.3 * rq.standard_normal((count, w.d))
        return _cast(w, q)
    ps = ps or structure(w, b, g)
    if w.structure == "ar1":
        nblk = w.n // 64
        out = np.zeros((count, w.d))
        for i in range(count):
            m = int(rq.integers(1, 9))
            blocks = rq.integers(0, nblk, size=m)
            acc = np.zeros(w.d)
            for blk in blocks:
                acc += ps.latent[blk * 64:(blk + 1) * 64].mean(axis=0)
            out[i] = acc / math.sqrt(m)
        return _cast(w, out)
    nseg = ps.centroids.shape[0]
    if w.structure != "mixed":
        if block is not None:
            lim = max(1, int(np.searchsorted(ps.seg_start, w.block * block, side="left")))
        else:
            lim = nseg
        j = rq.integers(0, lim, size=count)
        out = w.amp * ps.centroids[j] + w.noise * rq.standard_normal((count, w.d))
        return _cast(w, out)
    out = np.zeros((count, w.d))
    for i in range(count):
        h = g * w.group + i
        m = min((1, 8, 64)[(w.heads * b + h) % 3], nseg)
        tg = rq.choice(nseg, size=m, replace=False)
        direction = ps.centroids[tg].sum(axis=0) / math.sqrt(m)
        out[i] = w.amp * direction + w.noise * rq.standard_normal(w.d)
    return _cast(w, out)


def batch_inputs(w: Workload, rot: int = 0, threads: int = 8, unstructured: bool = False,
                 rotations: int = 1):
    """All pairs: K, V float32 [B][H_kv][n][d]; Q float32 [rotations][B][H_q][d];
    refs float32 [H_kv][R][d]."""
    B, H = w.batch, w.kv_heads
    K = np.empty((B, H, w.n, w.d), dtype=np.float32)
    V = np.empty((B, H, w.n, w.d), dtype=np.float32)
    Q = np.empty((rotations, B, w.heads, w.d), dtype=np.float32)

    def one(bg):
        b, g = bg
        ps = None if unstructured else structure(w, b, g)
        k, v = pair_kv(w, b, g, unstructured=unstructured, ps=ps)
        K[b, g] = k
        V[b, g] = v
        for r in range(rotations):
            Q[r, b, g * w.group:(g + 1) * w.group] = pair_queries(
                w, b, g, rot=rot + r, unstructured_keys=k if unstructured else None, ps=ps)

    pairs = [(b, g) for b in range(B) for g in range(H)]
    if threads > 1 and len(pairs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, pairs))
    else:
        for bg in pairs:
            one(bg)
    R = np.stack([refs(w, g) for g in range(H)])
    return K, V, Q, R


# ---- length sweep: nested keys -------------------------------------------------
#
# A self-similar structure, for measuring how a walk's cost grows with the
# context: segments of `seg` keys share a unit centroid, and the centroids
# nest in tiers of 4 at every scale -- one direction at the top, and each
# tier's 4 children of a direction drawn around it (direction + 0.6 * a
# random unit vector, renormalised), until there is a centroid per segment.
# key = amp * segment centroid + noise * N(0, I/d); a query targets one
# segment ("asks about one place"): amp * centroid + noise * N(0, I/d).
# Stream ids 10.. keep these draws apart from the five workloads above.

S_NEST_KEYS, S_NEST_QUERIES, S_NEST_REFS = 10, 11, 12


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _nested_centroids(n, d, seed, seg):
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 100, seed, S_NEST_KEYS]))
    nseg = (n + seg - 1) // seg
    cent = _unit(rng.standard_normal((1, d)))
    while cent.shape[0] < nseg:
        kids = np.repeat(cent, 4, axis=0)
        cent = _unit(kids + 0.6 * _unit(rng.standard_normal(kids.shape)))
    return cent[:nseg], rng


def nested_keys(n, d, seed=0, seg=64, amp=1.0, noise=0.1):
    """float32 [n][d] keys of the length sweep (see above), drawn in float32
    in fixed 1M-row slices (so memory stays bounded at 16M keys)."""
    cent, rng = _nested_centroids(n, d, seed, seg)
    cent = (amp * cent).astype(np.float32)
    out = np.empty((n, d), np.float32)
    sl = 1 << 20
    scale = np.float32(noise / math.sqrt(d))
    for a in range(0, n, sl):
        b = min(n, a + sl)
        out[a:b] = cent[np.arange(a, b) // seg] + scale * rng.standard_normal((b - a, d), dtype=np.float32)
    return out


def nested_queries(n, d, count, seed=0, seg=64, amp=1.0, noise=0.1):
    """float32 [count][d] one-place queries for nested_keys(n, d, seed)."""
    cent, _ = _nested_centroids(n, d, seed, seg)
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 100, seed, S_NEST_QUERIES]))
    j = rng.integers(0, cent.shape[0], size=count)
    q = amp * cent[j] + noise * rng.standard_normal((count, d)) / math.sqrt(d)
    return q.astype(np.float32)


def nested_refs(r, d, seed=0):
    """float32 [r][d] reference queries N(0, 1)/sqrt(d) of the length sweep."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 100, seed, S_NEST_REFS]))
    return (rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float32)


def nested_values(n, d, seed=0):
    """float32 [n][d] values N(0, 1) for the length sweep's keys."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 100, seed, 13]))
    out = np.empty((n, d), np.float32)
    sl = 1 << 20
    for a in range(0, n, sl):
        b = min(n, a + sl)
        out[a:b] = rng.standard_normal((b - a, d), dtype=np.float32)
    return out


# ---- constructed caches for particular code paths -----------------------------
#
# Stream ids 20.. keep these draws apart from everything above.

S_TIED, S_FLATQ = 20, 21


def repeated_chunk_pair(w: Workload, g: int, seed: int = 0):
    """One (sequence, KV head) pair whose cache is a single chunk of w.chunk
    random keys repeated end to end (every node of a level then holds the
    same summary, so every score of a step ties), random values, and G
    random queries N(0, 4).  float32 arrays, bf16-exact for bf16 workloads:
    K, V [n][d], Q [G][d]."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 200, seed, g, S_TIED]))
    pat = _cast(w, rng.standard_normal((w.chunk, w.d)).astype(np.float32))
    K = np.tile(pat, (w.n // w.chunk + 1, 1))[: w.n]
    V = _cast(w, rng.standard_normal((w.n, w.d)).astype(np.float32))
    Q = _cast(w, (2.0 * rng.standard_normal((w.group, w.d))).astype(np.float32))
    return np.ascontiguousarray(K), V, Q


def small_queries(w: Workload, count: int, scale: float, seed: int = 0) -> np.ndarray:
    """float32 [count][d] queries N(0, scale^2) (bf16-exact for bf16): with a
    small scale every node scores about the same."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 200, seed, S_FLATQ]))
    return _cast(w, (scale * rng.standard_normal((count, w.d))).astype(np.float32))
