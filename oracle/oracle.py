"""fp64 CPU oracle for tree-structured KV search (ZHA) -- Python wrapper.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It loads the plain C
oracle (``zha_oracle.c``, built here with gcc) and shares no code with the GPU
library.  Every function follows the page "How does a tree of summaries search
a context? How ZHA works" ([ZHA lesson]); see ``zha_oracle.c`` for the section
each step restates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zha_oracle.c")
_LIB = os.path.join(_HERE, "libzha_oracle.so")

TOPP = 0
TOPK = 1
MAX_LEVELS = 12


class WalkStats(ctypes.Structure):
    _fields_ = [
        ("scored", ctypes.c_int32 * MAX_LEVELS),
        ("opened", ctypes.c_int32 * MAX_LEVELS),
        ("steps", ctypes.c_int32),
        ("forced", ctypes.c_int32 * MAX_LEVELS),
        ("keys_read", ctypes.c_int64),
        ("comparisons", ctypes.c_int64),
        ("unforced_scored", ctypes.c_int64),
        ("gap", ctypes.c_double),
    ]


def build_lib(force: bool = False) -> str:
    """Compile the C oracle with gcc (IEEE double, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build_lib()
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.ora_level_nodes.restype = ctypes.c_int64
        L.ora_level_nodes.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        L.ora_round_bf16.restype = ctypes.c_double
        L.ora_round_bf16.argtypes = [ctypes.c_double]
        L.ora_summarize.restype = None
        L.ora_summarize.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                    dp, dp, dp, dp, dp, ctypes.c_int]
        L.ora_node_score.restype = ctypes.c_double
        L.ora_node_score.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, dp]
        L.ora_build.restype = None
        L.ora_build.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_double, dp, dp, dp, dp, ctypes.c_int]
        L.ora_walk.restype = ctypes.c_int
        L.ora_walk.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_double, dp, dp, dp, ctypes.c_int,
                               ctypes.c_double, i32p, ctypes.c_int, i64p, i64p,
                               ctypes.POINTER(WalkStats)]
        L.ora_attend.restype = None
        L.ora_attend.argtypes = [ctypes.c_int64, i64p, ctypes.c_int, ctypes.c_double,
                                 dp, dp, dp, dp, dp]
        L.ora_mass_kept.restype = ctypes.c_double
        L.ora_mass_kept.argtypes = [ctypes.c_int64, ctypes.c_int64, i64p, ctypes.c_int,
                                    ctypes.c_double, dp, dp]
        _lib = L
    return _lib


def _dp(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def level_nodes(n: int, c: int, l: int) -> int:
    return int(lib().ora_level_nodes(n, c, l))


@dataclass
class Tree:
    """Levels 1..L of one (sequence, KV head) tree, in fp64."""
    n: int
    d: int
    c: int
    R: int
    L: int
    s: float
    k: np.ndarray      # [nodes][R][d], levels concatenated bottom-up
    b: np.ndarray      # [nodes][R]
    offsets: list      # offsets[l] = first node of level l (index 1..L), offsets[L+1] = total

    def level(self, l: int):
        a, z = self.offsets[l], self.offsets[l + 1]
        return self.k[a:z], self.b[a:z]

    def nodes_at(self, l: int) -> int:
        return self.offsets[l + 1] - self.offsets[l]


def round_bf16(x: float) -> float:
    """x rounded to the nearest bfloat16 value, ties to even (``ora_round_bf16``)."""
    return float(lib().ora_round_bf16(float(x)))


def summarize(child_k, child_b, refs, s: float, key_bf16: bool = False):
    """One node from children [c][R][d] / [c][R] (see ``ora_summarize``)."""
    ck, cb, rf = _f64(child_k), _f64(child_b), _f64(refs)
    c, R, d = ck.shape
    nk = np.zeros((R, d))
    nb = np.zeros(R)
    lib().ora_summarize(c, R, d, float(s), _dp(ck), _dp(cb), _dp(rf), _dp(nk), _dp(nb), int(key_bf16))
    return nk, nb


def node_score(node_k, node_b, q, s: float) -> float:
    nk, nb, qq = _f64(node_k), _f64(node_b), _f64(q)
    R, d = nk.shape
    return float(lib().ora_node_score(R, d, float(s), _dp(nk), _dp(nb), _dp(qq)))


def build(keys, refs, c: int, L: int, s: float, key_bf16: bool = False) -> Tree:
    keys, refs = _f64(keys), _f64(refs)
    n, d = keys.shape
    R = refs.shape[0]
    offs = [0, 0]
    for l in range(1, L + 1):
        offs.append(offs[-1] + level_nodes(n, c, l))
    total = offs[L + 1]
    tk = np.zeros((max(total, 1), R, d))
    tb = np.zeros((max(total, 1), R))
    lib().ora_build(n, d, c, R, L, float(s), _dp(keys), _dp(refs), _dp(tk), _dp(tb), int(key_bf16))
    return Tree(n, d, c, R, L, float(s), tk[:total], tb[:total], offs)


def walk(tree: Tree, q, mode: int = TOPP, p: float = 0.9, ksched=(1,)):
    """One walk; returns (selected token indices ascending, stats dict)."""
    qq = _f64(q)
    ks = np.ascontiguousarray(np.asarray(ksched, dtype=np.int32).reshape(-1))
    sel = np.zeros(max(tree.n, 1), dtype=np.int64)
    nsel = ctypes.c_int64(0)
    st = WalkStats()
    tk = tree.k if tree.k.shape[0] else np.zeros((1, tree.R, tree.d))
    tb = tree.b if tree.b.shape[0] else np.zeros((1, tree.R))
    rc = lib().ora_walk(tree.n, tree.d, tree.c, tree.R, tree.L, tree.s,
                        _dp(np.ascontiguousarray(tk)), _dp(np.ascontiguousarray(tb)),
                        _dp(qq), int(mode), float(p),
                        ks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(ks.size),
                        sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        ctypes.byref(nsel), ctypes.byref(st))
    if rc != 0:
        raise ValueError("ora_walk rejected its arguments")
    steps = st.steps
    stats = dict(
        steps=steps,
        scored=[st.scored[i] for i in range(steps)],
        opened=[st.opened[i] for i in range(steps)],
        forced=[st.forced[i] for i in range(steps)],
        keys_read=int(st.keys_read),
        comparisons=int(st.comparisons),
        unforced_scored=int(st.unforced_scored),
        gap=float(st.gap),
    )
    return sel[: nsel.value].copy(), stats


def attend(sel, q, K, V, s: float):
    """Softmax attention over the listed original keys; returns (out[d], lse)."""
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    qq, KK, VV = _f64(q), _f64(K), _f64(V)
    d = qq.shape[0]
    out = np.zeros(d)
    lse = ctypes.c_double(0.0)
    lib().ora_attend(sel.size, sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), d, float(s),
                     _dp(qq), _dp(KK), _dp(VV), _dp(out), ctypes.byref(lse))
    return out, lse.value


def mass_kept(sel, q, K, s: float) -> float:
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    qq, KK = _f64(q), _f64(K)
    n, d = KK.shape
    return float(lib().ora_mass_kept(n, sel.size, sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     d, float(s), _dp(qq), _dp(KK)))


def blocks_of(sel: np.ndarray, c: int, n: int):
    """Split a selected token list into (level-1 block ids, raw tail tokens)."""
    sel = np.asarray(sel, dtype=np.int64)
    full = c * (n // c)
    body = sel[sel < full]
    tail = sel[sel >= full]
    blocks = np.unique(body // c)
    return blocks, tail
