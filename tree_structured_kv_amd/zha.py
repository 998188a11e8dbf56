"""ctypes binding of libzha (include/zha.h), argument marshalling only.

Every step of the path runs in the HIP kernels of ``libzha.so``; this module
turns torch tensors into device pointers and the caller's current stream into
a ``hipStream_t``.  The library must have been built
(``python -m tree_structured_kv_amd.build``); importing this module without it
raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzha.so")

MAX_LEVELS = 12
MAX_STEPS = 12
TOPP, TOPK = 0, 1
F32, BF16 = 0, 1
FLAG_CAND_OVERFLOW, FLAG_SEL_OVERFLOW, FLAG_NONFINITE = 1, 2, 4
PATH_TIE_SELECT, PATH_LONG_LIST, PATH_LDS_SPILL = 1, 2, 4
ENGINE_AUTO, ENGINE_PERSISTENT, ENGINE_LEVEL_SYNC, ENGINE_UNION, ENGINE_BLOCK, ENGINE_FUSED = 0, 1, 2, 3, 4, 5
ENGINES = {"auto": ENGINE_AUTO, "persistent": ENGINE_PERSISTENT, "level-sync": ENGINE_LEVEL_SYNC,
           "union": ENGINE_UNION, "block": ENGINE_BLOCK, "fused": ENGINE_FUSED}
ATTN_AUTO, ATTN_PER_WALK, ATTN_UNION = 0, 1, 2
ATTN_ENGINES = {"auto": ATTN_AUTO, "per-walk": ATTN_PER_WALK, "union": ATTN_UNION}

STATUS = {0: "ZHA_OK", 1: "ZHA_ERR_ARG", 2: "ZHA_ERR_SHAPE", 3: "ZHA_ERR_ALIGN",
          4: "ZHA_ERR_CAPACITY", 5: "ZHA_ERR_WORKSPACE", 6: "ZHA_ERR_UNSUPPORTED",
          7: "ZHA_ERR_HIP"}


class Geometry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("num_refs", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("sharpness", ctypes.c_float),
                ("summary_dtype", ctypes.c_int32)]


class Select(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("p", ctypes.c_float),
                ("k", ctypes.c_int32 * MAX_STEPS), ("num_k", ctypes.c_int32),
                ("max_blocks_per_walk", ctypes.c_int32), ("max_candidates", ctypes.c_int32),
                ("engine", ctypes.c_int32), ("attn_engine", ctypes.c_int32)]


class TreeHandle(ctypes.Structure):
    _fields_ = [("geom", Geometry), ("n_tokens", ctypes.c_int64),
                ("tree_mem", ctypes.c_void_p), ("tree_bytes", ctypes.c_uint64),
                ("refs", ctypes.c_void_p),
                ("level_cap", ctypes.c_int64 * (MAX_LEVELS + 1)),
                ("key_off", ctypes.c_uint64 * (MAX_LEVELS + 1)),
                ("bias_off", ctypes.c_uint64 * (MAX_LEVELS + 1))]


class WalkStats(ctypes.Structure):
    _fields_ = [("scored", ctypes.c_int32 * MAX_STEPS), ("opened", ctypes.c_int32 * MAX_STEPS),
                ("steps", ctypes.c_int32), ("keys_read", ctypes.c_int32),
                ("blocks", ctypes.c_int32), ("unforced_scored", ctypes.c_int32),
                ("comparisons", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("paths", ctypes.c_uint32)]


STATS_WORDS = ctypes.sizeof(WalkStats) // 4   # int32 words per stats record

EXPORTS = ["zha_tree_bytes", "zha_depth_for", "zha_tree_init", "zha_build", "zha_append",
           "zha_search_workspace_bytes", "zha_search_engine", "zha_search", "zha_visited_words", "zha_attn_workspace_bytes", "zha_attn_engine",
           "zha_sparse_attn", "zha_sparse_attn_noalloc", "zha_forward_workspace_bytes", "zha_forward",
           "zha_dense_workspace_bytes", "zha_dense_topk_attn", "zha_dense_topp_attn", "zha_bw_probe",
           "zha_status_string"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tree_structured_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, u64, i64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32
    gp, sp, tp = ctypes.POINTER(Geometry), ctypes.POINTER(Select), ctypes.POINTER(TreeHandle)
    sig = {
        "zha_tree_bytes": (u64, [gp]),
        "zha_depth_for": (i32, [i64, i32, i64]),
        "zha_tree_init": (i32, [tp, gp, vp, u64, vp]),
        "zha_build": (i32, [tp, vp, i64, vp]),
        "zha_append": (i32, [tp, vp, i64, vp]),
        "zha_search_workspace_bytes": (u64, [tp, sp, i32]),
        "zha_search_engine": (i32, [tp, sp, i32]),
        "zha_attn_engine": (i32, [tp, sp, i32]),
        "zha_search": (i32, [tp, vp, i32, sp, vp, vp, vp, vp, vp, vp, u64, vp]),
        "zha_visited_words": (u64, [tp]),
        "zha_attn_workspace_bytes": (u64, [tp, sp, i32]),
        "zha_sparse_attn": (i32, [tp, vp, i32, vp, vp, sp, vp, vp, vp, vp, u64, vp]),
        "zha_sparse_attn_noalloc": (i32, [tp, vp, i32, vp, vp, sp, vp, vp, vp, vp]),
        "zha_forward_workspace_bytes": (u64, [tp, sp, i32]),
        "zha_forward": (i32, [tp, i64, vp, i32, vp, vp, sp, vp, vp, vp, vp, u64, vp]),
        "zha_dense_workspace_bytes": (u64, [tp, i32]),
        "zha_dense_topk_attn": (i32, [tp, vp, vp, vp, vp, i32, vp, vp, vp, u64, vp]),
        "zha_dense_topp_attn": (i32, [tp, vp, vp, vp, ctypes.c_float, i32, vp, vp, vp, vp, vp, u64, vp]),
        "zha_bw_probe": (i32, [vp, u64, vp, vp]),
        "zha_status_string": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


class ZhaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({lib.zha_status_string(code).decode()})")


def _check(code: int, what: str):
    if code != 0:
        raise ZhaError(code, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# The C ABI takes bare pointers and cannot see how large a buffer is, so the
# binding checks every tensor it passes: on the GPU, contiguous, of the dtype
# and element count the layout in include/zha.h fixes (ZhaError otherwise,
# before anything is enqueued).  Raw integer pointers are passed unchecked.
_ERR_ARG, _ERR_SHAPE = 1, 2


def _on_gpu(t) -> bool:
    return t.device.type == "cuda"


def _need(t, name, dtype=None, numel=None, min_numel=None, min_bytes=None):
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise ZhaError(_ERR_ARG, f"{name}: expected a torch tensor or a device pointer")
    if not _on_gpu(t):
        raise ZhaError(_ERR_ARG, f"{name}: tensor is on {t.device}, not on the GPU")
    if not t.is_contiguous():
        raise ZhaError(_ERR_SHAPE, f"{name}: tensor is not contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ZhaError(_ERR_SHAPE, f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ZhaError(_ERR_SHAPE, f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ZhaError(_ERR_SHAPE, f"{name}: {t.numel()} elements, expected at least {min_numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ZhaError(_ERR_SHAPE, f"{name}: {t.numel() * t.element_size()} bytes, expected at least {min_bytes}")


def _geom_of(t):
    g = t.geom
    dt = torch.bfloat16 if g.dtype == BF16 else torch.float32
    walks = g.batch * g.num_kv_heads * g.group_size
    return g, dt, walks


def _need_cache(t, k_cache, name):
    g, dt, _ = _geom_of(t)
    _need(k_cache, name, dt, numel=g.batch * g.num_kv_heads * g.max_tokens * g.head_dim)


def _need_rows(t, x, name, q_per_head):
    g, dt, walks = _geom_of(t)
    _need(x, name, dt, numel=walks * q_per_head * g.head_dim)


def _need_lists(t, sel, sel_blocks, sel_count, q_per_head):
    _, _, walks = _geom_of(t)
    W = walks * q_per_head
    _need(sel_blocks, "sel_blocks", torch.int32, min_numel=W * sel.max_blocks_per_walk)
    _need(sel_count, "sel_count", torch.int32, min_numel=W)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_geometry(batch, kv_heads, group, head_dim, chunk, refs, levels, dtype, max_tokens,
                  sharpness, summary="f32") -> Geometry:
    return Geometry(batch, kv_heads, group, head_dim, chunk, refs, levels,
                    BF16 if dtype in ("bf16", BF16, torch.bfloat16) else F32,
                    int(max_tokens), float(sharpness),
                    BF16 if summary in ("bf16", BF16, torch.bfloat16) else F32)


def make_select(mode="topp", p=0.9, k=(1,), max_blocks=1024, max_candidates=0, engine="auto",
                attn="auto") -> Select:
    s = Select()
    s.mode = TOPK if mode in ("topk", TOPK) else TOPP
    s.p = float(p)
    ks = list(k) if hasattr(k, "__len__") else [int(k)]
    s.num_k = len(ks)
    for i in range(MAX_STEPS):
        s.k[i] = int(ks[min(i, len(ks) - 1)])
    s.max_blocks_per_walk = int(max_blocks)
    s.max_candidates = int(max_candidates)
    s.engine = ENGINES[engine] if isinstance(engine, str) else int(engine)
    s.attn_engine = ATTN_ENGINES[attn] if isinstance(attn, str) else int(attn)
    return s


# ---- the C entry points, same names ------------------------------------------

def zha_tree_bytes(geom: Geometry) -> int:
    return int(lib.zha_tree_bytes(ctypes.byref(geom)))


def zha_depth_for(n_tokens: int, chunk: int, max_top: int = 64) -> int:
    return int(lib.zha_depth_for(int(n_tokens), int(chunk), int(max_top)))


def zha_tree_init(geom: Geometry, tree_mem, refs) -> TreeHandle:
    _need(tree_mem, "tree_mem", min_bytes=zha_tree_bytes(geom))
    _need(refs, "refs", torch.float32, numel=geom.num_kv_heads * geom.num_refs * geom.head_dim)
    t = TreeHandle()
    nbytes = tree_mem.numel() * tree_mem.element_size()
    _check(lib.zha_tree_init(ctypes.byref(t), ctypes.byref(geom), _ptr(tree_mem), nbytes, _ptr(refs)),
           "zha_tree_init")
    return t


def zha_build(t: TreeHandle, k_cache, n_tokens: int, stream=None):
    _need_cache(t, k_cache, "k_cache")
    _check(lib.zha_build(ctypes.byref(t), _ptr(k_cache), int(n_tokens), _stream(stream)), "zha_build")


def zha_append(t: TreeHandle, k_cache, n_new: int, stream=None):
    _need_cache(t, k_cache, "k_cache")
    _check(lib.zha_append(ctypes.byref(t), _ptr(k_cache), int(n_new), _stream(stream)), "zha_append")


def zha_search_workspace_bytes(t: TreeHandle, sel: Select, q_per_head: int = 1) -> int:
    return int(lib.zha_search_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), q_per_head))


def zha_search_engine(t: TreeHandle, sel: Select, q_per_head: int = 1) -> str | None:
    """Name of the engine zha_search runs for these arguments (None: invalid)."""
    e = int(lib.zha_search_engine(ctypes.byref(t), ctypes.byref(sel), q_per_head))
    return {v: k for k, v in ENGINES.items()}.get(e) if e > 0 else None


def zha_attn_engine(t: TreeHandle, sel: Select, q_per_head: int = 1) -> str | None:
    """Name of the attention path zha_sparse_attn runs (None: invalid)."""
    e = int(lib.zha_attn_engine(ctypes.byref(t), ctypes.byref(sel), q_per_head))
    return {v: k for k, v in ATTN_ENGINES.items()}.get(e) if e > 0 else None


def zha_search(t: TreeHandle, q, sel: Select, sel_blocks, sel_count, stats, status, ws,
               q_per_head: int = 1, stream=None, visited=None):
    _need_rows(t, q, "q", q_per_head)
    _need_lists(t, sel, sel_blocks, sel_count, q_per_head)
    W = _geom_of(t)[2] * q_per_head
    _need(stats, "stats", min_bytes=W * ctypes.sizeof(WalkStats))
    _need(status, "status", min_bytes=4)
    _need(visited, "visited", min_bytes=4 * zha_visited_words(t))
    _need(ws, "ws")
    wsb = ws.numel() * ws.element_size()
    _check(lib.zha_search(ctypes.byref(t), _ptr(q), q_per_head, ctypes.byref(sel), _ptr(sel_blocks),
                          _ptr(sel_count), _ptr(stats), _ptr(status), _ptr(visited), _ptr(ws), wsb,
                          _stream(stream)),
           "zha_search")


def zha_visited_words(t: TreeHandle) -> int:
    return int(lib.zha_visited_words(ctypes.byref(t)))


def zha_attn_workspace_bytes(t: TreeHandle, sel: Select, q_per_head: int = 1) -> int:
    return int(lib.zha_attn_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), q_per_head))


def zha_sparse_attn(t: TreeHandle, q, k_cache, v_cache, sel: Select, sel_blocks, sel_count, out, ws,
                    q_per_head: int = 1, stream=None):
    _need_rows(t, q, "q", q_per_head)
    _need_rows(t, out, "out", q_per_head)
    _need_cache(t, k_cache, "k_cache")
    _need_cache(t, v_cache, "v_cache")
    _need_lists(t, sel, sel_blocks, sel_count, q_per_head)
    _need(ws, "ws")
    wsb = ws.numel() * ws.element_size()
    _check(lib.zha_sparse_attn(ctypes.byref(t), _ptr(q), q_per_head, _ptr(k_cache), _ptr(v_cache),
                               ctypes.byref(sel), _ptr(sel_blocks), _ptr(sel_count), _ptr(out),
                               _ptr(ws), wsb, _stream(stream)),
           "zha_sparse_attn")


def zha_sparse_attn_noalloc(t: TreeHandle, q, k_cache, v_cache, sel: Select, sel_blocks, sel_count, out,
                            q_per_head: int = 1, stream=None):
    _need_rows(t, q, "q", q_per_head)
    _need_rows(t, out, "out", q_per_head)
    _need_cache(t, k_cache, "k_cache")
    _need_cache(t, v_cache, "v_cache")
    _need_lists(t, sel, sel_blocks, sel_count, q_per_head)
    _check(lib.zha_sparse_attn_noalloc(ctypes.byref(t), _ptr(q), q_per_head, _ptr(k_cache), _ptr(v_cache),
                                       ctypes.byref(sel), _ptr(sel_blocks), _ptr(sel_count), _ptr(out),
                                       _stream(stream)),
           "zha_sparse_attn_noalloc")


def zha_forward_workspace_bytes(t: TreeHandle, sel: Select, q_per_head: int = 1) -> int:
    return int(lib.zha_forward_workspace_bytes(ctypes.byref(t), ctypes.byref(sel), q_per_head))


def zha_forward(t: TreeHandle, n_new: int, q, k_cache, v_cache, sel: Select, out, stats, status, ws,
                q_per_head: int = 1, stream=None):
    _need_rows(t, q, "q", q_per_head)
    _need_rows(t, out, "out", q_per_head)
    _need_cache(t, k_cache, "k_cache")
    _need_cache(t, v_cache, "v_cache")
    _need(stats, "stats", min_bytes=_geom_of(t)[2] * q_per_head * ctypes.sizeof(WalkStats))
    _need(status, "status", min_bytes=4)
    _need(ws, "ws")
    wsb = ws.numel() * ws.element_size()
    _check(lib.zha_forward(ctypes.byref(t), int(n_new), _ptr(q), q_per_head, _ptr(k_cache),
                           _ptr(v_cache), ctypes.byref(sel), _ptr(out), _ptr(stats), _ptr(status),
                           _ptr(ws), wsb, _stream(stream)),
           "zha_forward")


def zha_dense_workspace_bytes(t: TreeHandle, max_budget: int) -> int:
    return int(lib.zha_dense_workspace_bytes(ctypes.byref(t), int(max_budget)))


def zha_dense_topk_attn(t: TreeHandle, q, k_cache, v_cache, budget, max_budget: int, out, ws,
                        sel_tokens=None, stream=None):
    walks = _geom_of(t)[2]
    _need_rows(t, q, "q", 1)
    _need_rows(t, out, "out", 1)
    _need_cache(t, k_cache, "k_cache")
    _need_cache(t, v_cache, "v_cache")
    _need(budget, "budget", torch.int32, min_numel=walks)
    _need(sel_tokens, "sel_tokens", torch.int32, min_numel=walks * int(max_budget))
    _need(ws, "ws")
    wsb = ws.numel() * ws.element_size()
    _check(lib.zha_dense_topk_attn(ctypes.byref(t), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(budget), int(max_budget), _ptr(out), _ptr(sel_tokens),
                                   _ptr(ws), wsb, _stream(stream)),
           "zha_dense_topk_attn")


def zha_dense_topp_attn(t: TreeHandle, q, k_cache, v_cache, p: float, max_budget: int, out, ws,
                        sel_tokens=None, sel_count=None, status=None, stream=None):
    walks = _geom_of(t)[2]
    _need_rows(t, q, "q", 1)
    _need_rows(t, out, "out", 1)
    _need_cache(t, k_cache, "k_cache")
    _need_cache(t, v_cache, "v_cache")
    _need(sel_tokens, "sel_tokens", torch.int32, min_numel=walks * int(max_budget))
    _need(sel_count, "sel_count", torch.int32, min_numel=walks)
    _need(status, "status", min_bytes=4)
    _need(ws, "ws")
    wsb = ws.numel() * ws.element_size()
    _check(lib.zha_dense_topp_attn(ctypes.byref(t), _ptr(q), _ptr(k_cache), _ptr(v_cache), float(p),
                                   int(max_budget), _ptr(out), _ptr(sel_tokens), _ptr(sel_count),
                                   _ptr(status), _ptr(ws), wsb, _stream(stream)),
           "zha_dense_topp_attn")


def zha_bw_probe(buf, sink, stream=None):
    _need(buf, "buf")
    _need(sink, "sink", torch.float32, min_numel=1)
    nbytes = buf.numel() * buf.element_size()
    _check(lib.zha_bw_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "zha_bw_probe")


# ---- a small convenience owner of the device buffers ----------------------------

def torch_dtype(geom: Geometry):
    return torch.bfloat16 if geom.dtype == BF16 else torch.float32


def stats_to_dicts(stats_words: torch.Tensor):
    """Decode a host int32 tensor [walks][STATS_WORDS] into dicts."""
    raw = stats_words.contiguous().cpu().numpy()
    out = []
    for row in raw:
        st = WalkStats.from_buffer_copy(row.tobytes())
        steps = st.steps
        out.append(dict(steps=steps, scored=list(st.scored)[:steps], opened=list(st.opened)[:steps],
                        keys_read=st.keys_read, blocks=st.blocks,
                        unforced_scored=st.unforced_scored, comparisons=st.comparisons,
                        flags=st.flags, paths=st.paths))
    return out


class Index:
    """Device buffers of one tree set plus the calls on them (no arithmetic)."""

    def __init__(self, geom: Geometry, refs: torch.Tensor, device="cuda"):
        self.geom = geom
        self.device = torch.device(device)
        self.refs = refs.to(device=self.device, dtype=torch.float32).contiguous()
        nbytes = zha_tree_bytes(geom)
        if nbytes == 0:
            raise ZhaError(6, "zha_tree_bytes")
        self.tree_mem = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.handle = zha_tree_init(geom, self.tree_mem, self.refs)

    @property
    def n_tokens(self) -> int:
        return int(self.handle.n_tokens)

    @property
    def walks(self) -> int:
        g = self.geom
        return g.batch * g.num_kv_heads * g.group_size

    def build(self, k_cache, n_tokens, stream=None):
        zha_build(self.handle, k_cache, n_tokens, stream)

    def append(self, k_cache, n_new, stream=None):
        zha_append(self.handle, k_cache, n_new, stream)

    def level(self, l: int):
        """(keys [B][H_kv][cap][R][D], biases [B][H_kv][cap][R]) views of level l."""
        g, h = self.geom, self.handle
        cap = h.level_cap[l]
        nk = g.batch * g.num_kv_heads * cap * g.num_refs * g.head_dim
        nb = g.batch * g.num_kv_heads * cap * g.num_refs
        if g.summary_dtype == BF16:
            k = self.tree_mem[h.key_off[l]: h.key_off[l] + 2 * nk].view(torch.bfloat16)
        else:
            k = self.tree_mem[h.key_off[l]: h.key_off[l] + 4 * nk].view(torch.float32)
        b = self.tree_mem[h.bias_off[l]: h.bias_off[l] + 4 * nb].view(torch.float32)
        return (k.view(g.batch, g.num_kv_heads, cap, g.num_refs, g.head_dim),
                b.view(g.batch, g.num_kv_heads, cap, g.num_refs))

    def search_buffers(self, sel: Select, qph: int = 1):
        W = self.walks * qph
        return dict(
            sel_blocks=torch.empty(W, sel.max_blocks_per_walk, dtype=torch.int32, device=self.device),
            sel_count=torch.empty(W, dtype=torch.int32, device=self.device),
            stats=torch.zeros(W, STATS_WORDS, dtype=torch.int32, device=self.device),
            status=torch.zeros(1, dtype=torch.int32, device=self.device),
            ws=torch.empty(max(zha_search_workspace_bytes(self.handle, sel, qph), 16), dtype=torch.uint8,
                           device=self.device),
        )

    def search(self, q, sel: Select, bufs=None, stream=None, visited=None, qph: int = 1):
        bufs = bufs or self.search_buffers(sel, qph)
        zha_search(self.handle, q, sel, bufs["sel_blocks"], bufs["sel_count"], bufs["stats"],
                   bufs["status"], bufs["ws"], qph, stream, visited)
        return bufs

    def engine(self, sel: Select, qph: int = 1):
        return zha_search_engine(self.handle, sel, qph)

    def attn_engine(self, sel: Select, qph: int = 1):
        return zha_attn_engine(self.handle, sel, qph)

    def visited_bitmap(self):
        """A zeroed bitmap for zha_search's `visited` output: [pairs][words]."""
        g = self.geom
        words = zha_visited_words(self.handle) // (g.batch * g.num_kv_heads)
        return torch.zeros(g.batch * g.num_kv_heads, words, dtype=torch.int32, device=self.device)

    def attn_workspace(self, sel: Select, qph: int = 1):
        return torch.empty(max(zha_attn_workspace_bytes(self.handle, sel, qph), 16), dtype=torch.uint8,
                           device=self.device)

    def sparse_attn(self, q, k_cache, v_cache, sel: Select, sel_blocks, sel_count, out=None, ws=None,
                    stream=None, qph: int = 1):
        if out is None:
            out = torch.empty_like(q)
        if ws is None:
            ws = self.attn_workspace(sel, qph)
        zha_sparse_attn(self.handle, q, k_cache, v_cache, sel, sel_blocks, sel_count, out, ws, qph, stream)
        return out

    def dense_workspace(self, max_budget: int):
        return torch.empty(max(zha_dense_workspace_bytes(self.handle, max_budget), 16), dtype=torch.uint8,
                           device=self.device)

    def dense_topk_attn(self, q, k_cache, v_cache, budget, max_budget, out=None, ws=None,
                        sel_tokens=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        if ws is None:
            ws = self.dense_workspace(max_budget)
        zha_dense_topk_attn(self.handle, q, k_cache, v_cache, budget, max_budget, out, ws,
                            sel_tokens, stream)
        return out

    def dense_topp_attn(self, q, k_cache, v_cache, p, max_budget, out=None, ws=None, sel_tokens=None,
                        sel_count=None, status=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        if ws is None:
            ws = self.dense_workspace(max_budget)
        zha_dense_topp_attn(self.handle, q, k_cache, v_cache, p, max_budget, out, ws, sel_tokens, sel_count,
                            status, stream)
        return out

    def forward_workspace(self, sel: Select, qph: int = 1):
        return torch.empty(max(zha_forward_workspace_bytes(self.handle, sel, qph), 16), dtype=torch.uint8,
                           device=self.device)

    def forward(self, n_new, q, k_cache, v_cache, sel: Select, out, stats, status, ws, stream=None,
                qph: int = 1):
        zha_forward(self.handle, n_new, q, k_cache, v_cache, sel, out, stats, status, ws, qph, stream)
        return out
