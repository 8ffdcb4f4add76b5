"""ctypes binding of libfsa.so (include/fsa.h).

Argument marshalling only: torch tensors are passed as raw device pointers and
the current torch stream as the HIP stream; every step of the computation
runs in the library's kernels.  There is no fallback: if libfsa.so is missing
or a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfsa.so")
# debug build whose kernels poison their LDS (see build.py); tests only
POISON_LIB_PATH = os.path.join(_PKG, "libfsa_poison.so")

FSA_OK, FSA_ERR_INVALID_ARG, FSA_ERR_UNSUPPORTED, FSA_ERR_WORKSPACE, FSA_ERR_HIP = range(5)

EXPORTED = (
    "fsa_last_error", "fsa_import_kv_plain", "fsa_append_kv", "fsa_build_page_meta", "fsa_meta_bytes",
    "fsa_quest_scores", "fsa_max_work_items", "fsa_select_pages",
    "fsa_sparse_decode_workspace_bytes", "fsa_sparse_decode_attn",
    "fsa_dense_decode_workspace_bytes", "fsa_dense_decode_attn", "fsa_validate_inputs", "fsa_describe_step",
    "fsa_append_decode_attn", "fsa_device_memory", "fsa_read_probe", "fsa_sparse_decode_attn_noalloc",
    "fsa_sparse_decode_attn_launches", "fsa_build_flags", "fsa_set_one_launch", "fsa_one_launch_stalls",
)


class FsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fsa status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pool_pages", ctypes.c_int32)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("prefix_tokens", ctypes.c_int32), ("window_tokens", ctypes.c_int32),
                ("budget_pages", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None
_opened = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfsa.so and declare its signatures (raises if it is not built).
    Later calls return the library in use (see ``using``)."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = _open(path)
        return _lib


@contextlib.contextmanager
def using(path: str):
    """Run the binding's calls on another build of the library (same ABI), e.g.
    the LDS-poison debug build, inside the ``with`` block."""
    global _lib
    load()
    with _lock:
        prev, _lib = _lib, _open(path)
    try:
        yield _lib
    finally:
        with _lock:
            _lib = prev


def _open(path: str) -> ctypes.CDLL:
    if path in _opened:
        return _opened[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m free_sparse_attention_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    D, C = ctypes.POINTER(Dims), LayerCfg
    sig = {
        "fsa_last_error": (ctypes.c_char_p, []),
        "fsa_import_kv_plain": (i32, [D, vp, vp, vp, vp, vp]),
        "fsa_append_kv": (i32, [D, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "fsa_build_page_meta": (i32, [D, vp, vp, vp, vp, vp]),
        "fsa_meta_bytes": (sz, [D]),
        "fsa_quest_scores": (i32, [D, C, i32, vp, vp, vp, vp, vp]),
        "fsa_max_work_items": (i32, [D, C, i32]),
        "fsa_select_pages": (i32, [D, C, i32, vp, vp, vp, vp, vp, vp, vp]),
        "fsa_sparse_decode_workspace_bytes": (sz, [D, C, i32]),
        "fsa_sparse_decode_attn": (i32, [D, C, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fsa_sparse_decode_attn_noalloc": (i32, [D, C, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "fsa_sparse_decode_attn_launches": (i32, [D, C, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, i32,
                                                  vp]),
        "fsa_dense_decode_workspace_bytes": (sz, [D, i32]),
        "fsa_dense_decode_attn": (i32, [D, f32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fsa_validate_inputs": (i32, [D, i32, i32, vp, vp, vp, vp, vp]),
        "fsa_describe_step": (i32, [D, C, i32, ctypes.POINTER(i32), i32]),
        "fsa_append_decode_attn": (i32, [D, i32, vp, vp, vp, vp, C, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]),
        "fsa_device_memory": (i32, [ctypes.POINTER(i32), i32]),
        "fsa_read_probe": (i32, [vp, sz, vp, vp]),
        "fsa_build_flags": (i32, []),
        "fsa_set_one_launch": (i32, [i32]),
        "fsa_one_launch_stalls": (i32, [ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _opened[path] = L
    return L


def _check(status: int) -> None:
    if status != FSA_OK:
        raise FsaError(status, load().fsa_last_error().decode())


def _p(t: torch.Tensor | None, name: str, dtype_size: int | None = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype_size is not None and t.element_size() != dtype_size:
        raise ValueError(f"{name}: element size {t.element_size()}, expected {dtype_size}")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return _p(t, name)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dims(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, num_pool_pages, page_size=16) -> Dims:
    return Dims(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_pool_pages)


def cfg(prefix_tokens, window_tokens, budget_pages) -> LayerCfg:
    return LayerCfg(prefix_tokens, window_tokens, budget_pages)


def import_kv_plain(d: Dims, k_plain, v_plain, k_cache, v_cache, stream=None):
    _check(load().fsa_import_kv_plain(ctypes.byref(d), _p(k_plain, "k_plain", 2), _p(v_plain, "v_plain", 2),
                                      _p(k_cache, "k_cache", 2), _p(v_cache, "v_cache", 2), _stream(stream)))


def append_kv(d: Dims, n_new, k_new, v_new, page_table, seq_lens, seq_lens_out, k_cache, v_cache, meta,
              stream=None):
    _check(load().fsa_append_kv(ctypes.byref(d), int(n_new), _p(k_new, "k_new", 2), _p(v_new, "v_new", 2),
                                _i32(page_table, "page_table"), _i32(seq_lens, "seq_lens"),
                                _i32(seq_lens_out, "seq_lens_out"), _p(k_cache, "k_cache", 2),
                                _p(v_cache, "v_cache", 2), _p(meta, "meta", 2), _stream(stream)))


def build_page_meta(d: Dims, k_cache, page_table, seq_lens, meta, stream=None):
    _check(load().fsa_build_page_meta(ctypes.byref(d), _p(k_cache, "k_cache", 2), _i32(page_table, "page_table"),
                                      _i32(seq_lens, "seq_lens"), _p(meta, "meta", 2), _stream(stream)))


def meta_bytes(d: Dims) -> int:
    n = load().fsa_meta_bytes(ctypes.byref(d))
    if n == 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    return n


def quest_scores(d: Dims, c: LayerCfg, max_seq_len, q, meta, seq_lens, scores, stream=None):
    _check(load().fsa_quest_scores(ctypes.byref(d), c, int(max_seq_len), _p(q, "q", 2), _p(meta, "meta", 2),
                                   _i32(seq_lens, "seq_lens"), _p(scores, "scores", 4), _stream(stream)))


STEP_INFO = ("plan", "replicas", "per_replica", "xcd_grouped", "prefetch", "pw_workgroups", "slots", "select_cols",
             "pw_items_per_wave", "one_launch", "score_tasks")
PLANS = {0: "dense", 1: "wide", 2: "narrow"}


def describe_step(d: Dims, c: LayerCfg, max_seq_len) -> dict:
    """How the sparse step of these shapes runs on the current device (host only)."""
    buf = (ctypes.c_int32 * len(STEP_INFO))()
    n = load().fsa_describe_step(ctypes.byref(d), c, int(max_seq_len), buf, len(STEP_INFO))
    if n < 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    r = {k: int(buf[i]) for i, k in enumerate(STEP_INFO[:n])}
    r["plan"] = PLANS[r["plan"]]
    return r


MEMORY_INFO = ("memory_clock_khz", "memory_bus_width_bits", "compute_units", "l2_bytes")


def device_memory() -> dict:
    """The current device's memory clock, bus width, CU count and L2 size."""
    buf = (ctypes.c_int32 * len(MEMORY_INFO))()
    n = load().fsa_device_memory(buf, len(MEMORY_INFO))
    if n < 0:
        raise FsaError(FSA_ERR_HIP, load().fsa_last_error().decode())
    return {k: int(buf[i]) for i, k in enumerate(MEMORY_INFO[:n])}


def build_flags() -> int:
    """fsa_build_flags of the library in use: bit 0 = LDS-poison debug build."""
    return int(load().fsa_build_flags())


def set_one_launch(mode: int) -> int:
    """When the one-launch form of the wide plan is used (process-wide): 0
    never (the default), 1 for unit counts that are multiples of 8, 2 wherever
    it applies.  Returns the previous mode."""
    return int(load().fsa_set_one_launch(int(mode)))


def one_launch_stalls() -> int:
    """Waits the one-launch kernel gave up on since the library was loaded
    (nonzero: some step's result is wrong).  Synchronises the device."""
    n = ctypes.c_int64(0)
    _check(load().fsa_one_launch_stalls(ctypes.byref(n)))
    return int(n.value)


def read_probe(buf, sink, stream=None):
    """One plain streaming read of the device tensor buf (the read ceiling)."""
    _check(load().fsa_read_probe(_p(buf, "buf"), buf.numel() * buf.element_size(), _p(sink, "sink"),
                                 _stream(stream)))


def max_work_items(d: Dims, c: LayerCfg, max_seq_len) -> int:
    n = load().fsa_max_work_items(ctypes.byref(d), c, int(max_seq_len))
    if n < 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    return n


def select_pages(d: Dims, c: LayerCfg, max_seq_len, scores, page_table, seq_lens, sel_pages=None, work=None,
                 counts=None, stream=None):
    _check(load().fsa_select_pages(ctypes.byref(d), c, int(max_seq_len), _p(scores, "scores", 4),
                                   _i32(page_table, "page_table"), _i32(seq_lens, "seq_lens"),
                                   _i32(sel_pages, "sel_pages"), _i32(work, "work"), _i32(counts, "counts"),
                                   _stream(stream)))


def sparse_decode_workspace_bytes(d: Dims, c: LayerCfg, max_seq_len) -> int:
    n = load().fsa_sparse_decode_workspace_bytes(ctypes.byref(d), c, int(max_seq_len))
    if n == 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    return n


def sparse_decode_attn(d: Dims, c: LayerCfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table,
                       seq_lens, out, sel_pages, workspace, stream=None):
    _check(load().fsa_sparse_decode_attn(
        ctypes.byref(d), c, float(sm_scale), int(max_seq_len), _p(q, "q", 2), _p(k_cache, "k_cache", 2),
        _p(v_cache, "v_cache", 2), _p(meta, "meta", 2), _i32(page_table, "page_table"),
        _i32(seq_lens, "seq_lens"), _p(out, "out", 2), _i32(sel_pages, "sel_pages"),
        _p(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # FSA_NOALLOC_SCRATCH_BYTES in include/fsa.h


def sparse_decode_attn_noalloc(d: Dims, c: LayerCfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table,
                               seq_lens, out, sel_pages, stream=None):
    """fsa_sparse_decode_attn with the library's own per-GPU workspace (no allocation)."""
    _check(load().fsa_sparse_decode_attn_noalloc(
        ctypes.byref(d), c, float(sm_scale), int(max_seq_len), _p(q, "q", 2), _p(k_cache, "k_cache", 2),
        _p(v_cache, "v_cache", 2), _p(meta, "meta", 2), _i32(page_table, "page_table"),
        _i32(seq_lens, "seq_lens"), _p(out, "out", 2), _i32(sel_pages, "sel_pages"), _stream(stream)))


def sparse_decode_attn_launches(d: Dims, c: LayerCfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table,
                                seq_lens, out, sel_pages, workspace, first, last, stream=None) -> int:
    """Only launches first..last of the decode step (measurement); returns the step's launch count."""
    n = load().fsa_sparse_decode_attn_launches(
        ctypes.byref(d), c, float(sm_scale), int(max_seq_len), _p(q, "q", 2), _p(k_cache, "k_cache", 2),
        _p(v_cache, "v_cache", 2), _p(meta, "meta", 2), _i32(page_table, "page_table"),
        _i32(seq_lens, "seq_lens"), _p(out, "out", 2), _i32(sel_pages, "sel_pages"),
        _p(workspace, "workspace"), workspace.numel() * workspace.element_size(), int(first), int(last),
        _stream(stream))
    if n < 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    return n


def append_decode_attn(d: Dims, n_new, k_new, v_new, seq_lens, seq_lens_out, c: LayerCfg, sm_scale, max_seq_len,
                       q, k_cache, v_cache, meta, page_table, out, sel_pages, workspace, stream=None):
    _check(load().fsa_append_decode_attn(
        ctypes.byref(d), int(n_new), _p(k_new, "k_new", 2), _p(v_new, "v_new", 2), _i32(seq_lens, "seq_lens"),
        _i32(seq_lens_out, "seq_lens_out"), c, float(sm_scale), int(max_seq_len), _p(q, "q", 2),
        _p(k_cache, "k_cache", 2), _p(v_cache, "v_cache", 2), _p(meta, "meta", 2), _i32(page_table, "page_table"),
        _p(out, "out", 2), _i32(sel_pages, "sel_pages"), _p(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def dense_decode_workspace_bytes(d: Dims, max_seq_len) -> int:
    n = load().fsa_dense_decode_workspace_bytes(ctypes.byref(d), int(max_seq_len))
    if n == 0:
        raise FsaError(FSA_ERR_INVALID_ARG, load().fsa_last_error().decode())
    return n


def dense_decode_attn(d: Dims, sm_scale, max_seq_len, q, k_cache, v_cache, page_table, seq_lens, out,
                      workspace, stream=None):
    _check(load().fsa_dense_decode_attn(
        ctypes.byref(d), float(sm_scale), int(max_seq_len), _p(q, "q", 2), _p(k_cache, "k_cache", 2),
        _p(v_cache, "v_cache", 2), _i32(page_table, "page_table"), _i32(seq_lens, "seq_lens"),
        _p(out, "out", 2), _p(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def validate_inputs(d: Dims, max_seq_len, q, page_table, seq_lens, scratch=None, stream=None, n_new=0) -> None:
    """Debug check of device inputs (synchronises); raises FsaError naming a violation.
    With n_new > 0 the lengths are checked as they will be after appending n_new tokens."""
    if scratch is None:
        scratch = torch.empty(4, dtype=torch.int32, device=page_table.device)
    _check(load().fsa_validate_inputs(
        ctypes.byref(d), int(n_new), int(max_seq_len), _p(q, "q", 2) if q is not None else None,
        _i32(page_table, "page_table"), _i32(seq_lens, "seq_lens"), _i32(scratch, "scratch"), _stream(stream)))
