"""ctypes front end of the plain C++ oracle in ``oracle.cpp``.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` use it; nothing in the library's product path does.
Every function here only moves arrays in and out; the arithmetic is in
``oracle.cpp`` (see its header for the method and the readings taken).  The
functions keep the names of the float64 numpy oracle in ``reference.py``,
which stays as an independent cross-check that must agree to 1e-12.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build_lib(force: bool = True) -> str:
    """Compile oracle.cpp with g++ into liboracle.so; returns its path."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lpthread"],
                       check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                build_lib(force=False)
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            sig = {
                "ora_bf16_decode": (None, [vp, i64, vp]),
                "ora_gather": (None, [vp, vp, i32, i32, i32, i32, i32, vp]),
                "ora_page_minmax": (None, [vp, i32, i32, i32, vp, vp]),
                "ora_candidates": (i32, [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int)]),
                "ora_quest_bound": (None, [vp, vp, vp, i32, i32, i32, vp]),
                "ora_group_score": (None, [vp, i32, i32, vp]),
                "ora_select_topk": (i32, [vp, vp, i32, i32, vp]),
                "ora_selection_margin": (f64, [vp, i32, i32]),
                "ora_attended_mask": (None, [i32, i32, i32, i32, vp, i32, vp]),
                "ora_attend": (None, [vp, vp, vp, vp, i32, i32, i32, f64, vp]),
                "ora_build_meta": (None, [vp, vp, vp, i32, i32, i32, i32, i32, vp, i32]),
                "ora_decode_units": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                           vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, i32]),
            }
            for name, (res, args) in sig.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------------ single steps

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().ora_bf16_decode(_ptr(b), b.size, _ptr(out))
    return out


def gather_keys(pool: np.ndarray, page_table: np.ndarray, b: int, g: int, L: int) -> np.ndarray:
    """Keys (or values) of tokens [0, L) of sequence b, KV head g: float64 [L][D]."""
    pool = np.ascontiguousarray(pool, dtype=np.uint16)
    row = _i32(page_table[b])
    _, hkv, S, D = pool.shape
    out = np.empty((L, D), np.float64)
    lib().ora_gather(_ptr(pool), _ptr(row), hkv, D, S, g, L, _ptr(out))
    return out


def page_minmax(keys: np.ndarray, S: int):
    """Elementwise min and max of every page's valid keys: (m, M), each [ceil(L/S)][D]."""
    k = _f64(keys)
    L, D = k.shape
    n = -(-L // S)
    m = np.empty((n, D))
    M = np.empty((n, D))
    lib().ora_page_minmax(_ptr(k), L, D, S, _ptr(m), _ptr(M))
    return m, M


def build_meta(k_pool: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray) -> dict:
    """Metadata of every mapped page in use: {(phys, g): (m[D], M[D])} float64."""
    out = {}
    S = k_pool.shape[2]
    for b, L in enumerate(seq_lens):
        for g in range(k_pool.shape[1]):
            m, M = page_minmax(gather_keys(k_pool, page_table, b, g, int(L)), S)
            for p in range(m.shape[0]):
                out[(int(page_table[b, p]), g)] = (m[p], M[p])
    return out


def regions(L: int, prefix: int, window: int):
    """(Pe, Ws): the prefix is [0, Pe), the window [Ws, L), the middle [Pe, Ws)."""
    return min(prefix, L), max(0, L - window)


def candidate_pages(L: int, prefix: int, window: int, S: int) -> np.ndarray:
    """Logical pages that meet the middle region (empty if there is none)."""
    c_lo = ctypes.c_int(0)
    C = lib().ora_candidates(int(L), int(prefix), int(window), int(S), ctypes.byref(c_lo))
    return np.arange(c_lo.value, c_lo.value + C, dtype=np.int64)


def quest_bound(q: np.ndarray, m: np.ndarray, M: np.ndarray) -> np.ndarray:
    """U[h][c] = sum_i max(q[h,i] m[c,i], q[h,i] M[c,i])."""
    q, m, M = _f64(q), _f64(m), _f64(M)
    G, D = q.shape
    C = m.shape[0]
    U = np.empty((G, C))
    lib().ora_quest_bound(_ptr(q), _ptr(m), _ptr(M), G, C, D, _ptr(U))
    return U


def group_score(U: np.ndarray) -> np.ndarray:
    """The group's score of each page: the largest per-head bound."""
    U = _f64(U)
    G, C = U.shape
    s = np.empty(C)
    lib().ora_group_score(_ptr(U), G, C, _ptr(s))
    return s


def select_topk(scores: np.ndarray, pages: np.ndarray, budget: int) -> np.ndarray:
    """The k = min(budget, C) best pages (ties to the lower id), ascending."""
    s, p = _f64(scores), _i32(pages)
    sel = np.empty(max(len(p), 1), np.int32)
    k = lib().ora_select_topk(_ptr(s), _ptr(p), len(p), int(budget), _ptr(sel))
    return sel[:k].astype(np.int64)


def selection_margin(scores: np.ndarray, budget: int) -> float:
    """(s_(k) - s_(k+1)) / |s_(k)| of the decreasing scores; inf when nothing is left out."""
    s = _f64(scores)
    return float(lib().ora_selection_margin(_ptr(s), len(s), int(budget)))


def attended_mask(L: int, prefix: int, window: int, S: int, selected) -> np.ndarray:
    """Boolean mask over [0, L): prefix, window and every token of a selected page."""
    sel = _i32(np.asarray(list(selected), dtype=np.int64).reshape(-1))
    mask = np.empty(L, np.uint8)
    lib().ora_attended_mask(int(L), int(prefix), int(window), int(S), _ptr(sel), len(sel), _ptr(mask))
    return mask.astype(bool)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray, sm_scale: float) -> np.ndarray:
    """Two-pass softmax attention of every head of q over the masked tokens."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    mk = np.ascontiguousarray(mask, dtype=np.uint8)
    G, D = q.shape
    out = np.empty((G, D))
    lib().ora_attend(_ptr(q), _ptr(K), _ptr(V), _ptr(mk), K.shape[0], G, D, float(sm_scale), _ptr(out))
    return out


# ------------------------------------------------------------------ composed, on gathered arrays

def unit_inputs(wl, b: int, g: int, q_bits=None):
    """float64 q of the group [G][D] (query heads g G .. g G + G - 1) and K, V [L][D]."""
    G = wl.hq // wl.hkv
    qb = wl.q if q_bits is None else q_bits
    q = bf16_to_f64(qb[b, g * G:(g + 1) * G])
    L = int(wl.seq_lens[b])
    return q, gather_keys(wl.k_pool, wl.page_table, b, g, L), gather_keys(wl.v_pool, wl.page_table, b, g, L)


def sparse_decode_unit(q, K, V, L, cfg, S, sm_scale, selected=None) -> dict:
    """One (sequence, KV head): scores, selection, mask and output, step by step.
    ``selected`` replaces the oracle's own selection for the attention."""
    prefix, window, budget = cfg
    m, M = page_minmax(K, S)
    cand = candidate_pages(L, prefix, window, S)
    U = quest_bound(q, m[cand], M[cand])
    s = group_score(U)
    sel = select_topk(s, cand, budget) if selected is None else np.asarray(selected)
    mask = attended_mask(L, prefix, window, S, sel)
    out = attend(q, K, V, mask, sm_scale)
    return dict(candidates=cand, scores=s, bounds=U, selected=sel, mask=mask, out=out,
                margin=selection_margin(s, budget), meta=(m, M))


def dense_decode_unit(q, K, V, sm_scale) -> np.ndarray:
    """Plain attention over all tokens [0, L)."""
    return attend(q, K, V, np.ones(K.shape[0], dtype=bool), sm_scale)


# ------------------------------------------------------------------ whole units from the pool

def build_meta_all(wl, nthreads=None) -> np.ndarray:
    """Metadata of every unit, [B][Hkv][max_pages][2][D] (min row, max row; NaN past a length)."""
    meta = np.full((wl.batch, wl.hkv, wl.max_pages, 2, wl.d), np.nan)
    lib().ora_build_meta(_ptr(np.ascontiguousarray(wl.k_pool)), _ptr(_i32(wl.page_table)), _ptr(_i32(wl.seq_lens)),
                         wl.batch, wl.hkv, wl.d, wl.page, wl.max_pages, _ptr(meta), nthreads or default_threads())
    return meta


def decode_units(wl, units, q_bits=None, cfg=None, sel_in=None, dense=False, meta=None, want_meta=False,
                 nthreads=None) -> dict:
    """The decode step of the listed (b, g) units of a workload, from its pool.

    ``sel_in`` ([n_units][*] pages, -1 padded) makes each unit attend those pages
    (with its prefix and window) instead of the oracle's own selection; ``dense``
    attends every token.  Returns scores [n][max_pages] (NaN except candidates),
    sel [n][budget] (-1 padded), margin [n], k [n], out [n][G][D] and, with
    want_meta, meta [n][max_pages][2][D] (NaN past the length)."""
    cfg = tuple(cfg if cfg is not None else wl.cfg)
    units = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    n = units.shape[0]
    G = wl.hq // wl.hkv
    qb = np.ascontiguousarray(wl.q if q_bits is None else q_bits, dtype=np.uint16)
    budget = int(cfg[2])
    scores = np.full((n, wl.max_pages), np.nan)
    sel = np.full((n, max(budget, 1)), -1, np.int32)
    margin = np.empty(n)
    k = np.empty(n, np.int32)
    out = np.empty((n, G, wl.d))
    mo = np.full((n, wl.max_pages, 2, wl.d), np.nan) if want_meta else None
    si, stride = None, 0
    if sel_in is not None:
        rows = [np.asarray(r, dtype=np.int64).reshape(-1) for r in sel_in]
        stride = max(1, max(len(r) for r in rows))
        si = np.full((n, stride), -1, np.int32)
        for j, r in enumerate(rows):
            si[j, :len(r)] = r
    rc = lib().ora_decode_units(
        _ptr(qb), _ptr(np.ascontiguousarray(wl.k_pool)), _ptr(np.ascontiguousarray(wl.v_pool)),
        _ptr(_i32(wl.page_table)), _ptr(_i32(wl.seq_lens)), wl.batch, wl.hq, wl.hkv, wl.d, wl.page, wl.max_pages,
        int(cfg[0]), int(cfg[1]), budget, float(wl.sm_scale), _ptr(meta), _ptr(units), n, _ptr(si), stride,
        int(bool(dense)), _ptr(scores), _ptr(sel), _ptr(margin), _ptr(k), _ptr(mo), _ptr(out),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("ora_decode_units rejected its arguments")
    r = dict(scores=scores, sel=sel[:, :budget], margin=margin, k=k, out=out)
    if want_meta:
        r["meta"] = mo
    return r
