"""ctypes front end of the counter-based generator in ``synth.c``."""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libfsa_synth.so")
_lock = threading.Lock()
_lib = None


def build_lib(force: bool = True) -> str:
    """Compile synth.c with gcc (OpenMP) into libfsa_synth.so; returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build_lib(force=False)
            L = ctypes.CDLL(_LIB)
            u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
            L.synth_stream_key.restype = u64
            L.synth_stream_key.argtypes = [u64, u64]
            L.synth_bf16_from_double.restype = ctypes.c_uint16
            L.synth_bf16_from_double.argtypes = [ctypes.c_double]
            for name in ("synth_uniform", "synth_normal_f64", "synth_normal_bf16", "synth_raw_u64"):
                f = getattr(L, name)
                f.restype = None
                f.argtypes = [u64, u64, i64, vp]
            L.synth_fill_pool_seq.restype = None
            L.synth_fill_pool_seq.argtypes = [u64, i32, i64, i64, i32, i32, i32, vp, vp, vp]
            L.synth_fill_tokens.restype = None
            L.synth_fill_tokens.argtypes = [u64, i32, i64, i64, i32, i32, vp, vp]
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_key(seed: int, stream: int) -> int:
    return int(lib().synth_stream_key(seed & (2**64 - 1), stream & (2**64 - 1)))


def uniform(key: int, n: int, idx0: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform(key, idx0, n, _ptr(out))
    return out


def normal_f64(key: int, n: int, idx0: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal_f64(key, idx0, n, _ptr(out))
    return out


def normal_bf16(key: int, n: int, idx0: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(key, idx0, n, _ptr(out))
    return out


def raw_u64(key: int, n: int, idx0: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_raw_u64(key, idx0, n, _ptr(out))
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to fp32 (nearest-even), then to bf16 (nearest-even); finite inputs."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def fill_pool_seq(key: int, b: int, t0: int, t1: int, hkv: int, d: int, page: int,
                  page_row: np.ndarray, scale: np.ndarray | None, pool: np.ndarray) -> None:
    page_row = np.ascontiguousarray(page_row, dtype=np.int32)
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float64)
    lib().synth_fill_pool_seq(key, b, t0, t1, hkv, d, page, _ptr(page_row),
                              None if sc is None else _ptr(sc), _ptr(pool))


def fill_tokens(key: int, b: int, t0: int, n: int, hkv: int, d: int,
                scale: np.ndarray | None) -> np.ndarray:
    out = np.empty((n, hkv, d), np.uint16)
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float64)
    lib().synth_fill_tokens(key, b, t0, n, hkv, d, None if sc is None else _ptr(sc), _ptr(out))
    return out
