"""The C-ABI library loads, exports every entry point of include/fsa.h, and
rejects bad host arguments before touching a GPU (no device needed)."""
import ctypes
import os
import re

import pytest

import free_sparse_attention_amd as fsa
from free_sparse_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfsa.so is not built (run python -m free_sparse_attention_amd.build)")
    return fsa.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def _d(**kw):
    base = dict(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64, max_pages_per_seq=256, num_pool_pages=256)
    base.update(kw)
    return fsa.dims(**base)


def test_workspace_sizing_and_bad_shapes(lib):
    c = fsa.cfg(64, 256, 32)
    assert fsa.sparse_decode_workspace_bytes(_d(), c, 4096) > 0
    assert fsa.dense_decode_workspace_bytes(_d(), 4096) > 0
    assert fsa.max_work_items(_d(), c, 4096) == 4 + 32 + 17
    assert fsa.meta_bytes(_d()) == 1 * 2 * 16 * 16 * 2 * 64 * 2
    for bad, status in ((dict(head_dim=96), _lib.FSA_ERR_UNSUPPORTED), (dict(num_q_heads=7), _lib.FSA_ERR_INVALID_ARG),
                        (dict(num_q_heads=34, num_kv_heads=2), _lib.FSA_ERR_UNSUPPORTED),
                        (dict(batch=0), _lib.FSA_ERR_INVALID_ARG)):
        assert lib.fsa_sparse_decode_workspace_bytes(ctypes.byref(_d(**bad)), c, 4096) == 0
        with pytest.raises(fsa.FsaError) as e:
            fsa.sparse_decode_workspace_bytes(_d(**bad), c, 4096)
        assert "dims" in str(e.value)
        st = lib.fsa_quest_scores(ctypes.byref(_d(**bad)), c, 4096, None, None, None, None, None)
        assert st == status
    # page size other than 16
    assert lib.fsa_build_page_meta(ctypes.byref(_d(page_size=32)), None, None, None, None, None) == _lib.FSA_ERR_UNSUPPORTED


def test_bad_cfg_len_and_pointers(lib):
    d = _d()
    p = ctypes.c_void_p(16)  # never dereferenced: every check runs before a launch
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(0, 0, 0), 4096, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"attends to nothing" in lib.fsa_last_error()
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(-1, 0, 4), 4096, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(64, 256, 32), 4097, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(64, 256, 32), 4096, p, None, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"meta" in lib.fsa_last_error()
    assert lib.fsa_append_kv(ctypes.byref(d), 0, p, p, p, p, None, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_kv(ctypes.byref(d), 1, p, p, p, p, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"alias" in lib.fsa_last_error()
    need = fsa.sparse_decode_workspace_bytes(d, fsa.cfg(64, 256, 32), 4096)
    st = lib.fsa_sparse_decode_attn(ctypes.byref(d), fsa.cfg(64, 256, 32), 0.125, 4096, p, p, p, p, p, p, p, None,
                                    p, need - 1, None)
    assert st == _lib.FSA_ERR_WORKSPACE
    st = lib.fsa_sparse_decode_attn(ctypes.byref(d), fsa.cfg(64, 256, 32), 0.0, 4096, p, p, p, p, p, p, p, None,
                                    p, need, None)
    assert st == _lib.FSA_ERR_INVALID_ARG
    st = lib.fsa_dense_decode_attn(ctypes.byref(d), 0.125, 4096, p, p, p, p, p, p, p, 0, None)
    assert st == _lib.FSA_ERR_WORKSPACE
    # combined append + decode: the append's and the step's checks, before any launch
    c = fsa.cfg(64, 256, 32)
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 0, p, p, p, p, c, 0.125, 4096, p, p, p, p, p, p, None, p, need,
                                      None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, p, c, 0.125, 4096, p, p, p, p, p, p, None, p, need,
                                      None) == _lib.FSA_ERR_INVALID_ARG
    assert b"alias" in lib.fsa_last_error()
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, None, c, 0.125, 4096, p, p, p, p, p, p, None, p,
                                      need, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, ctypes.c_void_p(32), c, 0.125, 4096, p, p, p, p,
                                      p, p, None, p, need - 1, None) == _lib.FSA_ERR_WORKSPACE
    # the validator checks its host arguments before any launch
    assert lib.fsa_validate_inputs(ctypes.byref(d), 4096, p, p, p, None, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"scratch" in lib.fsa_last_error()
    assert lib.fsa_validate_inputs(ctypes.byref(d), 0, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG


def _plan(B, hq, hkv, D, L, P, W, budget):
    n = (L + 15) // 16 + 8
    return fsa.describe_step(fsa.dims(B, hq, hkv, D, n, B * n), fsa.cfg(P, W, budget), L)


def test_step_plans_on_256_cus(lib):
    """Host-side planning (no device here: the library assumes MI355X's 256
    CUs).  Shapes of the 64k, 256k and ragged serving workloads, a short
    context and a many-replica case."""
    p = _plan(4, 16, 4, 128, 65536, 128, 1024, 128)
    assert (p["plan"], p["replicas"], p["per_replica"], p["xcd_grouped"], p["prefetch"], p["select_cols"]) == \
        ("wide", 8, 16, 1, 1, 4)
    assert p["slots"] == p["pw_workgroups"] + p["replicas"]
    p = _plan(4, 32, 4, 128, 262144, 128, 4096, 256)  # one XCD's share of selected K/V (4 MiB) > half its L2
    assert (p["plan"], p["replicas"], p["per_replica"], p["xcd_grouped"], p["prefetch"], p["select_cols"]) == \
        ("wide", 8, 32, 1, 0, 16)
    p = _plan(16, 32, 8, 128, 262144, 128, 2048, 256)  # 128 units: replicas would not fit
    assert (p["plan"], p["replicas"], p["xcd_grouped"], p["prefetch"]) == ("narrow", 0, 0, 0)
    p = _plan(9, 8, 1, 64, 6400, 32, 256, 224)  # 9 x 14 replicas fit, but 28 per XCD do not fit half an XCD
    assert (p["plan"], p["replicas"], p["xcd_grouped"], p["prefetch"]) == ("wide", 14, 0, 0)
    p = _plan(4, 16, 4, 128, 2048, 128, 1024, 128)  # every candidate fits the budget
    assert p["plan"] == "dense" and p["replicas"] == 0
    assert _plan(1, 8, 1, 128, 400001, 128, 4096, 256)["select_cols"] == 32


def test_describe_step_rejects_bad_arguments(lib):
    d = fsa.dims(1, 8, 2, 64, 100, 100)
    buf = (ctypes.c_int32 * 8)()
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 1600, None, 8) == -1
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 1600, buf, 3) == 3
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 10 ** 9, buf, 8) == -1


def test_measurement_helpers_check_their_arguments(lib):
    sink = ctypes.c_void_p(256)  # never dereferenced: every call below fails before any launch
    for buf, nbytes in ((None, 1024), (ctypes.c_void_p(4096), 0), (ctypes.c_void_p(4096), 1000),
                        (ctypes.c_void_p(4104), 1024)):
        assert lib.fsa_read_probe(buf, nbytes, sink, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_read_probe(ctypes.c_void_p(4096), 1024, None, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_device_memory(None, 4) == -1
    info = (ctypes.c_int32 * 4)()
    n = lib.fsa_device_memory(info, 4)
    if n == -1:  # no device here
        assert lib.fsa_last_error()
    else:
        assert n == 4 and info[0] > 0 and info[1] > 0 and info[2] > 0


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library the binding raises; nothing falls back to a CPU path."""
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load("/nonexistent/libfsa.so")
