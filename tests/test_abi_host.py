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
    # the validator checks its host arguments before any launch
    assert lib.fsa_validate_inputs(ctypes.byref(d), 4096, p, p, p, None, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"scratch" in lib.fsa_last_error()
    assert lib.fsa_validate_inputs(ctypes.byref(d), 0, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
