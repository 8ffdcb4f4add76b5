"""CPU oracle of combined sparse decode attention (test infrastructure only).

The oracle is the plain C++ implementation in ``oracle.cpp``, reached through
the ctypes front end ``oracle.cpp`` module; its functions are re-exported here.
``reference`` is an independent float64 numpy implementation of the same
steps, kept as a cross-check that must agree with it to 1e-12.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU baseline of ``bench.py`` import
this package; the library's product path never does.
"""
from .cpp import (  # noqa: F401
    attend,
    attended_mask,
    bf16_to_f64,
    build_lib,
    build_meta,
    build_meta_all,
    candidate_pages,
    decode_units,
    default_threads,
    dense_decode_unit,
    gather_keys,
    group_score,
    page_minmax,
    quest_bound,
    regions,
    select_topk,
    selection_margin,
    sparse_decode_unit,
    unit_inputs,
)
from . import reference  # noqa: F401
