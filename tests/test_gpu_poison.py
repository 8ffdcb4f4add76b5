"""Parity on the LDS-poison debug build (libfsa_poison.so).

In that build every kernel fills its LDS with a NaN pattern when it starts and
where a later stage reuses an earlier stage's LDS (the selection's space
becoming the attention merge), so a read of LDS that no stage of the kernel
wrote shows up as NaN or garbage in the scores, selections, work lists or
outputs.  The cases below rerun parity checks of the other GPU test modules,
unchanged, with the binding switched to that build: every kernel and both
step plans, the stand-alone selection, the dense path, the append, 16 and 32
pages per selection thread, the 64k and 256k workloads, and the one-launch
form of the step against the separate launches.
"""
import os

import pytest

import tests.test_gpu_one_launch as O
import tests.test_gpu_parity as P
import tests.test_gpu_workloads as W
from free_sparse_attention_amd import _lib

pytestmark = pytest.mark.gpu

CASES = [
    (P.test_tiny_end_to_end, {}),
    (P.test_shapes, {"d": 64, "hq": 12, "hkv": 4}),
    (P.test_many_units_both_step_plans, {"budget": 40}),
    (P.test_many_units_both_step_plans, {"budget": 80}),
    (P.test_wide_plan_replicas_spread_over_xcds, {}),
    (P.test_longest_contexts_32_pages_per_thread, {}),
    (P.test_configs_and_degenerate_regions, {"cfg": (37, 53, 6)}),
    (P.test_short_sequences, {"L": 17}),
    (P.test_all_scores_tie_takes_lowest_ids, {}),
    (P.test_full_budget_equals_dense, {}),
    (P.test_append_matches_rebuild_and_oracle, {}),
    (W.test_ctx64k_all_units, {}),
    (W.test_ctx256k_all_units, {}),
    (O.test_one_launch_equals_separate_launches, {"case": "b4_h4_ragged"}),
    (O.test_one_launch_equals_separate_launches, {"case": "b3_h2_d64"}),
]


@pytest.fixture
def poisoned():
    if not os.path.exists(_lib.POISON_LIB_PATH):
        pytest.fail(f"{_lib.POISON_LIB_PATH} is not built; run `python -m free_sparse_attention_amd.build`")
    with _lib.using(_lib.POISON_LIB_PATH) as L:
        assert L.fsa_build_flags() & 1, "the debug library does not poison its LDS"
        yield L
    assert _lib.load().fsa_build_flags() == 0  # the release build is back in use


@pytest.mark.parametrize("fn,kw", CASES, ids=[f"{f.__name__}{'-' + '-'.join(map(str, k.values())) if k else ''}"
                                               for f, k in CASES])
def test_parity_with_poisoned_lds(poisoned, fn, kw):
    fn(**kw)
