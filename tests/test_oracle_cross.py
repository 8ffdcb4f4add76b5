"""The C++ oracle's whole-unit path from the pool (``oracle.decode_units``, the
one the GPU parity tests and the CPU baseline call) against its own pinned
steps composed one by one, and against the independent float64 numpy oracle
(``oracle.reference``): the two implementations must agree to 1e-12."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import reference as R

S = 16


def _cases():
    yield synth.make_workload("tiny")
    yield synth.workloads.build(name="x1", seed=41, batch=3, hq=16, hkv=4, d=128, seq_lens=(3000, 777, 1601),
                                prefix=32, window=200, budget=9, k_sigma=0.5, n_needles=4, permuted=True)
    yield synth.workloads.build(name="x2", seed=42, batch=2, hq=12, hkv=4, d=64, seq_lens=(1, 513), prefix=7,
                                window=33, budget=3, k_sigma=0.3, permuted=True)
    yield synth.workloads.build(name="x3", seed=43, batch=2, hq=8, hkv=1, d=64, seq_lens=(2049, 600), prefix=0,
                                window=0, budget=5, permuted=False)


@pytest.mark.parametrize("wl", list(_cases()), ids=lambda w: w.name)
def test_pool_path_equals_steps_and_numpy(wl):
    units = [(b, g) for b in range(wl.batch) for g in range(wl.hkv)]
    r = oracle.decode_units(wl, units, want_meta=True)
    for j, (b, g) in enumerate(units):
        L = int(wl.seq_lens[b])
        q, K, V = oracle.unit_inputs(wl, b, g)
        steps = oracle.sparse_decode_unit(q, K, V, L, wl.cfg, S, wl.sm_scale)
        npy = R.sparse_decode_unit(*R.unit_inputs(wl, b, g), L, wl.cfg, S, wl.sm_scale)
        cand = steps["candidates"]
        assert np.array_equal(cand, npy["candidates"])
        # scores: the same sums in the same order (C++), within rounding of numpy's
        assert np.array_equal(r["scores"][j, cand], steps["scores"])
        assert np.allclose(steps["scores"], npy["scores"], rtol=1e-12, atol=1e-12)
        k = int(r["k"][j])
        assert r["sel"][j, :k].tolist() == steps["selected"].tolist() == npy["selected"].tolist()
        assert (r["sel"][j, k:] == -1).all()
        assert r["margin"][j] == steps["margin"] or (math.isinf(r["margin"][j]) and math.isinf(steps["margin"]))
        assert np.allclose(r["margin"][j], npy["margin"], rtol=1e-9) or math.isinf(npy["margin"])
        assert np.allclose(r["out"][j], steps["out"], rtol=1e-12, atol=1e-12)
        assert np.allclose(r["out"][j], npy["out"], rtol=1e-12, atol=1e-12)
        n = -(-L // S)
        assert np.array_equal(r["meta"][j, :n, 0], steps["meta"][0]) and np.array_equal(r["meta"][j, :n, 1],
                                                                                         steps["meta"][1])
        assert np.array_equal(steps["meta"][0], npy["meta"][0]) and np.array_equal(steps["meta"][1], npy["meta"][1])


def test_pool_path_with_given_selection_dense_and_meta():
    wl = synth.workloads.build(name="x4", seed=44, batch=2, hq=8, hkv=2, d=64, seq_lens=(2500, 1800), prefix=64,
                               window=128, budget=6, k_sigma=0.5, n_needles=3, permuted=True)
    units = [(0, 1), (1, 0)]
    own = oracle.decode_units(wl, units)
    given = [[5, 9, 40], [3]]
    r = oracle.decode_units(wl, units, sel_in=given)
    dense = oracle.decode_units(wl, units, dense=True)
    meta = oracle.build_meta_all(wl)
    with_meta = oracle.decode_units(wl, units, meta=meta)
    for j, (b, g) in enumerate(units):
        L = int(wl.seq_lens[b])
        q, K, V = R.unit_inputs(wl, b, g)
        ref = R.attend(q, K, V, R.attended_mask(L, 64, 128, S, given[j]), wl.sm_scale)
        assert np.allclose(r["out"][j], ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(dense["out"][j], R.dense_decode_unit(q, K, V, wl.sm_scale), rtol=1e-12, atol=1e-12)
        # a given selection changes only the attention, not the oracle's own scores and selection
        assert np.array_equal(r["sel"][j], own["sel"][j])
        assert np.array_equal(with_meta["out"][j], own["out"][j]) and np.array_equal(with_meta["sel"][j],
                                                                                    own["sel"][j])


def test_pool_path_invariant_under_page_permutation_and_finds_needles():
    a = synth.make_workload("tiny", permuted=False)
    b = synth.make_workload("tiny", permuted=True)
    ra, rb = oracle.decode_units(a, [(0, 0), (0, 1)]), oracle.decode_units(b, [(0, 0), (0, 1)])
    assert np.array_equal(ra["out"], rb["out"]) and np.array_equal(ra["sel"], rb["sel"])
    pages = set((a.needles[0] // S).tolist())
    for j in range(2):
        assert pages <= set(ra["sel"][j].tolist())


def test_pool_path_rejects_bad_units():
    wl = synth.make_workload("tiny")
    for bad in ([(1, 0)], [(0, 2)], [(-1, 0)]):
        with pytest.raises(ValueError):
            oracle.decode_units(wl, bad)
