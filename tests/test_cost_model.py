"""The per-layer decode-cost model (host only): it reproduces the MI355X step
times it was fitted to, predicts step times it was not fitted to (the 12
layer configurations of the 12-layer sweep and G 8 with a 2048 window, within
15%), its terms are physical (non-negative), and it orders configurations the
way the measurements do."""
import json

import pytest

from free_sparse_attention_amd import cost_model as cm


@pytest.fixture(scope="module")
def model():
    return cm.load()


def _shape(r):
    return cm.StepShape(r["batch"], r["q_heads"], r["kv_heads"], r["head_dim"], r["seq_len"], r["prefix"], r["window"],
                        r["budget_pages"])


def test_reproduces_the_measurements(model):
    rows = json.load(open(cm._DATA))["rows"]
    assert len(rows) >= 40
    for r in rows:
        s = _shape(r)
        assert abs(model.dense_us(s) - r["dense_us"]) <= 0.12 * r["dense_us"], r
        assert abs(model.sparse_us(s) - r["sparse_us"]) <= 0.15 * r["sparse_us"], r


def test_terms_are_physical(model):
    t = model.terms
    assert all(v >= 0 for v in t.values())
    # the dense kernel streams K/V at several TB/s: 1 MB costs well under a microsecond
    assert 0.05 < t["d_kv_us_per_mb"] < 0.5


def test_orders_configurations(model):
    base = cm.StepShape(4, 16, 4, 128, 65536, 128, 1024, 128)
    longer = cm.StepShape(4, 16, 4, 128, 262144, 128, 1024, 128)
    bigger_budget = cm.StepShape(4, 16, 4, 128, 65536, 128, 1024, 1024)
    assert model.sparse_us(longer) > model.sparse_us(base)
    assert model.sparse_us(bigger_budget) > model.sparse_us(base)
    assert model.dense_us(longer) > 3 * model.dense_us(base)
    assert model.layer_cost(base)["speedup_vs_dense"] > 2.0


def test_budget_covering_every_candidate_costs_dense(model):
    s = cm.StepShape(4, 16, 4, 128, 4096, 128, 1024, 1024)
    assert model.sparse_us(s) == model.dense_us(s)


def test_predicts_points_it_was_not_fitted_to(model):
    """Out of sample: the measured steps of cost_model_holdout.json
    (bench.py --holdout) that are not calibration points (15 of its 16)."""
    fit = {(r["q_heads"], r["seq_len"], r["prefix"], r["window"], r["budget_pages"])
           for r in json.load(open(cm._DATA))["rows"]}
    rows = [r for r in json.load(open(cm._HOLDOUT))["rows"]  # one sweep layer is also a calibration point
            if (r["q_heads"], r["seq_len"], r["prefix"], r["window"], r["budget_pages"]) not in fit]
    assert len(rows) >= 12
    for r in rows:
        s = _shape(r)
        assert abs(model.sparse_us(s) - r["sparse_us"]) <= 0.15 * r["sparse_us"], r
        assert abs(model.dense_us(s) - r["dense_us"]) <= 0.15 * r["dense_us"], r


def test_plan_features_come_from_the_library(model):
    """The model's plan terms are the library's own planner's (fsa_describe_step)."""
    from free_sparse_attention_amd import _lib
    s = cm.StepShape(4, 32, 4, 128, 262144, 128, 4096, 256)
    f = cm._features(s, 256)
    n = -(-s.seq_len // 16)
    p = _lib.describe_step(_lib.dims(4, 32, 4, 128, n, 4 * n), _lib.cfg(128, 4096, 256), s.seq_len)
    assert f["cols"] == p["select_cols"] and f["ipw"] == -(-p["per_replica"] // 16) and not f["narrow"]
