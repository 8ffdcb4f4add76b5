"""Per-layer decode-cost model of the combined sparse attention step.

The method's per-layer configuration search weighs the accuracy of a layer's
(prefix, window, budget) choice against its estimated decoding cost (paper,
analysis page "Methodology").  This module supplies that estimate for this
library on MI355X: predicted microseconds of one ``fsa_sparse_decode_attn``
call (and of the dense baseline) for given shapes and configuration, fitted
by non-negative least squares to step times measured on the device
(``bench.py --calibrate``, stored in ``cost_model_data.json``).

Terms, per step (sums over the B x Hkv (sequence, KV head) units):

* sparse, when some sequence has more candidate pages than the budget:
  ``c0 + c_meta * metadata MB + c_cols * pages-per-thread of the selection
  + c_ipw * selected pages per wave (wide plan) + c_narrow * [narrow plan]
  + c_narrow_sel * selected K/V MB (narrow plan)``;
* otherwise the step runs the dense kernels: the dense cost;
* dense: ``d0 + d_kv * K/V MB``.

The plan terms (which plan, pages per selection thread, selected pages per
replica) are the library's own, read from ``fsa_describe_step``; the fit is
checked against measured points it was not fitted to
(``cost_model_holdout.json``, ``bench.py --holdout``).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass

import numpy as np

PAGE = 16
_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_model_data.json")
_HOLDOUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_model_holdout.json")


@dataclass(frozen=True)
class StepShape:
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    seq_len: int
    prefix: int
    window: int
    budget_pages: int


def _features(s: StepShape, compute_units: int) -> dict:
    """Byte counts of the step, and its launch plan as the library itself
    plans it (fsa_describe_step: host only; without a device the library
    plans for MI355X's 256 compute units)."""
    from . import _lib

    units = s.batch * s.kv_heads
    n = -(-s.seq_len // PAGE)
    pe, ws = min(s.prefix, s.seq_len), max(0, s.seq_len - s.window)
    cand = (-(-ws // PAGE) - pe // PAGE) if pe < ws else 0
    k = min(s.budget_pages, cand)
    d = _lib.dims(s.batch, s.q_heads, s.kv_heads, s.head_dim, n, s.batch * n)
    plan = _lib.describe_step(d, _lib.cfg(s.prefix, s.window, s.budget_pages), s.seq_len)
    wide = plan["plan"] == "wide"
    page_kv = 2 * PAGE * s.head_dim * 2  # K and V bytes of one page of one KV head
    return {
        "all_taken": plan["plan"] == "dense",
        "meta_mb": units * cand * 4 * s.head_dim / 1e6,
        "sel_mb": units * k * page_kv / 1e6,
        "dense_mb": units * n * page_kv / 1e6,
        "cols": plan["select_cols"],
        # selected pages each wave of a selection replica attends (wide plan)
        "ipw": -(-plan["per_replica"] // 16) if wide else 0,
        "narrow": int(plan["plan"] == "narrow"),
    }


def _sparse_row(f: dict) -> list:
    return [1.0, f["meta_mb"], f["cols"], (1 - f["narrow"]) * f["ipw"], f["narrow"], f["narrow"] * f["sel_mb"]]


SPARSE_TERMS = ("c0_us", "c_meta_us_per_mb", "c_cols_us", "c_ipw_us", "c_narrow_us", "c_narrow_sel_us_per_mb")
DENSE_TERMS = ("d0_us", "d_kv_us_per_mb")


class CostModel:
    """Fitted decode-cost model; see the module docstring for its terms."""

    def __init__(self, rows: list[dict], compute_units: int = 256):
        from scipy.optimize import nnls

        self.compute_units = compute_units
        shapes = [StepShape(r["batch"], r["q_heads"], r["kv_heads"], r["head_dim"], r["seq_len"], r["prefix"],
                            r["window"], r["budget_pages"]) for r in rows]
        feats = [_features(s, compute_units) for s in shapes]
        xd = np.array([[1.0, f["dense_mb"]] for f in feats])
        self.dense_coef = nnls(xd, np.array([r["dense_us"] for r in rows]))[0]
        idx = [i for i, f in enumerate(feats) if not f["all_taken"]]
        xs = np.array([_sparse_row(feats[i]) for i in idx])
        self.sparse_coef = nnls(xs, np.array([rows[i]["sparse_us"] for i in idx]))[0]

    @property
    def terms(self) -> dict:
        return dict(zip(SPARSE_TERMS + DENSE_TERMS, [float(c) for c in self.sparse_coef] +
                        [float(c) for c in self.dense_coef]))

    def dense_us(self, s: StepShape) -> float:
        f = _features(s, self.compute_units)
        return float(self.dense_coef @ np.array([1.0, f["dense_mb"]]))

    def sparse_us(self, s: StepShape) -> float:
        f = _features(s, self.compute_units)
        if f["all_taken"]:
            return self.dense_us(s)
        return float(self.sparse_coef @ np.array(_sparse_row(f)))

    def layer_cost(self, s: StepShape) -> dict:
        """Predicted sparse and dense step times and their ratio for one layer."""
        sp, de = self.sparse_us(s), self.dense_us(s)
        return {"sparse_us": sp, "dense_us": de, "speedup_vs_dense": de / sp}


def load(path: str = _DATA) -> CostModel:
    """The model fitted to the packaged MI355X measurements."""
    data = json.load(open(path))
    return CostModel(data["rows"], data.get("compute_units", 256))
