"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-worked case from
tests/golden/ (handworked.json, bf16_patterns.json), a closed form, an
invariant of the definition, a library routine (torch CPU attention in
float64), or brute force on tiny inputs.  They are chosen so that a dropped
term, a wrong sign, a wrong index or a transposed operand in the oracle fails
at least one of them.  Every pin runs against both implementations: the plain
C++ oracle (``oracle``, the one the GPU parity tests use) and the independent
float64 numpy one (``oracle.reference``).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GOLD = json.load(open(os.path.join(GOLDEN, "handworked.json")))
rng = np.random.default_rng(1234)


@pytest.fixture(params=["cpp", "numpy"])
def ora(request):
    return oracle if request.param == "cpp" else oracle.reference


def _bf16(x):
    """Nearest-even bf16 values of x (test data only), via the input generator's rounding."""
    return synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(np.asarray(x, dtype=np.float64)))


# ----------------------------------------------------------------- metadata

def test_page_minmax_contains_and_attains(ora):
    """m <= k <= M for every valid token, and both ends are attained (the definition of min/max)."""
    L, S, D = 77, 16, 9
    K = _bf16(rng.normal(size=(L, D)))
    m, M = ora.page_minmax(K, S)
    assert m.shape == (5, D)
    for p in range(5):
        blk = K[p * S:min(p * S + S, L)]
        assert (blk >= m[p]).all() and (blk <= M[p]).all()
        assert ((blk == m[p]).any(axis=0)).all() and ((blk == M[p]).any(axis=0)).all()


def test_page_minmax_ignores_tokens_past_length(ora):
    """Only tokens < L count on the last page: garbage after L must not move m or M."""
    S, D = 16, 4
    K = _bf16(rng.normal(size=(40, D)))
    m1, M1 = ora.page_minmax(K[:37], S)
    K2 = K.copy()
    K2[37:] = 1e4
    m2, M2 = ora.page_minmax(K2[:37], S)
    assert (m1 == m2).all() and (M1 == M2).all()
    assert (M1[2] < 100).all()


def test_page_minmax_zero_sign(ora):
    """A page holding -0 and +0 in one channel stores +0 at both ends."""
    K = np.zeros((3, 2))
    K[0, 0] = -0.0
    K[1, 0] = 0.0
    K[2, 0] = -0.0
    K[:, 1] = [-0.0, -0.0, -0.0]
    m, M = ora.page_minmax(K, 16)
    assert not np.signbit(m).any() and not np.signbit(M).any()


def test_gather_and_meta_follow_page_table(ora):
    """Metadata of a permuted pool equals that of the contiguous pool, page for page."""
    a = synth.make_workload("tiny", seq_lens=(300,), permuted=False, n_needles=0)
    b = synth.make_workload("tiny", seq_lens=(300,), permuted=True, n_needles=0)
    assert not (a.page_table == b.page_table).all()
    for g in range(2):
        Ka = ora.gather_keys(a.k_pool, a.page_table, 0, g, 300)
        Kb = ora.gather_keys(b.k_pool, b.page_table, 0, g, 300)
        assert (Ka == Kb).all()
    ma = ora.build_meta(a.k_pool, a.page_table, a.seq_lens)
    mb = ora.build_meta(b.k_pool, b.page_table, b.seq_lens)
    for p in range(-(-300 // 16)):
        for g in range(2):
            x = ma[(int(a.page_table[0, p]), g)]
            y = mb[(int(b.page_table[0, p]), g)]
            assert (x[0] == y[0]).all() and (x[1] == y[1]).all()


# ----------------------------------------------------------------- Quest bound

def test_quest_bound_handworked(ora):
    c = GOLD["quest_bound"]
    U = ora.quest_bound(np.array(c["q"]), np.array(c["m"]), np.array(c["M"]))
    assert np.array_equal(U, np.array(c["U"]))
    assert np.array_equal(ora.group_score(U), np.array(c["group_score"]))


@pytest.mark.parametrize("seed", range(5))
def test_quest_bound_is_an_upper_bound(seed, ora):
    """max over a page's keys of q.k never exceeds the bound (brute force, every page and head)."""
    r = np.random.default_rng(seed)
    L, S, D, G = 200, 16, 32, 4
    K = _bf16(r.normal(size=(L, D)) * np.exp(0.5 * r.normal(size=D)))
    q = _bf16(r.normal(size=(G, D)))
    m, M = ora.page_minmax(K, S)
    U = ora.quest_bound(q, m, M)
    for p in range(m.shape[0]):
        blk = K[p * S:min(p * S + S, L)]
        dots = q @ blk.T                                   # [G][tokens]
        slack = 1e-12 * (np.abs(q) @ np.abs(blk).T).max()
        assert (dots.max(axis=1) <= U[:, p] + slack).all()


def test_quest_bound_tight_cases(ora):
    """Single-token page, or a page of identical keys: the bound equals q.k exactly."""
    r = np.random.default_rng(7)
    D, G = 16, 3
    q = _bf16(r.normal(size=(G, D)))
    k = _bf16(r.normal(size=(1, D)))
    m, M = ora.page_minmax(k, 16)
    assert np.allclose(ora.quest_bound(q, m, M)[:, 0], (q @ k.T)[:, 0], rtol=0, atol=1e-12)
    same = np.repeat(k, 16, axis=0)
    m, M = ora.page_minmax(same, 16)
    assert np.allclose(ora.quest_bound(q, m, M)[:, 0], (q @ k.T)[:, 0], rtol=0, atol=1e-12)


def test_quest_bound_closed_forms(ora):
    """K = 0 gives 0; q >= 0 elementwise gives q.M; q <= 0 gives q.m."""
    r = np.random.default_rng(8)
    D = 12
    z = np.zeros((1, D))
    q = _bf16(r.normal(size=(2, D)))
    assert (ora.quest_bound(q, z, z) == 0).all()
    m = _bf16(r.normal(size=(3, D)) - 1)
    M = m + np.abs(_bf16(r.normal(size=(3, D))))
    qp = np.abs(q)
    assert np.allclose(ora.quest_bound(qp, m, M), qp @ M.T, rtol=0, atol=1e-12)
    qn = -np.abs(q)
    assert np.allclose(ora.quest_bound(qn, m, M), qn @ m.T, rtol=0, atol=1e-12)


def test_group_score_bounds_every_head(ora):
    """The group score bounds q_h . k for every head of the group and every key of the page."""
    r = np.random.default_rng(9)
    L, S, D, G = 96, 16, 16, 8
    K = _bf16(r.normal(size=(L, D)))
    q = _bf16(r.normal(size=(G, D)))
    m, M = ora.page_minmax(K, S)
    s = ora.group_score(ora.quest_bound(q, m, M))
    for p in range(L // S):
        assert (q @ K[p * S:(p + 1) * S].T).max() <= s[p] + 1e-9


# ----------------------------------------------------------------- selection

def _rank_select(scores, pages, budget):
    """Brute force: a page is kept iff fewer than k pages beat it (higher score, or equal and lower id)."""
    k = min(budget, len(pages))
    keep = []
    for i in range(len(pages)):
        beaten = sum(1 for j in range(len(pages))
                     if scores[j] > scores[i] or (scores[j] == scores[i] and pages[j] < pages[i]))
        if beaten < k:
            keep.append(int(pages[i]))
    return sorted(keep)


def test_topk_handworked(ora):
    for case in ("topk", "topk_budget4"):
        c = GOLD[case]
        got = ora.select_topk(np.array(c["scores"]), np.array(c["pages"]), c["budget"])
        assert got.tolist() == c["selected"]


@pytest.mark.parametrize("seed", range(20))
def test_topk_matches_rank_bruteforce_with_ties(seed, ora):
    r = np.random.default_rng(seed)
    C = int(r.integers(1, 40))
    pages = np.sort(r.choice(200, size=C, replace=False)) + 3
    scores = r.choice([-1.5, 0.0, 2.25, 7.0], size=C).astype(np.float64)
    scores[scores == 0.0] = r.choice([0.0, -0.0], size=(scores == 0.0).sum())
    for budget in (0, 1, 2, C // 2, C - 1, C, C + 5):
        got = ora.select_topk(scores, pages, budget).tolist()
        assert got == _rank_select(scores, pages, budget)


def test_topk_all_equal_takes_first_candidates(ora):
    """With K = 0 every score is 0 and the tie rule picks the first k candidate ids."""
    wl = synth.make_workload("tiny", n_needles=0)
    wl.k_pool[:] = 0
    q, K, V = ora.unit_inputs(wl, 0, 0)
    r = ora.sparse_decode_unit(q, K, V, 4096, wl.cfg, 16, wl.sm_scale)
    assert (r["scores"] == 0).all()
    assert r["selected"].tolist() == r["candidates"][:32].tolist()


def test_needle_pages_are_selected(ora):
    """Any page can be selected: every planted needle's page is in the selection."""
    wl = synth.make_workload("tiny")
    for g in range(wl.hkv):
        q, K, V = ora.unit_inputs(wl, 0, g)
        r = ora.sparse_decode_unit(q, K, V, 4096, wl.cfg, 16, wl.sm_scale)
        needle_pages = set((wl.needles[0] // 16).tolist())
        assert needle_pages <= set(r["selected"].tolist())


# ----------------------------------------------------------------- union of token sets

def test_mask_handworked(ora):
    c = GOLD["mask"]
    mask = ora.attended_mask(c["L"], c["prefix"], c["window"], c["S"], c["selected"])
    assert np.nonzero(mask)[0].tolist() == c["tokens"]
    assert ora.candidate_pages(c["L"], c["prefix"], c["window"], c["S"]).tolist() == c["candidates"]


@pytest.mark.parametrize("seed", range(10))
def test_mask_per_token_bruteforce_and_count(seed, ora):
    r = np.random.default_rng(seed)
    S = 16
    L = int(r.integers(1, 300))
    P, W = int(r.integers(0, 80)), int(r.integers(0, 120))
    cand = ora.candidate_pages(L, P, W, S)
    sel = sorted(r.choice(cand, size=min(len(cand), int(r.integers(0, 5))), replace=False).tolist()) if len(cand) else []
    mask = ora.attended_mask(L, P, W, S, sel)
    for t in range(L):
        expect = t < P or t >= L - W or (t // S) in sel
        assert mask[t] == expect
    # count closed form: prefix + window (disjoint part) + middle tokens of selected pages
    Pe, Ws = min(P, L), max(0, L - W)
    count = Pe + (L - max(Ws, Pe)) + sum(max(0, min(p * S + S, Ws) - max(p * S, Pe)) for p in sel)
    assert mask.sum() == count
    # every candidate page intersects the middle region, and no other page does
    for p in range(-(-L // S)):
        meets = max(p * S, Pe) < min(p * S + S, Ws)
        assert meets == (p in cand.tolist())


# ----------------------------------------------------------------- attention

def test_attend_handworked(ora):
    c = GOLD["attend"]
    out = ora.attend(np.array(c["q"]), np.array(c["K"]), np.array(c["V"]), np.ones(2, bool), math.log(3.0))
    assert np.allclose(out, np.array(c["out"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_attend_matches_torch_sdpa_float64(seed, ora):
    """Library routine: torch CPU scaled_dot_product_attention (float64) with a boolean mask."""
    r = np.random.default_rng(seed)
    G, L, D = 4, 130, 32
    q, K, V = r.normal(size=(G, D)), r.normal(size=(L, D)), r.normal(size=(L, D))
    mask = r.random(L) < 0.4
    mask[5] = True
    scale = 1 / math.sqrt(D)
    got = ora.attend(q, K, V, mask, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(K)[None, None].expand(1, G, L, D),
        torch.tensor(V)[None, None].expand(1, G, L, D),
        attn_mask=torch.tensor(mask)[None, None, None, :], scale=scale)[0, :, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attend_constant_v_and_equal_logits(ora):
    r = np.random.default_rng(3)
    G, L, D = 2, 50, 8
    q, K = r.normal(size=(G, D)), r.normal(size=(L, D))
    v = r.normal(size=D)
    mask = r.random(L) < 0.5
    out = ora.attend(q, K, np.tile(v, (L, 1)), mask, 0.3)
    assert np.allclose(out, np.tile(v, (G, 1)), rtol=0, atol=1e-14)
    V = r.normal(size=(L, D))
    out = ora.attend(q, np.zeros((L, D)), V, mask, 0.3)     # all logits 0: plain mean
    assert np.allclose(out, np.tile(V[mask].mean(axis=0), (G, 1)), rtol=0, atol=1e-13)


def test_full_budget_equals_dense_attention(ora):
    """Budget >= every page: the sparse step is dense attention (also torch SDPA)."""
    wl = synth.make_workload("tiny", budget=10**6)
    for g in range(wl.hkv):
        q, K, V = ora.unit_inputs(wl, 0, g)
        r = ora.sparse_decode_unit(q, K, V, 4096, wl.cfg, 16, wl.sm_scale)
        assert r["mask"].all()
        dense = ora.dense_decode_unit(q, K, V, wl.sm_scale)
        assert np.array_equal(r["out"], dense)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, :, None, :], torch.tensor(K)[None, None].expand(1, 4, 4096, 64),
            torch.tensor(V)[None, None].expand(1, 4, 4096, 64), scale=wl.sm_scale)[0, :, 0, :].numpy()
        assert np.allclose(dense, ref, rtol=1e-12, atol=1e-12)


def test_output_invariant_under_page_permutation(ora):
    a = synth.make_workload("tiny", permuted=False)
    b = synth.make_workload("tiny", permuted=True)
    for g in range(2):
        ra = ora.sparse_decode_unit(*ora.unit_inputs(a, 0, g), 4096, a.cfg, 16, a.sm_scale)
        rb = ora.sparse_decode_unit(*ora.unit_inputs(b, 0, g), 4096, b.cfg, 16, b.sm_scale)
        assert np.array_equal(ra["out"], rb["out"])
        assert np.array_equal(ra["selected"], rb["selected"])


def test_no_budget_is_prefix_plus_window(ora):
    """budget = 0: exactly the prefix and the window, checked against torch SDPA with that mask."""
    wl = synth.make_workload("tiny", budget=0)
    q, K, V = ora.unit_inputs(wl, 0, 1)
    r = ora.sparse_decode_unit(q, K, V, 4096, wl.cfg, 16, wl.sm_scale)
    assert len(r["selected"]) == 0
    mask = np.zeros(4096, bool)
    mask[:64] = True
    mask[4096 - 256:] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(K)[None, None].expand(1, 4, 4096, 64),
        torch.tensor(V)[None, None].expand(1, 4, 4096, 64),
        attn_mask=torch.tensor(mask)[None, None, None, :], scale=wl.sm_scale)[0, :, 0, :].numpy()
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- pins of the decode of bf16, the
# selection margin and the query-head grouping

def _value(expr: str) -> float:
    """Value of a fixture expression such as '2^-133' or '(2 - 2^-7) * 2^127'."""
    return float(eval(expr.replace("^", "**"), {"__builtins__": {}}, {"inf": math.inf}))


def test_bf16_decode_fixed_patterns(ora):
    """Bit patterns whose values the bf16 format defines (sign, 8-bit exponent, 7-bit fraction)."""
    pats = json.load(open(os.path.join(GOLDEN, "bf16_patterns.json")))["patterns"]
    bits = np.array([int(b, 16) for b, _, _ in pats], dtype=np.uint16)
    got = ora.bf16_to_f64(bits)
    for (b, expr, _), v in zip(pats, got):
        want = _value(expr)
        assert v == want and math.copysign(1.0, v) == math.copysign(1.0, want), (b, v, want)
    # and as a whole pool: every decoded key equals the pattern's value, page table applied
    wl = synth.make_workload("tiny", seq_lens=(40,), n_needles=0)
    wl.k_pool[:] = 0x3F80
    wl.k_pool[wl.page_table[0, 1], 1, 3, 5] = 0xC020
    K = ora.gather_keys(wl.k_pool, wl.page_table, 0, 1, 40)
    assert K[16 + 3, 5] == -2.5 and (np.delete(K.reshape(-1), (16 + 3) * 64 + 5) == 1.0).all()


def test_selection_margin_handworked(ora):
    c = GOLD["selection_margin"]
    for scores in (c["scores"], c["shuffled"]):
        for budget, want in c["cases"]:
            got = ora.selection_margin(np.array(scores), budget)
            want = math.inf if want == "inf" else want
            assert got == pytest.approx(want, rel=1e-15, abs=0), (scores, budget)
    for budget, want in c["negative_cases"]:
        assert ora.selection_margin(np.array(c["negative_scores"]), budget) == pytest.approx(want, rel=1e-15)


def _head_group_workload():
    c = GOLD["head_groups"]
    wl = synth.workloads.build(name="heads", seed=0, batch=1, hq=4, hkv=2, d=2, seq_lens=(2,), prefix=0, window=0,
                               budget=1)
    wl.q[0] = synth.f64_to_bf16_bits(np.array(c["q"]))
    for g in range(2):
        wl.k_pool[wl.page_table[0, 0], g, :2, :] = synth.f64_to_bf16_bits(np.array(c["keys"]))
    return wl, c


def test_query_heads_map_to_contiguous_groups(ora):
    """Query head h reads KV head h / G: a group whose heads are all zero scores exactly 0."""
    wl, c = _head_group_workload()
    for g in range(2):
        q, K, V = ora.unit_inputs(wl, 0, g)
        r = ora.sparse_decode_unit(q, K, V, 2, wl.cfg, 16, wl.sm_scale)
        assert r["scores"].tolist() == [c["group_scores"][g]], g
    if hasattr(ora, "decode_units"):  # the C++ oracle's path from the pool, used by the GPU parity tests
        r = ora.decode_units(wl, [(0, 0), (0, 1)])
        assert r["scores"][:, 0].tolist() == c["group_scores"]
