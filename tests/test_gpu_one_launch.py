"""The one-launch form of the wide plan against the separate launches.

Both forms run the same scoring, selection and prefix/window code, write the
same partial slots and merge them with the same arithmetic (combine_core.h),
so on the same inputs their outputs and selected pages must be bit-identical
(the separate launches are checked against the oracle by the other GPU
modules).  The form is off by default; here it is forced (mode 2), for unit
counts that are not multiples of 8 too.  Each case also checks that no wait of
the one-launch kernel was given up (the stall count stays zero), across more
calls than there are synchronisation slots, in a replayed HIP graph and
through the per-launch call.
"""
import sys

import numpy as np
import pytest
import torch

import free_sparse_attention_amd as fsa
import synth
from tests.gpu_harness import DeviceWorkload, bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fsa.load()
    yield
    fsa.set_one_launch(0)


def _need_256_cus():
    cus = fsa.device_memory()["compute_units"]
    if cus != 256:  # the one-launch form needs 8 XCDs of 32 CUs (MI355X as one partition)
        pytest.skip(f"the one-launch form needs a 256-CU device, this one has {cus}")


# (workload, overrides): units below, at and above one per XCD; G 4, 8 and 1;
# head dims 64 and 128; sequences without candidates; ragged lengths
CASES = {
    "tiny": ("tiny", {}),
    "b4_h4_ragged": ("ctx64k", dict(seq_lens=(16000, 21111, 9000, 30001))),
    "b4_g8_40k": ("ctx256k", dict(seq_lens=(40000, 36000, 47000, 52000), window=2048)),
    "b3_h2_d64": ("tiny", dict(batch=3, hq=8, hkv=2, seq_lens=(6000, 300, 8191), budget=24)),
    "b16_h4_64units": ("ctx64k", dict(batch=16, seq_lens=tuple(6000 + 700 * i for i in range(16)), budget=32,
                                      window=512)),
    "b2_h8_g1": ("tiny", dict(batch=2, hq=8, hkv=8, seq_lens=(9000, 12000), budget=16)),
}


def _both(dw, cfg=None):
    """(out bits, selected pages) of the one-launch and of the separate-launch form."""
    res = []
    for mode in (2, 0):
        fsa.set_one_launch(mode)
        desc = fsa.describe_step(dw.dims, dw.cfg(cfg), dw.max_seq_len)
        out, sel = dw.sparse(cfg=cfg)
        torch.cuda.synchronize()
        res.append((desc, bits(out), None if sel is None else sel.cpu().numpy()))
    fsa.set_one_launch(0)
    return res


@pytest.mark.parametrize("case", list(CASES))
def test_one_launch_equals_separate_launches(case):
    _need_256_cus()
    name, over = CASES[case]
    wl = synth.make_workload(name, **over)
    dw = DeviceWorkload(wl)
    say(f"[one-launch] {case}: B={wl.batch} Hq={wl.hq} Hkv={wl.hkv} D={wl.d} lens={list(wl.seq_lens)} cfg={wl.cfg}")
    before = fsa.one_launch_stalls()
    (d1, o1, s1), (d0, o0, s0) = _both(dw)
    assert d1["plan"] == "wide" and d1["one_launch"] == 1 and d1["score_tasks"] >= 1, d1
    assert d0["one_launch"] == 0
    assert np.array_equal(o1, o0), f"{case}: outputs differ"
    if s1 is not None:
        assert np.array_equal(s1, s0), f"{case}: selected pages differ"
    assert fsa.one_launch_stalls() == before


def test_slots_reused_graph_replays_and_launches_one_at_a_time():
    _need_256_cus()
    wl = synth.make_workload("ctx64k", seq_lens=(12000, 15000, 9000, 20000))
    dw = DeviceWorkload(wl)
    before = fsa.one_launch_stalls()
    fsa.set_one_launch(1)  # 16 units: mode 1 applies
    assert fsa.describe_step(dw.dims, dw.cfg(), dw.max_seq_len)["one_launch"] == 1
    ws = dw.workspace()
    out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.bfloat16, device="cuda")
    ref, _ = dw.sparse(ws=ws, want_sel=False)
    ref = bits(ref)
    # more calls in a row than there are synchronisation slots
    for i in range(80):
        dw.sparse(ws=ws, out=out, want_sel=False)
        if i % 20 == 19:
            torch.cuda.synchronize()
            assert np.array_equal(bits(out), ref), f"call {i}"
    # a captured step, replayed with eager steps and synchronisations between replays
    stream = torch.cuda.Stream()
    gout = torch.zeros_like(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        dw.sparse(ws=ws, out=gout, want_sel=False)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fsa.sparse_decode_attn(dw.dims, dw.cfg(), wl.sm_scale, dw.max_seq_len, dw.q, dw.k_cache, dw.v_cache,
                                   dw.meta, dw.page_table, dw.seq_lens, gout, None, ws, stream)
    for r in range(4):
        gout.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(gout), ref), f"replay {r}"
        dw.sparse(ws=ws, out=out, want_sel=False)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref)
    # the step's launches issued one call at a time
    n = fsa.sparse_decode_attn_launches(dw.dims, dw.cfg(), wl.sm_scale, dw.max_seq_len, dw.q, dw.k_cache, dw.v_cache,
                                        dw.meta, dw.page_table, dw.seq_lens, out, None, ws, 0, 0)
    assert n == 1
    out.zero_()
    for j in range(n):
        fsa.sparse_decode_attn_launches(dw.dims, dw.cfg(), wl.sm_scale, dw.max_seq_len, dw.q, dw.k_cache,
                                        dw.v_cache, dw.meta, dw.page_table, dw.seq_lens, out, None, ws, j, j)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), ref)
    fsa.set_one_launch(0)
    assert fsa.one_launch_stalls() == before
