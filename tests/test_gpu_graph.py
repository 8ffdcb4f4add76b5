"""The append and the decode step are graph-capturable: they allocate,
memset and synchronise nothing.  A captured [append one token, decode] pair,
replayed several times with eager work in between, gives bit for bit the
results of the same calls run eagerly (the pair is idempotent: every replay
writes the same token at the same position).  The same holds for the combined
append + decode call."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import DeviceWorkload, bits, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(dw, kn, vn, lens_a, lens_b, out, sel, ws, msl, stream, combined):
    import free_sparse_attention_amd as fsa
    wl = dw.wl
    if combined:
        fsa.append_decode_attn(dw.dims, 1, kn, vn, lens_a, lens_b, dw.cfg(), wl.sm_scale, msl, dw.q, dw.k_cache,
                               dw.v_cache, dw.meta, dw.page_table, out, sel, ws, stream)
        return
    fsa.append_kv(dw.dims, 1, kn, vn, dw.page_table, lens_a, lens_b, dw.k_cache, dw.v_cache, dw.meta, stream)
    fsa.sparse_decode_attn(dw.dims, dw.cfg(), wl.sm_scale, msl, dw.q, dw.k_cache, dw.v_cache, dw.meta,
                           dw.page_table, lens_b, out, sel, ws, stream)


@pytest.mark.parametrize("combined", [False, True], ids=["separate", "combined"])
@pytest.mark.parametrize("lens", [(16384, 15000, 12001, 9999), (65536,) * 4])
def test_graph_replays_match_eager(lens, combined):
    wl = synth.make_workload("ctx64k", seq_lens=lens, extra_tokens=64)
    kk, kv, _ = wl.keys()
    kn = np.stack([synth.core.fill_tokens(kk, b, int(wl.seq_lens[b]), 1, wl.hkv, wl.d, wl.k_scale)
                   for b in range(wl.batch)])
    vn = np.stack([synth.core.fill_tokens(kv, b, int(wl.seq_lens[b]), 1, wl.hkv, wl.d, None)
                   for b in range(wl.batch)])
    kn, vn = to_dev_bf16(kn), to_dev_bf16(vn)
    msl = int(wl.seq_lens.max()) + 1

    def run(graph):
        dw = DeviceWorkload(wl)
        lens_a = dw.seq_lens
        lens_b = torch.empty_like(lens_a)
        out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.bfloat16, device="cuda")
        sel = torch.empty((wl.batch, wl.hkv, wl.cfg[2]), dtype=torch.int32, device="cuda")
        ws = dw.workspace(max_seq_len=msl)
        if not graph:
            _pair(dw, kn, vn, lens_a, lens_b, out, sel, ws, msl, torch.cuda.current_stream(), combined)
            torch.cuda.synchronize()
            return [(bits(out), sel.cpu().numpy(), lens_b.cpu().numpy(), bits(dw.meta))]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            _pair(dw, kn, vn, lens_a, lens_b, out, sel, ws, msl, s, combined)  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _pair(dw, kn, vn, lens_a, lens_b, out, sel, ws, msl, torch.cuda.current_stream(), combined)
        res = []
        for rep in range(3):
            out.zero_()
            sel.fill_(-9)
            g.replay()
            torch.cuda.synchronize()
            res.append((bits(out), sel.cpu().numpy(), lens_b.cpu().numpy(), bits(dw.meta)))
            # eager work between replays
            dense = dw.dense(max_seq_len=msl)
            torch.cuda.synchronize()
            assert torch.isfinite(dense.float()).all()
        return res

    ref = run(False)[0]
    for i, got in enumerate(run(True)):
        assert np.array_equal(got[0], ref[0]), f"replay {i}: output differs"
        assert np.array_equal(got[1], ref[1]), f"replay {i}: selection differs"
        assert np.array_equal(got[2], ref[2]), f"replay {i}: lengths differ"
        assert np.array_equal(got[3], ref[3]), f"replay {i}: metadata differs"
