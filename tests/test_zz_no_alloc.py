"""The allocation-free decode step (fsa_sparse_decode_attn_noalloc) against
fsa_sparse_decode_attn with a caller-owned workspace: two calls in a row, the
second on a smaller input, each bit for bit equal to the workspace call (same
kernels, same plan), and the first also checked against the oracle."""
import numpy as np
import pytest
import torch

import free_sparse_attention_amd as fsa
import oracle
import synth
from tests.gpu_harness import DeviceWorkload, bf16_f64, bits

pytestmark = pytest.mark.gpu
S = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fsa.load()


def _both(dw):
    wl = dw.wl
    c = dw.cfg()
    out_ws, sel_ws = dw.sparse()
    out_na = torch.full_like(out_ws, float("nan"))
    sel_na = torch.full_like(sel_ws, -7)
    fsa.sparse_decode_attn_noalloc(dw.dims, c, wl.sm_scale, dw.max_seq_len, dw.q, dw.k_cache, dw.v_cache, dw.meta,
                                   dw.page_table, dw.seq_lens, out_na, sel_na)
    torch.cuda.synchronize()
    return out_ws, sel_ws, out_na, sel_na


def test_noalloc_equals_workspace_call_twice_second_smaller():
    big = synth.workloads.build(name="noalloc_big", seed=31, batch=4, hq=16, hkv=4, d=128,
                                seq_lens=(20000, 17777, 12345, 20000), prefix=128, window=1024, budget=64,
                                k_sigma=0.5, n_needles=8, permuted=True)
    small = synth.workloads.build(name="noalloc_small", seed=32, batch=2, hq=8, hkv=2, d=64, seq_lens=(3000, 1111),
                                  prefix=32, window=256, budget=16, k_sigma=0.5, n_needles=4, permuted=True)
    for wl in (big, small):
        print(f"[noalloc] {wl.name} B={wl.batch} L={wl.seq_lens.tolist()}", flush=True)
        dw = DeviceWorkload(wl)
        out_ws, sel_ws, out_na, sel_na = _both(dw)
        assert np.array_equal(bits(out_na), bits(out_ws)), wl.name
        assert torch.equal(sel_na, sel_ws), wl.name
        # and the result is the method's: unit (0, 0) against the oracle on the GPU's selection
        q, K, V = oracle.unit_inputs(wl, 0, 0)
        L = int(wl.seq_lens[0])
        sel = [int(p) for p in sel_na[0, 0].cpu().numpy() if p >= 0]
        ref = oracle.attend(q, K, V, oracle.attended_mask(L, wl.cfg[0], wl.cfg[1], S, sel), wl.sm_scale)
        got = bf16_f64(out_na)[0, :wl.group]
        assert (np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref)).all()


def test_noalloc_rejects_a_step_beyond_its_scratch():
    d = fsa.dims(64, 64, 8, 128, 32768, 64 * 32768)
    need = fsa.sparse_decode_workspace_bytes(d, fsa.cfg(128, 1024, 128), 32768 * 16)
    assert need > fsa.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    i = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(fsa.FsaError, match="allocation-free"):
        fsa.sparse_decode_attn_noalloc(d, fsa.cfg(128, 1024, 128), 0.1, 32768 * 16, t, t, t, t, i, i, t, None)
