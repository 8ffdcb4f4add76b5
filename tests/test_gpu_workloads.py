"""GPU parity at the full sizes of the studied decode workloads, in the launch
configuration the benchmark times, against the C++ oracle.

* batch-4 decode at 64k context: every (sequence, KV head) unit, sparse and dense;
* batch-4 decode at 256k context, permuted pool, GQA 8: every unit, sparse and dense;
* the 12-layer sweep at 128k (per-layer prefix/window/budget): every unit's
  metadata, scores, selection and work list in every layer, outputs of every
  unit, the dense kernel on two units per layer; plus the dense check (budget =
  all pages equals full attention);
* the ragged 16-sequence serving batch: 64 steps of one-token append followed by
  a decode with a fresh query.  After every append the incrementally kept
  metadata equals a fresh rebuild bit for bit; at six steps (the last among
  them) every one of the 128 units is checked against the oracle (metadata,
  scores, selection, work list and output).
Every case prints the share of the output tolerance it uses.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_harness import DeviceWorkload, bf16_f64, to_dev_bf16
from tests.test_gpu_parity import S, check_out, run_and_check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_ctx64k_all_units():
    wl = synth.make_workload("ctx64k")
    dw, out, sel = run_and_check(wl)
    for b in range(wl.batch):          # planted needles are found for every KV head
        pages = set((wl.needles[b] // S).tolist())
        for g in range(wl.hkv):
            assert len(pages & set(sel[b, g].tolist())) >= 0.9 * len(pages)


def test_ctx256k_all_units():
    wl = synth.make_workload("ctx256k")
    run_and_check(wl)


@pytest.mark.parametrize("layer", range(12))
def test_sweep12_layer(layer):
    wl = synth.make_workload("sweep12", layer=layer)
    run_and_check(wl, dense_units=[(layer % 4, (layer // 4) % 4), ((layer + 2) % 4, 3)])


def test_sweep12_dense_check():
    """budget = all pages: the sparse step equals full attention (GPU dense kernel and oracle)."""
    wl = synth.make_workload("sweep12", layer=5)
    n = -(-int(wl.seq_lens.max()) // S)
    cfg = (wl.cfg[0], wl.cfg[1], n)
    dw, out, sel = run_and_check(wl, cfg=cfg)
    dense = bf16_f64(dw.dense())
    check_out(out, dense, "sparse(all pages) vs dense")


def test_ragged16_append_decode_64_steps():
    import free_sparse_attention_amd as fsa
    wl = synth.make_workload("ragged16")
    say(f"[ragged16] lengths {wl.seq_lens.tolist()}")
    dw = DeviceWorkload(wl)
    lens = torch.from_numpy(wl.seq_lens.copy()).cuda()
    lens2 = torch.empty_like(lens)
    rebuilt = torch.zeros_like(dw.meta)
    check_steps = {0, 13, 27, 40, 52, 63}
    kk, kv, _ = wl.keys()
    for step in range(64):
        L0 = lens.cpu().numpy()
        kn = np.empty((wl.batch, 1, wl.hkv, wl.d), np.uint16)
        vn = np.empty_like(kn)
        for b in range(wl.batch):
            kn[b] = synth.core.fill_tokens(kk, b, int(L0[b]), 1, wl.hkv, wl.d, wl.k_scale)
            vn[b] = synth.core.fill_tokens(kv, b, int(L0[b]), 1, wl.hkv, wl.d, None)
            t = int(L0[b])
            phys = wl.page_table[b, t // S]
            wl.k_pool[phys, :, t % S, :] = kn[b, 0]
            wl.v_pool[phys, :, t % S, :] = vn[b, 0]
        fsa.append_kv(dw.dims, 1, to_dev_bf16(kn), to_dev_bf16(vn), dw.page_table, lens, lens2, dw.k_cache,
                      dw.v_cache, dw.meta)
        lens, lens2 = lens2, lens
        dw.seq_lens = lens
        wl.seq_lens = (L0 + 1).astype(np.int32)
        dw.max_seq_len = int(wl.seq_lens.max())
        rebuilt.zero_()
        fsa.build_page_meta(dw.dims, dw.k_cache, dw.page_table, lens, rebuilt)
        assert torch.equal(rebuilt, dw.meta), f"incremental metadata differs from a rebuild at step {step}"
        q = wl.step_q(step)
        if step in check_steps:
            say(f"[ragged16] step {step}: decode parity")
            run_and_check(wl, q=q, dense=False, dw=dw, label=f"ragged16 step {step}")
        else:
            out, _ = dw.sparse(q=to_dev_bf16(q))
    torch.cuda.synchronize()
