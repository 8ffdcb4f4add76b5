"""The measurement helpers run on the device: the plain-read probe over a
buffer, and the device's memory properties (checked against torch's view of
the same device)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_read_probe_and_device_memory():
    import free_sparse_attention_amd as fsa
    props = fsa.device_memory()
    assert props["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert props["memory_clock_khz"] > 0 and props["memory_bus_width_bits"] > 0
    for nbytes in (16, 4096 + 16 * 37, 64 << 20):  # one word, a ragged tail, many rounds of the grid
        buf = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        fsa.read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) in (0, 0x9E3779B9 - (1 << 32))
    with pytest.raises(fsa.FsaError):
        fsa.read_probe(torch.zeros(24, dtype=torch.uint8, device="cuda"), sink)


@pytest.mark.parametrize("cfg,batch,hkv,want", [((128, 1024, 128), 4, 4, "wide"), ((128, 1024, 300), 16, 8, "narrow"),
                                                ((64, 4096, 10**5), 2, 2, "dense")])
def test_launches_one_at_a_time_equal_the_step(cfg, batch, hkv, want):
    """Running the step's launches one by one (the benchmark's per-launch timing)
    gives bit for bit the output of the whole step, in each step plan."""
    import numpy as np

    import free_sparse_attention_amd as fsa
    import synth
    from tests.gpu_harness import DeviceWorkload, bits
    wl = synth.workloads.build(name="parts", seed=51, batch=batch, hq=4 * hkv, hkv=hkv, d=128,
                               seq_lens=tuple(9000 + 1111 * i for i in range(batch)), prefix=cfg[0], window=cfg[1],
                               budget=cfg[2], k_sigma=0.5, permuted=True)
    dw = DeviceWorkload(wl)
    plan = fsa.describe_step(dw.dims, dw.cfg(), dw.max_seq_len)["plan"]
    assert plan == want
    ws = dw.workspace()
    ref, _ = dw.sparse(ws=ws, want_sel=False)
    ref = bits(ref)
    out = torch.zeros((wl.batch, wl.hq, wl.d), dtype=torch.bfloat16, device="cuda")
    def run(first, last):
        return fsa.sparse_decode_attn_launches(dw.dims, dw.cfg(), wl.sm_scale, dw.max_seq_len, dw.q, dw.k_cache,
                                               dw.v_cache, dw.meta, dw.page_table, dw.seq_lens, out, None, ws, first,
                                               last)
    n = run(0, 0)
    for j in range(1, n):
        run(j, j)
    torch.cuda.synchronize()
    assert n == {"wide": 3, "narrow": 4, "dense": 2}[plan]
    assert np.array_equal(bits(out), ref)
    out.zero_()
    run(0, n - 2)  # a prefix, then the rest
    run(n - 1, n - 1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), ref)
