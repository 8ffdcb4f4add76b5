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
