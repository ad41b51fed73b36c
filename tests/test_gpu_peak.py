"""The sustained-rate probe behind the roofline report's measured ceiling:
it runs on the device, writes its sink, and agrees with itself."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("fp8", [0, 1])
def test_peak_mfma_runs_and_is_deterministic(fp8):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(3)
    codes = torch.randint(-128, 128, (262144,), dtype=torch.int8, generator=g)
    codes[(codes == 127) | (codes == -1)] = 1
    ops = codes.to(dev)
    blocks = 8
    sinks = []
    for _ in range(2):
        sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
        pkg.llmint8_peak_mfma(fp8, ops.data_ptr(), ops.numel(), sink.data_ptr(), sink.numel() * 4,
                              blocks, 3, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        sinks.append(sink.cpu())
    assert torch.equal(sinks[0], sinks[1])
    assert (sinks[0] != 0).float().mean() > 0.5
