"""The streaming-read reference (nvfp4_stream_read, a measurement helper) runs
through the C ABI on the GPU, touches only its sink, and leaves the sink alone
for data whose lane sums cannot hit the sink's trigger constant."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402


@pytest.mark.parametrize("nbytes", [256 * 1024, 8 * 2 ** 20, 66060288])
def test_stream_read_runs_and_keeps_sink(nbytes):
    src = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    src[nbytes:] = 0xAB                                   # bytes past the read range
    sink = torch.full((256 + 64,), -1, dtype=torch.int32, device="cuda")
    g.nvfp4_stream_read(src, nbytes, sink[:256])
    torch.cuda.synchronize()
    assert bool((sink == -1).all())                       # zero data never triggers a sink write
    assert bool((src[nbytes:] == 0xAB).all()) and bool((src[:nbytes] == 0).all())


def test_stream_read_rejects_bad_size():
    src = torch.zeros(2 ** 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_stream_read(src, 1000, sink)
