"""The streaming-read reference of the bench (libnvfp4bench.so, a measurement
helper outside the GEMV library) runs on the GPU in each read design, touches
only its sink, and leaves the sink alone for zero data."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_scaled_fp4_gemv_amd import benchlib  # noqa: E402


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("units", [1, 2, 15])
def test_stream_read_runs_and_keeps_sink(mode, units):
    nbytes = units * benchlib.stream_read_unit(mode)
    src = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    src[nbytes:] = 0xAB                                   # bytes past the read range
    sink = torch.full((256 + 64,), -1, dtype=torch.int32, device="cuda")
    benchlib.stream_read(src, nbytes, sink[:256], mode)
    torch.cuda.synchronize()
    assert bool((sink == -1).all())                       # zero data never triggers a sink write
    assert bool((src[nbytes:] == 0xAB).all()) and bool((src[:nbytes] == 0).all())


def test_stream_read_rejects_bad_arguments():
    src = torch.zeros(8 * 2 ** 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        benchlib.stream_read(src, 1000, sink, 0)
    with pytest.raises(RuntimeError):
        benchlib.stream_read(src, benchlib.stream_read_unit(0), sink, 7)
