"""GPU test of nvfp4_gemv_noalloc, the entry point that allocates nothing: its
split-K workspace is the library's fixed per-device scratch array. Called
through the C ABI and compared with nvfp4_gemv (the library-owned, allocated
workspace) bit for bit, and with the oracle to the parity bar, on calls in a
row whose shapes shrink, so that the second call runs on scratch the first one
left behind. Runs alone in a fresh process and after the other GPU tests."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402
from gpu_util import CANARY, CANARY_TAIL, DeviceInputs, run  # noqa: E402


def run_noalloc(dev: DeviceInputs, layout: str) -> np.ndarray:
    w = dev.inp.w
    n = w.L * w.M
    c = torch.empty(n + CANARY_TAIL, dtype=torch.float16, device="cuda")
    c.view(torch.int16).fill_(-1)
    g.nvfp4_gemv_noalloc(dev.a, dev.b, dev.sfa[layout], dev.sfb[layout], c[:n], w.M, w.K, w.L, layout)
    torch.cuda.synchronize()
    bits = c.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(bits[n:] == CANARY), "write past the end of c"
    return bits[:n].reshape(w.L, w.M).copy()


def check(M, K, L, layout, seed, dist="uniform"):
    w = synth.Workload(f"noalloc_{M}x{K}x{L}", M, K, L, dist, 0)
    inp = synth.make_inputs(w, seed)
    dev = DeviceInputs(inp)
    got = run_noalloc(dev, layout)
    want = run(dev, layout)                               # nvfp4_gemv: allocated workspace
    assert np.array_equal(got, want), f"{w.name} [{layout}]: differs from nvfp4_gemv"
    rep = oracle.check_report(got, oracle.gemv(inp, layout))
    assert rep == "", f"{w.name} [{layout}]\n{rep}"


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def test_scratch_covers_every_split_workspace_of_these_shapes():
    cap = g.nvfp4_gemv_noalloc_scratch_bytes()
    for M, K, L in [(127, 65536, 3), (5, 32768, 2), (64, 65536, 1), (1, 1 << 22, 1), (121, 65536, 2)]:
        assert 0 < g.nvfp4_gemv_workspace_bytes(M, K, L) <= cap


@pytest.mark.parametrize("layout", ["blocked", "plain"])
def test_calls_in_a_row_shrinking(layout):
    # split-K shapes (they use the scratch array), the second one smaller, then
    # a larger one again and a shape without a K-split
    check(127, 65536, 3, layout, seed=1)
    check(5, 32768, 2, layout, seed=2, dist="edge")
    check(64, 65536, 1, layout, seed=3)
    check(1000, 4096, 1, layout, seed=4)


def test_invalid_arguments_launch_nothing():
    w = synth.Workload("noalloc_bad", 128, 256, 1, "uniform", 0)
    dev = DeviceInputs(synth.make_inputs(w, 0))
    c = torch.empty(128, dtype=torch.float16, device="cuda")
    lib = g.lib()
    assert lib.nvfp4_gemv_noalloc(None, dev.b.data_ptr(), dev.sfa["plain"].data_ptr(), dev.sfb["plain"].data_ptr(),
                                  c.data_ptr(), 128, 256, 1, 0, None) == g.NVFP4_ERR_NULL_POINTER
    assert lib.nvfp4_gemv_noalloc(dev.a.data_ptr(), dev.b.data_ptr(), dev.sfa["plain"].data_ptr(),
                                  dev.sfb["plain"].data_ptr(), c.data_ptr(), 128, 48, 1, 0,
                                  None) == g.NVFP4_ERR_INVALID_SHAPE
