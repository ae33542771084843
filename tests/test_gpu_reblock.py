"""GPU parity of the device reblock (nvfp4_scales_to_blocked) against the
oracle's reblock: byte-exact, padding zero, no byte written past the output,
for aligned and unaligned plain inputs; and the GEMV fed by device-reblocked
scales equals the GEMV on the plain scales bit for bit."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402
from gpu_util import DeviceInputs, run, to_dev  # noqa: E402

CANARY = 0xA5
TAIL = 256


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def gpu_reblock(plain, rows, K, L, offset=0):
    """Reblock on the GPU; plain placed `offset` bytes into its buffer."""
    n = plain.size
    buf = torch.zeros(n + offset, dtype=torch.uint8, device="cuda")
    buf[offset:] = to_dev(plain.reshape(-1))
    need = g.nvfp4_blocked_scales_bytes(rows, K, L)
    out = torch.full((need + TAIL,), CANARY, dtype=torch.uint8, device="cuda")
    g.nvfp4_scales_to_blocked(buf[offset:], out[:need], rows, K, L)
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    assert np.all(host[need:] == CANARY), "write past the end of the blocked buffer"
    return host[:need].reshape(L, -1)


SHAPES = [(1, 32, 1), (1, 96, 3), (1, 16384, 1), (127, 4096, 3), (128, 2048, 2), (129, 32, 1),
          (300, 4128, 1), (1000, 7168, 2), (7168, 2048, 4), (4096, 7168, 8), (7, 1056, 5),
          # 32 tiles per workgroup (ragged rows, a partial last tile group)
          (129, 8192, 32), (100, 15872, 64), (7168, 16384, 1)]


@pytest.mark.parametrize("rows,K,L", SHAPES)
def test_reblock_matches_oracle(rows, K, L):
    plain = np.random.default_rng(rows + K + L).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    got = gpu_reblock(plain, rows, K, L)
    np.testing.assert_array_equal(got, oracle.reblock(plain, rows, K, L))


@pytest.mark.parametrize("offset", [1, 2, 3])
@pytest.mark.parametrize("rows,K,L", [(127, 4096, 2), (300, 96, 1)])
def test_reblock_unaligned_plain(rows, K, L, offset):
    plain = np.random.default_rng(offset).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    got = gpu_reblock(plain, rows, K, L, offset)
    np.testing.assert_array_equal(got, oracle.reblock(plain, rows, K, L))


def test_reblock_headline_sfa():
    w = synth.HEADLINE
    inp = synth.make_inputs(w, 0)
    got = gpu_reblock(inp.sfa_plain, w.M, w.K, w.L)
    np.testing.assert_array_equal(got, synth.to_blocked(inp.sfa_plain, pad=0))


@pytest.mark.parametrize("M,K,L", [(1000, 4096, 3), (127, 16384, 1), (7168, 2048, 4)])
def test_gemv_on_device_reblocked_scales(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=31, dist="edge")
    dev = DeviceInputs(inp)
    want = run(dev, "plain")
    sfa_b = torch.empty(g.nvfp4_blocked_scales_bytes(M, K, L), dtype=torch.uint8, device="cuda")
    sfb_b = torch.empty(g.nvfp4_blocked_scales_bytes(1, K, L), dtype=torch.uint8, device="cuda")
    g.nvfp4_scales_to_blocked(dev.sfa["plain"], sfa_b, M, K, L)
    g.nvfp4_scales_to_blocked(dev.sfb["plain"], sfb_b, 1, K, L)
    dev.sfa["blocked"], dev.sfb["blocked"] = sfa_b, sfb_b
    got = run(dev, "blocked")
    assert np.array_equal(got, want)


def test_reblock_invalid_arguments_launch_nothing():
    out = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    src = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_scales_to_blocked(src, out, 1, 48, 1)
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_scales_to_blocked(src, out[1:], 1, 32, 1)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
