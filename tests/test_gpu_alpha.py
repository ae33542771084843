"""GPU parity of the global float32 scale (nvfp4_gemv_scaled) against the oracle.

c = fp16(alpha * sum): the kernel multiplies its float32 row sum by alpha and
rounds once more to float16, so the bar is the usual one,
    |gpu - oracle| <= 1e-3 * |alpha| * sum_k |a*sfa*b*sfb| + 1 fp16 ulp(oracle),
against the oracle's exactly rounded fp16(alpha * exact sum). alpha = 1 must
reproduce nvfp4_gemv bit for bit, alpha = -1 must negate it exactly, and a
power of two must shift it exactly wherever both values are normal float16.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402
from gpu_util import DeviceInputs, run, zeroed_workspace  # noqa: E402
from test_oracle_alpha import one_row_with_sum, sticky_case  # noqa: E402

LAYOUTS = ["plain", "blocked"]
SHAPES = [(128, 256, 1), (7168, 2048, 4), (127, 16384, 3), (1000, 4096, 1), (300, 4128, 1),
          (5, 32768, 2)]


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def bits_equal(x, y):
    return np.array_equal(np.asarray(x, np.uint16), np.asarray(y, np.uint16))


def parity_scaled(inp, layout, alpha, **kw):
    got = run(DeviceInputs(inp), layout, alpha=alpha, **kw)
    ref = oracle.gemv(inp, layout, alpha=alpha)
    rep = oracle.check_report(got, ref)
    assert rep == "", f"{inp.w.name} [{layout}] alpha={alpha}\n{rep}"
    return got


@pytest.mark.parametrize("M,K,L", SHAPES)
def test_alpha_one_matches_unscaled_bit_exact(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=21, dist="edge")
    dev = DeviceInputs(inp)
    for layout in LAYOUTS:
        assert bits_equal(run(dev, layout, alpha=1.0), run(dev, layout)), layout


@pytest.mark.parametrize("M,K,L", SHAPES[:4])
def test_alpha_minus_one_negates(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=22)
    dev = DeviceInputs(inp)
    x = run(dev, "blocked")
    y = run(dev, "blocked", alpha=-1.0)
    np.testing.assert_array_equal(oracle.fp16_bits_to_double(y), -oracle.fp16_bits_to_double(x))


@pytest.mark.parametrize("k", [-22, -9, -1, 3, 5])
def test_power_of_two_alpha_shifts_exactly(k):
    inp = synth.random_inputs(1000, 4096, 2, seed=23)
    dev = DeviceInputs(inp)
    x = oracle.fp16_bits_to_double(run(dev, "plain"))
    y = oracle.fp16_bits_to_double(run(dev, "plain", alpha=2.0 ** k))
    ok = (np.abs(x) >= 2.0 ** -14) & (np.abs(x) * 2.0 ** k >= 2.0 ** -14) & (np.abs(x) * 2.0 ** k <= 32768)
    assert ok.sum() > 100
    np.testing.assert_array_equal(y[ok], x[ok] * 2.0 ** k)
    parity_scaled(inp, "plain", 2.0 ** k)


@pytest.mark.parametrize("M,K,L", SHAPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_random_alpha_parity(M, K, L, layout):
    rng = np.random.default_rng(M + K + L)
    inp = synth.random_inputs(M, K, L, seed=24, dist="edge" if M % 2 else "uniform")
    for alpha in [float(np.float32(rng.uniform(-3, 3))), float(np.float32(1.7e-5)),
                  float(np.float32(-913.25))]:
        parity_scaled(inp, layout, alpha)


@pytest.mark.parametrize("w", [synth.BALANCED, synth.HEADLINE], ids=lambda w: w.name)
def test_full_size_scaled(w):
    inp = synth.make_inputs(w, 0, 3)
    parity_scaled(inp, "blocked", float(np.float32(0.0123)))


def test_alpha_zero_gives_zero():
    inp = synth.random_inputs(1000, 4096, 1, seed=25)
    got = oracle.fp16_bits_to_double(run(DeviceInputs(inp), "blocked", alpha=0.0))
    assert np.all(got == 0)


@pytest.mark.parametrize("top,tail", [(63, 1), (64, 5)])
def test_sticky_tie_rows(top, tail):
    # rows whose exact scaled value sits just above a float16 tie: the float32
    # path lands within tolerance of the oracle's exactly rounded value
    S, ma = sticky_case(top, tail)
    inp = one_row_with_sum(S)
    parity_scaled(inp, "plain", float(ma) * 2.0 ** -34)
    parity_scaled(inp, "blocked", float(ma) * 2.0 ** -34)


@pytest.mark.parametrize("M,K,L", [(16, 32768, 1), (5, 32768, 2)])
def test_scaled_with_own_workspace(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=26)
    dev = DeviceInputs(inp)
    want = run(dev, "blocked", alpha=0.75)
    ws = zeroed_workspace(M, K, L)
    assert ws is not None
    for _ in range(2):
        assert bits_equal(run(dev, "blocked", workspace=ws, alpha=0.75), want)
    parity_scaled(inp, "blocked", 0.75, workspace=ws)


@pytest.mark.parametrize("alpha", [float("nan"), float("inf")])
def test_non_finite_alpha_launches_nothing(alpha):
    inp = synth.make_inputs(synth.TINY)
    dev = DeviceInputs(inp)
    c = torch.zeros(128, dtype=torch.float16, device="cuda")
    with pytest.raises(g.Nvfp4Error) as e:
        g.nvfp4_gemv_scaled(dev.a, dev.b, dev.sfa["plain"], dev.sfb["plain"], c, 128, 256, 1,
                            "plain", alpha)
    assert e.value.status == g.NVFP4_ERR_INVALID_SCALE
    torch.cuda.synchronize()
    assert torch.all(c == 0)
