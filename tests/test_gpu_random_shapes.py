"""GPU parity on seeded random shapes across the plan's branches (the shapes
of test_random_shapes_bounds.py, whose CPU mirrors walk the same grids):
both scale layouts against the oracle, within the tolerance, and plain and
blocked bit-identical."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DeviceInputs, run  # noqa: E402
from test_random_shapes_bounds import SHAPES  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


@pytest.mark.parametrize("M,K,L", SHAPES)
def test_random_shape_parity(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=M * 7 + K + L, dist="edge")
    dev = DeviceInputs(inp)
    outs = {}
    for layout in ("plain", "blocked"):
        got = run(dev, layout)
        rep = oracle.check_report(got, oracle.gemv(inp, layout))
        assert rep == "", f"{M}x{K}x{L} [{layout}]\n{rep}"
        outs[layout] = got
    assert np.array_equal(outs["plain"], outs["blocked"])
