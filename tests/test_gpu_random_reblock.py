"""GPU: the random reblock shapes of test_random_reblock_bounds.py (CPU
mirror first), byte for byte against the oracle, from an aligned and from an
unaligned plain buffer."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from test_gpu_reblock import gpu_reblock  # noqa: E402
from test_random_reblock_bounds import SHAPES  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


@pytest.mark.parametrize("rows,K,L", SHAPES)
@pytest.mark.parametrize("offset", [0, 4])
def test_random_reblock_matches_oracle(rows, K, L, offset):
    plain = np.random.default_rng(rows * K + L + offset).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    np.testing.assert_array_equal(gpu_reblock(plain, rows, K, L, offset), oracle.reblock(plain, rows, K, L))
