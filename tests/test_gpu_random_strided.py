"""GPU: the random strided cases of test_random_strided_bounds.py (whose CPU
mirrors walk the same launches) through nvfp4_gemv_strided: bit-identical to
the dense call, the gaps of the output untouched, within the oracle's
tolerance (the checks of test_gpu_strided.py)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from test_gpu_strided import test_strided_equals_dense as strided_equals_dense  # noqa: E402
from test_random_strided_bounds import CASES  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


@pytest.mark.parametrize("M,K,L,layout,over", CASES)
def test_random_strided_equals_dense(M, K, L, layout, over):
    strided_equals_dense(M, K, L, layout, over)
