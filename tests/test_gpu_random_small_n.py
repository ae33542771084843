"""GPU parity of the N-vector GEMM on the seeded random shapes of
test_random_small_n_bounds.py (whose CPU mirrors walk the same grids), both
scale layouts against the oracle (N independent GEMVs) within the tolerance."""
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from test_gpu_small_n import run_small_n  # noqa: E402
from test_oracle_small_n import inputs  # noqa: E402
from test_random_small_n_bounds import SHAPES  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


@pytest.mark.parametrize("M,N,K,L", SHAPES)
def test_random_small_n_parity(M, N, K, L):
    a, b, sfa, sfb = inputs(M, N, K, L, 3 * M + N + K + L)
    ref = oracle.gemm_small_n(a, b, sfa, sfb, M, N, K, L)
    for layout in ("plain", "blocked"):
        got = run_small_n(a, b, sfa, sfb, M, N, K, L, layout)
        rep = oracle.check_report(got, ref)
        assert rep == "", f"{M}x{N}x{K}x{L} [{layout}]\n{rep}"
