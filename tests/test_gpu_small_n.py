"""GPU parity of the N-vector skinny GEMM (nvfp4_gemm_small_n) against the
oracle (N independent GEMVs), within the GEMV's tolerance per output; plain
and blocked scales give bit-identical results; the global scale applies;
outputs outside c are untouched."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402
from gpu_util import to_dev  # noqa: E402
from test_oracle_small_n import inputs  # noqa: E402

TAIL = 64


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def blocked_rows(plain):
    """Plain scales [L][rows][K/16] -> blocked bytes [L][per batch] (synth's view
    chain), padding bytes E4M3 NaN: a product that read one would show it."""
    return synth.to_blocked(plain)


def run_small_n(a, b, sfa, sfb, M, N, K, L, layout, alpha=1.0):
    c = torch.full((L * N * M + TAIL,), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    if layout == "blocked":
        sfa, sfb = blocked_rows(sfa), blocked_rows(sfb)
    g.nvfp4_gemm_small_n(to_dev(a), to_dev(b), to_dev(sfa), to_dev(sfb), c[:L * N * M], M, N, K, L, layout, alpha)
    torch.cuda.synchronize()
    bits = c.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(bits[L * N * M:] == 0xFFFF), "write past the end of c"
    return bits[:L * N * M].reshape(L, N, M)


CASES = [(1, 1, 32, 1), (7, 3, 96, 2), (128, 2, 2048, 1), (300, 4, 20480, 2), (1000, 8, 4096, 3),
         (7168, 8, 2048, 1), (129, 5, 16384, 1), (4096, 2, 7168, 2), (64, 7, 65536, 1),
         # N = 2 through the GEMV kernel (ragged M, several batches, segmented K),
         # and N = 2 where a K-split is needed (the skinny kernel)
         (1000, 2, 4096, 3), (300, 2, 20480, 2), (127, 2, 16384, 1),
         # matrix-core kernels over many batches, ragged M and K (a last step of
         # fewer than 4 chunks; no whole step at all for K = 96); blocked scales
         # with K <= 16384 take the staged kernel, plain scales and K > 16384 the
         # unstaged one
         (300, 4, 1056, 120), (100, 8, 160, 300), (33, 3, 96, 5),
         # 128-row blocks whose workgroups own no row below M, a single 4-block group
         (5, 3, 768, 2), (127, 5, 2304, 3), (300, 6, 4352, 1), (1, 8, 256, 1), (129, 7, 256, 2),
         (1000, 4, 7168, 2), (128, 4, 1280, 5), (20, 3, 64, 1), (7168, 3, 16384, 1),
         # N = 2 on the matrix-core kernels (blocked, K >= 4096, 128 workgroups or
         # more): streamed, up-front; and short rows through the GEMV kernel
         (4100, 2, 4224, 1), (2000, 2, 4224, 5), (4100, 2, 256, 1),
         # wide grids with a ragged last 128-row block, two batches
         (5000, 5, 1056, 1), (3000, 8, 4160, 2)]


@pytest.mark.parametrize("M,N,K,L", CASES)
def test_small_n_parity(M, N, K, L):
    a, b, sfa, sfb = inputs(M, N, K, L, M + N + K)
    ref = oracle.gemm_small_n(a, b, sfa, sfb, M, N, K, L)
    outs = {}
    for layout in ("plain", "blocked"):
        got = run_small_n(a, b, sfa, sfb, M, N, K, L, layout)
        rep = oracle.check_report(got, ref)
        assert rep == "", f"{layout}\n{rep}"
        outs[layout] = got
    # the same kernel runs for both layouts except for N = 2 with K >= 4096 and
    # 128 workgroups or more, where blocked scales take a matrix-core kernel and
    # plain scales the GEMV's
    if not (N == 2 and K >= 4096 and L * -(-M // 128) * 4 >= 128):
        assert np.array_equal(outs["plain"], outs["blocked"])


@pytest.mark.parametrize("N", [4, 2])
def test_small_n_alpha_and_edge_codes(N):
    M, K, L = 1000, 4096, 2
    inp = [synth.random_inputs(M, K, L, seed=60 + n, dist="edge") for n in range(N)]
    a = inp[0].a
    b = np.stack([x.b.reshape(L, K // 2) for x in inp], axis=1)
    sfa = inp[0].sfa_plain
    sfb = np.stack([x.sfb_plain for x in inp], axis=1)
    for alpha in (1.0, -0.375):
        ref = oracle.gemm_small_n(a, b, sfa, sfb, M, N, K, L, alpha=alpha)
        got = run_small_n(a, b, sfa, sfb, M, N, K, L, "blocked", alpha)
        assert oracle.check_report(got, ref) == ""


@pytest.mark.parametrize("M,N,K,L", [(7168, 8, 16384, 1), (7168, 4, 16384, 1), (4096, 4, 7168, 8),
                                     (7168, 2, 16384, 1)])
def test_small_n_headline_shape(M, N, K, L):
    """The bench's shapes (N = 4 and 8 on the headline A, the batched A): sampled
    rows of the first and last vector against the oracle."""
    a, b, sfa, sfb = inputs(M, N, K, L, 5)
    got = run_small_n(a, b, sfa, sfb, M, N, K, L, "blocked")
    rows = np.arange(0, M, 97)
    for n in (0, N - 1):
        ref = oracle.gemm_small_n(a[:, rows], b[:, n:n + 1], sfa[:, rows], sfb[:, n:n + 1], rows.size, 1, K, L)
        col = oracle.Result(ref.c[:, 0], ref.s_f64[:, 0], ref.s_abs[:, 0], ref.s_exact[:, 0], ref.nan[:, 0])
        assert oracle.check(got[:, n, rows], col).all()
