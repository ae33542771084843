"""GPU: the library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed. Every replay, with eager calls and synchronisations between the
replays, gives the eager call's output bit for bit (the kernels are
deterministic); a replay reads the inputs as they are at replay time; and the
split-K tickets, which the kernels reset themselves, leave later eager calls
correct. Covers the main GEMV kernel (one and several batches), the row and
wide-row kernels, the split-K path through the library's workspace and through
the allocation-free scratch array, the skinny GEMM's kernels and the reblock.
The library's one-time set-up (workspace allocation, scratch clear) happens in
the eager calls before the capture."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_gemv_amd as g  # noqa: E402
from gpu_util import DeviceInputs, to_dev  # noqa: E402
from test_oracle_small_n import inputs as small_n_inputs  # noqa: E402

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def bits(t):
    torch.cuda.synchronize()
    return t.cpu().view(torch.int16).numpy().view(np.uint16).copy()


def poison(t):
    t.view(torch.int16).fill_(-1)        # 0xFFFF: an output the replay does not write stays NaN


def capture(fn):
    """fn() once on a side stream (as torch asks before a capture), then
    captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def check_replays(graph, out, want, eager_between):
    for _ in range(REPLAYS):
        poison(out)
        graph.replay()
        assert np.array_equal(bits(out), want), "a replay differs from the eager call"
        eager_between()


# main kernel (one batch; several batches, b's inputs first), row kernel,
# wide-row kernel, split-K, tiny
GEMV_SHAPES = [(1000, 16384, 1), (7168, 2048, 4), (1000, 4096, 1), (127, 16384, 3), (64, 65536, 1),
               (128, 256, 1)]


@pytest.mark.parametrize("M,K,L", GEMV_SHAPES)
@pytest.mark.parametrize("entry", ["default", "noalloc"])
def test_gemv_graph_replays(M, K, L, entry):
    layout = "blocked"
    call = g.nvfp4_gemv if entry == "default" else g.nvfp4_gemv_noalloc
    inp0 = synth.random_inputs(M, K, L, seed=41, dist="edge")
    inp1 = synth.random_inputs(M, K, L, seed=42, dist="edge")
    d0, d1 = DeviceInputs(inp0), DeviceInputs(inp1)
    c = torch.empty(L * M, dtype=torch.float16, device="cuda")
    c1 = torch.empty_like(c)

    def gemv(d, out):
        call(d.a, d.b, d.sfa[layout], d.sfb[layout], out, M, K, L, layout)

    poison(c)
    gemv(d0, c)
    want0 = bits(c)
    rep = oracle.check_report(want0.reshape(L, M), oracle.gemv(inp0, layout))
    assert rep == "", rep
    poison(c1)
    gemv(d1, c1)
    want1 = bits(c1)

    graph = capture(lambda: gemv(d0, c))

    def eager_between():
        poison(c1)
        gemv(d1, c1)
        assert np.array_equal(bits(c1), want1), "an eager call between replays differs"

    check_replays(graph, c, want0, eager_between)
    # new contents in the captured input buffers: the replay reads them
    for dst, src in ((d0.a, d1.a), (d0.b, d1.b), (d0.sfa[layout], d1.sfa[layout]),
                     (d0.sfb[layout], d1.sfb[layout])):
        dst.copy_(src)
    poison(c)
    graph.replay()
    assert np.array_equal(bits(c), want1), "the replay did not read the new inputs"


# streamed matrix-core kernel (N = 4, 128 workgroups), up-front kernel (N = 3,
# 384 workgroups), two vectors through the GEMV kernel
SMALL_N = [(4096, 4, 4096, 1), (4096, 3, 2048, 3), (1000, 2, 4096, 3)]


@pytest.mark.parametrize("M,N,K,L", SMALL_N)
def test_small_n_graph_replays(M, N, K, L):
    def dev_operands(seed):
        a, b, sfa, sfb = small_n_inputs(M, N, K, L, seed)
        return [to_dev(x) for x in (a, b, synth.to_blocked(sfa), synth.to_blocked(sfb))]

    ops0, ops1 = dev_operands(51), dev_operands(52)
    c = torch.empty(L * N * M, dtype=torch.float16, device="cuda")
    c1 = torch.empty_like(c)

    def gemm(ops, out):
        g.nvfp4_gemm_small_n(*ops, out, M, N, K, L, "blocked")

    poison(c)
    gemm(ops0, c)
    want0 = bits(c)
    poison(c1)
    gemm(ops1, c1)
    want1 = bits(c1)

    graph = capture(lambda: gemm(ops0, c))

    def eager_between():
        poison(c1)
        gemm(ops1, c1)
        assert np.array_equal(bits(c1), want1)

    check_replays(graph, c, want0, eager_between)
    for dst, src in zip(ops0, ops1):
        dst.copy_(src)
    poison(c)
    graph.replay()
    assert np.array_equal(bits(c), want1), "the replay did not read the new inputs"


@pytest.mark.parametrize("rows,K,L", [(7168, 16384, 1), (7168, 2048, 4)])
def test_reblock_graph_replays(rows, K, L):
    rng = np.random.default_rng(rows + K + L)
    p0 = rng.integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    p1 = rng.integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    d0, d1 = to_dev(p0), to_dev(p1)
    nbytes = g.nvfp4_blocked_scales_bytes(rows, K, L)
    out = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    want0 = oracle.reblock(p0, rows, K, L).reshape(-1)
    want1 = oracle.reblock(p1, rows, K, L).reshape(-1)

    graph = capture(lambda: g.nvfp4_scales_to_blocked(d0, out, rows, K, L))
    for _ in range(REPLAYS):
        out.fill_(0xAB)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want0)
        scratch = torch.empty_like(out)
        g.nvfp4_scales_to_blocked(d1, scratch, rows, K, L)
        torch.cuda.synchronize()
        assert np.array_equal(scratch.cpu().numpy(), want1)
    d0.copy_(d1)
    out.fill_(0xAB)
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want1)
