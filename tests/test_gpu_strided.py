"""GPU parity of strided operands (nvfp4_gemv_strided).

Each operand is embedded in a larger device buffer at the positions its
strides name; the gaps hold codes that would change the result if read (A/B
code 0x77, scale 0x7F = NaN) and the output gaps hold a canary. The strided
call must equal the dense call on the same values bit for bit (the launch plan
depends only on M, K, L), match the oracle, and leave every gap untouched.
Batch stride 0 broadcasts one batch: the reference then repeats batch 0.
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
from test_kernel_bounds import STRIDED, strided  # noqa: E402

C_CANARY = 0xFFFF


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def embed(rows_per_batch, row_bytes, L, batch_stride, row_stride, fill):
    """A host buffer with row r of batch l at l*batch_stride + r*row_stride,
    plus the (l, r) -> offset map; rows_per_batch * row_bytes dense bytes each."""
    extent = (L - 1) * batch_stride + (rows_per_batch - 1) * row_stride + row_bytes
    buf = np.full(extent + 64, fill, np.uint8)
    return buf


def place(buf, dense, batch_stride, row_stride):
    """Copy dense [L][rows][row_bytes] into buf at the strided positions."""
    L, rows, rb = dense.shape
    for l in range(L):
        for r in range(rows):
            o = l * batch_stride + r * row_stride
            buf[o:o + rb] = dense[l, r]


def broadcast_batch0(inp, sd, layout):
    """Inputs whose operands with batch stride 0 repeat batch 0 in every batch."""
    w = inp.w
    a = synth.unpack_nibbles(inp.a)
    b = synth.unpack_nibbles(inp.b)
    sfa, sfb = inp.sfa_plain.copy(), inp.sfb_plain.copy()
    if sd["a_batch"] == 0:
        a[:] = a[0]
    if sd["b_batch"] == 0:
        b[:] = b[0]
    if sd["sfa_batch"] == 0:
        sfa[:] = sfa[0]
    if sd["sfb_batch"] == 0:
        sfb[:] = sfb[0]
    return synth.from_codes(a, b, sfa, sfb, name=w.name)


@pytest.mark.parametrize("M,K,L,layout,over", STRIDED)
def test_strided_equals_dense(M, K, L, layout, over):
    lay = "blocked" if layout else "plain"
    sd = strided(M, K, L, layout, **over)
    inp = broadcast_batch0(synth.random_inputs(M, K, L, seed=M + K, dist="edge"), sd, layout)
    dense_bits = run(DeviceInputs(inp), lay)
    nkb = K // 16
    # A and B
    a_host = embed(M, K // 2, L, sd["a_batch"], sd["a_row"], 0x77)
    place(a_host, inp.a.reshape(L, M, K // 2), sd["a_batch"], sd["a_row"])
    b_host = embed(1, K // 2, L, sd["b_batch"], 0, 0x77)
    place(b_host, inp.b.reshape(L, 1, K // 2), sd["b_batch"], 0)
    # scales
    if layout:
        per_a = inp.sfa_blocked.shape[-1]
        sfa_host = embed(1, per_a, L, sd["sfa_batch"], 0, 0x7F)
        place(sfa_host, inp.sfa_blocked.reshape(L, 1, per_a), sd["sfa_batch"], 0)
        per_b = inp.sfb_blocked.shape[-1]
        sfb_host = embed(1, per_b, L, sd["sfb_batch"], 0, 0x7F)
        place(sfb_host, inp.sfb_blocked.reshape(L, 1, per_b), sd["sfb_batch"], 0)
    else:
        sfa_host = embed(M, nkb, L, sd["sfa_batch"], sd["sfa_row"], 0x7F)
        place(sfa_host, inp.sfa_plain.reshape(L, M, nkb), sd["sfa_batch"], sd["sfa_row"])
        sfb_host = embed(1, nkb, L, sd["sfb_batch"], 0, 0x7F)
        place(sfb_host, inp.sfb_plain.reshape(L, 1, nkb), sd["sfb_batch"], 0)
    dev = [torch.from_numpy(x).to("cuda") for x in (a_host, b_host, sfa_host, sfb_host)]
    c_len = (L - 1) * sd["c_batch"] + M
    c = torch.full((c_len + 64,), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    ws = zeroed_workspace(M, K, L)
    g.nvfp4_gemv_strided(*dev, c, M, K, L, lay, sd, workspace=ws)
    torch.cuda.synchronize()
    bits = c.cpu().view(torch.int16).numpy().view(np.uint16)
    got = np.stack([bits[l * sd["c_batch"]:l * sd["c_batch"] + M] for l in range(L)])
    assert np.array_equal(got, dense_bits), "strided result differs from the dense call"
    mask = np.ones(bits.size, bool)
    for l in range(L):
        mask[l * sd["c_batch"]:l * sd["c_batch"] + M] = False
    assert np.all(bits[mask] == C_CANARY), "write outside the strided output rows"
    assert oracle.check(got, oracle.gemv(inp, lay)).all()


def test_pages_harness_b_padding():
    """B as the pages' harness hands it: N padded to 128 rows per batch."""
    M, K, L = 4096, 7168, 8
    inp = synth.random_inputs(M, K, L, seed=3)
    b128 = np.zeros((L, 128, K // 2), np.uint8)
    b128[:, 0] = inp.b.reshape(L, K // 2)
    sd = g.nvfp4_gemv_dense_strides(M, K, L, "blocked")
    sd["b_batch"] = 128 * (K // 2)
    dev = DeviceInputs(inp)
    c = torch.empty(L * M, dtype=torch.float16, device="cuda")
    g.nvfp4_gemv_strided(dev.a, torch.from_numpy(b128).to("cuda"), dev.sfa["blocked"], dev.sfb["blocked"],
                         c, M, K, L, "blocked", sd)
    torch.cuda.synchronize()
    got = c.cpu().view(torch.int16).numpy().view(np.uint16).reshape(L, M)
    assert np.array_equal(got, run(dev, "blocked"))


def test_invalid_strides_launch_nothing():
    inp = synth.make_inputs(synth.TINY)
    dev = DeviceInputs(inp)
    c = torch.zeros(128, dtype=torch.float16, device="cuda")
    sd = g.nvfp4_gemv_dense_strides(128, 256, 1, "plain")
    sd["a_row"] = 100
    with pytest.raises(g.Nvfp4Error) as e:
        g.nvfp4_gemv_strided(dev.a, dev.b, dev.sfa["plain"], dev.sfb["plain"], c, 128, 256, 1, "plain", sd)
    assert e.value.status == g.NVFP4_ERR_INVALID_STRIDE
    torch.cuda.synchronize()
    assert torch.all(c == 0)
