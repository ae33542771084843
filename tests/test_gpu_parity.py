"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bar (float16 output of a float32-accumulated sum):
    |gpu - oracle| <= 1e-3 * sum_k |a*sfa*b*sfb| + 1 fp16 ulp(oracle)
with the float16 overflow edge handled by oracle.check. Decode of every E2M1
and E4M3 code, the hand cases and the sign flip are checked bit-exactly (all
partial sums there are exact in float32). Plain and blocked scale layouts must
give bit-identical outputs.
"""
import json
import os

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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = ["plain", "blocked"]


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def parity(inp, layout, **kw):
    got = run(DeviceInputs(inp), layout, **kw)
    ref = oracle.gemv(inp, layout)
    rep = oracle.check_report(got, ref)
    assert rep == "", f"{inp.w.name} [{layout}]\n{rep}"
    return got, ref


def bits_equal(x, y):
    return np.array_equal(np.asarray(x, np.uint16), np.asarray(y, np.uint16))


# ---------------------------------------------------------------- decode, bit-exact

@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_every_e2m1_code_of_a(layout):
    # row m: a single nonzero element k = 0 with code m; b = 1, scales = 1
    a = np.zeros((1, 16, 32), np.uint8)
    a[0, :, 0] = np.arange(16)
    inp = synth.from_codes(a, np.full((1, 32), 2, np.uint8), np.full((1, 16, 2), 0x38, np.uint8),
                           np.full((1, 2), 0x38, np.uint8))
    got, ref = parity(inp, layout)
    assert bits_equal(got, ref.c)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_every_e2m1_code_of_b(layout):
    # batch l: b has code l at k = 5; a = 1 everywhere; scales = 1
    b = np.zeros((16, 32), np.uint8)
    b[:, 5] = np.arange(16)
    inp = synth.from_codes(np.full((16, 4, 32), 2, np.uint8), b,
                           np.full((16, 4, 2), 0x38, np.uint8), np.full((16, 2), 0x38, np.uint8))
    got, ref = parity(inp, layout)
    assert bits_equal(got, ref.c)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_every_e4m3_code_of_sfa(layout):
    # row m: scale code m on block 0 (NaN codes give NaN rows)
    a = np.zeros((1, 256, 32), np.uint8)
    a[0, :, 3] = 2
    sfa = np.full((1, 256, 2), 0x38, np.uint8)
    sfa[0, :, 0] = np.arange(256)
    inp = synth.from_codes(a, np.full((1, 32), 2, np.uint8), sfa, np.full((1, 2), 0x38, np.uint8))
    got, ref = parity(inp, layout)
    fin = ~np.isnan(ref.value)
    assert bits_equal(got[fin], ref.c[fin])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_every_e4m3_code_of_sfb(layout):
    # batch l: b's scale code l on block 1
    L = 256
    a = np.zeros((L, 2, 32), np.uint8)
    a[:, :, 20] = 2
    sfb = np.full((L, 2), 0x38, np.uint8)
    sfb[:, 1] = np.arange(256)
    inp = synth.from_codes(a, np.full((L, 32), 2, np.uint8), np.full((L, 2, 2), 0x38, np.uint8), sfb)
    got, ref = parity(inp, layout)
    fin = ~np.isnan(ref.value)
    assert bits_equal(got[fin], ref.c[fin])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_positions_pair_with_their_b_and_scales(layout):
    # row m is one-hot at k = m (a = 1); b and both scales vary with k, so any
    # mix-up of element order, nibble order or scale block shows
    M = K = 128
    a = np.zeros((1, M, K), np.uint8)
    a[0, np.arange(M), np.arange(K)] = 2
    b = (np.arange(K) % 15 + 1).astype(np.uint8).reshape(1, K)
    sfa = (0x30 + np.arange(M * K // 16) % 16).astype(np.uint8).reshape(1, M, K // 16)
    sfb = (0x28 + 3 * np.arange(K // 16) % 24).astype(np.uint8).reshape(1, K // 16)
    inp = synth.from_codes(a, b, sfa, sfb)
    got, ref = parity(inp, layout)
    assert bits_equal(got, ref.c)


# ---------------------------------------------------------------- hand cases

HAND = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_hand_cases_bit_exact(case, layout):
    inp = synth.from_codes(np.array(case["a_codes"], np.uint8).reshape(1, 1, 32),
                           np.array(case["b_codes"], np.uint8).reshape(1, 32),
                           np.array(case["sfa"], np.uint8).reshape(1, 1, 2),
                           np.array(case["sfb"], np.uint8).reshape(1, 2))
    got = run(DeviceInputs(inp), layout)
    assert float(oracle.fp16_bits_to_double(got)[0, 0]) == float(case["fp16"])


# ---------------------------------------------------------------- workloads

MAIN = [synth.TINY, synth.BALANCED, synth.BATCHED, synth.HEADLINE, synth.SHARD]


@pytest.mark.parametrize("w", MAIN, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1])
def test_workloads_full_size(w, seed):
    inp = synth.make_inputs(w, 0, seed)
    dev = DeviceInputs(inp)
    outs = {}
    for layout in LAYOUTS:
        got = run(dev, layout)
        ref = oracle.gemv(inp, layout)
        rep = oracle.check_report(got, ref)
        assert rep == "", f"{w.name} seed {seed} [{layout}]\n{rep}"
        outs[layout] = got
    assert bits_equal(outs["plain"], outs["blocked"]), "layout changed the arithmetic"


@pytest.mark.parametrize("w", synth.EDGE, ids=lambda w: w.name)
def test_edge_sweep(w):
    inp = synth.make_inputs(w)
    dev = DeviceInputs(inp)
    outs = {}
    for layout in LAYOUTS:
        got = run(dev, layout)
        ref = oracle.gemv(inp, layout)
        rep = oracle.check_report(got, ref)
        assert rep == "", f"{w.name} [{layout}]\n{rep}"
        outs[layout] = got
    assert bits_equal(outs["plain"], outs["blocked"])


ODD = [(1, 32, 1), (2, 64, 3), (31, 96, 2), (33, 160, 1), (129, 2080, 2), (300, 4128, 1),
       (1, 16384, 1), (5, 32768, 1), (257, 7168, 2), (64, 224, 5), (1000, 1024, 1), (3, 4096, 7),
       (64, 65536, 1), (300, 20480, 2),
       # the multi-row kernel: ragged M and K, a partial last copy of SFA lines
       (6017, 2048, 1), (7168, 96, 1), (8100, 1056, 1), (2000, 3104, 3),
       # K-splits whose chunk count does not divide evenly: the slices start on
       # 4-block groups (an odd chunk count per slice once read the wrong pairs)
       (102, 55872, 2), (90, 46272, 1)]


@pytest.mark.parametrize("M,K,L", ODD)
@pytest.mark.parametrize("dist", ["uniform", "edge"])
def test_odd_shapes(M, K, L, dist):
    inp = synth.random_inputs(M, K, L, seed=M + K + L, dist=dist)
    for layout in LAYOUTS:
        parity(inp, layout)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("w", [synth.TINY, synth.EDGE[8], synth.BALANCED], ids=lambda w: w.name)
def test_sign_flip_negates_bit_exact(w):
    inp = synth.make_inputs(w)
    flipped = synth.Inputs(inp.w, inp.a ^ np.uint8(0x88), inp.b, inp.sfa_plain, inp.sfb_plain,
                           inp.sfa_blocked, inp.sfb_blocked)
    x = oracle.fp16_bits_to_double(run(DeviceInputs(inp), "blocked"))
    y = oracle.fp16_bits_to_double(run(DeviceInputs(flipped), "blocked"))
    np.testing.assert_array_equal(y, -x)


@pytest.mark.parametrize("M,K,L", [(7168, 16384, 1), (127, 65536, 3), (1000, 4096, 1)])
def test_deterministic(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=3)
    dev = DeviceInputs(inp)
    first = run(dev, "blocked")
    for _ in range(3):
        assert bits_equal(run(dev, "blocked"), first)


def test_batch_slices_match_single_batch_calls():
    inp = synth.make_inputs(synth.Workload("slices", 1000, 4096, 3, "uniform", 9))
    full = run(DeviceInputs(inp), "blocked")
    for l in range(3):
        one = synth.from_codes(synth.unpack_nibbles(inp.a[l:l + 1]), synth.unpack_nibbles(inp.b[l:l + 1]),
                               inp.sfa_plain[l:l + 1], inp.sfb_plain[l:l + 1])
        got = run(DeviceInputs(one), "blocked")
        ref = oracle.gemv(one, "blocked")
        assert oracle.check(got, ref).all()
        pa, pb = g.nvfp4_gemv_plan(1000, 4096, 3), g.nvfp4_gemv_plan(1000, 4096, 1)
        same_kernel = all(pa[k] == pb[k] for k in ("threads_per_wg", "lanes_per_row"))
        if pa["k_splits"] == pb["k_splits"] == 1 and same_kernel:
            assert bits_equal(got[0], full[l])      # same per-row summation order
        else:
            assert oracle.check(full[l:l + 1], ref).all()


# ---------------------------------------------------------------- entry points and streams

@pytest.mark.parametrize("M,K,L", [(16, 32768, 1), (127, 65536, 3), (1000, 16384, 3), (7168, 2048, 4), (5, 32768, 2)])
def test_ex_with_own_workspace_matches_default(M, K, L):
    inp = synth.random_inputs(M, K, L, seed=11)
    dev = DeviceInputs(inp)
    want = run(dev, "blocked")
    ws = zeroed_workspace(M, K, L)
    for _ in range(2):            # second call checks the counters were reset
        assert bits_equal(run(dev, "blocked", workspace=ws), want)
    if ws is not None:
        # the same workspace serves a smaller shape afterwards
        small = synth.random_inputs(33, 8192, 1, seed=12)
        assert g.nvfp4_gemv_workspace_bytes(33, 8192, 1) <= ws.numel()
        parity(small, "plain", workspace=ws)


def test_non_default_stream():
    inp = synth.random_inputs(1000, 4096, 2, seed=13)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run(DeviceInputs(inp), "blocked", stream=s)
    assert oracle.check(got, oracle.gemv(inp, "blocked")).all()


def test_invalid_arguments_launch_nothing():
    inp = synth.make_inputs(synth.TINY)
    dev = DeviceInputs(inp)
    c = torch.zeros(128, dtype=torch.float16, device="cuda")
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_gemv(dev.a, dev.b, dev.sfa["plain"], dev.sfb["plain"], c, 128, 255, 1, "plain")
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_gemv(dev.a, dev.b, dev.sfa["plain"], dev.sfb["plain"], c, 128, 256, 1, 7)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
