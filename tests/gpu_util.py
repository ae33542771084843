"""Helpers for the GPU tests: move seeded inputs to the device, call the HIP
library through its C ABI (the Python binding), and read results back."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_fp4_gemv_amd as g

CANARY = 0xFFFF        # fp16 NaN pattern around / after the output
CANARY_TAIL = 64       # extra output elements that must stay untouched


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


class DeviceInputs:
    def __init__(self, inp):
        self.inp = inp
        self.a = to_dev(inp.a)
        self.b = to_dev(inp.b)
        self.sfa = {"plain": to_dev(inp.sfa_plain), "blocked": to_dev(inp.sfa_blocked)}
        self.sfb = {"plain": to_dev(inp.sfb_plain), "blocked": to_dev(inp.sfb_blocked)}


def run(dev: DeviceInputs, layout: str, workspace=None, stream=None, alpha=None) -> np.ndarray:
    """One GEMV call; returns the float16 bits [L][M]. Checks the canary tail.
    With ``alpha`` the call goes through nvfp4_gemv_scaled."""
    w = dev.inp.w
    n = w.L * w.M
    c = torch.empty(n + CANARY_TAIL, dtype=torch.float16, device="cuda")
    c.view(torch.int16).fill_(-1)          # 0xFFFF everywhere: unwritten outputs stay NaN
    c_out = c[:n]
    if alpha is not None:
        g.nvfp4_gemv_scaled(dev.a, dev.b, dev.sfa[layout], dev.sfb[layout], c_out, w.M, w.K, w.L,
                            layout, alpha, workspace, stream=stream)
    elif workspace is None:
        g.nvfp4_gemv(dev.a, dev.b, dev.sfa[layout], dev.sfb[layout], c_out, w.M, w.K, w.L,
                     layout, stream)
    else:
        g.nvfp4_gemv_ex(dev.a, dev.b, dev.sfa[layout], dev.sfb[layout], c_out, w.M, w.K, w.L,
                        layout, workspace, stream=stream)
    torch.cuda.synchronize()
    bits = c.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(bits[n:] == CANARY), "write past the end of c"
    return bits[:n].reshape(w.L, w.M).copy()


def zeroed_workspace(M: int, K: int, L: int) -> torch.Tensor | None:
    nbytes = g.nvfp4_gemv_workspace_bytes(M, K, L)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
