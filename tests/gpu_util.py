"""Helpers shared by the GPU parity tests: moving seeded cases to the device
through the library's own packing, and comparing with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

# output tolerance, relative to max|y_ref| over the compared outputs
TOL = {O.F16: 2e-3, O.BF16: 5e-3}


def note(msg: str):
    """Print a progress line that reaches the terminal even under capture."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def torch_dtype(dt):
    import torch
    return torch.float16 if dt == O.F16 else torch.bfloat16


def bits_to_device(bits, dt, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch_dtype(dt))


def device_to_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceCase:
    """A synth.Case packed by libw4a16's host packing and uploaded."""

    def __init__(self, case, device="cuda:0"):
        import torch
        import int4_weight_only_linear_amd as L
        self.case = case
        self.wq_host = L.w4a16_pack_weights(case.q)
        self.zpk_host = None if case.zp is None else L.w4a16_pack_zeros(case.zp)
        self.wq = torch.from_numpy(self.wq_host).to(device)
        self.zp = None if self.zpk_host is None else torch.from_numpy(self.zpk_host).to(device)
        self.s = bits_to_device(case.s_bits, case.dtype, device)
        self.x = bits_to_device(case.x_bits, case.dtype, device)
        self.bias = None if case.bias_bits is None else bits_to_device(case.bias_bits, case.dtype, device)

    def set_x(self, x_bits, device="cuda:0"):
        self.case.x_bits = x_bits
        self.case.M = x_bits.shape[0]
        self.x = bits_to_device(x_bits, self.case.dtype, device)

    def run(self, path=0, out=None) -> np.ndarray:
        import torch
        import int4_weight_only_linear_amd as L
        y = L.w4a16_linear_path(self.x, self.wq, self.s, self.zp, self.bias,
                                group_size=self.case.group, path=path, out=out)
        torch.cuda.synchronize()
        return device_to_bits(y)


def oracle_rows(case, rows=None) -> np.ndarray:
    """Oracle y for all rows, or for the given 8-aligned row blocks (float64)."""
    c = case
    if rows is None:
        zpk = None if c.zp is None else O.pack_zeros(c.zp)
        return O.linear_ref(c.x_bits, O.pack_weights(c.q), c.s_bits, zpk, c.bias_bits,
                            c.M, c.N, c.K, c.group, c.dtype)
    rows = np.asarray(rows)
    zpk = None if c.zp is None else O.pack_zeros(c.zp[rows])
    bias = None if c.bias_bits is None else c.bias_bits[rows]
    return O.linear_ref(c.x_bits, O.pack_weights(c.q[rows]), c.s_bits[rows], zpk, bias,
                        c.M, len(rows), c.K, c.group, c.dtype)


def sample_rows(N: int, seed=0, blocks: int = 2) -> np.ndarray:
    """The first and last 16 rows plus a few random 8-row blocks (8-aligned)."""
    rng = np.random.default_rng(seed)
    starts = {0, 8, max(0, N - 16), max(0, N - 8)}
    nb = N // 8
    for b in rng.choice(nb, size=min(blocks, nb), replace=False):
        starts.add(int(b) * 8)
    rows = sorted({r for s in starts for r in range(s, min(s + 8, N))})
    return np.array(rows)


def assert_close(y_bits, ref64, dt, what=""):
    y = O.act_bits_to_f64(y_bits, dt)
    assert y.shape == ref64.shape, (y.shape, ref64.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    scale = float(np.abs(ref64).max())
    err = float(np.abs(y - ref64).max())
    bound = TOL[dt] * scale
    assert err <= bound, f"{what}: max|dy| = {err:.4g} > {bound:.4g} (= {TOL[dt]} * {scale:.4g})"
    return err / scale if scale else 0.0
