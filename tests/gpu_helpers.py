"""Helpers for the GPU parity tests: drive the HIP path through the binding and
compare with the oracle.  Imported only by tests marked ``gpu``."""

from __future__ import annotations

import numpy as np
import torch

from hybrid_model_ssm_amd import replayssm as rs

DEV = "cuda"


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    rs.lib()  # fail loudly when the HIP library was not built


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def fp32_violation(got, ref, rel=1e-4):
    """Largest ratio |got - ref| / (rel * (1 + |ref|)); <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / (rel * (1.0 + np.abs(ref))))) if ref.size else 0.0


def assert_fp32_close(got, ref, what="", rel=1e-4):
    v = fp32_violation(got, ref, rel)
    assert v <= 1.0, f"{what}: max |d|/({rel}(1+|ref|)) = {v:.3g}"


def rms_violation(got, ref, rel=2e-2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / (rel * rms))


class GpuMamba2:
    """The replay path on the GPU for one layer, with ping-pong cursors."""

    def __init__(self, desc: rs.Mamba2Desc, static, lowp=False, ckpt=None):
        self.desc = desc
        ck = to_dev(static.ckpt, torch.float32) if ckpt is None else ckpt
        self.state = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=ck)
        self.A = to_dev(static.A, torch.float32)
        self.D = to_dev(static.D, torch.float32)
        self.dt_bias = to_dev(static.dt_bias, torch.float32)
        B = desc.batch
        self.cur = [torch.zeros(B, dtype=torch.int32, device=DEV), torch.zeros(B, dtype=torch.int32, device=DEV)]
        self.flip = 0
        self.out = torch.empty(B, desc.nheads, desc.headdim, dtype=torch.float32, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        if lowp:
            self.flush()

    @property
    def cursor(self):
        return self.cur[self.flip]

    def inputs(self, s):
        io = self.desc.torch_io
        return [to_dev(s[k], io) for k in ("x", "z", "B", "C", "dt_raw")]

    def step(self, s):
        x, z, B, C, dt = self.inputs(s)
        rs.mamba2_decode(self.desc, self.state, self.cur[self.flip], self.cur[1 - self.flip], x, z, B, C, dt,
                         self.dt_bias, self.A, self.D, self.out, self.err)
        self.flip ^= 1
        return self.out

    def flush(self):
        rs.mamba2_flush(self.desc, self.state, self.cur[self.flip], self.cur[1 - self.flip], self.A, self.err)
        self.flip ^= 1


class GpuConventional:
    def __init__(self, desc: rs.Mamba2Desc, static):
        self.desc = desc
        self.state = to_dev(static.ckpt, torch.float32)
        self.A = to_dev(static.A, torch.float32)
        self.D = to_dev(static.D, torch.float32)
        self.dt_bias = to_dev(static.dt_bias, torch.float32)
        self.out = torch.empty(desc.batch, desc.nheads, desc.headdim, dtype=torch.float32, device=DEV)

    def step(self, s):
        io = self.desc.torch_io
        x, z, B, C, dt = [to_dev(s[k], io) for k in ("x", "z", "B", "C", "dt_raw")]
        rs.selective_state_update(self.desc, self.state, x, z, B, C, dt, self.dt_bias, self.A, self.D, self.out)
        return self.out


def degenerate_gdn_gates(s, t):
    """Set gates at their limits, by value head, in one step's (or round's) inputs in place:
    head 0 alpha = 0 (the state is cleared), head 1 alpha = 1e-4 (the product of a
    window's gates falls below the smallest fp32 number), head 2 alpha = 1 (no decay),
    head 3 beta = 0 (nothing is written), head 4 alpha = 1e-4 on odd t only."""
    al, be = s["alpha"], s["beta"]
    al[..., 0] = 0.0
    al[..., 1] = 1e-4
    al[..., 2] = 1.0
    be[..., 3] = 0.0
    if t % 2:
        al[..., 4] = 1e-4
    return s


def extreme_mamba2_dt(s, t):
    """Set dt inputs at their extremes, by head, in one step's (or round's) inputs in place:
    head 0 dt_raw = 60 (dt ~ 60: the window's decay exp(A sum dt) underflows to 0 in
    fp32), head 1 dt_raw = -60 (dt ~ 1e-26: no update, no decay), head 2 alternates the
    two by t, head 3 dt_raw = 30.  All four values are exact in bf16."""
    dt = s["dt_raw"]
    dt[..., 0] = 60.0
    dt[..., 1] = -60.0
    dt[..., 2] = 60.0 if t % 2 else -60.0
    dt[..., 3] = 30.0
    return s
