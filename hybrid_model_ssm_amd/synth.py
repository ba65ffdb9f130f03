"""Seeded synthetic inputs for the decode path.

This module is shared by the HIP path's callers (tests, bench) and by the CPU
oracle's callers.  It only draws random numbers and rounds them to the
precision the GPU receives; it holds none of the method's arithmetic.

Workloads (shapes of the pages' evaluation: batch 256, an FP32 state of up to
4 MiB per sequence per layer, window L = 16 -- "ReplaySSM Caches Inputs Instead
of State..." sections "Why SSM layers slow down hybrid models" and "Evaluation
and reported results"):

==================  ==========================================================
name                shape
==================  ==========================================================
mamba2_tiny         B=2, H=4, P=16, N=16, G=1, L=4, 64 steps, f32 inputs
mamba2_h64          B=256, H=64, P=64, N=128, G=8, L=16, 256 steps, bf16 io
mamba2_h128         B=256, H=128, P=64, N=128, G=8, L=16, 1024 steps, bf16 io
mamba2_spec_h128    as mamba2_h128; 256 rounds of 4 positions (3 drafts + 1)
gdn_hv32            B=256, HV=32, HK=16, dk=dv=128, L=16, 512 steps, bf16 io
==================  ==========================================================

Distributions (Mamba2): ``x, z ~ N(0,1)``; ``B, C ~ N(0,1)/sqrt(dstate)``;
``dt_raw ~ N(0,1)``; ``softplus(dt_bias) ~ U[1e-3, 1e-1]`` per head (so
``dt_bias = log(expm1(u))``); ``A = -exp(U[0, ln 16])``; ``D ~ N(0,1)``; initial
checkpoint ``~ N(0, 0.1^2)`` (standard deviation 0.1).

Distributions (GDN): ``q, k ~ N(0,1)`` L2-normalised in float32 and then
rounded; ``v ~ N(0,1)``; ``beta = sigmoid(N(0,1))``; ``alpha =
exp(-softplus(N(0,1) - 2))``; initial state ``~ N(0, 0.1^2)``.

Draw order is fixed: static parameters (A, D, dt_bias, checkpoint), then per
step ``x, z, B, C, dt_raw`` (speculative rounds: all positions of one round,
then the accepted-draft count ``k ~ U{0..T}`` of every sequence; GDN: ``q, k,
v, beta-logit, alpha-logit``).  bf16 rounding is round-to-nearest-even.
Arrays come back as float32 holding exactly the values the GPU receives; cast
with ``torch.from_numpy(a).to(torch.bfloat16)`` (exact for these values).
"""

from __future__ import annotations

import dataclasses

import numpy as np

WORKLOADS = {
    "mamba2_tiny": dict(kind="mamba2", batch=2, nheads=4, headdim=16, dstate=16, ngroups=1,
                        buffer_len=4, steps=64, io="f32", seed=1000),
    "mamba2_h64": dict(kind="mamba2", batch=256, nheads=64, headdim=64, dstate=128, ngroups=8,
                       buffer_len=16, steps=256, io="bf16", seed=1001),
    "mamba2_h128": dict(kind="mamba2", batch=256, nheads=128, headdim=64, dstate=128, ngroups=8,
                        buffer_len=16, steps=1024, io="bf16", seed=1002),
    "mamba2_spec_h128": dict(kind="mamba2_spec", batch=256, nheads=128, headdim=64, dstate=128,
                             ngroups=8, buffer_len=16, rounds=256, n_pos=4, io="bf16", seed=1003),
    "gdn_hv32": dict(kind="gdn", batch=256, num_v_heads=32, num_k_heads=16, dk=128, dv=128,
                     buffer_len=16, steps=512, io="bf16", seed=1004),
    "gdn_spec_hv32": dict(kind="gdn_spec", batch=256, num_v_heads=32, num_k_heads=16, dk=128, dv=128,
                          buffer_len=16, rounds=256, n_pos=4, io="bf16", seed=1005),
}


def round_bf16(a):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return out.reshape(a.shape)


def _io(a, io):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if io == "bf16" else a


@dataclasses.dataclass
class Mamba2Static:
    A: np.ndarray          # [H] f32, negative
    D: np.ndarray          # [H] f32
    dt_bias: np.ndarray    # [H] f32
    ckpt: np.ndarray       # [B,H,P,N] f32


class Mamba2Inputs:
    """Seeded Mamba2 decode inputs.  ``static`` is drawn at construction."""

    def __init__(self, batch, nheads, headdim, dstate, ngroups, io="bf16", seed=0,
                 ckpt_std=0.1, draw_ckpt=True):
        self.batch, self.nheads, self.headdim, self.dstate, self.ngroups = batch, nheads, headdim, dstate, ngroups
        self.io = io
        self.rng = np.random.Generator(np.random.PCG64(seed))
        rng = self.rng
        A = -np.exp(rng.uniform(0.0, np.log(16.0), size=nheads))
        D = rng.standard_normal(nheads)
        u = rng.uniform(1e-3, 1e-1, size=nheads)
        dt_bias = np.log(np.expm1(u))
        if draw_ckpt:
            ckpt = rng.standard_normal((batch, nheads, headdim, dstate), dtype=np.float32) * np.float32(ckpt_std)
        else:
            ckpt = np.zeros((batch, nheads, headdim, dstate), np.float32)
        self.static = Mamba2Static(A.astype(np.float32), D.astype(np.float32),
                                   dt_bias.astype(np.float32), ckpt.astype(np.float32))

    def step(self, n_pos=None):
        """One step's inputs (or one speculative round's, with a position axis after batch)."""
        rng = self.rng
        lead = (self.batch,) if n_pos is None else (self.batch, n_pos)
        H, P, N, G = self.nheads, self.headdim, self.dstate, self.ngroups
        x = rng.standard_normal(lead + (H, P), dtype=np.float32)
        z = rng.standard_normal(lead + (H, P), dtype=np.float32)
        s = np.float32(1.0 / np.sqrt(N))
        B = rng.standard_normal(lead + (G, N), dtype=np.float32) * s
        C = rng.standard_normal(lead + (G, N), dtype=np.float32) * s
        dt_raw = rng.standard_normal(lead + (H,), dtype=np.float32)
        return dict(x=_io(x, self.io), z=_io(z, self.io), B=_io(B, self.io), C=_io(C, self.io),
                    dt_raw=_io(dt_raw, self.io))

    def accepted(self, n_drafts):
        """Accepted draft count per sequence, ``k ~ U{0..n_drafts}``; keep ``k + 1`` positions."""
        return self.rng.integers(0, n_drafts + 1, size=self.batch).astype(np.int32)


@dataclasses.dataclass
class GDNStatic:
    ckpt: np.ndarray       # [B,HV,dv,dk] f32


class GDNInputs:
    def __init__(self, batch, num_v_heads, num_k_heads, dk, dv, io="bf16", seed=0, ckpt_std=0.1):
        self.batch, self.HV, self.HK, self.dk, self.dv = batch, num_v_heads, num_k_heads, dk, dv
        self.io = io
        self.rng = np.random.Generator(np.random.PCG64(seed))
        ckpt = self.rng.standard_normal((batch, num_v_heads, dv, dk), dtype=np.float32) * np.float32(ckpt_std)
        self.static = GDNStatic(ckpt.astype(np.float32))

    def step(self, n_pos=None):
        """One step's inputs (or one speculative round's, with a position axis after batch)."""
        rng = self.rng
        Bt, HV, HK, dk, dv = self.batch, self.HV, self.HK, self.dk, self.dv
        lead = (Bt,) if n_pos is None else (Bt, n_pos)
        q = rng.standard_normal(lead + (HK, dk), dtype=np.float32)
        k = rng.standard_normal(lead + (HK, dk), dtype=np.float32)
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal(lead + (HV, dv), dtype=np.float32)
        bl = rng.standard_normal(lead + (HV,))
        al = rng.standard_normal(lead + (HV,))
        beta = (1.0 / (1.0 + np.exp(-bl))).astype(np.float32)
        sp = np.log1p(np.exp(al - 2.0))
        alpha = np.exp(-sp).astype(np.float32)
        return dict(q=_io(q, self.io), k=_io(k, self.io), v=_io(v, self.io), alpha=alpha, beta=beta)

    def accepted(self, n_drafts):
        """Accepted draft count per sequence, ``k ~ U{0..n_drafts}``; keep ``k + 1`` positions."""
        return self.rng.integers(0, n_drafts + 1, size=self.batch).astype(np.int32)


def mamba2_inputs(name, **over):
    w = dict(WORKLOADS[name])
    w.update(over)
    return Mamba2Inputs(w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"],
                        io=w["io"], seed=w["seed"])


def gdn_inputs(name, **over):
    w = dict(WORKLOADS[name])
    w.update(over)
    return GDNInputs(w["batch"], w["num_v_heads"], w["num_k_heads"], w["dk"], w["dv"],
                     io=w["io"], seed=w["seed"])
