#!/usr/bin/env python3
"""Decode throughput of the ReplaySSM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--only headline]

Headline (``value``): Mamba2 replay decode, one layer, B=256, H=128, P=64, N=128,
G=8, L=16, bf16 inputs, fp32 checkpoint reads -- seq-tokens/s = batch * K / time
for exactly K timed decode steps (one kernel launch each, flushes included at their
true rate of one step in L).  Inputs sit in HBM before the timed region: a pool of
2L pre-drawn steps is cycled.  ``roofline`` gives the replay kernel's algorithmic
HBM bytes per launch divided by its average launch time (HIP events on the launch
stream) against the 8 TB/s peak; ``traffic`` is the counter-measured HBM bytes per
launch from the committed rocprofv3 summary when it matches the current kernel
source, else null.  ``cpu_baseline`` times the fp64 CPU oracle (replay form) on a
sample of the same workload, its sequences sharded over worker processes on the host's
cores (forked before the GPU is touched), and checks the GPU outputs for that sample.

Measured beside the headline, each with its own timed region: the in-library
conventional read-update-write kernel on the same inputs, the headline steps captured
as a graph and replayed, the bf16, fp16 and fp8 read
copies, the state-and-output decode route, the B=256/H=64 layer, speculative
verification (4 positions, commit) against the per-position snapshot baseline, and the
Gated DeltaNet layer (replay decode and conventional; speculative verification against
its snapshot baseline).  ``ceiling`` reports plain device read and copy bandwidth.

Auxiliary modes used to make the committed rocprofv3 summaries:
    --calibrate-copy        also run a plain 1 GiB device copy (counter calibration)
    --pmc-summarize FETCH_DIR WRITE_DIR  turn two rocprofv3 --pmc runs into a summary
    --stats-summarize STATS_DIR          turn a rocprofv3 --kernel-trace --stats run into a summary
    --precision-sweep       output error of emulated read and recurrence precisions
                            (bf16, fp16, fp8) against fp32, over 1024 steps
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Mamba2 decode seq-tokens/s at B=256, L=16 + achieved HBM GB/s vs peak"
PEAK_GBPS = 8000.0
HEADLINE = "mamba2_h128"
KERNEL_SOURCES = ["hybrid_model_ssm_amd/csrc/mamba2_kernels.h", "hybrid_model_ssm_amd/csrc/device_common.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "mamba2_replay_decode_h128_pmc.txt")
STATS_SUMMARY = os.path.join(ROOT, "profiles", "mamba2_replay_decode_h128_kernel_stats.txt")
REPLAY_KERNEL_TAG = "mamba2_replay_kernel<64, 128, unsigned short, 0, 0>"
GDN_KERNEL_TAG = "gdn_replay_kernel<128, 128, unsigned short, 0>"
# kernels with committed HBM counter summaries: the kernel, the sources its hash covers,
# the summary file and its title lines
COUNTED = {
    "headline": dict(tag=REPLAY_KERNEL_TAG, sources=KERNEL_SOURCES, summary=PMC_SUMMARY,
                     title=["# rocprofv3 HBM counters: Mamba2 replay decode kernel, workload mamba2_h128",
                            "# (B=256 H=128 P=64 N=128 G=8 L=16, bf16 io, fp32 checkpoint reads)"]),
    "gdn": dict(tag=GDN_KERNEL_TAG,
                sources=["hybrid_model_ssm_amd/csrc/gdn_kernels.hip", "hybrid_model_ssm_amd/csrc/device_common.h"],
                summary=os.path.join(ROOT, "profiles", "gdn_replay_decode_hv32_pmc.txt"),
                title=["# rocprofv3 HBM counters: Gated DeltaNet replay decode kernel, workload gdn_hv32",
                       "# (B=256 HV=32 HK=16 dk=dv=128 L=16, bf16 io; 544 dispatches = 34 windows, flushes "
                       "included)"]),
}
COPY_BYTES = 1 << 30
MiB = float(1 << 20)


def _code_only(text):
    """Source text without comments and blank space, so that editing a comment does not
    mark counters taken on the same code as stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------------
# algorithmic byte models (what the method must move per launch)
# ------------------------------------------------------------------------------------

def lp_copy_bytes(P, N, lowp):
    """Bytes of one head's read copy: 2 per element (bf16, fp16), or 1 per element plus
    a 4-byte scale per row (fp8)."""
    kind = "bf16" if lowp is True else lowp
    if not kind:
        return 0
    return P * N + 4 * P if kind == "fp8" else 2 * P * N


def mamba2_replay_bytes(B, H, P, N, G, L, io, c, lowp=False):
    """One decode step for B sequences all at cursor c (records stored before it)."""
    fold = c + 1 == L
    if fold:
        state = P * N * 4 * 2 + lp_copy_bytes(P, N, lowp)
    else:
        state = lp_copy_bytes(P, N, lowp) if lowp else P * N * 4
    per_h = state + 2 * P * io + io + P * 4 + c * (P * io + 4) + (0 if fold else P * io + 4)
    per_g = 2 * N * io + c * N * io + (0 if fold else N * io)
    return B * H * per_h + B * G * per_g


def mamba2_conventional_bytes(B, H, P, N, G, io):
    return B * H * (2 * P * N * 4 + 2 * P * io + io + P * 4) + B * G * 2 * N * io


def spec_round_bytes(H, P, N, G, L, io, T, committed, lowp=False):
    """One verify round; ``committed`` holds each sequence's committed count."""
    tot = 0
    for cm in committed:
        fold = cm + T > L
        if fold:
            state = 2 * P * N * 4 + lp_copy_bytes(P, N, lowp)
        else:
            state = lp_copy_bytes(P, N, lowp) if lowp else P * N * 4
        per_h = state + T * (2 * P * io + io + P * 4) + cm * (P * io + 4) + T * (P * io + 4)
        per_g = T * 2 * N * io + cm * N * io + T * N * io
        tot += H * per_h + G * per_g
    return tot


def spec_baseline_bytes(B, H, P, N, G, io, T):
    return B * H * (P * N * 4 * (1 + T) + T * (2 * P * io + io + P * 4)) + B * G * T * 2 * N * io


def gdn_replay_bytes(B, HV, HK, dk, dv, L, io, c):
    fold = c + 1 == L
    state = dv * dk * 4 * (2 if fold else 1)
    per_hv = state + dv * io + 8 + dv * 4 + c * (dv * io + 8) + (0 if fold else dv * io + 8)
    per_hk = 2 * dk * io + c * dk * io + (0 if fold else dk * io)
    return B * HV * per_hv + B * HK * per_hk


def gdn_window_bytes():
    """Average algorithmic bytes per GDN decode launch over one window (gdn_hv32)."""
    from hybrid_model_ssm_amd import synth
    w = synth.WORKLOADS["gdn_hv32"]
    B, HV, HK, dk, dv, L = w["batch"], w["num_v_heads"], w["num_k_heads"], w["dk"], w["dv"], w["buffer_len"]
    return sum(gdn_replay_bytes(B, HV, HK, dk, dv, L, 2, c) for c in range(L)) / L


def gdn_conventional_bytes(B, HV, HK, dk, dv, io):
    return B * HV * (2 * dv * dk * 4 + dv * io + 8 + dv * 4) + B * HK * 2 * dk * io


def gdn_spec_round_bytes(HV, HK, dk, dv, L, io, T, committed):
    """One Gated DeltaNet verify round; ``committed`` holds each sequence's committed count."""
    tot = 0
    for cm in committed:
        state = dv * dk * 4 * (2 if cm + T > L else 1)
        per_hv = state + T * (dv * io + 8 + dv * 4) + cm * (dv * io + 8) + T * (dv * io + 8)
        per_hk = T * 2 * dk * io + cm * dk * io + T * dk * io
        tot += HV * per_hv + HK * per_hk
    return tot


def gdn_spec_baseline_bytes(B, HV, HK, dk, dv, io, T):
    return B * HV * (dv * dk * 4 * (1 + T) + T * (dv * io + 8 + dv * 4)) + B * HK * T * 2 * dk * io


# ------------------------------------------------------------------------------------
# timing
# ------------------------------------------------------------------------------------

class Timer:
    """HIP events on the current (launch) stream around exactly ``n`` launches."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, launch, first, n):
        torch = self.torch
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for i in range(first, first + n):
            launch(i)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return e0.elapsed_time(e1) / 1e3, wall


def _check(st, name):
    if st != 0:
        from hybrid_model_ssm_amd import replayssm as rs
        raise rs.ReplaySSMError(st, name)


class Mamba2Bench:
    """Device buffers and pre-marshalled launch arguments for one Mamba2 workload."""

    def __init__(self, torch, rs, synth, name, pool=32, lowp=False, conventional=False, seed_override=None,
                 state_and_output=False):
        import ctypes
        self.torch, self.rs = torch, rs
        w = dict(synth.WORKLOADS[name])
        self.w = w
        self.B, self.H, self.P, self.N, self.G, self.L = (w["batch"], w["nheads"], w["headdim"], w["dstate"],
                                                          w["ngroups"], w["buffer_len"])
        self.io = 2 if w["io"] == "bf16" else 4
        gen = synth.mamba2_inputs(name) if seed_override is None else synth.mamba2_inputs(name, seed=seed_override)
        st = gen.static
        self.static = st
        dev = "cuda"
        f32 = torch.float32
        self.desc = rs.Mamba2Desc(self.B, self.H, self.P, self.N, self.G, self.L,
                                  rs.BF16 if w["io"] == "bf16" else rs.F32, True)
        iot = self.desc.torch_io
        t = lambda a, d: torch.from_numpy(a).to(dev).to(d)  # noqa: E731
        self.ckpt0 = t(st.ckpt, f32)
        self.A, self.D, self.bias = t(st.A, f32), t(st.D, f32), t(st.dt_bias, f32)
        self.pool_np = [gen.step() for _ in range(pool)]
        self.pool = [{k: t(v, iot) for k, v in s.items()} for s in self.pool_np]
        self.out = torch.empty(self.B, self.H, self.P, dtype=f32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.conventional = conventional
        self.lowp = lowp
        L = rs.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.stream = stream
        if conventional:
            self.state_conv = self.ckpt0.clone()
            d = self.desc.c()
            self._keep = [d]
            self.args = [(ctypes.byref(d), self.state_conv.data_ptr(),
                          *(p[k].data_ptr() for k in ("x", "z", "B", "C", "dt_raw")),
                          self.bias.data_ptr(), self.A.data_ptr(), self.D.data_ptr(), self.out.data_ptr(), stream)
                         for p in self.pool]
            self.fn = L.replayssm_selective_state_update
        else:
            self.state = rs.Mamba2State.allocate(self.desc, lowp=lowp, ckpt=self.ckpt0.clone())
            self.cur = [torch.zeros(self.B, dtype=torch.int32, device=dev) for _ in range(2)]
            d, s = self.desc.c(), self.state.c()
            self._keep = [d, s]
            if lowp:  # create the read copy: a flush of the empty buffer (cursors stay 0)
                rs.mamba2_flush(self.desc, self.state, self.cur[0], self.cur[1], self.A, self.err)
            self.args = []
            for i in range(2 * pool):
                p = self.pool[i % pool]
                self.args.append((ctypes.byref(d), ctypes.byref(s), self.cur[i % 2].data_ptr(),
                                  self.cur[1 - i % 2].data_ptr(),
                                  *(p[k].data_ptr() for k in ("x", "z", "B", "C", "dt_raw")),
                                  self.bias.data_ptr(), self.A.data_ptr(), self.D.data_ptr(),
                                  self.out.data_ptr(), self.err.data_ptr(), stream))
            self.fn = L.replayssm_mamba2_decode_state_and_output if state_and_output else L.replayssm_mamba2_decode

    def launch(self, i):
        a = self.args[i % len(self.args)]
        st = self.fn(*a)
        if st:
            _check(st, self.fn.__name__)

    def bytes_of_step(self, i):
        """Algorithmic bytes of the i-th launch (0-based) from a fresh state."""
        if self.conventional:
            return mamba2_conventional_bytes(self.B, self.H, self.P, self.N, self.G, self.io)
        return mamba2_replay_bytes(self.B, self.H, self.P, self.N, self.G, self.L, self.io, i % self.L, self.lowp)


def time_mamba2(torch, rs, synth, name, steps, warmup, **kw):
    b = Mamba2Bench(torch, rs, synth, name, **kw)
    for i in range(warmup):
        b.launch(i)
    secs, wall = Timer(torch).run(b.launch, warmup, steps)
    if not b.conventional:
        exp = (warmup + steps) % b.L
        if not torch.equal(b.cur[(warmup + steps) % 2], torch.full_like(b.cur[0], exp)):
            raise RuntimeError("cursor check failed after the timed region")
        if b.err.item() != 0:
            raise RuntimeError("device error flag set")
    nbytes = sum(b.bytes_of_step(i) for i in range(warmup, warmup + steps))
    res = dict(seq_tokens_per_s=b.B * steps / secs, ms_per_step=secs * 1e3 / steps, seconds=secs, wall_s=wall,
               bytes_per_step_MiB=nbytes / steps / MiB, hbm_gbps=nbytes / secs / 1e9,
               frac_of_peak=nbytes / secs / 1e9 / PEAK_GBPS, steps=steps)
    return res, b


def time_mamba2_graph(torch, rs, synth, name, steps, warmup):
    """The same decode steps captured as one graph of two windows (2L launches, so that
    flushes keep their rate and the ping-pong cursors line up) and replayed: the launch
    overhead of single calls taken out.  Times steps // (2L) replays."""
    b = Mamba2Bench(torch, rs, synth, name)
    W = 2 * b.L
    warm = -(-warmup // W) * W
    for i in range(warm):
        b.launch(i)
    torch.cuda.synchronize()
    import ctypes
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)   # the capturing stream
        for j in range(W):
            a = b.args[(warm + j) % len(b.args)]
            _check(b.fn(*a[:-1], cap), b.fn.__name__)
    nrep = max(1, steps // W)
    probe = b.state.ckpt[0, 0].clone()
    g.replay()                       # one untimed replay; its two flushes must change the checkpoint
    torch.cuda.synchronize()
    if torch.equal(probe, b.state.ckpt[0, 0]):
        raise RuntimeError("the captured graph did not run the decode steps")
    secs, wall = Timer(torch).run(lambda r: g.replay(), 0, nrep)
    n = nrep * W
    done = warm + W + n
    if not torch.equal(b.cur[done % 2], torch.full_like(b.cur[0], done % b.L)):
        raise RuntimeError("cursor check failed after the graph replays")
    if b.err.item() != 0:
        raise RuntimeError("device error flag set")
    nbytes = sum(b.bytes_of_step(i) for i in range(n))
    del g, b
    return dict(seq_tokens_per_s=synth.WORKLOADS[name]["batch"] * n / secs, ms_per_step=secs * 1e3 / n,
                steps=n, launches_per_graph=W, bytes_per_step_MiB=nbytes / n / MiB, hbm_gbps=nbytes / secs / 1e9,
                frac_of_peak=nbytes / secs / 1e9 / PEAK_GBPS)


def time_spec(torch, rs, synth, rounds, warmup, baseline=False, lowp=False):
    import ctypes
    import numpy as np
    w = synth.WORKLOADS["mamba2_spec_h128"]
    B, H, P, N, G, L, T = w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"], w["buffer_len"], w["n_pos"]
    io = 2
    gen = synth.mamba2_inputs("mamba2_spec_h128")
    st = gen.static
    dev = "cuda"
    f32 = torch.float32
    t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    pool_n = 32
    pool, keeps = [], []
    for _ in range(pool_n):
        s = gen.step(n_pos=T)
        pool.append({k: t(v, torch.bfloat16) for k, v in s.items()})
        keeps.append(gen.accepted(T - 1) + 1)
    keep_dev = [torch.from_numpy(k.astype(np.int32)).to(dev) for k in keeps]
    A, D, bias = t(st.A, f32), t(st.D, f32), t(st.dt_bias, f32)
    out = torch.empty(B, T, H, P, dtype=f32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    Lb = rs.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    d = desc.c()
    if baseline:
        snaps = torch.empty(B, T, H, P, N, dtype=f32, device=dev)
        snaps[:, 0] = t(st.ckpt, f32)
        slots = [torch.from_numpy((keeps[(r - 1) % pool_n] - 1).astype(np.int32)).to(dev) for r in range(pool_n)]
        slots[0] = torch.zeros(B, dtype=torch.int32, device=dev)

        def launch(r):
            p = pool[r % pool_n]
            _check(Lb.replayssm_mamba2_spec_baseline(ctypes.byref(d), snaps.data_ptr(), slots[r % pool_n].data_ptr(),
                                                     T, *(p[k].data_ptr() for k in ("x", "z", "B", "C", "dt_raw")),
                                                     bias.data_ptr(), A.data_ptr(), D.data_ptr(), out.data_ptr(),
                                                     stream), "spec_baseline")
        keep_state = [snaps]
    else:
        state = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=t(st.ckpt, f32))
        s_c = state.c()
        head = torch.zeros(B, dtype=torch.int32, device=dev)
        com = torch.zeros(B, dtype=torch.int32, device=dev)
        flushed = torch.zeros(B, dtype=torch.int32, device=dev)
        if lowp:
            z0, z1 = torch.zeros_like(head), torch.zeros_like(head)
            rs.mamba2_flush(desc, state, z0, z1, A, err)

        def launch(r):
            p = pool[r % pool_n]
            _check(Lb.replayssm_mamba2_spec_verify(ctypes.byref(d), ctypes.byref(s_c), head.data_ptr(), com.data_ptr(),
                                                   T, None, *(p[k].data_ptr() for k in ("x", "z", "B", "C", "dt_raw")),
                                                   bias.data_ptr(), A.data_ptr(), D.data_ptr(), out.data_ptr(),
                                                   flushed.data_ptr(), err.data_ptr(), stream), "spec_verify")
            _check(Lb.replayssm_commit(B, L, T, head.data_ptr(), com.data_ptr(), flushed.data_ptr(),
                                       keep_dev[r % pool_n].data_ptr(), None, err.data_ptr(), stream), "commit")
        keep_state = [state, s_c]
    for r in range(warmup):
        launch(r)
    secs, wall = Timer(torch).run(launch, warmup, rounds)
    accepted = sum(int(keeps[r % pool_n].sum()) for r in range(warmup, warmup + rounds))
    # host model of the cursors (integer rules of the commit call) for the byte count
    hd = np.zeros(B, np.int64)
    cm = np.zeros(B, np.int64)
    nbytes = 0
    n_flush = 0
    for r in range(warmup + rounds):
        fl = cm + T > L
        if r >= warmup:
            nbytes += spec_baseline_bytes(B, H, P, N, G, io, T) if baseline else \
                spec_round_bytes(H, P, N, G, L, io, T, cm, lowp)
            n_flush += int(fl.sum())
        hd = np.where(fl, (hd + cm) % L, hd)
        cm = np.where(fl, 0, cm) + keeps[r % pool_n]
    if not baseline:
        if not (np.array_equal(head.cpu().numpy(), hd.astype(np.int32)) and
                np.array_equal(com.cpu().numpy(), cm.astype(np.int32))):
            raise RuntimeError("speculative cursors disagree with the host model")
        if err.item() != 0:
            raise RuntimeError("device error flag set")
    del keep_state
    return dict(accepted_tokens_per_s=accepted / secs, positions_per_s=B * T * rounds / secs,
                ms_per_round=secs * 1e3 / rounds, rounds=rounds, bytes_per_round_MiB=nbytes / rounds / MiB,
                hbm_gbps=nbytes / secs / 1e9, frac_of_peak=nbytes / secs / 1e9 / PEAK_GBPS,
                accepted_per_round=accepted / rounds / B,
                flush_fraction=(n_flush / (B * rounds)) if not baseline else None)


def time_gdn(torch, rs, synth, steps, warmup, conventional=False):
    import ctypes
    import numpy as np
    w = synth.WORKLOADS["gdn_hv32"]
    B, HV, HK, dk, dv, L = w["batch"], w["num_v_heads"], w["num_k_heads"], w["dk"], w["dv"], w["buffer_len"]
    gen = synth.gdn_inputs("gdn_hv32")
    st = gen.static
    dev = "cuda"
    t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    pool = []
    for _ in range(32):
        s = gen.step()
        pool.append({"q": t(s["q"], torch.bfloat16), "k": t(s["k"], torch.bfloat16), "v": t(s["v"], torch.bfloat16),
                     "alpha": t(s["alpha"], torch.float32), "beta": t(s["beta"], torch.float32)})
    out = torch.empty(B, HV, dv, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    Lb = rs.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    d = desc.c()
    keys = ("q", "k", "v", "alpha", "beta")
    if conventional:
        S = t(st.ckpt, torch.float32)

        def launch(i):
            p = pool[i % 32]
            _check(Lb.replayssm_gdn_conventional_decode(ctypes.byref(d), S.data_ptr(), *(p[k].data_ptr() for k in keys),
                                                        out.data_ptr(), stream), "gdn_conventional")
        keep = [S]
    else:
        state = rs.GdnState.allocate(desc, ckpt=t(st.ckpt, torch.float32))
        s_c = state.c()
        cur = [torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(2)]

        def launch(i):
            p = pool[i % 32]
            _check(Lb.replayssm_gdn_decode(ctypes.byref(d), ctypes.byref(s_c), cur[i % 2].data_ptr(),
                                           cur[1 - i % 2].data_ptr(), *(p[k].data_ptr() for k in keys),
                                           out.data_ptr(), err.data_ptr(), stream), "gdn_decode")
        keep = [state, s_c, cur]
    for i in range(warmup):
        launch(i)
    secs, wall = Timer(torch).run(launch, warmup, steps)
    if conventional:
        nbytes = steps * gdn_conventional_bytes(B, HV, HK, dk, dv, 2)
    else:
        nbytes = sum(gdn_replay_bytes(B, HV, HK, dk, dv, L, 2, i % L) for i in range(warmup, warmup + steps))
        if err.item() != 0:
            raise RuntimeError("device error flag set")
    del keep
    return dict(seq_tokens_per_s=B * steps / secs, ms_per_step=secs * 1e3 / steps, steps=steps,
                bytes_per_step_MiB=nbytes / steps / MiB, hbm_gbps=nbytes / secs / 1e9,
                frac_of_peak=nbytes / secs / 1e9 / PEAK_GBPS)


def time_gdn_spec(torch, rs, synth, rounds, warmup, baseline=False):
    import ctypes
    import numpy as np
    w = synth.WORKLOADS["gdn_spec_hv32"]
    B, HV, HK, dk, dv, L, T = (w[k] for k in ("batch", "num_v_heads", "num_k_heads", "dk", "dv", "buffer_len",
                                               "n_pos"))
    io = 2
    gen = synth.gdn_inputs("gdn_spec_hv32")
    st = gen.static
    dev = "cuda"
    t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    pool_n = 32
    pool, keeps = [], []
    for _ in range(pool_n):
        s = gen.step(n_pos=T)
        pool.append({"q": t(s["q"], torch.bfloat16), "k": t(s["k"], torch.bfloat16), "v": t(s["v"], torch.bfloat16),
                     "alpha": t(s["alpha"], torch.float32), "beta": t(s["beta"], torch.float32)})
        keeps.append(gen.accepted(T - 1) + 1)
    keep_dev = [torch.from_numpy(k.astype(np.int32)).to(dev) for k in keeps]
    keys = ("q", "k", "v", "alpha", "beta")
    out = torch.empty(B, T, HV, dv, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    Lb = rs.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    d = desc.c()
    if baseline:
        snaps = torch.empty(B, T, HV, dv, dk, dtype=torch.float32, device=dev)
        snaps[:, 0] = t(st.ckpt, torch.float32)
        slots = [torch.from_numpy((keeps[(r - 1) % pool_n] - 1).astype(np.int32)).to(dev) for r in range(pool_n)]
        slots[0] = torch.zeros(B, dtype=torch.int32, device=dev)

        def launch(r):
            p = pool[r % pool_n]
            _check(Lb.replayssm_gdn_spec_baseline(ctypes.byref(d), snaps.data_ptr(), slots[r % pool_n].data_ptr(), T,
                                                  *(p[k].data_ptr() for k in keys), out.data_ptr(), stream),
                   "gdn_spec_baseline")
        keep_state = [snaps]
    else:
        state = rs.GdnState.allocate(desc, ckpt=t(st.ckpt, torch.float32))
        s_c = state.c()
        head = torch.zeros(B, dtype=torch.int32, device=dev)
        com = torch.zeros(B, dtype=torch.int32, device=dev)
        flushed = torch.zeros(B, dtype=torch.int32, device=dev)

        def launch(r):
            p = pool[r % pool_n]
            _check(Lb.replayssm_gdn_spec_verify(ctypes.byref(d), ctypes.byref(s_c), head.data_ptr(), com.data_ptr(), T,
                                                None, *(p[k].data_ptr() for k in keys), out.data_ptr(), flushed.data_ptr(),
                                                err.data_ptr(), stream), "gdn_spec_verify")
            _check(Lb.replayssm_commit(B, L, T, head.data_ptr(), com.data_ptr(), flushed.data_ptr(),
                                       keep_dev[r % pool_n].data_ptr(), None, err.data_ptr(), stream), "commit")
        keep_state = [state, s_c]
    for r in range(warmup):
        launch(r)
    secs, wall = Timer(torch).run(launch, warmup, rounds)
    accepted = sum(int(keeps[r % pool_n].sum()) for r in range(warmup, warmup + rounds))
    hd = np.zeros(B, np.int64)
    cm = np.zeros(B, np.int64)
    nbytes = 0
    n_flush = 0
    for r in range(warmup + rounds):
        fl = cm + T > L
        if r >= warmup:
            nbytes += gdn_spec_baseline_bytes(B, HV, HK, dk, dv, io, T) if baseline else \
                gdn_spec_round_bytes(HV, HK, dk, dv, L, io, T, cm)
            n_flush += int(fl.sum())
        hd = np.where(fl, (hd + cm) % L, hd)
        cm = np.where(fl, 0, cm) + keeps[r % pool_n]
    if not baseline:
        if not (np.array_equal(head.cpu().numpy(), hd.astype(np.int32)) and
                np.array_equal(com.cpu().numpy(), cm.astype(np.int32))):
            raise RuntimeError("speculative cursors disagree with the host model")
        if err.item() != 0:
            raise RuntimeError("device error flag set")
    del keep_state
    return dict(accepted_tokens_per_s=accepted / secs, positions_per_s=B * T * rounds / secs,
                ms_per_round=secs * 1e3 / rounds, rounds=rounds, bytes_per_round_MiB=nbytes / rounds / MiB,
                hbm_gbps=nbytes / secs / 1e9, frac_of_peak=nbytes / secs / 1e9 / PEAK_GBPS,
                accepted_per_round=accepted / rounds / B,
                flush_fraction=(n_flush / (B * rounds)) if not baseline else None)


SWEEP_WINDOWS = ((0, 16), (16, 64), (64, 256), (256, 1024))


def precision_sweep(torch, rs, synth, batch=32):
    """Emulated read and recurrence precisions (not timed).  Every configuration runs the
    same 1024 decode steps from the same inputs; its outputs are compared with an fp32
    conventional run, as sqrt(sum (y - y32)^2 / sum y32^2) over the steps of each window.

    replay  rec=f32 read=X   fp32 checkpoint; non-flush steps read a copy in format X
    replay  rec=X   read=X   checkpoint rounded to X at every flush (and at the start),
                             so the recurrence runs in X; non-flush steps read it
    conv    rec=X            conventional update, state rounded to X after every step
    """
    import numpy as np
    dev = "cuda"
    nsteps = SWEEP_WINDOWS[-1][1]
    names = {rs.F32: "f32", rs.BF16: "bf16", rs.F16: "f16", rs.FP8_E4M3: "fp8"}
    lowp_kind = {rs.BF16: "bf16", rs.F16: "f16", rs.FP8_E4M3: "fp8"}
    rows = []

    def window_errors(sq_err, sq_ref):
        return [float(np.sqrt(sq_err[a:b].sum() / sq_ref[a:b].sum())) for a, b in SWEEP_WINDOWS]

    # ---- Mamba2 -------------------------------------------------------------------------
    gen = synth.mamba2_inputs(HEADLINE, batch=batch)
    w = dict(synth.WORKLOADS[HEADLINE])
    H, P, N, G, L = w["nheads"], w["headdim"], w["dstate"], w["ngroups"], w["buffer_len"]
    desc = rs.Mamba2Desc(batch, H, P, N, G, L, rs.BF16, True)
    f32 = torch.float32
    t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
    st = gen.static
    ckpt0 = t(st.ckpt, f32)
    A, D, bias = t(st.A, f32), t(st.D, f32), t(st.dt_bias, f32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    cfgs = [dict(route="conv", rec=rs.F32, read=rs.F32)]
    cfgs += [dict(route="replay", rec=rs.F32, read=r) for r in (rs.F32, rs.BF16, rs.F16, rs.FP8_E4M3)]
    cfgs += [dict(route="replay", rec=r, read=r) for r in (rs.BF16, rs.F16, rs.FP8_E4M3)]
    cfgs += [dict(route="conv", rec=r, read=r) for r in (rs.BF16, rs.F16, rs.FP8_E4M3)]
    for c in cfgs:
        ck = ckpt0.clone()
        rs.emulate_precision(ck, c["rec"])
        c["out"] = torch.empty(batch, H, P, dtype=f32, device=dev)
        c["sq"] = torch.zeros(nsteps, dtype=torch.float64, device=dev)
        if c["route"] == "conv":
            c["state"] = ck
        else:
            lowp = lowp_kind.get(c["read"]) if c["rec"] == rs.F32 else False
            c["state"] = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=ck)
            c["cur"] = [torch.zeros(batch, dtype=torch.int32, device=dev) for _ in range(2)]
            if lowp:   # make the read copy: a flush of the empty buffer
                rs.mamba2_flush(desc, c["state"], c["cur"][0], c["cur"][1], A, err)
    ref_sq = torch.zeros(nsteps, dtype=torch.float64, device=dev)
    for i in range(nsteps):
        s = gen.step()
        x, z, Bm, Cm = (t(s[k], torch.bfloat16) for k in ("x", "z", "B", "C"))
        dt = t(s["dt_raw"], torch.bfloat16)
        for c in cfgs:
            if c["route"] == "conv":
                rs.selective_state_update(desc, c["state"], x, z, Bm, Cm, dt, bias, A, D, c["out"])
                rs.emulate_precision(c["state"], c["rec"])
            else:
                cur = c["cur"]
                rs.mamba2_decode(desc, c["state"], cur[i % 2], cur[1 - i % 2], x, z, Bm, Cm, dt, bias, A, D,
                                 c["out"], err)
                if i % L == L - 1:
                    rs.emulate_precision(c["state"].ckpt, c["rec"])
        y32 = cfgs[0]["out"].double()
        ref_sq[i] = (y32 * y32).sum()
        for c in cfgs[1:]:
            c["sq"][i] = ((c["out"].double() - y32) ** 2).sum()
    if err.item() != 0:
        raise RuntimeError("device error flag set in the precision sweep")
    ref = ref_sq.cpu().numpy()
    for c in cfgs[1:]:
        rows.append(dict(layer="mamba2", route=c["route"], rec=names[c["rec"]],
                         read=names[c["read"]] if c["route"] == "replay" else names[c["rec"]],
                         rel_rms=window_errors(c["sq"].cpu().numpy(), ref)))
    del cfgs

    # ---- Gated DeltaNet (no read copies: recurrence precision only) ------------------------
    gw = dict(synth.WORKLOADS["gdn_hv32"])
    HV, HK, dk, dv, GL = gw["num_v_heads"], gw["num_k_heads"], gw["dk"], gw["dv"], gw["buffer_len"]
    ggen = synth.gdn_inputs("gdn_hv32", batch=batch)
    gdesc = rs.GdnDesc(batch, HV, HK, dk, dv, GL, rs.BF16)
    S0 = t(ggen.static.ckpt, f32)
    gcfgs = [dict(route="conv", rec=rs.F32)]
    gcfgs += [dict(route="replay", rec=r) for r in (rs.F32, rs.BF16, rs.F16, rs.FP8_E4M3)]
    gcfgs += [dict(route="conv", rec=r) for r in (rs.BF16, rs.F16, rs.FP8_E4M3)]
    for c in gcfgs:
        ck = S0.clone()
        rs.emulate_precision(ck, c["rec"])
        c["out"] = torch.empty(batch, HV, dv, dtype=f32, device=dev)
        c["sq"] = torch.zeros(nsteps, dtype=torch.float64, device=dev)
        if c["route"] == "conv":
            c["state"] = ck
        else:
            c["state"] = rs.GdnState.allocate(gdesc, ckpt=ck)
            c["cur"] = [torch.zeros(batch, dtype=torch.int32, device=dev) for _ in range(2)]
    ref_sq = torch.zeros(nsteps, dtype=torch.float64, device=dev)
    for i in range(nsteps):
        s = ggen.step()
        q, k, v = (t(s[n], torch.bfloat16) for n in ("q", "k", "v"))
        al, be = t(s["alpha"], f32), t(s["beta"], f32)
        for c in gcfgs:
            if c["route"] == "conv":
                rs.gdn_conventional_decode(gdesc, c["state"], q, k, v, al, be, c["out"])
                rs.emulate_precision(c["state"], c["rec"])
            else:
                cur = c["cur"]
                rs.gdn_decode(gdesc, c["state"], cur[i % 2], cur[1 - i % 2], q, k, v, al, be, c["out"], err)
                if i % GL == GL - 1:
                    rs.emulate_precision(c["state"].ckpt, c["rec"])
        y32 = gcfgs[0]["out"].double()
        ref_sq[i] = (y32 * y32).sum()
        for c in gcfgs[1:]:
            c["sq"][i] = ((c["out"].double() - y32) ** 2).sum()
    if err.item() != 0:
        raise RuntimeError("device error flag set in the precision sweep")
    ref = ref_sq.cpu().numpy()
    for c in gcfgs[1:]:
        rows.append(dict(layer="gdn", route=c["route"], rec=names[c["rec"]],
                         read=names[c["rec"]], rel_rms=window_errors(c["sq"].cpu().numpy(), ref)))
    return dict(batch=batch, steps=nsteps, windows=[list(wd) for wd in SWEEP_WINDOWS],
                workloads=[f"{HEADLINE} at B={batch}", f"gdn_hv32 at B={batch}"],
                reference="conventional update in fp32 on the same inputs", rows=rows)


PROBE_LIB = os.path.join(ROOT, "hybrid_model_ssm_amd", "libreplayssm_probes.so")
# (name, mode, rows per thread, tiles per workgroup, non-temporal loads, non-temporal stores,
# in place): mode 0 reads, mode 1 reads and writes
PROBES = [(f"read_{'nt' if ntl else 'plain'}_r{r}_tpw{t}", 0, r, t, ntl, 0, False)
          for r in (1, 2, 8) for t in (1, 4, 16) for ntl in (0, 1)]
PROBES += [(f"{'inplace' if ip else 'copy'}_{'nt' if ntl else 'plain'}_{'nt' if nts else 'plain'}_r{r}_tpw{t}",
            1, r, t, ntl, nts, ip)
           for ip in (True, False) for r in (1, 2, 8) for t in (1, 4, 16) for ntl in (0, 1) for nts in (0, 1)]


def probe_lib():
    """The benchmark's bandwidth probes (built beside the library; not part of its C ABI)."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise FileNotFoundError(f"{PROBE_LIB} is missing: run python -m hybrid_model_ssm_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.replayssm_probe_pass_floats.restype = ctypes.c_int64
    lib.replayssm_probe_stream.restype = ctypes.c_int
    lib.replayssm_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
    return lib


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def ceiling(torch, reps=20, repeats=3):
    """Device bandwidth ceilings from the hand-written streaming probes (1 GiB of fp32 in
    the replay kernel's [64, 128] tile shape; read, in-place read+write, and copy), each the
    median of ``repeats`` timed regions of ``reps`` launches (HIP events on the launch
    stream); GB/s counts bytes read plus bytes written.  torch's elementwise copy (1 GiB in,
    1 GiB out) is timed beside them: it is the kernel the HBM counters are calibrated on."""
    import ctypes
    lib = probe_lib()
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.empty(n // lib.replayssm_probe_pass_floats(), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(3):
            fn()
        secs = []
        for _ in range(repeats):
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            secs.append(e0.elapsed_time(e1) / 1e3 / reps)
        return _median(secs)

    probes = {}
    for name, mode, rpt, tpw, ntl, nts, inplace in PROBES:
        dst = a if inplace else b

        def launch():
            st = lib.replayssm_probe_stream(a.data_ptr(), dst.data_ptr(), sink.data_ptr(), n, rpt, tpw, mode,
                                            ntl, nts, 1.0, stream)
            if st:
                raise RuntimeError(f"probe {name} failed with status {st}")
        secs = timed(launch)
        moved = COPY_BYTES * (1 if mode == 0 else 2)
        probes[name] = dict(gbps=moved / secs / 1e9, us=secs * 1e6)
    torch_copy = timed(lambda: torch.mul(a, 1.0, out=b))
    torch_inplace = timed(lambda: a.mul_(1.0))
    del a, b, sink
    best = lambda pre: max((v["gbps"], k) for k, v in probes.items() if k.startswith(pre))  # noqa: E731
    r, i, c = best("read_"), best("inplace_"), best("copy_")
    return dict(read_gbps=r[0], read_probe=r[1], inplace_rw_gbps=i[0], inplace_rw_probe=i[1],
                copy_gbps=c[0], copy_probe=c[1], torch_copy_gbps=2 * COPY_BYTES / torch_copy / 1e9,
                torch_inplace_gbps=2 * COPY_BYTES / torch_inplace / 1e9,
                probes=probes,
                note="hand-written HIP streaming probes (libreplayssm_probes.so), 1 GiB fp32 in [64,128] tiles, "
                     "256 threads, tpw = tiles per workgroup (16: replay decode shape, 1: conventional shape); "
                     "rw GB/s counts read + written bytes; median of 3 timed regions of 20 launches")


# ------------------------------------------------------------------------------------
# CPU oracle leg
# ------------------------------------------------------------------------------------

_ORACLE_JOB = None   # (static, step inputs, L, G): set before the pool forks, read by the workers


def _oracle_shard(span):
    """One worker's share of the CPU baseline: the oracle's replay form on sequences
    [b0, b1) of the sample, every step; returns its outputs and its compute time."""
    import numpy as np
    from oracle import mamba2 as om  # the oracle is test infrastructure; used only here
    b0, b1 = span
    st, steps_in, L, G = _ORACLE_JOB
    rep = om.Mamba2Replay(st.ckpt[b0:b1], L, st.A, st.D, st.dt_bias, G)
    t0 = time.perf_counter()
    outs = [rep.step(**{k: v[b0:b1] for k, v in s.items()})[0] for s in steps_in]
    return b0, time.perf_counter() - t0, np.stack(outs)


def cpu_oracle_run(synth, nseq, steps):
    """Time the fp64 oracle (replay form) on ``nseq`` sequences of the headline workload for
    ``steps`` steps, the sequences sharded over a pool of worker processes (one per host
    core this process may use, at most 16).  Must run before this process touches the GPU:
    the workers are forked from it.  The inputs are the ones the GPU run draws (the same
    seeded generator, the same order)."""
    global _ORACLE_JOB
    import multiprocessing
    import numpy as np
    gen = synth.mamba2_inputs(HEADLINE)
    st = gen.static
    steps_in = [gen.step() for _ in range(steps)]
    w = synth.WORKLOADS[HEADLINE]
    _ORACLE_JOB = (st, steps_in, w["buffer_len"], w["ngroups"])
    workers = max(1, min(16, len(os.sched_getaffinity(0)), nseq))
    cuts = [round(i * nseq / workers) for i in range(workers + 1)]
    spans = [(cuts[i], cuts[i + 1]) for i in range(workers) if cuts[i + 1] > cuts[i]]
    with multiprocessing.get_context("fork").Pool(len(spans)) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_shard, spans)
        wall = time.perf_counter() - t0
    _ORACLE_JOB = None
    res.sort(key=lambda r: r[0])
    outs = np.concatenate([r[2] for r in res], axis=1)   # [steps, nseq, H, P]
    return dict(nseq=nseq, steps=steps, workers=len(spans), wall=wall,
                worker_seconds=max(r[1] for r in res), outs=outs)


def cpu_baseline(torch, rs, synth, run):
    """The CPU baseline line from an oracle run (``cpu_oracle_run``), and the check of the
    GPU's outputs for the same sequences and inputs against it."""
    import numpy as np
    nseq, steps = run["nseq"], run["steps"]
    b = Mamba2Bench(torch, rs, synth, HEADLINE, pool=max(steps, 1))
    worst = 0.0
    for i in range(steps):
        b.launch(i)
        g = b.out[:nseq].cpu().numpy()
        o = run["outs"][i]
        worst = max(worst, float(np.max(np.abs(g - o) / (1e-4 * (1 + np.abs(o))))))
    secs = run["wall"]
    return dict(value=nseq * steps / secs, unit="seq-tokens/s", cores=run["workers"], kind="oracle",
                sample=f"{nseq} of {b.B} sequences x {steps} decode steps ({steps // b.L} L={b.L} windows with "
                       f"their flushes) of the {HEADLINE} workload, NumPy float64 replay form, sequences "
                       f"sharded over {run['workers']} worker processes (wall time of the pool)",
                seconds=secs, worker_seconds_max=run["worker_seconds"],
                gpu_parity_max_violation=worst, gpu_parity_ok=worst <= 1.0)


# ------------------------------------------------------------------------------------
# rocprofv3 counter summary
# ------------------------------------------------------------------------------------

def _read_counter_csv(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _avg_counter(rows, name_pred, counter):
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not name_pred(r.get("Kernel_Name", "")):
            continue
        key = (r.get("Dispatch_Id"), r.get("Kernel_Name"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)


def pmc_summarize(fetch_dir, write_dir, command, which="headline", algorithmic=None):
    """Summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) for the kernel
    COUNTED[which], scaled by what the same counters read for the 1 GiB calibration copy;
    ``algorithmic``: the byte model's average bytes per dispatch, for the ratio."""
    spec = COUNTED[which]
    out_path = spec["summary"]
    fr, wr = _read_counter_csv(fetch_dir), _read_counter_csv(write_dir)
    is_replay = lambda n: spec["tag"] in n  # noqa: E731
    is_copy = lambda n: "MulFunctor" in n  # the calibration kernel: 1 GiB read + 1 GiB write  # noqa: E731
    f_rep, nf = _avg_counter(fr, is_replay, "FETCH_SIZE")
    w_rep, nw = _avg_counter(wr, is_replay, "WRITE_SIZE")
    f_cpy, _ = _avg_counter(fr, is_copy, "FETCH_SIZE")
    w_cpy, _ = _avg_counter(wr, is_copy, "WRITE_SIZE")
    if None in (f_rep, w_rep, f_cpy, w_cpy):
        raise RuntimeError("missing counters for the replay kernel or the calibration copy")
    f_scale = COPY_BYTES / (f_cpy * 1024.0)
    w_scale = COPY_BYTES / (w_cpy * 1024.0)
    traffic = f_rep * 1024.0 * f_scale + w_rep * 1024.0 * w_scale
    lines = spec["title"] + [
        f"command: {command}",
        f"kernel: rssm::{spec['tag']}",
        f"kernel_source_sha256_16: {kernel_source_hash(spec['sources'])}",
        f"dispatches: fetch {nf}, write {nw}",
        f"FETCH_SIZE_KiB_per_dispatch: {f_rep:.1f}",
        f"WRITE_SIZE_KiB_per_dispatch: {w_rep:.1f}",
        f"copy_calibration: {COPY_BYTES} B device copy reads FETCH_SIZE {f_cpy:.1f} KiB, WRITE_SIZE {w_cpy:.1f} KiB",
        f"scale_fetch: {f_scale:.4f}",
        f"scale_write: {w_scale:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
    ]
    if algorithmic:
        lines += [f"algorithmic_bytes_per_launch: {algorithmic:.0f}",
                  f"traffic_over_algorithmic: {traffic / algorithmic:.4f}"]
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summarize(stats_dir, out_path, command, steps=0, warmup=0):
    """Write the per-kernel summary of a ``rocprofv3 --kernel-trace --stats`` run."""
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_stats.csv under {stats_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    lines = ["# rocprofv3 --kernel-trace --stats: kernels of one bench.py run (sorted by total time)",
             f"command: {command}",
             f"kernel_source_sha256_16: {kernel_source_hash()}",
             "calls | avg_us | min_us | max_us | total_ms | kernel"]
    for r in rows:
        lines.append("%5d | %8.1f | %8.1f | %8.1f | %8.2f | %s" % (
            int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e6, r["Name"][:160]))
    # the headline run is the first warmup+steps dispatches of the replay kernel; the same
    # kernel instance also serves later workloads of the run, so take them from the trace
    traces = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    if traces and steps:
        disp = [r for r in csv.DictReader(open(traces[0])) if REPLAY_KERNEL_TAG in r["Kernel_Name"]]
        disp.sort(key=lambda r: int(r["Start_Timestamp"]))
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp[:warmup + steps]]
        timed = dur[warmup:warmup + steps]
        if timed:
            lines.append(f"headline kernel: rssm::{REPLAY_KERNEL_TAG}")
            lines.append(f"headline timed dispatches: {len(timed)} (after {warmup} warmup), "
                         f"average {sum(timed) / len(timed):.1f} us, min {min(timed):.1f}, max {max(timed):.1f}")
            # every sequence starts at cursor 0, so dispatch i runs at cursor i mod L and the
            # dispatch at cursor L-1 is the flush step; split the time by the kind of step
            from hybrid_model_ssm_amd import synth
            w = synth.WORKLOADS[HEADLINE]
            L = w["buffer_len"]
            shape = (w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"], L, 2)
            for name, cs in (("non-flush", range(L - 1)), ("flush", [L - 1])):
                d = [t for i, t in enumerate(dur[:warmup + steps]) if i >= warmup and i % L in cs]
                nbytes = sum(mamba2_replay_bytes(*shape, c) for c in cs) / len(cs)
                if d:
                    avg = sum(d) / len(d)
                    lines.append(f"headline {name} steps (cursor {cs[0]}..{cs[-1]}): {len(d)} dispatches, "
                                 f"average {avg:.1f} us, min {min(d):.1f}, max {max(d):.1f}; "
                                 f"{nbytes / 1e6:.1f} MB algorithmic -> {nbytes / avg / 1e3:.0f} GB/s")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:12]))


def committed_traffic(which="headline"):
    """Counter-measured bytes per launch from the committed summary, if it matches the source."""
    spec = COUNTED[which]
    path = spec["summary"]
    if not os.path.exists(path):
        return None, "no counter summary committed"
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(spec["sources"]):
        return None, "kernel source changed since the counters were taken"
    return float(kv["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)


# ------------------------------------------------------------------------------------

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="timed decode steps of the headline")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--only", default="all",
                    help="all, headline, or a comma list of: conventional,graph,bf16,f16,fp8,so,h64,spec,gdn,"
                         "gdn_spec")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=256)
    ap.add_argument("--cpu-steps", type=int, default=32)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--pmc-kernel", default="headline", choices=sorted(COUNTED),
                    help="kernel whose counters --pmc-summarize reads")
    ap.add_argument("--stats-summarize", metavar="STATS_DIR")
    ap.add_argument("--precision-sweep", action="store_true",
                    help="print the emulated read/recurrence precision sweep (one JSON line) and exit")
    args = ap.parse_args(argv)

    if args.stats_summarize:
        stats_summarize(args.stats_summarize, STATS_SUMMARY, args.pmc_command, args.steps, args.warmup)
        return 0
    if args.pmc_summarize:
        pmc_summarize(args.pmc_summarize[0], args.pmc_summarize[1], args.pmc_command, args.pmc_kernel,
                      algorithmic=gdn_window_bytes() if args.pmc_kernel == "gdn" else None)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode path has no cross-GPU exchange); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    # the CPU oracle's worker pool is forked before this process touches the GPU
    oracle_run = None
    if not args.no_cpu_baseline and not args.precision_sweep:
        from hybrid_model_ssm_amd import synth as synth_cpu
        oracle_run = cpu_oracle_run(synth_cpu, args.cpu_seqs, args.cpu_steps)
        print(f"[bench] cpu oracle: {args.cpu_seqs} sequences x {args.cpu_steps} steps on "
              f"{oracle_run['workers']} worker processes in {oracle_run['wall']:.1f} s", file=sys.stderr, flush=True)

    import torch
    from hybrid_model_ssm_amd import replayssm as rs
    from hybrid_model_ssm_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rs.lib()
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    if args.precision_sweep:
        print(json.dumps({"precision_sweep": precision_sweep(torch, rs, synth)}), flush=True)
        return 0

    head, hb = time_mamba2(torch, rs, synth, HEADLINE, args.steps, args.warmup)
    print(f"[bench] headline {head['seq_tokens_per_s']:.4g} seq-tok/s, {head['hbm_gbps']:.0f} GB/s",
          file=sys.stderr, flush=True)
    del hb
    torch.cuda.empty_cache()
    launches = args.steps
    nbytes_per_launch = head["bytes_per_step_MiB"] * MiB
    avg_s = head["seconds"] / launches
    traffic, traffic_src = committed_traffic()
    roofline = dict(bound="hbm", achieved=nbytes_per_launch / avg_s / 1e9, peak=PEAK_GBPS, unit="GB/s",
                    frac=nbytes_per_launch / avg_s / 1e9 / PEAK_GBPS, traffic=traffic,
                    traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    traffic_source=traffic_src,
                    kernel=f"rssm::{REPLAY_KERNEL_TAG}", algorithmic_bytes_per_launch=nbytes_per_launch,
                    avg_launch_us=avg_s * 1e6, launches=launches)

    variants = {}
    conv = None
    groups = {"conventional", "graph", "bf16", "f16", "fp8", "so", "h64", "spec", "gdn", "gdn_spec"} \
        if args.only == "all" else \
        set() if args.only == "headline" else set(args.only.split(","))
    if "conventional" in groups:
        conv, _ = time_mamba2(torch, rs, synth, HEADLINE, args.steps, args.warmup, conventional=True)
        torch.cuda.empty_cache()
        variants["mamba2_h128_conventional"] = conv
    if "graph" in groups:
        variants["mamba2_h128_replay_graph"] = time_mamba2_graph(torch, rs, synth, HEADLINE, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if "bf16" in groups:
        variants["mamba2_h128_bf16_read"], _ = time_mamba2(torch, rs, synth, HEADLINE, args.steps, args.warmup,
                                                           lowp=True)
        torch.cuda.empty_cache()
    for kind in ("f16", "fp8"):
        if kind in groups:
            variants[f"mamba2_h128_{kind}_read"], _ = time_mamba2(torch, rs, synth, HEADLINE, args.steps,
                                                                  args.warmup, lowp=kind)
            torch.cuda.empty_cache()
    if "so" in groups:
        variants["mamba2_h128_state_and_output"], _ = time_mamba2(torch, rs, synth, HEADLINE, args.steps,
                                                                  args.warmup, state_and_output=True)
        torch.cuda.empty_cache()
    if "h64" in groups:
        variants["mamba2_h64_replay"], _ = time_mamba2(torch, rs, synth, "mamba2_h64", 256, 32)
        torch.cuda.empty_cache()
        variants["mamba2_h64_conventional"], _ = time_mamba2(torch, rs, synth, "mamba2_h64", 256, 32,
                                                             conventional=True)
        torch.cuda.empty_cache()
    if "spec" in groups:
        variants["spec_h128_verify"] = time_spec(torch, rs, synth, 256, 32)
        torch.cuda.empty_cache()
        variants["spec_h128_snapshot_baseline"] = time_spec(torch, rs, synth, 256, 32, baseline=True)
        torch.cuda.empty_cache()
    if "gdn" in groups:
        variants["gdn_hv32_replay"] = time_gdn(torch, rs, synth, 512, 32)
        tr, src = committed_traffic("gdn")
        variants["gdn_hv32_replay"].update(traffic_bytes_per_launch=tr, traffic_source=src,
                                           algorithmic_bytes_per_launch=gdn_window_bytes())
        torch.cuda.empty_cache()
        variants["gdn_hv32_conventional"] = time_gdn(torch, rs, synth, 512, 32, conventional=True)
        torch.cuda.empty_cache()
    if "gdn_spec" in groups:
        variants["gdn_spec_hv32_verify"] = time_gdn_spec(torch, rs, synth, 256, 32)
        torch.cuda.empty_cache()
        variants["gdn_spec_hv32_snapshot_baseline"] = time_gdn_spec(torch, rs, synth, 256, 32, baseline=True)
        torch.cuda.empty_cache()
    if variants:
        print("[bench] variants done", file=sys.stderr, flush=True)
    ceil = ceiling(torch) if (args.only == "all" or args.calibrate_copy) else None
    cpu = None
    if oracle_run is not None:
        cpu = cpu_baseline(torch, rs, synth, oracle_run)
        print(f"[bench] cpu baseline {cpu['value']:.4g} seq-tok/s in {cpu['seconds']:.1f}s", file=sys.stderr,
              flush=True)
        if not cpu["gpu_parity_ok"]:
            raise RuntimeError(f"GPU outputs disagree with the oracle: {cpu['gpu_parity_max_violation']}")

    w = synth.WORKLOADS[HEADLINE]
    line = {
        "metric": METRIC,
        "value": head["seq_tokens_per_s"],
        "unit": "seq-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "batch": w["batch"], "nheads": w["nheads"], "headdim": w["headdim"],
                   "dstate": w["dstate"], "ngroups": w["ngroups"], "buffer_len": w["buffer_len"],
                   "io_dtype": w["io"], "checkpoint": "f32", "checkpoint_reads": "f32",
                   "parallelism": "single GPU"},
        "hbm_gbps": head["hbm_gbps"],
        "hbm_frac_of_peak": head["frac_of_peak"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "speedup_vs_conventional": (head["seq_tokens_per_s"] / conv["seq_tokens_per_s"]) if conv else None,
        "variants": variants,
        "ceiling": ceil,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
