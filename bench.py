#!/usr/bin/env python3
"""Decode throughput of the ReplaySSM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--repeats R] [--only headline]

Headline (``value``): Mamba2 replay decode, one layer, B=256, H=128, P=64, N=128,
G=8, L=16, bf16 inputs, fp32 checkpoint reads -- seq-tokens/s = batch * K / time of
exactly K decode launches (one kernel launch each), the median of R timed regions.
Every region starts at a flush step, so it holds ceil(K/L) flushes (exactly the true
rate of one in L when K is a multiple of L, more otherwise); the untimed steps that
bring the cursors there are counted in ``timing.setup_steps``.  Inputs sit in HBM
before a region starts: a pool of 2L pre-drawn steps is cycled.  ``roofline`` gives
the replay kernel's algorithmic HBM bytes per launch divided by its average launch
time (HIP events on the launch stream) against the 8 TB/s peak; ``traffic`` is the
counter-measured HBM bytes per launch from the committed rocprofv3 summary when it
matches the current kernel source, else null (``traffic_gbps`` and ``traffic_frac``: those
bytes over the same launch time, against the peak).  ``step_split`` times two further
windows launch by launch: flush and non-flush steps.  ``cpu_baseline`` times the fp64
CPU oracle (replay and conventional forms, three workloads) on a sample of each, its
sequences sharded over worker processes on the host's cores (forked before the GPU is
touched), and checks the GPU outputs of the headline sample.

Measured beside the headline, each the median of R regions over whole windows (decode)
or the workload's rounds (speculative): the in-library conventional read-update-write
kernel, the headline steps captured as a graph and replayed, the bf16, fp16 and fp8 read
copies, the state-and-output decode route, the B=256/H=64 layer, speculative
verification (4 positions, commit) against the per-position snapshot baseline, and the
Gated DeltaNet layer (replay decode and conventional; speculative verification against
its snapshot baseline).  Each variant carries its counter traffic when a matching
summary is committed.  ``ceiling`` reports the device's streaming limits from the
hand-written probes (read, in-place read+write, copy, and reads followed by a block of
writes, which prices writes inside a read stream); ``device_model`` times the headline's
bytes at those rates and gives the measured steps as a fraction of it.

Auxiliary modes used to make the committed rocprofv3 summaries:
    --profile-variant NAME   W+K untimed dispatches of one variant and the 1 GiB
                             calibration copy (run under rocprofv3 --pmc)
    --pmc-summarize FETCH_DIR WRITE_DIR PROFILE_JSON   two --pmc runs into a summary
    --sq-summarize PROFILE_JSON PASS_DIR...   SQ instruction-counter passes into a summary
    --stats-summarize STATS_DIR BENCH_JSON   a --kernel-trace --stats run of the default
                             command into a summary
    --precision-sweep        output error of emulated read and recurrence precisions
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
REPLAY_KERNEL_TAG = "mamba2_replay_kernel<64, 128, unsigned short, 0, 0>"
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


def mamba2_replay_rw(B, H, P, N, G, L, io, c):
    """The bytes of ``mamba2_replay_bytes`` (fp32 reads) split as (read, written, flushed
    checkpoint): the last is the part of both that is the checkpoint read and written back
    in place (0 unless the step folds)."""
    fold = c + 1 == L
    ck = P * N * 4
    rd_h = ck + 2 * P * io + io + c * (P * io + 4)
    wr_h = P * 4 + (ck if fold else P * io + 4)
    rd_g = 2 * N * io + c * N * io
    wr_g = 0 if fold else N * io
    return B * H * rd_h + B * G * rd_g, B * H * wr_h + B * G * wr_g, (B * H * ck if fold else 0)


def step_model_seconds(read, written, inplace, read_bps, inplace_bps, write_seconds):
    """A step's time at the device's own rates: reads at the read probe's rate, the flushed
    checkpoint read and written at the in-place probe's rate (bytes read plus written), and
    every other write at the measured cost of writes inside a read stream
    (``write_seconds(bytes)``)."""
    return (read - inplace) / read_bps + 2 * inplace / inplace_bps + write_seconds(written - inplace)


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
# runners: one kind of dispatch on device-resident inputs
# ------------------------------------------------------------------------------------

def _check(st, name):
    if st != 0:
        from hybrid_model_ssm_amd import replayssm as rs
        raise rs.ReplaySSMError(st, name)


class Runner:
    """One workload variant.  ``launch(i)`` enqueues dispatch i (a decode step or a
    speculative round, counted from the fresh state) on the current stream;
    ``bytes_of(i)`` and ``tokens_of(i)`` are its algorithmic HBM bytes and the tokens
    it completes; ``check(n)`` validates the device state after n dispatches.  ``period``
    is the number of dispatches per window (decode: L, so a flush every L steps)."""

    unit = "seq-tokens/s"
    period = 1
    tag = None       # kernel name as rocprofv3 prints it
    sources = None   # kernel sources the counters depend on

    def bytes_of(self, i):
        raise NotImplementedError

    def tokens_of(self, i):
        return self.B

    def check(self, n):
        pass


MAMBA2_SOURCES = ["hybrid_model_ssm_amd/csrc/mamba2_kernels.h", "hybrid_model_ssm_amd/csrc/device_common.h"]
GDN_SOURCES = ["hybrid_model_ssm_amd/csrc/gdn_kernels.hip", "hybrid_model_ssm_amd/csrc/device_common.h"]
LP_CODE = {False: 0, "bf16": 1, "f16": 2, "fp8": 3}


class Mamba2Runner(Runner):
    """Mamba2 autoregressive decode: replay (fp32 reads or a read copy, output-only or
    state-and-output route) or the conventional read-update-write kernel."""

    def __init__(self, torch, rs, synth, name, pool=32, lowp=False, conventional=False, state_and_output=False):
        import ctypes
        self.torch, self.rs = torch, rs
        w = dict(synth.WORKLOADS[name])
        self.w = w
        self.B, self.H, self.P, self.N, self.G, self.L = (w["batch"], w["nheads"], w["headdim"], w["dstate"],
                                                          w["ngroups"], w["buffer_len"])
        self.io = 2 if w["io"] == "bf16" else 4
        self.period = 1 if conventional else self.L
        gen = synth.mamba2_inputs(name)
        st = gen.static
        dev = "cuda"
        f32 = torch.float32
        self.desc = rs.Mamba2Desc(self.B, self.H, self.P, self.N, self.G, self.L,
                                  rs.BF16 if w["io"] == "bf16" else rs.F32, True)
        iot = self.desc.torch_io
        t = lambda a, d: torch.from_numpy(a).to(dev).to(d)  # noqa: E731
        ckpt0 = t(st.ckpt, f32)
        self.A, self.D, self.bias = t(st.A, f32), t(st.D, f32), t(st.dt_bias, f32)
        self.pool = [{k: t(v, iot) for k, v in gen.step().items()} for _ in range(pool)]
        self.out = torch.empty(self.B, self.H, self.P, dtype=f32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.conventional, self.lowp = conventional, lowp
        Lb = rs.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        shape = f"{self.P}, {self.N}, {'unsigned short' if self.io == 2 else 'float'}"
        if conventional:
            self.state = ckpt0
            d = self.desc.c()
            self._keep = [d]
            self.args = [(ctypes.byref(d), self.state.data_ptr(),
                          *(p[k].data_ptr() for k in ("x", "z", "B", "C", "dt_raw")),
                          self.bias.data_ptr(), self.A.data_ptr(), self.D.data_ptr(), self.out.data_ptr(), stream)
                         for p in self.pool]
            self.fn = Lb.replayssm_selective_state_update
            self.tag = f"mamba2_conventional_kernel<{shape}, false>"
        else:
            self.state = rs.Mamba2State.allocate(self.desc, lowp=lowp, ckpt=ckpt0)
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
            self.fn = Lb.replayssm_mamba2_decode_state_and_output if state_and_output else Lb.replayssm_mamba2_decode
            self.tag = f"mamba2_replay_kernel<{shape}, {LP_CODE[lowp]}, {3 if state_and_output else 0}>"
        self.sources = MAMBA2_SOURCES

    def launch(self, i):
        st = self.fn(*self.args[i % len(self.args)])
        if st:
            _check(st, self.fn.__name__)

    def bytes_of(self, i):
        if self.conventional:
            return mamba2_conventional_bytes(self.B, self.H, self.P, self.N, self.G, self.io)
        return mamba2_replay_bytes(self.B, self.H, self.P, self.N, self.G, self.L, self.io, i % self.L, self.lowp)

    def check(self, n):
        if self.conventional:
            return
        torch = self.torch
        if not torch.equal(self.cur[n % 2], torch.full_like(self.cur[0], n % self.L)):
            raise RuntimeError("cursor check failed")
        if self.err.item() != 0:
            raise RuntimeError("device error flag set")


class SpecRunner(Runner):
    """Mamba2 or Gated DeltaNet speculative rounds (verify + commit) on the circular
    buffer, or the per-position snapshot baseline.  Round r uses pool entry r % pool; the
    kept counts come from the workload's seeded generator."""

    unit = "accepted tokens/s"

    def __init__(self, torch, rs, synth, name, baseline=False, pool=32):
        import ctypes
        import numpy as np
        self.torch = torch
        w = dict(synth.WORKLOADS[name])
        self.gdn = w["kind"] == "gdn_spec"
        self.baseline = baseline
        self.T, self.L, self.B = w["n_pos"], w["buffer_len"], w["batch"]
        T, L, B = self.T, self.L, self.B
        dev = "cuda"
        f32 = torch.float32
        t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
        gen = synth.gdn_inputs(name) if self.gdn else synth.mamba2_inputs(name)
        st = gen.static
        if self.gdn:
            self.HV, self.HK, self.dk, self.dv = w["num_v_heads"], w["num_k_heads"], w["dk"], w["dv"]
            keys = ("q", "k", "v", "alpha", "beta")
            types = {"q": torch.bfloat16, "k": torch.bfloat16, "v": torch.bfloat16, "alpha": f32, "beta": f32}
            desc = rs.GdnDesc(B, self.HV, self.HK, self.dk, self.dv, L, rs.BF16)
            self.out = torch.empty(B, T, self.HV, self.dv, dtype=f32, device=dev)
            per_state = (self.HV, self.dv, self.dk)
        else:
            self.H, self.P, self.N, self.G = w["nheads"], w["headdim"], w["dstate"], w["ngroups"]
            keys = ("x", "z", "B", "C", "dt_raw")
            types = {k: torch.bfloat16 for k in keys}
            desc = rs.Mamba2Desc(B, self.H, self.P, self.N, self.G, L, rs.BF16, True)
            self.out = torch.empty(B, T, self.H, self.P, dtype=f32, device=dev)
            per_state = (self.H, self.P, self.N)
            self.A, self.D, self.bias = t(st.A, f32), t(st.D, f32), t(st.dt_bias, f32)
        self.pool, self.keeps = [], []
        for _ in range(pool):
            s = gen.step(n_pos=T)
            self.pool.append({k: t(s[k], types[k]) for k in keys})
            self.keeps.append(gen.accepted(T - 1) + 1)
        self.keep_dev = [torch.from_numpy(k.astype(np.int32)).to(dev) for k in self.keeps]
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        Lb = rs.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        d = desc.c()
        self._keep = [d]
        io_name = "unsigned short"
        if baseline:
            # every snapshot slot starts as the initial state; round r reads the slot of the
            # last position kept in round r - 1
            self.snaps = t(st.ckpt, f32).unsqueeze(1).repeat(1, T, *([1] * len(per_state))).contiguous()
            self.slots = [torch.from_numpy((self.keeps[(r - 1) % pool] - 1).astype(np.int32)).to(dev)
                          for r in range(pool)]
            if self.gdn:
                fn = Lb.replayssm_gdn_spec_baseline
                self.args = [(ctypes.byref(d), self.snaps.data_ptr(), self.slots[r].data_ptr(), T,
                              *(p[k].data_ptr() for k in keys), self.out.data_ptr(), stream)
                             for r, p in enumerate(self.pool)]
                self.tag = f"gdn_conventional_kernel<{self.dk}, {self.dv}, {io_name}, true>"
            else:
                fn = Lb.replayssm_mamba2_spec_baseline
                self.args = [(ctypes.byref(d), self.snaps.data_ptr(), self.slots[r].data_ptr(), T,
                              *(p[k].data_ptr() for k in keys), self.bias.data_ptr(), self.A.data_ptr(),
                              self.D.data_ptr(), self.out.data_ptr(), stream) for r, p in enumerate(self.pool)]
                self.tag = f"mamba2_conventional_kernel<{self.P}, {self.N}, {io_name}, true>"
            self.calls = [(fn, a) for a in self.args]
        else:
            z = lambda: torch.zeros(B, dtype=torch.int32, device=dev)  # noqa: E731
            self.head, self.com, self.flushed = z(), z(), z()
            if self.gdn:
                self.state = rs.GdnState.allocate(desc, ckpt=t(st.ckpt, f32))
                s_c = self.state.c()
                fn = Lb.replayssm_gdn_spec_verify
                self.args = [(ctypes.byref(d), ctypes.byref(s_c), self.head.data_ptr(), self.com.data_ptr(), T, None,
                              *(p[k].data_ptr() for k in keys), self.out.data_ptr(), self.flushed.data_ptr(),
                              self.err.data_ptr(), stream) for p in self.pool]
                self.tag = f"gdn_replay_kernel<{self.dk}, {self.dv}, {io_name}, 2>"
            else:
                self.state = rs.Mamba2State.allocate(desc, ckpt=t(st.ckpt, f32))
                s_c = self.state.c()
                fn = Lb.replayssm_mamba2_spec_verify
                self.args = [(ctypes.byref(d), ctypes.byref(s_c), self.head.data_ptr(), self.com.data_ptr(), T, None,
                              *(p[k].data_ptr() for k in keys), self.bias.data_ptr(), self.A.data_ptr(),
                              self.D.data_ptr(), self.out.data_ptr(), self.flushed.data_ptr(), self.err.data_ptr(),
                              stream) for p in self.pool]
                self.tag = f"mamba2_replay_kernel<{self.P}, {self.N}, {io_name}, 0, 2>"
            self._keep.append(s_c)
            commit = Lb.replayssm_commit
            self.calls = [(fn, a, (B, L, T, self.head.data_ptr(), self.com.data_ptr(), self.flushed.data_ptr(),
                                   self.keep_dev[r].data_ptr(), None, self.err.data_ptr(), stream))
                          for r, a in enumerate(self.args)]
            self.commit = commit
        self.sources = GDN_SOURCES if self.gdn else MAMBA2_SOURCES
        self._model = None

    def launch(self, r):
        c = self.calls[r % len(self.calls)]
        _check(c[0](*c[1]), c[0].__name__)
        if not self.baseline:
            _check(self.commit(*c[2]), "replayssm_commit")

    def _cursor_model(self, n):
        """Per-round algorithmic bytes and fold counts of rounds 0..n-1 (host model of the
        commit rule), and the cursors after them."""
        import numpy as np
        hd = np.zeros(self.B, np.int64)
        cm = np.zeros(self.B, np.int64)
        out = []
        for r in range(n):
            fl = cm + self.T > self.L
            if self.baseline:
                nb = (gdn_spec_baseline_bytes(self.B, self.HV, self.HK, self.dk, self.dv, 2, self.T) if self.gdn else
                      spec_baseline_bytes(self.B, self.H, self.P, self.N, self.G, 2, self.T))
            else:
                nb = (gdn_spec_round_bytes(self.HV, self.HK, self.dk, self.dv, self.L, 2, self.T, cm) if self.gdn else
                      spec_round_bytes(self.H, self.P, self.N, self.G, self.L, 2, self.T, cm))
            out.append((nb, int(fl.sum())))
            hd = np.where(fl, (hd + cm) % self.L, hd)
            cm = np.where(fl, 0, cm) + self.keeps[r % len(self.keeps)]
        return out, hd, cm

    def bytes_of(self, r):
        if self._model is None or len(self._model) <= r:
            self._model = self._cursor_model(max(r + 1, 4096))[0]
        return self._model[r][0]

    def folds_of(self, r):
        self.bytes_of(r)
        return self._model[r][1]

    def tokens_of(self, r):
        return int(self.keeps[r % len(self.keeps)].sum())

    def check(self, n):
        import numpy as np
        if self.baseline:
            return
        _, hd, cm = self._cursor_model(n)
        if not (np.array_equal(self.head.cpu().numpy(), hd.astype(np.int32)) and
                np.array_equal(self.com.cpu().numpy(), cm.astype(np.int32))):
            raise RuntimeError("speculative cursors disagree with the host model")
        if self.err.item() != 0:
            raise RuntimeError("device error flag set")


class GdnRunner(Runner):
    """Gated DeltaNet autoregressive decode: replay, or the conventional kernel."""

    def __init__(self, torch, rs, synth, name="gdn_hv32", conventional=False, pool=32):
        import ctypes
        import numpy as np
        self.torch = torch
        w = synth.WORKLOADS[name]
        self.B, self.HV, self.HK, self.dk, self.dv, self.L = (w[k] for k in ("batch", "num_v_heads", "num_k_heads",
                                                                            "dk", "dv", "buffer_len"))
        self.conventional = conventional
        self.period = 1 if conventional else self.L
        gen = synth.gdn_inputs(name)
        st = gen.static
        dev = "cuda"
        t = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)  # noqa: E731
        desc = rs.GdnDesc(self.B, self.HV, self.HK, self.dk, self.dv, self.L, rs.BF16)
        keys = ("q", "k", "v", "alpha", "beta")
        self.pool = []
        for _ in range(pool):
            s = gen.step()
            self.pool.append({"q": t(s["q"], torch.bfloat16), "k": t(s["k"], torch.bfloat16),
                              "v": t(s["v"], torch.bfloat16), "alpha": t(s["alpha"], torch.float32),
                              "beta": t(s["beta"], torch.float32)})
        self.out = torch.empty(self.B, self.HV, self.dv, dtype=torch.float32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        Lb = rs.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        d = desc.c()
        self._keep = [d]
        if conventional:
            self.S = t(st.ckpt, torch.float32)
            self.fn = Lb.replayssm_gdn_conventional_decode
            self.args = [(ctypes.byref(d), self.S.data_ptr(), *(p[k].data_ptr() for k in keys), self.out.data_ptr(),
                          stream) for p in self.pool]
            self.tag = f"gdn_conventional_kernel<{self.dk}, {self.dv}, unsigned short, false>"
        else:
            self.state = rs.GdnState.allocate(desc, ckpt=t(st.ckpt, torch.float32))
            s_c = self.state.c()
            self._keep.append(s_c)
            self.cur = [torch.zeros(self.B, dtype=torch.int32, device=dev) for _ in range(2)]
            self.fn = Lb.replayssm_gdn_decode
            self.args = [(ctypes.byref(d), ctypes.byref(s_c), self.cur[i % 2].data_ptr(), self.cur[1 - i % 2].data_ptr(),
                          *(self.pool[i % pool][k].data_ptr() for k in keys), self.out.data_ptr(),
                          self.err.data_ptr(), stream) for i in range(2 * pool)]
            self.tag = f"gdn_replay_kernel<{self.dk}, {self.dv}, unsigned short, 0>"
        self.sources = GDN_SOURCES

    def launch(self, i):
        st = self.fn(*self.args[i % len(self.args)])
        if st:
            _check(st, self.fn.__name__)

    def bytes_of(self, i):
        if self.conventional:
            return gdn_conventional_bytes(self.B, self.HV, self.HK, self.dk, self.dv, 2)
        return gdn_replay_bytes(self.B, self.HV, self.HK, self.dk, self.dv, self.L, 2, i % self.L)

    def check(self, n):
        if self.conventional:
            return
        torch = self.torch
        if not torch.equal(self.cur[n % 2], torch.full_like(self.cur[0], n % self.L)):
            raise RuntimeError("cursor check failed")
        if self.err.item() != 0:
            raise RuntimeError("device error flag set")


# variant name -> (group of --only, constructor, workload, dispatches per timed region or None for
# the headline's whole windows)
VARIANTS = {
    "mamba2_h128_conventional": ("conventional", lambda T, R, S: Mamba2Runner(T, R, S, HEADLINE, conventional=True),
                                 HEADLINE, None),
    "mamba2_h128_bf16_read": ("bf16", lambda T, R, S: Mamba2Runner(T, R, S, HEADLINE, lowp="bf16"), HEADLINE, None),
    "mamba2_h128_f16_read": ("f16", lambda T, R, S: Mamba2Runner(T, R, S, HEADLINE, lowp="f16"), HEADLINE, None),
    "mamba2_h128_fp8_read": ("fp8", lambda T, R, S: Mamba2Runner(T, R, S, HEADLINE, lowp="fp8"), HEADLINE, None),
    "mamba2_h128_state_and_output": ("so", lambda T, R, S: Mamba2Runner(T, R, S, HEADLINE, state_and_output=True),
                                     HEADLINE, None),
    "mamba2_h64_replay": ("h64", lambda T, R, S: Mamba2Runner(T, R, S, "mamba2_h64"), "mamba2_h64", 256),
    "mamba2_h64_conventional": ("h64", lambda T, R, S: Mamba2Runner(T, R, S, "mamba2_h64", conventional=True),
                                "mamba2_h64", 256),
    "spec_h128_verify": ("spec", lambda T, R, S: SpecRunner(T, R, S, "mamba2_spec_h128"), "mamba2_spec_h128", 256),
    "spec_h128_snapshot_baseline": ("spec", lambda T, R, S: SpecRunner(T, R, S, "mamba2_spec_h128", baseline=True),
                                    "mamba2_spec_h128", 256),
    "gdn_hv32_replay": ("gdn", lambda T, R, S: GdnRunner(T, R, S), "gdn_hv32", 512),
    "gdn_hv32_conventional": ("gdn", lambda T, R, S: GdnRunner(T, R, S, conventional=True), "gdn_hv32", 512),
    "gdn_spec_hv32_verify": ("gdn_spec", lambda T, R, S: SpecRunner(T, R, S, "gdn_spec_hv32"), "gdn_spec_hv32", 256),
    "gdn_spec_hv32_snapshot_baseline": ("gdn_spec", lambda T, R, S: SpecRunner(T, R, S, "gdn_spec_hv32",
                                                                               baseline=True), "gdn_spec_hv32", 256),
}
GROUPS = ["conventional", "graph", "bf16", "f16", "fp8", "so", "h64", "spec", "gdn", "gdn_spec"]


# ------------------------------------------------------------------------------------
# timing
# ------------------------------------------------------------------------------------

def timed_region(torch, launch, first, n):
    """HIP events on the current (launch) stream around exactly ``n`` launches; returns
    the seconds between them."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(first, first + n):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


def measure(torch, r, warmup, n, repeats, start_at=None):
    """Time ``repeats`` regions of exactly ``n`` dispatches of runner ``r`` after
    ``warmup`` untimed ones.  With ``start_at`` (a position within r.period), untimed
    dispatches before the warmup and between regions make every region start at that
    position (for decode: the flush step).  Returns the region results (seconds, bytes,
    tokens, folds) and the dispatch count."""
    i = 0
    setup = 0
    if start_at is not None:
        setup = (start_at - warmup) % r.period
        for _ in range(setup):
            r.launch(i)
            i += 1
    for _ in range(warmup):
        r.launch(i)
        i += 1
    regions = []
    for _ in range(repeats):
        if start_at is not None:
            while i % r.period != start_at:
                r.launch(i)
                i += 1
        secs = timed_region(torch, r.launch, i, n)
        regions.append(dict(seconds=secs, first=i, bytes=sum(r.bytes_of(j) for j in range(i, i + n)),
                            tokens=sum(r.tokens_of(j) for j in range(i, i + n)),
                            flushes=sum(1 for j in range(i, i + n) if j % r.period == r.period - 1)
                            if r.period > 1 else None))
        i += n
    r.check(i)
    return regions, setup, i


def summarize(regions, n, unit_key="per_dispatch"):
    """The median region by throughput, with every region's throughput."""
    rates = [g["tokens"] / g["seconds"] for g in regions]
    order = sorted(range(len(regions)), key=lambda k: rates[k])
    med = regions[order[len(order) // 2]]
    secs = med["seconds"]
    return dict(value=med["tokens"] / secs, ms_per_dispatch=secs * 1e3 / n, dispatches_per_region=n,
                regions=len(regions), values_per_region=rates, bytes_per_dispatch_MiB=med["bytes"] / n / MiB,
                hbm_gbps=med["bytes"] / secs / 1e9, frac_of_peak=med["bytes"] / secs / 1e9 / PEAK_GBPS,
                flush_dispatches_per_region=med["flushes"])


def per_step_split(torch, r, first, n):
    """Duration of every dispatch of ``n`` (events between consecutive launches on the
    launch stream), split into flush steps (the last position of each window) and the
    others; ``first`` is the dispatch index to start at.  Returns averages in us."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for k in range(n):
        r.launch(first + k)
        ev[k + 1].record()
    torch.cuda.synchronize()
    dur = [ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(n)]
    fl = [d for k, d in enumerate(dur) if (first + k) % r.period == r.period - 1]
    nf = [d for k, d in enumerate(dur) if (first + k) % r.period != r.period - 1]
    fb = [r.bytes_of(first + k) for k in range(n) if (first + k) % r.period == r.period - 1]
    nb = [r.bytes_of(first + k) for k in range(n) if (first + k) % r.period != r.period - 1]
    res = dict(dispatches=n, flush_us=sum(fl) / len(fl) if fl else None,
               nonflush_us=sum(nf) / len(nf) if nf else None)
    if fl:
        res["flush_gbps"] = (sum(fb) / len(fb)) / (res["flush_us"] * 1e3)
    if nf:
        res["nonflush_gbps"] = (sum(nb) / len(nb)) / (res["nonflush_us"] * 1e3)
    return res, first + n


def time_variant(torch, rs, synth, name, K, W, repeats):
    """One variant of VARIANTS, timed over whole windows (decode) or the workload's
    rounds, the median of ``repeats`` regions, with the counter traffic of its committed
    summary when that matches the current source."""
    group, make, workload, n = VARIANTS[name]
    r = make(torch, rs, synth)
    if n is None:                                   # headline shapes: whole windows covering K
        n = max(2 * r.period, -(-K // r.period) * r.period)
    w = -(-W // r.period) * r.period
    regions, _, _ = measure(torch, r, w, n, repeats)
    res = summarize(regions, n)
    res.update(unit=r.unit, workload=workload, kernel=f"rssm::{r.tag}")
    tr = committed_traffic(name)
    if tr is not None:
        tg = tr["traffic"] / (res["ms_per_dispatch"] * 1e-3) / 1e9
        res.update(traffic_bytes_per_launch=tr["traffic"], traffic_over_algorithmic=tr["ratio"],
                   traffic_gbps=tg, traffic_frac_of_peak=tg / PEAK_GBPS, traffic_source=tr["source"])
    else:
        res.update(traffic_bytes_per_launch=None, traffic_source=committed_traffic_reason(name))
    del r
    torch.cuda.empty_cache()
    return res


def time_graph(torch, rs, synth, K, W, repeats):
    """The headline steps captured as one graph of two windows (2L launches, so that
    flushes keep their rate and the ping-pong cursors line up) and replayed: launch
    overhead taken out.  Each region replays it ceil(K / 2L) times."""
    import ctypes
    r = Mamba2Runner(torch, rs, synth, HEADLINE)
    Wn = 2 * r.L
    warm = -(-W // Wn) * Wn
    for i in range(warm):
        r.launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)   # the capturing stream
        for j in range(Wn):
            a = r.args[(warm + j) % len(r.args)]
            _check(r.fn(*a[:-1], cap), r.fn.__name__)
    nrep = max(1, -(-K // Wn))
    probe = r.state.ckpt[0, 0].clone()
    g.replay()                       # one untimed replay; its two flushes must change the checkpoint
    torch.cuda.synchronize()
    if torch.equal(probe, r.state.ckpt[0, 0]):
        raise RuntimeError("the captured graph did not run the decode steps")
    done = warm + Wn
    n = nrep * Wn
    regions = []
    for _ in range(repeats):
        secs = timed_region(torch, lambda _i: g.replay(), 0, nrep)
        regions.append(dict(seconds=secs, bytes=sum(r.bytes_of(i) for i in range(n)), tokens=r.B * n,
                            flushes=n // r.L))
        done += n
    r.check(done)
    res = summarize(regions, n)
    res.update(unit=r.unit, workload=HEADLINE, launches_per_graph=Wn, kernel=f"rssm::{r.tag}")
    del g, r
    torch.cuda.empty_cache()
    return res


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
# in place, tile order): mode 0 reads, modes 1 and 2 read and write; order 0 blocked (a workgroup's
# tiles consecutive), 1 skewed, 2 interleaved (workgroup w's tile t at t * grid + w)
PROBE_ORDERS = {1: "_skew", 2: "_ilv"}
PROBES = [(f"read_{'nt' if ntl else 'plain'}_r{r}_tpw{t}", 0, r, t, ntl, 0, False, 0)
          for r in (1, 2, 8) for t in (1, 4, 16) for ntl in (0, 1)]
PROBES += [(f"{'inplace' if ip else 'copy'}_{'nt' if ntl else 'plain'}_{'nt' if nts else 'plain'}_r{r}_tpw{t}",
            1, r, t, ntl, nts, ip, 0)
           for ip in (True, False) for r in (1, 2, 8) for t in (1, 4, 16) for ntl in (0, 1) for nts in (0, 1)]
PROBES += [(f"{kind}_nt_nt_r{r}_tpw{t}{PROBE_ORDERS[o]}", 0 if kind == "read" else 1, r, t, 1, 1,
            kind == "inplace", o)
           for o in (1, 2) for kind in ("read", "inplace", "copy") for r in (1, 2, 8) for t in (4, 16)]
# mode 2: the next tile's loads alternate with the current tile's stores
PROBES += [(f"{'inplace' if ip else 'copy'}_alt_nt_nt_r{r}_tpw{t}", 2, r, t, 1, 1, ip, 0)
           for ip in (True, False) for r in (2, 8) for t in (4, 16)]


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
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
    lib.replayssm_probe_rtw_read_floats.restype = ctypes.c_int64
    lib.replayssm_probe_read_then_write.restype = ctypes.c_int
    lib.replayssm_probe_read_then_write.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                    ctypes.c_int64, ctypes.c_void_p]
    return lib


# floats each workgroup of the read-then-write probe stores after reading its 512 KiB
# (2048 workgroups: 0 to 128 MiB written per launch)
RTW_WRITE_FLOATS = (0, 256, 512, 1024, 2048, 4096, 16384)


def write_cost_seconds(nbytes, points):
    """Seconds that ``nbytes`` written inside a read stream add, interpolated linearly in
    the read-then-write probe's (MiB written, seconds) points (the first at 0 MiB; past
    the last point, its last segment's slope): the cost per byte is not constant -- the
    first MiB written cost the most."""
    pts = sorted(points)
    x = nbytes / MiB
    x0, t0 = pts[0]
    for x1, t1 in pts[1:]:
        if x <= x1 or (x1, t1) == pts[-1]:
            return (t0 + (t1 - t0) * (x - x0) / (x1 - x0)) - pts[0][1]
        x0, t0 = x1, t1
    return 0.0


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
    for name, mode, rpt, tpw, ntl, nts, inplace, order in PROBES:
        dst = a if inplace else b

        def launch():
            st = lib.replayssm_probe_stream(a.data_ptr(), dst.data_ptr(), sink.data_ptr(), n, rpt, tpw, mode,
                                            ntl, nts, order, 1.0, stream)
            if st:
                raise RuntimeError(f"probe {name} failed with status {st}")
        secs = timed(launch)
        moved = COPY_BYTES * (1 if mode == 0 else 2)
        probes[name] = dict(gbps=moved / secs / 1e9, us=secs * 1e6)
    # a byte written inside a read stream: the read-then-write probe at several block sizes
    rtw_grid = n // lib.replayssm_probe_rtw_read_floats()
    rtw = []
    for wf in RTW_WRITE_FLOATS:
        def launch_rtw(wf=wf):
            st = lib.replayssm_probe_read_then_write(a.data_ptr(), b.data_ptr(), sink.data_ptr(), n, wf, stream)
            if st:
                raise RuntimeError(f"read-then-write probe failed with status {st}")
        rtw.append((rtw_grid * wf * 4 / MiB, timed(launch_rtw)))
    torch_copy = timed(lambda: torch.mul(a, 1.0, out=b))
    torch_inplace = timed(lambda: a.mul_(1.0))
    del a, b, sink
    best = lambda pre: max((v["gbps"], k) for k, v in probes.items() if k.startswith(pre))  # noqa: E731
    r, i, c = best("read_"), best("inplace_"), best("copy_")
    return dict(read_gbps=r[0], read_probe=r[1], inplace_rw_gbps=i[0], inplace_rw_probe=i[1],
                copy_gbps=c[0], copy_probe=c[1], torch_copy_gbps=2 * COPY_BYTES / torch_copy / 1e9,
                torch_inplace_gbps=2 * COPY_BYTES / torch_inplace / 1e9,
                probes=probes,
                read_then_write=dict(written_MiB=[p[0] for p in rtw], us=[p[1] * 1e6 for p in rtw],
                                     note="1 GiB read in the replay shape (16 tiles of 32 KiB per workgroup), "
                                          "then a block stored by each workgroup (non-temporal)"),
                note="hand-written HIP streaming probes (libreplayssm_probes.so), 1 GiB fp32 in [64,128] tiles, "
                     "256 threads, tpw = tiles per workgroup (16: replay decode shape, 1: conventional shape); "
                     "rw GB/s counts read + written bytes; median of 3 timed regions of 20 launches")




# ------------------------------------------------------------------------------------
# CPU oracle leg
# ------------------------------------------------------------------------------------

_ORACLE_JOB = None   # (kind, static, step inputs, params): set before the pool forks, read by the workers

# (workload, form, share of the sample's sequences): the oracle's replay form (O-2, O-5)
# and its conventional recurrence (O-1, O-4); the first is the baseline line's value, the
# others run on a quarter of its sequences to keep the leg short
ORACLE_JOBS = [(HEADLINE, "replay", 1.0), (HEADLINE, "conventional", 0.25), ("mamba2_h64", "replay", 0.25),
               ("mamba2_h64", "conventional", 0.25), ("gdn_hv32", "replay", 0.25), ("gdn_hv32", "conventional", 0.25)]


def _oracle_shard(span):
    """One worker's share of a CPU-baseline job: the oracle on sequences [b0, b1) of the
    sample, every step; returns its outputs and its compute time."""
    from threadpoolctl import threadpool_limits   # the oracle (test infrastructure) is used only here
    b0, b1 = span
    kind, form, st, steps_in, prm = _ORACLE_JOB
    sl = lambda s: {k: v[b0:b1] for k, v in s.items()}  # noqa: E731
    # one BLAS thread per worker: the workers already use every core
    with threadpool_limits(limits=1):
        return _oracle_shard_run(b0, b1, kind, form, st, steps_in, prm, sl)


def _oracle_shard_run(b0, b1, kind, form, st, steps_in, prm, sl):
    import numpy as np
    from oracle import gdn as og
    from oracle import mamba2 as om
    t0 = time.perf_counter()
    outs = []
    if kind == "mamba2" and form == "replay":
        rep = om.Mamba2Replay(st.ckpt[b0:b1], prm["L"], st.A, st.D, st.dt_bias, prm["G"])
        outs = [rep.step(**sl(s))[0] for s in steps_in]
    elif kind == "mamba2":
        h = st.ckpt[b0:b1].astype(np.float64)
        for s in steps_in:
            h, o = om.conventional_step(h, **sl(s), dt_bias=st.dt_bias, A=st.A, D=st.D)
            outs.append(o)
    elif form == "replay":
        rep = og.GDNReplay(st.ckpt[b0:b1], prm["L"], prm["HK"])
        outs = [rep.step(**sl(s))[0] for s in steps_in]
    else:
        S = st.ckpt[b0:b1].astype(np.float64)
        for s in steps_in:
            S, o = og.conventional_step(S, **sl(s))
            outs.append(o)
    return b0, time.perf_counter() - t0, np.stack(outs)


def cpu_oracle_run(synth, nseq, steps):
    """Time the fp64 oracle on ``nseq`` sequences (times the job's share) of each
    ORACLE_JOBS workload for ``steps`` steps, the sequences sharded over a pool of worker processes (one per host core this
    process may use, at most 16).  Must run before this process touches the GPU: the
    workers are forked from it.  The inputs are the ones the GPU runs draw (the same
    seeded generators, the same order).  Returns one result per job; the first holds the
    outputs for the GPU check."""
    global _ORACLE_JOB
    import multiprocessing
    import numpy as np
    results = []
    inputs = {}
    for name, form, share in ORACLE_JOBS:
        n = max(1, int(round(nseq * share)))
        workers = max(1, min(16, len(os.sched_getaffinity(0)), n))
        cuts = [round(i * n / workers) for i in range(workers + 1)]
        spans = [(cuts[i], cuts[i + 1]) for i in range(workers) if cuts[i + 1] > cuts[i]]
        w = synth.WORKLOADS[name]
        kind = "gdn" if w["kind"] == "gdn" else "mamba2"
        if name not in inputs:
            gen = synth.gdn_inputs(name) if kind == "gdn" else synth.mamba2_inputs(name)
            inputs[name] = (gen.static, [gen.step() for _ in range(steps)])
        st, steps_in = inputs[name]
        if nseq > w["batch"]:
            raise ValueError("--cpu-seqs exceeds the batch")
        prm = dict(L=w["buffer_len"], G=w.get("ngroups"), HK=w.get("num_k_heads"))
        _ORACLE_JOB = (kind, form, st, steps_in, prm)
        with multiprocessing.get_context("fork").Pool(len(spans)) as pool:
            t0 = time.perf_counter()
            res = pool.map(_oracle_shard, spans)
            wall = time.perf_counter() - t0
        _ORACLE_JOB = None
        res.sort(key=lambda x: x[0])
        out = dict(workload=name, form=form, nseq=n, steps=steps, workers=len(spans), wall=wall,
                   worker_seconds=max(x[1] for x in res), value=n * steps / wall)
        if not results:
            out["outs"] = np.concatenate([x[2] for x in res], axis=1)   # [steps, nseq, H, P]
        results.append(out)
    return results


def cpu_baseline(torch, rs, synth, runs):
    """The CPU baseline line from the oracle runs (``cpu_oracle_run``), and the check of the
    GPU's outputs for the first run's sequences and inputs against it."""
    import numpy as np
    run = runs[0]
    nseq, steps = run["nseq"], run["steps"]
    r = Mamba2Runner(torch, rs, synth, HEADLINE, pool=max(steps, 1))
    worst = 0.0
    for i in range(steps):
        r.launch(i)
        g = r.out[:nseq].cpu().numpy()
        o = run["outs"][i]
        worst = max(worst, float(np.max(np.abs(g - o) / (1e-4 * (1 + np.abs(o))))))
    r.check(steps)
    del r
    torch.cuda.empty_cache()
    secs = run["wall"]
    return dict(value=run["value"], unit="seq-tokens/s", cores=run["workers"], kind="oracle",
                sample=f"{nseq} of 256 sequences x {steps} decode steps ({steps // 16} L=16 windows with their "
                       f"flushes) of the {HEADLINE} workload, NumPy float64 replay form, sequences sharded over "
                       f"{run['workers']} worker processes (wall time of the pool)",
                seconds=secs, worker_seconds_max=run["worker_seconds"],
                gpu_parity_max_violation=worst, gpu_parity_ok=worst <= 1.0,
                runs=[{k: v for k, v in x.items() if k != "outs"} for x in runs])


# ------------------------------------------------------------------------------------
# rocprofv3 summaries
# ------------------------------------------------------------------------------------

# summary file of each profiled variant (named for the kernel and the workload)
PMC_FILES = {
    "headline": "mamba2_replay_decode_h128_pmc.txt",
    "mamba2_h128_conventional": "mamba2_conventional_h128_pmc.txt",
    "mamba2_h128_bf16_read": "mamba2_replay_decode_h128_bf16read_pmc.txt",
    "mamba2_h128_f16_read": "mamba2_replay_decode_h128_f16read_pmc.txt",
    "mamba2_h128_fp8_read": "mamba2_replay_decode_h128_fp8read_pmc.txt",
    "mamba2_h128_state_and_output": "mamba2_state_and_output_h128_pmc.txt",
    "mamba2_h64_replay": "mamba2_replay_decode_h64_pmc.txt",
    "mamba2_h64_conventional": "mamba2_conventional_h64_pmc.txt",
    "spec_h128_verify": "mamba2_spec_verify_h128_pmc.txt",
    "spec_h128_snapshot_baseline": "mamba2_spec_snapshot_baseline_h128_pmc.txt",
    "gdn_hv32_replay": "gdn_replay_decode_hv32_pmc.txt",
    "gdn_hv32_conventional": "gdn_conventional_hv32_pmc.txt",
    "gdn_spec_hv32_verify": "gdn_spec_verify_hv32_pmc.txt",
    "gdn_spec_hv32_snapshot_baseline": "gdn_spec_snapshot_baseline_hv32_pmc.txt",
}
STATS_SUMMARY = os.path.join(ROOT, "profiles", "mamba2_replay_decode_h128_kernel_stats.txt")


def make_runner(torch, rs, synth, name):
    if name == "headline":
        return Mamba2Runner(torch, rs, synth, HEADLINE)
    return VARIANTS[name][1](torch, rs, synth)


def profile_variant(torch, rs, synth, name, K, W, out_path):
    """The dispatches a counter run profiles: ``W`` then ``K`` dispatches of one variant
    (rounded to whole windows for decode), untimed, then the 1 GiB calibration copy.
    Writes the kernel name, its dispatch count and their average algorithmic bytes."""
    r = make_runner(torch, rs, synth, name)
    n = -(-(W + K) // r.period) * r.period
    for i in range(n):
        r.launch(i)
    torch.cuda.synchronize()
    r.check(n)
    info = dict(variant=name, kernel=r.tag, sources=r.sources, dispatches=n,
                algorithmic_bytes_per_dispatch=sum(r.bytes_of(i) for i in range(n)) / n)
    del r
    torch.cuda.empty_cache()
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)   # the counter calibration: 1 GiB read + 1 GiB write
    torch.cuda.synchronize()
    os.makedirs(os.path.dirname(os.path.abspath(out_path)), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(info, f)
    print(json.dumps(info))


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


SQ_SIMDS = 1024          # 256 CUs x 4 SIMDs
SQ_CLOCK_HZ = 2.4e9


def sq_summarize(info_path, dirs, command):
    """Summary of rocprofv3 --pmc runs of SQ instruction counters (one run per pass, each
    directory one pass) of one profiled variant: counts per dispatch and per wave, and the
    time the vector ALUs and the matrix cores would need for them if the work were spread
    evenly over the chip's 1024 SIMDs (one wave64 vector instruction per 4 cycles at
    2.4 GHz; matrix-core busy cycles as counted), to set against the kernel's time."""
    info = json.load(open(info_path))
    name = info["variant"]
    out_path = os.path.join(ROOT, "profiles", PMC_FILES[name].replace("_pmc.txt", "_sq.txt"))
    rows = []
    for d in dirs:
        rows.extend(_read_counter_csv(d))
    is_kernel = lambda n: info["kernel"] in n  # noqa: E731
    names = sorted({r["Counter_Name"] for r in rows if is_kernel(r.get("Kernel_Name", ""))})
    avg = {}
    for c in names:
        v, n = _avg_counter(rows, is_kernel, c)
        avg[c] = (v, n)
    waves = avg.get("SQ_WAVES", (None, 0))[0]
    lines = [f"# rocprofv3 SQ instruction counters: {name} ({VARIANTS[name][2] if name in VARIANTS else HEADLINE})",
             f"command: {command}",
             f"kernel: {info['kernel']}",
             f"kernel_source_sha256_16: {kernel_source_hash(info['sources'])}",
             "counter | per dispatch | per wave | dispatches"]
    for c in names:
        v, n = avg[c]
        lines.append(f"{c} | {v:.4g} | {v / waves:.1f} | {n}" if waves else f"{c} | {v:.4g} | - | {n}")
    if "SQ_INSTS_VALU" in avg:
        lines.append(f"vector ALU issue time if spread over {SQ_SIMDS} SIMDs: "
                     f"{avg['SQ_INSTS_VALU'][0] * 4 / SQ_SIMDS / SQ_CLOCK_HZ * 1e6:.1f} us per dispatch")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        lines.append(f"matrix-core busy time if spread over {SQ_SIMDS} SIMDs: "
                     f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'][0] / SQ_SIMDS / SQ_CLOCK_HZ * 1e6:.1f} us per dispatch")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_summarize(fetch_dir, write_dir, info_path, command):
    """Summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of one profiled
    variant, scaled by what the same counters read for the 1 GiB calibration copy."""
    info = json.load(open(info_path))
    name = info["variant"]
    out_path = os.path.join(ROOT, "profiles", PMC_FILES[name])
    fr, wr = _read_counter_csv(fetch_dir), _read_counter_csv(write_dir)
    is_kernel = lambda n: info["kernel"] in n  # noqa: E731
    is_copy = lambda n: "MulFunctor" in n  # the calibration kernel: 1 GiB read + 1 GiB write  # noqa: E731
    f_k, nf = _avg_counter(fr, is_kernel, "FETCH_SIZE")
    w_k, nw = _avg_counter(wr, is_kernel, "WRITE_SIZE")
    f_c, _ = _avg_counter(fr, is_copy, "FETCH_SIZE")
    w_c, _ = _avg_counter(wr, is_copy, "WRITE_SIZE")
    if None in (f_k, w_k, f_c, w_c):
        raise RuntimeError(f"missing counters for {info['kernel']} or the calibration copy")
    if nf != info["dispatches"] or nw != info["dispatches"]:
        raise RuntimeError(f"profiled {nf}/{nw} dispatches of {info['kernel']}, the run made {info['dispatches']}")
    f_scale = COPY_BYTES / (f_c * 1024.0)
    w_scale = COPY_BYTES / (w_c * 1024.0)
    traffic = f_k * 1024.0 * f_scale + w_k * 1024.0 * w_scale
    alg = info["algorithmic_bytes_per_dispatch"]
    lines = [f"# rocprofv3 HBM counters: {name} ({VARIANTS[name][2] if name in VARIANTS else HEADLINE})",
             f"command: {command}",
             f"kernel: rssm::{info['kernel']}",
             f"kernel_source_sha256_16: {kernel_source_hash(info['sources'])}",
             f"dispatches: {nf} (fetch run), {nw} (write run)",
             f"FETCH_SIZE_KiB_per_dispatch: {f_k:.1f}",
             f"WRITE_SIZE_KiB_per_dispatch: {w_k:.1f}",
             f"copy_calibration: {COPY_BYTES} B device copy reads FETCH_SIZE {f_c:.1f} KiB, WRITE_SIZE {w_c:.1f} KiB",
             f"scale_fetch: {f_scale:.4f}",
             f"scale_write: {w_scale:.4f}",
             f"fetch_bytes_per_launch: {f_k * 1024.0 * f_scale:.0f}",
             f"write_bytes_per_launch: {w_k * 1024.0 * w_scale:.0f}",
             f"traffic_bytes_per_launch: {traffic:.0f}",
             f"algorithmic_bytes_per_launch: {alg:.0f}",
             f"traffic_over_algorithmic: {traffic / alg:.4f}"]
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _summary_kv(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def committed_traffic(name):
    """Counter-measured bytes per launch of a variant from its committed summary, if the
    summary matches the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", PMC_FILES[name])
    if not os.path.exists(path):
        return None
    kv = _summary_kv(path)
    sources = MAMBA2_SOURCES if "mamba2" in kv.get("kernel", "") else GDN_SOURCES
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    return dict(traffic=float(kv["traffic_bytes_per_launch"]), ratio=float(kv["traffic_over_algorithmic"]),
                fetch=float(kv["fetch_bytes_per_launch"]), write=float(kv["write_bytes_per_launch"]),
                source=os.path.relpath(path, ROOT))


def committed_traffic_reason(name):
    path = os.path.join(ROOT, "profiles", PMC_FILES[name])
    if not os.path.exists(path):
        return "no counter summary committed"
    return "kernel source changed since the counters were taken"


def stats_summarize(stats_dir, out_path, command, bench_json):
    """Write the per-kernel summary of a ``rocprofv3 --kernel-trace --stats`` run of the
    default bench command, with the headline kernel's dispatches split into flush and
    non-flush steps (the headline runner's dispatches come first and step the cursor by
    one each, from 0)."""
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_stats.csv under {stats_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    tag = REPLAY_KERNEL_TAG
    lines = ["# rocprofv3 --kernel-trace --stats: kernels of one bench.py run (sorted by total time)",
             f"command: {command}",
             f"kernel_source_sha256_16: {kernel_source_hash(MAMBA2_SOURCES)}",
             "calls | avg_us | min_us | max_us | total_ms | kernel"]
    for r in rows:
        lines.append("%5d | %8.1f | %8.1f | %8.1f | %8.2f | %s" % (
            int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e6, r["Name"][:160]))
    traces = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    hd = line["headline_dispatches"]
    if traces:
        disp = [r for r in csv.DictReader(open(traces[0])) if tag in r["Kernel_Name"]]
        disp.sort(key=lambda r: int(r["Start_Timestamp"]))
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp[:hd["total"]]]
        timed = [d for i, d in enumerate(dur) if any(f <= i < f + line["steps"] for f in hd["timed_firsts"])]
        lines.append(f"headline kernel: rssm::{tag}")
        lines.append(f"headline timed dispatches: {len(timed)} ({len(hd['timed_firsts'])} regions of "
                     f"{line['steps']}), average {sum(timed) / len(timed):.1f} us, min {min(timed):.1f}, "
                     f"max {max(timed):.1f}; bench median region average {line['roofline']['avg_launch_us']:.1f} us")
        from hybrid_model_ssm_amd import synth
        w = synth.WORKLOADS[HEADLINE]
        L = w["buffer_len"]
        shape = (w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"], L, 2)
        for nm, cs in (("non-flush", range(L - 1)), ("flush", [L - 1])):
            d = [t for i, t in enumerate(dur) if i % L in cs]
            nbytes = sum(mamba2_replay_bytes(*shape, c) for c in cs) / len(cs)
            if d:
                avg = sum(d) / len(d)
                lines.append(f"headline {nm} steps (cursor {cs[0]}..{cs[-1]}): {len(d)} dispatches, "
                             f"average {avg:.1f} us, min {min(d):.1f}, max {max(d):.1f}; "
                             f"{nbytes / 1e6:.1f} MB algorithmic -> {nbytes / avg / 1e3:.0f} GB/s")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:14]))


# ------------------------------------------------------------------------------------

def headline_device_model(synth, ceil, split, head, K):
    """The headline's steps timed at the device's own rates from this run's probes (see
    ``step_model_seconds``), against the measured per-step split and timed regions."""
    w = synth.WORKLOADS[HEADLINE]
    B, H, P, N, G, L = w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"], w["buffer_len"]
    io = 2 if w["io"] == "bf16" else 4
    read_bps = ceil["read_gbps"] * 1e9
    inplace_name = "inplace_nt_nt_r8_tpw16"          # the replay kernel's shape
    inplace_bps = ceil["probes"][inplace_name]["gbps"] * 1e9
    rtw = ceil["read_then_write"]
    points = [(m, us * 1e-6) for m, us in zip(rtw["written_MiB"], rtw["us"])]
    wsec = lambda nbytes: write_cost_seconds(nbytes, points)  # noqa: E731
    steps = [mamba2_replay_rw(B, H, P, N, G, L, io, c) for c in range(L)]
    secs = [step_model_seconds(r, wr, ip, read_bps, inplace_bps, wsec) for r, wr, ip in steps]
    nonflush = sum(secs[:-1]) / (L - 1)
    flushes = head["flush_dispatches_per_region"]
    region = (flushes * secs[-1] + (K - flushes) * nonflush) / K
    window = sum(secs) / L
    window_bytes = sum(r + wr for r, wr, _ in steps) / L
    return dict(read_gbps=ceil["read_gbps"], read_probe=ceil["read_probe"], inplace_gbps=inplace_bps / 1e9,
                inplace_probe=inplace_name,
                nonflush_written_MiB=steps[0][1] / MiB, nonflush_write_us=wsec(steps[0][1]) * 1e6,
                nonflush_us=nonflush * 1e6, flush_us=secs[-1] * 1e6, window_us_per_step=window * 1e6,
                window_frac_of_peak=window_bytes / window / 1e9 / PEAK_GBPS,
                region_us_per_step=region * 1e6,
                measured_of_model=dict(nonflush=nonflush * 1e6 / split["nonflush_us"],
                                       flush=secs[-1] * 1e6 / split["flush_us"],
                                       region=region * 1e3 / head["ms_per_dispatch"]),
                note="reads at the best read probe, the flushed checkpoint at the in-place probe in the "
                     "replay kernel's shape, other writes at the read-then-write probe's extra time for "
                     "their volume")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="decode steps per timed region of the headline")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--repeats", type=int, default=5, help="timed regions per measurement (median reported)")
    ap.add_argument("--only", default="all",
                    help="all, headline, or a comma list of: " + ",".join(GROUPS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=256)
    ap.add_argument("--cpu-steps", type=int, default=32)
    ap.add_argument("--profile-variant", metavar="NAME", choices=["headline"] + sorted(VARIANTS),
                    help="run W+K dispatches of one variant untimed and the calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--profile-out", default="profile_variant.json")
    ap.add_argument("--pmc-summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "PROFILE_JSON"))
    ap.add_argument("--sq-summarize", nargs="+", metavar="PROFILE_JSON PASS_DIR",
                    help="SQ instruction-counter passes of one profiled variant into a summary")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--stats-summarize", nargs=2, metavar=("STATS_DIR", "BENCH_JSON"))
    ap.add_argument("--precision-sweep", action="store_true",
                    help="print the emulated read/recurrence precision sweep (one JSON line) and exit")
    args = ap.parse_args(argv)

    if args.stats_summarize:
        stats_summarize(args.stats_summarize[0], STATS_SUMMARY, args.pmc_command, args.stats_summarize[1])
        return 0
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize, args.pmc_command)
        return 0
    if args.sq_summarize:
        sq_summarize(args.sq_summarize[0], args.sq_summarize[1:], args.pmc_command)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode path has no cross-GPU exchange); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.repeats < 1:
        print("--steps and --repeats must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    # the CPU oracle's worker pool is forked before this process touches the GPU
    oracle_runs = None
    if not args.no_cpu_baseline and not args.precision_sweep and not args.profile_variant:
        from hybrid_model_ssm_amd import synth as synth_cpu
        oracle_runs = cpu_oracle_run(synth_cpu, args.cpu_seqs, args.cpu_steps)
        for x in oracle_runs:
            print(f"[bench] cpu oracle {x['workload']} {x['form']}: {x['nseq']} sequences x {x['steps']} steps on "
                  f"{x['workers']} worker processes in {x['wall']:.1f} s", file=sys.stderr, flush=True)

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
    if args.profile_variant:
        profile_variant(torch, rs, synth, args.profile_variant, args.steps, args.warmup, args.profile_out)
        return 0

    # ---- headline: every timed region starts at a flush step, so a region of K steps holds
    # ceil(K / L) flushes (K a multiple of L: exactly K / L, the true rate) --------------------
    hr = Mamba2Runner(torch, rs, synth, HEADLINE)
    L = hr.L
    regions, setup, done = measure(torch, hr, args.warmup, args.steps, args.repeats, start_at=L - 1)
    head = summarize(regions, args.steps)
    while done % L:                       # the per-step split covers two whole windows
        hr.launch(done)
        done += 1
    split, done = per_step_split(torch, hr, done, 2 * L)
    hr.check(done)
    head_dispatches = dict(total=done, setup=setup, timed_firsts=[g["first"] for g in regions])
    del hr
    torch.cuda.empty_cache()
    print(f"[bench] headline {head['value']:.4g} seq-tok/s, {head['hbm_gbps']:.0f} GB/s "
          f"(flush steps {split['flush_us']:.1f} us, others {split['nonflush_us']:.1f} us)",
          file=sys.stderr, flush=True)
    avg_s = head["ms_per_dispatch"] / 1e3
    nbytes_per_launch = head["bytes_per_dispatch_MiB"] * MiB
    tr = committed_traffic("headline")
    roofline = dict(bound="hbm", achieved=nbytes_per_launch / avg_s / 1e9, peak=PEAK_GBPS, unit="GB/s",
                    frac=nbytes_per_launch / avg_s / 1e9 / PEAK_GBPS, traffic=tr["traffic"] if tr else None,
                    traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    traffic_over_algorithmic=tr["ratio"] if tr else None,
                    traffic_gbps=tr["traffic"] / avg_s / 1e9 if tr else None,
                    traffic_frac=tr["traffic"] / avg_s / 1e9 / PEAK_GBPS if tr else None,
                    traffic_source=tr["source"] if tr else committed_traffic_reason("headline"),
                    kernel=f"rssm::{REPLAY_KERNEL_TAG}", algorithmic_bytes_per_launch=nbytes_per_launch,
                    avg_launch_us=avg_s * 1e6, launches=args.steps)

    groups = set(GROUPS) if args.only == "all" else set(args.only.split(",")) - {"headline"}   # the headline always runs
    unknown = groups - set(GROUPS)
    if unknown:
        print(f"unknown --only groups: {sorted(unknown)}", file=sys.stderr)
        return 2
    variants = {}
    for name, (group, _, _, _) in VARIANTS.items():
        if group in groups:
            variants[name] = time_variant(torch, rs, synth, name, args.steps, args.warmup, args.repeats)
            print(f"[bench] {name}: {variants[name]['value']:.4g} {variants[name]['unit']}, "
                  f"{variants[name]['hbm_gbps']:.0f} GB/s", file=sys.stderr, flush=True)
    if "graph" in groups:
        variants["mamba2_h128_replay_graph"] = time_graph(torch, rs, synth, args.steps, args.warmup, args.repeats)
    ceil = ceiling(torch) if args.only == "all" else None
    cpu = None
    if oracle_runs is not None:
        cpu = cpu_baseline(torch, rs, synth, oracle_runs)
        print(f"[bench] cpu baseline {cpu['value']:.4g} seq-tok/s in {cpu['seconds']:.1f}s", file=sys.stderr,
              flush=True)
        if not cpu["gpu_parity_ok"]:
            raise RuntimeError(f"GPU outputs disagree with the oracle: {cpu['gpu_parity_max_violation']}")

    model = headline_device_model(synth, ceil, split, head, args.steps) if ceil else None
    conv = variants.get("mamba2_h128_conventional")
    ratios = {}
    pairs = [("mamba2_h128", None, "mamba2_h128_conventional"),
             ("mamba2_h64", "mamba2_h64_replay", "mamba2_h64_conventional"),
             ("gdn_hv32", "gdn_hv32_replay", "gdn_hv32_conventional"),
             ("mamba2_spec_h128", "spec_h128_verify", "spec_h128_snapshot_baseline"),
             ("gdn_spec_hv32", "gdn_spec_hv32_verify", "gdn_spec_hv32_snapshot_baseline")]
    for wl, rep_name, conv_name in pairs:
        rv = head if rep_name is None else variants.get(rep_name)
        cv = variants.get(conv_name)
        if rv and cv:
            ent = dict(speedup=rv["value"] / cv["value"],
                       algorithmic_bytes_ratio=cv["bytes_per_dispatch_MiB"] / rv["bytes_per_dispatch_MiB"])
            rt = tr if rep_name is None else committed_traffic(rep_name)
            ct = committed_traffic(conv_name)
            if rt and ct:
                ent["measured_traffic_ratio"] = ct["traffic"] / rt["traffic"]
            ratios[wl] = ent
    w = synth.WORKLOADS[HEADLINE]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "seq-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_dispatch"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "batch": w["batch"], "nheads": w["nheads"], "headdim": w["headdim"],
                   "dstate": w["dstate"], "ngroups": w["ngroups"], "buffer_len": w["buffer_len"],
                   "io_dtype": w["io"], "checkpoint": "f32", "checkpoint_reads": "f32",
                   "parallelism": "single GPU"},
        "timing": {"timed_regions": args.repeats, "statistic": "median region",
                   "values_per_region": head["values_per_region"],
                   "flush_steps_per_region": head["flush_dispatches_per_region"],
                   "flush_steps_true_rate": args.steps / L,
                   "region_start": "a flush step (cursor L-1)", "setup_steps": setup},
        "step_split": split,
        "headline_dispatches": head_dispatches,
        "hbm_gbps": head["hbm_gbps"],
        "hbm_frac_of_peak": head["frac_of_peak"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "speedup_vs_conventional": (head["value"] / conv["value"]) if conv else None,
        "replay_vs_conventional": ratios,
        "variants": variants,
        "ceiling": ceil,
        "device_model": model,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
