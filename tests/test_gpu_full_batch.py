"""GPU parity over the whole batch of each full-size workload, at its real shape, for the
first 2L+1 steps (two flushes) or the first rounds of its speculative run.

The full runs (test_gpu_full_runs.py) follow 8 sampled sequences over every step; these
tests follow every one of the 256 sequences over the start of the run, where an indexing
mistake in any row, head or group of the grid would show: every output element, every
flushed checkpoint and the cursors of the whole batch against the oracle.  The Mamba2
autoregressive runs are checked against the oracle's conventional recurrence (the textbook
per-step update), GDN against its replay form and the speculative runs against the
speculative oracle with its commits.  Bars: max |d| <= 1e-4 (1 + |ref|) elementwise;
cursors, head, committed and flushed bit for bit.
"""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from hybrid_model_ssm_amd import synth
from oracle import gdn as og
from oracle import mamba2 as om
from tests.gpu_helpers import DEV, GpuMamba2, assert_fp32_close, require_gpu
from tests.test_gpu_gdn import GpuGdn
from tests.test_gpu_spec import GpuSpec

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mamba2_h64", "mamba2_h128"])
def test_mamba2_whole_batch_first_steps(name):
    w = synth.WORKLOADS[name]
    gen = synth.mamba2_inputs(name)
    st = gen.static
    B, L = w["batch"], w["buffer_len"]
    desc = rs.Mamba2Desc(B, w["nheads"], w["headdim"], w["dstate"], w["ngroups"], L, rs.BF16, True)
    gpu = GpuMamba2(desc, st)
    h = st.ckpt.astype(np.float64)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        h, ref = om.conventional_step(h, **s, dt_bias=st.dt_bias, A=st.A, D=st.D)
        assert_fp32_close(gpu.step(s).cpu().numpy(), ref, f"{name} step {t}")
        assert torch.equal(gpu.cursor, torch.full((B,), t % L, dtype=torch.int32, device=DEV)), f"step {t}"
        if t % L == 0:
            assert_fp32_close(gpu.state.ckpt.cpu().numpy(), h, f"{name} checkpoint step {t}")
        if t % 8 == 0:
            print(f"[whole batch] {name} step {t} of {2 * L + 1}", flush=True)
    assert gpu.err.item() == 0


@pytest.mark.timeout(600)
def test_mamba2_spec_whole_batch_first_rounds():
    name = "mamba2_spec_h128"
    w = synth.WORKLOADS[name]
    T = w["n_pos"]
    gen = synth.mamba2_inputs(name)
    st = gen.static
    B, L = w["batch"], w["buffer_len"]
    desc = rs.Mamba2Desc(B, w["nheads"], w["headdim"], w["dstate"], w["ngroups"], L, rs.BF16, True)
    gpu = GpuSpec(desc, st, T)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, w["ngroups"])
    n_flush = 0
    for r in range(12):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"{name} round {r}")
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, fl_ref.astype(np.int32)), f"round {r}"
        if fl.any():
            rows = torch.from_numpy(np.flatnonzero(fl)).to(DEV)
            assert_fp32_close(gpu.state.ckpt[rows].cpu().numpy(), spec.ckpt[fl.astype(bool)],
                              f"{name} round {r} folded checkpoints")
        n_flush += int(fl.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.head.cpu().numpy(), spec.head.astype(np.int32)), f"round {r}"
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32)), f"round {r}"
        if (r + 1) % 4 == 0:
            print(f"[whole batch] {name} round {r + 1} of 12", flush=True)
    assert n_flush > B and gpu.err.item() == 0      # most sequences fold at least twice


@pytest.mark.timeout(600)
def test_gdn_whole_batch_first_steps():
    name = "gdn_hv32"
    w = synth.WORKLOADS[name]
    gen = synth.gdn_inputs(name)
    st = gen.static
    B, HV, HK, dk, dv, L = (w[k] for k in ("batch", "num_v_heads", "num_k_heads", "dk", "dv", "buffer_len"))
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdn(desc, st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    n_flush = 0
    for t in range(1, 2 * L + 2):
        s = gen.step()
        ref, flushed = rep.step(**s)
        assert_fp32_close(gpu.step(s).cpu().numpy(), ref, f"{name} step {t}")
        assert torch.equal(gpu.cursor, torch.full((B,), t % L, dtype=torch.int32, device=DEV)), f"step {t}"
        if flushed.all():
            n_flush += 1
            assert_fp32_close(gpu.state.ckpt.cpu().numpy(), rep.ckpt, f"{name} checkpoint step {t}")
        else:
            assert not flushed.any()
        if t % 8 == 0:
            print(f"[whole batch] {name} step {t} of {2 * L + 1}", flush=True)
    assert n_flush == 2 and gpu.err.item() == 0
