"""GPU parity: Mamba2 speculative verification on the circular record buffer, the
commit/reset cursor calls, and the per-position snapshot baseline, against the
fp64 oracle.  flushed/head/committed are compared bit for bit; outputs at
max |d| <= 1e-4 (1 + |ref|) (fp32 reads) or 2e-2 RMS (bf16 reads)."""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from hybrid_model_ssm_amd import synth
from oracle import mamba2 as om
from tests.gpu_helpers import DEV, assert_fp32_close, extreme_mamba2_dt, require_gpu, rms_violation, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class GpuSpec:
    def __init__(self, desc, static, n_pos, lowp=False):
        self.desc, self.n_pos = desc, n_pos
        B = desc.batch
        self.state = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=to_dev(static.ckpt, torch.float32))
        self.A = to_dev(static.A, torch.float32)
        self.D = to_dev(static.D, torch.float32)
        self.dt_bias = to_dev(static.dt_bias, torch.float32)
        z = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
        self.head, self.committed, self.flushed = z(), z(), z()
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.out = torch.empty(B, n_pos, desc.nheads, desc.headdim, dtype=torch.float32, device=DEV)
        if lowp:
            rs.mamba2_flush(desc, self.state, z(), z(), self.A, self.err)

    def verify(self, s):
        io = self.desc.torch_io
        x, z, B, C, dt = [to_dev(s[k], io) for k in ("x", "z", "B", "C", "dt_raw")]
        rs.mamba2_spec_verify(self.desc, self.state, self.head, self.committed, self.n_pos, x, z, B, C, dt,
                              self.dt_bias, self.A, self.D, self.out, self.flushed, self.err)
        return self.out

    def commit(self, n_keep):
        rs.commit(self.desc.batch, self.desc.buffer_len, self.n_pos, self.head, self.committed, self.flushed,
                  torch.from_numpy(np.asarray(n_keep, np.int32)).to(DEV), self.err)


def _setup(B, H, P, N, G, L, seed, lowp=False, n_pos=4):
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=seed)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    return gen, st, desc, GpuSpec(desc, st, n_pos, lowp=lowp)


def test_spec_rounds_match_oracle_and_rollback_is_free():
    B, H, P, N, G, L, T = 8, 16, 64, 128, 2, 16, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=21)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    n_flush = 0
    for r in range(40):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ck_before = gpu.state.ckpt.clone()
        ref, fl_ref = spec.verify(**s)
        out = gpu.verify(s).cpu().numpy()
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, fl_ref.astype(np.int32)), f"round {r}"
        assert_fp32_close(out, ref, f"round {r}")
        for b in range(B):
            if not fl[b]:
                assert torch.equal(gpu.state.ckpt[b], ck_before[b]), f"round {r}: checkpoint of seq {b} written"
            else:
                assert_fp32_close(gpu.state.ckpt[b].cpu().numpy(), spec.ckpt[b], f"round {r} seq {b} flush")
        n_flush += int(fl.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.head.cpu().numpy(), spec.head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32))
    assert n_flush > 0 and gpu.err.item() == 0


def test_spec_every_draft_rejected_keeps_checkpoint_bit_identical():
    B, H, P, N, G, L, T = 4, 8, 64, 128, 2, 16, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=22)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    ck0 = gpu.state.ckpt.clone()
    for r in range(L - T + 1):          # committed grows by one per round: no flush yet
        s = gen.step(n_pos=T)
        ref, _ = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"round {r}")
        assert gpu.flushed.sum().item() == 0
        assert torch.equal(gpu.state.ckpt, ck0)
        spec.commit(np.ones(B, int))
        gpu.commit(np.ones(B, int))


def test_spec_full_size_sampled():
    """Speculative workload at full shape (B=256, H=128, P=64, N=128, G=8, L=16, 4
    positions): 12 rounds, 8 sampled sequences against the oracle, cursors of the
    whole batch bit for bit."""
    w = synth.WORKLOADS["mamba2_spec_h128"]
    B, H, P, N, G, L, T = w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"], w["buffer_len"], w["n_pos"]
    gen = synth.mamba2_inputs("mamba2_spec_h128")
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    gpu = GpuSpec(desc, st, T)
    sample = np.array([0, 3, 64, 127, 128, 190, 254, 255])
    spec = om.Mamba2Spec(st.ckpt[sample], L, st.A, st.D, st.dt_bias, G)
    allspec_head = np.zeros(B, np.int64)
    allspec_com = np.zeros(B, np.int64)
    for r in range(12):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**{k: v[sample] for k, v in s.items()})
        out = gpu.verify(s)
        assert_fp32_close(out[torch.from_numpy(sample).to(DEV)].cpu().numpy(), ref, f"round {r}")
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, (allspec_com + T > L).astype(np.int32))
        assert np.array_equal(fl[sample], fl_ref.astype(np.int32))
        spec.commit(n_keep[sample])
        gpu.commit(n_keep)
        allspec_head = np.where(fl == 1, (allspec_head + allspec_com) % L, allspec_head)
        allspec_com = np.where(fl == 1, 0, allspec_com) + n_keep
        assert np.array_equal(gpu.head.cpu().numpy(), allspec_head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), allspec_com.astype(np.int32))
    assert gpu.err.item() == 0


def test_spec_bf16_read_copy():
    B, H, P, N, G, L, T = 8, 16, 64, 128, 2, 16, 4
    gen, st, desc, lp = _setup(B, H, P, N, G, L, seed=23, lowp=True)
    fp = GpuSpec(desc, st, T)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    for r in range(24):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, _ = spec.verify(**s)
        o_lp = lp.verify(s).cpu().numpy()
        o_fp = fp.verify(s).cpu().numpy()
        for j in range(T):
            v = rms_violation(o_lp[:, j], ref[:, j])
            assert v <= 1.0, f"round {r} pos {j}: {v:.3g}"
        assert_fp32_close(o_fp, ref, f"round {r}")
        assert torch.equal(lp.state.ckpt, fp.state.ckpt)
        assert torch.equal(lp.flushed, fp.flushed)
        spec.commit(n_keep)
        lp.commit(n_keep)
        fp.commit(n_keep)


def test_snapshot_baseline_matches_conventional_oracle():
    B, H, P, N, G, T = 4, 8, 64, 128, 2, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=24)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, 16, rs.BF16, True)
    snaps = torch.zeros(B, T, H, P, N, dtype=torch.float32, device=DEV)
    snaps[:, 0] = to_dev(st.ckpt, torch.float32)
    slot = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.empty(B, T, H, P, dtype=torch.float32, device=DEV)
    A, D, bias = (to_dev(a, torch.float32) for a in (st.A, st.D, st.dt_bias))
    h_kept = st.ckpt.astype(np.float64)
    for r in range(6):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        x, z, Bm, C, dt = [to_dev(s[k], torch.bfloat16) for k in ("x", "z", "B", "C", "dt_raw")]
        rs.mamba2_spec_baseline(desc, snaps, slot, T, x, z, Bm, C, dt, bias, A, D, out)
        h = h_kept
        hs = []
        for j in range(T):
            h, o = om.conventional_step(h, **{k: v[:, j] for k, v in s.items()}, dt_bias=st.dt_bias, A=st.A, D=st.D)
            hs.append(h)
            assert_fp32_close(out[:, j].cpu().numpy(), o, f"round {r} pos {j}")
            assert_fp32_close(snaps[:, j].cpu().numpy(), h, f"round {r} snapshot {j}")
        h_kept = np.stack([hs[n_keep[b] - 1][b] for b in range(B)])
        slot.copy_(torch.from_numpy((n_keep - 1).astype(np.int32)))


def test_commit_rejects_out_of_range_and_reset():
    B, L, T = 4, 16, 4
    head = torch.tensor([3, 5, 15, 0], dtype=torch.int32, device=DEV)
    com = torch.tensor([14, 2, 12, 0], dtype=torch.int32, device=DEV)
    flushed = torch.tensor([1, 0, 0, 0], dtype=torch.int32, device=DEV)
    n_keep = torch.tensor([4, 0, 3, 5], dtype=torch.int32, device=DEV)  # seq 1, 3 invalid
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rs.commit(B, L, T, head, com, flushed, n_keep, err)
    assert err.item() & rs.DEVERR_CURSOR
    assert head.cpu().tolist() == [(3 + 14) % 16, 5, 15, 0]
    assert com.cpu().tolist() == [4, 2, 15, 0]
    rs.reset_cursors(B, head, com, torch.tensor([0, 2, 9], dtype=torch.int32, device=DEV))
    assert head.cpu().tolist() == [0, 5, 0, 0] and com.cpu().tolist() == [0, 2, 0, 0]
    cur = torch.tensor([3, 4, 5, 6], dtype=torch.int32, device=DEV)
    rs.reset_cursors(B, None, cur)
    assert cur.cpu().tolist() == [0, 0, 0, 0]


def test_spec_positions_equal_buffer_length():
    """n_pos = L: every round after the first folds the committed records first."""
    B, H, P, N, G, L, T = 3, 4, 64, 64, 1, 4, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=25, n_pos=T)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    for r in range(10):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"round {r}")
        assert np.array_equal(gpu.flushed.cpu().numpy(), fl_ref.astype(np.int32))
        assert bool(fl_ref.all()) == (r > 0)
        spec.commit(n_keep)
        gpu.commit(n_keep)
    assert gpu.err.item() == 0


@pytest.mark.parametrize("B", [256, 300])
def test_spec_full_batch_small_heads(B):
    """All sequences of a full batch (H=8, G=2, P=64, N=128, L=16, 4 positions) for 10
    rounds: every output, flushed flag and cursor against the oracle.  Workgroups take
    the folding sequences first; B=300 spans two 256-sequence chunks of that ordering."""
    H, P, N, G, L, T = 8, 64, 128, 2, 16, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=26)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    n_flush = 0
    for r in range(10):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"round {r}")
        assert np.array_equal(gpu.flushed.cpu().numpy(), fl_ref.astype(np.int32))
        n_flush += int(fl_ref.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.head.cpu().numpy(), spec.head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32))
    assert n_flush > B // 2 and gpu.err.item() == 0


def test_spec_batch_above_ranking_limit():
    """A batch above the speculative ranking's limit (1024 sequences) keeps batch order:
    B=1100 (H=2, G=1, P=N=16, L=16, 4 positions) for 6 rounds with folds, every output,
    flushed flag and cursor against the oracle."""
    B, H, P, N, G, L, T = 1100, 2, 16, 16, 1, 16, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=27)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    n_flush = 0
    for r in range(6):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"round {r}")
        assert np.array_equal(gpu.flushed.cpu().numpy(), fl_ref.astype(np.int32))
        n_flush += int(fl_ref.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.head.cpu().numpy(), spec.head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32))
    assert n_flush > 0 and gpu.err.item() == 0


def test_spec_extreme_dt():
    """Speculative rounds with dt at its extremes (see extreme_mamba2_dt) over several
    folds: outputs, flush flags, folded checkpoints and cursors against the oracle."""
    B, H, P, N, G, L, T = 4, 8, 64, 128, 2, 8, 4
    gen, st, desc, gpu = _setup(B, H, P, N, G, L, seed=23, n_pos=T)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    n_flush = 0
    for r in range(2 * L):
        s = extreme_mamba2_dt(gen.step(n_pos=T), r)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        out = gpu.verify(s).cpu().numpy()
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, fl_ref.astype(np.int32)), f"round {r}"
        assert np.isfinite(out).all(), f"round {r}"
        assert_fp32_close(out, ref, f"round {r}")
        for b in range(B):
            if fl[b]:
                assert_fp32_close(gpu.state.ckpt[b].cpu().numpy(), spec.ckpt[b], f"round {r} seq {b} flush")
        n_flush += int(fl.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32))
    assert n_flush >= 2 and gpu.err.item() == 0
