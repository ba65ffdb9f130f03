"""GPU parity: Gated DeltaNet speculative verification on the circular record buffer
against the fp64 oracle.  flushed/head/committed bit for bit; outputs and folded
checkpoints at max |d| <= 1e-4 (1 + |ref|) (the kernel reads the fp32 checkpoint; bf16
inputs are exact bf16 values on both sides)."""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from hybrid_model_ssm_amd import synth
from oracle import gdn as og
from tests.gpu_helpers import DEV, assert_fp32_close, degenerate_gdn_gates, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class GpuGdnSpec:
    def __init__(self, desc, static, n_pos):
        self.desc, self.n_pos = desc, n_pos
        B = desc.batch
        self.state = rs.GdnState.allocate(desc, ckpt=to_dev(static.ckpt, torch.float32))
        z = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
        self.head, self.committed, self.flushed = z(), z(), z()
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.out = torch.empty(B, n_pos, desc.num_v_heads, desc.dv, dtype=torch.float32, device=DEV)

    def verify(self, s):
        io = self.desc.torch_io
        q, k, v = (to_dev(s[n], io) for n in ("q", "k", "v"))
        al, be = (to_dev(s[n], torch.float32) for n in ("alpha", "beta"))
        rs.gdn_spec_verify(self.desc, self.state, self.head, self.committed, self.n_pos, q, k, v, al, be,
                           self.out, self.flushed, self.err)
        return self.out

    def commit(self, n_keep):
        rs.commit(self.desc.batch, self.desc.buffer_len, self.n_pos, self.head, self.committed, self.flushed,
                  torch.from_numpy(np.asarray(n_keep, np.int32)).to(DEV), self.err)


SHAPES = [  # B, HV, HK, dk, dv, L, n_pos, io
    (2, 4, 2, 64, 64, 5, 3, "f32"),
    (3, 8, 4, 128, 128, 16, 4, "bf16"),
    (2, 12, 2, 128, 64, 6, 2, "bf16"),     # 6 value heads per q/k head: two workgroups each
    (2, 2, 1, 64, 128, 4, 1, "f32"),       # one position: autoregressive decode on the ring
    (2, 4, 4, 128, 128, 4, 4, "bf16"),     # n_pos = L: every round after the first folds
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}HV{}HK{}dk{}dv{}L{}T{}{}".format(*s))
def test_gdn_spec_rounds_match_oracle(shape):
    B, HV, HK, dk, dv, L, T, io = shape
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io=io, seed=41)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16 if io == "bf16" else rs.F32)
    gpu = GpuGdnSpec(desc, st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
    n_flush = 0
    for r in range(3 * L):
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
                assert_fp32_close(gpu.state.ckpt[b].cpu().numpy(), spec.ckpt[b], f"round {r} seq {b} fold")
        n_flush += int(fl.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
        assert np.array_equal(gpu.head.cpu().numpy(), spec.head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), spec.committed.astype(np.int32))
    assert n_flush > 0 and gpu.err.item() == 0


def test_gdn_spec_every_draft_rejected_keeps_checkpoint_bit_identical():
    B, HV, HK, dk, dv, L, T = 4, 8, 4, 128, 128, 16, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=42)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdnSpec(desc, st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
    ck0 = gpu.state.ckpt.clone()
    for r in range(L - T + 1):          # committed grows by one per round: no fold yet
        s = gen.step(n_pos=T)
        ref, _ = spec.verify(**s)
        assert_fp32_close(gpu.verify(s).cpu().numpy(), ref, f"round {r}")
        assert gpu.flushed.sum().item() == 0
        assert torch.equal(gpu.state.ckpt, ck0)
        spec.commit(np.ones(B, int))
        gpu.commit(np.ones(B, int))


def test_gdn_spec_full_size_sampled():
    """Gated DeltaNet speculative workload at full shape (B=256, 32 value heads, 16 q/k
    heads, dk = dv = 128, L=16, 4 positions): 12 rounds, 8 sampled sequences against the
    oracle, cursors of the whole batch bit for bit."""
    w = synth.WORKLOADS["gdn_spec_hv32"]
    B, HV, HK, dk, dv, L, T = (w[k] for k in ("batch", "num_v_heads", "num_k_heads", "dk", "dv",
                                               "buffer_len", "n_pos"))
    gen = synth.gdn_inputs("gdn_spec_hv32")
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdnSpec(desc, st, T)
    sample = np.array([0, 5, 64, 127, 128, 191, 250, 255])
    spec = og.GDNSpec(st.ckpt[sample], L, HK)
    all_head = np.zeros(B, np.int64)
    all_com = np.zeros(B, np.int64)
    for r in range(12):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**{k: v[sample] for k, v in s.items()})
        out = gpu.verify(s)
        assert_fp32_close(out[torch.from_numpy(sample).to(DEV)].cpu().numpy(), ref, f"round {r}")
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, (all_com + T > L).astype(np.int32))
        assert np.array_equal(fl[sample], fl_ref.astype(np.int32))
        spec.commit(n_keep[sample])
        gpu.commit(n_keep)
        all_head = np.where(fl == 1, (all_head + all_com) % L, all_head)
        all_com = np.where(fl == 1, 0, all_com) + n_keep
        assert np.array_equal(gpu.head.cpu().numpy(), all_head.astype(np.int32))
        assert np.array_equal(gpu.committed.cpu().numpy(), all_com.astype(np.int32))
    assert gpu.err.item() == 0


def test_gdn_snapshot_baseline_matches_conventional_oracle():
    B, HV, HK, dk, dv, T = 3, 8, 4, 128, 128, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=44)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, 16, rs.BF16)
    snaps = torch.zeros(B, T, HV, dv, dk, dtype=torch.float32, device=DEV)
    snaps[:, 0] = to_dev(st.ckpt, torch.float32)
    slot = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.empty(B, T, HV, dv, dtype=torch.float32, device=DEV)
    S_kept = st.ckpt.astype(np.float64)
    for r in range(6):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        q, k, v = (to_dev(s[n], torch.bfloat16) for n in ("q", "k", "v"))
        al, be = (to_dev(s[n], torch.float32) for n in ("alpha", "beta"))
        rs.gdn_spec_baseline(desc, snaps, slot, T, q, k, v, al, be, out)
        S = S_kept
        states = []
        for j in range(T):
            S, o = og.conventional_step(S, **{n: a[:, j] for n, a in s.items()})
            states.append(S)
            assert_fp32_close(out[:, j].cpu().numpy(), o, f"round {r} pos {j}")
            assert_fp32_close(snaps[:, j].cpu().numpy(), S, f"round {r} snapshot {j}")
        S_kept = np.stack([states[n_keep[b] - 1][b] for b in range(B)])
        slot.copy_(torch.from_numpy((n_keep - 1).astype(np.int32)))


def test_gdn_spec_bad_cursor_skips_sequence():
    B, HV, HK, dk, dv, L, T = 3, 4, 2, 64, 64, 8, 2
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="f32", seed=43)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.F32)
    gpu = GpuGdnSpec(desc, st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
    gpu.committed.copy_(torch.tensor([0, L + 1, 0], dtype=torch.int32))   # sequence 1 invalid
    gpu.out.fill_(7.0)
    gpu.flushed.fill_(5)
    s = gen.step(n_pos=T)
    ref, _ = spec.verify(**s)
    out = gpu.verify(s).cpu().numpy()
    assert gpu.err.item() & rs.DEVERR_CURSOR
    assert np.all(out[1] == 7.0) and gpu.flushed[1].item() == 0      # skipped: reports no flush
    assert torch.equal(gpu.state.rec_v[1], torch.zeros_like(gpu.state.rec_v[1]))
    assert_fp32_close(out[[0, 2]], ref[[0, 2]], "valid sequences")


def test_gdn_spec_rejects_bad_arguments():
    desc = rs.GdnDesc(2, 4, 2, 128, 128, 8, rs.BF16)
    st = rs.GdnState.allocate(desc)
    T = 4
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=DEV)  # noqa: E731
    q, k, v = z(2, T, 2, 128), z(2, T, 2, 128), z(2, T, 4, 128)
    al, be = z(2, T, 4, dt=torch.float32), z(2, T, 4, dt=torch.float32)
    out = z(2, T, 4, 128, dt=torch.float32)
    hd, cm, fl = (z(2, dt=torch.int32) for _ in range(3))
    with pytest.raises(rs.ReplaySSMError):
        rs.gdn_spec_verify(desc, st, hd, cm, 9, q, k, v, al, be, out, fl)      # n_pos > L
    with pytest.raises(rs.ReplaySSMError):
        rs.gdn_spec_verify(desc, st, hd, hd, T, q, k, v, al, be, out, fl)      # head aliases committed
    big = rs.GdnDesc(2, 8, 2, 128, 128, 64, rs.F32)
    with pytest.raises(rs.ReplaySSMError):                                     # LDS staging too large
        rs.gdn_spec_verify(big, rs.GdnState.allocate(big), hd, cm, 64, z(2, 64, 2, 128, dt=torch.float32),
                           z(2, 64, 2, 128, dt=torch.float32), z(2, 64, 8, 128, dt=torch.float32),
                           z(2, 64, 8, dt=torch.float32), z(2, 64, 8, dt=torch.float32),
                           z(2, 64, 8, 128, dt=torch.float32), fl)


@pytest.mark.parametrize("B", [256, 300])
def test_gdn_spec_full_batch_small_heads(B):
    """All sequences of a full batch (4 value heads, 2 q/k heads, dk = dv = 128, L=16,
    4 positions) for 10 rounds against the oracle.  Workgroups take the folding
    sequences first; B=300 spans two 256-sequence chunks of that ordering."""
    HV, HK, dk, dv, L, T = 4, 2, 128, 128, 16, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=45)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdnSpec(desc, st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
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


def test_gdn_spec_batch_above_ranking_limit():
    """A batch above the speculative ranking's limit (1024 sequences) keeps batch order:
    B=1100 (2 value heads, 1 q/k head, dk = dv = 64, L=16, 4 positions) for 6 rounds with
    folds against the oracle."""
    B, HV, HK, dk, dv, L, T = 1100, 2, 1, 64, 64, 16, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=46)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdnSpec(desc, st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
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


def test_gdn_spec_degenerate_gates():
    """Speculative rounds with gates at their limits (alpha = 0, alpha = 1e-4 so that a
    window's gate products underflow in fp32, alpha = 1, beta = 0) over several folds:
    outputs, flush flags and folded checkpoints against the oracle."""
    B, HV, HK, dk, dv, L, T = 2, 8, 4, 128, 128, 8, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=43)
    st = gen.static
    gpu = GpuGdnSpec(rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16), st, T)
    spec = og.GDNSpec(st.ckpt, L, HK)
    n_flush = 0
    for r in range(2 * L):
        s = degenerate_gdn_gates(gen.step(n_pos=T), r)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        out = gpu.verify(s).cpu().numpy()
        fl = gpu.flushed.cpu().numpy()
        assert np.array_equal(fl, fl_ref.astype(np.int32)), f"round {r}"
        assert np.isfinite(out).all(), f"round {r}"
        assert_fp32_close(out, ref, f"round {r}")
        for b in range(B):
            if fl[b]:
                assert_fp32_close(gpu.state.ckpt[b].cpu().numpy(), spec.ckpt[b], f"round {r} seq {b} fold")
        n_flush += int(fl.sum())
        spec.commit(n_keep)
        gpu.commit(n_keep)
    assert n_flush >= 2
