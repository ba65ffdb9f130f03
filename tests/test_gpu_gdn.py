"""GPU parity: Gated DeltaNet replay decode and the conventional GDN kernel against the
fp64 oracle (max |d| <= 1e-4 (1 + |ref|); cursors bit for bit)."""

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


class GpuGdn:
    def __init__(self, desc, static):
        self.desc = desc
        B = desc.batch
        self.state = rs.GdnState.allocate(desc, ckpt=to_dev(static.ckpt, torch.float32))
        self.cur = [torch.zeros(B, dtype=torch.int32, device=DEV), torch.zeros(B, dtype=torch.int32, device=DEV)]
        self.flip = 0
        self.out = torch.empty(B, desc.num_v_heads, desc.dv, dtype=torch.float32, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.conv_state = to_dev(static.ckpt, torch.float32)
        self.conv_out = torch.empty_like(self.out)

    @property
    def cursor(self):
        return self.cur[self.flip]

    def _in(self, s):
        io = self.desc.torch_io
        return ([to_dev(s[k], io) for k in ("q", "k", "v")] +
                [to_dev(s[k], torch.float32) for k in ("alpha", "beta")])

    def step(self, s):
        q, k, v, al, be = self._in(s)
        rs.gdn_decode(self.desc, self.state, self.cur[self.flip], self.cur[1 - self.flip], q, k, v, al, be,
                      self.out, self.err)
        self.flip ^= 1
        return self.out

    def conventional(self, s):
        q, k, v, al, be = self._in(s)
        rs.gdn_conventional_decode(self.desc, self.conv_state, q, k, v, al, be, self.conv_out)
        return self.conv_out

    def flush(self):
        rs.gdn_flush(self.desc, self.state, self.cur[self.flip], self.cur[1 - self.flip], self.err)
        self.flip ^= 1


SHAPES = [  # B, HV, HK, dk, dv, L, io
    (2, 4, 2, 64, 64, 4, "f32"),
    (3, 4, 4, 128, 128, 5, "bf16"),
    (2, 6, 2, 128, 64, 4, "bf16"),
    (2, 2, 1, 64, 128, 3, "f32"),
    (4, 8, 4, 128, 128, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}HV{}HK{}dk{}dv{}L{}{}".format(*s))
def test_gdn_replay_and_conventional(shape):
    B, HV, HK, dk, dv, L, io = shape
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io=io, seed=31)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16 if io == "bf16" else rs.F32)
    gpu = GpuGdn(desc, st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    S = st.ckpt.astype(np.float64)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        S, ref = og.conventional_step(S, **s)
        rref, _ = rep.step(**s)
        out = gpu.step(s).cpu().numpy()
        assert_fp32_close(out, ref, f"{shape} replay step {t}")
        assert_fp32_close(out, rref, f"{shape} replay vs replay-oracle step {t}")
        assert_fp32_close(gpu.conventional(s).cpu().numpy(), ref, f"{shape} conventional step {t}")
        assert_fp32_close(gpu.conv_state.cpu().numpy(), S, f"{shape} conventional state step {t}")
        assert np.array_equal(gpu.cursor.cpu().numpy(), np.full(B, t % L, np.int32))
        if t % L == 0:
            assert_fp32_close(gpu.state.ckpt.cpu().numpy(), S, f"{shape} checkpoint step {t}")
    assert gpu.err.item() == 0


def test_gdn_mixed_cursor_phases_with_preloaded_records():
    """Sequences start at different cursors with records already in their buffers (k and v
    rows, and the slot-major alpha/beta rows), so one launch mixes flushing and
    non-flushing sequences: outputs, cursors and every folded checkpoint against the
    oracle over two flushes of each sequence."""
    B, HV, HK, dk, dv, L = 5, 4, 2, 128, 128, 8
    rng = np.random.default_rng(7)
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=31)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdn(desc, st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    cursors = np.array([0, 7, 3, 6, 1], np.int32)
    kk = rng.standard_normal((B, HK, L, dk))
    rec_k = synth.round_bf16((kk / np.linalg.norm(kk, axis=-1, keepdims=True)).astype(np.float32))
    rec_v = synth.round_bf16(rng.standard_normal((B, HV, L, dv)).astype(np.float32))
    rec_al = rng.uniform(0.5, 1.0, (B, L, HV)).astype(np.float32)
    rec_be = rng.uniform(0.0, 1.0, (B, L, HV)).astype(np.float32)
    gpu.state.rec_k.copy_(to_dev(rec_k, torch.bfloat16))
    gpu.state.rec_v.copy_(to_dev(rec_v, torch.bfloat16))
    gpu.state.rec_alpha.copy_(to_dev(rec_al, torch.float32))
    gpu.state.rec_beta.copy_(to_dev(rec_be, torch.float32))
    gpu.cur[0].copy_(torch.from_numpy(cursors))
    for b in range(B):
        rep.records[b] = [(og.heads_of_kgroups(rec_k[b, :, s], HV), rec_v[b, :, s].astype(np.float64),
                           rec_al[b, s].astype(np.float64), rec_be[b, s].astype(np.float64))
                          for s in range(cursors[b])]
    for t in range(1, 2 * L + 2):
        s = gen.step()
        ref, flushed = rep.step(**s)
        assert_fp32_close(gpu.step(s).cpu().numpy(), ref, f"step {t}")
        assert np.array_equal(gpu.cursor.cpu().numpy(), rep.cursor)
        for b in np.nonzero(flushed)[0]:
            assert_fp32_close(gpu.state.ckpt[b].cpu().numpy(), rep.ckpt[b], f"seq {b} checkpoint step {t}")
    assert gpu.err.item() == 0


def test_gdn_full_size_sampled():
    """B=256, 32 value heads over 16 q/k heads, dk=dv=128, L=16: 2L+2 steps, 8 sampled
    sequences against the oracle."""
    w = synth.WORKLOADS["gdn_hv32"]
    gen = synth.gdn_inputs("gdn_hv32")
    st = gen.static
    B, L = w["batch"], w["buffer_len"]
    desc = rs.GdnDesc(B, w["num_v_heads"], w["num_k_heads"], w["dk"], w["dv"], L, rs.BF16)
    gpu = GpuGdn(desc, st)
    sample = np.array([0, 2, 50, 127, 128, 199, 254, 255])
    rep = og.GDNReplay(st.ckpt[sample], L, w["num_k_heads"])
    S = st.ckpt[sample].astype(np.float64)
    idx = torch.from_numpy(sample).to(DEV)
    for t in range(1, 2 * L + 3):
        s = gen.step()
        ss = {k: v[sample] for k, v in s.items()}
        ref, _ = rep.step(**ss)
        S, _ = og.conventional_step(S, **ss)
        out = gpu.step(s)
        assert_fp32_close(out[idx].cpu().numpy(), ref, f"step {t}")
        assert torch.equal(gpu.cursor, torch.full((B,), t % L, dtype=torch.int32, device=DEV))
        if t % L == 0:
            assert_fp32_close(gpu.state.ckpt[idx].cpu().numpy(), S, f"checkpoint step {t}")


def test_gdn_explicit_flush_and_bad_cursor():
    B, HV, HK, dk, dv, L = 3, 4, 2, 128, 128, 16
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=32)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdn(desc, st)
    S = st.ckpt.astype(np.float64)
    for t in range(6):
        s = gen.step()
        S, _ = og.conventional_step(S, **s)
        gpu.step(s)
    gpu.flush()
    assert gpu.cursor.cpu().tolist() == [0] * B
    assert_fp32_close(gpu.state.ckpt.cpu().numpy(), S, "explicit flush")
    ck = gpu.state.ckpt.clone()
    gpu.flush()
    assert torch.equal(gpu.state.ckpt, ck)
    gpu.cur[gpu.flip].copy_(torch.tensor([0, -1, 2], dtype=torch.int32))
    gpu.out.fill_(7.0)
    gpu.step(gen.step())
    assert gpu.err.item() & rs.DEVERR_CURSOR
    assert torch.all(gpu.out[1] == 7.0)
    assert gpu.cursor.cpu().tolist() == [1, -1, 3]


def test_gdn_L1_equals_conventional_kernel():
    B, HV, HK, dk, dv = 2, 4, 2, 128, 128
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=33)
    st = gen.static
    gpu = GpuGdn(rs.GdnDesc(B, HV, HK, dk, dv, 1, rs.BF16), st)
    for t in range(5):
        s = gen.step()
        o = gpu.step(s).clone()
        c = gpu.conventional(s)
        assert_fp32_close(o.cpu().numpy(), c.cpu().numpy(), f"step {t}", rel=1e-5)
        assert_fp32_close(gpu.state.ckpt.cpu().numpy(), gpu.conv_state.cpu().numpy(), f"state {t}", rel=1e-5)


def test_gdn_largest_window_L64():
    B, HV, HK, dk, dv, L = 2, 2, 1, 64, 64, 64
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=33)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdn(desc, st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        ref, flushed = rep.step(**s)
        assert_fp32_close(gpu.step(s).cpu().numpy(), ref, f"step {t}")
        if flushed.all():
            assert_fp32_close(gpu.state.ckpt.cpu().numpy(), rep.ckpt, f"checkpoint step {t}")
    assert np.array_equal(gpu.cursor.cpu().numpy(), np.full(B, (2 * L + 1) % L, np.int32))


def test_gdn_degenerate_gates():
    """Gates at their limits (alpha = 0, alpha = 1e-4 so that a window's gate products
    underflow in fp32, alpha = 1, beta = 0, see degenerate_gdn_gates) through two
    flushes: outputs and flushed checkpoints against the oracle, no NaN."""
    B, HV, HK, dk, dv, L = 2, 8, 2, 128, 128, 16
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=37)
    st = gen.static
    gpu = GpuGdn(rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16), st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    n_flush = 0
    for t in range(1, 2 * L + 2):
        s = degenerate_gdn_gates(gen.step(), t)
        ref, flushed = rep.step(**s)
        out = gpu.step(s).cpu().numpy()
        assert np.isfinite(out).all(), f"step {t}"
        assert_fp32_close(out, ref, f"step {t}")
        if flushed.all():
            n_flush += 1
            ck = gpu.state.ckpt.cpu().numpy()
            assert np.isfinite(ck).all(), f"checkpoint step {t}"
            assert_fp32_close(ck, rep.ckpt, f"checkpoint step {t}")
    assert n_flush == 2


def test_gdn_full_batch_small_heads():
    """Every one of B=256 sequences (4 value heads, 2 q/k heads, dk = dv = 128, L=16)
    for 2L+1 steps, two flushes included: outputs and flushed checkpoints of the whole
    batch against the oracle."""
    B, HV, HK, dk, dv, L = 256, 4, 2, 128, 128, 16
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=35)
    st = gen.static
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    gpu = GpuGdn(desc, st)
    rep = og.GDNReplay(st.ckpt, L, HK)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        ref, flushed = rep.step(**s)
        assert_fp32_close(gpu.step(s).cpu().numpy(), ref, f"step {t}")
        if flushed.all():
            assert_fp32_close(gpu.state.ckpt.cpu().numpy(), rep.ckpt, f"checkpoint step {t}")
    assert np.array_equal(gpu.cursor.cpu().numpy(), np.full(B, (2 * L + 1) % L, np.int32))
    assert gpu.err.item() == 0
