"""GPU parity: low-precision read copies of the Mamba2 checkpoint (bf16, fp16, OCP E4M3
fp8 with row scales) against the read-copy oracle.

* The copy an explicit flush makes from a synthetic checkpoint equals the oracle's
  encoding bit for bit (codes and row scales), ties and subnormals included.
* Before the first flush the copy in use is the oracle's copy of the initial
  checkpoint, so outputs must match a replay from the dequantized copy at
  max |d| <= 1e-4 (1 + |ref|).
* At every step, outputs stay within the error the copy's rounding allows:
  |d| <= |g(z)| decay (eps . |C|) + 1e-4 (1 + |ref|), eps = half a unit in the last
  place of the format at each checkpoint element (oracle.readcopy.copy_error_bound),
  where decay (eps . |C|) g(z) is computed by a replay of eps with x = 0, D = 0.
* Flushes read and write fp32: the fp32 checkpoint trajectory is bit-identical to
  the run without a copy, and each refreshed copy is within eps of the oracle state.
"""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from hybrid_model_ssm_amd import synth
from oracle import mamba2 as om
from oracle import readcopy as rc
from tests.gpu_helpers import DEV, GpuMamba2, assert_fp32_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu

KINDS = ["bf16", "f16", "fp8"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _copy_values(state, kind):
    """Values the kernels read from a copy on the device (float64, host)."""
    if kind == "fp8":
        return rc.fp8_values(state.ckpt_lp.cpu().numpy(), state.lp_scale.cpu().numpy())
    return state.ckpt_lp.to(torch.float64).cpu().numpy()


def _oracle_copy(h, kind):
    if kind == "fp8":
        return rc.fp8_values(*rc.fp8_copy(h))
    return rc.bf16_copy(h) if kind == "bf16" else rc.f16_copy(h)


def _eps(h, kind):
    scale = rc.fp8_copy(h)[1] if kind == "fp8" else None
    return rc.copy_error_bound(h, kind, scale) * (1 + 1e-6) + 1e-30


def _assert_copy_near_state(state, kind, h, what):
    """The refreshed copy against the oracle state: the copy's own rounding (eps at h)
    plus what the fp32 fold may differ from fp64 (1e-5 relative, 2e-6 absolute for
    checkpoint entries of order 0.1 built from terms of order 1)."""
    got = _copy_values(state, kind)
    e = _eps(h, kind) + 1e-5 * np.abs(h) + 2e-6
    worst = float(np.max(np.abs(got - h) / e))
    assert worst <= 1.0, f"{what}: {worst:.3g} of the bound"


def _special_checkpoint(B, H, P, N, seed):
    rng = np.random.default_rng(seed)
    h = (0.1 * rng.standard_normal((B, H, P, N))).astype(np.float32)
    h[0, 0, 0] = 0.0                                            # zero row
    row = np.full(N, 2.0 ** -12, np.float32)                    # scale 1: exact ties for fp8
    ties = [448.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 0.0146484375, -232.0, 240.0, -0.0]
    row[:len(ties)] = ties
    h[0, 0, 1] = row
    h[0, 1, 3] *= np.float32(1e-5)                              # subnormal codes under one large entry
    h[0, 1, 3, 5] = 2.5
    h[1, 2, 7] = -h[1, 2, 7]
    return h


@pytest.mark.parametrize("kind", KINDS)
def test_copy_made_by_flush_is_the_oracle_encoding(kind):
    B, H, P, N, G, L = 2, 4, 64, 128, 2, 4
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    h = _special_checkpoint(B, H, P, N, seed=61)
    st = rs.Mamba2State.allocate(desc, lowp=kind, ckpt=torch.from_numpy(h).to(DEV))
    z = torch.zeros(B, dtype=torch.int32, device=DEV)
    rs.mamba2_flush(desc, st, z, torch.ones_like(z), torch.full((H,), -1.0, device=DEV))
    assert np.array_equal(st.ckpt.cpu().numpy(), h)              # an empty buffer leaves it as is
    if kind == "fp8":
        codes, scale = rc.fp8_copy(h)
        assert np.array_equal(st.ckpt_lp.cpu().numpy(), codes)
        assert np.array_equal(st.lp_scale.cpu().numpy(), scale)
    else:
        assert np.array_equal(_copy_values(st, kind), _oracle_copy(h, kind))


def _run(kind, B=4, H=8, P=64, N=128, G=2, L=8, seed=62, steps=None):
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=seed)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    lp = GpuMamba2(desc, st, lowp=kind)
    fp = GpuMamba2(desc, st)
    rep = om.Mamba2Replay(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    rep_q = om.Mamba2Replay(_oracle_copy(st.ckpt, kind), L, st.A, st.D, st.dt_bias, G)
    erep = om.Mamba2Replay(_eps(st.ckpt.astype(np.float64), kind), L, st.A, np.zeros(H), st.dt_bias, G)
    for t in range(1, (steps or 2 * L + 2) + 1):
        s = gen.step()
        ref, flushed = rep.step(**s)
        ref_q, _ = rep_q.step(**s)
        bound, _ = erep.step(x=np.zeros_like(s["x"]), z=s["z"], B=s["B"], C=np.abs(s["C"]), dt_raw=s["dt_raw"])
        out = lp.step(s).cpu().numpy()
        fp.step(s)
        tol = np.abs(bound) + 1e-4 * (1 + np.abs(ref))
        worst = float(np.max(np.abs(out - ref) / tol))
        assert worst <= 1.0, f"{kind} step {t}: {worst:.3g} of the bound"
        if t < L:
            assert_fp32_close(out, ref_q, f"{kind} step {t} vs replay of the copy")
        if flushed.all():
            assert torch.equal(lp.state.ckpt, fp.state.ckpt), f"{kind} step {t}: fp32 checkpoint differs"
            assert_fp32_close(lp.state.ckpt.cpu().numpy(), rep.ckpt, f"{kind} checkpoint step {t}")
            _assert_copy_near_state(lp.state, kind, rep.ckpt, f"{kind} copy step {t}")
            erep.ckpt = _eps(rep.ckpt, kind)
    assert lp.err.item() == 0


@pytest.mark.parametrize("kind", KINDS)
def test_decode_reads_the_copy_within_its_rounding(kind):
    _run(kind)


# heads per workgroup that take every path of the copy-tile ring: fewer heads than
# buffers, the unrolled loop, and each count of heads left for its tail (3 buffers for
# bf16 and fp16, 4 for fp8)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("heads", [3, 5, 6, 7, 11, 13])
def test_copy_ring_heads_per_workgroup(kind, heads):
    _run(kind, B=2, H=heads, P=64, N=128, G=1, L=4, seed=64 + heads)


@pytest.mark.parametrize("shape", [(2, 4, 64, 16, 1, 4), (2, 4, 128, 64, 2, 5), (2, 4, 32, 256, 2, 4)],
                         ids=lambda s: "P{}N{}".format(s[2], s[3]))
def test_fp8_copy_other_tile_shapes(shape):
    B, H, P, N, G, L = shape
    _run("fp8", B, H, P, N, G, L, seed=63)


def test_spec_verify_with_fp8_copy():
    B, H, P, N, G, L, T = 8, 16, 64, 128, 2, 16, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=64)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    state = rs.Mamba2State.allocate(desc, lowp="fp8", ckpt=to_dev(st.ckpt, torch.float32))
    fp_state = rs.Mamba2State.allocate(desc, ckpt=to_dev(st.ckpt, torch.float32))
    A, D, bias = (to_dev(a, torch.float32) for a in (st.A, st.D, st.dt_bias))
    zi = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
    head, com, fl = zi(), zi(), zi()
    head2, com2, fl2 = zi(), zi(), zi()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rs.mamba2_flush(desc, state, zi(), zi() + 1, A, err)           # create the copy
    out = torch.empty(B, T, H, P, dtype=torch.float32, device=DEV)
    out2 = torch.empty_like(out)
    spec = om.Mamba2Spec(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    espec = om.Mamba2Spec(_eps(st.ckpt.astype(np.float64), "fp8"), L, st.A, np.zeros(H), st.dt_bias, G)
    for r in range(20):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        ref, fl_ref = spec.verify(**s)
        bound, _ = espec.verify(x=np.zeros_like(s["x"]), z=s["z"], B=s["B"], C=np.abs(s["C"]), dt_raw=s["dt_raw"])
        x, z, Bm, C, dt = [to_dev(s[k], torch.bfloat16) for k in ("x", "z", "B", "C", "dt_raw")]
        rs.mamba2_spec_verify(desc, state, head, com, T, x, z, Bm, C, dt, bias, A, D, out, fl, err)
        rs.mamba2_spec_verify(desc, fp_state, head2, com2, T, x, z, Bm, C, dt, bias, A, D, out2, fl2, err)
        o = out.cpu().numpy()
        tol = np.abs(bound) + 1e-4 * (1 + np.abs(ref))
        worst = float(np.max(np.abs(o - ref) / tol))
        assert worst <= 1.0, f"round {r}: {worst:.3g} of the bound"
        assert np.array_equal(fl.cpu().numpy(), fl_ref.astype(np.int32))
        assert torch.equal(state.ckpt, fp_state.ckpt)
        for b in np.nonzero(fl_ref)[0]:
            espec.ckpt[b] = _eps(spec.ckpt[b], "fp8")
        keep = torch.from_numpy(n_keep.astype(np.int32)).to(DEV)
        rs.commit(B, L, T, head, com, fl, keep, err)
        rs.commit(B, L, T, head2, com2, fl2, keep, err)
        spec.commit(n_keep)
        espec.commit(n_keep)
    assert err.item() == 0


def test_state_and_output_route_refreshes_fp8_copy():
    B, H, P, N, G, L = 2, 4, 64, 128, 2, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=65)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    g = GpuMamba2(desc, st, lowp="fp8")
    rep = om.Mamba2Replay(st.ckpt, L, st.A, st.D, st.dt_bias, G)
    for t in range(1, L + 1):
        s = gen.step()
        ref, _ = rep.step(**s)
        x, z, Bm, C, dt = g.inputs(s)
        rs.mamba2_decode_state_and_output(desc, g.state, g.cur[g.flip], g.cur[1 - g.flip], x, z, Bm, C, dt,
                                          g.dt_bias, g.A, g.D, g.out, g.err)
        g.flip ^= 1
        assert_fp32_close(g.out.cpu().numpy(), ref, f"step {t}")       # this route reads fp32
    _assert_copy_near_state(g.state, "fp8", rep.ckpt, "copy after the flush")
