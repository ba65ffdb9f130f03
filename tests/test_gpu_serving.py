"""GPU parity for the serving features: state slots (a pool of state rows addressed
through a per-batch-row map, -1 = pad row), and a per-sequence position count for
speculative verification (0 = pad row), for Mamba2 and Gated DeltaNet.

Outputs against the fp64 oracle at max |d| <= 1e-4 (1 + |ref|); cursors bit for bit.
Pool rows that no batch row names, and the outputs of pad rows, must stay untouched
byte for byte; a run through the slot map must give the same bytes as the same
sequences held in a dense state."""

import numpy as np
import pytest
import torch

from hybrid_model_ssm_amd import replayssm as rs
from hybrid_model_ssm_amd import synth
from oracle import gdn as og
from oracle import mamba2 as om
from tests.gpu_helpers import DEV, assert_fp32_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu

SLOTS = np.array([3, -1, 0, 8, 5, -1], np.int32)   # 6 batch rows over a pool of 9
POOL = 9


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _pool_ckpt(rng, shape):
    return (0.1 * rng.standard_normal((POOL,) + shape)).astype(np.float32)


def _state_bytes(st):
    return {k: v.clone() for k, v in vars(st).items() if isinstance(v, torch.Tensor) and k != "slot"}


def _assert_rows_untouched(before, st, rows, what):
    for k, v in before.items():
        now = getattr(st, k)
        for r in rows:
            assert torch.equal(now[r], v[r]), f"{what}: pool row {r} of {k} written"


@pytest.mark.parametrize("lowp", [False, "fp8"])
def test_mamba2_decode_through_slots(lowp):
    B, H, P, N, G, L = len(SLOTS), 8, 64, 128, 2, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=71)
    st = gen.static
    pool = _pool_ckpt(np.random.default_rng(72), (H, P, N))
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    A, D, bias = (to_dev(a, torch.float32) for a in (st.A, st.D, st.dt_bias))
    live = np.nonzero(SLOTS >= 0)[0]
    unused = [r for r in range(POOL) if r not in SLOTS]
    # the pool, and the same live sequences in a dense state (pad rows take slot 0's copy)
    sp = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=torch.from_numpy(pool).to(DEV), num_slots=POOL)
    sp.slot = _i32(SLOTS)
    dense_ck = pool[np.where(SLOTS >= 0, SLOTS, 0)]
    sd = rs.Mamba2State.allocate(desc, lowp=lowp, ckpt=torch.from_numpy(dense_ck).to(DEV))
    zi = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    if lowp:
        rs.mamba2_flush(desc, sp, zi(), zi(), A, err)
        rs.mamba2_flush(desc, sd, zi(), zi(), A, err)
    before = _state_bytes(sp)
    rep = om.Mamba2Replay(dense_ck[live], L, st.A, st.D, st.dt_bias, G)
    cp, cd = [zi(), zi()], [zi(), zi()]
    op = torch.full((B, H, P), 7.0, device=DEV)
    od = torch.empty_like(op)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        x, z, Bm, C, dt = [to_dev(s[k], torch.bfloat16) for k in ("x", "z", "B", "C", "dt_raw")]
        f = (t - 1) % 2
        rs.mamba2_decode(desc, sp, cp[f], cp[1 - f], x, z, Bm, C, dt, bias, A, D, op, err)
        rs.mamba2_decode(desc, sd, cd[f], cd[1 - f], x, z, Bm, C, dt, bias, A, D, od, err)
        ref, _ = rep.step(**{k: v[live] for k, v in s.items()})
        o = op.cpu().numpy()
        if not lowp:
            assert_fp32_close(o[live], ref, f"step {t}")
        assert torch.equal(op[live], od[live]), f"step {t}: slot run differs from the dense run"
        assert np.all(o[SLOTS < 0] == 7.0), f"step {t}: pad row output written"
        cur = cp[1 - f].cpu().numpy()
        assert np.array_equal(cur[live], np.full(live.size, t % L)) and np.all(cur[SLOTS < 0] == 0)
    for b in live:
        assert torch.equal(sp.ckpt[SLOTS[b]], sd.ckpt[b]), f"row {b}: checkpoint"
        assert torch.equal(sp.rec_x[SLOTS[b]], sd.rec_x[b]) and torch.equal(sp.rec_dt[SLOTS[b]], sd.rec_dt[b])
        if lowp:
            assert torch.equal(sp.ckpt_lp[SLOTS[b]], sd.ckpt_lp[b]) and torch.equal(sp.lp_scale[SLOTS[b]],
                                                                                    sd.lp_scale[b])
    _assert_rows_untouched(before, sp, unused, "decode")
    assert err.item() == 0


def test_bad_slot_is_flagged_and_skipped():
    B, H, P, N, G, L = 3, 4, 64, 128, 2, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=73)
    st = gen.static
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    sp = rs.Mamba2State.allocate(desc, num_slots=4)
    sp.slot = _i32([1, 4, 0])                          # 4 is past the pool
    A, D, bias = (to_dev(a, torch.float32) for a in (st.A, st.D, st.dt_bias))
    cin = _i32([2, 3, 0])
    cout = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full((B, H, P), 7.0, device=DEV)
    s = gen.step()
    x, z, Bm, C, dt = [to_dev(s[k], torch.bfloat16) for k in ("x", "z", "B", "C", "dt_raw")]
    rs.mamba2_decode(desc, sp, cin, cout, x, z, Bm, C, dt, bias, A, D, out, err)
    assert err.item() == rs.DEVERR_SLOT
    assert cout.cpu().tolist() == [3, 3, 1] and torch.all(out[1] == 7.0)


def _spec_round_inputs(gen, T):
    s = gen.step(n_pos=T)
    return s, gen.accepted(T - 1) + 1


@pytest.mark.parametrize("H,G", [(8, 2), (34, 1)], ids=["one_wg_per_group", "three_wgs_per_group"])
def test_mamba2_spec_with_slots_and_variable_positions(H, G):
    B, P, N, L, T = len(SLOTS), 64, 128, 8, 4
    gen = synth.Mamba2Inputs(B, H, P, N, G, io="bf16", seed=74)
    st = gen.static
    rng = np.random.default_rng(75)
    pool = _pool_ckpt(rng, (H, P, N))
    desc = rs.Mamba2Desc(B, H, P, N, G, L, rs.BF16, True)
    A, D, bias = (to_dev(a, torch.float32) for a in (st.A, st.D, st.dt_bias))
    sp = rs.Mamba2State.allocate(desc, ckpt=torch.from_numpy(pool).to(DEV), num_slots=POOL)
    sp.slot = _i32(SLOTS)
    before = _state_bytes(sp)
    live = np.nonzero(SLOTS >= 0)[0]
    specs = {b: om.Mamba2Spec(pool[SLOTS[b]][None], L, st.A, st.D, st.dt_bias, G) for b in live}
    zi = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
    head, com, fl = zi(), zi(), zi()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(B, T, H, P, dtype=torch.float32, device=DEV)
    n_flush = 0
    for r in range(24):
        s, n_keep = _spec_round_inputs(gen, T)
        tb = rng.integers(0, T + 1, size=B).astype(np.int32)
        tb[0] = T if r % 3 == 0 else tb[0]
        tb[SLOTS < 0] = 0                     # pad rows carry no positions, so commit skips them
        n_keep = np.minimum(n_keep, np.maximum(tb, 1)).astype(np.int32)
        out.fill_(7.0)
        fl.fill_(5)
        x, z, Bm, C, dt = [to_dev(s[k], torch.bfloat16) for k in ("x", "z", "B", "C", "dt_raw")]
        nps = _i32(tb)
        rs.mamba2_spec_verify(desc, sp, head, com, T, x, z, Bm, C, dt, bias, A, D, out, fl, err, n_pos_seq=nps)
        o, f = out.cpu().numpy(), fl.cpu().numpy()
        for b in range(B):
            if SLOTS[b] < 0 or tb[b] == 0:
                assert np.all(o[b] == 7.0) and f[b] == 0, f"round {r} row {b}: pad row written"
                continue
            ref, fr = specs[b].verify(**{k: v[b:b + 1, :tb[b]] for k, v in s.items()})
            assert_fp32_close(o[b, :tb[b]], ref[0], f"round {r} row {b}")
            assert np.all(o[b, tb[b]:] == 7.0), f"round {r} row {b}: position past its count written"
            assert f[b] == fr[0]
            n_flush += int(f[b])
            specs[b].commit(n_keep[b:b + 1])
        rs.commit(B, L, T, head, com, fl, _i32(n_keep), err, n_pos_seq=nps)
        hd, cm = head.cpu().numpy(), com.cpu().numpy()
        for b in specs:
            assert hd[b] == specs[b].head[0] and cm[b] == specs[b].committed[0], f"round {r} row {b}: cursors"
    assert n_flush > 0 and err.item() == 0
    _assert_rows_untouched(before, sp, [r for r in range(POOL) if r not in SLOTS], "spec")


def test_commit_checks_keep_against_positions():
    B, L, T = 3, 16, 4
    head, com = _i32([0, 2, 5]), _i32([3, 4, 6])
    fl = _i32([0, 0, 0])
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rs.commit(B, L, T, head, com, fl, _i32([2, 3, 1]), err, n_pos_seq=_i32([2, 2, 0]))
    assert err.item() & rs.DEVERR_CURSOR                  # row 1 keeps 3 of 2 positions
    assert com.cpu().tolist() == [5, 4, 6]                 # row 2 had no positions: unchanged


@pytest.mark.parametrize("HV,HK", [(4, 2), (12, 2)], ids=["one_wg_per_kgroup", "two_wgs_per_kgroup"])
def test_gdn_spec_with_slots_and_variable_positions(HV, HK):
    B, dk, dv, L, T = len(SLOTS), 128, 128, 8, 4
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="bf16", seed=76)
    rng = np.random.default_rng(77)
    pool = _pool_ckpt(rng, (HV, dv, dk))
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.BF16)
    sp = rs.GdnState.allocate(desc, ckpt=torch.from_numpy(pool).to(DEV), num_slots=POOL)
    sp.slot = _i32(SLOTS)
    before = _state_bytes(sp)
    live = np.nonzero(SLOTS >= 0)[0]
    specs = {b: og.GDNSpec(pool[SLOTS[b]][None], L, HK) for b in live}
    zi = lambda: torch.zeros(B, dtype=torch.int32, device=DEV)  # noqa: E731
    head, com, fl = zi(), zi(), zi()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(B, T, HV, dv, dtype=torch.float32, device=DEV)
    n_flush = 0
    for r in range(24):
        s = gen.step(n_pos=T)
        n_keep = gen.accepted(T - 1) + 1
        tb = rng.integers(0, T + 1, size=B).astype(np.int32)
        tb[SLOTS < 0] = 0
        n_keep = np.minimum(n_keep, np.maximum(tb, 1)).astype(np.int32)
        out.fill_(7.0)
        q, k, v = (to_dev(s[n], torch.bfloat16) for n in ("q", "k", "v"))
        al, be = (to_dev(s[n], torch.float32) for n in ("alpha", "beta"))
        nps = _i32(tb)
        rs.gdn_spec_verify(desc, sp, head, com, T, q, k, v, al, be, out, fl, err, n_pos_seq=nps)
        o, f = out.cpu().numpy(), fl.cpu().numpy()
        for b in range(B):
            if SLOTS[b] < 0 or tb[b] == 0:
                assert np.all(o[b] == 7.0) and f[b] == 0, f"round {r} row {b}: pad row written"
                continue
            ref, fr = specs[b].verify(**{kk: vv[b:b + 1, :tb[b]] for kk, vv in s.items()})
            assert_fp32_close(o[b, :tb[b]], ref[0], f"round {r} row {b}")
            assert np.all(o[b, tb[b]:] == 7.0)
            assert f[b] == fr[0]
            n_flush += int(f[b])
            specs[b].commit(n_keep[b:b + 1])
        rs.commit(B, L, T, head, com, fl, _i32(n_keep), err, n_pos_seq=nps)
        hd, cm = head.cpu().numpy(), com.cpu().numpy()
        for b in specs:
            assert hd[b] == specs[b].head[0] and cm[b] == specs[b].committed[0], f"round {r} row {b}: cursors"
    assert n_flush > 0 and err.item() == 0
    _assert_rows_untouched(before, sp, [r for r in range(POOL) if r not in SLOTS], "gdn spec")


def test_gdn_decode_through_slots():
    B, HV, HK, dk, dv, L = len(SLOTS), 6, 2, 64, 128, 4      # 3 value heads per q/k head
    gen = synth.GDNInputs(B, HV, HK, dk, dv, io="f32", seed=78)
    pool = _pool_ckpt(np.random.default_rng(79), (HV, dv, dk))
    desc = rs.GdnDesc(B, HV, HK, dk, dv, L, rs.F32)
    sp = rs.GdnState.allocate(desc, ckpt=torch.from_numpy(pool).to(DEV), num_slots=POOL)
    sp.slot = _i32(SLOTS)
    before = _state_bytes(sp)
    live = np.nonzero(SLOTS >= 0)[0]
    rep = og.GDNReplay(pool[SLOTS[live]], L, HK)
    cur = [torch.zeros(B, dtype=torch.int32, device=DEV) for _ in range(2)]
    out = torch.full((B, HV, dv), 7.0, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for t in range(1, 2 * L + 2):
        s = gen.step()
        q, k, v = (to_dev(s[n], torch.float32) for n in ("q", "k", "v"))
        al, be = (to_dev(s[n], torch.float32) for n in ("alpha", "beta"))
        f = (t - 1) % 2
        rs.gdn_decode(desc, sp, cur[f], cur[1 - f], q, k, v, al, be, out, err)
        ref, _ = rep.step(**{kk: vv[live] for kk, vv in s.items()})
        o = out.cpu().numpy()
        assert_fp32_close(o[live], ref, f"step {t}")
        assert np.all(o[SLOTS < 0] == 7.0)
        if t % L == 0:
            assert_fp32_close(sp.ckpt[_i32(SLOTS[live]).long()].cpu().numpy(), rep.ckpt, f"checkpoint step {t}")
    _assert_rows_untouched(before, sp, [r for r in range(POOL) if r not in SLOTS], "gdn decode")
    assert err.item() == 0
