"""Pins for the Gated DeltaNet oracle (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import gdn as og
from hybrid_model_ssm_amd import synth


def _rand_step(rng, Bt, HV, HK, dk, dv):
    q = rng.standard_normal((Bt, HK, dk))
    k = rng.standard_normal((Bt, HK, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=rng.standard_normal((Bt, HV, dv)),
                alpha=np.exp(-np.log1p(np.exp(rng.standard_normal((Bt, HV)) - 2))),
                beta=1 / (1 + np.exp(-rng.standard_normal((Bt, HV)))))


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "gdn_hand.json")))
    S = np.array(g["S0"])[None, None]
    rep = og.GDNReplay(S, g["buffer_len"], 1, scale=g["scale"])
    for i, st in enumerate(g["steps"]):
        q = np.array(st["q"])[None, None]
        k = np.array(st["k"])[None, None]
        v = np.array(st["v"])[None, None]
        al = np.array([[st["alpha"]]])
        be = np.array([[st["beta"]]])
        S, o = og.conventional_step(S, q, k, v, al, be, scale=g["scale"])
        assert np.allclose(S[0, 0], np.array(st["S"]), atol=1e-12)
        assert np.allclose(o[0, 0], np.array(st["o"]), atol=1e-12)
        ro, fl = rep.step(q, k, v, al, be)
        assert np.allclose(ro[0, 0], np.array(st["o"]), atol=1e-12)
        if fl[0]:
            assert np.allclose(rep.ckpt[0, 0], np.array(st["S"]), atol=1e-12)


def test_value_heads_share_key_heads():
    kq = np.arange(2 * 3, dtype=float).reshape(1, 2, 3)
    e = og.heads_of_kgroups(kq, 4)
    assert np.array_equal(e[0, 1], kq[0, 0]) and np.array_equal(e[0, 2], kq[0, 1])


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(20)
    Bt, HV, HK, dk, dv = 2, 4, 2, 5, 3
    S0 = 0.1 * rng.standard_normal((Bt, HV, dv, dk))
    rep = og.GDNReplay(S0, 4, HK)
    S = S0.copy()
    prod = np.ones((Bt, HV))
    for t in range(7):
        s = _rand_step(rng, Bt, HV, HK, dk, dv)
        s["beta"][:] = 0.0
        prod *= s["alpha"]
        S, o = og.conventional_step(S, **s)
        ro, _ = rep.step(**s)
        qh = np.repeat(s["q"], HV // HK, axis=1)
        ref = og.default_scale(dk) * prod[:, :, None] * np.einsum("bhij,bhj->bhi", S0, qh)
        assert np.allclose(o, ref, atol=1e-14)
        assert np.allclose(ro, ref, atol=1e-14)


def test_delta_rule_writes_value_exactly():
    # alpha = beta = 1 and a unit axis key: S_t k_t = v_t, so q = k reads back scale * v.
    rng = np.random.default_rng(21)
    Bt, HV, HK, dk, dv = 1, 2, 1, 4, 3
    S0 = rng.standard_normal((Bt, HV, dv, dk))
    rep = og.GDNReplay(S0, 3, HK)
    S = S0.copy()
    for t in range(5):
        j = t % dk
        k = np.zeros((Bt, HK, dk)); k[..., j] = 1.0
        v = rng.standard_normal((Bt, HV, dv))
        one = np.ones((Bt, HV))
        S, o = og.conventional_step(S, k, k, v, one, one)
        ro, _ = rep.step(k, k, v, one, one)
        assert np.array_equal(o, og.default_scale(dk) * v)
        assert np.allclose(ro, og.default_scale(dk) * v, atol=1e-13)


@pytest.mark.parametrize("L", [1, 2, 4, 5])
def test_replay_matches_conventional(L):
    rng = np.random.default_rng(22)
    Bt, HV, HK, dk, dv = 2, 4, 2, 6, 5
    S0 = 0.1 * rng.standard_normal((Bt, HV, dv, dk))
    rep = og.GDNReplay(S0, L, HK)
    S = S0.copy()
    for t in range(1, 21):
        s = _rand_step(rng, Bt, HV, HK, dk, dv)
        S, o = og.conventional_step(S, **s)
        ro, fl = rep.step(**s)
        assert np.max(np.abs(ro - o)) <= 1e-12
        assert bool(fl.all()) == (t % L == 0)
        if t % L == 0:
            assert np.max(np.abs(rep.ckpt - S)) <= 1e-12


def test_matrix_fold_matches_rowwise_updates_and_partial_flush():
    rng = np.random.default_rng(23)
    Bt, HV, HK, dk, dv = 1, 2, 1, 4, 3
    S0 = rng.standard_normal((Bt, HV, dv, dk))
    rep = og.GDNReplay(S0, 8, HK)
    S = S0.copy()
    for t in range(5):
        s = _rand_step(rng, Bt, HV, HK, dk, dv)
        # row-wise form of one step: S[i,:] <- alpha (S[i,:] - beta (S[i,:].k) k) + beta v[i] k
        kh = np.repeat(s["k"], HV // HK, axis=1)
        for h in range(HV):
            for i in range(dv):
                row = S[0, h, i]
                S[0, h, i] = s["alpha"][0, h] * (row - s["beta"][0, h] * (row @ kh[0, h]) * kh[0, h]) \
                    + s["beta"][0, h] * s["v"][0, h, i] * kh[0, h]
        rep.step(**s)
    assert list(rep.cursor) == [5]
    rep.flush()
    assert np.max(np.abs(rep.ckpt - S)) <= 1e-12
    before = rep.ckpt.copy()
    rep.flush()
    assert np.array_equal(rep.ckpt, before)


def test_synth_gdn_inputs_shapes_and_ranges():
    gen = synth.GDNInputs(4, 4, 2, 8, 8, io="bf16", seed=5)
    s = gen.step()
    assert s["q"].shape == (4, 2, 8) and s["v"].shape == (4, 4, 8)
    assert np.all((s["beta"] > 0) & (s["beta"] < 1))
    assert np.all((s["alpha"] > 0) & (s["alpha"] < 1))
    assert np.allclose(np.linalg.norm(s["k"].astype(np.float64), axis=-1), 1.0, atol=1e-2)
    assert np.array_equal(synth.round_bf16(s["q"]), s["q"])


def test_gdn_spec_outputs_equal_conventional_on_kept_and_draft_streams():
    rng = np.random.default_rng(24)
    Bt, HV, HK, dk, dv, L, T = 2, 4, 2, 6, 5, 7, 3
    S0 = 0.1 * rng.standard_normal((Bt, HV, dv, dk))
    spec = og.GDNSpec(S0, L, HK)
    S_kept = S0.copy()
    n_flush = 0
    for r in range(30):
        steps = [_rand_step(rng, Bt, HV, HK, dk, dv) for _ in range(T)]
        ins = {key: np.stack([s[key] for s in steps], 1) for key in steps[0]}
        com_before = spec.committed.copy()
        ck_before = spec.ckpt.copy()
        out, flushed = spec.verify(**ins)
        assert np.array_equal(flushed.astype(bool), com_before + T > L)
        n_flush += int(flushed.sum())
        for b in range(Bt):
            if not flushed[b]:
                assert np.array_equal(spec.ckpt[b], ck_before[b])   # output-only verify
        S = S_kept.copy()
        states = []
        for j in range(T):
            S, o = og.conventional_step(S, **steps[j])
            states.append(S)
            assert np.max(np.abs(out[:, j] - o)) <= 1e-12
        n_keep = rng.integers(1, T + 1, size=Bt)
        spec.commit(n_keep)
        S_kept = np.stack([states[n_keep[b] - 1][b] for b in range(Bt)])
        assert np.all((spec.committed >= 1) & (spec.committed <= L))
    assert n_flush > 0
    # folding what remains reproduces the kept conventional state
    for b in range(Bt):
        com, head = int(spec.committed[b]), int(spec.head[b])
        slots = [(head + i) % L for i in range(com)]
        ck = og.fold_matrix_form(spec.ckpt[b], spec.ring_k[b, slots], spec.ring_v[b, slots],
                                 spec.ring_alpha[b, slots], spec.ring_beta[b, slots])
        assert np.max(np.abs(ck - S_kept[b])) <= 1e-12


def test_gdn_spec_hand_example_single_position(golden_dir):
    # one position per round is the autoregressive hand example (buffer 2 -> flush every 2)
    g = json.load(open(os.path.join(golden_dir, "gdn_hand.json")))
    spec = og.GDNSpec(np.array(g["S0"])[None, None], g["buffer_len"], 1, scale=g["scale"])
    for st in g["steps"]:
        ins = dict(q=np.array(st["q"])[None, None, None], k=np.array(st["k"])[None, None, None],
                   v=np.array(st["v"])[None, None, None], alpha=np.array([[[st["alpha"]]]]),
                   beta=np.array([[[st["beta"]]]]))
        out, _ = spec.verify(**ins)
        assert np.allclose(out[0, 0, 0], np.array(st["o"]), atol=1e-12)
        spec.commit([1])


def _spec_rounds_vs_conventional(rng, spec, S_kept, rounds, Bt, HV, HK, dk, dv, T):
    """Run speculative rounds and check every output against the conventional recurrence
    continued from each sequence's kept state; returns the kept states after the rounds."""
    for _ in range(rounds):
        steps = [_rand_step(rng, Bt, HV, HK, dk, dv) for _ in range(T)]
        ins = {key: np.stack([s[key] for s in steps], 1) for key in steps[0]}
        out, _ = spec.verify(**ins)
        S = S_kept.copy()
        states = []
        for j in range(T):
            S, o = og.conventional_step(S, **steps[j])
            states.append(S)
            assert np.max(np.abs(out[:, j] - o)) <= 1e-12
        n_keep = rng.integers(1, T + 1, size=Bt)
        spec.commit(n_keep)
        S_kept = np.stack([states[n_keep[b] - 1][b] for b in range(Bt)])
    return S_kept


def test_gdn_spec_reset_starts_a_fresh_sequence():
    """reset() sets head and committed of the listed sequences to 0 and touches nothing
    else; with the caller's new checkpoint in place, a reset sequence then follows the
    conventional recurrence from that checkpoint (the records it held are dropped) while
    the other sequences continue theirs."""
    rng = np.random.default_rng(26)
    Bt, HV, HK, dk, dv, L, T = 3, 4, 2, 6, 5, 7, 3
    S0 = 0.1 * rng.standard_normal((Bt, HV, dv, dk))
    spec = og.GDNSpec(S0, L, HK)
    S_kept = _spec_rounds_vs_conventional(rng, spec, S0.copy(), 5, Bt, HV, HK, dk, dv, T)
    head0, com0, ck0 = spec.head.copy(), spec.committed.copy(), spec.ckpt.copy()
    assert com0[1] >= 1                     # the sequence to reset holds committed records
    spec.reset([1])
    assert spec.head[1] == 0 and spec.committed[1] == 0
    assert np.array_equal(spec.head[[0, 2]], head0[[0, 2]])
    assert np.array_equal(spec.committed[[0, 2]], com0[[0, 2]])
    assert np.array_equal(spec.ckpt, ck0)   # cursors only
    S_new = 0.1 * rng.standard_normal((HV, dv, dk))
    spec.ckpt[1] = S_new                    # the caller supplies the new sequence's checkpoint
    S_kept[1] = S_new
    _spec_rounds_vs_conventional(rng, spec, S_kept, 6, Bt, HV, HK, dk, dv, T)


def test_fixed_key_and_gates_reduce_to_an_iir_filter():
    """With a fixed unit key k and fixed alpha, beta, the state's component along k,
    s_t = S_t k, obeys s_t = alpha (1 - beta) s_{t-1} + beta v_t (a first-order IIR filter
    that scipy's lfilter, unused by the oracle, computes), and the rest decays by alpha
    per step: S_t = s_t k^T + alpha^t S_0 (I - k k^T).  Both oracle forms, across
    flushes, must match it for varying q and v."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(31)
    Bt, HV, HK, dk, dv, L, T = 1, 4, 2, 6, 5, 4, 11
    S0 = 0.3 * rng.standard_normal((Bt, HV, dv, dk))
    k = rng.standard_normal((Bt, HK, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    alpha = rng.uniform(0.5, 0.99, (Bt, HV))
    beta = rng.uniform(0.05, 0.95, (Bt, HV))
    steps = []
    for _ in range(T):
        s = _rand_step(rng, Bt, HV, HK, dk, dv)
        s.update(k=k, alpha=alpha, beta=beta)
        steps.append(s)
    kh = og.heads_of_kgroups(k, HV)[0]                           # [HV, dk]
    vs = np.stack([s["v"][0] for s in steps])                    # [T, HV, dv]
    ref_S = np.empty((T, HV, dv, dk))
    for h in range(HV):
        pole = alpha[0, h] * (1 - beta[0, h])
        s0 = S0[0, h] @ kh[h]
        sk, _ = lfilter([1.0], [1.0, -pole], beta[0, h] * vs[:, h], axis=0, zi=(pole * s0)[None])
        perp = S0[0, h] - np.outer(s0, kh[h])
        for t in range(T):
            ref_S[t, h] = np.outer(sk[t], kh[h]) + alpha[0, h] ** (t + 1) * perp
    scale = og.default_scale(dk)
    S = S0.copy()
    rep = og.GDNReplay(S0, L, HK)
    for t, s in enumerate(steps):
        qh = og.heads_of_kgroups(s["q"], HV)[0]
        ref_o = scale * np.einsum("hij,hj->hi", ref_S[t], qh)
        S, o = og.conventional_step(S, **s)
        assert np.allclose(S[0], ref_S[t], rtol=0, atol=1e-13)
        assert np.allclose(o[0], ref_o, rtol=0, atol=1e-13)
        ro, flushed = rep.step(**s)
        assert np.allclose(ro[0], ref_o, rtol=0, atol=1e-13)
        if flushed[0]:
            assert np.allclose(rep.ckpt[0], ref_S[t], rtol=0, atol=1e-13)
