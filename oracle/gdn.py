"""Gated DeltaNet decode oracle, float64 -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The Gated DeltaNet rule is the second SSM layer type the pages treat ("ReplaySSM
(a vLLM research fork)" -- "Core implementation files" lists a GDN
autoregressive replay kernel beside the Mamba2 ones; "ReplaySSM Caches Inputs
Instead of State..." -- "Why SSM layers slow down hybrid models" names GDN as a
layer of the hybrid models).  The recurrence is the standard gated delta rule
with a state ``S`` of shape ``[dv, dk]`` per value head::

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t q_t                     (scale defaults to 1/sqrt(dk))

Value head ``hv`` reads the q/k head ``hv // (HV // HK)``.

Replay form ("How ReplaySSM works": a checkpoint and a buffer of records,
outputs evaluated with no state written back, the records merged into the
checkpoint once per window).  Writing ``M_s = alpha_s (I - beta_s k_s k_s^T)``,
``S_t = S_ckpt M_1 ... M_t + sum_s beta_s v_s k_s^T M_{s+1} ... M_t``, so::

    S_t q = S_ckpt u + acc,   with u, acc from carrying q back:
        u <- q;  for s = t down to 1:  kappa = k_s . u
                                        acc  += beta_s * kappa * v_s
                                        u     = alpha_s * (u - beta_s * kappa * k_s)

The fold at a flush is written in the matrix form above (suffix products of the
``M_s``), which is a different computation from both the per-step recurrence
and the carry-back.

Arrays: state ``[batch, HV, dv, dk]``; ``q, k`` ``[batch, HK, dk]``; ``v``
``[batch, HV, dv]``; ``alpha, beta`` ``[batch, HV]``.
"""

from __future__ import annotations

import numpy as np


def heads_of_kgroups(qk, num_v_heads):
    """Repeat ``[..., HK, dk]`` to ``[..., HV, dk]`` (value head hv uses hv // (HV/HK))."""
    HK = qk.shape[-2]
    if num_v_heads % HK:
        raise ValueError("num_v_heads must be a multiple of num_k_heads")
    return np.repeat(np.asarray(qk, dtype=np.float64), num_v_heads // HK, axis=-2)


def default_scale(dk):
    return 1.0 / np.sqrt(dk)


# --------------------------------------------------------------------------------------
# O-4: conventional per-step recurrence
# --------------------------------------------------------------------------------------

def conventional_step(S, q, k, v, alpha, beta, scale=None):
    """One conventional step for a batch.  Returns ``(S_new, o)``."""
    S = np.asarray(S, dtype=np.float64)
    HV, dv, dk = S.shape[1:]
    scale = default_scale(dk) if scale is None else scale
    qh = heads_of_kgroups(q, HV)
    kh = heads_of_kgroups(k, HV)
    v = np.asarray(v, dtype=np.float64)
    al = np.asarray(alpha, dtype=np.float64)[:, :, None, None]
    be = np.asarray(beta, dtype=np.float64)[:, :, None, None]
    Sk = np.einsum("bhij,bhj->bhi", S, kh)                         # S k
    S_new = al * (S - be * Sk[..., :, None] * kh[..., None, :]) + be * v[..., :, None] * kh[..., None, :]
    o = scale * np.einsum("bhij,bhj->bhi", S_new, qh)
    return S_new, o


# --------------------------------------------------------------------------------------
# O-5: replay form
# --------------------------------------------------------------------------------------

def carry_back(q_h, ks, vs, alphas, betas):
    """Carry ``q`` back through the window's records, one sequence.

    ``q_h`` [HV,dk]; ``ks`` [c,HV,dk], ``vs`` [c,HV,dv], ``alphas``, ``betas``
    [c,HV], oldest first with the current step last.  Returns ``(u, acc)`` so
    that ``S_t q = S_ckpt u + acc``.
    """
    u = np.array(q_h, dtype=np.float64, copy=True)
    acc = np.zeros(vs.shape[1:], dtype=np.float64)
    for s in range(len(ks) - 1, -1, -1):
        kappa = np.einsum("hj,hj->h", ks[s], u)
        acc += (betas[s] * kappa)[:, None] * vs[s]
        u = alphas[s][:, None] * (u - (betas[s] * kappa)[:, None] * ks[s])
    return u, acc


def fold_matrix_form(Sc, ks, vs, alphas, betas):
    """``S_ckpt M_1..M_c + sum_s beta_s v_s k_s^T M_{s+1}..M_c``, one sequence."""
    Sc = np.asarray(Sc, dtype=np.float64)
    HV, dv, dk = Sc.shape
    c = len(ks)
    if c == 0:
        return Sc.copy()
    eye = np.eye(dk)
    M = [alphas[s][:, None, None] * (eye[None] - betas[s][:, None, None] * ks[s][:, :, None] * ks[s][:, None, :])
         for s in range(c)]
    suffix = [None] * (c + 1)                # suffix[s] = M_s ... M_{c-1} (0-based)
    suffix[c] = np.broadcast_to(eye, (HV, dk, dk)).copy()
    for s in range(c - 1, -1, -1):
        suffix[s] = M[s] @ suffix[s + 1]
    S_new = Sc @ suffix[0]
    for s in range(c):
        S_new = S_new + betas[s][:, None, None] * (vs[s][:, :, None] * ks[s][:, None, :]) @ suffix[s + 1]
    return S_new


class GDNReplay:
    """Autoregressive replay decode for a batch, each sequence with its own cursor."""

    def __init__(self, ckpt, buffer_len, num_k_heads, scale=None):
        self.ckpt = np.array(ckpt, dtype=np.float64, copy=True)
        self.Bt, self.HV, self.dv, self.dk = self.ckpt.shape
        self.HK = int(num_k_heads)
        self.L = int(buffer_len)
        self.scale = default_scale(self.dk) if scale is None else scale
        self.records = [[] for _ in range(self.Bt)]   # (k [HV,dk] expanded, v, alpha, beta)

    @property
    def cursor(self):
        return np.array([len(r) for r in self.records], dtype=np.int32)

    def step(self, q, k, v, alpha, beta):
        qh = heads_of_kgroups(q, self.HV)
        kh = heads_of_kgroups(k, self.HV)
        v = np.asarray(v, dtype=np.float64)
        alpha = np.asarray(alpha, dtype=np.float64)
        beta = np.asarray(beta, dtype=np.float64)
        out = np.empty((self.Bt, self.HV, self.dv))
        flushed = np.zeros(self.Bt, dtype=bool)
        for b in range(self.Bt):
            window = self.records[b] + [(kh[b], v[b], alpha[b], beta[b])]
            ks = np.stack([r[0] for r in window])
            vs = np.stack([r[1] for r in window])
            als = np.stack([r[2] for r in window])
            bes = np.stack([r[3] for r in window])
            u, acc = carry_back(qh[b], ks, vs, als, bes)
            out[b] = self.scale * (np.einsum("hij,hj->hi", self.ckpt[b], u) + acc)
            if len(window) == self.L:
                self.ckpt[b] = fold_matrix_form(self.ckpt[b], ks, vs, als, bes)
                self.records[b] = []
                flushed[b] = True
            else:
                self.records[b] = window
        return out, flushed

    def flush(self, seqs=None):
        for b in range(self.Bt) if seqs is None else seqs:
            rec = self.records[b]
            if rec:
                self.ckpt[b] = fold_matrix_form(self.ckpt[b], np.stack([r[0] for r in rec]),
                                                np.stack([r[1] for r in rec]),
                                                np.stack([r[2] for r in rec]),
                                                np.stack([r[3] for r in rec]))
            self.records[b] = []


# --------------------------------------------------------------------------------------
# speculative verification on a circular buffer
# --------------------------------------------------------------------------------------

class GDNSpec:
    """Speculative verify for the gated delta rule, with the cursor rules of ``Mamba2Spec``.

    The pages give Gated DeltaNet the same speculative treatment as Mamba2 ("ReplaySSM (a
    vLLM research fork)" -- "Core implementation files": a GDN speculative decode kernel on
    a circular buffer with its own commit and reset calls).  Per sequence the buffer holds
    ``committed`` records from slot ``head``.  verify: if ``committed + n_pos > L`` the
    committed records are folded into the checkpoint first (``flushed = 1``); the
    positions' records go to slots ``(head + committed + j) % L``; position ``j``'s output
    carries its q back through positions ``j..0`` and the committed records.  commit: if
    the round flushed, ``head += committed`` and ``committed = 0``; then ``committed +=
    n_keep``.  Records are kept per value head here (the q/k head's k expanded).
    """

    def __init__(self, ckpt, buffer_len, num_k_heads, scale=None):
        self.ckpt = np.array(ckpt, dtype=np.float64, copy=True)
        self.Bt, self.HV, self.dv, self.dk = self.ckpt.shape
        self.HK = int(num_k_heads)
        self.L = int(buffer_len)
        self.scale = default_scale(self.dk) if scale is None else scale
        self.ring_k = np.zeros((self.Bt, self.L, self.HV, self.dk))
        self.ring_v = np.zeros((self.Bt, self.L, self.HV, self.dv))
        self.ring_alpha = np.zeros((self.Bt, self.L, self.HV))
        self.ring_beta = np.zeros((self.Bt, self.L, self.HV))
        self.head = np.zeros(self.Bt, dtype=np.int64)
        self.committed = np.zeros(self.Bt, dtype=np.int64)
        self.flushed = np.zeros(self.Bt, dtype=np.int64)

    def verify(self, q, k, v, alpha, beta):
        """Inputs ``q, k [Bt,n_pos,HK,dk]``, ``v [Bt,n_pos,HV,dv]``, ``alpha, beta [Bt,n_pos,HV]``.
        Returns ``(out [Bt,n_pos,HV,dv], flushed [Bt])``."""
        n_pos = np.asarray(q).shape[1]
        if not 1 <= n_pos <= self.L:
            raise ValueError("need 1 <= n_pos <= buffer_len")
        qh = heads_of_kgroups(q, self.HV)
        kh = heads_of_kgroups(k, self.HV)
        v = np.asarray(v, dtype=np.float64)
        alpha = np.asarray(alpha, dtype=np.float64)
        beta = np.asarray(beta, dtype=np.float64)
        out = np.empty((self.Bt, n_pos, self.HV, self.dv))
        for b in range(self.Bt):
            head, com = int(self.head[b]), int(self.committed[b])
            slots = [(head + i) % self.L for i in range(com)]
            ks = [self.ring_k[b, s] for s in slots]
            vs = [self.ring_v[b, s] for s in slots]
            als = [self.ring_alpha[b, s] for s in slots]
            bes = [self.ring_beta[b, s] for s in slots]
            if com + n_pos > self.L:
                if com:
                    self.ckpt[b] = fold_matrix_form(self.ckpt[b], np.stack(ks), np.stack(vs),
                                                    np.stack(als), np.stack(bes))
                ks, vs, als, bes = [], [], [], []
                self.flushed[b] = 1
            else:
                self.flushed[b] = 0
            for j in range(n_pos):
                slot = (head + com + j) % self.L
                self.ring_k[b, slot] = kh[b, j]
                self.ring_v[b, slot] = v[b, j]
                self.ring_alpha[b, slot] = alpha[b, j]
                self.ring_beta[b, slot] = beta[b, j]
                ks.append(kh[b, j])
                vs.append(v[b, j])
                als.append(alpha[b, j])
                bes.append(beta[b, j])
                u, acc = carry_back(qh[b, j], np.stack(ks), np.stack(vs), np.stack(als), np.stack(bes))
                out[b, j] = self.scale * (np.einsum("hij,hj->hi", self.ckpt[b], u) + acc)
        return out, self.flushed.copy()

    def commit(self, n_keep):
        n_keep = np.asarray(n_keep, dtype=np.int64)
        for b in range(self.Bt):
            if self.flushed[b]:
                self.head[b] = (self.head[b] + self.committed[b]) % self.L
                self.committed[b] = 0
            self.committed[b] += n_keep[b]
            self.flushed[b] = 0

    def reset(self, seqs=None):
        for b in range(self.Bt) if seqs is None else seqs:
            self.head[b] = 0
            self.committed[b] = 0
