"""Mamba2 decode oracle, float64 -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Three pieces, each written from its source and kept separate from the others:

* ``conventional_step`` -- the read-update-write recurrence that conventional
  decoding runs at every step: load the state, update it, read the output from
  it, store it ("ReplaySSM Caches Inputs Instead of State..." -- "Why SSM layers
  slow down hybrid models").  The update is the standard Mamba2 selective
  state update with a scalar decay per head::

      dt  = softplus(dt_raw + dt_bias[h])       (or dt_raw + dt_bias[h])
      h   = exp(dt * A[h]) * h + dt * outer(x, B)
      y   = h @ C + D[h] * x
      out = y * silu(z) = y * z * sigmoid(z)

  ``B`` and ``C`` belong to the group ``g = h // (nheads // ngroups)``.

* ``Mamba2Replay`` -- the replay form ("How ReplaySSM works"): the state held as
  a checkpoint and a ring of the latest input records.  Each step appends its record and evaluates
  y from the checkpoint plus the records, writing no state back; once the
  buffer holds L records they are merged into the checkpoint, which is written
  once, and the buffer starts empty again.  Unrolling the
  recurrence over the window (records ``s`` oldest first, the current step
  last) gives, with ``lam_s = sum of dt_r over the records after s``::

      decay = exp(A * sum_s dt_s)
      w_s   = dt_s * exp(A * lam_s)
      y     = decay * (Hc @ C_t) + sum_s w_s * (B_s . C_t) * x_s + D * x_t
      fold:   Hc <- decay * Hc + sum_s w_s * outer(x_s, B_s)

  The decay is formed from summed ``dt`` (log space), not from a running
  product as in ``conventional_step``: the two sides reach the same numbers by
  different arithmetic, which is what the tests compare.

* ``Mamba2Spec`` -- speculative verification on a circular buffer ("ReplaySSM"
  README, benefit "Cheap rollback": rejected inputs are discarded by moving a
  buffer pointer and verification is output-only; "How ReplaySSM works": draft
  inputs are appended to the buffer instead of snapshotting the state).  The
  cursor rules (flush when the uncommitted capacity runs out, commit of a kept
  prefix) are the plainest reading of those sentences; they are listed with
  the other readings in the design notes.

Arrays: checkpoint/state ``[batch, nheads, headdim, dstate]``; ``x, z``
``[batch, nheads, headdim]``; ``B, C`` ``[batch, ngroups, dstate]``; ``dt_raw``
``[batch, nheads]``; ``A, D, dt_bias`` ``[nheads]``.  All arithmetic is float64;
inputs are whatever exact values the GPU receives, upcast.
"""

from __future__ import annotations

import numpy as np

SOFTPLUS_THRESHOLD = 20.0


def softplus(u):
    """log(1 + exp(u)), returning u itself above the usual threshold of 20."""
    u = np.asarray(u, dtype=np.float64)
    return np.where(u > SOFTPLUS_THRESHOLD, u, np.log1p(np.exp(np.minimum(u, SOFTPLUS_THRESHOLD))))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate(y, z):
    """out = y * silu(z)."""
    z = np.asarray(z, dtype=np.float64)
    return y * z * sigmoid(z)


def heads_of_groups(Bg, nheads):
    """Repeat group vectors ``[..., G, N]`` to heads ``[..., H, N]`` (head h uses group h // (H/G))."""
    G = Bg.shape[-2]
    if nheads % G:
        raise ValueError("nheads must be a multiple of ngroups")
    return np.repeat(np.asarray(Bg, dtype=np.float64), nheads // G, axis=-2)


def dt_of(dt_raw, dt_bias, dt_softplus=True):
    u = np.asarray(dt_raw, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)
    return softplus(u) if dt_softplus else u


# --------------------------------------------------------------------------------------
# O-1: conventional read-update-write recurrence
# --------------------------------------------------------------------------------------

def conventional_step(h, x, z, B, C, dt_raw, dt_bias, A, D, dt_softplus=True):
    """One conventional decode step for a batch.  Returns ``(h_new, out)``.

    ``h`` [Bt,H,P,N]; the state is multiplied by ``exp(dt*A)`` (a per-step
    product) and receives ``dt * outer(x, B)``; the output is read from the
    updated state.
    """
    h = np.asarray(h, dtype=np.float64)
    H = h.shape[1]
    x = np.asarray(x, dtype=np.float64)
    Bh = heads_of_groups(B, H)
    Ch = heads_of_groups(C, H)
    dt = dt_of(dt_raw, dt_bias, dt_softplus)                      # [Bt,H]
    a = np.exp(dt * np.asarray(A, dtype=np.float64)[None, :])     # [Bt,H]
    h_new = a[:, :, None, None] * h + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :]
    y = np.einsum("bhpn,bhn->bhp", h_new, Ch) + np.asarray(D, dtype=np.float64)[None, :, None] * x
    return h_new, gate(y, z)


# --------------------------------------------------------------------------------------
# O-2: replay form (checkpoint + buffer of records)
# --------------------------------------------------------------------------------------

def window_coefficients(dts, A):
    """``dts`` [c, H], oldest record first and the newest last.

    Returns ``(decay [H], w [c, H])`` with ``decay = exp(A * sum dt)`` and
    ``w_s = dt_s * exp(A * lam_s)``, ``lam_s`` the sum of ``dt`` over the
    records after ``s`` (zero for the newest).
    """
    dts = np.asarray(dts, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    incl = np.cumsum(dts, axis=0)          # sum over r <= s
    total = incl[-1]
    lam = total[None, :] - incl            # sum over r > s
    lam[-1] = 0.0
    decay = np.exp(A * total)
    w = dts * np.exp(A[None, :] * lam)
    return decay, w


def replay_output(Hc, xs, Bs_h, dts, x_t, z_t, C_h, A, D):
    """Output of one step from the checkpoint and the window, one sequence.

    ``Hc`` [H,P,N]; ``xs`` [c,H,P], ``Bs_h`` [c,H,N], ``dts`` [c,H] hold the
    window's records oldest first with the current step's record last;
    ``C_h`` [H,N] is C_t expanded to heads.
    """
    decay, w = window_coefficients(dts, A)
    r = np.einsum("hpn,hn->hp", Hc, C_h)                  # Hc @ C_t
    beta = np.einsum("shn,hn->sh", Bs_h, C_h)             # B_s . C_t
    y = decay[:, None] * r + np.einsum("sh,shp->hp", w * beta, xs) + np.asarray(D)[:, None] * x_t
    return gate(y, z_t)


def fold_records(Hc, xs, Bs_h, dts, A):
    """Fold the window's records into the checkpoint, one sequence: ``decay*Hc + sum_s w_s outer(x_s, B_s)``."""
    if len(dts) == 0:
        return np.array(Hc, dtype=np.float64, copy=True)
    decay, w = window_coefficients(dts, A)
    return decay[:, None, None] * Hc + np.einsum("sh,shp,shn->hpn", w, xs, Bs_h)


class Mamba2Replay:
    """Autoregressive replay decode for a batch of sequences, each with its own cursor.

    The step that brings the buffer to ``buffer_len`` records flushes: its own
    record is folded together with the stored ones, the checkpoint is replaced
    and the buffer is cleared.  So a buffer never stores more than L-1 records
    between steps, and with every cursor starting at 0 the flushes land on the
    steps whose 1-based number is a multiple of L.
    """

    def __init__(self, ckpt, buffer_len, A, D, dt_bias, ngroups, dt_softplus=True):
        self.ckpt = np.array(ckpt, dtype=np.float64, copy=True)
        self.Bt, self.H, self.P, self.N = self.ckpt.shape
        if buffer_len < 1:
            raise ValueError("buffer_len must be >= 1")
        self.L = int(buffer_len)
        self.G = int(ngroups)
        self.A = np.asarray(A, dtype=np.float64)
        self.D = np.asarray(D, dtype=np.float64)
        self.dt_bias = np.asarray(dt_bias, dtype=np.float64)
        self.dt_softplus = bool(dt_softplus)
        # records per sequence: lists of (x [H,P], B [G,N], dt [H]) oldest first
        self.records = [[] for _ in range(self.Bt)]

    @property
    def cursor(self):
        return np.array([len(r) for r in self.records], dtype=np.int32)

    def step(self, x, z, B, C, dt_raw):
        """Returns ``(out [Bt,H,P], flushed [Bt] bool)``."""
        x = np.asarray(x, dtype=np.float64)
        z = np.asarray(z, dtype=np.float64)
        B = np.asarray(B, dtype=np.float64)
        C = np.asarray(C, dtype=np.float64)
        dt = dt_of(dt_raw, self.dt_bias, self.dt_softplus)
        out = np.empty((self.Bt, self.H, self.P))
        flushed = np.zeros(self.Bt, dtype=bool)
        for b in range(self.Bt):
            window = self.records[b] + [(x[b], B[b], dt[b])]
            xs = np.stack([r[0] for r in window])
            Bs_h = heads_of_groups(np.stack([r[1] for r in window]), self.H)
            dts = np.stack([r[2] for r in window])
            C_h = heads_of_groups(C[b], self.H)
            out[b] = replay_output(self.ckpt[b], xs, Bs_h, dts, x[b], z[b], C_h, self.A, self.D)
            if len(window) == self.L:
                self.ckpt[b] = fold_records(self.ckpt[b], xs, Bs_h, dts, self.A)
                self.records[b] = []
                flushed[b] = True
            else:
                self.records[b] = window
        return out, flushed

    def flush(self, seqs=None):
        """Fold whatever records sequences hold (0..L-1) and clear their buffers."""
        for b in range(self.Bt) if seqs is None else seqs:
            rec = self.records[b]
            if rec:
                xs = np.stack([r[0] for r in rec])
                Bs_h = heads_of_groups(np.stack([r[1] for r in rec]), self.H)
                dts = np.stack([r[2] for r in rec])
                self.ckpt[b] = fold_records(self.ckpt[b], xs, Bs_h, dts, self.A)
            self.records[b] = []


# --------------------------------------------------------------------------------------
# O-3: speculative verification on a circular buffer
# --------------------------------------------------------------------------------------

class Mamba2Spec:
    """Speculative decode with a circular record buffer of ``buffer_len`` slots.

    Per sequence the buffer holds ``committed`` records starting at slot
    ``head``.  A round presents ``n_pos`` positions (the last accepted token
    and the drafts):

    * verify: if ``committed + n_pos > L`` the committed records are folded
      into the checkpoint first (``flushed = 1``; the window is then empty);
      the ``n_pos`` records are written at slots ``(head + committed + j) % L``
      and position ``j``'s output is the replay output over the committed
      records followed by positions ``0..j``.  Verify writes the checkpoint
      only when it flushes and leaves ``head``/``committed`` unchanged.
    * commit: if the round flushed, ``head = (head + committed) % L`` and
      ``committed = 0``; then ``committed += n_keep`` (the kept prefix,
      ``1 <= n_keep <= n_pos``).  Rejected records are dropped by not counting
      them -- the checkpoint is not touched.
    """

    def __init__(self, ckpt, buffer_len, A, D, dt_bias, ngroups, dt_softplus=True):
        self.ckpt = np.array(ckpt, dtype=np.float64, copy=True)
        self.Bt, self.H, self.P, self.N = self.ckpt.shape
        self.L = int(buffer_len)
        self.G = int(ngroups)
        self.A = np.asarray(A, dtype=np.float64)
        self.D = np.asarray(D, dtype=np.float64)
        self.dt_bias = np.asarray(dt_bias, dtype=np.float64)
        self.dt_softplus = bool(dt_softplus)
        self.ring_x = np.zeros((self.Bt, self.L, self.H, self.P))
        self.ring_B = np.zeros((self.Bt, self.L, self.G, self.N))
        self.ring_dt = np.zeros((self.Bt, self.L, self.H))
        self.head = np.zeros(self.Bt, dtype=np.int64)
        self.committed = np.zeros(self.Bt, dtype=np.int64)
        self.flushed = np.zeros(self.Bt, dtype=np.int64)

    def verify(self, x, z, B, C, dt_raw):
        """Inputs ``[Bt, n_pos, ...]``.  Returns ``(out [Bt,n_pos,H,P], flushed [Bt])``."""
        x = np.asarray(x, dtype=np.float64)
        z = np.asarray(z, dtype=np.float64)
        B = np.asarray(B, dtype=np.float64)
        C = np.asarray(C, dtype=np.float64)
        n_pos = x.shape[1]
        if not 1 <= n_pos <= self.L:
            raise ValueError("need 1 <= n_pos <= buffer_len")
        dt = dt_of(dt_raw, self.dt_bias[None, :], self.dt_softplus)   # [Bt,n_pos,H]
        out = np.empty((self.Bt, n_pos, self.H, self.P))
        for b in range(self.Bt):
            head, com = int(self.head[b]), int(self.committed[b])
            slots = [(head + i) % self.L for i in range(com)]
            xs = [self.ring_x[b, s] for s in slots]
            Bs = [self.ring_B[b, s] for s in slots]
            ds = [self.ring_dt[b, s] for s in slots]
            if com + n_pos > self.L:
                if com:
                    self.ckpt[b] = fold_records(self.ckpt[b], np.stack(xs),
                                                heads_of_groups(np.stack(Bs), self.H),
                                                np.stack(ds), self.A)
                xs, Bs, ds = [], [], []
                self.flushed[b] = 1
            else:
                self.flushed[b] = 0
            for j in range(n_pos):
                slot = (head + com + j) % self.L
                self.ring_x[b, slot] = x[b, j]
                self.ring_B[b, slot] = B[b, j]
                self.ring_dt[b, slot] = dt[b, j]
                xs.append(x[b, j])
                Bs.append(B[b, j])
                ds.append(dt[b, j])
                out[b, j] = replay_output(self.ckpt[b], np.stack(xs),
                                          heads_of_groups(np.stack(Bs), self.H), np.stack(ds),
                                          x[b, j], z[b, j], heads_of_groups(C[b, j], self.H),
                                          self.A, self.D)
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
        idx = range(self.Bt) if seqs is None else seqs
        for b in idx:
            self.head[b] = 0
            self.committed[b] = 0
