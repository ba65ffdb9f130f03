"""ctypes binding of libreplayssm (the C ABI in ``include/replayssm.h``).

Argument marshalling only: every function takes torch tensors, checks that they
are contiguous device tensors of the expected dtype, and passes their data
pointers and the current HIP stream to the library function of the same name.
All computation happens in the library's HIP kernels.  A non-OK status raises
``ReplaySSMError``; a missing library raises ``ReplaySSMLibraryMissing``.

PyTorch must be imported before the library is loaded so that both use the one
HIP runtime that torch ships.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; REPLAYSSM_LIB may name another build of the same library
LIB_PATH = os.environ.get("REPLAYSSM_LIB") or os.path.join(_HERE, "libreplayssm.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
F32, BF16, F16, FP8_E4M3 = 0, 1, 2, 3
DEVERR_CURSOR, DEVERR_SLOT = 1, 2
MAX_BUFFER_LEN = 64

EXPORTED = (
    "replayssm_status_string", "replayssm_version",
    "replayssm_mamba2_decode", "replayssm_mamba2_decode_state_and_output", "replayssm_mamba2_flush",
    "replayssm_mamba2_spec_verify",
    "replayssm_commit", "replayssm_reset_cursors", "replayssm_selective_state_update",
    "replayssm_mamba2_spec_baseline", "replayssm_gdn_decode", "replayssm_gdn_flush",
    "replayssm_gdn_spec_verify", "replayssm_gdn_conventional_decode", "replayssm_gdn_spec_baseline",
    "replayssm_emulate_precision",
)


class ReplaySSMError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        super().__init__(f"{func}: {status_string(status)} (status {status})")


class ReplaySSMLibraryMissing(ImportError):
    pass


class Mamba2DescC(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("ngroups", ctypes.c_int32), ("buffer_len", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32)]


class Mamba2StateC(ctypes.Structure):
    _fields_ = [("ckpt", ctypes.c_void_p), ("ckpt_lp", ctypes.c_void_p), ("rec_x", ctypes.c_void_p),
                ("rec_B", ctypes.c_void_p), ("rec_dt", ctypes.c_void_p), ("lp_dtype", ctypes.c_int32),
                ("lp_scale", ctypes.c_void_p), ("slot", ctypes.c_void_p), ("num_slots", ctypes.c_int32)]


class GdnDescC(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_v_heads", ctypes.c_int32), ("num_k_heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("buffer_len", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class GdnStateC(ctypes.Structure):
    _fields_ = [("ckpt", ctypes.c_void_p), ("rec_k", ctypes.c_void_p), ("rec_v", ctypes.c_void_p),
                ("rec_alpha", ctypes.c_void_p), ("rec_beta", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """Load the library (once).  Raises ReplaySSMLibraryMissing if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ReplaySSMLibraryMissing(
            f"{LIB_PATH} is missing; build it with `python -m hybrid_model_ssm_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.replayssm_status_string.restype = ctypes.c_char_p
    L.replayssm_status_string.argtypes = [ctypes.c_int]
    L.replayssm_version.restype = ctypes.c_int32
    L.replayssm_version.argtypes = []
    D, S = ctypes.POINTER(Mamba2DescC), ctypes.POINTER(Mamba2StateC)
    GD, GS = ctypes.POINTER(GdnDescC), ctypes.POINTER(GdnStateC)
    sig = {
        "replayssm_mamba2_decode": [D, S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_mamba2_decode_state_and_output": [D, S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_mamba2_flush": [D, S, _P, _P, _P, _P, _P],
        "replayssm_mamba2_spec_verify": [D, S, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_commit": [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_reset_cursors": [_I, _P, _P, _P, _I, _P],
        "replayssm_selective_state_update": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_mamba2_spec_baseline": [D, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_gdn_decode": [GD, GS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_gdn_flush": [GD, GS, _P, _P, _P, _P],
        "replayssm_gdn_spec_verify": [GD, GS, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_gdn_conventional_decode": [GD, _P, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_gdn_spec_baseline": [GD, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P],
        "replayssm_emulate_precision": [_P, ctypes.c_int64, _I, _I, _P, _P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    _lib = L
    return L


def status_string(status):
    return lib().replayssm_status_string(int(status)).decode()


def version():
    return int(lib().replayssm_version())


# --------------------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------------------

def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, func):
    if status != OK:
        raise ReplaySSMError(status, func)


_IO_TORCH = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass
class Mamba2Desc:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    buffer_len: int
    io_dtype: int = BF16
    dt_softplus: bool = True

    def c(self):
        return Mamba2DescC(self.batch, self.nheads, self.headdim, self.dstate, self.ngroups,
                           self.buffer_len, self.io_dtype, int(bool(self.dt_softplus)))

    @property
    def torch_io(self):
        return _IO_TORCH[self.io_dtype]


@dataclasses.dataclass
class Mamba2State:
    """Device buffers of one Mamba2 layer's replay state (see ``replayssm_mamba2_state``)."""
    ckpt: torch.Tensor
    rec_x: torch.Tensor
    rec_B: torch.Tensor
    rec_dt: torch.Tensor
    ckpt_lp: torch.Tensor | None = None
    lp_scale: torch.Tensor | None = None      # [B,H,P] f32 row scales of an fp8 copy
    slot: torch.Tensor | None = None          # [batch] int32 state row of each batch row (-1: pad)

    @staticmethod
    def allocate(desc: Mamba2Desc, device="cuda", lowp=False, ckpt=None, num_slots=None):
        """``lowp``: False (no read copy), True or "bf16", "f16", or "fp8" (e4m3 codes
        as uint8 with f32 row scales).  ``num_slots``: rows of a state pool addressed
        through ``slot`` (default: one row per batch row)."""
        H, P, N, G, L = desc.nheads, desc.headdim, desc.dstate, desc.ngroups, desc.buffer_len
        B = desc.batch if num_slots is None else int(num_slots)
        io = desc.torch_io
        if ckpt is None:
            ckpt = torch.zeros(B, H, P, N, dtype=torch.float32, device=device)
        kind = "bf16" if lowp is True else (lowp or None)
        if kind not in (None, "bf16", "f16", "fp8"):
            raise ValueError(f"unknown read copy {lowp!r}")
        lp_t = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.uint8}.get(kind)
        return Mamba2State(
            ckpt=ckpt,
            rec_x=torch.zeros(B, H, L, P, dtype=io, device=device),
            rec_B=torch.zeros(B, G, L, N, dtype=io, device=device),
            rec_dt=torch.zeros(B, L, H, dtype=torch.float32, device=device),
            ckpt_lp=torch.zeros(B, H, P, N, dtype=lp_t, device=device) if kind else None,
            lp_scale=torch.zeros(B, H, P, dtype=torch.float32, device=device) if kind == "fp8" else None,
        )

    @property
    def lp_dtype(self):
        if self.ckpt_lp is None:
            return F32
        return {torch.bfloat16: BF16, torch.float16: F16, torch.uint8: FP8_E4M3}[self.ckpt_lp.dtype]

    def c(self):
        return Mamba2StateC(_ptr(self.ckpt, torch.float32, "ckpt"),
                            _ptr(self.ckpt_lp, None, "ckpt_lp"),
                            _ptr(self.rec_x, None, "rec_x"), _ptr(self.rec_B, None, "rec_B"),
                            _ptr(self.rec_dt, torch.float32, "rec_dt"), self.lp_dtype,
                            _ptr(self.lp_scale, torch.float32, "lp_scale"), _ptr(self.slot, torch.int32, "slot"),
                            self.ckpt.shape[0])


@dataclasses.dataclass
class GdnDesc:
    batch: int
    num_v_heads: int
    num_k_heads: int
    dk: int
    dv: int
    buffer_len: int
    io_dtype: int = BF16
    scale: float = 0.0

    def c(self):
        return GdnDescC(self.batch, self.num_v_heads, self.num_k_heads, self.dk, self.dv,
                        self.buffer_len, self.io_dtype, float(self.scale))

    @property
    def torch_io(self):
        return _IO_TORCH[self.io_dtype]


@dataclasses.dataclass
class GdnState:
    ckpt: torch.Tensor
    rec_k: torch.Tensor
    rec_v: torch.Tensor
    rec_alpha: torch.Tensor
    rec_beta: torch.Tensor
    slot: torch.Tensor | None = None          # [batch] int32 state row of each batch row (-1: pad)

    @staticmethod
    def allocate(desc: GdnDesc, device="cuda", ckpt=None, num_slots=None):
        HV, HK, dk, dv, L = desc.num_v_heads, desc.num_k_heads, desc.dk, desc.dv, desc.buffer_len
        B = desc.batch if num_slots is None else int(num_slots)
        io = desc.torch_io
        if ckpt is None:
            ckpt = torch.zeros(B, HV, dv, dk, dtype=torch.float32, device=device)
        return GdnState(ckpt=ckpt,
                        rec_k=torch.zeros(B, HK, L, dk, dtype=io, device=device),
                        rec_v=torch.zeros(B, HV, L, dv, dtype=io, device=device),
                        rec_alpha=torch.zeros(B, L, HV, dtype=torch.float32, device=device),
                        rec_beta=torch.zeros(B, L, HV, dtype=torch.float32, device=device))

    def c(self):
        return GdnStateC(_ptr(self.ckpt, torch.float32, "ckpt"), _ptr(self.rec_k, None, "rec_k"),
                         _ptr(self.rec_v, None, "rec_v"), _ptr(self.rec_alpha, torch.float32, "rec_alpha"),
                         _ptr(self.rec_beta, torch.float32, "rec_beta"), _ptr(self.slot, torch.int32, "slot"),
                         self.ckpt.shape[0])


# --------------------------------------------------------------------------------------
# entry points (same names as the C ABI, without the prefix)
# --------------------------------------------------------------------------------------

def mamba2_decode(desc, state, cursor_in, cursor_out, x, z, B, C, dt_raw, dt_bias, A, D, out,
                  err_flags=None, stream=None):
    io = desc.torch_io
    st = lib().replayssm_mamba2_decode(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(cursor_in, torch.int32, "cursor_in"), _ptr(cursor_out, torch.int32, "cursor_out"),
        _ptr(x, io, "x"), _ptr(z, io, "z"), _ptr(B, io, "B"), _ptr(C, io, "C"), _ptr(dt_raw, io, "dt_raw"),
        _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(A, torch.float32, "A"), _ptr(D, torch.float32, "D"),
        _ptr(out, torch.float32, "out"), _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_mamba2_decode")


def mamba2_decode_state_and_output(desc, state, cursor_in, cursor_out, x, z, B, C, dt_raw, dt_bias, A, D, out,
                                   err_flags=None, stream=None):
    io = desc.torch_io
    st = lib().replayssm_mamba2_decode_state_and_output(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(cursor_in, torch.int32, "cursor_in"), _ptr(cursor_out, torch.int32, "cursor_out"),
        _ptr(x, io, "x"), _ptr(z, io, "z"), _ptr(B, io, "B"), _ptr(C, io, "C"), _ptr(dt_raw, io, "dt_raw"),
        _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(A, torch.float32, "A"), _ptr(D, torch.float32, "D"),
        _ptr(out, torch.float32, "out"), _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_mamba2_decode_state_and_output")


def mamba2_flush(desc, state, cursor_in, cursor_out, A, err_flags=None, stream=None):
    st = lib().replayssm_mamba2_flush(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(cursor_in, torch.int32, "cursor_in"), _ptr(cursor_out, torch.int32, "cursor_out"),
        _ptr(A, torch.float32, "A"), _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_mamba2_flush")


def mamba2_spec_verify(desc, state, head, committed, n_pos, x, z, B, C, dt_raw, dt_bias, A, D, out,
                       flushed, err_flags=None, stream=None, n_pos_seq=None):
    io = desc.torch_io
    st = lib().replayssm_mamba2_spec_verify(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(head, torch.int32, "head"), _ptr(committed, torch.int32, "committed"), int(n_pos),
        _ptr(n_pos_seq, torch.int32, "n_pos_seq"),
        _ptr(x, io, "x"), _ptr(z, io, "z"), _ptr(B, io, "B"), _ptr(C, io, "C"), _ptr(dt_raw, io, "dt_raw"),
        _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(A, torch.float32, "A"), _ptr(D, torch.float32, "D"),
        _ptr(out, torch.float32, "out"), _ptr(flushed, torch.int32, "flushed"),
        _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_mamba2_spec_verify")


def commit(batch, buffer_len, n_pos, head, committed, flushed, n_keep, err_flags=None, stream=None,
           n_pos_seq=None):
    st = lib().replayssm_commit(int(batch), int(buffer_len), int(n_pos),
                                _ptr(head, torch.int32, "head"), _ptr(committed, torch.int32, "committed"),
                                _ptr(flushed, torch.int32, "flushed"), _ptr(n_keep, torch.int32, "n_keep"),
                                _ptr(n_pos_seq, torch.int32, "n_pos_seq"),
                                _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_commit")


def emulate_precision(data, dtype, row_scale=None, stream=None):
    """Round the fp32 tensor ``data`` (rows along its last dimension) in place to the
    values of ``dtype`` (BF16, F16, or FP8_E4M3 with one scale per row, written to
    ``row_scale`` if given; F32 leaves it unchanged)."""
    if not isinstance(data, torch.Tensor) or data.dim() < 1:
        raise TypeError("data must be a tensor with at least one dimension")
    row_len = int(data.shape[-1])
    rows = int(data.numel() // row_len) if row_len else 0
    if row_scale is not None and row_scale.numel() != rows:
        raise ValueError(f"row_scale must hold {rows} values")
    st = lib().replayssm_emulate_precision(_ptr(data, torch.float32, "data"), rows, row_len, int(dtype),
                                           _ptr(row_scale, torch.float32, "row_scale"), _stream(stream))
    _check(st, "replayssm_emulate_precision")


def reset_cursors(batch, head, cursor, seq_idx=None, stream=None):
    n = 0 if seq_idx is None else int(seq_idx.numel())
    st = lib().replayssm_reset_cursors(int(batch), _ptr(head, torch.int32, "head"),
                                       _ptr(cursor, torch.int32, "cursor"),
                                       _ptr(seq_idx, torch.int32, "seq_idx"), n, _stream(stream))
    _check(st, "replayssm_reset_cursors")


def selective_state_update(desc, state, x, z, B, C, dt_raw, dt_bias, A, D, out, stream=None):
    io = desc.torch_io
    st = lib().replayssm_selective_state_update(
        ctypes.byref(desc.c()), _ptr(state, torch.float32, "state"),
        _ptr(x, io, "x"), _ptr(z, io, "z"), _ptr(B, io, "B"), _ptr(C, io, "C"), _ptr(dt_raw, io, "dt_raw"),
        _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(A, torch.float32, "A"), _ptr(D, torch.float32, "D"),
        _ptr(out, torch.float32, "out"), _stream(stream))
    _check(st, "replayssm_selective_state_update")


def mamba2_spec_baseline(desc, snapshots, slot_in, n_pos, x, z, B, C, dt_raw, dt_bias, A, D, out,
                         stream=None):
    io = desc.torch_io
    st = lib().replayssm_mamba2_spec_baseline(
        ctypes.byref(desc.c()), _ptr(snapshots, torch.float32, "snapshots"),
        _ptr(slot_in, torch.int32, "slot_in"), int(n_pos),
        _ptr(x, io, "x"), _ptr(z, io, "z"), _ptr(B, io, "B"), _ptr(C, io, "C"), _ptr(dt_raw, io, "dt_raw"),
        _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(A, torch.float32, "A"), _ptr(D, torch.float32, "D"),
        _ptr(out, torch.float32, "out"), _stream(stream))
    _check(st, "replayssm_mamba2_spec_baseline")


def gdn_decode(desc, state, cursor_in, cursor_out, q, k, v, alpha, beta, out, err_flags=None, stream=None):
    io = desc.torch_io
    st = lib().replayssm_gdn_decode(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(cursor_in, torch.int32, "cursor_in"), _ptr(cursor_out, torch.int32, "cursor_out"),
        _ptr(q, io, "q"), _ptr(k, io, "k"), _ptr(v, io, "v"),
        _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"),
        _ptr(out, torch.float32, "out"), _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_gdn_decode")


def gdn_flush(desc, state, cursor_in, cursor_out, err_flags=None, stream=None):
    st = lib().replayssm_gdn_flush(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(cursor_in, torch.int32, "cursor_in"), _ptr(cursor_out, torch.int32, "cursor_out"),
        _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_gdn_flush")


def gdn_spec_verify(desc, state, head, committed, n_pos, q, k, v, alpha, beta, out, flushed,
                    err_flags=None, stream=None, n_pos_seq=None):
    io = desc.torch_io
    st = lib().replayssm_gdn_spec_verify(
        ctypes.byref(desc.c()), ctypes.byref(state.c()),
        _ptr(head, torch.int32, "head"), _ptr(committed, torch.int32, "committed"), int(n_pos),
        _ptr(n_pos_seq, torch.int32, "n_pos_seq"),
        _ptr(q, io, "q"), _ptr(k, io, "k"), _ptr(v, io, "v"),
        _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"),
        _ptr(out, torch.float32, "out"), _ptr(flushed, torch.int32, "flushed"),
        _ptr(err_flags, torch.int32, "err_flags"), _stream(stream))
    _check(st, "replayssm_gdn_spec_verify")


def gdn_conventional_decode(desc, state, q, k, v, alpha, beta, out, stream=None):
    io = desc.torch_io
    st = lib().replayssm_gdn_conventional_decode(
        ctypes.byref(desc.c()), _ptr(state, torch.float32, "state"),
        _ptr(q, io, "q"), _ptr(k, io, "k"), _ptr(v, io, "v"),
        _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"),
        _ptr(out, torch.float32, "out"), _stream(stream))
    _check(st, "replayssm_gdn_conventional_decode")


def gdn_spec_baseline(desc, snapshots, slot_in, n_pos, q, k, v, alpha, beta, out, stream=None):
    io = desc.torch_io
    st = lib().replayssm_gdn_spec_baseline(
        ctypes.byref(desc.c()), _ptr(snapshots, torch.float32, "snapshots"),
        _ptr(slot_in, torch.int32, "slot_in"), int(n_pos),
        _ptr(q, io, "q"), _ptr(k, io, "k"), _ptr(v, io, "v"),
        _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"),
        _ptr(out, torch.float32, "out"), _stream(stream))
    _check(st, "replayssm_gdn_spec_baseline")
