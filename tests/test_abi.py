"""Host-side tests of the C ABI: the library loads, exports every function that
include/replayssm.h declares, and rejects invalid arguments before touching the GPU.

No call here reaches a kernel launch: every call carries at least one invalid
argument or is one the header documents as launching nothing (precision emulation to
F32, or of zero rows), and the pointers are fake addresses that are never
dereferenced.  The
module is skipped where a GPU is visible so that a regression in the validation
could never launch a kernel on fake pointers.
"""

import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

from hybrid_model_ssm_amd import replayssm as rs  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only ABI checks")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rs.LIB_PATH):
        from hybrid_model_ssm_amd import build
        build.build()
    return rs.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int32_t|replayssm_status)\s+(replayssm_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("replayssm_mamba2_decode", "replayssm_mamba2_flush", "replayssm_mamba2_spec_verify",
              "replayssm_commit", "replayssm_reset_cursors", "replayssm_gdn_decode", "replayssm_gdn_flush",
              "replayssm_gdn_spec_verify", "replayssm_selective_state_update"):
        assert n in names
    assert set(names) == set(rs.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert rs.status_string(0) == "ok"
    assert rs.status_string(1) == "invalid argument"
    assert rs.status_string(2) == "unsupported shape"
    assert rs.status_string(3) == "HIP launch failure"
    assert rs.status_string(99) == "unknown status"
    assert rs.version() == 300


# fake, 256-byte aligned device addresses (never dereferenced)
def fake(i):
    return 0x7f0000000000 + 0x100000 * i


def m2desc(**kw):
    d = dict(batch=4, nheads=8, headdim=64, dstate=128, ngroups=2, buffer_len=16, io_dtype=rs.BF16,
             dt_softplus=1)
    d.update(kw)
    return rs.Mamba2DescC(**d)


def m2state(**kw):
    d = dict(ckpt=fake(1), ckpt_lp=None, rec_x=fake(2), rec_B=fake(3), rec_dt=fake(4))
    d.update(kw)
    return rs.Mamba2StateC(**d)


def decode(L, desc=None, state=None, **kw):
    a = dict(cin=fake(5), cout=fake(6), x=fake(7), z=fake(8), B=fake(9), C=fake(10), dt=fake(11),
             bias=fake(12), A=fake(13), D=fake(14), out=fake(15), err=None)
    a.update(kw)
    desc = desc if desc is not None else m2desc()
    state = state if state is not None else m2state()
    return L.replayssm_mamba2_decode(ctypes.byref(desc), ctypes.byref(state), a["cin"], a["cout"], a["x"],
                                     a["z"], a["B"], a["C"], a["dt"], a["bias"], a["A"], a["D"], a["out"],
                                     a["err"], None)


INV, UNS = rs.ERR_INVALID_ARGUMENT, rs.ERR_UNSUPPORTED


@pytest.mark.parametrize("desc_kw,expect", [
    (dict(batch=0), INV), (dict(nheads=0), INV), (dict(ngroups=3), INV), (dict(buffer_len=0), INV),
    (dict(buffer_len=65), INV), (dict(io_dtype=7), INV), (dict(headdim=48), UNS), (dict(dstate=24), UNS),
    (dict(headdim=128, dstate=256), UNS), (dict(headdim=0), INV),
])
def test_mamba2_decode_rejects_bad_desc(L, desc_kw, expect):
    # a bad x pointer as well, so that no variant could ever launch
    assert decode(L, desc=m2desc(**desc_kw), x=None) in (expect, INV)
    assert decode(L, desc=m2desc(**desc_kw), cout=fake(5)) == expect


def test_mamba2_decode_rejects_bad_pointers(L):
    assert L.replayssm_mamba2_decode(None, ctypes.byref(m2state()), *([fake(1)] * 11), None, None) == INV
    assert decode(L, state=m2state(ckpt=None), cout=fake(5)) == INV
    assert decode(L, state=m2state(ckpt=fake(1) + 4), cout=fake(5)) == INV      # 16-byte alignment
    assert decode(L, state=m2state(ckpt_lp=fake(20) + 8), cout=fake(5)) == INV
    assert decode(L, state=m2state(ckpt_lp=fake(1)), cout=fake(5)) == INV        # copy aliases ckpt
    assert decode(L, state=m2state(rec_B=None), cout=fake(5)) == INV
    assert decode(L, cout=fake(5)) == INV                                         # cursor_in == cursor_out
    assert decode(L, cin=None) == INV
    assert decode(L, x=fake(7) + 2, cout=fake(5)) == INV
    assert decode(L, out=fake(15) + 1, cout=fake(5)) == INV
    assert decode(L, D=None, cout=fake(5)) == INV
    assert decode(L, err=fake(16) + 2, cout=fake(5)) == INV


def test_mamba2_read_copy_kinds(L):
    ok = dict(cout=fake(6))
    # the read copy's dtype must name a read-copy format; fp8 needs its row scales
    assert decode(L, state=m2state(ckpt_lp=fake(20), lp_dtype=rs.F32), **ok) == INV
    assert decode(L, state=m2state(ckpt_lp=fake(20), lp_dtype=9), **ok) == INV
    assert decode(L, state=m2state(ckpt_lp=fake(20), lp_dtype=rs.FP8_E4M3, lp_scale=None), **ok) == INV
    assert decode(L, state=m2state(ckpt_lp=fake(20), lp_dtype=rs.FP8_E4M3, lp_scale=fake(21) + 2), **ok) == INV
    # without a read copy its dtype and scales are ignored
    assert decode(L, state=m2state(lp_dtype=9), x=None, **ok) == INV     # still rejected for x only
    assert rs.Mamba2StateC.lp_dtype.offset == 40 and rs.Mamba2StateC.lp_scale.offset == 48
    assert rs.Mamba2StateC.slot.offset == 56 and rs.Mamba2StateC.num_slots.offset == 64
    assert rs.GdnStateC.slot.offset == 40 and rs.GdnStateC.num_slots.offset == 48


def test_state_slot_validation(L):
    ok = dict(cout=fake(6))
    assert decode(L, state=m2state(slot=fake(22), num_slots=0), **ok) == INV
    assert decode(L, state=m2state(slot=fake(22) + 2, num_slots=8), **ok) == INV
    assert decode(L, state=m2state(slot=fake(22), num_slots=1 << 30), **ok) == INV


def test_mamba2_window_limit_is_unsupported(L):
    # headdim 128 with L=64: one head's fold rows (headdim * L elements) exceed what the
    # replay kernel stages per head
    assert decode(L, desc=m2desc(headdim=128, buffer_len=64)) == UNS
    assert decode(L, desc=m2desc(headdim=128, dstate=128, buffer_len=33)) == UNS


def test_mamba2_flush_and_spec_validation(L):
    d, s = m2desc(), m2state()
    assert L.replayssm_mamba2_flush(ctypes.byref(d), ctypes.byref(s), fake(5), fake(5), fake(13), None, None) == INV
    assert L.replayssm_mamba2_flush(ctypes.byref(d), ctypes.byref(s), fake(5), fake(6), None, None, None) == INV

    def spec(n_pos, head=fake(5), com=fake(6), flushed=fake(17), x=fake(7), nps=None):
        return L.replayssm_mamba2_spec_verify(ctypes.byref(d), ctypes.byref(s), head, com, n_pos, nps, x, fake(8),
                                              fake(9), fake(10), fake(11), fake(12), fake(13), fake(14),
                                              fake(15), flushed, None, None)
    assert spec(0, x=None) == INV
    assert spec(17, x=None) == INV
    assert spec(4, head=fake(6), x=None) == INV
    assert spec(4, flushed=fake(5), x=None) == INV
    assert spec(0) == INV and spec(17) == INV and spec(4, head=fake(6)) == INV and spec(4, flushed=fake(6)) == INV
    assert spec(4, nps=fake(18) + 2) == INV                                       # misaligned counts


def test_cursor_call_validation(L):
    C = L.replayssm_commit
    assert C(0, 16, 4, fake(1), fake(2), fake(3), fake(4), None, None, None) == INV
    assert C(4, 0, 1, fake(1), fake(2), fake(3), fake(4), None, None, None) == INV
    assert C(4, 16, 17, fake(1), fake(2), fake(3), fake(4), None, None, None) == INV
    assert C(4, 16, 0, fake(1), fake(2), fake(3), fake(4), None, None, None) == INV
    assert C(4, 16, 4, fake(1), fake(1), fake(3), fake(4), None, None, None) == INV
    assert C(4, 16, 4, fake(1), fake(2), None, fake(4), None, None, None) == INV
    assert C(4, 16, 4, fake(1), fake(2), fake(3), fake(4), fake(5) + 1, None, None) == INV
    R = L.replayssm_reset_cursors
    assert R(0, fake(1), fake(2), None, 0, None) == INV
    assert R(4, fake(1), None, None, 0, None) == INV
    assert R(4, fake(1), fake(1), None, 0, None) == INV
    assert R(4, fake(1), fake(2), fake(3), -1, None) == INV


def test_conventional_validation(L):
    d = m2desc(buffer_len=0)   # ignored by the conventional call
    args = [fake(i) for i in range(7, 16)]
    assert L.replayssm_selective_state_update(ctypes.byref(d), None, *args, None) == INV
    assert L.replayssm_selective_state_update(ctypes.byref(m2desc(ngroups=3)), fake(1), *args, None) == INV
    assert L.replayssm_mamba2_spec_baseline(ctypes.byref(d), fake(1), fake(2), 0, *args, None) == INV
    assert L.replayssm_mamba2_spec_baseline(ctypes.byref(d), fake(1), None, 4, *args, None) == INV


def gdesc(**kw):
    d = dict(batch=4, num_v_heads=8, num_k_heads=4, dk=128, dv=128, buffer_len=16, io_dtype=rs.BF16, scale=0.0)
    d.update(kw)
    return rs.GdnDescC(**d)


def test_gdn_validation(L):
    s = rs.GdnStateC(fake(1), fake(2), fake(3), fake(4), fake(5))

    def dec(desc, cin=fake(6), cout=fake(7), q=fake(8)):
        return L.replayssm_gdn_decode(ctypes.byref(desc), ctypes.byref(s), cin, cout, q, fake(9), fake(10),
                                      fake(11), fake(12), fake(13), None, None)
    assert dec(gdesc(num_k_heads=3), cout=fake(6)) == INV
    assert dec(gdesc(dk=96), cout=fake(6)) == UNS
    assert dec(gdesc(dv=32), cout=fake(6)) == UNS
    assert dec(gdesc(buffer_len=0), cout=fake(6)) == INV
    assert dec(gdesc(scale=-1.0), cout=fake(6)) == INV
    assert dec(gdesc(), cout=fake(6)) == INV
    assert dec(gdesc(), q=None) == INV
    assert dec(gdesc(), q=fake(8) + 4, cout=fake(6)) == INV
    assert L.replayssm_gdn_flush(ctypes.byref(gdesc()), ctypes.byref(s), fake(6), fake(6), None, None) == INV
    assert L.replayssm_gdn_conventional_decode(ctypes.byref(gdesc()), None, fake(8), fake(9), fake(10),
                                               fake(11), fake(12), fake(13), None) == INV

    def spec(desc, hd=fake(6), cm=fake(7), n_pos=4, fl=fake(14)):
        return L.replayssm_gdn_spec_verify(ctypes.byref(desc), ctypes.byref(s), hd, cm, n_pos, None, fake(8), fake(9),
                                           fake(10), fake(11), fake(12), fake(13), fl, None, None)
    assert spec(gdesc(), n_pos=0) == INV
    assert spec(gdesc(), n_pos=17) == INV                    # beyond buffer_len
    assert spec(gdesc(), cm=fake(6)) == INV                  # head aliases committed
    assert spec(gdesc(), fl=fake(7)) == INV                  # flushed aliases committed
    assert spec(gdesc(), fl=None) == INV
    assert spec(gdesc(dk=96)) == UNS
    # staging of 64 + 64 rows for four value heads exceeds one workgroup's LDS
    assert spec(gdesc(buffer_len=64, num_v_heads=16, io_dtype=rs.F32), n_pos=64) == UNS

    def snap(desc, sn=fake(1), slot=fake(2), n_pos=4):
        return L.replayssm_gdn_spec_baseline(ctypes.byref(desc), sn, slot, n_pos, fake(8), fake(9), fake(10),
                                             fake(11), fake(12), fake(13), None)
    assert snap(gdesc(), n_pos=0) == INV
    assert snap(gdesc(), sn=None) == INV
    assert snap(gdesc(), slot=None) == INV
    assert snap(gdesc(dv=96)) == UNS


def test_binding_refuses_host_tensors(L):
    desc = rs.Mamba2Desc(1, 1, 16, 16, 1, 4, rs.F32)
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        rs._ptr(t, torch.float32, "t")
    with pytest.raises(TypeError):
        rs._ptr([1, 2], None, "t")
    assert desc.c().headdim == 16


def test_emulate_precision_validation(L):
    E = L.replayssm_emulate_precision
    assert E(fake(1), 8, 6, rs.BF16, None, None) == INV              # row length not a multiple of 4
    assert E(fake(1), 8, 0, rs.BF16, None, None) == INV
    assert E(fake(1), -1, 8, rs.BF16, None, None) == INV
    assert E(fake(1), 8, 8, 7, None, None) == INV                    # no such dtype
    assert E(fake(1) + 4, 8, 8, rs.F16, None, None) == INV           # data not 16-byte aligned
    assert E(None, 8, 8, rs.F16, None, None) == INV
    assert E(fake(1), 8, 8, rs.FP8_E4M3, fake(2) + 2, None) == INV   # misaligned scales
    # documented to launch nothing
    assert E(fake(1), 8, 8, rs.F32, None, None) == rs.OK
    assert E(fake(1), 0, 8, rs.FP8_E4M3, None, None) == rs.OK


def test_probe_library_rejects_invalid_arguments_before_launching():
    """The benchmark's streaming probes (libreplayssm_probes.so, not part of the C ABI
    above): one 16-byte access per thread per pass, and every invalid argument returns 1
    before anything is launched (fake, never dereferenced pointers)."""
    import bench
    if not os.path.exists(bench.PROBE_LIB):
        from hybrid_model_ssm_amd import build
        build.build()
    P = bench.probe_lib()
    pf = P.replayssm_probe_pass_floats()
    assert pf == 256 * 4
    src, dst, sink = 0x100000, 0x200000, 0x300000
    n = pf * 8 * 16            # one workgroup of 16 tiles of 8 rows per thread

    def call(**kw):
        a = dict(src=src, dst=dst, sink=sink, n=n, rpt=8, tpw=16, mode=1, ntl=1, nts=1, order=0)
        a.update(kw)
        return P.replayssm_probe_stream(a["src"], a["dst"], a["sink"], a["n"], a["rpt"], a["tpw"], a["mode"],
                                        a["ntl"], a["nts"], a["order"], 1.0, None)

    for bad in (dict(src=0), dict(src=src + 4), dict(n=0), dict(n=n + 4), dict(rpt=3), dict(tpw=2),
                dict(mode=3), dict(mode=-1), dict(mode=0, sink=0), dict(mode=1, dst=0), dict(mode=2, dst=dst + 8),
                dict(order=3), dict(order=1, tpw=1, n=pf * 8)):
        assert call(**bad) == 1, bad


def test_read_then_write_probe_rejects_invalid_arguments_before_launching():
    """The read-then-write probe reads 16 tiles of [64, 128] fp32 per workgroup; each
    invalid argument returns 1 before anything is launched (fake pointers)."""
    import bench
    if not os.path.exists(bench.PROBE_LIB):
        from hybrid_model_ssm_amd import build
        build.build()
    P = bench.probe_lib()
    per_wg = P.replayssm_probe_rtw_read_floats()
    assert per_wg == 64 * 128 * 16
    src, dst, sink = 0x100000, 0x200000, 0x300000

    def call(**kw):
        a = dict(src=src, dst=dst, sink=sink, n=per_wg, wf=1024)
        a.update(kw)
        return P.replayssm_probe_read_then_write(a["src"], a["dst"], a["sink"], a["n"], a["wf"], None)

    for bad in (dict(src=0), dict(src=src + 4), dict(sink=0), dict(n=0), dict(n=per_wg + 4), dict(wf=-1024),
                dict(wf=1022), dict(dst=0), dict(dst=dst + 8)):
        assert call(**bad) == 1, bad


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """With no built library the binding raises on first use; there is no other route."""
    monkeypatch.setattr(rs, "_lib", None)
    monkeypatch.setattr(rs, "LIB_PATH", str(tmp_path / "libreplayssm.so"))
    with pytest.raises(rs.ReplaySSMLibraryMissing, match="missing"):
        rs.lib()
    with pytest.raises(rs.ReplaySSMLibraryMissing):      # every wrapper loads through lib()
        rs.version()
