"""Host-side checks of bench.py: byte models, argument handling, profile parsing."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

MiB = 1 << 20


def _window_avg(fn, L, **kw):
    return sum(fn(c=c, L=L, **kw) for c in range(L)) / L / MiB


def test_mamba2_byte_model_headline():
    # B=256, H=128, P=64, N=128, G=8, L=16, bf16 io: state 1088 + io 17.06 + records 39.0 MiB
    avg = _window_avg(lambda c, L: bench.mamba2_replay_bytes(256, 128, 64, 128, 8, L, 2, c), 16)
    assert avg == pytest.approx(1144.1, abs=0.05)
    lp = _window_avg(lambda c, L: bench.mamba2_replay_bytes(256, 128, 64, 128, 8, L, 2, c, True), 16)
    assert lp == pytest.approx(696.1, abs=0.05)
    assert bench.mamba2_conventional_bytes(256, 128, 64, 128, 8, 2) / MiB == pytest.approx(2065.06, abs=0.01)
    # the state part alone: 15 reads + one read and write per window of a 1 GiB checkpoint
    state_only = (15 * 1024 + 2048) / 16
    assert state_only == 1088


def test_read_copy_byte_models():
    # non-flush steps read 2 bytes per element (bf16, fp16) or 1 plus a 4-byte row scale (fp8)
    f32 = bench.mamba2_replay_bytes(1, 1, 64, 128, 1, 16, 2, 3)
    for kind, per_head in (("bf16", 2 * 64 * 128), ("f16", 2 * 64 * 128), ("fp8", 64 * 128 + 4 * 64)):
        got = bench.mamba2_replay_bytes(1, 1, 64, 128, 1, 16, 2, 3, kind)
        assert f32 - got == 4 * 64 * 128 - per_head
        flush = bench.mamba2_replay_bytes(1, 1, 64, 128, 1, 16, 2, 15, kind)
        assert flush - bench.mamba2_replay_bytes(1, 1, 64, 128, 1, 16, 2, 15) == per_head
    avg = _window_avg(lambda c, L: bench.mamba2_replay_bytes(256, 128, 64, 128, 8, L, 2, c, "fp8"), 16)
    # codes 256 MiB + row scales 8 MiB per read; the flush writes fp32 and the copy
    assert avg == pytest.approx(15 / 16 * (256 + 8) + (2048 + 264) / 16 + 17.06 + 39.0, abs=0.1)


def test_mamba2_byte_model_h64_and_gdn():
    assert _window_avg(lambda c, L: bench.mamba2_replay_bytes(256, 64, 64, 128, 8, L, 2, c), 16) == \
        pytest.approx(574.65, abs=0.01)
    assert _window_avg(lambda c, L: bench.gdn_replay_bytes(256, 32, 16, 128, 128, L, 2, c), 16) == \
        pytest.approx(577.9, abs=0.05)
    assert bench.gdn_conventional_bytes(256, 32, 16, 128, 128, 2) / MiB == pytest.approx(1032.06, abs=0.01)


def test_spec_byte_model_flush_and_plain_rounds():
    H, P, N, G, L, T = 128, 64, 128, 8, 16, 4
    plain = bench.spec_round_bytes(H, P, N, G, L, 2, T, [0])
    flush = bench.spec_round_bytes(H, P, N, G, L, 2, T, [13])
    # a flushing round writes the checkpoint: one more P*N*4 per head
    assert flush - plain - 13 * (H * (P * 2 + 4) + G * N * 2) == H * P * N * 4
    assert bench.spec_baseline_bytes(1, H, P, N, G, 2, T) == H * (P * N * 4 * 5 + T * (2 * P * 2 + 2 + P * 4)) + \
        G * T * 2 * N * 2


def test_gdn_spec_byte_model():
    HV, HK, dk, dv, L, T = 32, 16, 128, 128, 16, 4
    plain = bench.gdn_spec_round_bytes(HV, HK, dk, dv, L, 2, T, [0])
    fold = bench.gdn_spec_round_bytes(HV, HK, dk, dv, L, 2, T, [13])
    # a folding round writes the checkpoint (dv*dk*4 per value head) and reads 13 records
    assert fold - plain - 13 * (HV * (dv * 2 + 8) + HK * dk * 2) == HV * dv * dk * 4
    assert plain == HV * (dv * dk * 4 + T * (dv * 2 + 8 + dv * 4) + T * (dv * 2 + 8)) + HK * (T * 3 * dk * 2)
    assert bench.gdn_spec_baseline_bytes(1, HV, HK, dk, dv, 2, T) == \
        HV * (dv * dk * 4 * 5 + T * (dv * 2 + 8 + dv * 4)) + HK * T * 2 * dk * 2


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_only():
    a = "int f(int x) { return x + 1; }  // one\n/* two */"
    b = "int f(int x) {\n  return x + 1;\n}  // changed comment"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)


def test_committed_counter_summary_parses():
    traffic, src = bench.committed_traffic()
    assert traffic is None or traffic > 1e9
    assert isinstance(src, str)
    traffic, src = bench.committed_traffic("gdn")
    assert traffic is None or traffic > 1e8
    assert isinstance(src, str)


def test_gdn_window_bytes_matches_step_models():
    L = 16
    per = [bench.gdn_replay_bytes(256, 32, 16, 128, 128, L, 2, c) for c in range(L)]
    assert bench.gdn_window_bytes() == sum(per) / L
    # the flush step reads and writes the state once: twice the state bytes of a read
    assert per[L - 1] - per[0] > 256 * 32 * 128 * 128 * 4 * 0.99
