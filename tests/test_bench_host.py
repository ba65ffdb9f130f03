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


def test_committed_counter_summaries_parse():
    for name in bench.PMC_FILES:
        tr = bench.committed_traffic(name)
        if tr is None:
            assert isinstance(bench.committed_traffic_reason(name), str)
        else:
            assert tr["traffic"] > 1e8 and 0.5 < tr["ratio"] < 2.0 and tr["source"].startswith("profiles/")


def test_gdn_flush_step_moves_the_state_twice():
    L = 16
    per = [bench.gdn_replay_bytes(256, 32, 16, 128, 128, L, 2, c) for c in range(L)]
    # the flush step reads and writes the state once: twice the state bytes of a read
    assert per[L - 1] - per[0] > 256 * 32 * 128 * 128 * 4 * 0.99


class _FakeRunner(bench.Runner):
    """Records dispatch indices; period L like a decode runner."""

    def __init__(self, L):
        self.period, self.B, self.launched = L, 4, []

    def launch(self, i):
        assert i == len(self.launched), "dispatches must be launched in order"
        self.launched.append(i)

    def bytes_of(self, i):
        return 100 if i % self.period == self.period - 1 else 10


@pytest.mark.parametrize("K,W,L", [(20, 5, 16), (1024, 32, 16), (7, 0, 4), (16, 16, 16), (1, 3, 16)])
def test_headline_regions_start_at_a_flush(monkeypatch, K, W, L):
    """Every timed region starts at the flush step and so holds ceil(K / L) flushes; the
    warmup is W launches after the setup steps."""
    calls = []

    def fake_timed(torch, launch, first, n):
        for i in range(first, first + n):
            launch(i)
        calls.append((first, n))
        return 1e-3 * n

    monkeypatch.setattr(bench, "timed_region", fake_timed)
    r = _FakeRunner(L)
    regions, setup, done = bench.measure(None, r, W, K, 3, start_at=L - 1)
    assert (setup + W) % L == L - 1 and setup < L
    assert [g["first"] % L for g in regions] == [L - 1] * 3
    assert all(g["flushes"] == -(-K // L) for g in regions)
    assert [c[1] for c in calls] == [K] * 3 and done == len(r.launched)
    res = bench.summarize(regions, K)
    assert res["value"] == pytest.approx(4 * K / (1e-3 * K))
    assert res["flush_dispatches_per_region"] == -(-K // L)


def test_summarize_takes_the_median_region():
    regions = [dict(seconds=s, bytes=1000, tokens=10, flushes=1) for s in (3.0, 1.0, 2.0, 5.0, 4.0)]
    res = bench.summarize(regions, 10)
    assert res["value"] == pytest.approx(10 / 3.0)
    assert sorted(res["values_per_region"]) == pytest.approx(sorted(10 / s for s in (3.0, 1.0, 2.0, 5.0, 4.0)))


def test_pmc_summary_from_counter_files(tmp_path, monkeypatch):
    """Two counter runs (FETCH_SIZE, WRITE_SIZE) of one variant become a summary scaled by
    the calibration copy, and committed_traffic reads it back."""
    def write_csv(d, counter, kern_val, copy_val):
        d.mkdir()
        with open(d / "x_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for i in range(4):
                f.write(f'{i},"rssm::gdn_conventional_kernel<128, 128, unsigned short, false>(rssm::GdnArgs)",'
                        f"{counter},{kern_val}\n")
            f.write(f'9,"void at::native::vectorized_elementwise_kernel<4, MulFunctor>",{counter},{copy_val}\n')
    write_csv(tmp_path / "f", "FETCH_SIZE", 1000.0, 524288.0)     # copy reads 1 GiB as 512 MiB
    write_csv(tmp_path / "w", "WRITE_SIZE", 2000.0, 1048576.0)
    info = dict(variant="gdn_hv32_conventional", kernel="gdn_conventional_kernel<128, 128, unsigned short, false>",
                sources=bench.GDN_SOURCES, dispatches=4, algorithmic_bytes_per_dispatch=5000.0 * 1024)
    ij = tmp_path / "info.json"
    ij.write_text(bench.json.dumps(info))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "feedfacefeedface")
    bench.pmc_summarize(str(tmp_path / "f"), str(tmp_path / "w"), str(ij), "cmd")
    tr = bench.committed_traffic("gdn_hv32_conventional")
    assert tr["fetch"] == pytest.approx(2000.0 * 1024) and tr["write"] == pytest.approx(2000.0 * 1024)
    assert tr["traffic"] == pytest.approx(4000.0 * 1024) and tr["ratio"] == pytest.approx(0.8)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "0000000000000000")
    assert bench.committed_traffic("gdn_hv32_conventional") is None


def test_sq_summary_from_counter_passes(tmp_path, monkeypatch):
    """SQ instruction-counter passes of one variant become per-dispatch and per-wave counts
    and the ALU time they would need spread over the chip's SIMDs."""
    kern = "rssm::gdn_replay_kernel<128, 128, unsigned short, 2>(rssm::GdnArgs)"

    def write_pass(d, counters):
        d.mkdir()
        with open(d / "x_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for i in range(3):
                for c, v in counters.items():
                    # two rows per dispatch and counter (the tool splits some counters): they add up
                    f.write(f'{i},"{kern}",{c},{v / 2}\n{i},"{kern}",{c},{v / 2}\n')
            f.write('7,"void other_kernel()",SQ_WAVES,5\n')
    write_pass(tmp_path / "p1", {"SQ_WAVES": 1000.0, "SQ_INSTS_VALU": 614.4e6 / 1000})
    write_pass(tmp_path / "p2", {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 2.4e3})
    info = dict(variant="gdn_spec_hv32_verify", kernel="gdn_replay_kernel<128, 128, unsigned short, 2>",
                sources=bench.GDN_SOURCES, dispatches=3)
    ij = tmp_path / "info.json"
    ij.write_text(bench.json.dumps(info))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "feedfacefeedface")
    bench.sq_summarize(str(ij), [str(tmp_path / "p1"), str(tmp_path / "p2")], "cmd")
    text = (tmp_path / "profiles" / "gdn_spec_verify_hv32_sq.txt").read_text()
    assert "SQ_WAVES | 1000 | 1.0 | 3" in text
    assert "SQ_INSTS_VALU | 6.144e+05 | 614.4 | 3" in text
    # 614400 wave instructions x 4 cycles / 1024 SIMDs / 2.4 GHz = 1.0 us
    assert "vector ALU issue time if spread over 1024 SIMDs: 1.0 us per dispatch" in text
    assert "matrix-core busy time if spread over 1024 SIMDs: 1.0 us per dispatch" in text


def test_headline_byte_split_adds_up():
    # reads plus writes are the byte model's total at every cursor; only the folding step
    # moves the checkpoint in place, 1 GiB each way
    for c in range(16):
        rd, wr, ip = bench.mamba2_replay_rw(256, 128, 64, 128, 8, 16, 2, c)
        assert rd + wr == bench.mamba2_replay_bytes(256, 128, 64, 128, 8, 16, 2, c)
        assert ip == (1 << 30 if c == 15 else 0)
    rd, wr, _ = bench.mamba2_replay_rw(256, 128, 64, 128, 8, 16, 2, 0)
    assert wr == 256 * 128 * (64 * 4 + 64 * 2 + 4) + 256 * 8 * 128 * 2     # outputs and the appended records


def test_step_model_at_the_measured_rates():
    # reads at 7.12 TB/s, the flushed checkpoint at 5.52 TB/s, other writes at 0.65 us/MiB:
    # 160.3 us at cursor 0, 405.8 us for the flush, 180.2 us per step over a window
    wsec = lambda nbytes: nbytes / MiB * 0.65e-6  # noqa: E731
    secs = [bench.step_model_seconds(*bench.mamba2_replay_rw(256, 128, 64, 128, 8, 16, 2, c), 7.12e12, 5.52e12, wsec)
            for c in range(16)]
    assert secs[0] * 1e6 == pytest.approx(160.3, abs=0.1)
    assert secs[15] * 1e6 == pytest.approx(405.8, abs=0.1)
    assert sum(secs) / 16 * 1e6 == pytest.approx(180.2, abs=0.1)


def test_write_cost_interpolates_the_probe_points():
    pts = [(0.0, 1.0e-4), (8.0, 1.12e-4), (32.0, 1.22e-4), (128.0, 1.58e-4)]
    assert bench.write_cost_seconds(0, pts) == 0.0
    assert bench.write_cost_seconds(4 * MiB, pts) == pytest.approx(6.0e-6)          # half of the first segment
    assert bench.write_cost_seconds(20 * MiB, pts) == pytest.approx(1.7e-5)         # within the second
    assert bench.write_cost_seconds(256 * MiB, pts) == pytest.approx(1.06e-4)       # past the last: its slope
    assert bench.write_cost_seconds(4 * MiB, list(reversed(pts))) == pytest.approx(6.0e-6)   # any order


def test_headline_device_model_from_probe_numbers():
    """The bench line's device model, from a ceiling section shaped like the probes' output
    (reads 7.12 TB/s, in place 5.52 TB/s in the replay shape, 0.65 us per MiB written) and a
    measured split: the window average is the 180.2 us of the hand calculation."""
    from hybrid_model_ssm_amd import synth
    ceil = dict(read_gbps=7120.0, read_probe="read_nt_r8_tpw4",
                probes={"inplace_nt_nt_r8_tpw16": dict(gbps=5520.0, us=0.0)},
                read_then_write=dict(written_MiB=[0.0, 128.0], us=[150.0, 150.0 + 128 * 0.65]))
    split = dict(nonflush_us=175.0, flush_us=413.0)
    head = dict(flush_dispatches_per_region=2, ms_per_dispatch=0.2)
    m = bench.headline_device_model(synth, ceil, split, head, 20)
    assert m["window_us_per_step"] == pytest.approx(180.2, abs=0.1)
    assert m["flush_us"] == pytest.approx(405.8, abs=0.1)
    assert m["region_us_per_step"] == pytest.approx((2 * m["flush_us"] + 18 * m["nonflush_us"]) / 20)
    assert m["measured_of_model"]["flush"] == pytest.approx(405.8 / 413.0, abs=1e-3)
    assert 0.8 < m["window_frac_of_peak"] < 0.84
