"""CPU checks of the benchmark's bookkeeping: the kernel-source hash that keys the committed
profile records ignores comments and whitespace but not code, a record is used only when its hash
matches, the clock fields divide a run's own FLOP rate by the peak at that run's clock, and the
gather byte count of the 800-frame workload."""
import json
import os

import pytest

import bench


def _write(path, text):
    with open(path, "w") as fh:
        fh.write(text)


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    _write(src, "int a = 1;  // one\n\n// note\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("k.hip",))
    h0 = bench.kernel_source_hash()
    _write(src, "int a = 1;   // other words\n// more notes\n\n  int b = 2;\n")
    assert bench.kernel_source_hash() == h0
    _write(src, "int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash() != h0


def test_profile_records_follow_the_hash(tmp_path, monkeypatch):
    _write(tmp_path / "k.hip", "int a = 1;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("k.hip",))
    os.makedirs(tmp_path / "profiles")
    h = bench.kernel_source_hash()
    rec = {"source_sha256": h, "gfx_clock_ghz": 2.0, "duration_s": 0.5, "hbm_bytes_per_launch": 123.0}
    _write(tmp_path / "profiles" / "attn_w_clock.txt", "# summary\n\n" + json.dumps(rec) + "\n")
    _write(tmp_path / "profiles" / "attn_w_hbm_traffic.txt", "# summary\n\n" + json.dumps(rec) + "\n")
    assert bench.measured_traffic("w") == 123.0
    assert bench.measured_clock("w") == 2.0
    f = bench.clock_fields(1e15, "w", 256)
    peak = 256 * 4096 * 2.0e9 / 1e12
    assert f["peak_at_clock"] == pytest.approx(peak)
    assert f["frac_at_clock"] == pytest.approx(1e15 / 0.5 / 1e12 / peak)
    _write(tmp_path / "k.hip", "int a = 2;\n")  # code changed: records void
    assert bench.measured_traffic("w") is None
    assert bench.clock_fields(1e15, "w", 256)["frac_at_clock"] is None
    assert bench.measured_clock("missing") is None


def test_gather_bytes_800_frames():
    """Reads: the K/V rows of S and every dropped row (they feed the means); writes: the packed
    rows padded to 64, and S as int32."""
    desc = bench.WORKLOADS["sga6-800f"][0]
    c = {"n_kv": 202722, "n_mean": 799}
    T = 800 * 1374
    rows_read = 202722 + (T - 202722)
    rows_written = (202722 + 799 + 63) // 64 * 64
    assert bench.gather_bytes(desc, c) == 16 * (rows_read + rows_written) * 64 * 2 * 2 + 4 * 202722


def test_f16_workloads_mirror_their_exact_forms():
    for name in ("sga6-800f", "dense-32f", "g2f-200f", "sga9-200f"):
        d, _ = bench.WORKLOADS[name + "-f16"]
        assert d == dict(bench.WORKLOADS[name][0], prescale_q=True)
        assert bench.form_name(d).endswith("-f16")
