"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts, the dominant-kernel choice and roofline arithmetic,
the gating of recorded HBM traffic by the GEMM sources' hash, the timed
region's lead-in and the clock record's summary."""

import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one MI355X" in line["error"]


def test_quantizer_bytes():
    # 2048 x 4096 bf16 in (2 B), E4M3 out (1 B), 32 scale columns of 2048 floats
    assert bench.quant_bytes(2048, 4096) == 3 * 2048 * 4096 + 4 * 2048 * 32
    # rows padded to four in the scale layout
    assert bench.quant_bytes(1, 128) == 3 * 128 + 4 * 4 * 1


def test_gemm_bytes():
    m, n, k = 2048, 6144, 4096
    a, sa = m * k, 4 * m * (k // 128)
    b, sb = n * k, 4 * (n // 128) * (k // 128)
    d = 2 * m * n
    assert bench.gemm_bytes(m, n, k) == a + sa + b + sb + d
    # MX: one packed scale word per weight row and chunk
    assert bench.gemm_bytes(m, n, k, mx=True) == a + sa + b + 4 * n * (k // 128) + d
    # a partial last column block keeps its own scale row
    assert bench.gemm_bytes(17, 130, 256) - bench.gemm_bytes(17, 128, 256) == 2 * 256 + 4 * 2 + 2 * 17 * 2


def _row(name, m, n, k, kernel, gemm_s):
    return {"name": name, "m": m, "n": n, "k": k, "_kernel": kernel, "_gemm_s": gemm_s, "_flops": 2 * m * n * k,
            "_bytes": bench.gemm_bytes(m, n, k)}


def test_dominant_kernel_and_roofline():
    per = [_row("qkv", 2048, 6144, 4096, "tile256x192_w4x3", 60e-6),
           _row("o", 2048, 4096, 4096, "tile256x128_w4x2", 45e-6),
           _row("gate_up", 2048, 24576, 4096, "tile256x256_w4x2", 200e-6),
           _row("down", 2048, 4096, 12288, "tile256x128_w4x2", 120e-6)]
    # 256x128 runs twice (165 us in all) but 256x256 once for 200 us
    assert bench.dominant_kernel(per) == "tile256x256_w4x2"
    roof = bench.roofline_of(per)
    flops = 2 * 2048 * 24576 * 4096
    assert roof["kernel"] == "gemm_nt_kernel<tile256x256_w4x2>" and roof["launches_per_step"] == 1
    assert roof["achieved"] == pytest.approx(flops / 200e-6 / 1e12, abs=0.1)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 5000.0, abs=1e-4)
    assert roof["algorithmic_bytes_per_launch"] == bench.gemm_bytes(2048, 24576, 4096)
    # the timed region's own launch time takes precedence
    timed = bench.roofline_of(per, {"kernel": "tile256x256_w4x2", "mean_s": 250e-6, "launches": 20})
    assert timed["mean_launch_us"] == pytest.approx(250.0)
    assert timed["achieved"] == pytest.approx(flops / 250e-6 / 1e12, abs=0.1)
    # two launches of one kernel: per-launch figures are means
    two = bench.roofline_of([_row("o", 2048, 4096, 4096, "tile256x128_w4x2", 40e-6),
                             _row("down", 2048, 4096, 12288, "tile256x128_w4x2", 120e-6)])
    assert two["launches_per_step"] == 2 and two["mean_launch_us"] == pytest.approx(80.0)
    assert two["algorithmic_gflop_per_launch"] == pytest.approx(2 * 2048 * 4096 * (4096 + 12288) / 2 / 1e9, abs=1e-3)


def test_persistent_kernel_name():
    """A plan that walks its tiles persistently names that kernel."""
    roof = bench.roofline_of([_row("gate_up", 2048, 24576, 4096, "tile256x256_w4x2 persistent", 170e-6)])
    assert roof["kernel"] == "gemm_nt_persistent_kernel<tile256x256_w4x2>"


def test_recorded_traffic_is_gated_by_the_sources_hash(tmp_path, monkeypatch):
    h = bench.kernel_sources_hash()
    assert len(h) == 16 and h == bench.kernel_sources_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel": "gemm_nt_kernel<tile256x256_w4x2>", "bytes_per_launch": 123, "sources": h}
    stale = dict(rec, kernel="gemm_nt_kernel<tile256x128_w4x2>", sources="0" * 16)
    (prof / "t.md").write_text(f"traffic-record: {json.dumps(rec)}\ntraffic-record: {json.dumps(stale)}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the sources are read from the real tree; only profiles/ moves
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: h)
    assert bench.recorded_traffic("gemm_nt_kernel<tile256x256_w4x2>") == 123
    assert bench.recorded_traffic("gemm_nt_kernel<tile256x128_w4x2>") is None  # recorded for other sources
    assert bench.recorded_traffic("gemm_nt_kernel<tile128x128_w2x2>") is None


def test_lead_in_spins_only_where_the_host_falls_behind():
    """The timed region's lead-in: no spin kernel where the host enqueues the
    steps in under half their device time (a sleeping GPU lowers its clock),
    a spin of 1.5x the host time + 2 ms otherwise."""
    spins = []
    ahead = object.__new__(bench.GpuAhead)
    ahead.spin = spins.append
    ahead.lead_in(host_s=100 * 0.15e-3, gpu_s=100 * 0.41e-3)  # the prefill step
    assert spins == []
    ahead.lead_in(host_s=100 * 0.05e-3, gpu_s=100 * 0.02e-3)  # small kernels
    assert spins == [pytest.approx(1.5 * 100 * 0.05e-3 + 2e-3)]


def test_clock_summary_counts_refreshes():
    """The clock record: medians over the valid samples (65535 marks a
    metric the firmware does not report), the XCDs' median, and how many
    distinct metric refreshes the samples hold."""
    s = bench.SmiSampler.__new__(bench.SmiSampler)
    s.samples = [(2000, 1400, 0.0, 1990.0)] * 50 + [(2040, 1398, 1.0, 2010.0)] * 60 + [(65535, None, 2.0, None)]
    out = s.summary()
    assert out["samples"] == 110 and out["distinct_readings"] == 2
    assert out["gfxclk_mhz_median"] == 2040.0 and out["gfxclk_mhz_min"] == 2000.0
    assert out["xcd_gfxclk_mhz_median"] == 2010.0
    assert out["socket_power_w_median"] == 1398.0 and out["socket_power_w_max"] == 1400.0
    s.samples = []
    assert s.summary() is None
