"""Host-side pieces of bench.py (no GPU): the shader-clock sampler's parsing
of the driver's clock-level file, and the gate that takes HBM traffic from a
committed counter summary only while it matches the kernel source."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _sampler(tmp_path, text):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text(text)
    s = bench.ClockSampler()
    s.path = str(f)
    return s


def test_clock_reading_takes_the_starred_level(tmp_path):
    assert _sampler(tmp_path, "0: 500Mhz\n1: 1785Mhz *\n2: 2400Mhz\n")._read() == 1785
    assert _sampler(tmp_path, "0: 500Mhz *\n1: 2400Mhz\n")._read() == 500


def test_clock_reading_skips_deep_sleep(tmp_path):
    assert _sampler(tmp_path, "S: 95Mhz *\n0: 500Mhz\n1: 2400Mhz\n")._read() is None


def test_clock_summary(tmp_path):
    s = _sampler(tmp_path, "0: 500Mhz\n1: 1700Mhz *\n2: 2400Mhz\n")
    assert s.summary() is None
    s.samples = [1700, 1800, 1750]
    sm = s.summary()
    assert (sm["median"], sm["min"], sm["max"], sm["samples"]) == (1750.0, 1700.0, 1800.0, 3)


def test_clock_sampler_without_a_file_reports_none(tmp_path):
    s = bench.ClockSampler()
    s.path = None
    with s:
        pass
    assert s.summary() is None


def test_clock_sampler_thread_collects(tmp_path):
    s = _sampler(tmp_path, "0: 500Mhz\n1: 1650Mhz *\n2: 2400Mhz\n")
    import time

    with s:
        time.sleep(0.05)
    assert s.samples and set(s.samples) == {1650}


def test_traffic_only_for_the_profiled_source(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    h = bench.kernel_source_hash(str(src))
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic(str(summary), str(src)) == 123456.0
    src.write_text("kernel source, changed\n")
    assert bench.measured_traffic(str(summary), str(src)) is None
