"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the reading of the
committed counter summary (kept only while it matches the kernel sources) and the sysfs clock
parser."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_is_read_only_for_matching_sources(tmp_path, monkeypatch):
    b = load_bench()
    for which in ("decode", "prefill"):
        f = tmp_path / f"traffic_{which}.md"
        monkeypatch.setitem(b.TRAFFIC_FILES, which, str(f))
        f.write_text("x\nsource_sha256_16 = %s\ntraffic_bytes_per_launch = 1234.0\n" % b.kernel_source_hash(which))
        assert b.measured_traffic(which) == 1234
        f.write_text("source_sha256_16 = 0000000000000000\ntraffic_bytes_per_launch = 1234.0\n")
        assert b.measured_traffic(which) is None
        f.write_text("source_sha256_16 = %s\n" % b.kernel_source_hash(which))  # no figure
        assert b.measured_traffic(which) is None
        monkeypatch.setitem(b.TRAFFIC_FILES, which, str(tmp_path / "missing.md"))
        assert b.measured_traffic(which) is None


def test_divisor_and_byte_counts():
    b = load_bench()
    assert b._divisor_at_most(20, 8) == 5 and b._divisor_at_most(20, 4) == 4 and b._divisor_at_most(7, 4) == 1
    import workloads as W
    # the survey's algorithmic bytes: weights + fp16 scale and zero + x + y + int16 pair index and fp32
    # angle per channel per stage (4 K D) + fp32 channel scale (4 D)
    M, D, N, K = 64, 4096, 14336, 8
    assert W.algorithmic_bytes(M, D, N, K) == N * D // 2 + N * D // 32 + 2 * M * D + 2 * M * N + 4 * K * D + 4 * D
    assert W.plain_bytes(M, D, N) == N * D // 2 + N * D // 32 + 2 * M * D + 2 * M * N


def test_sclk_parser(tmp_path, monkeypatch):
    b = load_bench()
    import glob as glob_mod

    real_glob = glob_mod.glob
    monkeypatch.setattr(glob_mod, "glob", lambda p: real_glob(p.replace("/sys/class/drm", str(tmp_path))))
    assert b.read_sclk_mhz() is None  # nothing there
    d = tmp_path / "card0" / "device"
    d.mkdir(parents=True)
    (d / "pp_dpm_sclk").write_text("S: 95Mhz\n0: 500Mhz\n1: 2400Mhz *\n")
    assert b.read_sclk_mhz() == {"now": 2400, "max_level": 2400}
    (d / "pp_dpm_sclk").write_text("0: 500Mhz *\n1: 1900Mhz\n2: 2400Mhz\n")
    assert b.read_sclk_mhz() == {"now": 500, "max_level": 2400}
    (d / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 2400Mhz\n")  # no current level marked
    assert b.read_sclk_mhz() == {"now": None, "max_level": 2400}
