"""CPU: the benchmark's host-side helpers (no GPU needed)."""
import pytest

import bench
from dense_mixed_precision_amd.workloads import WORKLOADS


def test_roofline_bound_follows_arithmetic_intensity():
    # ridge = 2516.6 TFLOP/s / 8 TB/s = 315 FLOP/byte
    assert bench.roofline_entry(WORKLOADS["square8192"], 1.0)["bound"] == "mfma"     # AI 2048
    assert bench.roofline_entry(WORKLOADS["square2048"], 1.0)["bound"] == "mfma"     # AI 512
    assert bench.roofline_entry(WORKLOADS["tallskinny32768x128x4096"], 1.0)["bound"] == "hbm"  # AI 120
    assert bench.roofline_entry(WORKLOADS["ragged1000x800x617"], 1.0)["bound"] == "hbm"


def test_roofline_achieved_is_algorithmic_work_over_time():
    w = WORKLOADS["square2048"]
    r = bench.roofline_entry(w, 0.025)  # 25 us
    assert abs(r["achieved"] - 2 * 2048**3 / 25e-6 / 1e12) < 0.01
    assert abs(r["frac"] - r["achieved"] / bench.PEAK_F16_TFLOPS) < 1e-4
    w = WORKLOADS["tallskinny32768x128x4096"]
    r = bench.roofline_entry(w, 0.05)
    assert abs(r["achieved"] - w.algorithmic_bytes / 50e-6 / 1e9) < 0.1
    assert r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS


def test_secondary_warmup_is_about_40ms_of_gpu_time():
    assert bench.warmup_for(WORKLOADS["square8192"], 1000) >= 20      # ~1 ms per launch
    assert bench.warmup_for(WORKLOADS["square2048"], 1000) == 1000    # capped by --warmup
    assert bench.warmup_for(WORKLOADS["square8192"], 2) == 3          # at least 3


def test_measured_traffic_follows_the_kernel_code_digest(tmp_path, monkeypatch):
    """L2-miss bytes come from a committed counter summary only while the
    device code it was taken on is unchanged."""
    digest = "0123456789abcdef"
    prof = tmp_path / "profiles"
    prof.mkdir()
    text = ("# L2-miss bytes\nkernel_code_digest: {d}\nl2_miss_read_bytes_per_launch: 3000\n"
            "l2_miss_write_bytes_per_launch: 1000\n")
    (prof / "l2_miss_bytes_square2048.txt").write_text(text.format(d=digest))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_code_digest", lambda lib=None: digest)
    t = bench.measured_traffic("square2048", 0.001)
    assert t["bytes_per_launch"] == 4000 and t["GBps"] == 4.0
    roof = bench.with_traffic(bench.roofline_entry(WORKLOADS["square2048"], 0.025), t)
    assert roof["traffic"] == 4000 and roof["traffic_detail"]["read_bytes"] == 3000
    (prof / "l2_miss_bytes_square2048.txt").write_text(text.format(d="0" * 16))
    assert bench.measured_traffic("square2048", 0.001) is None
    assert bench.measured_traffic("square8192", 0.001) is None
    assert bench.with_traffic({"bound": "mfma"}, None)["traffic"] is None
    # no library built: no digest, no reuse
    monkeypatch.setattr(bench, "kernel_code_digest", lambda lib=None: None)
    (prof / "l2_miss_bytes_square2048.txt").write_text(text.format(d=digest))
    assert bench.measured_traffic("square2048", 0.001) is None


def test_spread_reports_median_and_cv():
    s = bench.spread([0.010, 0.012, 0.011, 0.011])
    assert s["median_us"] == 11.0 and s["n"] == 4
    assert abs(s["cv"] - (0.0007071 / 0.011)) < 1e-3
    assert bench.spread([0.02])["cv"] == 0.0


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_timeline_summary_reads_the_record_layout():
    """Synthetic records with a 2 GHz shader clock: 2 us to the first tile,
    1.2 us between tiles, 0.5 us to the loop end, 0.3 us of epilogue."""
    import numpy as np

    nwg, ntiles, ghz = 16, 5, 2.0
    rec = np.zeros((nwg, 48), dtype=np.uint64)
    for b in range(nwg):
        rt0, mt0 = 1000 + b, 5_000_000 + 37 * b
        cyc = [mt0, mt0 + 4000]                       # start, tile 0 after 2 us
        for _ in range(1, ntiles):
            cyc.append(cyc[-1] + 2400)                # 1.2 us per tile
        loop_end = cyc[-1] + 1000
        epi_end = loop_end + 600
        rec[b, 0], rec[b, 1] = rt0, mt0
        for t in range(ntiles):
            rec[b, 2 + t] = cyc[1 + t]
        rec[b, 43], rec[b, 44], rec[b, 45] = ntiles, loop_end, epi_end
        rec[b, 46] = rt0 + round((epi_end - mt0) / ghz / 10)   # 100 MHz ticks
        rec[b, 47] = ((b % 8) << 32) | 0x123
    s = bench.timeline_summary(rec, nwg)
    assert s["k_tiles"] == ntiles and s["workgroups"] == nwg
    assert abs(s["shader_clock_GHz"] - ghz) < 0.01
    assert abs(s["first_tile_us"] - 2.0) < 0.01
    assert s["tile_interval_us"] == [1.2] * (ntiles - 1)
    assert abs(s["last_recorded_tile_to_loop_end_us"] - 0.5) < 0.01
    assert abs(s["epilogue_us"] - 0.3) < 0.01
    assert s["start_skew_us"]["max"] == 0.15
    assert sorted(s["xcd_end_us"]) == list(range(8))


def test_kernel_code_digest_covers_the_device_code_only(tmp_path):
    """The digest is that of the library's .hip_fatbin section (the kernels'
    code objects): a byte changed inside the section changes it, a byte
    changed elsewhere (host code) does not."""
    import hashlib
    import os

    lib = os.path.join(bench.ROOT, bench.PRODUCT_LIB)
    if not os.path.exists(lib):
        pytest.skip("product library not built")
    data = bytearray(open(lib, "rb").read())
    off, size = bench._elf_section(bytes(data), b".hip_fatbin")
    assert size > 0
    d0 = bench.kernel_code_digest(lib)
    assert d0 == hashlib.sha256(bytes(data[off:off + size])).hexdigest()[:16]
    host = tmp_path / "host.so"
    data_h = bytearray(data)
    data_h[off - 1] ^= 0xFF
    data_h[off + size] ^= 0xFF
    host.write_bytes(bytes(data_h))
    assert bench.kernel_code_digest(str(host)) == d0
    dev = tmp_path / "dev.so"
    data_d = bytearray(data)
    data_d[off + size // 2] ^= 0xFF
    dev.write_bytes(bytes(data_d))
    assert bench.kernel_code_digest(str(dev)) != d0
    assert bench.kernel_code_digest(str(tmp_path / "missing.so")) is None


def test_copy_bound_adds_the_loop_at_the_copy_rate_to_the_measured_phases():
    w = WORKLOADS["square2048"]
    cfg = {"bm": 128, "bn": 128}
    tl = {"shader_clock_GHz": 2.0, "k_tiles": 16, "first_tile_us": 2.5, "epilogue_us": 1.5}
    fill = {"per_cu_bytes_per_clk": {"hit_2MiB_lds16_d2_1cu": 40.0, "hit_2MiB_lds16_d2_32cu": 32.0,
                                     "hit_2MiB_lds16_d8_32cu": 25.0}}
    b = bench.copy_bound(w, cfg, tl, fill, 0.025)
    copy = (128 + 128) * 2048 * 2
    assert b["copy_bytes_per_workgroup"] == copy and b["copy_bytes_per_clk"] == 32.0
    loop = copy / 32.0 / 2000.0 * 15 / 16            # us: bytes / (B/clk) / (clk per us), less the first tile
    assert abs(b["loop_us"] - loop) < 1e-3
    assert abs(b["bound_us"] - (loop + 4.0)) < 1e-3
    assert abs(b["frac_of_bound"] - (loop + 4.0) / 25.0) < 1e-3


def test_sweep_tool_parses_its_arguments(monkeypatch):
    """The factory sweep's command line (the GPU part runs on the device only)."""
    import sys

    from dense_mixed_precision_amd import sweep
    monkeypatch.setattr(sys, "argv", ["sweep", "--shapes", "256x512,1024x2048", "--ks", "256,8192",
                                      "--configs", "35,36,41"])
    a = sweep.parse()
    assert (a.shapes, a.ks, a.configs, a.rounds, a.candidates) == ("256x512,1024x2048", "256,8192", "35,36,41",
                                                                    5, False)
    monkeypatch.setattr(sys, "argv", ["sweep", "--triples", "256x96x5000", "--splits", "0,1,8"])
    a = sweep.parse()
    assert (a.triples, a.splits, a.configs) == ("256x96x5000", "0,1,8", None)
