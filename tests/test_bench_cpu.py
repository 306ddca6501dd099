"""bench.py's host-side roofline logic (no GPU): the counter-bound label and
the VALU issue block derived from a profile's counters."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _stats(us):
    return {"median_us": us, "p10_us": us, "p90_us": us, "mean_us": us, "reps": 1}


def _block(prof, us=50.0, kind="mfma", work=1e9, peak=157.3):
    cold = {"single_launch": _stats(us), "warm_single_launch": _stats(us)}
    return bench.roofline(kind, work, _stats(us), cold, prof, peak)


def test_valu_bound_kernel_gets_an_alu_block():
    # 64 lanes x 1e6 wave instructions in 10 us, VALU issue the busiest unit
    prof = {"file": "x.md", "rocprof_avg_us": 10.0, "mfma_busy_pct": 10.0,
            "valu_issue_pct": 60.0, "valu_lane_ops_per_launch": 64e6,
            "hbm_bytes_per_launch": 1e6}
    b = _block(prof, us=10.0)
    assert b["counter_bound"] == "valu"
    v = bench.valu_roofline(b, prof, _stats(10.0))
    assert v["bound"] == "alu" and v["unit"] == "T lane-ops/s (issued)"
    assert abs(v["achieved"] - 6.4) < 1e-12  # 64e6 / 10 us = 6.4e12 lane-ops/s
    # the peak is 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    assert abs(v["peak"] - 256 * 4 * 16 * 2.4e9 / 1e12) < 1e-9
    assert abs(v["frac"] - v["achieved"] / v["peak"]) < 1e-15


def test_hbm_or_mfma_bound_kernels_get_none():
    # counted bytes at 6.4 TB/s over the profiled duration: HBM is the busiest
    prof = {"file": "x.md", "rocprof_avg_us": 10.0, "mfma_busy_pct": 5.0,
            "valu_issue_pct": 40.0, "valu_lane_ops_per_launch": 64e6,
            "hbm_bytes_per_launch": 64e6}
    b = _block(prof, us=10.0, kind="hbm", work=50e6, peak=8000.0)
    assert b["counter_bound"] == "hbm"
    assert bench.valu_roofline(b, prof, _stats(10.0)) is None
    prof2 = dict(prof, mfma_busy_pct=70.0, hbm_bytes_per_launch=1e6)
    b2 = _block(prof2, us=10.0)
    assert b2["counter_bound"] == "mfma"
    assert bench.valu_roofline(b2, prof2, _stats(10.0)) is None


def test_no_profile_means_no_counter_blocks():
    b = _block(None)
    assert "counter_bound" not in b and b["traffic"] is None
    assert bench.valu_roofline(b, None, _stats(50.0)) is None
