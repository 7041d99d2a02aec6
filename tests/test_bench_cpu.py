"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic work
per step against the budget table of the workloads (NS flops N*sum(3p^2q +
p^3), elementwise bytes 12 + 6 per bf16 element), and the traffic figure's
guard on the kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from muon_step_03_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


# (workload, NS algorithmic TFLOP per step, elementwise GB per step): the
# per-configuration budget of the workloads (five iterations; head 12 and
# tail 6 bytes per bf16 element)
BUDGET = [("gpt160m", 1.142, 1.529), ("gpt400m", 5.412, 5.436), ("moe1b", 26.167, 54.585),
          ("stress2k", 813.6, 425.2)]


@pytest.mark.parametrize("name,tflop,gb", BUDGET)
def test_algorithmic_work_matches_budget(name, tflop, gb):
    w = wl.WORKLOADS[name]
    work = bench.matrix_work(w.groups, 2)
    ns = 5 * (work["gram"] + work["poly"] + work["update"])
    assert ns / 1e12 == pytest.approx(tflop, rel=1e-3)
    assert (work["head_bytes"] + work["tail_bytes"]) / 1e9 == pytest.approx(gb, rel=1e-3)


def test_matrix_work_closed_form():
    """One 256x512 and one 512x256 matrix: p = 256, q = 512 for both."""
    class G:
        def __init__(self, count, rows, cols):
            self.count, self.rows, self.cols = count, rows, cols
    work = bench.matrix_work([G(1, 256, 512), G(1, 512, 256)], 4)
    p, q = 256, 512
    assert work["gram"] == 2 * p * p * q
    assert work["poly"] == 2 * p ** 3
    assert work["update"] == 2 * 2 * p * p * q
    assert work["head_bytes"] == 2 * p * q * 16      # fp32: G r 4, M r 4 + w 4, X0 w 4
    assert work["tail_bytes"] == 2 * p * q * 12
    assert work["update_bytes"] == 2 * (p * p + 2 * p * q) * 4   # B r, X r, X' w


def test_traffic_figure_needs_matching_sources(tmp_path, monkeypatch):
    """The committed counter summary is used only while the kernel sources
    hash to the value recorded with it."""
    f = tmp_path / "ns_update_moe1b_hbm_traffic.md"
    f.write_text("traffic_bytes_per_launch: 123456\n"
                 f"kernel_source_sha256: `{bench.kernel_source_hash()}`\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "ns_update_{}_hbm_traffic.md"))
    assert bench.measured_traffic("moe1b") == 123456
    assert bench.measured_traffic("gpt400m") is None
    f.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: `0000`\n")
    assert bench.measured_traffic("moe1b") is None


def test_default_workload_is_the_largest_full_model():
    """The headline is timed on the MoE model (the largest full model of the
    workloads), and the other workloads are listed to be timed after it."""
    ap_args = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = ap_args
    assert args.workload == "moe1b"
    assert max(wl.WORKLOADS[n].n_elements for n in ("gpt160m", "gpt400m", "moe1b")) == \
        wl.WORKLOADS["moe1b"].n_elements
    names = {(n, v) for n, v, _, _ in bench.EXTRAS}
    assert {("gpt160m", "muon"), ("gpt400m", "muon"), ("gpt400m", "muongs"),
            ("stress2k", "muon"), ("fp32_256x512", "muon")} <= names


def test_roofline_picks_the_lower_roof():
    """Below the ridge point (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B) the HBM roof
    bounds a launch, above it the MFMA roof; the reported fraction is the
    bounding roof's, and the MoE-1B update (216 flop/B) is HBM-bound."""
    peak = bench.PEAK_MFMA["bf16"]
    r = bench.roofline(216e9, 1e9, 1e-3, peak)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(1e9 / 1e-3 / bench.PEAK_HBM)
    assert r["mfma_view"]["frac"] == pytest.approx(216e9 / 1e-3 / peak)
    r = bench.roofline(410e9, 1e9, 1e-3, peak)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(410e9 / 1e-3 / peak)
    w = bench.matrix_work(wl.WORKLOADS["moe1b"].groups, 2)
    assert w["update"] / w["update_bytes"] < peak / bench.PEAK_HBM
    w = bench.matrix_work(wl.WORKLOADS["gpt400m"].groups, 2)
    assert w["update"] / w["update_bytes"] > peak / bench.PEAK_HBM
