"""Host-side pieces of bench.py (no GPU): the metric's flop count against the
figures derived independently for the five workloads, the per-phase split, the
Llama owner share, the traffic-summary lookup, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from matrix_optimizer_muon_amd.workloads import workload  # noqa: E402

# effective GFLOP per step, Σ k·(4m²n + 2m³) with k = 5, worked out by hand per
# workload (m = short side, n = long side)
EXPECTED_GFLOP = {
    "single_256x512": 5 * (4 * 256**2 * 512 + 2 * 256**3) / 1e9,
    "layer_d2048": 5 * (4 * (4 * 2048**3 + 2 * 2048**3)
                        + 3 * (4 * 2048**2 * 5632 + 2 * 2048**3)) / 1e9,
    "merged_small": 5 * (256 * (4 * 512**3 + 2 * 512**3)
                         + 128 * (4 * 256**2 * 1024 + 2 * 256**3)) / 1e9,
    "mlp_moe_large": 5 * (4 * (4 * 8192**2 * 28672 + 2 * 8192**3)
                          + 64 * (4 * 1408**2 * 2048 + 2 * 1408**3)) / 1e9,
}


@pytest.mark.parametrize("name", sorted(EXPECTED_GFLOP))
def test_ns_flops_matches_hand_count(name):
    wl = workload(name)
    assert bench.ns_flops(wl.tensors, 5) / 1e9 == pytest.approx(EXPECTED_GFLOP[name], rel=1e-12)


def test_phase_flops_add_up_to_the_metric():
    for name in EXPECTED_GFLOP:
        wl = workload(name)
        pf = bench.phase_flops(wl.tensors)
        assert 5 * (pf["gram"] + pf["square"] + pf["apply"]) == bench.ns_flops(wl.tensors, 5)


def test_llama_owner_share():
    """Slot 0 of the 32-layer model under the LPT rule: 29 matrices, 17 of 4096²,
    8 tall 11008×4096 and 4 wide 4096×11008, 87.6 TFLOP per step."""
    wl, share = bench.select_share("llama_d4096")
    ts = [wl.tensors[i] for i in share]
    shapes = sorted(tuple(t.shape) for t in ts)
    assert len(ts) == 29
    assert shapes.count((4096, 4096)) == 17
    assert shapes.count((11008, 4096)) == 8
    assert shapes.count((4096, 11008)) == 4
    assert len({t.layer for t in ts}) == 29            # one matrix per layer at most
    expect = 5 * (17 * 6 * 4096**3 + 12 * (4 * 4096**2 * 11008 + 2 * 4096**3))
    assert bench.ns_flops(ts, 5) == expect
    assert expect / 1e9 == pytest.approx(87617, rel=1e-4)


def test_measured_traffic_lookup(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("apply", "layer_d2048") is None          # no summary
    f = tmp_path / "traffic_apply_layer_d2048.md"
    f.write_text(f"# x\n\n- kernels_sha256: `{bench.kernels_sha256()}`\n- hbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("apply", "layer_d2048") == 123456.0
    f.write_text("# x\n\n- kernels_sha256: `0000`\n- hbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("apply", "layer_d2048") is None          # other sources


def test_committed_traffic_summaries_parse():
    for kernel, wl in (("apply", "layer_d2048"), ("adamw", "adamw_stream")):
        path = os.path.join(bench.PROFILES, f"traffic_{kernel}_{wl}.md")
        assert os.path.exists(path), path
        fields = dict(l.strip()[2:].split(":", 1) for l in open(path) if l.strip().startswith("- ") and ":" in l)
        assert float(fields["hbm_bytes_per_launch"].strip().strip("`")) > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_lpt_summary_of_the_llama_share():
    """The bench line's partition summary: 8 slots whose loads add up to the
    whole 32-layer model, slot 0 owning 29 matrices, max/mean 1.0207; none for
    a workload stepped whole."""
    s = bench.lpt_summary("llama_d4096")
    model = 32 * (4 * 4096 * 4096 + 3 * 4096 * 11008)
    assert s["slots"] == 8 and s["owner_slot"] == 0 and s["owned_matrices"] == 29
    assert sum(s["slot_loads_elements"]) == model
    assert s["max_over_mean"] == 1.0207
    assert bench.lpt_summary("mlp_moe_large") is None


def test_measured_mfma_busy_lookup(tmp_path, monkeypatch):
    """The counter summary behind the line's `counters`: read only while it was
    taken on the current kernel sources; the committed headline one parses."""
    got = bench.measured_mfma_busy("mlp_moe_large")
    if got is not None:                   # the committed summary matches these sources
        assert {"gram", "square", "apply (0 < t < k-1)"} <= set(got["kernels"])
        assert all(0 <= v["mfma_busy"] <= 1 and 0.5 < v["clock_ghz"] < 2.5 for v in got["kernels"].values())
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_mfma_busy("layer_d2048") is None
    f = tmp_path / "mfma_busy_layer_d2048.md"
    table = ("| kernel | dispatches | average (us) | clock (GHz) | MFMA busy | MFMA instructions / dispatch |\n"
             "|---|---|---|---|---|---|\n| gram | 15 | 100.0 | 1.75 | 64.5% | 1.1e+08 |\n")
    f.write_text(f"# x\n\n- kernels_sha256: `{bench.kernels_sha256()}`\n\n{table}")
    assert bench.measured_mfma_busy("layer_d2048")["kernels"] == {"gram": {"clock_ghz": 1.75, "mfma_busy": 0.645}}
    f.write_text(f"# x\n\n- kernels_sha256: `0000`\n\n{table}")
    assert bench.measured_mfma_busy("layer_d2048") is None
