"""Host-side pieces of bench.py (CPU only): the algorithmic byte count behind
`value` and `roofline.achieved`, and the rule that reports measured HBM
traffic only for the kernel sources it was measured on."""
import json
import os

import numpy as np
import pytest

import bench
import moe_inputs as mi

PER_EXPERT_S1 = 3 * 768 * 2048 + 3 * 768 * 2048 // 32    # 4,866,048 B: gate, up and down rows + scales
PER_EXPERT_S2 = 3 * 1536 * 4096 + 3 * 1536 * 4096 // 32  # 19,464,192 B


def test_per_expert_bytes():
    assert PER_EXPERT_S1 == 4_866_048 and PER_EXPERT_S2 == 19_464_192


@pytest.mark.parametrize("B", [1, 2, 8, 32])
def test_layer_bytes_formula(B):
    """D distinct experts' rows and scales + x read and y written (2H each per token)
    + h written and read (2 * 2I per slot) + ids read twice and a router weight (12 B per slot)."""
    H, I, k = 2048, 768, 8
    ids, _ = mi.route_uniform(mi.routing_seed("batch_sweep", B), B, 128, k)
    d = bench.layer_bytes(ids, H, I, k)
    D = len(set(ids.ravel().tolist()))
    assert d["distinct"] == D
    assert d["total"] == D * PER_EXPERT_S1 + 2 * 2 * B * H + 2 * 2 * B * k * I + 12 * B * k
    assert d["total"] == d["gate_up"] + d["down"]
    # gate/up carries two thirds of every expert's bytes, down one third
    assert d["gate_up"] - (2 * B * H + 2 * B * k * I + 4 * B * k) == D * (2 * 768 * 2048 + 2 * 768 * 2048 // 32)


def test_layer_bytes_one_token_matches_the_worked_figure():
    """One token, 8 distinct experts: 38.96 MB per layer."""
    ids = np.arange(8, dtype=np.int32).reshape(1, 8)
    assert abs(bench.layer_bytes(ids, 2048, 768, 8)["total"] / 1e6 - 38.96) < 0.005


def test_duplicate_experts_counted_once():
    ids = np.array([[3, 3, 5, 7], [5, 3, 9, 11]], np.int32)
    assert bench.layer_bytes(ids, 2048, 768, 4)["distinct"] == 5


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    """profiles/traffic.json is used while its hash equals the current kernel sources' hash."""
    h = bench.kernel_source_hash()
    assert len(h) == 16
    root = tmp_path
    (root / "profiles").mkdir()
    data = {"source_hash": h, "kernels": {"gate_up": {"bytes": 123}}}
    (root / "profiles" / "traffic.json").write_text(json.dumps(data))
    monkeypatch.setattr(bench, "ROOT", str(root))
    # the hash is computed from the sources under ROOT too: point it back at the real tree
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    assert bench.measured_traffic("gate_up") == 123
    assert bench.measured_traffic("down") is None
    data["source_hash"] = "0" * 16
    (root / "profiles" / "traffic.json").write_text(json.dumps(data))
    assert bench.measured_traffic("gate_up") is None


def test_traffic_reported_only_for_its_kernel_and_workload(tmp_path, monkeypatch):
    """The counters were taken on one kernel at one workload: another batch size,
    shape or routing, or the table's other kernel at that size, gets None."""
    h = bench.kernel_source_hash()
    wl = {"B": 32, "H": 2048, "I": 768, "E": 128, "k": 8, "routing": "uniform"}
    data = {"source_hash": h, "workload": wl,
            "kernels": {"gate_up": {"template_name": "moe_gate_up_grouped_mfma_w64", "bytes": 123}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(data))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    assert bench.measured_traffic("gate_up", "moe_gate_up_grouped_mfma_w64", dict(wl)) == 123
    assert bench.measured_traffic("gate_up", "moe_gate_up_3d_batched_w64", dict(wl)) is None
    assert bench.measured_traffic("gate_up", "moe_gate_up_grouped_mfma_w64", dict(wl, B=1)) is None
    assert bench.measured_traffic("gate_up", "moe_gate_up_grouped_mfma_w64", dict(wl, routing="zipf")) is None


def test_committed_traffic_names_its_workload():
    d = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic.json")))
    assert d["workload"] == {"B": 32, "H": 2048, "I": 768, "E": 128, "k": 8, "routing": "uniform"}
    assert set(d["kernels"]) == {"gate_up", "down"}


def test_source_hash_covers_the_build_flags(tmp_path, monkeypatch):
    """A change of the compiler flags changes the hash (and so voids stored counters)."""
    h = bench.kernel_source_hash()
    root = tmp_path
    (root / "moe_gate_up_amd").mkdir()
    os.symlink(os.path.join(bench.ROOT, "moe_gate_up_amd", "csrc"), root / "moe_gate_up_amd" / "csrc")
    src = open(os.path.join(bench.ROOT, "moe_gate_up_amd", "build.py")).read()
    (root / "moe_gate_up_amd" / "build.py").write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.kernel_source_hash() == h
    (root / "moe_gate_up_amd" / "build.py").write_text(src + "\n# -O2\n")
    assert bench.kernel_source_hash() != h


def test_source_hash_covers_every_kernel_source():
    csrc = os.path.join(bench.ROOT, "moe_gate_up_amd", "csrc")
    files = [f for f in os.listdir(csrc) if f.endswith((".hpp", ".hip"))]
    assert "moe_decode.hip" in files and "router.hpp" in files and len(files) >= 8


@pytest.mark.parametrize("B,expect", [
    (1, "gate_up per-slot, down per-token"),
    (8, "gate_up per-slot, down matrix-core grouped"),
    (32, "gate_up matrix-core grouped, down matrix-core grouped"),
])
def test_kernel_choice_names_the_table_s_kernels(B, expect):
    # the names bench prints beside each timed row come from the library's own
    # plan calls (host-only: no GPU needed), H=2048, I=768, 128 experts, top-8
    assert bench.kernel_choice(B, 2048, 768, 128, 8) == expect
