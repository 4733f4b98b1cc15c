"""Per-workload parity report of the layer (the built-in kernel choice) against
the oracle, in the style of the blog post's "Hardware efficiency" section
(minimum cosine and maximum absolute difference over every batch size).

For each of the five synthetic workloads and each of its batch sizes, the
whole batch goes through moe_decode_gate_up + moe_decode_down and h and y are
compared with the oracle element by element: max |got - ref|, the worst ratio
to the bound 2e-3 + 1e-2 |ref|, the minimum per-row cosine and the number of
elements that differ at all.  The table is printed (run pytest with -s) and,
when MOE_PARITY_REPORT names a file, written there as JSON.
"""
import json
import os

import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi
import oracle
from tests.test_gpu_parity import DevLayer, check, run_gpu, wide_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _row(workload, B, routing, D, x, ids, w, dev, h_ref=None, y_ref=None):
    if h_ref is None:
        h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    h, y = run_gpu(D, x, ids, w, dev)
    ph, py = check(h, y, h_ref, y_ref, B, ids.shape[1], f"report {workload} B={B} {routing}", own=(D, ids, w))
    vg, _, _ = mg.moe_decode_gate_up_plan(B, D.H, D.I, D.E, ids.shape[1])
    vd, _, _ = mg.moe_decode_down_plan(B, D.H, D.I, D.E, ids.shape[1])
    r = {"workload": workload, "B": B, "routing": routing, "gate_up_variant": vg, "down_variant": vd}
    for name, p in (("h", ph), ("y", py)):
        r.update({f"{name}_max_abs": p["max_abs"], f"{name}_worst_ratio": round(p["worst_ratio"], 4),
                  f"{name}_min_cos": p["min_cos"], f"{name}_n_diff": p["n_diff"], f"{name}_n": p["n"]})
    return r


def test_parity_report(dev, s2):
    s = mi.SHAPES["S1"]
    s1 = DevLayer(mi.make_layer(mi.layer_seed("single_b1"), s["H"], s["I"], s["E"]), dev)
    rows = []

    def s1_case(workload, B, routing, D=s1, layer=None):
        seed = mi.routing_seed(workload, B, routing) if layer is None else mi.routing_seed(workload, B, layer=layer)
        x = mi.make_x(seed, B, D.H)
        ids, w = mi.make_routing(routing, seed, B, D.E, 8)
        rows.append(_row(workload, B, routing, D, x, ids, w, dev))

    s1_case("single_b1", 1, "uniform")
    for B in (1, 2, 4, 8, 16, 32):
        s1_case("batch_sweep", B, "uniform")
    for routing in ("zipf", "adversarial", "contiguous"):
        s1_case("routing_stress", 32, routing)
    d24 = DevLayer(mi.make_layer(mi.layer_seed("decode_step", 24), s["H"], s["I"], s["E"]), dev)
    for B in (1, 8, 32):
        s1_case("decode_step", B, "uniform", D=d24, layer=24)
    del d24
    for B in (1, 16, 32, 64):
        x, ids, w, h_ref, y_ref = wide_case(s2, B)
        rows.append(_row("wide_layers", B, "uniform", s2, x, ids, w, dev, h_ref, y_ref))

    hdr = ("workload", "B", "routing", "h max|d|", "h min cos", "h diff", "y max|d|", "y min cos", "y diff")
    print("\n| " + " | ".join(hdr) + " |\n|" + "---|" * len(hdr))
    for r in rows:
        print(f"| {r['workload']} | {r['B']} | {r['routing']} | {r['h_max_abs']:.3g} | {r['h_min_cos']:.9f} | "
              f"{r['h_n_diff']}/{r['h_n']} | {r['y_max_abs']:.3g} | {r['y_min_cos']:.9f} | {r['y_n_diff']}/{r['y_n']} |")
    worst = {"h_max_abs": max(r["h_max_abs"] for r in rows), "y_max_abs": max(r["y_max_abs"] for r in rows),
             "h_min_cos": min(r["h_min_cos"] for r in rows), "y_min_cos": min(r["y_min_cos"] for r in rows),
             "h_diff_frac": max(r["h_n_diff"] / r["h_n"] for r in rows),
             "y_diff_frac": max(r["y_n_diff"] / r["y_n"] for r in rows)}
    print("over all workloads:", worst, flush=True)
    out = os.environ.get("MOE_PARITY_REPORT")
    if out:
        with open(out, "w") as f:
            json.dump({"rows": rows, "worst": worst}, f, indent=1)
    assert all(np.isfinite([r["h_max_abs"], r["y_max_abs"]]).all() for r in rows)
