"""Checks against the figures the pages print (tests/golden/pages_figures.json), CPU only."""
import json
import os

import numpy as np
import pytest

import moe_inputs as mi

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))["figures"]


def v(name):
    return G[name]["value"]


def test_workload_shape_matches_pages():
    s = mi.SHAPES["S1"]
    assert s["E"] == v("experts_total") and s["k"] == v("experts_routed_per_token") and s["H"] == v("hidden_size")


def test_per_expert_buffer_closed_form():
    # the conventional path's per-expert bf16 output buffer: k rows of H bf16 values per token
    s = mi.SHAPES["S1"]
    assert s["k"] * s["H"] * 2 == v("per_expert_buffer_bytes_per_token")


def test_bandwidth_fraction_consistent():
    assert round(v("sustained_TBps_at_B32") / v("copy_peak_TBps"), 2) == v("fraction_of_copy_peak")


def test_max_abs_diff_is_one_bf16_step(orc):
    # 0.001953 is 2^-9 printed to 6 decimals: one bf16 step for magnitudes in [0.25, 0.5)
    step = orc.bf16_value(orc.bf16_rne(0.25) + 1) - 0.25
    assert step == 2.0 ** -9 and round(step, 6) == v("max_abs_diff")


def test_accuracy_ratio_reproduced(orc):
    """The emulated conventional path (MXFP8 activations, bf16 per-expert buffer) is
    about 1.4x further than warp decode from the full-precision layer."""
    H, I, E, k, B = 2048, 768, 16, 8, 4
    L = mi.make_layer(0, H, I, E, keep_fp32=True)
    x = mi.make_x(0, B, H)
    ids, w = mi.route_uniform(0, B, E, k)
    args = (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    _, y_wd = orc.layer(x, ids, w, *args)
    y_cv = orc.conventional(x, ids, w, *args)
    T = orc.truth_layer(x, ids, w, L.f_gate, L.f_up, L.f_down)
    err = lambda y: np.linalg.norm(orc.bf16_to_f64(y) - T) / np.linalg.norm(T)
    assert err(y_cv) / err(y_wd) == pytest.approx(v("closer_to_fp32_reference"), abs=0.1)
