"""GPU parity of the router step (moe_decode_route and the router prologue
fused into gate/up, moe_decode_gate_up_routed) against the oracle's router,
through the C ABI.

Bar: ids bit-exact (the selection compares FP32 logits, exact on both sides);
routing weights |got - ref| <= 4e-6 ref + 1e-9.  The GPU computes
exp(l_j - l_0) in FP32: the rounded difference costs |l_j - l_0| * 2^-24
relative (N(0,1) logits: below 1e-6), expf about 2^-23, the k-term sum and the
division k * 2^-24 at most; the FP64 oracle is exact by comparison.  The h and
y produced with the selected experts meet the layer's bar (the same check as
the layer parity tests).
"""
import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi
import oracle
from tests.test_gpu_parity import DevLayer, _t, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def check_route(ids, w, logits, k, what):
    ri, rw = oracle.route(logits, k)
    bad = np.argwhere(ids != ri)
    assert bad.size == 0, (what, bad[:5], ids[tuple(bad[0])] if bad.size else None)
    err = np.abs(w.astype(np.float64) - rw)
    tol = 4e-6 * rw + 1e-9
    print(f"{what}: ids exact, weights max rel err {np.max(err / np.maximum(rw, 1e-30)):.2e}", flush=True)
    assert np.all(err <= tol), (what, np.max(err - tol))


def run_route(logits, k, dev):
    B, E = logits.shape
    ids = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((B, k), float("nan"), dtype=torch.float32, device=dev)
    mg.moe_decode_route(_t(logits, dev), ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def tied(seed, B, E):
    g = np.random.default_rng(seed)
    v = (g.integers(-6, 7, size=(B, E)) / 4.0).astype(np.float32)
    v[g.random((B, E)) < 0.1] = -0.0   # -0 and +0 are equal logits
    return v


ROUTE_SHAPES = [
    # B, E, k
    (1, 128, 8), (5, 128, 8), (33, 128, 8), (64, 128, 8), (7, 100, 6), (3, 64, 64), (2, 1, 1),
    (6, 256, 16), (9, 1000, 8), (4, 1024, 64), (130, 32, 4), (3, 65, 60), (2, 513, 3),
]


@pytest.mark.parametrize("shape", ROUTE_SHAPES, ids=[str(s) for s in ROUTE_SHAPES])
def test_route_kernel(dev, shape):
    B, E, k = shape
    for what, logits in (("normal", np.random.default_rng(B * E + k).standard_normal((B, E)).astype(np.float32)),
                         ("ties", tied(B + E + k, B, E))):
        ids, w = run_route(logits, k, dev)
        check_route(ids, w, logits, k, f"route {shape} {what}")


def test_route_kernel_special_values(dev):
    B, E, k = 4, 128, 8
    logits = np.zeros((B, E), np.float32)                      # all equal: ids 0..k-1, weights 1/k
    logits[1] = np.float32(-3.5)
    logits[2] = np.linspace(-1e30, 1e30, E, dtype=np.float32)  # huge gaps: one weight 1, the rest 0
    logits[3, ::2] = np.float32(1e-38)                         # tiny values next to zeros
    ids, w = run_route(logits, k, dev)
    check_route(ids, w, logits, k, "route special values")
    assert np.array_equal(ids[0], np.arange(k)) and np.all(w[0] == np.float32(1 / k))


def test_route_workload_logits(dev):
    """The 128-expert, top-8 router at B = 1..64 on the workload's N(0,1) logits."""
    for B in (1, 8, 32, 64):
        logits = mi.router_logits(mi.routing_seed("single_b1", B), B, 128)
        ids, w = run_route(logits, 8, dev)
        check_route(ids, w, logits, 8, f"route workload B={B}")


# ----------------------------------------------------------- fused into gate/up
def run_routed(D, x, logits, k, dev, variant=None, rows=None):
    B = x.shape[0]
    h = torch.empty((B, k, D.I), dtype=torch.int16, device=dev)
    ids = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((B, k), float("nan"), dtype=torch.float32, device=dev)
    y = torch.empty((B, D.H), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up_routed(_t(x, dev), _t(logits, dev), D.wg, D.sg, D.wu, D.su, h, ids, w,
                                 variant=variant, rows_per_wave=rows)
    mg.moe_decode_down(h, ids, w, D.wd, D.sd, y)
    torch.cuda.synchronize()
    return (h.cpu().numpy().view(np.uint16), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy().view(np.uint16))


def check_routed(D, x, logits, k, got, what):
    h, ids, w, y = got
    check_route(ids, w, logits, k, what)
    ri, rw = oracle.route(logits, k)
    Lh = D.L
    h_ref = oracle.gate_up(x, ri, Lh.w_gate, Lh.s_gate, Lh.w_up, Lh.s_up)
    y_ref = oracle.down(h_ref, ri, rw.astype(np.float32), Lh.w_down, Lh.s_down)
    check(h, y, h_ref, y_ref, x.shape[0], k, what, own=(D, ids, w))


ROUTED_SMALL = [
    # B, H, I, E, k: k % 4 == 0 shares x in LDS, k % 4 != 0 does not; E > 128 runs the router kernel first
    (1, 2048, 64, 8, 8), (3, 256, 96, 16, 4), (5, 256, 64, 8, 2), (4, 2080, 160, 6, 3), (2, 512, 64, 100, 6),
    (3, 256, 64, 200, 8), (2, 1024, 96, 128, 8),
]


@pytest.mark.parametrize("shape", ROUTED_SMALL, ids=[str(s) for s in ROUTED_SMALL])
def test_routed_gate_up_small(dev, shape):
    B, H, I, E, k = shape
    D = DevLayer(mi.make_layer(700 + ROUTED_SMALL.index(shape), H, I, E), dev)
    x = mi.make_x(71, B, H)
    logits = np.random.default_rng(B * E).standard_normal((B, E)).astype(np.float32)
    for variant in (mg.MOE_GATE_UP_PER_SLOT, mg.MOE_GATE_UP_EXPERT_GROUPED):
        got = run_routed(D, x, logits, k, dev, variant=variant)
        check_routed(D, x, logits, k, got, f"routed {shape} variant {variant}")


@pytest.fixture(scope="module")
def s1(dev):
    s = mi.SHAPES["S1"]
    return DevLayer(mi.make_layer(mi.layer_seed("single_b1"), s["H"], s["I"], s["E"]), dev)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_routed_gate_up_workload(dev, s1, B):
    """H=2048, I=768, 128 experts, top-8, with the workload's N(0,1) logits: the
    built-in choice (the fused prologue at 1 token; the router kernel, then the
    per-slot kernel at 8 and the grouped kernel at 32) and, at 8 and 32 tokens,
    the fused per-slot kernel too."""
    seed = mi.routing_seed("single_b1", B)
    x = mi.make_x(seed, B, s1.H)
    logits = mi.router_logits(seed, B, s1.E)
    check_routed(s1, x, logits, 8, run_routed(s1, x, logits, 8, dev), f"routed workload B={B}")
    if B > 1:
        got = run_routed(s1, x, logits, 8, dev, variant=mg.MOE_GATE_UP_PER_SLOT)
        check_routed(s1, x, logits, 8, got, f"routed workload B={B} fused per-slot")


def test_routed_matches_unfused_bitwise(dev, s1):
    """The fused prologue selects exactly what the router kernel selects, and gate/up
    on those ids gives the same bits as gate/up with the prologue."""
    B = 8
    x = mi.make_x(5, B, s1.H)
    logits = tied(5, B, s1.E)
    h, ids, w, _ = run_routed(s1, x, logits, 8, dev, variant=mg.MOE_GATE_UP_PER_SLOT)
    ids2, w2 = run_route(logits, 8, dev)
    assert np.array_equal(ids, ids2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))
    h2 = torch.empty((B, 8, s1.I), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(_t(x, dev), _t(ids2, dev), s1.wg, s1.sg, s1.wu, s1.su, h2,
                          variant=mg.MOE_GATE_UP_PER_SLOT)
    torch.cuda.synchronize()
    assert np.array_equal(h, h2.cpu().numpy().view(np.uint16))


def test_routed_empty_batch(dev, s1):
    x = torch.empty((0, s1.H), dtype=torch.int16, device=dev)
    lg = torch.empty((0, s1.E), dtype=torch.float32, device=dev)
    h = torch.empty((0, 8, s1.I), dtype=torch.int16, device=dev)
    ids = torch.empty((0, 8), dtype=torch.int32, device=dev)
    w = torch.empty((0, 8), dtype=torch.float32, device=dev)
    mg.moe_decode_gate_up_routed(x, lg, s1.wg, s1.sg, s1.wu, s1.su, h, ids, w, B=0, k=8)
    mg.moe_decode_route(lg, ids, w, B=0, k=8)
    torch.cuda.synchronize()
