"""GPU parity of the matrix-core expert-grouped gate/up kernel
(MOE_GATE_UP_EXPERT_GROUPED_MFMA) against the oracle, through the C ABI.

Same bar as the other layer tests (tests/test_gpu_parity.py): every element
|got - ref| <= 2e-3 + 1e-2 |ref| and every row's cosine >= 0.999995.  The kernel
rounds each scaled weight to bf16 (exact while it is a normal bf16) and sums in
FP32 in a different order than the vector-unit kernels, so a few bf16 outputs
may differ by one step.  Covered: small shapes (H a multiple of 2048, I from
32 to 2048, units of 1 to 16 slots, an expert cut into several units), every E4M3 code at
edge E8M0 scales including the shifted path for codes above 246, seeded random
shapes with uniform or skewed routing, the S1 and S2 workloads, determinism,
the kernel's limits (1024 slots over 1024 experts at H = 8192, one workgroup
per CU), out-of-range ids and the router step in front of it.
"""
import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi
import oracle
from oracle.compare import parity, passes
from tests.test_gpu_parity import DevLayer, _t, check, run_gpu, wide_case

pytestmark = pytest.mark.gpu

MFMA = (mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA, None)   # down: the table's choice


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


SMALL = [
    # B, H, I, E, k
    (1, 2048, 64, 8, 8),
    (3, 2048, 96, 16, 8),
    (2, 4096, 160, 8, 4),
    (2, 6144, 96, 4, 2),
    (3, 2048, 1536, 8, 8),
    (2, 8192, 64, 3, 2),
    (1, 2048, 2048, 8, 8),
    (5, 4096, 1280, 6, 3),
    (20, 2048, 96, 4, 4),     # 20 slots per expert: units of 16 and 4
    (40, 2048, 96, 16, 8),
    (64, 2048, 32, 128, 8),   # 512 slots over 128 experts; I = 32: two 16-neuron items per unit
    (7, 2048, 48 * 32, 5, 5),  # k = E: every expert in every token
]


@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(dev, shape):
    B, H, I, E, k = shape
    D = DevLayer(mi.make_layer(300 + SMALL.index(shape), H, I, E), dev)
    x = mi.make_x(31, B, H)
    ids, w = mi.route_uniform(31 + B, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev, variant=MFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"mfma {shape}", own=(D, ids, w))


@pytest.mark.parametrize("scale", [127, 120, 134, 1, 0, 246, 247, 253, 254, 255])
def test_every_e4m3_code_at_edge_scales(dev, scale):
    """Neuron n's gate row holds E4M3 code n in element 0 with E8M0 code `scale`
    (the rest of the row zero, scale 127), its up row 1.0, x = e_0: h[n] =
    bf16(SiLU(dec(n) * 2^(scale-127))).  Codes above 246 take the shifted path;
    NaN codes give NaN, infinite gates infinity (or -0)."""
    E, H, I, k, B = 1, 2048, 256, 1, 1
    wg = np.zeros((E, I, H), np.uint8)
    wg[0, :, 0] = np.arange(256, dtype=np.uint8)
    sg = np.full((E, I, H // 32), 127, np.uint8)
    sg[0, :, 0] = scale
    wu = np.zeros((E, I, H), np.uint8)
    wu[0, :, 0] = 0x38                   # E4M3 1.0
    su = np.full((E, I, H // 32), 127, np.uint8)
    x = np.zeros((B, H), np.uint16)
    x[0, 0] = 0x3F80                      # 1.0
    ids = np.zeros((B, k), np.int32)
    h = torch.empty((B, k, I), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(_t(x, dev), _t(ids, dev), _t(wg, dev), _t(sg, dev), _t(wu, dev), _t(su, dev), h,
                          variant=mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(h.cpu().numpy().view(np.uint16).ravel())
    ref = oracle.bf16_to_f64(oracle.gate_up(x, ids, wg, sg, wu, su).ravel())
    assert np.array_equal(np.isnan(got), np.isnan(ref)), np.nonzero(np.isnan(got) != np.isnan(ref))
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf])
    fin = np.isfinite(ref)
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref[fin])), (scale, np.max(err))


def test_big_codes_beside_small_ones(dev):
    """A row whose largest block code is 254 while its other blocks hold ordinary
    codes: the shifted path keeps the ordinary blocks exact (the row's sum is
    dominated by neither)."""
    B, H, I, E, k = 3, 2048, 64, 4, 2
    L = mi.make_layer(77, H, I, E)
    sg = L.s_gate.copy()
    sg[:, :, 5] = 254                     # one block of every gate row at 2^127
    wg = L.w_gate.copy()
    wg[:, :, 160:192] = 0                 # ... whose weights are zero: the sum is the ordinary blocks'
    x = mi.make_x(78, B, H)
    ids, w = mi.route_uniform(79, B, E, k)
    h = torch.empty((B, k, I), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(_t(x, dev), _t(ids, dev), _t(wg, dev), _t(sg, dev), _t(L.w_up, dev), _t(L.s_up, dev),
                          h, variant=mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA)
    torch.cuda.synchronize()
    ref = oracle.gate_up(x, ids, wg, sg, L.w_up, L.s_up)
    p = parity(h.cpu().numpy().view(np.uint16), ref, B * k)
    assert passes(p), p


def _random_case(i):
    g = np.random.default_rng(9500 + i)
    k = int(g.integers(1, 9))
    E = int(g.integers(k, 41))
    B = int(g.integers(1, 65))
    H = 2048 * int(g.integers(1, 3))
    I = 32 * int(g.integers(1, 49))
    while k * I > 16384:
        I -= 32
    return B, H, I, E, k, bool(g.integers(0, 2))


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(dev, i):
    B, H, I, E, k, skew = _random_case(i)
    D = DevLayer(mi.make_layer(9600 + i, H, I, E), dev)
    x = mi.make_x(9700 + i, B, H)
    ids, w = (mi.route_zipf if skew else mi.route_uniform)(9800 + i, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev, variant=MFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"mfma random {i}: B={B} H={H} I={I} E={E} k={k} skew={skew}",
          own=(D, ids, w))


@pytest.fixture(scope="module")
def s1(dev):
    s = mi.SHAPES["S1"]
    return DevLayer(mi.make_layer(mi.layer_seed("single_b1"), s["H"], s["I"], s["E"]), dev)


@pytest.mark.parametrize("B,routing", [(16, "uniform"), (32, "uniform"), (32, "zipf"), (32, "adversarial"),
                                       (64, "uniform"), (64, "zipf")])
def test_s1_workload(dev, s1, B, routing):
    seed = mi.routing_seed("routing_stress" if routing != "uniform" else "batch_sweep", B, routing)
    x = mi.make_x(seed, B, s1.H)
    ids, w = mi.make_routing(routing, seed, B, s1.E, 8)
    h, y = run_gpu(s1, x, ids, w, dev, variant=MFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    check(h, y, h_ref, y_ref, B, 8, f"mfma S1 B={B} {routing}", own=(s1, ids, w))
    h2, y2 = run_gpu(s1, x, ids, w, dev, variant=MFMA)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)


@pytest.mark.parametrize("B", [16, 32, 64])
def test_wide_layer(dev, s2, B):
    """Every token of the wide workload's batch (H=4096, I=1536)."""
    x, ids, w, h_ref, y_ref = wide_case(s2, B)
    h, y = run_gpu(s2, x, ids, w, dev, variant=MFMA)
    check(h, y, h_ref, y_ref, B, 8, f"mfma wide B={B}", own=(s2, ids, w))


@pytest.mark.parametrize("shape", [(1024, 8192, 32, 1024, 1), (96, 2048, 64, 512, 8)],
                         ids=["max: B*k=1024, E=1024, H=8192", "E=512, 1.5 slots per expert"])
def test_large_expert_counts(dev, shape):
    """The kernel's limits: 1024 slots over 1024 experts at H = 8192, where the
    slot index, the chunk buffers and the scale codes take over 80 KB of LDS and
    one workgroup runs per CU; and 768 slots over 512 experts, where the plain
    call picks the matrix cores by itself."""
    B, H, I, E, k = shape
    L = mi.make_layer(400 + E, H, I, E)
    x = mi.make_x(401, B, H)
    ids, _ = mi.route_uniform(402, B, E, k)
    h = torch.empty((B, k, I), dtype=torch.int16, device=dev)
    variant = mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA if E == 1024 else 0
    if variant == 0:
        assert mg.moe_decode_gate_up_plan(B, H, I, E, k)[0] == mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA
    mg.moe_decode_gate_up(_t(x, dev), _t(ids, dev), _t(L.w_gate, dev), _t(L.s_gate, dev), _t(L.w_up, dev),
                          _t(L.s_up, dev), h, variant=variant)
    torch.cuda.synchronize()
    ref = oracle.gate_up(x, ids, L.w_gate, L.s_gate, L.w_up, L.s_up)
    p = parity(h.cpu().numpy().view(np.uint16), ref, B * k)
    assert passes(p), p


def test_out_of_range_ids_give_nan(dev, s1):
    B, k = 40, 8
    x = mi.make_x(88, B, s1.H)
    ids, w = mi.route_uniform(88, B, s1.E, k)
    bad = ids.copy()
    bad[1, 3] = -1
    bad[2, 0] = s1.E
    h, y = run_gpu(s1, x, bad, w, dev, variant=MFMA)
    h_ref, _ = oracle.layer(x, ids, w, *s1.host())
    hv = oracle.bf16_to_f64(h)
    assert np.all(np.isnan(hv[1, 3])) and np.all(np.isnan(hv[2, 0]))
    mask = np.ones((B, k), bool)
    mask[1, 3] = mask[2, 0] = False
    assert passes(parity(h[mask], h_ref[mask], int(mask.sum())))


def test_routed(dev, s1):
    """The router kernel, then the matrix-core kernel on the ids it wrote."""
    B = 64
    seed = mi.routing_seed("batch_sweep", B)
    x = mi.make_x(seed, B, s1.H)
    logits = mi.router_logits(seed, B, s1.E)
    h = torch.empty((B, 8, s1.I), dtype=torch.int16, device=dev)
    ids = torch.empty((B, 8), dtype=torch.int32, device=dev)
    w = torch.empty((B, 8), dtype=torch.float32, device=dev)
    mg.moe_decode_gate_up_routed(_t(x, dev), _t(logits, dev), s1.wg, s1.sg, s1.wu, s1.su, h, ids, w,
                                 variant=mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA)
    torch.cuda.synchronize()
    ri, rw = oracle.route(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), ri)
    h_ref = oracle.gate_up(x, ri, s1.L.w_gate, s1.L.s_gate, s1.L.w_up, s1.L.s_up)
    p = parity(h.cpu().numpy().view(np.uint16), h_ref, B * 8)
    assert passes(p), p


def test_two_host_threads_two_streams(dev, s1):
    """Calls from two host threads on two streams, with shapes whose LDS needs
    differ (64 tokens over 128 experts; 4 tokens over 8 experts at I = 96), each
    thread launching 40 times before it synchronises: both results match the
    oracle (the library keeps no per-call state that one call could change under
    another)."""
    import threading

    small = DevLayer(mi.make_layer(500, 2048, 96, 8), dev)
    cases = []
    for D, B, E, seed in ((s1, 64, s1.E, 501), (small, 4, 8, 502)):
        x = mi.make_x(seed, B, D.H)
        ids, w = mi.route_uniform(seed, B, E, 8 if E > 8 else 4)
        cases.append((D, x, ids, w))
    out = [None, None]
    errs = []

    def work(i):
        try:
            D, x, ids, w = cases[i]
            B, k = ids.shape
            st = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(st):
                xd, idd = _t(x, dev), _t(ids, dev)
                h = torch.empty((B, k, D.I), dtype=torch.int16, device=dev)
                st.synchronize()
                for _ in range(40):
                    mg.moe_decode_gate_up(xd, idd, D.wg, D.sg, D.wu, D.su, h, stream=st,
                                          variant=mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA)
                st.synchronize()
                out[i] = h.cpu().numpy().view(np.uint16)
        except Exception as e:   # reported by the main thread
            errs.append(e)

    ts = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs, errs
    for (D, x, ids, w), h in zip(cases, out):
        ref = oracle.gate_up(x, ids, D.L.w_gate, D.L.s_gate, D.L.w_up, D.L.s_up)
        p = parity(h, ref, ids.size)
        assert passes(p), p


@pytest.mark.parametrize("n_experts", [11, 16, 21], ids=["last round 16 items", "last round 256", "last round 496"])
def test_partial_last_round(dev, s1, n_experts):
    """Two tokens routed so that exactly n_experts experts are used: 48 items per
    expert over a grid of 512, so the last round of the persistent grid holds
    16, 256 or 496 items.  Against the oracle, twice, bit-identical."""
    B, k = 2, 8
    ids = np.array([list(range(8)), list(range(n_experts - 8, n_experts))], np.int32)
    _, w = mi.route_uniform(870, B, s1.E, k)
    x = mi.make_x(871, B, s1.H)
    h, y = run_gpu(s1, x, ids, w, dev, variant=MFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    check(h, y, h_ref, y_ref, B, k, f"mfma last round, {n_experts} experts", own=(s1, ids, w))
    h2, y2 = run_gpu(s1, x, ids, w, dev, variant=MFMA)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)
