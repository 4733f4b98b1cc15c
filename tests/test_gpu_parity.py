"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Bar (per tensor h and y): every element |got - ref| <= 2e-3 + 1e-2 |ref| and
every token row's cosine >= 0.999995; the oracle rounds FP64 to bf16 once, the
GPU accumulates in FP32, so a few elements may differ by one bf16 step.
Covered: every E4M3 code and E8M0 edge scale through the real kernel, small
shapes spanning several tiles with ragged tails and every rows-per-wave
variant, 24 seeded random shapes (ragged H, I, E, k, B; both kernel families;
uniform or skewed routing), the five synthetic workloads at full size and
every token of their batches (the 48-layer workload on all 48 layers at 1
token, every fourth at 8 and layers 1, 24 and 47 at 32; the 8-layer wide
workload on layer 0 at every batch size and on layers 1-7 at 1 token),
empty batches, out-of-range expert ids, full coverage of the outputs
(sentinels and guard words), determinism and non-default streams.
"""
import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi
import oracle
from oracle.compare import parity, passes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _t(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


class DevLayer:
    def __init__(self, L, dev):
        self.L = L
        self.H, self.I, self.E = L.H, L.I, L.E
        self.wg, self.sg, self.wu, self.su, self.wd, self.sd = (
            _t(a, dev) for a in (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down))

    def host(self):
        L = self.L
        return (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)


# kernel families: (gate/up variant, down variant); None = the built-in table's choice
PER_SLOT = (mg.MOE_GATE_UP_PER_SLOT, mg.MOE_DOWN_PER_TOKEN)
GROUPED = (mg.MOE_GATE_UP_EXPERT_GROUPED, mg.MOE_DOWN_EXPERT_GROUPED)
FAMILIES = [PER_SLOT, GROUPED]
BOTH = (None, PER_SLOT, GROUPED)


def run_gpu(D, x, ids, w, dev, rows_gu=None, rows_dn=None, stream=None, variant=None):
    B, k = ids.shape
    vg, vd = variant if variant is not None else (None, None)
    xd, idd, wdv = _t(x, dev), _t(ids, dev), _t(w, dev)
    h = torch.empty((B, k, D.I), dtype=torch.int16, device=dev)
    y = torch.empty((B, D.H), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(xd, idd, D.wg, D.sg, D.wu, D.su, h, stream=stream, rows_per_wave=rows_gu, variant=vg)
    mg.moe_decode_down(h, idd, wdv, D.wd, D.sd, y, stream=stream, rows_per_wave=rows_dn, variant=vd)
    torch.cuda.synchronize()
    return h.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16)


# at most one element in N_DIFF_DIV may differ from the oracle's bf16 at all
N_DIFF_DIV = 200


def _few_flips(p):
    return p["n_diff"] <= max(8, p["n"] // N_DIFF_DIV)


def check(h, y, h_ref, y_ref, B, k, what="", own=None):
    """The layer's bar for h and y against the oracle (every element within
    2e-3 + 1e-2 |ref|, every row's cosine >= 0.999995, the same NaNs), plus a
    guard against systematic rounding errors: FP32 accumulation flips the bf16
    rounding of a few near-ties, a rounding mistake (e.g. truncation) about
    half of them.  h is compared with the oracle's h directly.  y depends on
    h, and one flipped h element moves every output of its token, so y's
    flips are counted against the oracle's down projection of the GPU's own h
    (own = (layer, ids, weights)); without `own`, only when h matched exactly."""
    ph = parity(h, h_ref, B * k)
    py = parity(y, y_ref, B)
    print(f"{what} h: {ph}\n{what} y: {py}", flush=True)
    assert passes(ph), (what, ph)
    assert passes(py), (what, py)
    assert _few_flips(ph), (what, "h", ph)
    if ph["n_diff"] == 0:
        assert _few_flips(py), (what, "y", py)
    elif own is not None:
        D, ids, w = own
        py_own = parity(y, oracle.down(h, ids, w, D.L.w_down, D.L.s_down), B)
        print(f"{what} y against the oracle's down of the GPU's h: {py_own}", flush=True)
        assert _few_flips(py_own), (what, "y from the GPU's h", py_own)
    return ph, py


# --------------------------------------------------------------- decode path
@pytest.mark.parametrize("scale", [127, 120, 134, 1, 0, 253, 255])
@pytest.mark.parametrize("dvariant", [mg.MOE_DOWN_PER_TOKEN, mg.MOE_DOWN_EXPERT_GROUPED])
def test_every_e4m3_code_through_down_kernel(dev, scale, dvariant):
    """y[o] = w * dec(code o) * 2^(scale-127) * h[0]: one product per output, so exact."""
    E, H, I, k, B = 1, 256, 32, 1, 1
    wd = np.zeros((E, H, I), np.uint8)
    wd[0, :, 0] = np.arange(256, dtype=np.uint8)
    sd = np.full((E, H, I // 32), scale, np.uint8)
    h = np.zeros((B, k, I), np.uint16)
    h[0, 0, 0] = 0x3F80   # 1.0
    ids = np.zeros((B, k), np.int32)
    w = np.ones((B, k), np.float32)
    y = torch.empty((B, H), dtype=torch.int16, device=dev)
    mg.moe_decode_down(_t(h, dev), _t(ids, dev), _t(w, dev), _t(wd, dev), _t(sd, dev), y, variant=dvariant)
    torch.cuda.synchronize()
    got = y.cpu().numpy().view(np.uint16)[0]
    ref = oracle.down(h, ids, w, wd, sd)[0]
    gv, rv = oracle.bf16_to_f64(got), oracle.bf16_to_f64(ref)
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    ok = ~np.isnan(rv)
    assert np.array_equal(gv[ok], rv[ok]), np.nonzero(gv != rv)


@pytest.mark.parametrize("scale", [127, 120, 134, 1, 0, 253, 255])
@pytest.mark.parametrize("gvariant", [mg.MOE_GATE_UP_PER_SLOT, mg.MOE_GATE_UP_EXPERT_GROUPED])
def test_every_e4m3_code_through_gate_up_kernel(dev, scale, gvariant):
    """Neuron n's gate row holds E4M3 code n in element 0 with E8M0 scale `scale`, its up
    row 1.0 * 2^0, and x = e_0: gate = dec(n) * 2^(scale-127) and up = 1 exactly, so
    h[n] = bf16(SiLU(gate)).  NaN codes (0x7F, 0xFF) and the NaN scale 255 give NaN, an
    infinite gate infinity (or -0); everything else meets the layer's bar."""
    E, H, I, k, B = 1, 32, 256, 1, 1
    wg = np.zeros((E, I, H), np.uint8)
    wg[0, :, 0] = np.arange(256, dtype=np.uint8)
    sg = np.full((E, I, H // 32), scale, np.uint8)
    wu = np.zeros((E, I, H), np.uint8)
    wu[0, :, 0] = 0x38                   # E4M3 1.0
    su = np.full((E, I, H // 32), 127, np.uint8)
    x = np.zeros((B, H), np.uint16)
    x[0, 0] = 0x3F80                      # 1.0
    ids = np.zeros((B, k), np.int32)
    h = torch.empty((B, k, I), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(_t(x, dev), _t(ids, dev), _t(wg, dev), _t(sg, dev), _t(wu, dev), _t(su, dev), h,
                          variant=gvariant)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(h.cpu().numpy().view(np.uint16).ravel())
    ref = oracle.bf16_to_f64(oracle.gate_up(x, ids, wg, sg, wu, su).ravel())
    assert np.array_equal(np.isnan(got), np.isnan(ref)), np.nonzero(np.isnan(got) != np.isnan(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(got[~fin & ~np.isnan(ref)], ref[~fin & ~np.isnan(ref)])   # infinities exactly
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref[fin])), (scale, np.max(err))


# Tiny block scales with activations large enough that the products are
# ordinary numbers again: a kernel that rounded the scaled weights to bf16
# subnormals (or flushed them) would miss by far more than the bar here, which
# is relative only.  The bf16 activation 2^p (p <= 100, so no FP32 partial sum
# overflows) brings dec(code) * 2^(scale - 127) * 2^p to at least 2^-36.
TINY_SCALES = [0, 1, 5, 9, 10, 27, 54, 63, 64, 100]


def _pow2_bf16(p):
    return np.uint16((p + 127) << 7)


@pytest.mark.parametrize("scale", TINY_SCALES)
@pytest.mark.parametrize("gvariant", [mg.MOE_GATE_UP_PER_SLOT, mg.MOE_GATE_UP_EXPERT_GROUPED,
                                      mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA])
def test_tiny_scales_through_gate_up_kernel(dev, scale, gvariant):
    """Every gate block of neuron n at E8M0 code `scale`, E4M3 code n in element 0
    (the rest zero), its up row 2^-p in element 0, x = 2^p e_0: gate = dec(n) *
    2^(scale - 127 + p), up = 1 exactly, h[n] = bf16(SiLU(gate)), checked to 1 %
    of its own size (zero exactly); the NaN codes give NaN."""
    E, H, I, k, B = 1, 2048, 256, 1, 1
    p = min(100, 124 - scale)     # |gate| <= 448 / 8: SiLU stays a normal number
    wg = np.zeros((E, I, H), np.uint8)
    wg[0, :, 0] = np.arange(256, dtype=np.uint8)
    sg = np.full((E, I, H // 32), scale, np.uint8)
    wu = np.zeros((E, I, H), np.uint8)
    wu[0, :, 0] = 0x38                   # E4M3 1.0
    su = np.full((E, I, H // 32), 127 - p, np.uint8)
    x = np.zeros((B, H), np.uint16)
    x[0, 0] = _pow2_bf16(p)
    ids = np.zeros((B, k), np.int32)
    h = torch.empty((B, k, I), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(_t(x, dev), _t(ids, dev), _t(wg, dev), _t(sg, dev), _t(wu, dev), _t(su, dev), h,
                          variant=gvariant)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(h.cpu().numpy().view(np.uint16).ravel())
    ref = oracle.bf16_to_f64(oracle.gate_up(x, ids, wg, sg, wu, su).ravel())
    assert np.array_equal(np.isnan(got), np.isnan(ref)), np.nonzero(np.isnan(got) != np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.all(np.isfinite(ref[fin])) and np.min(np.abs(ref[fin & (ref != 0)])) >= 2.0 ** -100   # normal
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= 1e-2 * np.abs(ref[fin])), (scale, np.nonzero(err > 1e-2 * np.abs(ref[fin])))


@pytest.mark.parametrize("scale", TINY_SCALES)
@pytest.mark.parametrize("dvariant", [mg.MOE_DOWN_PER_TOKEN, mg.MOE_DOWN_EXPERT_GROUPED,
                                      mg.MOE_DOWN_EXPERT_GROUPED_MFMA])
def test_tiny_scales_through_down_kernel(dev, scale, dvariant):
    """Every block of row o at E8M0 code `scale`, E4M3 code o in element 0, h =
    2^p e_0, router weight 1: y[o] = dec(o) * 2^(scale - 127 + p), one product,
    so exact."""
    E, H, I, k, B = 1, 256, 768, 1, 1
    p = min(100, 127 - scale)
    wd = np.zeros((E, H, I), np.uint8)
    wd[0, :, 0] = np.arange(256, dtype=np.uint8)
    sd = np.full((E, H, I // 32), scale, np.uint8)
    h = np.zeros((B, k, I), np.uint16)
    h[0, 0, 0] = _pow2_bf16(p)
    ids = np.zeros((B, k), np.int32)
    w = np.ones((B, k), np.float32)
    y = torch.empty((B, H), dtype=torch.int16, device=dev)
    mg.moe_decode_down(_t(h, dev), _t(ids, dev), _t(w, dev), _t(wd, dev), _t(sd, dev), y, variant=dvariant)
    torch.cuda.synchronize()
    gv = oracle.bf16_to_f64(y.cpu().numpy().view(np.uint16)[0])
    rv = oracle.bf16_to_f64(oracle.down(h, ids, w, wd, sd)[0])
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    ok = ~np.isnan(rv)
    assert np.min(np.abs(rv[ok & (rv != 0)])) >= 2.0 ** -40
    assert np.array_equal(gv[ok], rv[ok]), np.nonzero(gv != rv)


# --------------------------------------------------------------- small shapes
SMALL = [
    # B, H, I, E, k
    (1, 2048, 64, 8, 8),
    (3, 2048, 96, 16, 8),
    (5, 256, 64, 8, 2),
    (2, 4096, 160, 8, 4),
    (4, 2080, 800, 6, 3),     # ragged last pass (2080 = 2 x 1024 + 32), k*I = 2400
    (7, 32, 32, 4, 4),        # one 32-element block per row: most lanes clamped
    (2, 6144, 96, 4, 2),      # six passes over a row
    (3, 1024, 1536, 8, 8),    # twelve passes in down
    (2, 8192, 64, 3, 2),      # the widest supported rows
    (1, 2048, 2048, 8, 8),    # the longest supported down reduction (k*I = 16384)
]


@pytest.fixture(scope="module")
def small_layers(dev):
    return {s: DevLayer(mi.make_layer(100 + i, s[1], s[2], s[3]), dev) for i, s in enumerate(SMALL)}


@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
@pytest.mark.parametrize("rows", [None, 1, 2, 4, 8])
@pytest.mark.parametrize("variant", FAMILIES, ids=["per_slot", "grouped"])
def test_small_shapes_all_variants(dev, small_layers, shape, rows, variant):
    B, H, I, E, k = shape
    D = small_layers[shape]
    # register-feasible variants only (passes of 1024 elements per lane group);
    # the grouped down kernel takes 8 rows (I <= 1024) or 4
    n_gu, n_dn = -(-H // 1024), -(-(k * I) // 1024)
    cap = 16 if variant == PER_SLOT else 8
    rows_gu = rows if rows is None or rows * n_gu <= cap else None
    if variant == PER_SLOT:
        rows_dn = rows if rows is None or n_dn * (5 * rows + 8) <= 224 else None
    else:
        rows_dn = rows if rows == (8 if I <= 1024 else 4) else None
    x = mi.make_x(7, B, H)
    ids, w = mi.route_uniform(7, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev, rows_gu, rows_dn, variant=variant)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"{shape} rows={rows} variant={variant}", own=(D, ids, w))


def _random_case(i):
    """Seeded random shape within the kernels' limits, its routing and launch choices."""
    g = np.random.default_rng(9000 + i)
    k = int(g.integers(1, 9))
    E = int(g.integers(k, 41))
    B = int(g.integers(1, 41))
    H = 32 * int(g.integers(1, 97))      # up to 3072
    I = 32 * int(g.integers(1, 49))      # up to 1536
    while k * I > 16384:
        I -= 32
    variant = FAMILIES[int(g.integers(0, 2))]
    skew = bool(g.integers(0, 2))        # Zipf-like popularity: tokens share experts
    return B, H, I, E, k, variant, skew, int(g.integers(0, 4))


@pytest.mark.parametrize("i", range(24))
def test_random_shapes(dev, i):
    """Random shapes, ragged everywhere, both kernel families, random rows per wave
    (the table's choice when the draw is beyond a kernel's limits), uniform or
    skewed routing; against the oracle."""
    B, H, I, E, k, variant, skew, rsel = _random_case(i)
    D = DevLayer(mi.make_layer(9100 + i, H, I, E), dev)
    x = mi.make_x(9200 + i, B, H)
    ids, w = (mi.route_zipf if skew else mi.route_uniform)(9300 + i, B, E, k)
    n_gu, n_dn = -(-H // 1024), -(-(k * I) // 1024)
    rows = (1, 2, 4, 8)[rsel]
    if variant == PER_SLOT:
        rows_gu = rows if rows * n_gu <= 16 else None
        rows_dn = rows if n_dn * (5 * rows + 8) <= 224 else None
    else:
        rows_gu = rows if rows * n_gu <= 8 else None
        rows_dn = None
        if -(-I // 1024) > 2 or B > 64:   # beyond the grouped down kernel's limits
            variant = (mg.MOE_GATE_UP_EXPERT_GROUPED, mg.MOE_DOWN_PER_TOKEN)
    h, y = run_gpu(D, x, ids, w, dev, rows_gu, rows_dn, variant=variant)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"random {i}: B={B} H={H} I={I} E={E} k={k} variant={variant} "
                                    f"rows={rows_gu},{rows_dn} skew={skew}", own=(D, ids, w))


@pytest.mark.parametrize("variant", FAMILIES, ids=["per_slot", "grouped"])
def test_duplicate_ids_within_a_token(dev, small_layers, variant):
    """A token may list one expert twice; each slot is computed and summed on its own."""
    shape = (3, 2048, 96, 16, 8)
    B, H, I, E, k = shape
    D = small_layers[shape]
    x = mi.make_x(8, B, H)
    ids, w = mi.route_uniform(8, B, E, k)
    ids[0, 1] = ids[0, 0]
    ids[2, :] = 5
    h, y = run_gpu(D, x, ids, w, dev, variant=variant)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"duplicates variant={variant}", own=(D, ids, w))


@pytest.mark.parametrize("variant", FAMILIES, ids=["per_slot", "grouped"])
def test_one_expert_over_several_work_units(dev, small_layers, variant):
    """Every token routes its first slot to expert 3: 40 slots of one expert, more
    than one work unit holds (16 in gate/up, 8 in down), so the expert's slots are
    cut into several units that different workgroups process -- every workgroup
    must cut them the same way.  Checked against the oracle, and twice for
    bit-identical results."""
    shape = (3, 2048, 96, 16, 8)
    _, H, I, E, k = shape
    B = 40
    D = small_layers[shape]
    x = mi.make_x(9, B, H)
    ids, w = mi.route_uniform(9, B, E, k)
    for b in range(B):
        row = [e for e in ids[b] if e != 3][: k - 1]
        ids[b] = [3] + row + [e for e in range(E) if e != 3 and e not in row][: k - 1 - len(row)]
    assert (ids == 3).sum() == B and all(len(set(r)) == k for r in ids.tolist())
    h, y = run_gpu(D, x, ids, w, dev, variant=variant)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"one expert over several units, variant={variant}", own=(D, ids, w))
    h2, y2 = run_gpu(D, x, ids, w, dev, variant=variant)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)


# --------------------------------------------------------------- full-size workloads
@pytest.fixture(scope="module")
def s1(dev):
    s = mi.SHAPES["S1"]
    return DevLayer(mi.make_layer(mi.layer_seed("single_b1"), s["H"], s["I"], s["E"]), dev)


def _full(D, workload, B, routing, dev, it=0, variants=(None,)):
    seed = mi.routing_seed(workload, B, routing)
    x = mi.make_x(seed, B, D.H, it=it)
    ids, w = mi.make_routing(routing, seed, B, D.E, 8, it=it)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    for v in variants:
        h, y = run_gpu(D, x, ids, w, dev, variant=v)
        check(h, y, h_ref, y_ref, B, 8, f"{workload} B={B} {routing} variant={v}", own=(D, ids, w))


def test_single_layer_b1(dev, s1):
    _full(s1, "single_b1", 1, "uniform", dev)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 24, 32])
def test_batch_sweep(dev, s1, B):
    _full(s1, "batch_sweep", B, "uniform", dev, variants=BOTH)


# the built-in table's switch points at H=2048, E=128, k=8 (down on the matrix
# cores from 5 tokens, gate/up from 10; gate/up's work units of 8 slots, three
# workgroups per CU, up to 42 tokens, of 16 from 43) on either side, and the
# largest batches
@pytest.mark.parametrize("B", [4, 5, 9, 10, 42, 43, 64])
def test_table_switch_points_and_large_batches(dev, s1, B):
    _full(s1, "batch_sweep", B, "uniform", dev)


@pytest.mark.parametrize("routing", ["zipf", "adversarial", "contiguous"])
def test_routing_stress_b32(dev, s1, routing):
    _full(s1, "routing_stress", 32, routing, dev, variants=BOTH)


@pytest.mark.parametrize("layer", [1, 24, 47])
def test_decode_step_layers(dev, layer):
    s = mi.SHAPES["S1"]
    D = DevLayer(mi.make_layer(mi.layer_seed("decode_step", layer), s["H"], s["I"], s["E"]), dev)
    for B in (1, 8, 32):
        seed = mi.routing_seed("decode_step", B, layer=layer)
        x = mi.make_x(seed, B, D.H)
        ids, w = mi.route_uniform(seed, B, D.E, 8)
        h, y = run_gpu(D, x, ids, w, dev)
        h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
        check(h, y, h_ref, y_ref, B, 8, f"decode step layer={layer} B={B}", own=(D, ids, w))


def test_near_tie_in_h_and_the_y_bar(dev):
    """h is rounded to bf16 once, from an FP32 sum on the GPU and from the exact
    FP64 value in the oracle.  Where the exact value lies within a rounding
    error of the midpoint between two bf16 values, the two can round to
    neighbours, and a large h element moved by one bf16 step moves every output
    of its token (here by up to 0.0027, beyond the y bar's absolute part where
    y is small).  Seeded layer of 2048 x 1184, 22 experts, top-1, 45 tokens
    under Zipf routing, which has such a tie: every h element the GPU rounds
    differently from the oracle is either tiny (within the absolute part of the
    bar) or one step away from an exact value within 1/64 of a step of the
    midpoint; and y meets the bar against the oracle's down projection of the
    GPU's own h, which is what the down kernel is given."""
    B, H, I, E, k, seed = 45, 2048, 1184, 22, 1, 150162
    L = mi.make_layer(seed, H, I, E)
    D = DevLayer(L, dev)
    x = mi.make_x(seed, B, H)
    ids, w = mi.route_zipf(seed, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev)
    h_ref, _, _, h64 = oracle.gate_up(x, ids, L.w_gate, L.s_gate, L.w_up, L.s_up, fp64=True)
    ph = parity(h, h_ref, B * k)
    assert passes(ph) and _few_flips(ph), ph
    got = oracle.bf16_to_f64(h.ravel())
    ref = oracle.bf16_to_f64(h_ref.ravel())
    exact = h64.ravel()
    for j in np.nonzero(h.ravel() != h_ref.ravel())[0]:
        if abs(ref[j]) < 2.0 ** -4:
            continue   # inside the bar's absolute part, whatever the rounding
        step = abs(got[j] - ref[j])
        assert abs(int(h.ravel()[j]) - int(h_ref.ravel()[j])) == 1, (j, got[j], ref[j])
        assert abs(exact[j] - 0.5 * (got[j] + ref[j])) <= step / 64, (j, got[j], ref[j], exact[j])
    py_own = parity(y, oracle.down(h, ids, w, L.w_down, L.s_down), B)
    assert passes(py_own) and _few_flips(py_own), py_own
    print("y against the oracle's y:", parity(y, oracle.layer(x, ids, w, *D.host())[1], B), flush=True)


@pytest.mark.parametrize("group", range(6))
def test_decode_step_every_layer(dev, group):
    """Config 4 at full depth: every one of the 48 distinct layers (8 per
    test), each with its own weights and its own routing, at 1 token, and
    every fourth layer at 8 tokens too (32 tokens on layers 1, 24 and 47
    above)."""
    s = mi.SHAPES["S1"]
    for layer in range(8 * group, 8 * group + 8):
        D = DevLayer(mi.make_layer(mi.layer_seed("decode_step", layer), s["H"], s["I"], s["E"]), dev)
        for B in ((1, 8) if layer % 4 == 0 else (1,)):
            seed = mi.routing_seed("decode_step", B, layer=layer)
            x = mi.make_x(seed, B, D.H)
            ids, w = mi.route_uniform(seed, B, D.E, 8)
            h, y = run_gpu(D, x, ids, w, dev)
            h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
            check(h, y, h_ref, y_ref, B, 8, f"decode step layer={layer} B={B}", own=(D, ids, w))
        del D
        torch.cuda.empty_cache()


_WIDE_REF = {}


def wide_case(D, B):
    """Inputs and the oracle's h, y for the whole batch of B tokens of the wide
    workload's layer 0 (computed once per process)."""
    if B not in _WIDE_REF:
        seed = mi.routing_seed("wide_layers", B, layer=0)
        x = mi.make_x(seed, B, D.H)
        ids, w = mi.route_uniform(seed, B, D.E, 8)
        _WIDE_REF[B] = (x, ids, w) + tuple(oracle.layer(x, ids, w, *D.host()))
    return _WIDE_REF[B]


@pytest.mark.parametrize("B", [1, 16, 32, 64])
def test_wide_layer(dev, s2, B):
    """Every token of the batch, every kernel family."""
    x, ids, w, h_ref, y_ref = wide_case(s2, B)
    for v in BOTH:
        h, y = run_gpu(s2, x, ids, w, dev, variant=v)
        check(h, y, h_ref, y_ref, B, 8, f"wide layer B={B} variant={v}", own=(s2, ids, w))


@pytest.mark.parametrize("layer", range(1, 8))
def test_wide_every_layer(dev, layer):
    """Config 5 at full depth: layers 1-7 of the 8 distinct wide layers (layer 0
    is checked above at every batch size), each with its own weights and
    routing, at 1 token, and the last one at 16 tokens too."""
    s = mi.SHAPES["S2"]
    D = DevLayer(mi.make_layer(mi.layer_seed("wide_layers", layer), s["H"], s["I"], s["E"]), dev)
    for B in ((1, 16) if layer == 7 else (1,)):
        seed = mi.routing_seed("wide_layers", B, layer=layer)
        x = mi.make_x(seed, B, D.H)
        ids, w = mi.route_uniform(seed, B, D.E, 8)
        h, y = run_gpu(D, x, ids, w, dev)
        h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
        check(h, y, h_ref, y_ref, B, 8, f"wide layer {layer} B={B}", own=(D, ids, w))
    del D
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [4, 5, 27, 28])
def test_wide_layer_table_switch_point(dev, s2, B):
    """H=4096, I=1536: the built-in table moves down to the matrix cores at 5
    tokens, gate/up to the vector-unit grouped kernel at 5 and to the matrix
    cores at 28; every token on either side."""
    x, ids, w, h_ref, y_ref = wide_case(s2, B)
    h, y = run_gpu(s2, x, ids, w, dev)
    check(h, y, h_ref, y_ref, B, 8, f"wide layer B={B} built-in table", own=(s2, ids, w))


# --------------------------------------------------------------- properties
def test_output_coverage_and_guards(dev, s1):
    B, k, G = 5, 8, 4096
    x = mi.make_x(55, B, s1.H)
    ids, w = mi.route_uniform(55, B, s1.E, k)
    hbuf = torch.full((B * k * s1.I + 2 * G,), -1, dtype=torch.int16, device=dev)   # 0xFFFF = NaN sentinel
    ybuf = torch.full((B * s1.H + 2 * G,), -1, dtype=torch.int16, device=dev)
    h = hbuf[G:G + B * k * s1.I].view(B, k, s1.I)
    y = ybuf[G:G + B * s1.H].view(B, s1.H)
    xd, idd, wdv = _t(x, dev), _t(ids, dev), _t(w, dev)
    mg.moe_decode_gate_up(xd, idd, s1.wg, s1.sg, s1.wu, s1.su, h)
    mg.moe_decode_down(h, idd, wdv, s1.wd, s1.sd, y)
    torch.cuda.synchronize()
    hb, yb = hbuf.cpu().numpy().view(np.uint16), ybuf.cpu().numpy().view(np.uint16)
    assert np.all(hb[:G] == 0xFFFF) and np.all(hb[-G:] == 0xFFFF)
    assert np.all(yb[:G] == 0xFFFF) and np.all(yb[-G:] == 0xFFFF)
    assert not np.any(hb[G:-G] == 0xFFFF) and not np.any(yb[G:-G] == 0xFFFF)


@pytest.mark.parametrize("B", [8, 32])
def test_deterministic(dev, s1, B):
    """Same inputs, same bits, for both kernel families (the grouped kernels sort
    slots with LDS atomics; the sort is put back in slot order).  Token 0 lists
    one expert three times, so a timing-dependent slot order would show."""
    x = mi.make_x(66, B, s1.H)
    ids, w = mi.route_uniform(66, B, s1.E, 8)
    ids[0, 1] = ids[0, 2] = ids[0, 0]
    for v in BOTH:
        a = run_gpu(s1, x, ids, w, dev, variant=v)
        for _ in range(3):
            b = run_gpu(s1, x, ids, w, dev, variant=v)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), v


def test_nondefault_stream(dev, s1):
    x = mi.make_x(77, 4, s1.H)
    ids, w = mi.route_uniform(77, 4, s1.E, 8)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        h, y = run_gpu(s1, x, ids, w, dev, stream=st)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    check(h, y, h_ref, y_ref, 4, 8, "stream", own=(s1, ids, w))


def test_graph_replay_matches_eager(dev, s1):
    """Both kernels captured into one HIP graph; every replay (with eager work and
    synchronisations in between) reproduces the eager result bit for bit."""
    B, k = 6, 8
    x = mi.make_x(99, B, s1.H)
    ids, w = mi.route_uniform(99, B, s1.E, k)
    xd, idd, wdv = _t(x, dev), _t(ids, dev), _t(w, dev)
    h = torch.empty((B, k, s1.I), dtype=torch.int16, device=dev)
    y = torch.empty((B, s1.H), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(xd, idd, s1.wg, s1.sg, s1.wu, s1.su, h)
    mg.moe_decode_down(h, idd, wdv, s1.wd, s1.sd, y)
    torch.cuda.synchronize()
    h_eager, y_eager = h.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.moe_decode_gate_up(xd, idd, s1.wg, s1.sg, s1.wu, s1.su, h)
        mg.moe_decode_down(h, idd, wdv, s1.wd, s1.sd, y)
    for rep in range(4):
        h.fill_(-1)
        y.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_eager) and torch.equal(y, y_eager), rep
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    check(h.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16), h_ref, y_ref, B, k, "graph",
          own=(s1, ids, w))


def test_empty_batch(dev, s1):
    x = torch.empty((0, s1.H), dtype=torch.int16, device=dev)
    ids = torch.empty((0, 8), dtype=torch.int32, device=dev)
    w = torch.empty((0, 8), dtype=torch.float32, device=dev)
    h = torch.empty((0, 8, s1.I), dtype=torch.int16, device=dev)
    y = torch.empty((0, s1.H), dtype=torch.int16, device=dev)
    mg.moe_decode_gate_up(x, ids, s1.wg, s1.sg, s1.wu, s1.su, h)
    mg.moe_decode_down(h, ids, w, s1.wd, s1.sd, y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant", FAMILIES, ids=["per_slot", "grouped"])
def test_out_of_range_ids_give_nan_not_faults(dev, s1, variant):
    B, k = 4, 8
    x = mi.make_x(88, B, s1.H)
    ids, w = mi.route_uniform(88, B, s1.E, k)
    bad = ids.copy()
    bad[1, 3] = -1
    bad[2, 0] = s1.E
    h, y = run_gpu(s1, x, bad, w, dev, variant=variant)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    hv, yv = oracle.bf16_to_f64(h), oracle.bf16_to_f64(y)
    assert np.all(np.isnan(hv[1, 3])) and np.all(np.isnan(hv[2, 0]))
    assert np.all(np.isnan(yv[1])) and np.all(np.isnan(yv[2]))
    mask = np.ones((B, k), bool)
    mask[1, 3] = mask[2, 0] = False
    assert passes(parity(h[mask], h_ref[mask], int(mask.sum())))
    assert passes(parity(y[[0, 3]], y_ref[[0, 3]], 2))


def test_copy_and_read_peak_kernels(dev):
    n = 64 << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    mg.moe_decode_copy_peak(src, dst)
    mg.moe_decode_read_peak(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
