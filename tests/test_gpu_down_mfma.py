"""GPU parity of the matrix-core expert-grouped down kernel
(MOE_DOWN_EXPERT_GROUPED_MFMA) against the oracle, through the C ABI.

Same bar as the other layer tests (tests/test_gpu_parity.py): every element
|got - ref| <= 2e-3 + 1e-2 |ref|, every row's cosine >= 0.999995, at most one
element in 200 differing from the oracle's down projection of the same h.
The kernel forms 16-element chunk products on the matrix cores (bf16 inputs,
FP32 sums), scales each chunk by its E8M0 scale and adds the chunks in a
fixed order, so a few bf16 outputs may differ by one step from the FP64
oracle.  Covered: every E4M3 code at edge E8M0 scales (NaN code 255, 0, 1,
253, 254), rows shorter than one 256-element round and ragged tails, units of
1 to 8 slots and experts cut into several units, duplicates, k = E, random
shapes with uniform or skewed routing, the S1 and S2 workloads in full,
determinism, 1024 experts, out-of-range ids and empty batches.
"""
import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi
import oracle
from oracle.compare import parity, passes
from tests.test_gpu_parity import DevLayer, _few_flips, _t, check, run_gpu, wide_case

pytestmark = pytest.mark.gpu

DMFMA = (None, mg.MOE_DOWN_EXPERT_GROUPED_MFMA)   # gate/up: the table's choice


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def down_only(dev, h, ids, w, wd, sd, variant=mg.MOE_DOWN_EXPERT_GROUPED_MFMA):
    B, k, I = h.shape
    H = wd.shape[1]
    y = torch.full((B, H), -1, dtype=torch.int16, device=dev)
    mg.moe_decode_down(_t(h, dev), _t(ids, dev), _t(w, dev), _t(wd, dev), _t(sd, dev), y, variant=variant)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("scale", [127, 120, 134, 1, 0, 253, 254, 255])
def test_every_e4m3_code_at_edge_scales(dev, scale):
    """y[o] = w * dec(code o) * 2^(scale-127) * h[0]: one product per output (the
    rest of the row is zero), so exact; NaN codes and the NaN scale give NaN."""
    E, H, I, k, B = 1, 256, 768, 1, 1
    wd = np.zeros((E, H, I), np.uint8)
    wd[0, :, 0] = np.arange(256, dtype=np.uint8)
    sd = np.full((E, H, I // 32), 127, np.uint8)
    sd[0, :, 0] = scale
    h = np.zeros((B, k, I), np.uint16)
    h[0, 0, 0] = 0x3F80   # 1.0
    ids = np.zeros((B, k), np.int32)
    w = np.ones((B, k), np.float32)
    got = oracle.bf16_to_f64(down_only(dev, h, ids, w, wd, sd)[0])
    ref = oracle.bf16_to_f64(oracle.down(h, ids, w, wd, sd)[0])
    assert np.array_equal(np.isnan(got), np.isnan(ref)), np.nonzero(np.isnan(got) != np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), np.nonzero(got != ref)


def test_nan_scale_in_a_later_block_only_poisons_its_row(dev):
    """A NaN scale code in the last block of one row (the block a row's clamped
    chunk re-reads at I = 96) makes that output NaN and no other."""
    E, H, I, k, B = 2, 64, 96, 2, 3
    g = np.random.default_rng(600)
    wd = g.integers(0, 0x7E, (E, H, I), dtype=np.uint8)
    sd = np.full((E, H, I // 32), 120, np.uint8)
    sd[1, 5, 2] = 255
    h = mi.make_x(601, B * k, I).reshape(B, k, I)
    ids = np.array([[0, 1], [1, 0], [0, 0]], np.int32)
    w = np.full((B, k), 0.5, np.float32)
    got = oracle.bf16_to_f64(down_only(dev, h, ids, w, wd, sd))
    ref = oracle.bf16_to_f64(oracle.down(h, ids, w, wd, sd))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[0, 5]) and np.isnan(got[1, 5]) and not np.isnan(got[2, 5])
    ok = ~np.isnan(ref)
    assert np.all(np.abs(got[ok] - ref[ok]) <= 2e-3 + 1e-2 * np.abs(ref[ok]))


SMALL = [
    # B, H, I, E, k
    (1, 2048, 64, 8, 8),       # a quarter round: most chunks re-read the last one
    (3, 2048, 96, 16, 8),
    (5, 256, 64, 8, 2),
    (2, 4096, 160, 8, 4),
    (4, 2080, 800, 6, 3),      # ragged last round (800 = 3 x 256 + 32)
    (7, 32, 32, 4, 4),         # one block per row
    (3, 1024, 1536, 8, 8),     # six rounds, 8 wavefronts
    (2, 512, 2048, 8, 8),      # the longest rows (8 rounds)
    (20, 2048, 96, 4, 4),      # 20 slots per expert: units of 8, 8 and 4
    (40, 2048, 96, 16, 8),
    (64, 2048, 32, 128, 8),
    (7, 2048, 1536, 5, 5),     # k = E: every expert in every token
]


@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(dev, shape):
    B, H, I, E, k = shape
    D = DevLayer(mi.make_layer(800 + SMALL.index(shape), H, I, E), dev)
    x = mi.make_x(81, B, H)
    ids, w = mi.route_uniform(81 + B, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev, variant=DMFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"down mfma {shape}", own=(D, ids, w))


def _random_case(i):
    g = np.random.default_rng(9900 + i)
    k = int(g.integers(1, 9))
    E = int(g.integers(k, 41))
    B = int(g.integers(1, 97))
    H = 32 * int(g.integers(1, 97))
    I = 32 * int(g.integers(1, 65))     # up to 2048 (k * I <= 16384, B * k <= 768)
    return B, H, I, E, k, bool(g.integers(0, 2))


@pytest.mark.parametrize("i", range(16))
def test_random_shapes(dev, i):
    B, H, I, E, k, skew = _random_case(i)
    D = DevLayer(mi.make_layer(9950 + i, H, I, E), dev)
    x = mi.make_x(9970 + i, B, H)
    ids, w = (mi.route_zipf if skew else mi.route_uniform)(9990 + i, B, E, k)
    h, y = run_gpu(D, x, ids, w, dev, variant=DMFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, f"down mfma random {i}: B={B} H={H} I={I} E={E} k={k} skew={skew}",
          own=(D, ids, w))


def test_duplicates_and_one_expert_over_several_units(dev):
    """Token 0 lists one expert three times, every token routes slot 0 to expert
    3 (40 slots: units of 8 on different wavefronts); twice, bit-identical."""
    B, H, I, E, k = 40, 2048, 96, 16, 8
    D = DevLayer(mi.make_layer(850, H, I, E), dev)
    x = mi.make_x(851, B, H)
    ids, w = mi.route_uniform(852, B, E, k)
    for b in range(B):
        row = [e for e in ids[b] if e != 3][: k - 1]
        ids[b] = [3] + row + [e for e in range(E) if e != 3 and e not in row][: k - 1 - len(row)]
    ids[0, 1] = ids[0, 2] = ids[0, 0]
    h, y = run_gpu(D, x, ids, w, dev, variant=DMFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *D.host())
    check(h, y, h_ref, y_ref, B, k, "down mfma duplicates", own=(D, ids, w))
    h2, y2 = run_gpu(D, x, ids, w, dev, variant=DMFMA)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)


@pytest.fixture(scope="module")
def s1(dev):
    s = mi.SHAPES["S1"]
    return DevLayer(mi.make_layer(mi.layer_seed("single_b1"), s["H"], s["I"], s["E"]), dev)


@pytest.mark.parametrize("B,routing", [(1, "uniform"), (8, "uniform"), (16, "uniform"), (32, "uniform"),
                                       (32, "zipf"), (32, "adversarial"), (32, "contiguous"), (64, "uniform"),
                                       (64, "zipf")])
def test_s1_workload(dev, s1, B, routing):
    seed = mi.routing_seed("routing_stress" if routing != "uniform" else "batch_sweep", B, routing)
    x = mi.make_x(seed, B, s1.H)
    ids, w = mi.make_routing(routing, seed, B, s1.E, 8)
    h, y = run_gpu(s1, x, ids, w, dev, variant=DMFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    check(h, y, h_ref, y_ref, B, 8, f"down mfma S1 B={B} {routing}", own=(s1, ids, w))
    h2, y2 = run_gpu(s1, x, ids, w, dev, variant=DMFMA)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)


@pytest.mark.parametrize("B", [1, 16, 32, 64])
def test_wide_layer(dev, s2, B):
    x, ids, w, h_ref, y_ref = wide_case(s2, B)
    h, y = run_gpu(s2, x, ids, w, dev, variant=DMFMA)
    check(h, y, h_ref, y_ref, B, 8, f"down mfma wide B={B}", own=(s2, ids, w))


def test_many_experts(dev):
    """1024 slots over 1024 experts (the slot index's limits)."""
    B, H, I, E, k = 128, 64, 256, 1024, 8
    g = np.random.default_rng(860)
    wd = g.integers(0, 0x7E, (E, H, I), dtype=np.uint8) | (g.integers(0, 2, (E, H, I), dtype=np.uint8) << 7)
    sd = g.integers(110, 125, (E, H, I // 32), dtype=np.uint8)
    h = mi.make_x(861, B * k, I).reshape(B, k, I)
    ids, w = mi.route_uniform(862, B, E, k)
    got = down_only(dev, h, ids, w, wd, sd)
    ref = oracle.down(h, ids, w, wd, sd)
    p = parity(got, ref, B)
    assert passes(p) and _few_flips(p), p


def test_out_of_range_ids_give_nan(dev, s1):
    B, k = 40, 8
    x = mi.make_x(88, B, s1.H)
    ids, w = mi.route_uniform(88, B, s1.E, k)
    bad = ids.copy()
    bad[1, 3] = -1
    bad[2, 0] = s1.E
    h, y = run_gpu(s1, x, bad, w, dev, variant=DMFMA)
    h_ref, y_ref = oracle.layer(x, ids, w, *s1.host())
    yv = oracle.bf16_to_f64(y)
    assert np.all(np.isnan(yv[1])) and np.all(np.isnan(yv[2]))
    keep = [b for b in range(B) if b not in (1, 2)]
    assert passes(parity(y[keep], y_ref[keep], len(keep)))


def test_empty_batch(dev, s1):
    h = torch.empty((0, 8, s1.I), dtype=torch.int16, device=dev)
    ids = torch.empty((0, 8), dtype=torch.int32, device=dev)
    w = torch.empty((0, 8), dtype=torch.float32, device=dev)
    y = torch.empty((0, s1.H), dtype=torch.int16, device=dev)
    mg.moe_decode_down(h, ids, w, s1.wd, s1.sd, y, variant=mg.MOE_DOWN_EXPERT_GROUPED_MFMA)
    torch.cuda.synchronize()
