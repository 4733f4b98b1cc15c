"""Pins for the oracle's layer arithmetic (CPU only).

Each check fixes the oracle against something other than itself:
  * exact brute force (pure Python, rationals) on tiny shapes;
  * k=1 with router weight 1 reduces to a dense SwiGLU FFN of one expert,
    computed here with NumPy FP64 matrix products on weights decoded through
    PyTorch's float8 dtypes;
  * the combine is a sum over slots (permutation invariance) that is linear in
    the router weights, with w=0 giving +0 and one-hot w giving that expert;
  * magnitudes match a closed form (E[SiLU(g)^2] for g ~ N(0,1));
  * the emulated conventional path, which quantises activations to MXFP8, is
    further from the full-precision layer than the warp-decode arithmetic
    (direction of the accuracy claim in the blog post's "Accuracy improvement").
"""
import math

import numpy as np
import pytest
import torch
from scipy import integrate

import moe_inputs as mi
from oracle import brute


def _deq(q, s):
    """Dequantise with PyTorch float8 views (independent of the oracle's decoder)."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return v * np.repeat(sc, 32, axis=-1)


def _bf16_vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _is_nearest_bf16(bits, ref):
    """True where bf16 `bits` is a nearest bf16 value to the float64 `ref`
    (checked against both bf16 neighbours; ties accept either)."""
    bits = np.asarray(bits, np.uint16).astype(np.int64)
    v = _bf16_vals(bits)
    up = _bf16_vals(np.where(ref >= 0, bits + 1, bits - 1) & 0xFFFF)
    dn = _bf16_vals(np.where(ref >= 0, bits - 1, bits + 1) & 0xFFFF)
    d = np.abs(v - ref)
    return (d <= np.abs(up - ref)) & (d <= np.abs(dn - ref))


def _small(seed, B, H, I, E, k):
    L = mi.make_layer(seed, H, I, E, threads=1)
    x = mi.make_x(seed, B, H)
    ids, w = mi.route_uniform(seed, B, E, k)
    return L, x, ids, w


@pytest.mark.parametrize("B,H,I,E,k,seed", [(1, 64, 32, 4, 2, 1), (2, 64, 32, 4, 2, 2), (3, 64, 32, 4, 2, 3),
                                            (2, 32, 32, 4, 2, 4), (2, 96, 64, 6, 3, 5)])
def test_brute_force_equality(orc, B, H, I, E, k, seed):
    L, x, ids, w = _small(seed, B, H, I, E, k)
    h, y = orc.layer(x, ids, w, L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    hb, ht = brute.gate_up(x.ravel(), ids.ravel(), L.w_gate.ravel(), L.s_gate.ravel(),
                           L.w_up.ravel(), L.s_up.ravel(), B, H, I, k)
    hb, ht = np.array(hb, np.uint16), np.array(ht)
    assert np.all((hb == h.ravel()) | ht), np.nonzero((hb != h.ravel()) & ~ht)
    assert ht.sum() <= 1
    # down from the oracle's h so both sides see the same intermediate
    yb, yt = brute.down(h.ravel(), ids.ravel(), w.ravel(), L.w_down.ravel(), L.s_down.ravel(), B, H, I, k)
    yb, yt = np.array(yb, np.uint16), np.array(yt)
    assert np.all((yb == y.ravel()) | yt)
    assert yt.sum() <= 1


def test_k1_is_dense_swiglu_ffn(orc):
    B, H, I, E = 4, 256, 128, 3
    L = mi.make_layer(11, H, I, E, threads=1)
    x = mi.make_x(11, B, H)
    xv = _bf16_vals(x)
    Wg, Wu, Wd = _deq(L.w_gate, L.s_gate), _deq(L.w_up, L.s_up), _deq(L.w_down, L.s_down)
    for e in range(E):
        ids = np.full((B, 1), e, np.int32)
        w = np.ones((B, 1), np.float32)
        h, y = orc.layer(x, ids, w, L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
        g = xv @ Wg[e].T
        u = xv @ Wu[e].T
        pre_h = g / (1 + np.exp(-g)) * u
        assert _is_nearest_bf16(h[:, 0, :], pre_h).all()
        pre_y = _bf16_vals(h[:, 0, :]) @ Wd[e].T
        assert _is_nearest_bf16(y, pre_y).all()


def test_permutation_invariance(orc):
    B, H, I, E, k = 4, 128, 64, 16, 8
    L, x, ids, w = _small(21, B, H, I, E, k)
    args = (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    h, y = orc.layer(x, ids, w, *args)
    rng = np.random.default_rng(0)
    for _ in range(3):
        perm = np.stack([rng.permutation(k) for _ in range(B)])
        ids_p = np.take_along_axis(ids, perm, 1)
        w_p = np.take_along_axis(w, perm, 1)
        h_p, y_p = orc.layer(x, ids_p, w_p, *args)
        assert np.array_equal(h_p, np.take_along_axis(h, perm[:, :, None], 1))
        assert np.array_equal(y_p, y)


def test_router_weight_linearity_and_special_cases(orc):
    B, H, I, E, k = 3, 128, 64, 8, 4
    L, x, ids, w = _small(31, B, H, I, E, k)
    h = orc.gate_up(x, ids, L.w_gate, L.s_gate, L.w_up, L.s_up)
    rng = np.random.default_rng(1)
    w2 = rng.random((B, k)).astype(np.float32)
    a, b = 0.75, -1.25   # exact in binary; a*w + b*w2 is rounded to fp32, so compare with the rounded weights
    wc = (a * w.astype(np.float64) + b * w2.astype(np.float64)).astype(np.float32)
    _, Y1 = orc.down(h, ids, w, L.w_down, L.s_down, fp64=True)
    _, Y2 = orc.down(h, ids, w2, L.w_down, L.s_down, fp64=True)
    _, Yc = orc.down(h, ids, wc, L.w_down, L.s_down, fp64=True)
    # per-slot contributions are linear: recompute the combination from one-hot weights
    Ys = []
    for j in range(k):
        oh = np.zeros((B, k), np.float32); oh[:, j] = 1.0
        Ys.append(orc.down(h, ids, oh, L.w_down, L.s_down, fp64=True)[1])
    Ys = np.stack(Ys, 1)   # [B, k, H]
    for wv, Yv in ((w, Y1), (w2, Y2), (wc, Yc)):
        rebuilt = np.einsum("bk,bkh->bh", wv.astype(np.float64), Ys)
        assert np.allclose(Yv, rebuilt, rtol=1e-12, atol=1e-15)
    # Y(a*w + b*w2) = a*Y(w) + b*Y(w2), up to the fp32 rounding of the combined weights
    bound = 2.0 ** -23 * np.einsum("bk,bkh->bh", np.abs(wc.astype(np.float64)), np.abs(Ys)) + 1e-15
    assert np.all(np.abs(a * Y1 + b * Y2 - Yc) <= bound)
    # zero weights -> +0 exactly
    y0 = orc.down(h, ids, np.zeros((B, k), np.float32), L.w_down, L.s_down)
    assert np.all(y0 == 0)
    # one-hot weight on slot j == dense FFN of expert ids[:, j]
    for j in range(k):
        oh = np.zeros((B, k), np.float32); oh[:, j] = 1.0
        y_oh = orc.down(h, ids, oh, L.w_down, L.s_down)
        for bb in range(B):
            hs, ys = orc.layer(x[bb:bb + 1], ids[bb:bb + 1, j:j + 1], np.ones((1, 1), np.float32),
                               L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
            assert np.array_equal(hs[0, 0], h[bb, j])
            assert np.array_equal(ys[0], y_oh[bb])


def test_magnitudes_match_closed_form(orc):
    # g, u ~ N(0, 1) independent (x ~ N(0,1), rows ~ N(0, 1/H)) => E[h^2] = E[SiLU(g)^2]
    pdf = lambda t: math.exp(-t * t / 2) / math.sqrt(2 * math.pi)
    e_silu2, _ = integrate.quad(lambda t: (t / (1 + math.exp(-t))) ** 2 * pdf(t), -40, 40)
    assert e_silu2 == pytest.approx(0.3558, abs=2e-4)
    B, H, I, E, k = 16, 2048, 1024, 16, 8
    L, x, ids, w = _small(41, B, H, I, E, k)
    h = orc.gate_up(x, ids, L.w_gate, L.s_gate, L.w_up, L.s_up)
    hv = _bf16_vals(h)
    # 131072 samples of a heavy-tailed h^2: the sample mean's relative std is about 1.2%
    assert np.mean(hv ** 2) == pytest.approx(e_silu2, rel=0.06)
    y = orc.down(h, ids, w, L.w_down, L.s_down)
    # E[y^2] = E[sum_j w_j^2] * E[h^2] for independent rows of variance 1/I
    ew2 = np.mean(np.sum(w.astype(np.float64) ** 2, axis=1))
    assert np.mean(_bf16_vals(y) ** 2) == pytest.approx(ew2 * e_silu2, rel=0.15)


@pytest.mark.parametrize("B", [1, 4])
def test_conventional_path_is_less_accurate(orc, B):
    """Warp decode keeps activations bf16 and accumulators wide; the conventional path
    quantises them to MXFP8.  Against the unquantised full-precision layer the
    conventional output must be further away (blog post, "Accuracy improvement")."""
    H, I, E, k = 2048, 768, 16, 8
    L = mi.make_layer(0, H, I, E, keep_fp32=True)
    x = mi.make_x(0, B, H)
    ids, w = mi.route_uniform(0, B, E, k)
    args = (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    _, y_wd = orc.layer(x, ids, w, *args)
    y_cv = orc.conventional(x, ids, w, *args)
    T = orc.truth_layer(x, ids, w, L.f_gate, L.f_up, L.f_down)
    err = lambda y: np.linalg.norm(_bf16_vals(y) - T) / np.linalg.norm(T)
    e_wd, e_cv = err(y_wd), err(y_cv)
    assert e_cv > e_wd, (e_cv, e_wd)
    # the predicted ratio for quantising both GEMM inputs is about sqrt(2); only the direction is pinned
    assert 1.0 < e_cv / e_wd < 4.0


def _exact_bf16_bits(v):
    """bf16 bit patterns of float64 values that are bf16 values (checked)."""
    f = np.asarray(v, np.float64).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_bf16_vals(bits), np.asarray(v, np.float64)), "not bf16-representable"
    return bits


@pytest.mark.parametrize("k", [1, 3])
def test_conventional_is_the_composition_of_its_stages(orc, k):
    """The emulated conventional path equals its stages put together from the
    oracle's other functions (blog post, "The traditional MoE path" and
    "Accuracy improvement"): x quantised to MXFP8, the warp-decode gate/up on
    it, the intermediate quantised to MXFP8, each routed expert's down output
    rounded to bf16 on its own (the per-expert buffer), and the router-weighted
    combine rounded to bf16 once."""
    B, H, I, E = 4, 96, 64, 5
    L = mi.make_layer(31, H, I, E)
    x = mi.make_x(32, B, H)
    ids, w = mi.route_uniform(33, B, E, k)
    args = (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    y_cv = orc.conventional(x, ids, w, *args)
    xq = _exact_bf16_bits(orc.mx_fake_quant(_bf16_vals(x)))
    h = orc.gate_up(xq, ids, L.w_gate, L.s_gate, L.w_up, L.s_up)
    hq = _exact_bf16_bits(orc.mx_fake_quant(_bf16_vals(h)))
    per_expert = np.stack([_bf16_vals(orc.down(hq[:, j:j + 1], ids[:, j:j + 1], np.ones((B, 1), np.float32),
                                               L.w_down, L.s_down)) for j in range(k)], axis=1)   # [B, k, H]
    combine = np.zeros((B, H))
    for j in range(k):
        combine += w[:, j:j + 1].astype(np.float64) * per_expert[:, j]
    y_ref = np.array([[orc.bf16_rne(v) for v in row] for row in combine], np.uint16)
    assert np.array_equal(y_cv, y_ref), np.nonzero(y_cv != y_ref)
    # and quantisation did something: without it the warp-decode layer differs
    assert not np.array_equal(y_cv, orc.layer(x, ids, w, *args)[1])


def test_truth_layer_special_cases_and_invariants(orc):
    """The full-precision reference of the accuracy A/B (blog post, "Accuracy
    improvement"): with one routed expert of weight 1 it is PyTorch's own dense
    SwiGLU FFN (F.linear and F.silu in float64) on the unquantised draws; it is
    linear in the router weights and does not depend on the slot order."""
    import torch.nn.functional as Fn
    B, H, I, E, k = 3, 96, 64, 4, 3
    L = mi.make_layer(41, H, I, E, keep_fp32=True)
    x = mi.make_x(42, B, H)
    xt = torch.from_numpy(_bf16_vals(x))
    for e in range(E):
        ids1 = np.full((B, 1), e, np.int32)
        T = orc.truth_layer(x, ids1, np.ones((B, 1), np.float32), L.f_gate, L.f_up, L.f_down)
        g = Fn.linear(xt, torch.from_numpy(L.f_gate[e].astype(np.float64)))
        u = Fn.linear(xt, torch.from_numpy(L.f_up[e].astype(np.float64)))
        ref = Fn.linear(Fn.silu(g) * u, torch.from_numpy(L.f_down[e].astype(np.float64))).numpy()
        assert np.allclose(T, ref, rtol=1e-12, atol=1e-14)
    ids, w = mi.route_uniform(43, B, E, k)
    T = orc.truth_layer(x, ids, w, L.f_gate, L.f_up, L.f_down)
    parts = [orc.truth_layer(x, ids[:, j:j + 1], np.ones((B, 1), np.float32), L.f_gate, L.f_up, L.f_down)
             for j in range(k)]
    assert np.allclose(T, sum(w[:, j:j + 1].astype(np.float64) * parts[j] for j in range(k)), rtol=1e-12, atol=1e-14)
    perm = np.array([2, 0, 1])
    Tp = orc.truth_layer(x, ids[:, perm], w[:, perm], L.f_gate, L.f_up, L.f_down)
    assert np.allclose(T, Tp, rtol=1e-12, atol=1e-14)
