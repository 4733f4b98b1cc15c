"""Pins for the oracle's number formats (CPU only).

E4M3 and E8M0 decoding are checked against PyTorch's own float8_e4m3fn /
float8_e8m0fnu dtypes (a library routine, independent of the oracle's C
formula) and against landmark values fixed by the OCP 8-bit FP and MX
specifications.  bf16 rounding is checked against PyTorch's FP32->bf16
conversion on FP32-representable inputs and against hand-derived exact cases,
including one where rounding through FP32 first would give a different
answer.
"""
import math
import struct

import numpy as np
import pytest
import torch


def _torch_e4m3(q):
    return torch.tensor([q], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()


def _torch_e8m0(v):
    return torch.tensor([v], dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).item()


def _f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def test_e4m3_all_codes_match_torch(orc):
    for q in range(256):
        a, b = orc.e4m3(q), _torch_e4m3(q)
        if math.isnan(b):
            assert math.isnan(a), q
        else:
            assert a == b and math.copysign(1, a) == math.copysign(1, b), (q, a, b)


def test_e4m3_landmarks(orc):
    assert orc.e4m3(0x38) == 1.0          # exponent field 7 = bias
    assert orc.e4m3(0x7E) == 448.0        # largest finite
    assert orc.e4m3(0x01) == 2.0 ** -9    # smallest subnormal
    assert orc.e4m3(0x08) == 2.0 ** -6    # smallest normal
    assert orc.e4m3(0x07) == 7 * 2.0 ** -9
    assert orc.e4m3(0xB8) == -1.0
    z = orc.e4m3(0x80)
    assert z == 0.0 and math.copysign(1, z) < 0
    assert math.isnan(orc.e4m3(0x7F)) and math.isnan(orc.e4m3(0xFF))
    # no infinities: every non-NaN code is finite, and codes 0..0x7E increase strictly
    vals = [orc.e4m3(q) for q in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert all(orc.e4m3(q | 0x80) == -orc.e4m3(q) for q in range(0x7F))


def test_e8m0_all_codes(orc):
    for v in range(255):
        assert orc.e8m0(v) == _torch_e8m0(v) == 2.0 ** (v - 127), v
    assert math.isnan(orc.e8m0(255))
    assert orc.e8m0(0x7F) == 1.0 and orc.e8m0(0x80) == 2.0 and orc.e8m0(0) == 2.0 ** -127


def test_bf16_matches_torch_on_fp32_inputs(orc):
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around random significands, subnormals and the overflow edge
    base = rng.integers(0, 2 ** 31, size=2000, dtype=np.uint64).astype(np.uint32) & np.uint32(0xFFFF0000)
    extra = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base | 0x18000,
                            np.array([0x00000001, 0x00008000, 0x00018000, 0x7F7F7FFF, 0x7F7F8000,
                                      0x7F7FFFFF, 0x80000000, 0x7F800000, 0xFF800000], np.uint32)])
    allb = np.concatenate([bits, extra.astype(np.uint32)])
    f = allb.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([orc.bf16_rne(float(v)) for v in f], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(_f32_bits(f[i])), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_exact_cases(orc):
    one = 0x3F80
    assert orc.bf16_rne(1.0 + 2 ** -8) == one                 # tie -> even (mantissa 0)
    assert orc.bf16_rne(1.0 + 3 * 2 ** -8) == one + 2          # tie -> even (mantissa 2)
    assert orc.bf16_rne(1.0 + 2 ** -8 + 2 ** -40) == one + 1   # above the tie: FP32 would drop 2^-40
    assert orc.bf16_rne(1.0 + 2 ** -8 - 2 ** -40) == one
    assert orc.bf16_rne(-(1.0 + 2 ** -8 + 2 ** -40)) == 0x8000 | (one + 1)
    big = (2 - 2 ** -7) * 2.0 ** 127                            # largest finite bf16
    assert orc.bf16_rne(big) == 0x7F7F
    assert orc.bf16_rne((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80   # tie to the even neighbour 2^128 = inf
    assert orc.bf16_rne((2 - 2 ** -8) * 2.0 ** 127 * (1 - 2 ** -30)) == 0x7F7F
    assert orc.bf16_rne(2.0 ** -133) == 0x0001                  # smallest subnormal
    assert orc.bf16_rne(2.0 ** -134) == 0x0000                  # tie between 0 and 2^-133 -> 0
    assert orc.bf16_rne(1.5 * 2.0 ** -134) == 0x0001
    assert orc.bf16_rne(2.0 ** -134 + 2.0 ** -160) == 0x0001    # below FP32's subnormal range
    assert orc.bf16_rne(float("nan")) == 0x7FC0
    assert orc.bf16_rne(float("inf")) == 0x7F80
    assert orc.bf16_rne(-0.0) == 0x8000
    for bits in (0x3F80, 0x0001, 0x7F7F, 0xBEEF, 0x0080):
        assert orc.bf16_rne(orc.bf16_value(bits)) == bits


def test_silu_closed_form(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # silu(g) - silu(-g) = g
    for g in (0.1, 0.7, 3.0, 12.0):
        assert orc.silu(g) - orc.silu(-g) == pytest.approx(g, rel=1e-14)


def test_mx_fake_quant_properties(orc):
    rng = np.random.default_rng(5)
    v = rng.standard_normal(32 * 64) * np.exp2(rng.integers(-20, 20, 64)).repeat(32)
    q = orc.mx_fake_quant(v)
    blocks = v.reshape(-1, 32)
    qb = q.reshape(-1, 32)
    for b, bq in zip(blocks, qb):
        amax = np.abs(b).max()
        X = 2.0 ** (math.floor(math.log2(amax)) - 8)
        codes = bq / X
        # every element is an E4M3 value times the shared scale, and |error| <= half a spacing
        grid = np.array([_torch_e4m3(c) for c in range(0x7F)])
        assert np.all(np.isin(np.abs(codes), grid))
        a = np.abs(b) / X
        sat = a > 448
        assert np.all(np.abs(codes[sat]) == 448)
        a, c = a[~sat], np.abs(codes[~sat])
        spacing = np.where(a >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2 ** -6))) - 3), 2.0 ** -9)
        assert np.all(np.abs(c - a) <= spacing / 2)
    # idempotent
    assert np.array_equal(orc.mx_fake_quant(q), q)


def _torch_mx(v32):
    """MX fake quantisation of float32 values in blocks of 32 through PyTorch's own
    float8_e4m3fn conversion (round to nearest even): shared scale 2^(floor(log2
    amax) - 8) per block (OCP MX v1.0 with E4M3's largest exponent, 8), elements
    saturated to +-448 (torch itself does not saturate)."""
    out = np.zeros(v32.shape, np.float64)
    for i, blk in enumerate(v32.reshape(-1, 32)):
        amax = float(np.abs(blk).max())
        if amax == 0.0:
            continue
        X = 2.0 ** (math.floor(math.log2(amax)) - 8)
        a = torch.from_numpy((blk.astype(np.float64) / X).astype(np.float32))   # exact: X is a power of two
        a = a.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        out.reshape(-1, 32)[i] = a * X
    return out


def test_mx_fake_quant_matches_torch_e4m3(orc):
    """The oracle's MX quantise-dequantise of activations equals PyTorch's
    float8_e4m3fn rounding under the block's shared scale, on random float32
    blocks over a wide range of magnitudes and on blocks built from exact ties
    (halfway between two E4M3 values, normal and subnormal) and saturating
    values."""
    rng = np.random.default_rng(17)
    v = (rng.standard_normal(32 * 256) * np.exp2(rng.integers(-30, 30, 256)).repeat(32)).astype(np.float32)
    # a block with every element's magnitude tiny against the block max: E4M3 subnormals
    v[:32] = (rng.standard_normal(32) * 2.0 ** -14).astype(np.float32)
    v[0] = 300.0
    ties = np.array([300.0, 17.0, 19.0, -17.0, 25.0, 27.0, 3.0 * 2 ** -10, 5.0 * 2 ** -10, 7.0 * 2 ** -10,
                     -3.0 * 2 ** -10, 1.0625, 1.1875, 0.0, 2.0 ** -12, 460.0 / 512.0 * 256.0] + [1.0] * 17, np.float32)
    sat = np.array([500.0, -510.0, 449.0, 300.0] + [2.0] * 28, np.float32)   # block max 510: X = 1, 449..510 saturate
    v = np.concatenate([v, ties, sat])
    got = orc.mx_fake_quant(v.astype(np.float64))
    ref = _torch_mx(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), float(got[i]), float(ref[i])) for i in bad[:8]]
