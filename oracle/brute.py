"""Exact brute-force restatement of the layer for tiny shapes -- TEST INFRASTRUCTURE ONLY.

Pure Python, rational arithmetic (``fractions.Fraction``), written separately
from the C oracle to pin it: decoding works from the E4M3 bit fields as
fractions, dot products are exact, and bf16 rounding is done on the exact
rational value.  The only inexact step is SiLU's exponential, evaluated in
double; results whose exact value lies within ``TIE_REL`` of a bf16 rounding
boundary are reported as near ties so a caller can exempt them.

Layer definition: Cursor, "warp decode" blog post, "How the two kernels work"
(gate/up neuron = SiLU(gate . x) * (up . x); output = sum over the top-k
experts of router weight x down row . intermediate).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

TIE_REL = Fraction(1, 10**12)
_SILU_EPS = Fraction(1, 10**13)


def e4m3_exact(q: int) -> Fraction:
    """E4M3 code -> exact value.  Fields: sign | 4-bit exponent (bias 7) | 3-bit fraction.
    Exponent field 0 is subnormal (no implicit 1, exponent 1-7); S.1111.111 is NaN."""
    neg = bool(q & 0x80)
    ef, mf = (q >> 3) & 0xF, q & 0x7
    if ef == 0xF and mf == 0x7:
        raise ValueError("E4M3 NaN")
    lead = 0 if ef == 0 else 1
    exp = (1 if ef == 0 else ef) - 7
    val = (lead + Fraction(mf, 8)) * (Fraction(2) ** exp)
    return -val if neg else val


def e8m0_exact(v: int) -> Fraction:
    if v == 0xFF:
        raise ValueError("E8M0 NaN")
    return Fraction(2) ** (v - 127)


def bf16_bits_to_fraction(bits: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    return Fraction(f)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def bf16_round_exact(v: Fraction):
    """Exact rational -> (bf16 bits, near_tie).  Round to nearest, ties to even
    (Python's round() on a Fraction rounds half to even)."""
    if v == 0:
        return 0, False
    neg = v < 0
    a = -v if neg else v
    e = max(_floor_log2(a), -126)
    spacing = Fraction(2) ** (e - 7)
    scaled = a / spacing
    q = round(scaled)
    frac = scaled - math.floor(scaled)
    near_tie = abs(frac - Fraction(1, 2)) * spacing <= TIE_REL * a
    r = q * spacing
    if r >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = struct.unpack("<I", struct.pack("<f", float(r)))[0] >> 16
    return (bits | (0x8000 if neg else 0)), bool(near_tie)


def _row(codes, scales, row_index: int, C: int):
    base = row_index * C
    sbase = row_index * (C // 32)
    return [e4m3_exact(int(codes[base + c])) * e8m0_exact(int(scales[sbase + c // 32])) for c in range(C)]


def gate_up(x, ids, wg, sg, wu, su, B, H, I, k):
    """x: flat bf16 bits [B*H]; ids flat [B*k]; weights flat.  Returns (h bits, near-tie flags), flat [B*k*I]."""
    out, ties = [], []
    xs = [[bf16_bits_to_fraction(int(x[b * H + c])) for c in range(H)] for b in range(B)]
    for b in range(B):
        for j in range(k):
            e = int(ids[b * k + j])
            for n in range(I):
                g_row = _row(wg, sg, e * I + n, H)
                u_row = _row(wu, su, e * I + n, H)
                G = sum(w * xv for w, xv in zip(g_row, xs[b]))
                U = sum(w * xv for w, xv in zip(u_row, xs[b]))
                gf = float(G)
                silu = Fraction(gf / (1.0 + math.exp(-gf))) if gf > -700 else Fraction(0)
                v = silu * U
                bits, tie = bf16_round_exact(v)
                # SiLU in double carries ~1e-15 relative error: flag values whose
                # rounding would change under a 1e-13 relative perturbation.
                if v != 0:
                    lo = bf16_round_exact(v * (1 - _SILU_EPS))[0]
                    hi = bf16_round_exact(v * (1 + _SILU_EPS))[0]
                    tie = tie or lo != bits or hi != bits
                out.append(bits)
                ties.append(tie)
    return out, ties


def down(h, ids, w, wd, sd, B, H, I, k):
    """h: flat bf16 bits [B*k*I]; w: flat float32 router weights [B*k].  Returns (y bits, near-tie flags), flat [B*H]."""
    out, ties = [], []
    for b in range(B):
        hs = [[bf16_bits_to_fraction(int(h[(b * k + j) * I + i])) for i in range(I)] for j in range(k)]
        for o in range(H):
            Y = Fraction(0)
            for j in range(k):
                e = int(ids[b * k + j])
                d_row = _row(wd, sd, e * H + o, I)
                Y += Fraction(float(w[b * k + j])) * sum(wv * hv for wv, hv in zip(d_row, hs[j]))
            bits, tie = bf16_round_exact(Y)
            out.append(bits)
            ties.append(tie)
    return out, ties
