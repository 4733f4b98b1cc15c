"""The oracle's pins must catch plausible mistakes (CPU only).

Each case copies the oracle's C source, plants one mistake in the copy (a
dropped sign, a wrong exponent bias or index, swapped operands, a wrong
rounding rule, a dropped router weight, a wrong tie rule in the router, a
dropped quantisation step or a wrong MX rule in the conventional emulation ...),
builds it into a temporary library, and runs the pin tests against it.  At least one pin has to fail for
every planted mistake; the unmodified oracle passes all of them (the other test
modules).  The planted mistakes only ever live in a temporary copy.
"""
import contextlib
import os

import pytest

import oracle
from tests import test_oracle_formats as F
from tests import test_oracle_layer as L
from tests import test_oracle_router as RT

MUTATIONS = [
    ("e4m3 sign dropped", "return s ? -mag : mag;", "return mag;"),
    ("e4m3 exponent bias", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    ("e4m3 subnormal scale", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("e4m3 mantissa width", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(16 + m), e - 11)"),
    ("e8m0 bias", "ldexp(1.0, (int)v - 127)", "ldexp(1.0, (int)v - 128)"),
    ("scale block order", "c / ORC_BLOCK]", "(C / ORC_BLOCK - 1 - c / ORC_BLOCK)]"),
    ("gate/up rows swapped", "u += weight_at(wu, su, I, H, e, n, c) * xv;", "u += weight_at(wg, sg, I, H, e, n, c) * xv;"),
    ("x token index", "orc_bf16_value(x[b * H + c])", "orc_bf16_value(x[c])"),
    ("expert slot index", "long e = ids[b * k + j], c;", "long e = ids[b * k], c;"),
    ("silu sign", "return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    ("silu replaced by sigmoid", "return g / (1.0 + exp(-g));", "return 1.0 / (1.0 + exp(-g));"),
    ("router weight dropped", "y += (double)tw[b * k + j] * dot;", "y += dot;"),
    ("h slot index", "orc_bf16_value(h[(b * k + j) * I + i])", "orc_bf16_value(h[(b * k) * I + i])"),
    ("down row transposed index", "weight_at(wd, sd, H, I, e, o, i)", "weight_at(wd, sd, H, I, e, (o + 1) % H, i)"),
    ("bf16 ties away from zero", "r = nearbyint(a / spacing) * spacing;", "r = round(a / spacing) * spacing;"),
    ("bf16 truncation", "r = nearbyint(a / spacing) * spacing;", "r = floor(a / spacing) * spacing;"),
    ("bf16 via fp32 (double rounding)", "r = nearbyint(a / spacing) * spacing;",
     "r = nearbyint((double)(float)a / spacing) * spacing;"),
    ("bf16 significand width", "spacing = ldexp(1.0, ex - 1 - 7);", "spacing = ldexp(1.0, ex - 1 - 8);"),
    ("router ties to the higher id", "(double)l[i] > (double)l[best]", "(double)l[i] >= (double)l[best]"),
    ("router keeps the smallest logits", "(double)l[i] > (double)l[best]", "(double)l[i] < (double)l[best]"),
    ("router weights not renormalised", "- m) / z / s;", "- m) / z;"),
    ("router weight of the wrong slot", "w_out[b * k + j] = exp((double)l[ids_out[b * k + j]] - m)",
     "w_out[b * k + j] = exp((double)l[ids_out[b * k]] - m)"),
    # the emulated conventional path
    ("mx shared exponent", "X = ldexp(1.0, ex - 1 - 8);", "X = ldexp(1.0, ex - 1 - 7);"),
    ("mx saturation dropped", "if (a > 448.0)\n                a = 448.0;", "if (a > 448.0)\n                a = a;"),
    ("mx ties away from zero", "    return nearbyint(a / spacing) * spacing;", "    return round(a / spacing) * spacing;"),
    ("mx subnormal spacing", "        spacing = ldexp(1.0, -9);", "        spacing = ldexp(1.0, -10);"),
    ("mx significand width", "spacing = ldexp(1.0, ex - 1 - 3);", "spacing = ldexp(1.0, ex - 1 - 4);"),
    ("conventional x not quantised", "        orc_mx_fake_quant(xq, H);", "        (void)0;"),
    ("conventional h not quantised", "            orc_mx_fake_quant(hq, I);", "            (void)0;"),
    ("per-expert buffer not rounded", "acc[o] += (double)tw[b * k + j] * orc_bf16_value(orc_bf16_rne(d));",
     "acc[o] += (double)tw[b * k + j] * d;"),
    ("combine weight of the wrong slot", "acc[o] += (double)tw[b * k + j] * orc_bf16_value(orc_bf16_rne(d));",
     "acc[o] += (double)tw[b * k] * orc_bf16_value(orc_bf16_rne(d));"),
    ("conventional x of the wrong token", "xq[c] = orc_bf16_value(x[b * H + c]);", "xq[c] = orc_bf16_value(x[c]);"),
]

PINS = [
    ("e4m3 vs torch", lambda o: F.test_e4m3_all_codes_match_torch(o)),
    ("e4m3 landmarks", lambda o: F.test_e4m3_landmarks(o)),
    ("e8m0", lambda o: F.test_e8m0_all_codes(o)),
    ("bf16 vs torch", lambda o: F.test_bf16_matches_torch_on_fp32_inputs(o)),
    ("bf16 exact", lambda o: F.test_bf16_exact_cases(o)),
    ("silu", lambda o: F.test_silu_closed_form(o)),
    ("brute force", lambda o: L.test_brute_force_equality(o, 2, 64, 32, 4, 2, 2)),
    ("dense k=1", lambda o: L.test_k1_is_dense_swiglu_ffn(o)),
    ("permutation", lambda o: L.test_permutation_invariance(o)),
    ("linearity", lambda o: L.test_router_weight_linearity_and_special_cases(o)),
    ("router ranks", lambda o: RT.test_route_matches_rank_definition(o, 12, 5)),
    ("router k=2", lambda o: RT.test_route_k2_is_logistic_of_the_gap(o)),
    ("mx vs torch", lambda o: F.test_mx_fake_quant_matches_torch_e4m3(o)),
    ("conventional composition", lambda o: L.test_conventional_is_the_composition_of_its_stages(o, 3)),
]


@contextlib.contextmanager
def _oracle_lib(lib):
    old = oracle._lib
    oracle._lib = lib
    try:
        yield
    finally:
        oracle._lib = old


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    path = tmp_path / "moe_oracle_mut.c"
    path.write_text(mutated)
    so = str(tmp_path / f"libmut_{abs(hash(name))}.so")
    oracle.build(so, str(path))
    lib = oracle._bind(__import__("ctypes").CDLL(so))
    failed = []
    with _oracle_lib(lib):
        for pin_name, pin in PINS:
            try:
                pin(oracle)
            except (AssertionError, oracle.OracleError):
                failed.append(pin_name)
                break
    assert failed, f"no pin caught the planted mistake '{name}'"
