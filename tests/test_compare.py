"""The parity checker every GPU test relies on (oracle/compare.py), checked on
the CPU against planted differences: if it were lenient, the GPU parity tests
would pass vacuously.  The bar: |got - ref| <= 2e-3 + 1e-2 |ref| per element,
cosine >= 0.999995 per row, no NaN."""
import numpy as np

from oracle.compare import ATOL, MIN_COS, RTOL, bf16_to_f64, parity, passes


def _bits(v):
    """bf16 bits of float64 values (truncating float32 bits: exact for the values used here)."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _ref(rows=4, n=64, seed=0):
    rng = np.random.default_rng(seed)
    return _bits(rng.standard_normal((rows, n)))


def test_identical_passes_exactly():
    r = _ref()
    p = parity(r, r, 4)
    assert passes(p) and p["n_diff"] == 0 and p["max_abs"] == 0.0 and p["min_cos"] == 1.0


def test_element_bound_edges():
    r = np.full((2, 32), _bits(0.5)[()], np.uint16)            # ref = 0.5: bound 2e-3 + 5e-3 = 7e-3
    g = r.copy()
    g[1, 3] = _bits(0.5 + 0.0078125)[()]                        # +2^-7 > 7e-3: outside
    p = parity(g, r, 2)
    assert p["worst_ratio"] > 1.0 and not passes(p)
    g[1, 3] = _bits(0.5 + 0.00390625)[()]                       # +2^-8 < 7e-3: inside (one bf16 step at 0.5)
    p = parity(g, r, 2)
    assert p["worst_ratio"] <= 1.0 and p["n_diff"] == 1
    assert abs(p["worst_ratio"] - 0.00390625 / (ATOL + RTOL * 0.5)) < 1e-12


def test_cosine_catches_what_the_element_bound_allows():
    """Errors of one sign on a row of tiny values of both signs stay inside the
    absolute term of the element bound but turn the row (cosine ~0.55): the
    cosine must fail.  A sign flip of one row is caught too."""
    n = 64
    ref = np.tile([1e-3, -1e-3], (1, n // 2))
    got = ref + 1.5e-3                                          # each |diff| ~1.5e-3 < 2e-3 + 1e-5
    p = parity(_bits(got), _bits(ref), 1)
    assert p["worst_ratio"] <= 1.0
    assert p["min_cos"] < 0.6 and not passes(p)
    r = _ref(3)
    g = r.copy()
    g[2] ^= np.uint16(0x8000)
    p = parity(g, r, 3)
    assert p["min_cos"] < 0 and not passes(p)


def test_nan_anywhere_fails():
    r = _ref()
    g = r.copy()
    g[0, 5] = 0x7FC0
    assert not passes(parity(g, r, 4))
    assert not passes(parity(g, g, 4))                          # NaN on both sides is handled by the callers
    assert parity(g, r, 4)["nan_got"] == 1 and parity(g, r, 4)["nan_ref"] == 0


def test_zero_rows():
    z = np.zeros((2, 16), np.uint16)
    assert parity(z, z, 2)["min_cos"] == 1.0
    r = z.copy()
    r[1, 0] = _bits(1.0)[()]
    p = parity(z, r, 2)
    assert p["min_cos"] == 0.0 and not passes(p)


def test_rows_are_taken_as_given():
    r = _ref(4, 64)
    g = r.copy()
    g[3] = _ref(1, 64, seed=9)[0]                               # one unrelated row
    p = parity(g, r, 4)
    assert p["min_cos"] < 0.5 and not passes(p)
    assert parity(g.reshape(-1), r.reshape(-1), 4) == p          # flat input, same rows


def test_bf16_decoding():
    assert bf16_to_f64(np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80], np.uint16)).tolist() == [1.0, -1.0, 0.0, -0.0, np.inf]
