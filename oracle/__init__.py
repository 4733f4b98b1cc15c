"""CPU oracle for the output-centric MoE decode layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library and never imports it.

* ``moe_oracle.c`` (built into ``libmoe_oracle.so`` with gcc + OpenMP) is the
  plain FP64 definition of the layer; this module wraps it with ctypes.
* ``brute.py`` is an independent pure-Python restatement with exact rational
  arithmetic, used to pin the C code on tiny shapes.
* ``route`` is the top-k router step in front of the layer (``orc_route`` in
  the C code), kept to check the router prologue of the HIP library.
* ``truth_layer`` evaluates the layer with the *unquantised* FP32 weight draws
  and no rounding anywhere (the "full precision" reference of the accuracy
  claim), with NumPy matrix products in FP64.

Citations are to Cursor's "warp decode" blog post; see the header of
``moe_oracle.c`` for the passage each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None


def build(out: str = _LIB, src: str = _SRC, extra=()) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-Wno-unused-parameter", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    i, L = ctypes.c_int, ctypes.c_long
    lib.orc_e4m3.argtypes = [ctypes.c_uint8]; lib.orc_e4m3.restype = ctypes.c_double
    lib.orc_e8m0.argtypes = [ctypes.c_uint8]; lib.orc_e8m0.restype = ctypes.c_double
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]; lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_bf16_rne.argtypes = [ctypes.c_double]; lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_silu.argtypes = [ctypes.c_double]; lib.orc_silu.restype = ctypes.c_double
    lib.orc_set_threads.argtypes = [i]; lib.orc_set_threads.restype = i
    lib.orc_gate_up.argtypes = [P, P, P, P, P, P, P, P, P, P, i, i, i, i, i]; lib.orc_gate_up.restype = i
    lib.orc_down.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i]; lib.orc_down.restype = i
    lib.orc_conventional.argtypes = [P, P, P, P, P, P, P, P, P, P, P, i, i, i, i, i]; lib.orc_conventional.restype = i
    lib.orc_mx_fake_quant.argtypes = [P, L]; lib.orc_mx_fake_quant.restype = None
    lib.orc_route.argtypes = [P, P, P, i, i, i]; lib.orc_route.restype = i
    return lib


def load(path: str = _LIB):
    """Load (building first if absent) the C oracle."""
    global _lib
    with _lock:
        if path == _LIB and _lib is not None:
            return _lib
        if not os.path.exists(path):
            build(path)
        lib = _bind(ctypes.CDLL(path))
        if path == _LIB:
            _lib = lib
        return lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError({-1: "null pointer", -2: "bad shape", -3: "expert id out of range"}.get(rc, rc))


# ---------------------------------------------------------------- scalars
def e4m3(q: int) -> float:
    return load().orc_e4m3(q)


def e8m0(v: int) -> float:
    return load().orc_e8m0(v)


def bf16_rne(v: float) -> int:
    return load().orc_bf16_rne(v)


def bf16_value(b: int) -> float:
    return load().orc_bf16_value(b)


def silu(g: float) -> float:
    return load().orc_silu(g)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (0 = leave as is); returns the count in use."""
    return load().orc_set_threads(int(n))


# ---------------------------------------------------------------- tensors
def gate_up(x, ids, wg, sg, wu, su, *, E=None, fp64=False):
    """h[b,j,n] = bf16(SiLU(G) * U) for all (b, j, n); x is bf16 bits [B,H].

    Returns h bits [B,k,I] (uint16), or (h, G, U, Hx) with the unrounded FP64
    values when fp64=True."""
    x = _c(x, np.uint16); ids = _c(ids, np.int32)
    wg = _c(wg, np.uint8); sg = _c(sg, np.uint8); wu = _c(wu, np.uint8); su = _c(su, np.uint8)
    B, H = x.shape
    k = ids.shape[1]
    E_, I, H2 = wg.shape
    E = E or E_
    assert H2 == H
    h = np.empty((B, k, I), np.uint16)
    G = np.empty((B, k, I)) if fp64 else None
    U = np.empty((B, k, I)) if fp64 else None
    Hx = np.empty((B, k, I)) if fp64 else None
    _check(load().orc_gate_up(_p(x), _p(ids), _p(wg), _p(sg), _p(wu), _p(su), _p(h), _p(G), _p(U), _p(Hx), B, H, I, E, k))
    return (h, G, U, Hx) if fp64 else h


def down(h, ids, w, wd, sd, *, fp64=False):
    """y[b,o] = bf16(sum_j w[b,j] * Wd[ids[b,j],o,:] . h[b,j,:]); h is bf16 bits [B,k,I].

    Returns y bits [B,H] (uint16), or (y, Y) with the unrounded FP64 sum."""
    h = _c(h, np.uint16); ids = _c(ids, np.int32); w = _c(w, np.float32)
    wd = _c(wd, np.uint8); sd = _c(sd, np.uint8)
    B, k, I = h.shape
    E, H, I2 = wd.shape
    assert I2 == I
    y = np.empty((B, H), np.uint16)
    Y = np.empty((B, H)) if fp64 else None
    _check(load().orc_down(_p(h), _p(ids), _p(w), _p(wd), _p(sd), _p(y), _p(Y), B, H, I, E, k))
    return (y, Y) if fp64 else y


def layer(x, ids, w, wg, sg, wu, su, wd, sd):
    """Both kernels: returns (h bits [B,k,I], y bits [B,H])."""
    h = gate_up(x, ids, wg, sg, wu, su)
    return h, down(h, ids, w, wd, sd)


def conventional(x, ids, w, wg, sg, wu, su, wd, sd, *, fp64=False):
    """Emulated expert-centric path (activations quantised to MXFP8, bf16 per-expert buffer)."""
    x = _c(x, np.uint16); ids = _c(ids, np.int32); w = _c(w, np.float32)
    arrs = [_c(a, np.uint8) for a in (wg, sg, wu, su, wd, sd)]
    B, H = x.shape
    k = ids.shape[1]
    E, I, _ = arrs[0].shape
    y = np.empty((B, H), np.uint16)
    Y = np.empty((B, H)) if fp64 else None
    _check(load().orc_conventional(_p(x), _p(ids), _p(w), *[_p(a) for a in arrs], _p(y), _p(Y), B, H, I, E, k))
    return (y, Y) if fp64 else y


def mx_fake_quant(v):
    """MX (E4M3 + shared power-of-two per 32) quantise-dequantise of a float64 vector."""
    a = np.array(v, dtype=np.float64, copy=True).ravel()
    load().orc_mx_fake_quant(_p(a), a.size)
    return a.reshape(np.shape(v))


def route(logits, k):
    """Router step in front of the layer (reading in ``moe_oracle.c``, ``orc_route``):
    logits FP32 [B,E] -> (ids int32 [B,k], largest logit first, lower id first among
    equal logits; weights FP64 [B,k] = softmax over E renormalised over the k)."""
    logits = _c(logits, np.float32)
    B, E = logits.shape
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    _check(load().orc_route(_p(logits), _p(ids), _p(w), B, E, int(k)))
    return ids, w


def truth_layer(x, ids, w, f_gate, f_up, f_down):
    """Full-precision reference: FP32 weight draws (unquantised), bf16 x, FP64 everywhere,
    no rounding of h, y or the per-expert outputs.  Returns FP64 y [B,H]."""
    xv = bf16_to_f64(x)
    B = xv.shape[0]
    H = xv.shape[1]
    y = np.zeros((B, H))
    for b in range(B):
        for j in range(ids.shape[1]):
            e = int(ids[b, j])
            g = f_gate[e].astype(np.float64) @ xv[b]
            u = f_up[e].astype(np.float64) @ xv[b]
            hv = g / (1.0 + np.exp(-g)) * u
            y[b] += float(w[b, j]) * (f_down[e].astype(np.float64) @ hv)
    return y
