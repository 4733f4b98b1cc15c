"""Seeded generators for activations, routing and MXFP8 expert weights.

Everything here is input preparation.  Random draws use NumPy's PCG64 through
``SeedSequence(entropy=seed, spawn_key=(purpose, ...))`` so that every tensor,
expert slab and routing iteration has its own reproducible stream and can be
regenerated on its own (the 48-layer and 4096-wide workloads are too large to
hold as FP32 draws).

Weight packing follows the OCP Microscaling (MX) v1.0 layout that the pages
call MXFP8 (warp-decode post, "How the two kernels work"): E4M3 elements with
one E8M0 power-of-two scale per 32 consecutive elements along the reduction
dimension.  The quantiser below only has to *produce* valid MXFP8 bytes; the
layer consumes those bytes, so its exact rounding rule does not affect parity.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MX_BLOCK = 32          # elements per E8M0 scale
_E4M3_EMAX = 8         # exponent of the largest E4M3 binade (448 = 1.75 * 2**8)
_E4M3_MAX = 448.0

# Layer shapes of the synthetic workloads.  E=128 experts with top-8 routing and
# hidden size 2048 are the figures the pages use (sections "The traditional MoE
# path" and "Eliminating buffers"); I=768 and the 4096/1536 shape are the
# stated synthetic configurations.
SHAPES = {
    "S1": dict(H=2048, I=768, E=128, k=8),
    "S2": dict(H=4096, I=1536, E=128, k=8),
}

# Purposes (first element of the spawn key).
_P_WEIGHT, _P_X, _P_ROUTE, _P_ROUTE_W = 0, 1, 2, 3
_T_GATE, _T_UP, _T_DOWN = 0, 1, 2


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(int(k) for k in key)))


def _threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


# --------------------------------------------------------------------------
# Encoders used only to create inputs
# --------------------------------------------------------------------------
def _e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values with |v| <= 448 to the nearest E4M3 code (ties to even).

    Normal range (|v| >= 2**-6): round the FP32 significand to 3 bits in the
    integer domain (adding the rounding bias may carry into the exponent, which
    is the correct next binade) and rebias the exponent from 127 to 7.
    Subnormal range: the E4M3 spacing is 2**-9, so the code is rint(|v| * 512).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32)
    sign = (u >> 31).astype(np.uint32)
    mag = u & np.uint32(0x7FFFFFFF)
    rounded = (mag + np.uint32(0x7FFFF) + ((mag >> 20) & np.uint32(1))) >> 20
    normal_code = rounded.astype(np.int64) - (120 << 3)
    a = mag.view(np.float32)
    sub_code = np.rint(a * np.float32(512.0)).astype(np.int64)
    code = np.where(a >= np.float32(2.0 ** -6), normal_code, sub_code)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def _mx_pack(w: np.ndarray):
    """Pack an FP32 matrix [R, C] (C % 32 == 0) into E4M3 codes [R, C] + E8M0 codes [R, C/32].

    Scale exponent = floor(log2(block amax)) - 8, so the block maximum lands in
    E4M3's top binade; scaled values are saturated to +-448.  Scale codes are
    kept in [1, 253]; an all-zero block gets code 127 (scale 1).
    """
    R, C = w.shape
    blk = np.ascontiguousarray(w, dtype=np.float32).reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    e_amax = (amax.view(np.uint32) >> 23).astype(np.int64) - 127   # floor(log2 amax) for normal amax
    code = np.clip(e_amax - _E4M3_EMAX + 127, 1, 253)
    code = np.where(amax > 0, code, 127)
    inv_scale = ((254 - code).astype(np.uint32) << 23).view(np.float32)   # 2**(127 - code), exact
    scaled = blk * inv_scale[..., None]
    np.clip(scaled, -_E4M3_MAX, _E4M3_MAX, out=scaled)
    q = _e4m3_encode(scaled)
    return q.reshape(R, C), code.astype(np.uint8)


def bf16_bits_from_f32(f: np.ndarray) -> np.ndarray:
    """FP32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------
@dataclass
class Layer:
    """One MoE layer's MXFP8 expert weights, in the library's plain layout.

    w_gate, w_up: uint8 [E, I, H] E4M3 codes; s_gate, s_up: uint8 [E, I, H/32] E8M0 codes.
    w_down: uint8 [E, H, I] E4M3 codes;      s_down: uint8 [E, H, I/32] E8M0 codes.
    f_gate/f_up/f_down: the FP32 draws before quantisation (only when requested).
    """
    H: int
    I: int
    E: int
    seed: int
    w_gate: np.ndarray
    s_gate: np.ndarray
    w_up: np.ndarray
    s_up: np.ndarray
    w_down: np.ndarray
    s_down: np.ndarray
    f_gate: Optional[np.ndarray] = field(default=None, repr=False)
    f_up: Optional[np.ndarray] = field(default=None, repr=False)
    f_down: Optional[np.ndarray] = field(default=None, repr=False)

    @property
    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.w_gate, self.s_gate, self.w_up, self.s_up, self.w_down, self.s_down))


def _draw_slab(seed: int, tensor: int, e: int, rows: int, cols: int, fan_in: int) -> np.ndarray:
    g = _rng(seed, _P_WEIGHT, tensor, e)
    w = g.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(fan_in))
    return w


def make_layer(seed: int, H: int, I: int, E: int, keep_fp32: bool = False, threads: Optional[int] = None) -> Layer:
    """Draw W_gate, W_up ~ N(0, 1/H) [E,I,H] and W_down ~ N(0, 1/I) [E,H,I]; pack to MXFP8.

    Each (tensor, expert) slab has its own stream, so slabs are generated in
    parallel threads and the result does not depend on the thread count.
    """
    if H % MX_BLOCK or I % MX_BLOCK:
        raise ValueError("H and I must be multiples of 32")
    wg = np.empty((E, I, H), np.uint8); sg = np.empty((E, I, H // MX_BLOCK), np.uint8)
    wu = np.empty((E, I, H), np.uint8); su = np.empty((E, I, H // MX_BLOCK), np.uint8)
    wd = np.empty((E, H, I), np.uint8); sd = np.empty((E, H, I // MX_BLOCK), np.uint8)
    fg = np.empty((E, I, H), np.float32) if keep_fp32 else None
    fu = np.empty((E, I, H), np.float32) if keep_fp32 else None
    fd = np.empty((E, H, I), np.float32) if keep_fp32 else None
    jobs = []
    for e in range(E):
        jobs.append((_T_GATE, e, I, H, H, wg, sg, fg))
        jobs.append((_T_UP, e, I, H, H, wu, su, fu))
        jobs.append((_T_DOWN, e, H, I, I, wd, sd, fd))

    def run(job):
        t, e, rows, cols, fan, wq, ws, wf = job
        w = _draw_slab(seed, t, e, rows, cols, fan)
        q, s = _mx_pack(w)
        wq[e] = q
        ws[e] = s
        if wf is not None:
            wf[e] = w

    n = threads or _threads()
    if n <= 1:
        for j in jobs:
            run(j)
    else:
        with _cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(run, jobs))
    return Layer(H, I, E, seed, wg, sg, wu, su, wd, sd, fg, fu, fd)


# --------------------------------------------------------------------------
# Activations and routing
# --------------------------------------------------------------------------
def make_x(seed: int, B: int, H: int, it: int = 0) -> np.ndarray:
    """x ~ N(0,1) rounded to bf16; returned as uint16 bit patterns [B, H]."""
    f = _rng(seed, _P_X, it).standard_normal((B, H), dtype=np.float32)
    return bf16_bits_from_f32(f)


def _softmax_f32(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def router_logits(seed: int, B: int, E: int, it: int = 0) -> np.ndarray:
    """Router logits ~ N(0,1), FP32 [B,E] (the draw behind route_uniform)."""
    return _rng(seed, _P_ROUTE, it).standard_normal((B, E), dtype=np.float32)


def route_uniform(seed: int, B: int, E: int, k: int, it: int = 0):
    """Router logits ~ N(0,1) [B,E]; ids = top-k by descending logit (ties -> lower id);
    weights = softmax over the k selected logits (= softmax over E renormalised over the top-k)."""
    logits = router_logits(seed, B, E, it)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = _softmax_f32(np.take_along_axis(logits, ids.astype(np.int64), axis=1))
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def _fresh_weights(seed: int, B: int, k: int, it: int) -> np.ndarray:
    return _softmax_f32(_rng(seed, _P_ROUTE_W, it).standard_normal((B, k), dtype=np.float32))


def route_zipf(seed: int, B: int, E: int, k: int, s: float = 1.1, it: int = 0):
    """Zipf(s) expert popularity p(e) ~ (e+1)^-s; k distinct ids per token drawn without
    replacement proportionally to p (Gumbel-top-k); weights = softmax of k fresh N(0,1) logits."""
    g = _rng(seed, _P_ROUTE, it)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    u = g.random((B, E))
    keys = logp[None, :] - np.log(-np.log(np.clip(u, 1e-300, 1.0)))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    return np.ascontiguousarray(ids), _fresh_weights(seed, B, k, it)


def route_adversarial(seed: int, B: int, E: int, k: int, gap: int = 3, it: int = 0):
    """k distinct ids per token, uniform subject to every pairwise gap >= `gap` (rejection
    sampling); weights = softmax of k fresh N(0,1) logits."""
    if (k - 1) * gap + 1 > E:
        raise ValueError("gap too large for E and k")
    g = _rng(seed, _P_ROUTE, it)
    ids = np.empty((B, k), np.int32)
    for b in range(B):
        while True:
            c = g.choice(E, size=k, replace=False)
            if np.min(np.diff(np.sort(c))) >= gap:
                ids[b] = c
                break
    return ids, _fresh_weights(seed, B, k, it)


def route_contiguous(seed: int, B: int, E: int, k: int, it: int = 0):
    """Control routing: token b uses experts k*(b mod E/k) + {0..k-1} (adjacent rows)."""
    groups = E // k
    ids = np.array([[k * (b % groups) + j for j in range(k)] for b in range(B)], np.int32)
    return ids, _fresh_weights(seed, B, k, it)


_ROUTERS = {
    "uniform": route_uniform,
    "zipf": route_zipf,
    "adversarial": route_adversarial,
    "contiguous": route_contiguous,
}


def make_routing(kind: str, seed: int, B: int, E: int, k: int, it: int = 0):
    return _ROUTERS[kind](seed, B, E, k, it=it)


# --------------------------------------------------------------------------
# The five synthetic workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    "single_b1": dict(name="single layer, B=1", shape="S1", batches=(1,), routings=("uniform",), layers=1),
    "batch_sweep": dict(name="single layer, batch sweep", shape="S1", batches=(1, 2, 4, 8, 16, 32), routings=("uniform",),
                        layers=1),
    "routing_stress": dict(name="B=32 routing stress", shape="S1", batches=(32,),
                           routings=("zipf", "adversarial", "contiguous"), layers=1),
    "decode_step": dict(name="48-layer decode step", shape="S1", batches=(1, 8, 32), routings=("uniform",), layers=48),
    "wide_layers": dict(name="larger expert shape, 8 layers", shape="S2", batches=(1, 16, 32, 64), routings=("uniform",),
                        layers=8),
}

_ROUTE_BASE = {"zipf": 3000, "adversarial": 3100, "contiguous": 3200}


def layer_seed(workload: str, layer: int = 0) -> int:
    """Weight seed of layer `layer` of a workload (the three single-layer workloads share seed 0)."""
    if workload in ("single_b1", "batch_sweep", "routing_stress"):
        return 0
    if workload == "decode_step":
        return layer
    if workload == "wide_layers":
        return 5000 + layer
    raise ValueError(workload)


def routing_seed(workload: str, B: int, routing: str = "uniform", layer: int = 0) -> int:
    """Seed of the activation/routing stream; iteration r of that stream uses spawn key r."""
    if workload == "single_b1":
        return 0
    if workload == "batch_sweep":
        return 1000 + B
    if workload == "routing_stress":
        return _ROUTE_BASE[routing]
    if workload == "decode_step":
        return 4000 + layer
    if workload == "wide_layers":
        return 5000 + layer
    raise ValueError(workload)
