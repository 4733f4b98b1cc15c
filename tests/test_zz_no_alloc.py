"""GPU test of moe_decode_conventional_noalloc, the conventional path on the
library's fixed scratch buffer, through the C ABI.

Its result must equal moe_decode_conventional's (same kernels, caller-given
workspace) bit for bit, on two calls in a row where the second has a smaller
batch and so runs over what the first left in the buffer; and a HIP graph that
captures the call (it allocates nothing) reproduces the eager result on every
replay, with eager work in between.
"""
import numpy as np
import pytest
import torch

import moe_gate_up_amd as mg
import moe_inputs as mi

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


@pytest.fixture(scope="module")
def layer(dev):
    L = mi.make_layer(700, 2048, 768, 32)
    return [_t(a, dev) for a in (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)]


def _inputs(seed, B, dev):
    x = mi.make_x(seed, B, 2048)
    ids, w = mi.route_uniform(seed, B, 32, 8)
    return _t(x, dev), _t(ids, dev), _t(w, dev)


def _with_workspace(x, ids, w, W, dev):
    B = x.shape[0]
    ws = torch.empty(mg.moe_decode_conventional_workspace(B, 2048, 768, 32, 8), dtype=torch.uint8, device=dev)
    y = torch.empty((B, 2048), dtype=torch.int16, device=dev)
    mg.moe_decode_conventional(x, ids, w, *W, y, ws)
    torch.cuda.synchronize()
    return y


def test_noalloc_equals_workspace_path_on_two_calls(dev, layer):
    for seed, B in ((701, 32), (702, 5)):   # the second call is smaller than the first
        x, ids, w = _inputs(seed, B, dev)
        print(f"noalloc: B={B} H=2048 I=768 E=32 k=8 seed={seed}", flush=True)
        y = torch.full((B, 2048), -1, dtype=torch.int16, device=dev)
        mg.moe_decode_conventional_noalloc(x, ids, w, *layer, y)
        torch.cuda.synchronize()
        ref = _with_workspace(x, ids, w, layer, dev)
        assert torch.equal(y, ref), (B, int((y != ref).sum()))
        assert torch.isfinite(y.view(torch.bfloat16).float()).all()


def test_noalloc_captured_in_a_graph(dev, layer):
    B = 12
    x, ids, w = _inputs(703, B, dev)
    print(f"noalloc graph: B={B} H=2048 I=768 E=32 k=8", flush=True)
    y = torch.empty((B, 2048), dtype=torch.int16, device=dev)
    mg.moe_decode_conventional_noalloc(x, ids, w, *layer, y)
    torch.cuda.synchronize()
    eager = y.clone()
    assert torch.equal(eager, _with_workspace(x, ids, w, layer, dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.moe_decode_conventional_noalloc(x, ids, w, *layer, y)
    x2, ids2, w2 = _inputs(704, 20, dev)
    y2 = torch.empty((20, 2048), dtype=torch.int16, device=dev)
    for rep in range(4):
        y.fill_(-1)
        mg.moe_decode_conventional_noalloc(x2, ids2, w2, *layer, y2)   # eager work on the same buffer between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), rep


def test_noalloc_full_size_layer(dev):
    """The H=2048, I=768, 128-expert layer at 32 tokens and then 4 (4.2 MiB
    and 0.6 MiB of the 32 MiB buffer), each equal to the workspace path bit
    for bit."""
    s = mi.SHAPES["S1"]
    H, I, E, k = s["H"], s["I"], s["E"], s["k"]
    L = mi.make_layer(mi.layer_seed("single_b1"), H, I, E)
    W = [_t(a, dev) for a in (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)]
    for seed, B in ((711, 32), (712, 4)):
        print(f"noalloc full size: B={B} H={H} I={I} E={E} k={k} seed={seed}", flush=True)
        x = _t(mi.make_x(seed, B, H), dev)
        ids_h, w_h = mi.route_uniform(seed, B, E, k)
        ids, w = _t(ids_h, dev), _t(w_h, dev)
        y = torch.full((B, H), -1, dtype=torch.int16, device=dev)
        mg.moe_decode_conventional_noalloc(x, ids, w, *W, y)
        torch.cuda.synchronize()
        ws = torch.empty(mg.moe_decode_conventional_workspace(B, H, I, E, k), dtype=torch.uint8, device=dev)
        ref = torch.empty((B, H), dtype=torch.int16, device=dev)
        mg.moe_decode_conventional(x, ids, w, *W, ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (B, int((y != ref).sum()))
        assert torch.isfinite(y.view(torch.bfloat16).float()).all()
