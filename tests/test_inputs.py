"""Generator invariants (CPU only): routing rules, MXFP8 packing, reproducibility."""
import numpy as np
import pytest
import torch

import moe_inputs as mi


def test_uniform_routing_invariants():
    ids, w = mi.route_uniform(0, 64, 128, 8)
    assert ids.dtype == np.int32 and w.dtype == np.float32 and ids.shape == w.shape == (64, 8)
    assert np.all((ids >= 0) & (ids < 128))
    assert all(len(set(r)) == 8 for r in ids)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)            # slots in descending logit order
    # the same ids are the top-8 of the regenerated logits, weights = renormalised softmax over all 128
    logits = mi.gen._rng(0, mi.gen._P_ROUTE, 0).standard_normal((64, 128), dtype=np.float32).astype(np.float64)
    p = np.exp(logits - logits.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    top = np.argsort(-logits, 1, kind="stable")[:, :8]
    assert np.array_equal(top, ids)
    ren = np.take_along_axis(p, top, 1); ren /= ren.sum(1, keepdims=True)
    assert np.allclose(ren, w, rtol=1e-6)


def test_routing_reproducible_and_iteration_dependent():
    a = mi.route_uniform(1002, 4, 128, 8, it=3)
    b = mi.route_uniform(1002, 4, 128, 8, it=3)
    c = mi.route_uniform(1002, 4, 128, 8, it=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])


def test_zipf_routing_popularity():
    ids, w = mi.route_zipf(3000, 2000, 128, 8)
    assert all(len(set(r)) == 8 for r in ids[:200])
    cnt = np.bincount(ids.ravel(), minlength=128)
    assert cnt[0] > cnt[10] > cnt[100]       # popularity decreases with id
    assert np.allclose(w.sum(1), 1, atol=1e-6)


def test_adversarial_routing_gaps():
    ids, w = mi.route_adversarial(3100, 64, 128, 8)
    for r in ids:
        s = np.sort(r)
        assert len(set(r)) == 8 and np.min(np.diff(s)) >= 3


def test_contiguous_routing():
    ids, _ = mi.route_contiguous(3200, 32, 128, 8)
    assert np.array_equal(ids[0], np.arange(8)) and np.array_equal(ids[17], np.arange(8, 16))


def test_x_is_bf16_of_normal_draws():
    x = mi.make_x(0, 3, 2048)
    f = mi.gen._rng(0, mi.gen._P_X, 0).standard_normal((3, 2048), dtype=np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(x, ref)


def test_mx_packing_round_trip():
    L = mi.make_layer(9, 256, 64, 3, keep_fp32=True, threads=2)
    for q, s, f in ((L.w_gate, L.s_gate, L.f_gate), (L.w_up, L.s_up, L.f_up), (L.w_down, L.s_down, L.f_down)):
        assert q.dtype == np.uint8 and s.dtype == np.uint8
        assert s.shape == q.shape[:-1] + (q.shape[-1] // 32,)
        assert not np.any((q & 0x7F) == 0x7F)                 # no NaN codes
        assert np.all((s >= 1) & (s <= 253))                   # no E8M0 0x00 / 0xFF
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        sc = np.exp2(s.astype(np.float64) - 127)
        deq = v * np.repeat(sc, 32, -1)
        blk = f.reshape(*f.shape[:-1], -1, 32).astype(np.float64)
        amax = np.abs(blk).max(-1)
        # block max lands in E4M3's top binade [256, 512) before saturation at 448
        assert np.all(amax / sc >= 256) and np.all(amax / sc < 512)
        # error bound: half an E4M3 spacing at the top binade (2^5 * scale / 2) per element
        err = np.abs(deq.reshape(blk.shape) - blk)
        assert np.all(err <= np.maximum(16 * sc, amax - 448 * sc)[..., None] + 1e-30)


def test_layer_independent_of_thread_count():
    a = mi.make_layer(4, 64, 32, 4, threads=1)
    b = mi.make_layer(4, 64, 32, 4, threads=3)
    for n in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        assert np.array_equal(getattr(a, n), getattr(b, n))


def test_workload_table():
    assert mi.WORKLOADS["batch_sweep"]["batches"] == (1, 2, 4, 8, 16, 32)
    assert mi.SHAPES["S1"] == dict(H=2048, I=768, E=128, k=8)
    assert mi.layer_seed("single_b1") == 0 and mi.routing_seed("batch_sweep", 32) == 1032
