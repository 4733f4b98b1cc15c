"""Pins for the oracle's router step (CPU only).

The pages route each token to k of E experts and say nothing more; the
reading pinned here is the plain top-k router: the k largest logits, largest
first, the lower expert id first among equal logits, weighted by the softmax
over all E logits renormalised over the kept k.  Each check fixes the oracle
against something other than itself:
  * a pure-Python restatement by ranks (rank = experts with a larger logit +
    lower ids with an equal one), with the weights as 1 / sum_i exp(l_i - l_j)
    over the kept experts, on tiny inputs full of ties;
  * closed forms: k = 1 is the first argmax with weight 1, k = 2 is the
    logistic function of the logit gap, k = E is the full softmax;
  * invariances: an exact common shift of the logits changes nothing, and
    relabelling the experts relabels the ids.
"""
import math

import numpy as np
import pytest
from scipy import special

import moe_inputs as mi


def _brute(logits, k):
    ids, ws = [], []
    for row in np.asarray(logits, np.float32).tolist():
        E = len(row)
        rank = [sum(1 for j in range(E) if row[j] > row[i]) + sum(1 for j in range(i) if row[j] == row[i])
                for i in range(E)]
        kept = sorted((i for i in range(E) if rank[i] < k), key=lambda i: rank[i])
        ids.append(kept)
        ws.append([1.0 / sum(math.exp(row[i] - row[j]) for i in kept) for j in kept])
    return np.array(ids, np.int32), np.array(ws)


def _tied_logits(seed, B, E):
    """Logits from a small set of values (many ties), exact in FP32."""
    g = np.random.default_rng(seed)
    return (g.integers(-6, 7, size=(B, E)) / 4.0).astype(np.float32)


@pytest.mark.parametrize("E,k", [(1, 1), (5, 2), (7, 3), (12, 5), (16, 16), (70, 8)])
def test_route_matches_rank_definition(orc, E, k):
    for seed, maker in ((E, _tied_logits), (E + 1, lambda s, B, E: np.random.default_rng(s).standard_normal((B, E)).astype(np.float32))):
        logits = maker(seed, 6, E)
        ids, w = orc.route(logits, k)
        bi, bw = _brute(logits, k)
        assert np.array_equal(ids, bi)
        np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


def test_route_k1_is_first_argmax(orc):
    logits = _tied_logits(3, 40, 9)
    ids, w = orc.route(logits, 1)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))   # numpy: first occurrence of the max
    assert np.all(w == 1.0)


def test_route_k2_is_logistic_of_the_gap(orc):
    logits = np.random.default_rng(4).standard_normal((50, 16)).astype(np.float32)
    ids, w = orc.route(logits, 2)
    l0 = np.take_along_axis(logits, ids[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, ids[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], special.expit(l0 - l1), rtol=1e-14)
    np.testing.assert_allclose(w[:, 1], special.expit(l1 - l0), rtol=1e-13)


def test_route_k_equals_E_is_the_full_softmax(orc):
    logits = np.random.default_rng(5).standard_normal((8, 12)).astype(np.float32)
    ids, w = orc.route(logits, 12)
    assert np.array_equal(ids, np.argsort(-logits, axis=1, kind="stable"))
    full = special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13)


def test_route_invariances(orc):
    logits = _tied_logits(6, 20, 32)
    ids, w = orc.route(logits, 8)
    ids2, w2 = orc.route(logits + np.float32(3.0), 8)   # exact in FP32: quarters below 8
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w2, w, rtol=1e-14)
    # relabel experts: new id p[e] for old id e; distinct logits so no tie order changes
    d = np.random.default_rng(7).permutation(20 * 32).reshape(20, 32).astype(np.float32) / 64
    p = np.random.default_rng(8).permutation(32)
    relabelled = np.empty_like(d)
    relabelled[:, p] = d
    a, wa = orc.route(d, 8)
    b, wb = orc.route(relabelled, 8)
    assert np.array_equal(b, p[a])
    np.testing.assert_allclose(wb, wa, rtol=1e-14)


def test_route_properties_on_the_workload(orc):
    """128 experts, top-8, N(0,1) logits: ids distinct, every kept logit >= every
    dropped one, weights positive, non-increasing and summing to one; and the
    input generator's own top-k (argsort + FP32 softmax) agrees."""
    B, E, k = 64, 128, 8
    logits = mi.router_logits(mi.routing_seed("batch_sweep", B), B, E)
    ids, w = orc.route(logits, k)
    for b in range(B):
        kept = set(ids[b].tolist())
        assert len(kept) == k
        dropped = [logits[b, e] for e in range(E) if e not in kept]
        assert min(logits[b, ids[b]]) >= max(dropped)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)
    gi, gw = mi.route_uniform(mi.routing_seed("batch_sweep", B), B, E, k)
    assert np.array_equal(ids, gi)
    np.testing.assert_allclose(w, gw, rtol=2e-7)


def test_route_edge_cases(orc):
    ids, w = orc.route(np.zeros((0, 16), np.float32), 4)
    assert ids.shape == (0, 4) and w.shape == (0, 4)
    ids, w = orc.route(np.zeros((3, 16), np.float32), 4)   # all tied: ids 0..3, equal weights
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    assert np.all(w == 0.25)
    bad = np.zeros((2, 16), np.float32)
    for v in (np.nan, np.inf, -np.inf):
        bad[1, 5] = v
        with pytest.raises(orc.OracleError):
            orc.route(bad, 4)
    with pytest.raises(orc.OracleError):
        orc.route(np.zeros((2, 4), np.float32), 5)   # k > E
