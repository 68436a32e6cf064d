"""Pins of the oracle's router (top-K + weights) and align (sort + pad).

Compared with: hand cases with closed-form answers, a brute-force comparison
sort, scipy's softmax (a library routine) and structural invariants.
"""

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe


def _brute_topk(row, K):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:K]


def test_route_hand_cases():
    ids, w = moe.route(np.array([[1.0, 3.0, 3.0, 2.0]], np.float32), 2)
    assert ids.tolist() == [[1, 2]] and np.allclose(w, [[0.5, 0.5]], atol=0, rtol=1e-15)
    ids, w = moe.route(np.array([[0.0, math.log(3.0)]], np.float32), 2)
    assert ids.tolist() == [[1, 0]]
    # logits are float32: ln3 rounds, so the weights are 3/4, 1/4 to ~1e-8
    assert np.allclose(w, [[0.75, 0.25]], atol=1e-7)
    # -0.0 and +0.0 are equal: lower id first
    ids, _ = moe.route(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]
    ids, _ = moe.route(np.array([[0.0, -0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]


def test_route_all_equal_logits():
    ids, w = moe.route(np.full((3, 16), 0.25, np.float32), 5)
    assert (ids == np.arange(5)).all()
    assert np.allclose(w, 0.2, rtol=1e-15)


@pytest.mark.parametrize("E,K", [(8, 2), (16, 16), (256, 8), (128, 8), (7, 1), (64, 64)])
def test_route_matches_brute_force(E, K):
    rng = np.random.default_rng(E * 100 + K)
    lg = rng.standard_normal((40, E)).astype(np.float32)
    lg[::3] = rng.integers(0, 4, size=lg[::3].shape)        # tie-heavy rows
    ids, w = moe.route(lg, K)
    for t in range(lg.shape[0]):
        assert ids[t].tolist() == _brute_topk(lg[t], K)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (np.diff(w, axis=1) <= 1e-15).all()               # non-increasing


def test_route_weights_vs_scipy_softmax():
    rng = np.random.default_rng(5)
    lg = (rng.standard_normal((20, 12)) * 4).astype(np.float32)
    # K = E: the renormalised weights are the full softmax in sorted order
    ids, w = moe.route(lg, 12)
    p = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12)
    # no renormalisation: the softmax entries themselves
    ids, w = moe.route(lg, 3, renormalize=False)
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12)
    # K = 1 renormalised: weight exactly 1
    _, w = moe.route(lg, 1)
    assert (w == 1.0).all()
    # renormalised = softmax restricted to the chosen logits
    ids, w = moe.route(lg, 4)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-12)


def test_route_large_logits_finite():
    ids, w = moe.route(np.array([[1000.0, 990.0, -1000.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]] and np.isfinite(w).all()
    assert abs(w[0, 0] - 1 / (1 + math.exp(-10))) < 1e-12


def _brute_align(ids, E, BM):
    flat = np.asarray(ids).reshape(-1).tolist()
    P = len(flat)
    order = sorted(range(P), key=lambda i: (flat[i], i))
    out, blocks = [], []
    j = 0
    while j < P:
        e = flat[order[j]]
        run = []
        while j < P and flat[order[j]] == e:
            run.append(order[j])
            j += 1
        while len(run) % BM:
            run.append(P)
        out += run
        blocks += [e] * (len(run) // BM)
    return out, blocks


def _check_invariants(ids, E, BM, sorted_ids, block_expert, npp):
    flat = np.asarray(ids).reshape(-1)
    P = flat.size
    counts = np.bincount(flat, minlength=E)
    assert npp == int(sum(-(-c // BM) * BM for c in counts))
    assert sorted_ids.size == npp and block_expert.size == npp // BM
    real = sorted_ids[sorted_ids != P]
    assert np.array_equal(np.sort(real), np.arange(P))
    assert (np.diff(block_expert) >= 0).all()
    assert set(block_expert.tolist()) == set(np.nonzero(counts)[0].tolist())
    for b, e in enumerate(block_expert):
        blk = sorted_ids[b * BM:(b + 1) * BM]
        r = blk[blk != P]
        assert (flat[r] == e).all()
        assert (np.diff(r) > 0).all()
        # sentinels only after the real entries of the block
        nreal = r.size
        assert (blk[nreal:] == P).all()


@pytest.mark.parametrize("T,E,K,BM", [
    (4, 8, 2, 16), (1, 256, 8, 16), (64, 256, 8, 64), (64, 8, 2, 64),
    (37, 128, 8, 32), (300, 16, 4, 128), (5, 4, 4, 1), (0, 8, 2, 16),
])
def test_align_vs_brute_force(T, E, K, BM):
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = moe.route(lg, K) if T else (np.zeros((0, K), np.int32), None)
    s, b, npp = moe.align(ids, E, BM)
    bs, bb = _brute_align(ids, E, BM)
    assert s.tolist() == bs and b.tolist() == bb and npp == len(bs)
    _check_invariants(ids, E, BM, s, b, npp)


def test_align_single_expert_and_skew():
    ids = np.zeros((10, 1), np.int32)
    s, b, npp = moe.align(ids, 4, 4)
    assert npp == 12 and b.tolist() == [0, 0, 0]
    assert s.tolist() == list(range(10)) + [10, 10]
    ids = np.array([[3, 1], [3, 0], [3, 2]], np.int32)
    s, b, npp = moe.align(ids, 4, 2)
    assert s.tolist() == [3, 6, 1, 6, 5, 6, 0, 2, 4, 6]
    assert b.tolist() == [0, 1, 2, 3, 3]
