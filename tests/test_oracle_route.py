"""Pins of the oracle's router product and top-k softmax (CPU only)."""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle.moe import router_logits, topk_softmax


def _brute_topk(l32, k):
    T, E = l32.shape
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        row = [float(v) for v in l32[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        idx[t] = order
        m = max(row)
        p = [math.exp(v - m) for v in row]
        z = sum(p)
        p = [v / z for v in p]
        s = sum(p[e] for e in order)
        w[t] = [p[e] / s for e in order]
    return idx, w


def _planted(T, E, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    # exact ties inside the top-k, at the k-th boundary, and +0 / -0 pairs
    l[:, 3] = l[:, 1]
    l[::2, 5] = l[::2, 0]
    l[1::3, 2] = 0.0
    l[1::3, 6] = -0.0
    l[1::3, 7] = 10.0  # -> 0.0 and -0.0 compete for later slots
    l[5, :] = 1.25     # a whole row of ties
    return l


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (33, 10), (64, 8)])
def test_topk_matches_brute_force(E, k):
    l = _planted(40, E, seed=E * 7 + k)
    idx, w = topk_softmax(l, k)
    bi, bw = _brute_topk(l, k)
    assert np.array_equal(idx, bi)
    assert np.allclose(w, bw, rtol=1e-6, atol=0)


def test_signed_zero_is_a_tie_broken_by_index():
    l = np.array([[-0.0, 0.0, -1.0, -0.0]], np.float32)
    idx, w = topk_softmax(l, 3)
    assert idx.tolist() == [[0, 1, 3]]
    assert np.allclose(w, 1.0 / 3.0, rtol=1e-7)


def test_zero_router_gives_first_k_and_uniform_weights():
    x = np.random.default_rng(0).standard_normal((16, 32))
    l = router_logits(x, np.zeros((12, 32)))
    idx, w = topk_softmax(l, 5)
    assert np.array_equal(idx, np.tile(np.arange(5), (16, 1)))
    assert np.allclose(w, 0.2, rtol=1e-7)


def test_k_equals_E_is_full_softmax():
    l = np.random.default_rng(1).standard_normal((20, 9)).astype(np.float32)
    idx, w = topk_softmax(l, 9)
    ref = softmax(l.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx, 1), rtol=1e-6)


def test_renormalised_topk_of_softmax():
    """renorm(topk(softmax(l))) computed with scipy equals the oracle weights."""
    l = np.random.default_rng(2).standard_normal((50, 64)).astype(np.float32) * 3
    idx, w = topk_softmax(l, 10)
    p = softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6)


def test_topk_invariants():
    l = np.random.default_rng(4).standard_normal((200, 128)).astype(np.float32)
    idx, w = topk_softmax(l, 8)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in idx.tolist())
    vals = np.take_along_axis(l, idx, 1)
    kth = vals[:, -1:]
    others = l.copy()
    np.put_along_axis(others, idx, -np.inf, 1)
    assert np.all(others <= kth)


def test_router_logits_against_exact_sums():
    """fp64 product rounded to fp32 equals the correctly rounded exact dot
    product (math.fsum of exact bf16-representable products) to 1 fp32 ulp."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 512)).astype(np.float32).astype(np.float64)
    wr = (rng.standard_normal((16, 512)) / 22.6).astype(np.float32).astype(np.float64)
    l = router_logits(x, wr)
    for t in range(8):
        for e in range(16):
            exact = np.float32(math.fsum(float(a) * float(b) for a, b in zip(x[t], wr[e])))
            assert abs(float(l[t, e]) - float(exact)) <= float(np.spacing(np.abs(exact)))


# ---------------------------------------------------------------- softmax gating without renormalisation
def test_plain_softmax_weights_match_library_softmax():
    """renormalize=False: the weights are scipy's softmax over all experts,
    read at the selected indices."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    l = (rng.standard_normal((50, 40)) * 3).astype(np.float32)
    idx, w = topk_softmax(l, 6, renormalize=False)
    ref = softmax(l.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx.astype(np.int64), axis=1), rtol=1e-6, atol=0)
    assert np.array_equal(idx, topk_softmax(l, 6)[0])          # selection is unchanged
    assert np.all(w.sum(axis=1) < 1.0) and np.all(np.diff(w, axis=1) <= 0)


def test_plain_and_renormalised_agree_when_every_expert_is_selected():
    """k = E: both are the full softmax."""
    l = _planted(20, 9, seed=3)
    _, wr = topk_softmax(l, 9)
    _, wp = topk_softmax(l, 9, renormalize=False)
    assert np.allclose(wr, wp, rtol=1e-6, atol=0)


def test_plain_weights_are_renormalised_weights_times_selected_mass():
    """w_plain = w_renorm * (selected softmax mass), a closed form."""
    rng = np.random.default_rng(5)
    l = rng.standard_normal((30, 24)).astype(np.float32)
    idx, wr = topk_softmax(l, 4)
    _, wp = topk_softmax(l, 4, renormalize=False)
    l64 = l.astype(np.float64)
    mass = np.exp(np.take_along_axis(l64, idx.astype(np.int64), axis=1) - l64.max(axis=1, keepdims=True)).sum(axis=1) \
        / np.exp(l64 - l64.max(axis=1, keepdims=True)).sum(axis=1)
    assert np.allclose(wp, wr * mass[:, None], rtol=2e-6, atol=0)
