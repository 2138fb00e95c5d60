"""Pins for the fused LM-head oracle: closed forms, fp64 finite differences of
the backward, and gradient invariants."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import fused, logprob


def test_zero_weight_is_uniform():
    rng = np.random.default_rng(1)
    N, H, V = 4, 16, 37
    h = rng.normal(size=(N, H))
    W = np.zeros((V, H))
    r = fused.forward(h, W, rng.integers(0, V, N), 0.7, 0.95)
    np.testing.assert_allclose(r.lp_full, -math.log(V), rtol=0, atol=1e-13)
    np.testing.assert_allclose(r.h_trunc, math.log(V), rtol=0, atol=1e-13)
    assert np.all(r.size == V)


def test_dominant_weight_row_is_one_hot():
    rng = np.random.default_rng(2)
    N, H, V = 3, 8, 20
    h = rng.normal(size=(N, H))
    W = rng.normal(0, 0.01, size=(V, H))
    y = np.array([4, 4, 4])
    W[4] = 50.0 * h.mean(axis=0) / np.linalg.norm(h.mean(axis=0)) ** 2 * 10
    r = fused.forward(h, W, y, 1.0, 0.9)
    z = fused.logits(h, W)
    assert np.all(np.argmax(z, axis=1) == 4)
    assert np.all(r.lp_trunc == 0.0) and np.all(r.h_trunc == 0.0) and np.all(r.size == 1)


def test_matches_materialised_logits():
    rng = np.random.default_rng(3)
    N, H, V = 5, 12, 50
    h = rng.normal(size=(N, H))
    W = rng.normal(0, 0.5, size=(V, H))
    y = rng.integers(0, V, N)
    a = fused.forward(h, W, y, 0.7, 0.95)
    z = np.array([[float(np.dot(h[n], W[v])) for v in range(V)] for n in range(N)])
    b = logprob.logprob_from_logits(z, y, 0.7, 0.95)
    np.testing.assert_allclose(a.lp_trunc, b.lp_trunc, rtol=1e-12)
    np.testing.assert_allclose(a.h_trunc, b.h_trunc, rtol=1e-12)


def _loss(h, W, y, g_lp, g_H, T, p, k=0):
    r = fused.forward(h, W, y, T, p, k)
    lp = np.where(np.isfinite(r.lp_trunc), r.lp_trunc, 0.0)
    return float(np.dot(g_lp, lp) + np.dot(g_H, r.h_trunc))


@pytest.mark.parametrize("T,p,k", [(1.0, 1.0, 0), (0.7, 1.0, 0), (0.7, 0.9, 0), (1.8, 0.6, 0),
                                   (0.7, 1.0, 5), (1.2, 0.8, 9)])
def test_backward_finite_differences(T, p, k):
    rng = np.random.default_rng(int(T * 10 + p * 100 + k))
    N, V, H = 3, 17, 8
    h = rng.normal(size=(N, H))
    W = rng.normal(0, 0.7, size=(V, H))
    y = np.array([int(np.argmax(h[n] @ W.T)) for n in range(N)])   # inside any nucleus
    y[1] = int(np.argsort(h[1] @ W.T)[-2])
    g_lp = rng.normal(size=N)
    g_H = rng.normal(size=N)
    for n in range(N):                       # keep away from a nucleus boundary
        r = logprob.row(h[n] @ W.T, int(y[n]), T, p, k)
        assert r.flags & logprob.FLAG_BOUNDARY == 0
        if k:                                # the top-k set is a strict subset
            assert r.size <= k < V
    dh, dW = fused.backward(h, W, y, g_lp, g_H, T, p, k)
    eps = 1e-6
    num_h = np.zeros_like(h)
    for idx in np.ndindex(h.shape):
        hp, hm = h.copy(), h.copy()
        hp[idx] += eps
        hm[idx] -= eps
        num_h[idx] = (_loss(hp, W, y, g_lp, g_H, T, p, k) - _loss(hm, W, y, g_lp, g_H, T, p, k)) / (2 * eps)
    num_w = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        wp, wm = W.copy(), W.copy()
        wp[idx] += eps
        wm[idx] -= eps
        num_w[idx] = (_loss(h, wp, y, g_lp, g_H, T, p, k) - _loss(h, wm, y, g_lp, g_H, T, p, k)) / (2 * eps)
    np.testing.assert_allclose(dh, num_h, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dW, num_w, rtol=1e-6, atol=1e-8)


def test_lp_only_gradient_closed_form():
    # L = -mean lp at T = 1, p = 1: dL/dz = (softmax - onehot) / N
    rng = np.random.default_rng(4)
    N, V = 6, 30
    z = rng.normal(0, 2, size=(N, V))
    y = rng.integers(0, V, N)
    G = fused.grad_logits(z, y, -np.ones(N) / N, np.zeros(N), 1.0, 1.0)
    ref = scipy.special.softmax(z, axis=1)
    ref[np.arange(N), y] -= 1.0
    np.testing.assert_allclose(G, ref / N, rtol=1e-12, atol=1e-15)


def test_gradient_invariants():
    rng = np.random.default_rng(5)
    N, V, H = 4, 25, 6
    h = rng.normal(size=(N, H))
    W = rng.normal(0, 0.5, size=(V, H))
    y = rng.integers(0, V, N)
    g_lp, g_H = rng.normal(size=N), rng.normal(size=N)
    for p in (1.0, 0.8):
        G = fused.grad_logits(fused.logits(h, W), y, g_lp, g_H, 0.7, p)
        np.testing.assert_allclose(G.sum(axis=1), 0.0, atol=1e-14)      # softmax shift invariance
        dh, dW = fused.backward(h, W, y, g_lp, g_H, 0.7, p)
        np.testing.assert_allclose(dW.sum(axis=0), 0.0, atol=1e-13)
        c = rng.normal(size=H)
        dh2, _ = fused.backward(h, W + c[None, :], y, g_lp, g_H, 0.7, p)
        np.testing.assert_allclose(dh2, dh, rtol=1e-9, atol=1e-12)       # per-row logit shift
