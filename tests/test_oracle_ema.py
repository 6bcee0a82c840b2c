"""Pins for the fp64 gated-EMA oracle (CPU only).

The oracle computes out_t = f_t * out_{t-1} + x_t one channel at a time.  It is
trusted because of checks that come from outside that loop:

* a parallel prefix scan (Hillis-Steele doubling) built from the associative
  operator printed in RetNet issue #21, (x_a, f_a) o (x_b, f_b) =
  (x_a f_b + x_b, f_a f_b), combining whole spans in a different order;
* the closed form out_t = sum_{s<=t} (prod_{s<r<=t} f_r) x_s
  + (prod_{r<=t} f_r) out_0, built with explicit products;
* the page's own derivation: retention is the query contraction of the EMA of
  the key/value outer products with a constant factor, so the linear-attention
  oracle (pinned separately) must agree with this one on the same inputs;
* special cases: f == 0 returns x, f == 1 is numpy.cumsum, a single impulse
  under a constant factor decays geometrically;
* invariants: reverse == flip . forward . flip, continuation through the carried
  state, independence from the thread count.
"""
import numpy as np
import pytest

import oracle


def rng_inputs(seed, B=2, T=11, C=5):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, C))
    f = 1.0 / (1.0 + np.exp(-r.normal(1.0, 1.5, (B, T, C))))
    h0 = r.standard_normal((B, C))
    return x, f, h0


def prefix_scan_with_page_operator(x, f, h0):
    """Inclusive scan along time with the published operator, by doubling: after
    round r each position holds the combination of the 2^r positions ending at
    it.  The initial state enters as a leading element with factor 0."""
    B, T, C = x.shape
    X = np.concatenate([h0[:, None, :], x], axis=1)
    F = np.concatenate([np.zeros((B, 1, C)), f], axis=1)
    d = 1
    while d < T + 1:
        Xa, Fa = X[:, :-d], F[:, :-d]          # the earlier span (a)
        Xb, Fb = X[:, d:], F[:, d:]            # the later span (b)
        nX, nF = X.copy(), F.copy()
        nX[:, d:] = Xa * Fb + Xb               # (x_a, f_a) o (x_b, f_b)
        nF[:, d:] = Fa * Fb
        X, F = nX, nF
        d *= 2
    return X[:, 1:], X[:, -1]


def closed_form(x, f, h0):
    B, T, C = x.shape
    y = np.zeros((B, T, C))
    for t in range(T):
        acc = h0 * np.prod(f[:, : t + 1], axis=1)
        for s in range(t + 1):
            acc = acc + np.prod(f[:, s + 1 : t + 1], axis=1) * x[:, s]
        y[:, t] = acc
    return y


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_prefix_scan_of_the_page_operator(seed):
    x, f, h0 = rng_inputs(seed, T=13)
    y, s = oracle.ema(x, f, h0)
    ys, ss = prefix_scan_with_page_operator(x, f, h0)
    np.testing.assert_allclose(y, ys, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, ss, rtol=1e-12, atol=1e-12)


def test_matches_closed_form():
    x, f, h0 = rng_inputs(2, T=9)
    y, s = oracle.ema(x, f, h0)
    np.testing.assert_allclose(y, closed_form(x, f, h0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, y[:, -1], rtol=0, atol=0)


def test_retention_is_query_contraction_of_outer_product_ema():
    """RetNet issue #21 computes retention as einsum(Q, cumulative_ema(K v^T, gamma))."""
    r = np.random.default_rng(3)
    B, H, T, Dk, Dv = 1, 2, 10, 3, 4
    q = r.standard_normal((B, H, T, Dk))
    k = r.standard_normal((B, H, T, Dk))
    v = r.standard_normal((B, H, T, Dv))
    gam = np.array([0.7, 0.95])
    for reverse in (False, True):
        y_la, s_la, _ = oracle.la(q, k, v, gam, "head", reverse=reverse)
        for h in range(H):
            outer = np.einsum("ta,tc->tac", k[0, h], v[0, h]).reshape(1, T, Dk * Dv)
            rhs, st = oracle.ema(outer, np.full_like(outer, gam[h]), reverse=reverse)
            y = np.einsum("ta,tac->tc", q[0, h], rhs[0].reshape(T, Dk, Dv))
            np.testing.assert_allclose(y, y_la[0, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(st[0].reshape(Dk, Dv), s_la[0, h], rtol=1e-12, atol=1e-12)


def test_special_cases():
    x, f, h0 = rng_inputs(4)
    y, _ = oracle.ema(x, np.zeros_like(f), h0)
    np.testing.assert_array_equal(y, x)
    y, s = oracle.ema(x, np.ones_like(f), h0)
    np.testing.assert_allclose(y, np.cumsum(x, axis=1) + h0[:, None, :], rtol=1e-13, atol=1e-13)
    imp = np.zeros((1, 8, 1))
    imp[0, 0, 0] = 1.0
    y, s = oracle.ema(imp, np.full_like(imp, 0.5))
    np.testing.assert_array_equal(y[0, :, 0], 0.5 ** np.arange(8))


def test_reverse_is_flip_forward_flip():
    x, f, h0 = rng_inputs(5)
    yr, sr = oracle.ema(x, f, h0, reverse=True)
    yf, sf = oracle.ema(x[:, ::-1], f[:, ::-1], h0)
    np.testing.assert_array_equal(yr, yf[:, ::-1])
    np.testing.assert_array_equal(sr, sf)


def test_continuation_through_state():
    x, f, h0 = rng_inputs(6, T=20)
    y, s = oracle.ema(x, f, h0)
    y1, s1 = oracle.ema(x[:, :7], f[:, :7], h0)
    y2, s2 = oracle.ema(x[:, 7:], f[:, 7:], s1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(s2, s)


def test_thread_count_invariance():
    x, f, h0 = rng_inputs(7, B=3, T=50, C=33)
    a = oracle.ema(x, f, h0, threads=1)
    b = oracle.ema(x, f, h0, threads=4)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)
