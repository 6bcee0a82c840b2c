"""Pins for the oracle's per-element decay mode and its bidirectional forms (CPU only).

Per-element decay (RetNet issue #21: cumulative_ema takes factors shaped like
the values) gives each key channel its own factor g_t[i].  The oracle's ELEM
mode is trusted because of checks from outside its loop:

* the page's own construction, the EMA of the key/value outer products with
  factors broadcast along the value axis, computed by the separately pinned
  gated-EMA oracle and contracted with the query;
* the explicit parallel form, y_t = sum_{s<=t} sum_i q_t[i] k_s[i]
  (prod_{s<r<=t} g_r[i]) v_s plus the decayed initial state, with its
  normalised ratio, built with explicit products;
* a decomposition: without normalisation the output is the sum over key
  channels i of one-channel problems with the per-step decay g_t[i], each of
  which is the (pinned) STEP mode with Dk = 1;
* the special case of factors equal across channels, which is STEP mode.

The bidirectional encoder (the same page: combine a forward and a reverse
call) is read as the sum of the two outputs.  Its pins are the two-sided
quadratic form with the decay mask D[t,s] = prod of the factors strictly
between the two positions, counted from the later one, with the diagonal
counted twice, and, for the gated EMA, the two-sided closed form.
"""
import numpy as np
import pytest

import oracle


def rng_elem(seed, B=2, H=2, T=9, Dk=3, Dv=4, positive=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, Dk))
    k = r.standard_normal((B, H, T, Dk))
    v = r.standard_normal((B, H, T, Dv))
    if positive:
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    g = 1.0 / (1.0 + np.exp(-r.normal(1.5, 1.0, (B, H, T, Dk))))
    return q, k, v, g


def quadratic_elem(q, k, v, g, S0=None, z0=None, normalize=False, reverse=False):
    """Explicit parallel form with one factor product per key channel."""
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    y = np.zeros((B, H, T, Dv))
    order = list(range(T))[::-1] if reverse else list(range(T))
    pos = {t: n for n, t in enumerate(order)}        # visiting position of time t
    for b in range(B):
        for h in range(H):
            for t in range(T):
                num = np.zeros(Dv)
                den = 0.0
                for s in range(T):
                    if pos[s] > pos[t]:
                        continue
                    # factors of the steps visited after s, up to and including t
                    between = [order[n] for n in range(pos[s] + 1, pos[t] + 1)]
                    dec = np.prod(g[b, h, between], axis=0) if between else np.ones(Dk)
                    w = np.sum(q[b, h, t] * k[b, h, s] * dec)
                    num += w * v[b, h, s]
                    den += w
                upto = [order[n] for n in range(0, pos[t] + 1)]
                P = np.prod(g[b, h, upto], axis=0)
                if S0 is not None:
                    num += (q[b, h, t] * P) @ S0[b, h]
                if z0 is not None:
                    den += np.sum(q[b, h, t] * P * z0[b, h])
                y[b, h, t] = num / den if normalize else num
    return y


@pytest.mark.parametrize("reverse", [False, True])
def test_elem_is_query_contraction_of_outer_product_ema(reverse):
    """cumulative_ema(K v^T, factors) with factors[t, i, j] = g_t[i]."""
    q, k, v, g = rng_elem(0, B=1, H=2, T=10, Dk=3, Dv=4)
    S0 = np.random.default_rng(10).standard_normal((1, 2, 3, 4))
    y, s, _ = oracle.la(q, k, v, g, "elem", state_in=S0, reverse=reverse)
    T, Dk, Dv = 10, 3, 4
    for h in range(2):
        # the flattened state S[i, j] <-> i * Dv + j: key row i's factor on every column j
        outer = np.stack([np.outer(k[0, h, t], v[0, h, t]).ravel() for t in range(T)])[None]
        fac = np.repeat(g[0, h], Dv, axis=1)[None]
        rhs, st = oracle.ema(outer, fac, S0[0, h].reshape(1, Dk * Dv), reverse=reverse)
        ye = np.stack([q[0, h, t] @ rhs[0, t].reshape(Dk, Dv) for t in range(T)])
        np.testing.assert_allclose(y[0, h], ye, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s[0, h], st[0].reshape(Dk, Dv), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("normalize", [False, True])
def test_elem_matches_quadratic_form(normalize, reverse):
    q, k, v, g = rng_elem(1, positive=normalize)
    r = np.random.default_rng(11)
    S0 = r.standard_normal((2, 2, 3, 4))
    z0 = np.abs(r.standard_normal((2, 2, 3))) if normalize else None
    y, _, _ = oracle.la(q, k, v, g, "elem", state_in=S0, cum_k_in=z0,
                        normalize=normalize, reverse=reverse)
    ye = quadratic_elem(q, k, v, g, S0, z0, normalize=normalize, reverse=reverse)
    np.testing.assert_allclose(y, ye, rtol=1e-12, atol=1e-12)


def test_elem_is_sum_of_one_channel_step_problems():
    q, k, v, g = rng_elem(2, T=12, Dk=4, Dv=3)
    y, s, _ = oracle.la(q, k, v, g, "elem")
    acc = np.zeros_like(y)
    for i in range(4):
        yi, si, _ = oracle.la(q[..., i:i + 1], k[..., i:i + 1], v, g[..., i], "step")
        acc += yi
        np.testing.assert_allclose(s[:, :, i:i + 1, :], si, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, acc, rtol=1e-12, atol=1e-12)


def test_elem_with_equal_channels_is_step_mode():
    q, k, v, g = rng_elem(3, positive=True)
    gs = g[..., 0]
    ge = np.repeat(gs[..., None], q.shape[-1], axis=-1)
    z0 = np.abs(np.random.default_rng(12).standard_normal((2, 2, 3)))
    a = oracle.la(q, k, v, ge, "elem", cum_k_in=z0, normalize=True)
    b = oracle.la(q, k, v, gs, "step", cum_k_in=z0, normalize=True)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)


def test_elem_split_continuation():
    q, k, v, g = rng_elem(4, T=14, positive=True)
    y, s, z = oracle.la(q, k, v, g, "elem", normalize=True)
    y1, s1, z1 = oracle.la(q[:, :, :5], k[:, :, :5], v[:, :, :5], g[:, :, :5], "elem", normalize=True)
    y2, s2, z2 = oracle.la(q[:, :, 5:], k[:, :, 5:], v[:, :, 5:], g[:, :, 5:], "elem",
                           state_in=s1, cum_k_in=z1, normalize=True)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=2), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s2, s, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(z2, z, rtol=1e-13, atol=1e-13)


def two_sided_quadratic(q, k, v, g, normalize=False):
    """sum over all s of D2[t,s] (q_t.k_s) v_s with D2[t,s] = prod of the factors
    from the step after the earlier position through the later one, and the
    diagonal (the current token, included by both directions) counted twice."""
    B, H, T, Dk = q.shape
    y = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            gg = g[b, h]
            D = np.zeros((T, T))
            for t in range(T):
                for s in range(T):
                    if s < t:
                        D[t, s] = np.prod(gg[s + 1:t + 1])
                    elif s > t:
                        D[t, s] = np.prod(gg[t:s])
                    else:
                        D[t, s] = 2.0
            A = (q[b, h] @ k[b, h].T) * D
            if normalize:
                # each direction is normalised on its own, then the two are summed
                Af, Ar = np.tril(A), np.triu(A)
                np.fill_diagonal(Af, np.diag(A) / 2)
                np.fill_diagonal(Ar, np.diag(A) / 2)
                y[b, h] = (Af @ v[b, h]) / Af.sum(1)[:, None] + (Ar @ v[b, h]) / Ar.sum(1)[:, None]
            else:
                y[b, h] = A @ v[b, h]
    return y


@pytest.mark.parametrize("mode", ["none", "head", "step"])
def test_bidirectional_matches_two_sided_quadratic_form(mode):
    r = np.random.default_rng(5)
    B, H, T, Dk, Dv = 2, 2, 8, 3, 4
    q, k, v = (r.standard_normal((B, H, T, d)) for d in (Dk, Dk, Dv))
    if mode == "none":
        dec, g = None, np.ones((B, H, T))
    elif mode == "head":
        dec = np.array([0.6, 0.9])
        g = np.broadcast_to(dec[None, :, None], (B, H, T)).copy()
    else:
        dec = g = r.uniform(0.3, 1.0, (B, H, T))
    y = oracle.la_bidirectional(q, k, v, dec, mode)
    np.testing.assert_allclose(y, two_sided_quadratic(q, k, v, g), rtol=1e-12, atol=1e-12)


def test_bidirectional_normalized_matches_two_sided_ratios():
    r = np.random.default_rng(6)
    B, H, T, Dk, Dv = 1, 2, 7, 3, 4
    q, k = (np.abs(r.standard_normal((B, H, T, Dk))) + 0.1 for _ in range(2))
    v = r.standard_normal((B, H, T, Dv))
    dec = r.uniform(0.3, 1.0, (B, H, T))
    y = oracle.la_bidirectional(q, k, v, dec, "step", normalize=True)
    np.testing.assert_allclose(y, two_sided_quadratic(q, k, v, dec, normalize=True),
                               rtol=1e-12, atol=1e-12)


def test_bidirectional_elem_matches_two_one_sided_quadratic_forms():
    q, k, v, g = rng_elem(7, T=8)
    y = oracle.la_bidirectional(q, k, v, g, "elem")
    ye = quadratic_elem(q, k, v, g) + quadratic_elem(q, k, v, g, reverse=True)
    np.testing.assert_allclose(y, ye, rtol=1e-12, atol=1e-12)


def test_ema_bidirectional_matches_two_sided_closed_form():
    r = np.random.default_rng(8)
    B, T, C = 2, 9, 3
    x = r.standard_normal((B, T, C))
    f = r.uniform(0.1, 1.0, (B, T, C))
    y = oracle.ema_bidirectional(x, f)
    ye = np.zeros_like(x)
    for t in range(T):
        for s in range(T):
            if s <= t:
                ye[:, t] += np.prod(f[:, s + 1:t + 1], axis=1) * x[:, s]
            if s >= t:
                ye[:, t] += np.prod(f[:, t:s], axis=1) * x[:, s]
    np.testing.assert_allclose(y, ye, rtol=1e-12, atol=1e-12)
