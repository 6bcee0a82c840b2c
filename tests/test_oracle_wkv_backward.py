"""Pins for the fp64 WKV backward oracle (CPU only).

``oracle.wkv_backward`` runs the chain rule through the linear form of the
recurrence in reverse order.  It is trusted because of checks from outside
that loop:

* torch autograd, in float64, through the closed form of the output
  (RWKV-LM discussion #189 / issue #167: numerator and denominator as decayed,
  key-weighted sums over the earlier tokens plus the current token with the
  bonus u), written here with explicit powers of the decay;
* central finite differences of the (separately pinned) forward oracle along
  random directions of w, u, k and v;
* special cases: with one token and no state the output is v itself, so the
  gradients of k, u and w vanish and dv = dy.

The carried state's gradient (the planes aa, bb, pp) is pinned the same two
ways, and by an invariance: rescaling the state's representation (aa, bb, pp) ->
(aa e^c, bb e^c, pp - c) leaves every output unchanged, so the gradient is
orthogonal to that direction: d aa * aa + d bb * bb - d pp = 0.
"""
import numpy as np
import pytest
import torch

import oracle


def rng(seed, B=2, T=8, C=3, state=True):
    r = np.random.default_rng(seed)
    w = -np.exp(r.normal(0, 0.5, C))
    u = r.normal(0, 1, C)
    k = r.normal(0, 2, (B, T, C))
    v = r.normal(0, 1, (B, T, C))
    dy = r.normal(0, 1, (B, T, C))
    s0 = None
    if state:
        s0 = np.stack([r.normal(0, 1, (B, C)), np.abs(r.normal(0, 1, (B, C))) + 0.5, r.normal(0, 1, (B, C))])
    return w, u, k, v, dy, s0


def closed_form_torch(w, u, k, v, s0):
    B, T, C = k.shape
    ys = []
    for t in range(T):
        num = torch.zeros(B, C, dtype=torch.float64)
        den = torch.zeros(B, C, dtype=torch.float64)
        if s0 is not None:
            num = num + torch.exp(s0[2] + t * w) * s0[0]
            den = den + torch.exp(s0[2] + t * w) * s0[1]
        for i in range(t):
            f = torch.exp((t - 1 - i) * w + k[:, i])
            num = num + f * v[:, i]
            den = den + f
        cur = torch.exp(u + k[:, t])
        ys.append((num + cur * v[:, t]) / (den + cur))
    return torch.stack(ys, dim=1)


@pytest.mark.parametrize("state", [False, True])
def test_matches_autograd_of_closed_form(state):
    w, u, k, v, dy, s0 = rng(1, state=state)
    tw, tu, tk, tv = (torch.tensor(x, requires_grad=True) for x in (w, u, k, v))
    ts0 = None if s0 is None else torch.tensor(s0)
    y = closed_form_torch(tw, tu, tk, tv, ts0)
    torch.sum(y * torch.tensor(dy)).backward()
    got = oracle.wkv_backward(w, u, k, v, dy, s0)
    for name, a, b in zip(("dw", "du", "dk", "dv"), got, (tw.grad, tu.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_directional_finite_differences_of_the_forward_oracle():
    w, u, k, v, dy, s0 = rng(2, T=11, C=4)
    grads = oracle.wkv_backward(w, u, k, v, dy, s0)
    r = np.random.default_rng(3)
    eps = 1e-6
    args = [w, u, k, v]
    for a in range(4):
        d = r.standard_normal(args[a].shape)
        plus = [x.copy() for x in args]
        minus = [x.copy() for x in args]
        plus[a] = plus[a] + eps * d
        minus[a] = minus[a] - eps * d
        lp = np.sum(oracle.wkv(*plus, state_in=s0)[0] * dy)
        lm = np.sum(oracle.wkv(*minus, state_in=s0)[0] * dy)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(grads[a] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (a, fd, an)


def test_state_gradient_matches_autograd_of_closed_form():
    w, u, k, v, dy, s0 = rng(5)
    ts0 = torch.tensor(s0, requires_grad=True)
    y = closed_form_torch(*(torch.tensor(x) for x in (w, u, k, v)), ts0)
    torch.sum(y * torch.tensor(dy)).backward()
    *_, ds = oracle.wkv_backward(w, u, k, v, dy, s0, return_dstate=True)
    np.testing.assert_allclose(ds, ts0.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_state_gradient_finite_differences_and_representation_invariance():
    w, u, k, v, dy, s0 = rng(6, T=9, C=5)
    *_, ds = oracle.wkv_backward(w, u, k, v, dy, s0, return_dstate=True)
    eps = 1e-6
    for plane in range(3):
        d = np.random.default_rng(7 + plane).standard_normal(s0[plane].shape)
        sp, sm = s0.copy(), s0.copy()
        sp[plane] += eps * d
        sm[plane] -= eps * d
        fd = (np.sum(oracle.wkv(w, u, k, v, sp)[0] * dy) - np.sum(oracle.wkv(w, u, k, v, sm)[0] * dy)) / (2 * eps)
        an = float(np.sum(ds[plane] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (plane, fd, an)
    np.testing.assert_allclose(ds[0] * s0[0] + ds[1] * s0[1], ds[2], rtol=1e-12, atol=1e-13)


def test_state_gradient_without_state_is_zero():
    w, u, k, v, dy, _ = rng(8, state=False)
    *_, ds = oracle.wkv_backward(w, u, k, v, dy, None, return_dstate=True)
    np.testing.assert_array_equal(ds, 0.0)


def test_single_token_without_state():
    w, u, k, v, dy, _ = rng(4, T=1, state=False)
    dw, du, dk, dv = oracle.wkv_backward(w, u, k, v, dy)
    np.testing.assert_allclose(dv, dy, rtol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(du, 0.0, atol=1e-14)
    np.testing.assert_allclose(dw, 0.0, atol=1e-14)
