"""Pins for the fp64 linear-attention backward oracle (CPU only).

``oracle.la_backward`` applies the chain rule to the recurrence in reverse
order.  It is trusted because of checks from outside that loop:

* torch autograd, in float64, through an explicit parallel form of the
  forward pass written here (decay products built with torch.prod, the
  initial state and the final state as separate terms), for every decay mode,
  both time orders, with an initial state and a final-state gradient;
* central finite differences of the (separately pinned) forward oracle along
  random directions of every input;
* the flip invariant: the backward of the reversed call is the flipped
  backward of the forward call on flipped inputs.
"""
import numpy as np
import pytest
import torch

import oracle


def rng(seed, B=2, H=2, T=7, Dk=3, Dv=4, mode="step"):
    r = np.random.default_rng(seed)
    q, k = r.standard_normal((B, H, T, Dk)), r.standard_normal((B, H, T, Dk))
    v, dy = r.standard_normal((B, H, T, Dv)), r.standard_normal((B, H, T, Dv))
    S0, dSf = r.standard_normal((B, H, Dk, Dv)), r.standard_normal((B, H, Dk, Dv))
    g = {"none": None, "head": r.uniform(0.4, 0.95, H), "step": r.uniform(0.4, 0.95, (B, H, T)),
         "elem": r.uniform(0.4, 0.95, (B, H, T, Dk))}[mode]
    return q, k, v, dy, S0, dSf, g


def per_step_factors(g, mode, B, H, T, Dk):
    """[B,H,T,Dk] factor of each step and key row (differentiable in g)."""
    if mode == "none":
        return torch.ones(B, H, T, Dk, dtype=torch.float64)
    if mode == "head":
        return g[None, :, None, None].expand(B, H, T, Dk)
    if mode == "step":
        return g[..., None].expand(B, H, T, Dk)
    return g


def explicit_forward(q, k, v, G, S0):
    """y_t = sum_{s<=t} sum_i q_t[i] k_s[i] prod_{s<r<=t} G_r[i] v_s + (q_t * P_t) S0,
    S_final = sum_s (k_s * prod_{s<r<T} G_r) v_s^T + P_{T-1} * S0 (rows)."""
    B, H, T, Dk = q.shape
    ys, Sf = [], []
    for b in range(B):
        yb, Sb = [], []
        for h in range(H):
            rows = []
            for t in range(T):
                acc = (q[b, h, t] * torch.prod(G[b, h, :t + 1], dim=0)) @ S0[b, h]
                for s in range(t + 1):
                    dec = torch.prod(G[b, h, s + 1:t + 1], dim=0) if s < t else torch.ones(Dk, dtype=q.dtype)
                    acc = acc + torch.sum(q[b, h, t] * k[b, h, s] * dec) * v[b, h, s]
                rows.append(acc)
            yb.append(torch.stack(rows))
            S = torch.prod(G[b, h], dim=0)[:, None] * S0[b, h]
            for s in range(T):
                dec = torch.prod(G[b, h, s + 1:], dim=0) if s < T - 1 else torch.ones(Dk, dtype=q.dtype)
                S = S + torch.outer(k[b, h, s] * dec, v[b, h, s])
            Sb.append(S)
        ys.append(torch.stack(yb))
        Sf.append(torch.stack(Sb))
    return torch.stack(ys), torch.stack(Sf)


def autograd_reference(q, k, v, dy, S0, dSf, g, mode, reverse):
    B, H, T, Dk = q.shape
    leaves = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, S0)]
    gt = None if g is None else torch.tensor(g, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tS0 = leaves
    G = per_step_factors(gt, mode, B, H, T, Dk)
    flip = (lambda x: torch.flip(x, dims=[2])) if reverse else (lambda x: x)
    y, Sf = explicit_forward(flip(tq), flip(tk), flip(tv), flip(G), tS0)
    y = flip(y)
    L = torch.sum(y * torch.tensor(dy)) + torch.sum(Sf * torch.tensor(dSf))
    L.backward()
    out = [x.grad.numpy() for x in (tq, tk, tv)]
    out.append(None if gt is None else gt.grad.numpy())
    out.append(tS0.grad.numpy())
    return out


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mode", ["none", "head", "step", "elem"])
def test_matches_autograd_of_explicit_form(mode, reverse):
    q, k, v, dy, S0, dSf, g = rng(1, mode=mode)
    got = oracle.la_backward(q, k, v, dy, g, mode, S0, dSf, reverse=reverse)
    want = autograd_reference(q, k, v, dy, S0, dSf, g, mode, reverse)
    for name, a, b in zip(("dq", "dk", "dv", "dgamma", "dstate_in"), got, want):
        if b is None:
            assert a is None
            continue
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11, err_msg=name)


def loss(q, k, v, g, mode, S0, dy, dSf, reverse):
    y, S, _ = oracle.la(q, k, v, g, mode, S0, reverse=reverse)
    return float(np.sum(y * dy) + np.sum(S * dSf))


@pytest.mark.parametrize("mode,reverse", [("head", False), ("step", True), ("elem", False)])
def test_directional_finite_differences_of_the_forward_oracle(mode, reverse):
    q, k, v, dy, S0, dSf, g = rng(2, T=9, mode=mode)
    grads = oracle.la_backward(q, k, v, dy, g, mode, S0, dSf, reverse=reverse)
    r = np.random.default_rng(3)
    eps = 1e-6
    args = [q, k, v, g, S0]       # grads come back in the same order: dq, dk, dv, dgamma, dstate_in
    for a in range(len(args)):
        d = r.standard_normal(args[a].shape)
        plus = [x.copy() for x in args]
        minus = [x.copy() for x in args]
        plus[a] = plus[a] + eps * d
        minus[a] = minus[a] - eps * d
        fd = (loss(plus[0], plus[1], plus[2], plus[3], mode, plus[4], dy, dSf, reverse)
              - loss(minus[0], minus[1], minus[2], minus[3], mode, minus[4], dy, dSf, reverse)) / (2 * eps)
        an = float(np.sum(grads[a] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (a, fd, an)


def test_reverse_is_flipped_forward_backward():
    q, k, v, dy, S0, dSf, g = rng(4, T=8, mode="step")
    f = lambda x: np.ascontiguousarray(x[:, :, ::-1])
    a = oracle.la_backward(q, k, v, dy, g, "step", S0, dSf, reverse=True)
    b = oracle.la_backward(f(q), f(k), f(v), f(dy), f(g), "step", S0, dSf, reverse=False)
    for x, y in zip(a[:4], b[:4]):
        np.testing.assert_allclose(x, f(y), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(a[4], b[4], rtol=1e-13, atol=1e-13)


def test_no_state_terms_when_absent():
    """Without an initial state and a final-state gradient, the per-step decay
    gradient of the first visited step is zero (its factor scales a zero state)."""
    q, k, v, dy, _, _, g = rng(5, mode="step")
    _, _, _, dg, ds0 = oracle.la_backward(q, k, v, dy, g, "step")
    np.testing.assert_array_equal(dg[:, :, 0], 0.0)
    assert np.abs(ds0).max() > 0      # the initial state still receives a gradient


# ---------------------------------------------------------------------------
# the normalised form (flash-linear-attention issue #268: y = QKV / QK1 with a
# carried key sum): y_t = q_t^T S_t / q_t^T z_t
# ---------------------------------------------------------------------------

def rng_norm(seed, B=2, H=2, T=7, Dk=3, Dv=4, mode="step"):
    """Positive queries, keys and key sum (the page's feature-mapped attention), so
    the denominators stay away from zero."""
    r = np.random.default_rng(seed)
    q, k = r.uniform(0.2, 1.5, (B, H, T, Dk)), r.uniform(0.2, 1.5, (B, H, T, Dk))
    v, dy = r.standard_normal((B, H, T, Dv)), r.standard_normal((B, H, T, Dv))
    S0, dSf = r.standard_normal((B, H, Dk, Dv)), r.standard_normal((B, H, Dk, Dv))
    z0, dzf = r.uniform(0.5, 2.0, (B, H, Dk)), r.standard_normal((B, H, Dk))
    g = {"none": None, "head": r.uniform(0.4, 0.95, H), "step": r.uniform(0.4, 0.95, (B, H, T)),
         "elem": r.uniform(0.4, 0.95, (B, H, T, Dk))}[mode]
    return q, k, v, dy, S0, dSf, z0, dzf, g


def autograd_reference_norm(q, k, v, dy, S0, dSf, z0, dzf, g, mode, reverse):
    """Autograd of the ratio of two explicit parallel forms: the numerator with the
    values, the denominator with a single value channel of ones and the key sum as
    its initial state."""
    B, H, T, Dk = q.shape
    leaves = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, S0, z0)]
    gt = None if g is None else torch.tensor(g, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tS0, tz0 = leaves
    G = per_step_factors(gt, mode, B, H, T, Dk)
    flip = (lambda x: torch.flip(x, dims=[2])) if reverse else (lambda x: x)
    num, Sf = explicit_forward(flip(tq), flip(tk), flip(tv), flip(G), tS0)
    ones = torch.ones(B, H, T, 1, dtype=torch.float64)
    den, zf = explicit_forward(flip(tq), flip(tk), ones, flip(G), tz0[..., None])
    y = flip(num / den)
    L = torch.sum(y * torch.tensor(dy)) + torch.sum(Sf * torch.tensor(dSf)) + torch.sum(zf[..., 0] * torch.tensor(dzf))
    L.backward()
    out = [x.grad.numpy() for x in (tq, tk, tv)]
    out.append(None if gt is None else gt.grad.numpy())
    out += [tS0.grad.numpy(), tz0.grad.numpy()]
    return out


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mode", ["none", "head", "step", "elem"])
def test_normalized_matches_autograd_of_ratio_form(mode, reverse):
    q, k, v, dy, S0, dSf, z0, dzf, g = rng_norm(11, mode=mode)
    got = oracle.la_backward(q, k, v, dy, g, mode, S0, dSf, reverse=reverse, normalize=True,
                             cum_k_in=z0, dcum_k_out=dzf)
    want = autograd_reference_norm(q, k, v, dy, S0, dSf, z0, dzf, g, mode, reverse)
    for name, a, b in zip(("dq", "dk", "dv", "dgamma", "dstate_in", "dcum_k_in"), got, want):
        if b is None:
            assert a is None
            continue
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)


def loss_norm(q, k, v, g, mode, S0, z0, dy, dSf, dzf, reverse):
    y, S, z = oracle.la(q, k, v, g, mode, S0, z0, reverse=reverse, normalize=True)
    return float(np.sum(y * dy) + np.sum(S * dSf) + np.sum(z * dzf))


@pytest.mark.parametrize("mode,reverse", [("head", True), ("step", False), ("elem", True), ("none", False)])
def test_normalized_directional_finite_differences(mode, reverse):
    q, k, v, dy, S0, dSf, z0, dzf, g = rng_norm(12, T=9, mode=mode)
    grads = oracle.la_backward(q, k, v, dy, g, mode, S0, dSf, reverse=reverse, normalize=True,
                               cum_k_in=z0, dcum_k_out=dzf)
    r = np.random.default_rng(13)
    eps = 1e-6
    args = [q, k, v, g, S0, z0]   # the gradients come back in this order
    for a in range(len(args)):
        if args[a] is None:
            continue
        d = r.standard_normal(args[a].shape)
        plus = [None if x is None else x.copy() for x in args]
        minus = [None if x is None else x.copy() for x in args]
        plus[a] = plus[a] + eps * d
        minus[a] = minus[a] - eps * d
        fd = (loss_norm(plus[0], plus[1], plus[2], plus[3], mode, plus[4], plus[5], dy, dSf, dzf, reverse)
              - loss_norm(minus[0], minus[1], minus[2], minus[3], mode, minus[4], minus[5], dy, dSf, dzf,
                          reverse)) / (2 * eps)
        an = float(np.sum(grads[a] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (a, fd, an)


def test_normalized_query_gradient_is_orthogonal_to_the_query():
    """y_t does not change when q_t is scaled, so q_t . dq_t = 0 at every step."""
    q, k, v, dy, S0, dSf, z0, dzf, g = rng_norm(14, T=11, mode="step")
    dq = oracle.la_backward(q, k, v, dy, g, "step", S0, dSf, normalize=True, cum_k_in=z0, dcum_k_out=dzf)[0]
    assert np.abs(dq).max() > 1e-3
    np.testing.assert_allclose(np.sum(q * dq, axis=-1), 0.0, atol=1e-12)


@pytest.mark.parametrize("mode", ["head", "elem"])
def test_normalized_joint_key_scaling_identity(mode):
    """Scaling k, S0 and z0 together by a leaves every y_t unchanged and scales the
    final state and key sum by a, so  sum k.dk + <S0, dS0> + <z0, dz0> equals
    <dS_final, S_final> + <dz_final, z_final>."""
    q, k, v, dy, S0, dSf, z0, dzf, g = rng_norm(15, T=10, mode=mode)
    dq, dk, dv, dg, dS0, dz0 = oracle.la_backward(q, k, v, dy, g, mode, S0, dSf, normalize=True,
                                                  cum_k_in=z0, dcum_k_out=dzf)
    _, Sf, zf = oracle.la(q, k, v, g, mode, S0, z0, normalize=True)
    lhs = np.sum(k * dk) + np.sum(S0 * dS0) + np.sum(z0 * dz0)
    rhs = np.sum(dSf * Sf) + np.sum(dzf * zf)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def test_normalized_equal_values_give_no_query_key_or_decay_gradient():
    """All values equal to c and S0 = z0 c^T: every output is c whatever q, k and the
    factors are, so their gradients vanish (the values' do not)."""
    q, k, v, dy, _, _, z0, _, g = rng_norm(16, T=9, mode="elem")
    c = np.array([0.7, -1.3, 2.0, 0.1])
    v = np.broadcast_to(c, v.shape).copy()
    S0 = z0[..., None] * c
    dq, dk, dv, dg, dS0, dz0 = oracle.la_backward(q, k, v, dy, g, "elem", S0, normalize=True, cum_k_in=z0)
    for name, x in (("dq", dq), ("dk", dk), ("dgamma", dg)):
        np.testing.assert_allclose(x, 0.0, atol=1e-12, err_msg=name)
    assert np.abs(dv).max() > 1e-3


def test_normalized_reverse_is_flipped_forward_backward():
    q, k, v, dy, S0, dSf, z0, dzf, g = rng_norm(17, T=8, mode="step")
    f = lambda x: np.ascontiguousarray(x[:, :, ::-1])
    a = oracle.la_backward(q, k, v, dy, g, "step", S0, dSf, reverse=True, normalize=True, cum_k_in=z0,
                           dcum_k_out=dzf)
    b = oracle.la_backward(f(q), f(k), f(v), f(dy), f(g), "step", S0, dSf, reverse=False, normalize=True,
                           cum_k_in=z0, dcum_k_out=dzf)
    for x, y in zip(a[:4], b[:4]):
        np.testing.assert_allclose(x, f(y), rtol=1e-13, atol=1e-13)
    for x, y in zip(a[4:], b[4:]):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)
