"""Pins for the fp64 linear-attention oracle (CPU only).

The oracle is trusted only because of these checks, each of which comes from
outside the oracle's own recurrence:

* the worked examples printed on the tensortonic "cs336 linear attention
  duality" exercise page (exact small integers, ``tests/golden``);
* the parallel (quadratic) form that page requires to equal the recurrent
  one, generalised with the decay-mask D of RetNet issue #21, built here with
  explicit products, for causal and anti-causal (reverse) orders;
* a hand-worked decay example that fixes which factor multiplies what
  (cumulative_ema docstring in RetNet issue #21);
* invariants: reverse == flip . forward . flip, split/continuation through the
  carried state and key sum (flash-linear-attention issue #268), scale
  invariance of the normalised output;
* special cases: gamma == 1 is the plain cumulative sum (numpy.cumsum of the
  outer products, the page's hint), gamma_t == 0 restarts the state, equal
  keys turn the normalised output into a running mean of v.

Every random case uses Dk != Dv and non-symmetric data so that a transposed
operand, a dropped term or an off-by-one decay index fails at least one test.
"""
import json

import numpy as np
import pytest

import oracle
from decayed_recurrence_scans_amd import workloads as wl


def rng_inputs(seed, B=2, H=3, T=9, Dk=3, Dv=5, positive=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, Dk))
    k = r.standard_normal((B, H, T, Dk))
    v = r.standard_normal((B, H, T, Dv))
    if positive:
        q = np.abs(q) + 0.1
        k = np.abs(k) + 0.1
    return q, k, v


def gammas_for(mode, decay, B, H, T):
    """Per-(b,h,t) decay factor array for the explicit quadratic forms."""
    if mode == "none":
        return np.ones((B, H, T))
    if mode == "head":
        return np.broadcast_to(np.asarray(decay)[None, :, None], (B, H, T)).copy()
    return np.asarray(decay, dtype=np.float64)


def quadratic_forward(q, k, v, g, S0=None, z0=None, normalize=False):
    """Causal parallel form: y_t = sum_{s<=t} D[t,s] (q_t.k_s) v_s + P_t q_t S0,
    D[t,s] = prod_{r=s+1..t} g_r, P_t = prod_{r=0..t} g_r (explicit products)."""
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    y = np.zeros((B, H, T, Dv))
    S = np.zeros((B, H, Dk, Dv))
    Z = np.zeros((B, H, Dk))
    for b in range(B):
        for h in range(H):
            gg = g[b, h]
            D = np.zeros((T, T))
            for t in range(T):
                for s in range(t + 1):
                    D[t, s] = np.prod(gg[s + 1:t + 1])
            P = np.array([np.prod(gg[:t + 1]) for t in range(T)])
            A = (q[b, h] @ k[b, h].T) * D
            num = A @ v[b, h]
            den = A.sum(axis=1)
            if S0 is not None:
                num = num + P[:, None] * (q[b, h] @ S0[b, h])
            if z0 is not None:
                den = den + P * (q[b, h] @ z0[b, h])
            y[b, h] = num / den[:, None] if normalize else num
            S[b, h] = (D[T - 1][:, None] * k[b, h]).T @ v[b, h]
            Z[b, h] = (D[T - 1][:, None] * k[b, h]).sum(axis=0)
            if S0 is not None:
                S[b, h] += P[T - 1] * S0[b, h]
            if z0 is not None:
                Z[b, h] += P[T - 1] * z0[b, h]
    return y, S, Z


def quadratic_reverse(q, k, v, g, S0=None):
    """Anti-causal parallel form of the reversed scan:
    S_t = g_t S_{t+1} + k_t v_t^T  =>  y_t = sum_{s>=t} (prod_{r=t..s-1} g_r)(q_t.k_s) v_s
    + (prod_{r=t..T-1} g_r) q_t S0."""
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    y = np.zeros((B, H, T, Dv))
    S = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            gg = g[b, h]
            D = np.zeros((T, T))
            for t in range(T):
                for s in range(t, T):
                    D[t, s] = np.prod(gg[t:s])
            P = np.array([np.prod(gg[t:]) for t in range(T)])
            y[b, h] = ((q[b, h] @ k[b, h].T) * D) @ v[b, h]
            S[b, h] = (D[0][:, None] * k[b, h]).T @ v[b, h]
            if S0 is not None:
                y[b, h] += P[:, None] * (q[b, h] @ S0[b, h])
                S[b, h] += P[0] * S0[b, h]
    return y, S


# --------------------------------------------------------------------------
# worked examples printed on the exercise page
# --------------------------------------------------------------------------

def test_worked_examples_exact(golden_dir):
    data = json.loads((golden_dir / "la_worked_examples.json").read_text())
    assert len(data["examples"]) == 3
    for ex in data["examples"]:
        q = np.array(ex["q"], float)[:, None]     # (B,S,D) -> (B,1,S,D)
        k = np.array(ex["k"], float)[:, None]
        v = np.array(ex["v"], float)[:, None]
        y, S, _ = oracle.la(q, k, v)
        assert np.array_equal(y[:, 0], np.array(ex["output"], float))
        assert np.array_equal(S[:, 0], np.array(ex["final_state"], float))
        # parallel form (the page states both forms give the same output)
        yq, Sq, _ = quadratic_forward(q, k, v, np.ones(q.shape[:3]))
        assert np.array_equal(yq[:, 0], np.array(ex["output"], float))
        if "states_after_each_write" in ex:
            for T, want in enumerate(ex["states_after_each_write"], start=1):
                _, St, _ = oracle.la(q[:, :, :T], k[:, :, :T], v[:, :, :T])
                assert St.ravel()[0] == want


# --------------------------------------------------------------------------
# parallel (quadratic) forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["none", "head", "step"])
@pytest.mark.parametrize("with_state", [False, True])
def test_matches_causal_quadratic_form(mode, with_state):
    B, H, T, Dk, Dv = 2, 3, 9, 3, 5
    q, k, v = rng_inputs(10 + with_state, B, H, T, Dk, Dv)
    r = np.random.default_rng(99)
    decay = {"none": None, "head": r.uniform(0.3, 1.0, H),
             "step": r.uniform(0.2, 1.0, (B, H, T))}[mode]
    S0 = r.standard_normal((B, H, Dk, Dv)) if with_state else None
    y, S, _ = oracle.la(q, k, v, decay, mode, state_in=S0)
    yq, Sq, _ = quadratic_forward(q, k, v, gammas_for(mode, decay, B, H, T), S0)
    np.testing.assert_allclose(y, yq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sq, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["none", "head", "step"])
def test_reverse_matches_anticausal_quadratic_form(mode):
    B, H, T, Dk, Dv = 2, 2, 8, 4, 3
    q, k, v = rng_inputs(20, B, H, T, Dk, Dv)
    r = np.random.default_rng(21)
    decay = {"none": None, "head": r.uniform(0.3, 1.0, H),
             "step": r.uniform(0.2, 1.0, (B, H, T))}[mode]
    S0 = r.standard_normal((B, H, Dk, Dv))
    y, S, _ = oracle.la(q, k, v, decay, mode, state_in=S0, reverse=True)
    yq, Sq = quadratic_reverse(q, k, v, gammas_for(mode, decay, B, H, T), S0)
    np.testing.assert_allclose(y, yq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sq, rtol=1e-12, atol=1e-12)


def test_normalized_matches_quadratic_ratio():
    """QKV / QK1 (flash-linear-attention issue #268) with a cached state and key sum."""
    B, H, T, Dk, Dv = 2, 2, 11, 4, 6
    q, k, v = rng_inputs(30, B, H, T, Dk, Dv, positive=True)
    r = np.random.default_rng(31)
    S0 = r.standard_normal((B, H, Dk, Dv))
    z0 = np.abs(r.standard_normal((B, H, Dk))) + 1.0
    for mode, decay in [("none", None), ("step", r.uniform(0.5, 1.0, (B, H, T)))]:
        y, S, Z = oracle.la(q, k, v, decay, mode, S0, z0, normalize=True)
        yq, Sq, Zq = quadratic_forward(q, k, v, gammas_for(mode, decay, B, H, T), S0, z0,
                                       normalize=True)
        np.testing.assert_allclose(y, yq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, Sq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Z, Zq, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# index convention of the decay factor, worked by hand
# --------------------------------------------------------------------------

def test_decay_convention_by_hand():
    # gamma_t multiplies the state carried in from the previous visited step;
    # the first visited step's gamma multiplies state_in.
    q = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    k = np.ones((1, 1, 3, 1))
    v = np.array([1.0, 2.0, 4.0]).reshape(1, 1, 3, 1)
    g = np.array([0.5, 0.5, 0.25]).reshape(1, 1, 3)
    S0 = np.array([8.0]).reshape(1, 1, 1, 1)
    # forward: S = .5*8+1 = 5 ; .5*5+2 = 4.5 ; .25*4.5+4 = 5.125
    y, S, _ = oracle.la(q, k, v, g, "step", state_in=S0)
    assert y.ravel().tolist() == [5.0, 9.0, 15.375]
    assert S.ravel().tolist() == [5.125]
    # reverse: S = .25*8+4 = 6 (t=2) ; .5*6+2 = 5 (t=1) ; .5*5+1 = 3.5 (t=0)
    y, S, _ = oracle.la(q, k, v, g, "step", state_in=S0, reverse=True)
    assert y.ravel().tolist() == [3.5, 10.0, 18.0]
    assert S.ravel().tolist() == [3.5]


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("mode", ["none", "head", "step"])
def test_reverse_is_flip_forward_flip(mode, normalize):
    B, H, T, Dk, Dv = 2, 2, 13, 5, 3
    q, k, v = rng_inputs(40, B, H, T, Dk, Dv, positive=normalize)
    r = np.random.default_rng(41)
    decay = {"none": None, "head": r.uniform(0.3, 1.0, H),
             "step": r.uniform(0.2, 1.0, (B, H, T))}[mode]
    S0 = r.standard_normal((B, H, Dk, Dv))
    z0 = np.abs(r.standard_normal((B, H, Dk))) + 1 if normalize else None
    yr, Sr, Zr = oracle.la(q, k, v, decay, mode, S0, z0, reverse=True, normalize=normalize)
    f = lambda x: np.ascontiguousarray(np.flip(x, axis=2))
    fd = f(decay) if mode == "step" else decay
    yf, Sf, Zf = oracle.la(f(q), f(k), f(v), fd, mode, S0, z0, normalize=normalize)
    np.testing.assert_array_equal(yr, f(yf))
    np.testing.assert_array_equal(Sr, Sf)
    if normalize:
        np.testing.assert_array_equal(Zr, Zf)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("normalize", [False, True])
def test_split_continuation(normalize, reverse):
    """Running [0,T) in one call equals two calls chained through state and key sum."""
    B, H, T, Dk, Dv, T1 = 2, 2, 17, 4, 6, 7
    q, k, v = rng_inputs(50, B, H, T, Dk, Dv, positive=normalize)
    g = np.random.default_rng(51).uniform(0.4, 1.0, (B, H, T))
    y, S, Z = oracle.la(q, k, v, g, "step", normalize=normalize, reverse=reverse)
    first = slice(T1, T) if reverse else slice(0, T1)
    second = slice(0, T1) if reverse else slice(T1, T)
    c = lambda x, s: np.ascontiguousarray(x[:, :, s])
    ya, Sa, Za = oracle.la(c(q, first), c(k, first), c(v, first), c(g, first), "step",
                           normalize=normalize, reverse=reverse)
    yb, Sb, Zb = oracle.la(c(q, second), c(k, second), c(v, second), c(g, second), "step",
                           Sa, Za, normalize=normalize, reverse=reverse)
    np.testing.assert_allclose(y[:, :, first], ya, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[:, :, second], yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sb, rtol=1e-12, atol=1e-12)
    if normalize:
        np.testing.assert_allclose(Z, Zb, rtol=1e-12, atol=1e-12)


def test_normalized_scale_invariance():
    q, k, v = rng_inputs(60, positive=True)
    y1, _, _ = oracle.la(q, k, v, normalize=True)
    y2, _, _ = oracle.la(3.75 * q, k, v, normalize=True)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)


def test_normalized_equal_keys_is_running_mean():
    B, H, T, Dk, Dv = 1, 2, 10, 4, 3
    r = np.random.default_rng(70)
    q = np.abs(r.standard_normal((B, H, T, Dk))) + 0.2
    k = np.broadcast_to(np.abs(r.standard_normal((1, 1, 1, Dk))) + 0.5, (B, H, T, Dk)).copy()
    v = r.standard_normal((B, H, T, Dv))
    y, _, _ = oracle.la(q, k, v, normalize=True)
    mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(y, mean, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------

def test_unit_decay_is_plain_cumsum():
    B, H, T, Dk, Dv = 2, 2, 9, 3, 4
    q, k, v = rng_inputs(80, B, H, T, Dk, Dv)
    outer = k[..., :, None] * v[..., None, :]          # [B,H,T,Dk,Dv]
    S_all = np.cumsum(outer, axis=2)
    y_ref = np.einsum("bhtd,bhtde->bhte", q, S_all)
    for mode, decay in [("none", None), ("head", np.ones(H)), ("step", np.ones((B, H, T)))]:
        y, S, _ = oracle.la(q, k, v, decay, mode)
        np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, S_all[:, :, -1], rtol=1e-12, atol=1e-12)


def test_zero_decay_restarts_state():
    B, H, T, Dk, Dv = 1, 1, 6, 3, 2
    q, k, v = rng_inputs(90, B, H, T, Dk, Dv)
    g = np.full((B, H, T), 0.7)
    g[0, 0, 3] = 0.0
    S0 = np.random.default_rng(91).standard_normal((B, H, Dk, Dv))
    _, S3, _ = oracle.la(q[:, :, :4], k[:, :, :4], v[:, :, :4], g[:, :, :4], "step", S0)
    np.testing.assert_array_equal(S3[0, 0], np.outer(k[0, 0, 3], v[0, 0, 3]))
    y, _, _ = oracle.la(q, k, v, g, "step", S0)
    y_tail, _, _ = oracle.la(q[:, :, 3:], k[:, :, 3:], v[:, :, 3:], g[:, :, 3:], "step")
    np.testing.assert_allclose(y[:, :, 3:], y_tail, rtol=1e-13, atol=1e-13)


def test_thread_count_does_not_change_results():
    q, k, v = rng_inputs(95, B=3, H=4, T=20, Dk=5, Dv=7)
    g = np.random.default_rng(96).uniform(0.5, 1, (3, 4, 20))
    a = oracle.la(q, k, v, g, "step", threads=1)
    b = oracle.la(q, k, v, g, "step", threads=4)
    for x, y in zip(a[:2], b[:2]):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------
# the continuation workload's synthetic state
# --------------------------------------------------------------------------

def test_carried_state_workload_equals_concatenation():
    """S0/cum_k0 summed over the prefix, then continued, equals the tail of the
    plain run over prefix+segment (flash-linear-attention issue #268: the
    cached key sum plus the running sum of the new keys)."""
    B, H, T, Dk, Dv, P = 2, 2, 12, 8, 6, 20
    inp = wl.la_inputs(B, H, T, Dk, Dv, dtype="bf16", normalize=True, dist="elu1",
                       seed=7, prefix=P, return_prefix=True)
    y, S, Z = oracle.la(inp["q"], inp["k"], inp["v"], state_in=inp["state_in"],
                        cum_k_in=inp["cum_k_in"], normalize=True)
    qp = np.ones((B, H, P, Dk))
    cat = lambda a, b: np.concatenate([np.asarray(a.double()) if hasattr(a, "double") else a,
                                       np.asarray(b.double())], axis=2)
    yc, Sc, Zc = oracle.la(cat(qp, inp["q"]), cat(inp["prefix_k"], inp["k"]),
                           cat(inp["prefix_v"], inp["v"]), normalize=True)
    # S0 and cum_k0 were rounded to fp32 once; allow that rounding only
    np.testing.assert_allclose(y, yc[:, :, P:], rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(S, Sc, rtol=2e-6, atol=2e-5)
    np.testing.assert_allclose(Z, Zc, rtol=2e-6, atol=2e-5)
