"""Pins for the fp64 WKV oracle (CPU only).

The max-shifted recurrence quoted in RWKV-LM issue #167 computes, exactly up
to rounding, a plain weighted average.  Unrolled, with the state (aa, bb, pp)
standing for aa*e^pp and bb*e^pp:

    y_t = [e^{pp0 + t w} aa0 + sum_{i<t} e^{(t-1-i) w + k_i} v_i + e^{u + k_t} v_t]
        / [e^{pp0 + t w} bb0 + sum_{i<t} e^{(t-1-i) w + k_i}     + e^{u + k_t}    ]

The tests pin the oracle against that closed form (evaluated here directly,
O(T^2), with one common shift per output), against the scaled cumulative-sum
form of RWKV-LM discussion #189 where it does not overflow, against special
cases with textbook answers, against the split/continuation invariant, and
they check the segment-summary combine used by the time-parallel path.
"""
import numpy as np
import pytest

import oracle


def rand_case(seed, B=2, T=9, C=5, state=False, kscale=2.0):
    r = np.random.default_rng(seed)
    w = -np.exp(r.standard_normal(C))
    u = r.standard_normal(C)
    k = r.standard_normal((B, T, C)) * kscale
    v = r.standard_normal((B, T, C))
    s0 = None
    if state:
        s0 = np.stack([r.standard_normal((B, C)), np.abs(r.standard_normal((B, C))) + 0.3,
                       r.standard_normal((B, C)) * 3])
    return w, u, k, v, s0


def closed_form(w, u, k, v, s0=None):
    """Direct evaluation of the weighted average and of the canonical end state."""
    B, T, C = k.shape
    y = np.zeros((B, T, C))
    st = np.zeros((3, B, C))
    for b in range(B):
        for c in range(C):
            kk, vv, ww, uu = k[b, :, c], v[b, :, c], w[c], u[c]
            for t in range(T + 1):
                expo, num_w, den_w = [], [], []
                if s0 is not None:
                    expo.append(s0[2, b, c] + t * ww)
                    num_w.append(s0[0, b, c])
                    den_w.append(s0[1, b, c])
                for i in range(t):
                    expo.append((t - 1 - i) * ww + kk[i])
                    num_w.append(vv[i])
                    den_w.append(1.0)
                if t < T:
                    expo.append(uu + kk[t])
                    num_w.append(vv[t])
                    den_w.append(1.0)
                e = np.array(expo)
                m = e.max()
                f = np.exp(e - m)
                if t < T:
                    y[b, t, c] = (f @ np.array(num_w)) / (f @ np.array(den_w))
                else:  # end state, represented at the canonical scale m
                    st[:, b, c] = [f @ np.array(num_w), f @ np.array(den_w), m]
    return y, st


@pytest.mark.parametrize("with_state", [False, True])
def test_matches_closed_form(with_state):
    w, u, k, v, s0 = rand_case(1, state=with_state)
    y, st = oracle.wkv(w, u, k, v, s0)
    yc, stc = closed_form(w, u, k, v, s0)
    np.testing.assert_allclose(y, yc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[2], stc[2], rtol=0, atol=1e-12)   # canonical log-scale
    np.testing.assert_allclose(st[:2], stc[:2], rtol=1e-12, atol=1e-12)


def test_matches_closed_form_with_large_outliers():
    """Keys far beyond exp's range in either sign: the recurrence stays finite."""
    w, u, k, v, _ = rand_case(2, T=12, kscale=5.0)
    k[0, 3, :] = 700.0
    k[1, 5, :] = -700.0
    k[0, 8, 1] = 2000.0
    y, st = oracle.wkv(w, u, k, v)
    assert np.isfinite(y).all() and np.isfinite(st).all()
    yc, stc = closed_form(w, u, k, v)
    np.testing.assert_allclose(y, yc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[2], stc[2], rtol=1e-15, atol=1e-12)


def test_scaled_cumsum_form():
    """RWKV-LM discussion #189: scale numerator and denominator by the decay
    to the power -(t-1) and both become cumulative sums (valid while nothing
    overflows: small T, small keys)."""
    B, T, C = 2, 12, 4
    w, u, k, v, _ = rand_case(3, B, T, C, kscale=1.0)
    W = np.exp(w)                                    # multiplicative per-step decay
    i = np.arange(T)[None, :, None]
    a = W[None, None, :] ** (-i) * np.exp(k)         # W^{-i} e^{k_i}
    num_past = np.cumsum(a * v, axis=1) - a * v      # exclusive prefix sums
    den_past = np.cumsum(a, axis=1) - a
    cur = W[None, None, :] ** (-(i - 1)) * np.exp(u[None, None, :] + k)
    y_ref = (num_past + cur * v) / (den_past + cur)
    y, _ = oracle.wkv(w, u, k, v)
    np.testing.assert_allclose(y, y_ref, rtol=1e-10, atol=1e-12)


def test_single_step_from_zero_state_returns_v():
    w, u, k, v, _ = rand_case(4, T=1, kscale=30.0)
    y, st = oracle.wkv(w, u, k, v)
    np.testing.assert_array_equal(y, v)
    np.testing.assert_array_equal(st[2], k[:, 0, :])          # pp = k_0
    np.testing.assert_array_equal(st[0], v[:, 0, :])
    np.testing.assert_array_equal(st[1], np.ones_like(v[:, 0, :]))


def test_no_decay_no_bonus_no_keys_is_running_mean():
    B, T, C = 2, 15, 3
    r = np.random.default_rng(5)
    v = r.standard_normal((B, T, C))
    z = np.zeros(C)
    y, _ = oracle.wkv(z, z, np.zeros((B, T, C)), v)
    mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    np.testing.assert_allclose(y, mean, rtol=1e-13, atol=1e-13)


def test_huge_bonus_returns_current_value():
    w, u, k, v, _ = rand_case(6, kscale=1.0)
    y, _ = oracle.wkv(w, u + 60.0, k, v)
    np.testing.assert_allclose(y, v, rtol=1e-12, atol=1e-12)


def test_instant_decay_keeps_only_previous_token():
    w, u, k, v, _ = rand_case(7, kscale=1.5)
    w = np.full_like(w, -1e4)
    y, _ = oracle.wkv(w, u, k, v)
    np.testing.assert_array_equal(y[:, 0], v[:, 0])
    a = np.exp(k[:, :-1])                       # previous token, undecayed
    c = np.exp(u[None, None, :] + k[:, 1:])     # current token with bonus
    ref = (a * v[:, :-1] + c * v[:, 1:]) / (a + c)
    np.testing.assert_allclose(y[:, 1:], ref, rtol=1e-12, atol=1e-13)


def test_split_continuation():
    w, u, k, v, s0 = rand_case(8, T=20, state=True)
    y, st = oracle.wkv(w, u, k, v, s0)
    T1 = 7
    c = np.ascontiguousarray
    ya, sta = oracle.wkv(w, u, c(k[:, :T1]), c(v[:, :T1]), s0)
    yb, stb = oracle.wkv(w, u, c(k[:, T1:]), c(v[:, T1:]), sta)
    np.testing.assert_allclose(np.concatenate([ya, yb], 1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(stb, st, rtol=1e-13, atol=1e-13)


def combine(s1, s2, n2, w):
    """Segment-summary combine: (aa1,bb1,pp1) over an earlier span, then
    (aa2,bb2,pp2) over a later span of n2 steps.  The earlier sums decay by
    n2 steps (log-scale pp1 + n2 w); both are rescaled to the larger scale."""
    q = s1[2] + n2 * w
    m = np.maximum(q, s2[2])
    e1, e2 = np.exp(q - m), np.exp(s2[2] - m)
    return np.stack([s1[0] * e1 + s2[0] * e2, s1[1] * e1 + s2[1] * e2, m])


def test_segment_combine_is_exact_and_associative():
    """The time-parallel path rests on this: summaries of consecutive segments
    (each started from the empty state) combine into the whole run's state."""
    w, u, k, v, s0 = rand_case(9, B=2, T=24, C=6, state=True, kscale=4.0)
    c = np.ascontiguousarray
    cuts = [0, 5, 6, 15, 24]
    sums = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        _, s = oracle.wkv(w, u, c(k[:, a:b]), c(v[:, a:b]))
        sums.append((s, b - a))
    _, whole = oracle.wkv(w, u, k, v, s0)
    # left fold from the carried state
    acc = s0
    for s, n in sums:
        acc = combine(acc, s, n, w)
    np.testing.assert_allclose(acc, whole, rtol=1e-12, atol=1e-12)
    # right-leaning tree gives the same
    r23 = combine(sums[2][0], sums[3][0], sums[3][1], w)
    r123 = combine(sums[1][0], r23, sums[2][1] + sums[3][1], w)
    r0123 = combine(sums[0][0], r123, sums[1][1] + sums[2][1] + sums[3][1], w)
    tree = combine(s0, r0123, 24, w)
    np.testing.assert_allclose(tree, whole, rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_results():
    w, u, k, v, s0 = rand_case(10, B=3, T=30, C=17, state=True)
    a = oracle.wkv(w, u, k, v, s0, threads=1)
    b = oracle.wkv(w, u, k, v, s0, threads=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
