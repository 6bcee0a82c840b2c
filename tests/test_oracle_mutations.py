"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of ``oracle/oracle.c`` (a dropped
term, a wrong sign, a wrong index, a transposed operand, an ignored input),
compiles it into a temporary library, swaps it in for the real one and runs
the pins of ``test_oracle_la``, ``test_oracle_elem_bidir``, ``test_oracle_wkv`` or
``test_oracle_ema``.  At least one pin must
fail for every planted mistake; the real library is restored afterwards.
"""
import ctypes
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_elem_bidir as E
from tests import test_oracle_ema as M
from tests import test_oracle_la as L
from tests import test_oracle_la_backward as LB
from tests import test_oracle_wkv as W
from tests import test_oracle_wkv_backward as WB

LA_PINS = [
    lambda g: L.test_worked_examples_exact(g),
    lambda g: L.test_matches_causal_quadratic_form("step", True),
    lambda g: L.test_matches_causal_quadratic_form("head", False),
    lambda g: L.test_reverse_matches_anticausal_quadratic_form("step"),
    lambda g: L.test_normalized_matches_quadratic_ratio(),
    lambda g: L.test_decay_convention_by_hand(),
    lambda g: L.test_normalized_equal_keys_is_running_mean(),
    lambda g: L.test_carried_state_workload_equals_concatenation(),
]

WKV_PINS = [
    lambda g: W.test_matches_closed_form(True),
    lambda g: W.test_matches_closed_form(False),
    lambda g: W.test_scaled_cumsum_form(),
    lambda g: W.test_single_step_from_zero_state_returns_v(),
    lambda g: W.test_instant_decay_keeps_only_previous_token(),
    lambda g: W.test_no_decay_no_bonus_no_keys_is_running_mean(),
]

ELEM_PINS = [
    lambda g: E.test_elem_is_query_contraction_of_outer_product_ema(False),
    lambda g: E.test_elem_is_query_contraction_of_outer_product_ema(True),
    lambda g: E.test_elem_matches_quadratic_form(True, False),
    lambda g: E.test_elem_matches_quadratic_form(False, True),
    lambda g: E.test_elem_is_sum_of_one_channel_step_problems(),
    lambda g: E.test_elem_with_equal_channels_is_step_mode(),
]

BWD_PINS = [
    lambda g: LB.test_matches_autograd_of_explicit_form("head", False),
    lambda g: LB.test_matches_autograd_of_explicit_form("step", True),
    lambda g: LB.test_matches_autograd_of_explicit_form("elem", False),
    lambda g: LB.test_directional_finite_differences_of_the_forward_oracle("step", True),
    lambda g: LB.test_reverse_is_flipped_forward_backward(),
]

BWD_NORM_PINS = [
    lambda g: LB.test_normalized_matches_autograd_of_ratio_form("step", False),
    lambda g: LB.test_normalized_matches_autograd_of_ratio_form("elem", True),
    lambda g: LB.test_normalized_directional_finite_differences("head", True),
    lambda g: LB.test_normalized_query_gradient_is_orthogonal_to_the_query(),
    lambda g: LB.test_normalized_joint_key_scaling_identity("elem"),
    lambda g: LB.test_normalized_equal_values_give_no_query_key_or_decay_gradient(),
]

WBWD_PINS = [
    lambda g: WB.test_matches_autograd_of_closed_form(True),
    lambda g: WB.test_directional_finite_differences_of_the_forward_oracle(),
    lambda g: WB.test_single_token_without_state(),
    lambda g: WB.test_state_gradient_matches_autograd_of_closed_form(),
    lambda g: WB.test_state_gradient_finite_differences_and_representation_invariance(),
]

EMA_PINS = [
    lambda g: M.test_matches_prefix_scan_of_the_page_operator(0),
    lambda g: M.test_matches_closed_form(),
    lambda g: M.test_retention_is_query_contraction_of_outer_product_ema(),
    lambda g: M.test_special_cases(),
    lambda g: M.test_reverse_is_flip_forward_flip(),
    lambda g: M.test_continuation_through_state(),
]

MUTATIONS = [
    # linear attention
    ("la: decay dropped from the state update",
     "S[i * Dv + j] = gi * S[i * Dv + j] + kt[i] * vt[j];",
     "S[i * Dv + j] = S[i * Dv + j] + kt[i] * vt[j];", LA_PINS),
    ("la: key/value outer product transposed",
     "gi * S[i * Dv + j] + kt[i] * vt[j];", "gi * S[i * Dv + j] + kt[j % Dk] * vt[i % Dv];", LA_PINS),
    ("la: read-out contracts the wrong state index",
     "acc += qt[i] * S[i * Dv + j];", "acc += qt[i] * S[(j % Dk) * Dv + (i % Dv)];", LA_PINS),
    ("la: per-step decay taken one step late",
     "g = gamma[(b * H + h) * T + t];", "g = gamma[(b * H + h) * T + (t + 1) % T];", LA_PINS),
    ("la: reverse flag ignored",
     "long t = reverse ? (T - 1 - n) : n;\n            const double *qt = q + (unit * T + t) * Dk;\n"
     "            const double *kt = k + (unit * T + t) * Dk;\n            const double *vt = v + (unit * T + t) * Dv;\n"
     "            double g",
     "long t = n;\n            const double *qt = q + (unit * T + t) * Dk;\n"
     "            const double *kt = k + (unit * T + t) * Dk;\n            const double *vt = v + (unit * T + t) * Dv;\n"
     "            double g", LA_PINS),
    ("la bwd: reverse flag ignored in the backward sweep",
     "long t = reverse ? (T - 1 - n) : n;\n            const double *qt = q + (unit * T + t) * Dk;\n"
     "            const double *kt = k + (unit * T + t) * Dk;\n            const double *vt = v + (unit * T + t) * Dv;\n"
     "            const double *dyt",
     "long t = n;\n            const double *qt = q + (unit * T + t) * Dk;\n"
     "            const double *kt = k + (unit * T + t) * Dk;\n            const double *vt = v + (unit * T + t) * Dv;\n"
     "            const double *dyt", BWD_PINS),
    ("la: key sum not decayed", "z[i] = gi * z[i] + kt[i];", "z[i] = z[i] + kt[i];", LA_PINS),
    # per-element decay
    ("la elem: factor of the wrong key channel", "const double gi = ge ? ge[i] : g;",
     "const double gi = ge ? ge[(i + 1) % Dk] : g;", ELEM_PINS),
    ("la elem: factor indexed by the value column",
     "S[i * Dv + j] = gi * S[i * Dv + j] + kt[i] * vt[j];",
     "S[i * Dv + j] = (ge ? ge[j % Dk] : gi) * S[i * Dv + j] + kt[i] * vt[j];", ELEM_PINS),
    ("la elem: factor taken one step late", "ge = gamma + ((b * H + h) * T + t) * Dk;",
     "ge = gamma + ((b * H + h) * T + (t + 1) % T) * Dk;", ELEM_PINS),
    ("la elem: key sum not decayed", "z[i] = gi * z[i] + kt[i];",
     "z[i] = (ge ? 1.0 : gi) * z[i] + kt[i];", ELEM_PINS),
    ("la: initial state ignored",
     "S[i] = state_in ? state_in[unit * Dk * Dv + i] : 0.0;", "S[i] = 0.0;", LA_PINS),
    ("la: cached key sum ignored",
     "z[i] = (normalize && cum_k_in) ? cum_k_in[unit * Dk + i] : 0.0;", "z[i] = 0.0;", LA_PINS),
    ("la: normaliser uses the current key only",
     "den += qt[i] * z[i];", "den += qt[i] * kt[i];", LA_PINS),
    # linear-attention backward
    ("la bwd: query gradient from the entering state", "a += Sa[i * Dv + j] * an[j];",
     "a += Se[i * Dv + j] * an[j];", BWD_PINS),
    ("la bwd: decay gradient against the leaving state", "for (long i = 0; i < SZ; ++i) a += G[i] * Se[i];",
     "for (long i = 0; i < SZ; ++i) a += G[i] * Sa[i];", BWD_PINS),
    ("la bwd: key gradient contracts dy instead of v", "c += G[i * Dv + j] * vt[j];",
     "c += G[i * Dv + j] * dyt[j % Dv];", BWD_PINS),
    ("la bwd: state gradient not decayed", "G[i * Dv + j] *= gv[i];", "G[i * Dv + j] *= 1.0;", BWD_PINS),
    ("la bwd: final-state gradient ignored",
     "for (long i = 0; i < SZ; ++i) G[i] = dstate_out ? dstate_out[unit * SZ + i] : 0.0;",
     "for (long i = 0; i < SZ; ++i) G[i] = 0.0;", BWD_PINS),
    ("la bwd: factor of the wrong step", "                gv[i] = g;",
     "                gv[i] = (decay_mode == ORACLE_DECAY_STEP) ? gamma[unit * T + (t + 1) % T] : g;", BWD_PINS),
    ("la bwd: query term added after the decay",
     "for (long j = 0; j < Dv; ++j) G[i * Dv + j] += qt[i] * an[j];",
     "for (long j = 0; j < Dv; ++j) G[i * Dv + j] += 0.0 * qt[i] * an[j];", BWD_PINS),
    # normalised linear-attention backward
    ("la bwd norm: numerator gradient not divided by the denominator", "an[j] = dyt[j] / den;",
     "an[j] = dyt[j];", BWD_NORM_PINS),
    ("la bwd norm: denominator gradient sign", "cden = -dyy / den;", "cden = dyy / den;", BWD_NORM_PINS),
    ("la bwd norm: denominator gradient missing a 1/den", "cden = -dyy / den;", "cden = -dyy;",
     BWD_NORM_PINS),
    ("la bwd norm: query gradient misses the key-sum read-out", "dq[(unit * T + t) * Dk + i] = a + za[i] * cden;",
     "dq[(unit * T + t) * Dk + i] = a;", BWD_NORM_PINS),
    ("la bwd norm: query gradient reads the entering key sum", "dq[(unit * T + t) * Dk + i] = a + za[i] * cden;",
     "dq[(unit * T + t) * Dk + i] = a + ze[i] * cden;", BWD_NORM_PINS),
    ("la bwd norm: key gradient misses the key-sum term", "dk[(unit * T + t) * Dk + i] = c + Gz[i];",
     "dk[(unit * T + t) * Dk + i] = c;", BWD_NORM_PINS),
    ("la bwd norm: key-sum gradient not decayed", "Gz[i] *= gv[i];", "Gz[i] *= 1.0;", BWD_NORM_PINS),
    ("la bwd norm: final key-sum gradient ignored",
     "Gz[i] = (normalize && dcum_k_out) ? dcum_k_out[unit * Dk + i] : 0.0;", "Gz[i] = 0.0;", BWD_NORM_PINS),
    ("la bwd norm: cached key sum ignored in the recomputation",
     "zb[i] = (normalize && cum_k_in) ? cum_k_in[unit * Dk + i] : 0.0;", "zb[i] = 0.0;", BWD_NORM_PINS),
    ("la bwd norm: decay gradient misses the key-sum term (per channel)", "double a = Gz[i] * ze[i];",
     "double a = 0.0;", BWD_NORM_PINS),
    ("la bwd norm: decay gradient misses the key-sum term", "for (long i = 0; i < Dk; ++i) a += Gz[i] * ze[i];",
     "for (long i = 0; i < Dk; ++i) a += 0.0 * Gz[i] * ze[i];", BWD_NORM_PINS),
    # WKV
    ("wkv: bonus u dropped", "const struct wsum now = { v[i], 1.0, u[c] + k[i] };",
     "const struct wsum now = { v[i], 1.0, k[i] };", WKV_PINS),
    ("wkv: decay sign flipped", "const struct wsum past = { st.a, st.b, st.p + w[c] };",
     "const struct wsum past = { st.a, st.b, st.p - w[c] };", WKV_PINS),
    ("wkv: no decay", "const struct wsum past = { st.a, st.b, st.p + w[c] };",
     "const struct wsum past = { st.a, st.b, st.p };", WKV_PINS),
    ("wkv: weight of the current token dropped from the denominator",
     "const struct wsum now = { v[i], 1.0, u[c] + k[i] };",
     "const struct wsum now = { v[i], 0.0, u[c] + k[i] };", WKV_PINS),
    ("wkv: bonus applied when absorbing", "const struct wsum tok = { v[i], 1.0, k[i] };",
     "const struct wsum tok = { v[i], 1.0, u[c] + k[i] };", WKV_PINS),
    ("wkv: state planes swapped", "st.a = state_in[0 * B * C + unit];",
     "st.a = state_in[1 * B * C + unit];", WKV_PINS),
    ("wkv: join rescales the wrong side", "struct wsum r = { x.a * ex + y.a * ey, x.b * ex + y.b * ey, p };",
     "struct wsum r = { x.a * ey + y.a * ex, x.b * ex + y.b * ey, p };", WKV_PINS),
    # WKV backward
    ("wkv bwd: state gradient of pp misses the weight-sum part", "dpp = aa0 * daa + bb0 * dbb;",
     "dpp = aa0 * daa;", WBWD_PINS),
    ("wkv bwd: state gradient not scaled by e^pp", "daa = Abar * e0;", "daa = Abar;", WBWD_PINS),
    ("wkv bwd: decay factor missing from dw", "dw += ew * (A[t] * Abar + Bs[t] * Bbar);",
     "dw += (A[t] * Abar + Bs[t] * Bbar);", WBWD_PINS),
    ("wkv bwd: bonus term of dk dropped", "dk[i] = cur * (v[i] * r + s) + exp(k[i]) * (v[i] * Abar + Bbar);",
     "dk[i] = exp(k[i]) * (v[i] * Abar + Bbar);", WBWD_PINS),
    ("wkv bwd: numerator gradient not decayed", "Abar = r + ew * Abar;", "Abar = r + Abar;", WBWD_PINS),
    ("wkv bwd: dv reads the denominator gradient", "dv[i] = cur * r + exp(k[i]) * Abar;",
     "dv[i] = cur * r + exp(k[i]) * Bbar;", WBWD_PINS),
    ("wkv bwd: denominator gradient sign", "const double r = dy[i] / D, s = -dy[i] * yt / D;",
     "const double r = dy[i] / D, s = dy[i] * yt / D;", WBWD_PINS),
    # gated EMA
    ("ema: factor dropped", "h = f[i] * h + x[i];", "h = h + x[i];", EMA_PINS),
    ("ema: factor applied after the value is added", "h = f[i] * h + x[i];",
     "h = f[i] * (h + x[i]);", EMA_PINS),
    ("ema: factor taken one step late", "h = f[i] * h + x[i];",
     "h = f[(b * T + (t + 1) % T) * C + c] * h + x[i];", EMA_PINS),
    ("ema: reverse flag ignored", "long t = reverse ? (T - 1 - n) : n;\n            long i = (b * T + t) * C + c;",
     "long t = n;\n            long i = (b * T + t) * C + c;", EMA_PINS),
    ("ema: initial state ignored", "double h = state_in ? state_in[unit] : 0.0;", "double h = 0.0;", EMA_PINS),
    ("ema: output written before the update", "h = f[i] * h + x[i];\n            y[i] = h;",
     "y[i] = h;\n            h = f[i] * h + x[i];", EMA_PINS),
]


@pytest.fixture(scope="module")
def src_text():
    return oracle._SRC.read_text()


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pins, src_text, tmp_path, golden_dir):
    assert src_text.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src_text.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(str(so))
    mut.oracle_la.argtypes = real.oracle_la.argtypes
    mut.oracle_la.restype = None
    mut.oracle_wkv.argtypes = real.oracle_wkv.argtypes
    mut.oracle_wkv.restype = None
    mut.oracle_ema.argtypes = real.oracle_ema.argtypes
    mut.oracle_ema.restype = None
    mut.oracle_la_backward.argtypes = real.oracle_la_backward.argtypes
    mut.oracle_la_backward.restype = None
    mut.oracle_wkv_backward.argtypes = real.oracle_wkv_backward.argtypes
    mut.oracle_wkv_backward.restype = None
    failures = 0
    oracle._lib = mut
    try:
        with np.errstate(all="ignore"):
            for pin in pins:
                try:
                    pin(golden_dir)
                except AssertionError:
                    failures += 1
    finally:
        oracle._lib = real
    assert failures > 0, f"no pin caught the planted mistake: {name}"
