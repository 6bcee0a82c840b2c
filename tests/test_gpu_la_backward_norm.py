"""GPU parity of la_backward's step-by-step path (and of the fp32 chunked scans that
take the normalised form without factors for bf16 inputs) against the fp64 backward
oracle: the normalised form (flash-linear-attention issue #268: y = QKV / QK1
with a carried key sum, whose initial value also gets its gradient), one factor
per key channel (RetNet issue #21: factors of the values' own shape), and the
scalar modes forced onto that path."""
import numpy as np
import pytest
import torch

import decayed_recurrence_scans_amd as drs
import oracle
from decayed_recurrence_scans_amd import workloads as wl
from tests.tolerance import RTOL, assert_close, record_margin, worst_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "ddecay", "dstate_in", "dcum_k_in")


def dev(x):
    return None if x is None else x.to(DEV)


def case(B, H, T, Dk, Dv, dtype, mode, seed, normalize, with_state=True):
    inp = wl.la_inputs(B, H, T, Dk, Dv, dtype=dtype, mode=mode, normalize=normalize,
                       dist="elu1" if normalize else "scaled", seed=seed, random_state=with_state)
    dy, dsf = wl.output_gradients(B, H, T, Dk, Dv, dtype=dtype, seed=seed, with_state=with_state)
    dzf = None
    if normalize and with_state:
        dzf = torch.randn(B, H, Dk, generator=torch.Generator().manual_seed(seed + 31)).to(torch.float32)
    return inp, dy, dsf, dzf


def run(inp, dy, dsf, dzf, mode, reverse, normalize, force=None):
    q, k, v, dec, s0 = (dev(inp[n]) for n in ("q", "k", "v", "decay", "state_in"))
    g = drs.la_backward(q, k, v, dev(dy), dec, mode, s0, None, dev(dsf), reverse=reverse, normalize=normalize,
                        cum_k_in=dev(inp["cum_k_in"]) if normalize else None, dcum_k_out=dev(dzf), force=force)
    torch.cuda.synchronize()
    return [None if x is None else x.float().cpu().numpy() for x in g]


def reference(inp, dy, dsf, dzf, mode, reverse, normalize):
    if normalize:
        return oracle.la_backward(inp["q"], inp["k"], inp["v"], dy, inp["decay"], mode, inp["state_in"], dsf,
                                  reverse=reverse, normalize=True, cum_k_in=inp["cum_k_in"], dcum_k_out=dzf)
    return oracle.la_backward(inp["q"], inp["k"], inp["v"], dy, inp["decay"], mode, inp["state_in"], dsf,
                              reverse=reverse)


def slices(mode):
    """Slice dimensions of each gradient for the tolerance's rms term."""
    dg = {"none": 1, "head": 1, "step": 1, "elem": 2}[mode]
    return (2, 2, 2, dg, 2, 1)


def check(got, ref, dtype, mode, what, record=False):
    rtol = RTOL[dtype]
    ratios = {}
    for name, a, b, nd in zip(NAMES, got, ref, slices(mode)):
        if b is None:
            assert a is None, name
            continue
        ratios[name] = worst_ratio(a, b, rtol, nd)
        assert_close(a, b, rtol, nd, f"{what} {name}")
    if record:
        record_margin(what, **ratios)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["none", "head", "step", "elem"])
@pytest.mark.parametrize("reverse", [False, True])
def test_normalized_modes(dtype, mode, reverse):
    seed = 200 + 4 * ["none", "head", "step", "elem"].index(mode) + 2 * (dtype == "bf16") + reverse
    inp, dy, dsf, dzf = case(2, 3, 300, 64, 32, dtype, mode, seed, True)
    got = run(inp, dy, dsf, dzf, mode, reverse, True)
    check(got, reference(inp, dy, dsf, dzf, mode, reverse, True), dtype, mode,
          f"normalized {dtype} {mode} rev={reverse}")


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("mode", ["none", "head", "step", "elem"])
@pytest.mark.parametrize("reverse", [False, True])
def test_time_segments(normalize, mode, reverse):
    """Two (b, h) units over T = 1437: each sweep runs as 5 segments of 288 steps (the
    last 285) that fold the other segments' summaries into their entering state, and
    the factor gradient's sums are completed across segments.  fp32, strict bar."""
    seed = 400 + 4 * ["none", "head", "step", "elem"].index(mode) + 2 * normalize + reverse
    inp, dy, dsf, dzf = case(1, 2, 1437, 32, 32, "f32", mode, seed, normalize)
    got = run(inp, dy, dsf, dzf, mode, reverse, normalize, force="recurrent")
    check(got, reference(inp, dy, dsf, dzf, mode, reverse, normalize), "f32", mode,
          f"segments norm={normalize} {mode} rev={reverse}", record=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_elem_unnormalized(dtype, reverse, with_state):
    inp, dy, dsf, dzf = case(2, 2, 250, 32, 64, dtype, "elem", 300 + 2 * reverse + with_state, False, with_state)
    got = run(inp, dy, dsf, dzf, "elem", reverse, False)
    check(got, reference(inp, dy, dsf, dzf, "elem", reverse, False), dtype, "elem",
          f"elem {dtype} rev={reverse} state={with_state}")


@pytest.mark.parametrize("mode", ["none", "head", "step"])
def test_scalar_modes_forced_onto_the_step_by_step_path(mode):
    inp, dy, dsf, dzf = case(2, 2, 180, 64, 64, "f32", mode, 400, False)
    got = run(inp, dy, dsf, dzf, mode, True, False, force="recurrent")
    check(got, reference(inp, dy, dsf, dzf, mode, True, False), "f32", mode, f"forced {mode}")


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (128, 128), (32, 128), (128, 16), (16, 64)])
def test_normalized_head_dims(Dk, Dv):
    inp, dy, dsf, dzf = case(1, 2, 120, Dk, Dv, "bf16", "step", Dk + Dv, True)
    got = run(inp, dy, dsf, dzf, "step", False, True)
    check(got, reference(inp, dy, dsf, dzf, "step", False, True), "bf16", "step", f"{Dk}x{Dv}")


@pytest.mark.parametrize("T", [1, 2, 16, 17, 333])
def test_normalized_lengths(T):
    inp, dy, dsf, dzf = case(2, 2, T, 64, 64, "f32", "elem", 500 + T, True)
    got = run(inp, dy, dsf, dzf, "elem", T % 2 == 0, True)
    check(got, reference(inp, dy, dsf, dzf, "elem", T % 2 == 0, True), "f32", "elem", f"T={T}")


def test_zero_state_and_no_final_gradients():
    """No initial state, key sum or final-state gradients: the first visited step's
    factor gradient is zero (the oracle's is exactly zero; here it is the sum of
    every step's terms, which cancel to rounding)."""
    inp, dy, dsf, dzf = case(2, 2, 64, 32, 32, "f32", "step", 600, True, with_state=False)
    got = run(inp, dy, dsf, dzf, "step", False, True)
    ref = reference(inp, dy, dsf, dzf, "step", False, True)
    check(got, ref, "f32", "step", "no state")
    np.testing.assert_array_equal(ref[3][:, :, 0], 0.0)
    rms = np.sqrt(np.mean(ref[3] ** 2, axis=-1))
    assert np.all(np.abs(got[3][:, :, 0]) <= 1e-5 * rms)


def test_normalized_workload_backward():
    """The backward of the normalized workload at full size (B=4, H=16, T=4096,
    Dk=Dv=128, bf16, continuing from S0 / cum_k0), every unit, with final-state
    and key-sum gradients."""
    cfg = wl.LA_CONFIGS["normalized_bf16"]
    inp = wl.la_config_inputs(cfg)
    dy, dsf = wl.output_gradients(cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv, dtype=cfg.dtype, seed=cfg.seed,
                                  with_state=True)
    dzf = torch.randn(cfg.B, cfg.H, cfg.Dk, generator=torch.Generator().manual_seed(cfg.seed + 31))
    got = run(inp, dy, dsf, dzf, cfg.mode, False, True)
    ref = reference(inp, dy, dsf, dzf, cfg.mode, False, True)
    check(got, ref, cfg.dtype, cfg.mode, "normalized_bf16 backward", record=True)


def test_elem_workload_backward():
    """The backward of the per-key-channel workload at full size (B=4, H=16, T=4096,
    Dk=Dv=128, bf16, four time segments per sweep), every unit, with the factor
    gradient of every (b, h, t, key channel)."""
    cfg = wl.LA_CONFIGS["backward_elem_bf16"]
    inp = wl.la_config_inputs(cfg)
    dy, dsf = wl.output_gradients(cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv, dtype=cfg.dtype, seed=cfg.seed,
                                  with_state=inp["state_in"] is not None)
    got = run(inp, dy, dsf, None, cfg.mode, False, False)
    ref = reference(inp, dy, dsf, None, cfg.mode, False, False)
    check(got, ref, cfg.dtype, cfg.mode, "backward_elem_bf16", record=True)


@pytest.mark.parametrize("T", [200, 1437])
def test_bitwise_deterministic(T):
    inp, dy, dsf, dzf = case(2, 2, T, 64, 64, "bf16", "elem", 700, True)
    a = run(inp, dy, dsf, dzf, "elem", False, True)
    b = run(inp, dy, dsf, dzf, "elem", False, True)
    for x, y in zip(a, b):
        if x is not None:
            np.testing.assert_array_equal(x, y)


def test_leaves_the_lookback_counters_alone():
    """The step-by-step backward keeps off the workspace's first 256 bytes (the
    look-back counters that chunked calls sharing the workspace rely on): chunked
    forward and backward calls on the same workspace afterwards still match."""
    B, H, T, Dk, Dv = 2, 2, 700, 64, 64
    inp, dy, dsf, dzf = case(B, H, T, Dk, Dv, "bf16", "step", 800, True)
    need = max(drs.la_backward_workspace_bytes(B, H, T, Dk, Dv, normalize=True),
               drs.la_workspace_bytes(B, H, T, Dk, Dv))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    q, k, v, dec, s0 = (dev(inp[n]) for n in ("q", "k", "v", "decay", "state_in"))
    drs.la_backward(q, k, v, dev(dy), dec, "step", s0, None, dev(dsf), normalize=True,
                    cum_k_in=dev(inp["cum_k_in"]), dcum_k_out=dev(dzf), workspace=ws, force="recurrent")
    torch.cuda.synchronize()
    assert int(ws[:256].count_nonzero()) == 0
    for _ in range(2):
        y, s, _ = drs.la_forward(q, k, v, dec, "step", s0, workspace=ws)
        g = drs.la_backward(q, k, v, dev(dy), dec, "step", s0, s, dev(dsf), workspace=ws)
        torch.cuda.synchronize()
        yr, sr, _ = oracle.la(inp["q"], inp["k"], inp["v"], inp["decay"], "step", inp["state_in"])
        assert_close(y.float().cpu().numpy(), yr, RTOL["bf16"], 2, "forward after")
        gr = oracle.la_backward(inp["q"], inp["k"], inp["v"], dy, inp["decay"], "step", inp["state_in"], dsf)
        check([None if x is None else x.float().cpu().numpy() for x in g], gr, "bf16", "step", "chunked after")


@pytest.mark.parametrize("mode", ["none", "step"])
def test_normalized_fp32_long_sequence(mode):
    """fp32 over a long sequence: the factor gradient is a suffix sum over 2000 steps
    whose terms partly cancel; the margin under the fp32 bar is recorded."""
    inp, dy, dsf, dzf = case(2, 4, 2000, 64, 64, "f32", mode, 900, True)
    got = run(inp, dy, dsf, dzf, mode, mode == "step", True)
    check(got, reference(inp, dy, dsf, dzf, mode, mode == "step", True), "f32", mode,
          f"normalized fp32 T=2000 {mode}", record=True)


# ---- the normalised form without factors, bf16: unnormalised fp32 chunked scans ----------

@pytest.mark.parametrize("Dk,Dv,T,reverse", [(64, 64, 700, False), (64, 64, 700, True), (16, 16, 17, False),
                                             (32, 128, 333, True), (128, 16, 257, False), (128, 128, 1000, True)])
def test_normalized_chunked_scans(Dk, Dv, T, reverse):
    """bf16, no factor, T above the step-by-step limit: n, d and the five gradient
    products as fp32 scans on the chunked kernels (ragged last chunks, both visiting
    orders, every head-dimension pairing incl. the 16-wide padded operands), with
    initial state, key sum and final-state gradients."""
    inp, dy, dsf, dzf = case(2, 2, T, Dk, Dv, "bf16", "none", 900 + T + Dk, True)
    got = run(inp, dy, dsf, dzf, "none", reverse, True)
    check(got, reference(inp, dy, dsf, dzf, "none", reverse, True), "bf16", "none",
          f"chunked normalized {Dk}x{Dv} T={T} rev={reverse}")


def test_normalized_chunked_scans_zero_state():
    """No initial state, key sum or final gradients (every padded state absent)."""
    inp, dy, dsf, dzf = case(3, 2, 400, 64, 32, "bf16", "none", 950, True, with_state=False)
    got = run(inp, dy, dsf, dzf, "none", False, True)
    check(got, reference(inp, dy, dsf, dzf, "none", False, True), "bf16", "none", "chunked normalized, no state")


def test_normalized_chunked_matches_step_by_step():
    """The chunked fp32 scans and the forced step-by-step kernels (fp64) agree to the
    bf16 bar with each other as well as with the oracle."""
    inp, dy, dsf, dzf = case(2, 2, 600, 64, 64, "bf16", "none", 960, True)
    a = run(inp, dy, dsf, dzf, "none", False, True)
    b = run(inp, dy, dsf, dzf, "none", False, True, force="recurrent")
    ref = reference(inp, dy, dsf, dzf, "none", False, True)
    check(a, ref, "bf16", "none", "chunked")
    check(b, ref, "bf16", "none", "step by step")


@pytest.mark.parametrize("chunk", [16, 64])
def test_normalized_chunked_scans_explicit_chunk(chunk):
    """A chunk size given by the caller serves every scan of the fp32 path."""
    inp, dy, dsf, dzf = case(2, 3, 500, 64, 128, "bf16", "none", 970 + chunk, True)
    q, k, v, s0 = (dev(inp[n]) for n in ("q", "k", "v", "state_in"))
    g = drs.la_backward(q, k, v, dev(dy), None, "none", s0, None, dev(dsf), normalize=True,
                        cum_k_in=dev(inp["cum_k_in"]), dcum_k_out=dev(dzf), chunk=chunk)
    torch.cuda.synchronize()
    got = [None if x is None else x.float().cpu().numpy() for x in g]
    check(got, reference(inp, dy, dsf, dzf, "none", False, True), "bf16", "none", f"chunk {chunk}")


@pytest.mark.parametrize("mode", ["head", "step"])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_normalized_chunked_scans_factors(mode, reverse, with_state):
    """One factor per head or per step on the fp32-scan path: the reverse scans take the
    factor of the step visited next, the initial-state gradients the first visited
    step's factor, and the factor gradient the suffix sums of q . dq - k . dk plus the
    final state's and key sum's terms."""
    inp, dy, dsf, dzf = case(2, 3, 600, 64, 64, "bf16", mode, 990 + 2 * reverse + with_state, True,
                             with_state=with_state)
    got = run(inp, dy, dsf, dzf, mode, reverse, True)
    check(got, reference(inp, dy, dsf, dzf, mode, reverse, True), "bf16", mode,
          f"chunked normalized {mode} rev={reverse} state={with_state}")


def test_normalized_chunked_scans_step_decay_d128():
    inp, dy, dsf, dzf = case(2, 4, 2048, 128, 128, "bf16", "step", 999, True)
    got = run(inp, dy, dsf, dzf, "step", False, True)
    check(got, reference(inp, dy, dsf, dzf, "step", False, True), "bf16", "step", "chunked normalized step D=128")
