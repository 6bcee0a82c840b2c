"""GPU parity of wkv_forward (HIP, gfx950) against the fp64 oracle, both paths."""
import numpy as np
import pytest
import torch

import decayed_recurrence_scans_amd as drs
import oracle
from decayed_recurrence_scans_amd import workloads as wl
from tests.tolerance import RTOL, assert_close, record_margin, worst_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = RTOL["f32"]


def run_gpu(inp, force=None):
    y, s = drs.wkv_forward(*(inp[n].to(DEV) for n in ("w", "u", "k", "v")),
                           None if inp["state_in"] is None else inp["state_in"].to(DEV), force=force)
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


def run_ref(inp):
    return oracle.wkv(inp["w"], inp["u"], inp["k"], inp["v"], inp["state_in"])


def check_state(got, ref, what):
    """States compare in the sums they stand for: (aa, bb) rescaled to the
    oracle's log-scale pp, and pp itself to an absolute 1e-5 * (1 + |pp|)."""
    aa, bb, pp = got
    ra, rb, rp = ref
    scale = np.exp(np.clip(pp.astype(np.float64) - rp, -700, 700))
    assert_close(aa * scale, ra, TOL, 1, what + " aa")
    assert_close(bb * scale, rb, TOL, 1, what + " bb")
    assert np.all(np.abs(pp - rp) <= TOL * (1 + np.abs(rp))), what + " pp"


@pytest.mark.parametrize("force", [None, "seq", "scan", "chain", "rows"])
def test_full_size_config(force):
    cfg = wl.WKV_CONFIGS["wkv_f32"]
    inp = wl.wkv_config_inputs(cfg)
    y, s = run_gpu(inp, force)
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, f"wkv {force} y")
    check_state(s, sr, f"wkv {force}")
    scale = np.exp(np.clip(s[2].astype(np.float64) - sr[2], -700, 700))
    record_margin(f"wkv_f32 path={force or 'default'}", y=worst_ratio(y, yr, TOL, 2),
                  aa=worst_ratio(s[0] * scale, sr[0], TOL, 1), bb=worst_ratio(s[1] * scale, sr[1], TOL, 1))


@pytest.mark.parametrize("force", [None, "seq", "scan", "chain"])
@pytest.mark.parametrize("B,T,C", [(1, 1, 64), (2, 17, 1000), (1, 3000, 300), (3, 700, 129),
                                   (1, 5000, 64), (2, 257, 65), (1, 16384, 70)])
def test_shapes_and_paths(B, T, C, force):
    inp = wl.wkv_inputs(B, T, C, seed=B * 7 + T + C, random_state=True)
    y, s = run_gpu(inp, force)
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, f"B={B} T={T} C={C} {force} y")
    check_state(s, sr, f"B={B} T={T} C={C} {force}")


def test_few_channels_long_sequence_uses_scan():
    B, T, C = 1, 65536, 256
    assert drs.wkv_workspace_bytes(B, T, C) > 0        # the time-parallel path is chosen
    inp = wl.wkv_inputs(B, T, C, seed=77)
    y, s = run_gpu(inp)
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, "long y")
    check_state(s, sr, "long")


@pytest.mark.parametrize("force", ["seq", "scan", "chain"])
def test_state_in_place(force):
    inp = wl.wkv_inputs(2, 400, 256, seed=5, random_state=True)
    yr, sr = run_ref(inp)
    st = inp["state_in"].to(DEV).clone()
    y, s = drs.wkv_forward(*(inp[n].to(DEV) for n in ("w", "u", "k", "v")), st, state_out=st, force=force)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert_close(y.cpu().numpy(), yr, TOL, 2, "in place y")
    check_state(st.cpu().numpy(), sr, "in place")


def test_continuation_through_state():
    inp = wl.wkv_inputs(2, 300, 512, seed=6)
    k, v = inp["k"].to(DEV), inp["v"].to(DEV)
    w, u = inp["w"].to(DEV), inp["u"].to(DEV)
    y1, s1 = drs.wkv_forward(w, u, k[:, :123].contiguous(), v[:, :123].contiguous())
    y2, s2 = drs.wkv_forward(w, u, k[:, 123:].contiguous(), v[:, 123:].contiguous(), s1)
    torch.cuda.synchronize()
    yr, sr = run_ref(inp)
    assert_close(torch.cat([y1, y2], 1).cpu().numpy(), yr, TOL, 2, "continued y")
    check_state(s2.cpu().numpy(), sr, "continued")


def test_empty_state_first_output_is_v():
    inp = wl.wkv_inputs(2, 5, 300, seed=8, outlier_frac=0.05)
    y, _ = run_gpu(inp)
    assert np.array_equal(y[:, 0], inp["v"][:, 0].numpy())


@pytest.mark.parametrize("force", ["seq", "scan", "chain"])
def test_bitwise_deterministic(force):
    inp = wl.wkv_inputs(2, 600, 700, seed=10, random_state=True)
    a = run_gpu(inp, force)
    b = run_gpu(inp, force)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_workload_uses_chain_and_no_wait_gave_up():
    cfg = wl.WKV_CONFIGS["wkv_f32"]
    assert drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C) == \
        drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C, drs.DRS_FORCE_CHAIN) > 0
    assert drs.lookback_timeouts() == 0     # over every call of this module so far


@pytest.mark.parametrize("B,T,C", [(1, 3000, 300), (3, 700, 129), (1, 5000, 64), (2, 257, 65),
                                   (1, 16384, 70)])
def test_chain_own_aggregates(B, T, C):
    """The chained kernel with every earlier block's aggregate computed by the waiting
    waves from k and v (the path a wave takes when its wait runs out): the same
    result up to rounding, and the workspace counts the computed aggregates."""
    inp = wl.wkv_inputs(B, T, C, seed=B * 11 + T + C, random_state=True)
    ws = torch.zeros(drs.wkv_workspace_bytes(B, T, C, drs.DRS_FORCE_CHAIN), dtype=torch.uint8, device=DEV)
    s_in = None if inp["state_in"] is None else inp["state_in"].to(DEV)
    y, s = drs.wkv_forward(*(inp[n].to(DEV) for n in ("w", "u", "k", "v")), s_in,
                           force="chain", own_aggregates=True, workspace=ws)
    torch.cuda.synchronize()
    yr, sr = run_ref(inp)
    assert_close(y.cpu().numpy(), yr, TOL, 2, f"B={B} T={T} C={C} own y")
    check_state(s.cpu().numpy(), sr, f"B={B} T={T} C={C} own")
    assert drs.lookback_timeouts(ws) > 0


# The row-owning sweep (forced only; C a multiple of 4): spans of 8 or 16 steps,
# ragged last spans, channel counts that leave the last workgroup partly empty, a
# carried state, and the look-back that stops at an inclusive state or runs back to
# the initial state.
ROWS_SHAPES = [(1, 1, 64), (2, 17, 1000), (1, 3000, 300), (1, 5000, 64), (3, 700, 132),
               (2, 257, 1028), (8, 300, 4096), (1, 16384, 72)]


@pytest.mark.parametrize("B,T,C", ROWS_SHAPES)
def test_rows_shapes(B, T, C):
    inp = wl.wkv_inputs(B, T, C, seed=B * 13 + T + C, random_state=True)
    y, s = run_gpu(inp, "rows")
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, f"B={B} T={T} C={C} rows y")
    check_state(s, sr, f"B={B} T={T} C={C} rows")


@pytest.mark.parametrize("B,T,C", [(1, 3000, 300), (2, 257, 1028), (3, 700, 132)])
def test_rows_own_aggregates(B, T, C):
    """Every earlier span's summary computed by the waiting wave from k and v (the
    path a wave takes when its wait runs out): the same result up to rounding."""
    inp = wl.wkv_inputs(B, T, C, seed=B * 17 + T + C, random_state=True)
    ws = torch.zeros(drs.wkv_workspace_bytes(B, T, C, drs.DRS_FORCE_ROWS), dtype=torch.uint8, device=DEV)
    y, s = drs.wkv_forward(*(inp[n].to(DEV) for n in ("w", "u", "k", "v")), inp["state_in"].to(DEV),
                           force="rows", own_aggregates=True, workspace=ws)
    torch.cuda.synchronize()
    yr, sr = run_ref(inp)
    assert_close(y.cpu().numpy(), yr, TOL, 2, f"B={B} T={T} C={C} rows own y")
    check_state(s.cpu().numpy(), sr, f"B={B} T={T} C={C} rows own")
    assert drs.lookback_timeouts(ws) > 0


def test_rows_continuation_and_repeat():
    """Two calls that share a workspace (the counters re-armed in between), the
    second continuing from the first's state."""
    inp = wl.wkv_inputs(2, 300, 512, seed=9)
    k, v = inp["k"].to(DEV), inp["v"].to(DEV)
    w, u = inp["w"].to(DEV), inp["u"].to(DEV)
    ws = torch.zeros(drs.wkv_workspace_bytes(2, 300, 512, drs.DRS_FORCE_ROWS), dtype=torch.uint8, device=DEV)
    y1, s1 = drs.wkv_forward(w, u, k[:, :123].contiguous(), v[:, :123].contiguous(), force="rows", workspace=ws)
    y2, s2 = drs.wkv_forward(w, u, k[:, 123:].contiguous(), v[:, 123:].contiguous(), s1, force="rows",
                             workspace=ws)
    torch.cuda.synchronize()
    yr, sr = run_ref(inp)
    assert_close(torch.cat([y1, y2], 1).cpu().numpy(), yr, TOL, 2, "rows continued y")
    check_state(s2.cpu().numpy(), sr, "rows continued")
    assert drs.lookback_timeouts(ws) == 0


# The walk kernel (one workgroup walking all time blocks of 64 channels) serves
# shapes with at least 512 such channel groups; these cases reach it with a carried
# state (weights bb below 1 are rescaled on load), ragged sequence ends (T not a
# multiple of the 128-step block) and a ragged last channel group.
WALK_SHAPES = [(8, 300, 4096), (8, 129, 4100), (16, 64, 2048), (8, 1, 4096), (8, 1000, 4160)]


@pytest.mark.parametrize("B,T,C", WALK_SHAPES)
@pytest.mark.parametrize("state", [False, True])
def test_walk_shapes(B, T, C, state):
    assert B * ((C + 63) // 64) >= 512
    inp = wl.wkv_inputs(B, T, C, seed=B + T + C, random_state=state)
    y, s = run_gpu(inp)
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, f"walk B={B} T={T} C={C} y")
    check_state(s, sr, f"walk B={B} T={T} C={C}")


def test_walk_small_weights_state_and_in_place():
    """A carried state with weights bb far below 1 (and above): the walk kernel
    rescales it by a power of two; updated in place."""
    B, T, C = 8, 200, 4096
    inp = wl.wkv_inputs(B, T, C, seed=31, random_state=True)
    st = inp["state_in"].clone()
    st[1] = st[1] * torch.exp2(torch.randint(-40, 20, (B, C)).float())
    inp["state_in"] = st
    yr, sr = run_ref(inp)
    dst = st.to(DEV).clone()
    y, s = drs.wkv_forward(*(inp[n].to(DEV) for n in ("w", "u", "k", "v")), dst, state_out=dst)
    torch.cuda.synchronize()
    assert s.data_ptr() == dst.data_ptr()
    assert_close(y.cpu().numpy(), yr, TOL, 2, "walk small bb y")
    check_state(dst.cpu().numpy(), sr, "walk small bb")


def test_walk_bitwise_deterministic():
    inp = wl.wkv_inputs(8, 333, 4096, seed=12, random_state=True)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_walk_state_stays_the_largest_term():
    """A carried state with pp = 60 (the size of the workload's outlier keys): in the
    slowly decaying channels it outweighs every key for the whole sequence, so the
    final pp there is pp0 + T w (the canonical maximum), which must come out as is.
    (Far larger log-scales are beyond what fp32 anchors resolve to 1e-5: one
    rounding at pp = 200 already costs ~2e-5.)"""
    B, T, C = 8, 130, 4096
    inp = wl.wkv_inputs(B, T, C, seed=41, random_state=True, outlier_frac=0.0)
    st = inp["state_in"].clone()
    st[2] = 60.0
    w = inp["w"]
    assert int((60.0 + T * w > 40.0).sum()) > 50      # channels where the state stays on top
    inp["state_in"] = st
    y, s = run_gpu(inp)
    yr, sr = run_ref(inp)
    assert_close(y, yr, TOL, 2, "dominant state y")
    check_state(s, sr, "dominant state")
