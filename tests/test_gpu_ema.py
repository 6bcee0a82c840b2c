"""GPU parity of ema_forward (HIP, gfx950) against the fp64 oracle.

Shapes cover both kernels (walk: enough 64-channel units to fill the GPU;
look-back: few channels, one workgroup per time block), ragged T and C, the
reverse order, carried and in-place states.  Bar: tests/tolerance.py.
"""
import numpy as np
import pytest
import torch

import decayed_recurrence_scans_amd as drs
import oracle
from decayed_recurrence_scans_amd import workloads as wl
from tests.tolerance import RTOL, assert_close, record_margin, worst_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gpu(inp, reverse=False):
    s0 = None if inp["state_in"] is None else inp["state_in"].to(DEV)
    y, s = drs.ema_forward(inp["x"].to(DEV), inp["f"].to(DEV), s0, reverse=reverse)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), s.cpu().numpy()


def check(inp, dtype, reverse, what):
    y, s = run_gpu(inp, reverse)
    yr, sr = oracle.ema(inp["x"], inp["f"], inp["state_in"], reverse=reverse)
    assert_close(y, yr, RTOL[dtype], 2, what + " y")
    assert_close(s, sr, RTOL[dtype], 1, what + " state")


@pytest.mark.parametrize("reverse", [False, True])
def test_full_size_config(reverse):
    cfg = wl.EMA_CONFIGS["ema_bf16"]
    assert drs.ema_workspace_bytes(cfg.B, cfg.T, cfg.C, torch.bfloat16) == 0   # walk kernel
    inp = wl.ema_config_inputs(cfg)
    y, s = run_gpu(inp, reverse)
    yr, sr = oracle.ema(inp["x"], inp["f"], inp["state_in"], reverse=reverse)
    what = f"{cfg.name} rev={reverse}"
    assert_close(y, yr, RTOL[cfg.dtype], 2, what + " y")
    assert_close(s, sr, RTOL[cfg.dtype], 1, what + " state")
    record_margin(what, y=worst_ratio(y, yr, RTOL[cfg.dtype], 2), state=worst_ratio(s, sr, RTOL[cfg.dtype], 1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("B,T,C", [(1, 1, 64), (2, 17, 100), (1, 3000, 300), (3, 700, 129),
                                   (8, 300, 4096), (1, 20000, 64),
                                   (2, 3000, 1000), (3, 2100, 2000)])   # few groups, many blocks: walk
def test_shapes(B, T, C, dtype, reverse):
    inp = wl.ema_inputs(B, T, C, dtype=dtype, seed=B + T + C, random_state=True)
    check(inp, dtype, reverse, f"B={B} T={T} C={C} {dtype} rev={reverse}")


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("B,T,C", [(8, 300, 4094), (8, 300, 4095), (2, 9000, 130), (1, 9000, 2), (1, 8500, 66)])
def test_bf16_walk_channel_pairs(B, T, C, reverse):
    """The bf16 walk kernel takes two neighbouring channels per lane when C is even
    (a partial last group of 128 channels at 4094, 130, 66 and 2 channels) and one per
    lane when it is odd; carried state, updated in place."""
    assert drs.ema_workspace_bytes(B, T, C, torch.bfloat16) == 0   # walk mode
    inp = wl.ema_inputs(B, T, C, dtype="bf16", seed=B + T + C, random_state=True)
    yr, sr = oracle.ema(inp["x"], inp["f"], inp["state_in"], reverse=reverse)
    st = inp["state_in"].to(DEV).clone()
    y, _ = drs.ema_forward(inp["x"].to(DEV), inp["f"].to(DEV), st, reverse=reverse, state_out=st)
    torch.cuda.synchronize()
    what = f"bf16 walk B={B} T={T} C={C} rev={reverse}"
    assert_close(y.float().cpu().numpy(), yr, RTOL["bf16"], 2, what + " y")
    assert_close(st.cpu().numpy(), sr, RTOL["bf16"], 1, what + " state")


def test_both_kernels_are_exercised():
    dt = torch.float32
    assert drs.ema_workspace_bytes(1, 3000, 300, dt) > 0      # look-back
    assert drs.ema_workspace_bytes(8, 300, 4096, dt) == 0     # walk: 512 units
    assert drs.ema_workspace_bytes(1, 20000, 64, dt) == 0     # walk: too many time blocks to fold


@pytest.mark.parametrize("T,C", [(400, 256), (300, 4096 * 2)])
def test_state_in_place(T, C):
    inp = wl.ema_inputs(2, T, C, dtype="f32", seed=5, random_state=True)
    yr, sr = oracle.ema(inp["x"], inp["f"], inp["state_in"])
    st = inp["state_in"].to(DEV).clone()
    y, s = drs.ema_forward(inp["x"].to(DEV), inp["f"].to(DEV), st, state_out=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert_close(y.cpu().numpy(), yr, RTOL["f32"], 2, "in place y")
    assert_close(st.cpu().numpy(), sr, RTOL["f32"], 1, "in place state")


def test_continuation_through_state():
    inp = wl.ema_inputs(2, 700, 200, dtype="f32", seed=6)
    x, f = inp["x"].to(DEV), inp["f"].to(DEV)
    y1, s1 = drs.ema_forward(x[:, :333].contiguous(), f[:, :333].contiguous())
    y2, s2 = drs.ema_forward(x[:, 333:].contiguous(), f[:, 333:].contiguous(), s1)
    torch.cuda.synchronize()
    yr, sr = oracle.ema(inp["x"], inp["f"])
    assert_close(torch.cat([y1, y2], 1).cpu().numpy(), yr, RTOL["f32"], 2, "continued y")
    assert_close(s2.cpu().numpy(), sr, RTOL["f32"], 1, "continued state")


@pytest.mark.parametrize("B,T,C", [(2, 900, 300), (8, 600, 4096)])
def test_bitwise_deterministic(B, T, C):
    inp = wl.ema_inputs(B, T, C, dtype="f32", seed=10, random_state=True)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_zz_no_lookback_wait_gave_up():
    assert drs.lookback_timeouts() == 0


def test_walk_beyond_one_round():
    """Fewer than 512 channel groups but more (group, block) pairs than one resident
    round: the walk kernel runs (no workspace) instead of look-back workgroups."""
    assert drs.ema_workspace_bytes(2, 3000, 1000, torch.float32) == 0
    assert drs.ema_workspace_bytes(1, 3000, 300, torch.float32) > 0     # one round: look-back
