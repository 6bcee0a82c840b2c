"""GPU parity of the step-by-step linear-attention path (decode steps, short
sequences, per-key-channel decay) and of the bidirectional sums, against the
fp64 oracle (``tests/tolerance.py``: rtol 1e-5 fp32, 2e-2 bf16).
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


def dev(x):
    return None if x is None else x.to(DEV)


def gpu_la(inp, mode, normalize, reverse=False, force=None, state=True):
    y, s, z = drs.la_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), mode,
                             dev(inp["state_in"]) if state else None,
                             dev(inp["cum_k_in"]) if (state and normalize) else None,
                             reverse=reverse, normalize=normalize, force=force)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), s.cpu().numpy(), None if z is None else z.cpu().numpy()


def ref_la(inp, mode, normalize, reverse=False, state=True):
    return oracle.la(inp["q"], inp["k"], inp["v"], inp["decay"], mode,
                     inp["state_in"] if state else None,
                     inp["cum_k_in"] if (state and normalize) else None,
                     reverse=reverse, normalize=normalize)


def check(got, ref, dtype, normalize, what):
    rtol = RTOL[dtype]
    assert_close(got[0], ref[0], rtol, 2, f"{what} y")
    assert_close(got[1], ref[1], rtol, 2, f"{what} state")
    if normalize:
        assert_close(got[2], ref[2], rtol, 1, f"{what} cum_k")


def inputs(B, H, T, Dk, Dv, dtype, mode, normalize, seed):
    return wl.la_inputs(B, H, T, Dk, Dv, dtype=dtype, mode=mode, normalize=normalize,
                        dist="elu1" if normalize else "scaled", seed=seed, random_state=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["none", "head", "step", "elem"])
@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("T,reverse", [(1, False), (3, True), (16, False)])
def test_short_sequences(dtype, mode, normalize, T, reverse):
    inp = inputs(3, 2, T, 64, 32, dtype, mode, normalize, seed=100 + T)
    got = gpu_la(inp, mode, normalize, reverse)
    check(got, ref_la(inp, mode, normalize, reverse), dtype, normalize, f"T={T} {mode}")


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (16, 128), (128, 16), (32, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_dims(Dk, Dv, dtype):
    inp = inputs(2, 3, 5, Dk, Dv, dtype, "step", True, seed=Dk * 7 + Dv)
    check(gpu_la(inp, "step", True), ref_la(inp, "step", True), dtype, True, f"{Dk}x{Dv}")


@pytest.mark.parametrize("T", [17, 150, 333])
@pytest.mark.parametrize("mode", ["head", "elem"])
def test_forced_recurrent_long(T, mode):
    inp = inputs(2, 2, T, 64, 64, "bf16", mode, True, seed=T)
    got = gpu_la(inp, mode, True, force="recurrent")
    check(got, ref_la(inp, mode, True), "bf16", True, f"recurrent T={T}")


def test_forced_chunked_short():
    inp = inputs(2, 2, 7, 64, 64, "bf16", "step", True, seed=3)
    check(gpu_la(inp, "step", True, force="chunked"), ref_la(inp, "step", True), "bf16", True, "chunked T=7")


@pytest.mark.parametrize("reverse", [False, True])
def test_elem_mode_long_sequence(reverse):
    """Per-key-channel decay over a long sequence (default path)."""
    inp = inputs(1, 4, 700, 32, 64, "bf16", "elem", False, seed=11)
    check(gpu_la(inp, "elem", False, reverse), ref_la(inp, "elem", False, reverse), "bf16", False,
          "elem T=700")


def test_elem_mode_strong_and_zero_decay():
    inp = inputs(1, 2, 40, 16, 16, "f32", "elem", False, seed=12)
    g = inp["decay"].clone()
    g[..., 0] = 0.0          # channel 0 forgets everything each step
    g[:, :, 20, :] = 0.0     # every channel restarts at t = 20
    g[..., 1] = 1.0          # channel 1 never decays
    inp["decay"] = g
    check(gpu_la(inp, "elem", False), ref_la(inp, "elem", False), "f32", False, "elem edge")


def test_elem_with_forced_chunked_is_unsupported():
    inp = inputs(1, 1, 8, 16, 16, "f32", "elem", False, seed=13)
    with pytest.raises(drs.DrsError) as e:
        gpu_la(inp, "elem", False, force="chunked")
    assert e.value.status == drs.DRS_ERR_UNSUPPORTED


@pytest.mark.parametrize("T", [1, 9, 2500])
def test_state_and_key_sum_in_place(T):
    """state_out / cum_k_out are the very tensors passed in (both paths)."""
    inp = inputs(2, 4, T, 64, 64, "bf16", "head", True, seed=20 + T)
    ref = ref_la(inp, "head", True)
    S = dev(inp["state_in"]).clone()
    z = dev(inp["cum_k_in"]).clone()
    y, s1, z1 = drs.la_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), "head",
                               S, z, normalize=True, state_out=S, cum_k_out=z)
    torch.cuda.synchronize()
    assert s1.data_ptr() == S.data_ptr() and z1.data_ptr() == z.data_ptr()
    check((y.float().cpu().numpy(), S.cpu().numpy(), z.cpu().numpy()), ref, "bf16", True, f"in place T={T}")


@pytest.mark.parametrize("mode", ["head", "elem"])
def test_prefill_then_decode_steps(mode):
    """A prompt through the chunked path, then one token at a time with the state
    and key sum updated in place, equals the oracle on the whole sequence."""
    P, N = 300, 6
    full = inputs(2, 2, P + N, 64, 64, "bf16", mode, True, seed=31)
    ref = oracle.la(full["q"], full["k"], full["v"], full["decay"], mode, full["state_in"],
                    full["cum_k_in"], normalize=True)

    q, k, v = (dev(full[n]) for n in ("q", "k", "v"))
    dec = dev(full["decay"])
    S = dev(full["state_in"]).clone()
    z = dev(full["cum_k_in"]).clone()
    dslice = (lambda a, b: dec) if mode == "head" else (lambda a, b: dec[:, :, a:b].contiguous())
    y0, _, _ = drs.la_forward(q[:, :, :P].contiguous(), k[:, :, :P].contiguous(), v[:, :, :P].contiguous(),
                              dslice(0, P), mode, S, z, normalize=True, state_out=S, cum_k_out=z)
    ys = [y0]
    for t in range(P, P + N):
        yt, _, _ = drs.la_forward(q[:, :, t:t + 1].contiguous(), k[:, :, t:t + 1].contiguous(),
                                  v[:, :, t:t + 1].contiguous(), dslice(t, t + 1), mode, S, z,
                                  normalize=True, state_out=S, cum_k_out=z)
        ys.append(yt)
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2).float().cpu().numpy()
    check((y, S.cpu().numpy(), z.cpu().numpy()), ref, "bf16", True, f"prefill+decode {mode}")


def test_decode_workload():
    """The decode workload at full size: 1024 (b, h) states, one token each."""
    cfg = wl.LA_CONFIGS["decode_bf16"]
    inp = wl.la_config_inputs(cfg)
    ref = ref_la(inp, cfg.mode, cfg.normalize)
    S = dev(inp["state_in"])
    z = dev(inp["cum_k_in"])
    y, _, _ = drs.la_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), cfg.mode,
                             S, z, normalize=True, state_out=S, cum_k_out=z)
    torch.cuda.synchronize()
    got = (y.float().cpu().numpy(), S.cpu().numpy(), z.cpu().numpy())
    check(got, ref, "bf16", True, "decode_bf16")
    rt = RTOL["bf16"]
    record_margin("decode_bf16", y=worst_ratio(got[0], ref[0], rt, 2), state=worst_ratio(got[1], ref[1], rt, 2),
                  cum_k=worst_ratio(got[2], ref[2], rt, 1))


# ---- bidirectional sums ---------------------------------------------------------

BIDIR_RTOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,normalize", [("none", False), ("head", False), ("step", True), ("elem", False)])
@pytest.mark.parametrize("T", [5, 700])
def test_la_bidirectional(dtype, mode, normalize, T):
    inp = wl.la_inputs(2, 2, T, 32, 64, dtype=dtype, mode=mode, normalize=normalize,
                       dist="elu1" if normalize else "scaled", seed=40 + T)
    y = drs.la_bidirectional(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), mode,
                             normalize=normalize)
    torch.cuda.synchronize()
    ref = oracle.la_bidirectional(inp["q"], inp["k"], inp["v"], inp["decay"], mode, normalize=normalize)
    assert_close(y.float().cpu().numpy(), ref, BIDIR_RTOL[dtype], 2, f"bidir {mode} T={T}")


def test_la_bidirectional_workload():
    cfg = wl.LA_CONFIGS["bidir_retention_bf16"]
    inp = wl.la_config_inputs(cfg)
    y = drs.la_bidirectional(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), cfg.mode)
    torch.cuda.synchronize()
    ref = oracle.la_bidirectional(inp["q"], inp["k"], inp["v"], inp["decay"], cfg.mode)
    assert_close(y.float().cpu().numpy(), ref, BIDIR_RTOL["bf16"], 2, "bidir_retention_bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 300, 70), (1, 5000, 64),      # two calls and an add
                                   (8, 1024, 4096), (8, 333, 4100), (4, 5000, 8192),  # fused kernel
                                   (8, 333, 4101), (2, 9000, 130),   # fused: bf16 single channels, pairs
                                   (512, 3, 64), (2, 3000, 1000)])
def test_ema_bidirectional(dtype, B, T, C):
    inp = wl.ema_inputs(B, T, C, dtype=dtype, seed=T + C)
    y = drs.ema_bidirectional(dev(inp["x"]), dev(inp["f"]))
    torch.cuda.synchronize()
    ref = oracle.ema_bidirectional(inp["x"], inp["f"])
    assert_close(y.float().cpu().numpy(), ref, BIDIR_RTOL[dtype], 2, f"ema bidir {B}x{T}x{C}")


def test_ema_bidirectional_workload():
    """bidir_ema_bf16 at full size (the fused kernel), against the oracle everywhere."""
    cfg = wl.EMA_CONFIGS["bidir_ema_bf16"]
    inp = wl.ema_config_inputs(cfg)
    y = drs.ema_bidirectional(dev(inp["x"]), dev(inp["f"])).float().cpu().numpy()
    ref = oracle.ema_bidirectional(inp["x"], inp["f"])
    assert_close(y, ref, BIDIR_RTOL[cfg.dtype], 2, cfg.name)
    record_margin(cfg.name, y=worst_ratio(y, ref, BIDIR_RTOL[cfg.dtype], 2))


def test_bidirectional_then_chunked_call_shares_workspace():
    """The bidirectional tail never overwrites the counters that the next look-back
    call of the same (cached) workspace relies on."""
    a = wl.la_inputs(1, 2, 4, 64, 64, dtype="bf16", mode="head", seed=50)
    drs.la_bidirectional(dev(a["q"]), dev(a["k"]), dev(a["v"]), dev(a["decay"]), "head")
    b = wl.la_inputs(2, 4, 3000, 64, 64, dtype="bf16", mode="head", seed=51)
    got = gpu_la(b, "head", False, state=False)
    check(got, ref_la(b, "head", False, state=False), "bf16", False, "after bidir")
    assert drs.lookback_timeouts() == 0
