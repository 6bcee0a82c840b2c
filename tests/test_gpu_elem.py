"""GPU parity of the chunked per-key-channel decay kernel (bf16, MFMA, two
passes over time segments) against the fp64 oracle."""
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


def run(inp, reverse=False, force=None, state=True, decay=None):
    y, s, _ = drs.la_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]),
                             dev(inp["decay"]) if decay is None else decay, "elem",
                             dev(inp["state_in"]) if state else None, reverse=reverse, force=force)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), s.cpu().numpy()


def ref(inp, reverse=False, state=True):
    y, s, _ = oracle.la(inp["q"], inp["k"], inp["v"], inp["decay"], "elem",
                        inp["state_in"] if state else None, reverse=reverse)
    return y, s


def check(got, want, what):
    assert_close(got[0], want[0], RTOL["bf16"], 2, f"{what} y")
    assert_close(got[1], want[1], RTOL["bf16"], 2, f"{what} state")


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 64), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("reverse", [False, True])
def test_head_dims(Dk, Dv, reverse):
    inp = wl.la_inputs(2, 2, 333, Dk, Dv, dtype="bf16", mode="elem", seed=Dk + Dv, random_state=True)
    check(run(inp, reverse), ref(inp, reverse), f"{Dk}x{Dv} rev={reverse}")


@pytest.mark.parametrize("T", [17, 31, 32, 100, 1000, 3000])
def test_lengths(T):
    inp = wl.la_inputs(1, 3, T, 64, 32, dtype="bf16", mode="elem", seed=T, random_state=True)
    check(run(inp), ref(inp), f"T={T}")


@pytest.mark.parametrize("force", ["chunked", "recurrent"])
def test_paths_agree_with_oracle(force):
    inp = wl.la_inputs(2, 2, 200, 64, 64, dtype="bf16", mode="elem", seed=5, random_state=True)
    check(run(inp, force=force), ref(inp), force)


def test_strong_zero_and_unit_decay():
    """Factors of 0 restart a channel (up to the 2^-15 floor), 1 never decays."""
    inp = wl.la_inputs(1, 2, 300, 32, 32, dtype="bf16", mode="elem", seed=6)
    g = inp["decay"].clone()
    g[..., 0] = 0.0
    g[:, :, 150, :] = 0.0
    g[..., 1] = 1.0
    g[..., 2] = 1e-3
    g[:, :, 40:60, 3] = 0.02
    inp["decay"] = g
    check(run(inp, state=False), ref(inp, state=False), "edge factors")


def test_state_in_place():
    inp = wl.la_inputs(2, 2, 1000, 64, 64, dtype="bf16", mode="elem", seed=7, random_state=True)
    want = ref(inp)
    S = dev(inp["state_in"]).clone()
    y, s, _ = drs.la_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), "elem", S,
                             state_out=S)
    torch.cuda.synchronize()
    check((y.float().cpu().numpy(), S.cpu().numpy()), want, "in place")


def test_misaligned_factors_take_the_step_by_step_path():
    inp = wl.la_inputs(1, 2, 64, 32, 32, dtype="bf16", mode="elem", seed=8, random_state=True)
    flat = torch.empty(inp["decay"].numel() + 1, dtype=torch.float32, device=DEV)
    g = flat[1:].view(inp["decay"].shape)
    g.copy_(dev(inp["decay"]))
    assert g.data_ptr() % 16 == 4
    check(run(inp, decay=g), ref(inp), "misaligned factors")


def test_deterministic():
    inp = wl.la_inputs(2, 4, 1500, 64, 64, dtype="bf16", mode="elem", seed=9, random_state=True)
    a = run(inp)
    b = run(inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_elem_workload():
    cfg = wl.LA_CONFIGS["elem_decay_bf16"]
    inp = wl.la_config_inputs(cfg)
    got, want = run(inp, state=False), ref(inp, state=False)
    check(got, want, cfg.name)
    record_margin(cfg.name, y=worst_ratio(got[0], want[0], RTOL["bf16"], 2),
                  state=worst_ratio(got[1], want[1], RTOL["bf16"], 2))
