"""la_forward_noalloc -- the entry point for callers that cannot allocate -- called
through the C ABI (ctypes) and compared with la_forward on the same inputs: two
calls in a row, the second with a smaller input, then the other paths.  The two
entry points run the same kernels with the same plan, so the outputs must be
bitwise equal; both are also checked against the fp64 oracle at the usual bar."""
import ctypes

import numpy as np
import pytest
import torch

import decayed_recurrence_scans_amd as drs
import oracle
from decayed_recurrence_scans_amd import workloads as wl
from tests.tolerance import RTOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(c):
    """Runs one case through la_forward_noalloc and through la_forward (own zeroed
    workspace); returns the inputs and the two sets of outputs (CPU)."""
    lib = drs.load_library()
    B, H, T, Dk, Dv = c["B"], c["H"], c["T"], c["Dk"], c["Dv"]
    norm, mode = c["normalize"], c["mode"]
    inp = wl.la_inputs(B, H, T, Dk, Dv, dtype=c["dtype"], mode=mode, normalize=norm,
                       dist="elu1" if norm else "scaled", seed=c["seed"], random_state=True)
    g = lambda n: None if inp[n] is None else inp[n].to(DEV)
    q, k, v, dec, s0 = g("q"), g("k"), g("v"), g("decay"), g("state_in")
    z0 = g("cum_k_in") if norm else None
    dt = drs.DRS_BF16 if q.dtype == torch.bfloat16 else drs.DRS_F32
    m = {"none": 0, "head": 1, "step": 2, "elem": 3}[mode]
    flags = (drs.DRS_REVERSE if c["reverse"] else 0) | (drs.DRS_NORMALIZE if norm else 0)
    outs = []
    for entry in ("noalloc", "workspace"):
        y = torch.full((B, H, T, Dv), float("nan"), dtype=q.dtype, device=DEV)
        s = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device=DEV)
        z = torch.full((B, H, Dk), float("nan"), dtype=torch.float32, device=DEV) if norm else None
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = (ptr(q), ptr(k), ptr(v), dt, ptr(dec), m, ptr(s0), ptr(z0), ptr(y), ptr(s), ptr(z),
                B, H, T, Dk, Dv, 0, flags)
        if entry == "noalloc":
            st = lib.la_forward_noalloc(*args, stream)
        else:
            need = lib.la_workspace_bytes(B, H, T, Dk, Dv, dt, 0, flags & ~(drs.DRS_REVERSE | drs.DRS_NORMALIZE))
            ws = torch.zeros(max(int(need), 256), dtype=torch.uint8, device=DEV)
            st = lib.la_forward(*args, ptr(ws), ws.numel(), stream)
        assert st == drs.DRS_OK, f"{entry}: {drs.status_string(st)}"
        torch.cuda.synchronize()
        outs.append((y.float().cpu().numpy(), s.cpu().numpy(), None if z is None else z.cpu().numpy()))
    return inp, outs


def compare(c, inp, outs):
    (y1, s1, z1), (y2, s2, z2) = outs
    what = f"{c}"
    assert np.array_equal(y1, y2), what + ": y differs from la_forward's"
    assert np.array_equal(s1, s2), what + ": state differs from la_forward's"
    if z1 is not None:
        assert np.array_equal(z1, z2), what + ": key sum differs from la_forward's"
    ref = oracle.la(inp["q"], inp["k"], inp["v"], inp["decay"], c["mode"], inp["state_in"],
                    inp["cum_k_in"] if c["normalize"] else None, reverse=c["reverse"], normalize=c["normalize"])
    rt = RTOL[c["dtype"]]
    assert_close(y1, ref[0], rt, 2, what + " y")
    assert_close(s1, ref[1], rt, 2, what + " state")
    if z1 is not None:
        assert_close(z1, ref[2], rt, 1, what + " key sum")


def test_noalloc_two_calls_second_smaller():
    """The retention workload's shape, then a smaller per-step, normalized, reversed
    call in fp32: the second call runs on the scratch the first one left."""
    cases = [
        dict(B=8, H=8, T=2048, Dk=64, Dv=64, dtype="bf16", mode="head", normalize=False, reverse=False, seed=21),
        dict(B=2, H=3, T=500, Dk=32, Dv=64, dtype="f32", mode="step", normalize=True, reverse=True, seed=22),
    ]
    for c in cases:
        inp, outs = both(c)
        compare(c, inp, outs)


def test_noalloc_other_paths():
    """Per-key-channel factors (their own chunked kernel on the scratch), a decode
    step (no scratch), and the D = 128 two-pass kernel after them."""
    cases = [
        dict(B=1, H=2, T=300, Dk=64, Dv=64, dtype="bf16", mode="elem", normalize=False, reverse=False, seed=23),
        dict(B=3, H=2, T=1, Dk=128, Dv=128, dtype="bf16", mode="head", normalize=True, reverse=False, seed=24),
        dict(B=2, H=4, T=3000, Dk=128, Dv=128, dtype="bf16", mode="step", normalize=True, reverse=False, seed=25),
    ]
    for c in cases:
        inp, outs = both(c)
        compare(c, inp, outs)
