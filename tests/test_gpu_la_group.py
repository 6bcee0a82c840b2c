"""GPU tests of la_forward_group: several la_forward problems of one shape in one
call.  Where they share the chunked kernel they run as one launch; every result must
be bitwise that of the separate la_forward call (the same kernel, the same plan and
fold order), and the first problems are also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import decayed_recurrence_scans_amd as drs
import oracle
from decayed_recurrence_scans_amd import workloads as wl
from tests.tolerance import RTOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x):
    return None if x is None else x.to(DEV)


def problem(inp, mode, reverse, normalize):
    return dict(q=dev(inp["q"]), k=dev(inp["k"]), v=dev(inp["v"]), decay=dev(inp["decay"]), mode=mode,
                state_in=dev(inp["state_in"]), cum_k_in=dev(inp["cum_k_in"]) if normalize else None,
                reverse=reverse, normalize=normalize)


def single(pr):
    return drs.la_forward(pr["q"], pr["k"], pr["v"], pr["decay"], pr["mode"], pr["state_in"], pr["cum_k_in"],
                          reverse=pr["reverse"], normalize=pr["normalize"])


def same(a, b, what):
    for x, y in zip(a, b):
        if x is None:
            assert y is None, what
            continue
        assert torch.equal(x, y), what


@pytest.mark.parametrize("B,H,T,D,dtype,mode,normalize", [
    (8, 8, 2048, 64, "bf16", "head", False),      # the headline's forward and reverse scans
    (4, 16, 4096, 128, "bf16", "none", True),     # two-pass kernels, normalized, carried state
    (2, 3, 1000, 64, "f32", "step", False),       # ragged, fp32
    (1, 64, 4500, 64, "bf16", "head", False),     # multi-group segments, ragged
])
def test_forward_and_reverse_in_one_launch(B, H, T, D, dtype, mode, normalize):
    inp = wl.la_inputs(B, H, T, D, D, dtype=dtype, mode=mode, normalize=normalize,
                       dist="elu1" if normalize else "scaled", seed=T + D, random_state=True)
    probs = [problem(inp, mode, rev, normalize) for rev in (False, True)]
    got = drs.la_forward_group(probs)
    torch.cuda.synchronize()
    for pr, g in zip(probs, got):
        same(g, single(pr), f"{B}x{H}x{T}x{D} rev={pr['reverse']}")
    # the reverse problem against the oracle on a few units
    y = got[1][0].float().cpu().numpy()
    for b, h in [(0, 0), (B - 1, H - 1)]:
        sel = lambda x: None if x is None else x[b:b + 1, h:h + 1]
        dec = inp["decay"]
        dec = dec[h:h + 1] if mode == "head" else (dec[b:b + 1, h:h + 1] if mode == "step" else dec)
        yr, _, _ = oracle.la(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), dec, mode, sel(inp["state_in"]),
                             sel(inp["cum_k_in"]) if normalize else None, reverse=True, normalize=normalize)
        assert_close(y[b:b + 1, h:h + 1], yr, RTOL[dtype], 2, f"group reverse ({b},{h})")


def test_four_problems_with_their_own_inputs():
    """Four problems of one shape with different inputs, decays and directions."""
    B, H, T, D = 2, 4, 777, 64
    probs = []
    for i in range(4):
        inp = wl.la_inputs(B, H, T, D, D, dtype="bf16", mode="step", seed=50 + i, random_state=i % 2 == 0)
        probs.append(problem(inp, "step", i % 2 == 1, False))
    got = drs.la_forward_group(probs)
    torch.cuda.synchronize()
    for i, (pr, g) in enumerate(zip(probs, got)):
        same(g, single(pr), f"problem {i}")


def test_mixed_modes_run_one_after_another():
    """Problems that need different kernels (here per-head and per-step factors, and
    a short sequence on the step-by-step kernel) still give la_forward's results."""
    B, H, D = 2, 2, 64
    a = wl.la_inputs(B, H, 300, D, D, dtype="bf16", mode="head", seed=60)
    b = wl.la_inputs(B, H, 300, D, D, dtype="bf16", mode="step", seed=61)
    probs = [problem(a, "head", False, False), problem(b, "step", True, False)]
    got = drs.la_forward_group(probs)
    torch.cuda.synchronize()
    for pr, g in zip(probs, got):
        same(g, single(pr), "mixed")
    c = wl.la_inputs(B, H, 12, D, D, dtype="bf16", mode="head", seed=62)
    probs = [problem(c, "head", False, False), problem(c, "head", True, False)]
    got = drs.la_forward_group(probs)
    torch.cuda.synchronize()
    for pr, g in zip(probs, got):
        same(g, single(pr), "short")


def test_in_place_state_and_own_aggregates_in_a_group():
    """A problem updating its state in place (start-order ids within its own slice of
    the workspace) next to one that computes every earlier aggregate itself."""
    B, H, T, D = 2, 8, 3000, 64
    inp = wl.la_inputs(B, H, T, D, D, dtype="bf16", mode="head", seed=70, random_state=True)
    ref_y, ref_s, _ = single(problem(inp, "head", False, False))
    st = dev(inp["state_in"]).clone()
    p0 = problem(inp, "head", False, False)
    p0["state_in"] = st
    p0["state_out"] = st
    ws = torch.zeros(drs.la_forward_group_workspace_bytes(2, B, H, T, D, D), dtype=torch.uint8, device=DEV)
    p1 = problem(inp, "head", True, False)
    got = drs.la_forward_group([p0, p1], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got[0][0], ref_y) and torch.equal(st, ref_s)
    same(got[1], single(p1), "reverse next to in place")


def test_repeated_group_calls_rearm_every_slice():
    B, H, T, D = 2, 8, 2048, 64
    inp = wl.la_inputs(B, H, T, D, D, dtype="bf16", mode="head", seed=80)
    probs = [problem(inp, "head", rev, False) for rev in (False, True, False)]
    ws = torch.zeros(drs.la_forward_group_workspace_bytes(3, B, H, T, D, D), dtype=torch.uint8, device=DEV)
    first = drs.la_forward_group(probs, workspace=ws)
    first = [tuple(None if x is None else x.clone() for x in g) for g in first]
    for _ in range(3):
        again = drs.la_forward_group(probs, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        same(a, b, "repeat")
    assert drs.lookback_timeouts(ws) == 0


def test_graph_replays_match_eager():
    """The headline step captured into one HIP graph (two grouped calls on rotating
    inputs, the workspace created on the capture stream beforehand) and replayed
    several times, with eager calls on the same workspace in between: every replay's
    outputs are bitwise those of the eager calls, so the look-back flags and epochs
    stay valid across replays."""
    B, H, T, D = 4, 8, 2048, 64
    before = drs.lookback_timeouts()
    sets = []
    for seed in (1, 2):
        inp = wl.la_inputs(B, H, T, D, D, dtype="bf16", mode="head", seed=seed)
        sets.append(dict(q=dev(inp["q"]), k=dev(inp["k"]), v=dev(inp["v"]), decay=dev(inp["decay"])))
    outs = [[torch.empty(B, H, T, D, device=DEV, dtype=torch.bfloat16) for _ in range(2)] for _ in sets]

    def step(i):
        st = sets[i]
        drs.la_forward_group([dict(q=st["q"], k=st["k"], v=st["v"], decay=st["decay"], mode="head",
                                   reverse=rev, y=outs[i][j]) for j, rev in enumerate((False, True))])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in (0, 1, 0, 1):
            step(i)
        s.synchronize()
        want = [[y.clone() for y in o] for o in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step(0)
            step(1)
        for rep in range(4):
            for o in outs:
                for y in o:
                    y.zero_()
            g.replay()
            s.synchronize()
            for i in range(2):
                for j in range(2):
                    assert torch.equal(outs[i][j], want[i][j]), f"replay {rep} set {i} direction {j}"
            step(rep % 2)          # eager work on the same workspace between the replays
            s.synchronize()
            assert torch.equal(outs[rep % 2][0], want[rep % 2][0]), f"eager call after replay {rep}"
    torch.cuda.synchronize()
    assert drs.lookback_timeouts() == before   # no wait ran out in the replays
