"""GPU parity of the fused bidirectional linear-attention kernel (both scan orders
in one pass) against the fp64 oracle's forward-plus-reverse sum, and of the
composed path (two scans and a sum) where it is forced.  Tolerances: rtol 1e-5
fp32, 2e-2 bf16 (``tests/tolerance.py``).

The segment plans named per case follow the library's chunked plan (2048 target
waves, Dv / 16 waves per workgroup); the fused kernel takes plans whose segments
have at most four chunks, the composition the others.
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


def run(inp, mode, **kw):
    print(f"la_bidirectional {tuple(inp['q'].shape)} v{tuple(inp['v'].shape)} {inp['q'].dtype} {mode} {kw}",
          flush=True)
    y = drs.la_bidirectional(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"]), mode, **kw)
    torch.cuda.synchronize()
    return y


def ref(inp, mode):
    return oracle.la_bidirectional(inp["q"], inp["k"], inp["v"], inp["decay"], mode)


CASES = [
    # dtype, mode, (B, H, T, Dk, Dv): plan
    ("bf16", "head", (8, 8, 2000, 64, 64)),   # C 64, 32 chunks: 8 segments of 4 (last chunk: 16 rows)
    ("f32", "head", (2, 32, 1111, 64, 32)),   # C 32, 35 chunks: 12 segments of 3 (last: 2, 23 rows)
    ("f32", "none", (4, 16, 1000, 32, 64)),   # C 64, 16 chunks: 8 segments of 2 (last row block: 40)
    ("bf16", "none", (4, 4, 3000, 16, 16)),   # C 64, 47 chunks: one chunk per segment
    ("bf16", "head", (3, 5, 777, 32, 32)),    # 13 one-chunk segments, ragged
    ("f32", "head", (1, 2, 300, 16, 64)),     # short: a few segments
]


@pytest.mark.parametrize("dtype,mode,shape", CASES)
def test_fused_matches_oracle(dtype, mode, shape):
    B, H, T, Dk, Dv = shape
    inp = wl.la_inputs(B, H, T, Dk, Dv, dtype=dtype, mode=mode, seed=7 * T + Dk)
    y = run(inp, mode)
    assert_close(y.float().cpu().numpy(), ref(inp, mode), RTOL[dtype], 2, f"fused bidir {dtype} {mode} {shape}")
    assert drs.lookback_timeouts() == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_tiny_and_unit_factors(dtype):
    """One head per edge value of the factor: 0 (each step forgets everything before
    it), 1e-30 and 1e-12 (below fp32's reach over a chunk), 1e-3, 1/2 and 1 (no
    decay); several three-chunk segments, so the factors meet chunk and segment
    boundaries in both orders."""
    gam = torch.tensor([0.0, 1e-30, 1e-12, 1e-3, 0.5, 1.0], dtype=torch.float32)
    inp = wl.la_inputs(11, 6, 1500, 32, 64, dtype=dtype, mode="head", seed=3, gamma=gam)
    y = run(inp, "head")
    assert_close(y.float().cpu().numpy(), ref(inp, "head"), RTOL[dtype], 2, f"fused bidir edge factors {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_own_aggregates(dtype):
    """Every workgroup computes the other segments' aggregates (both orders) itself
    instead of waiting: the fallback path, to the same bar."""
    inp = wl.la_inputs(4, 16, 1000, 64, 64, dtype=dtype, mode="head", seed=11)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # a workspace of its own: the computed aggregates are counted in it
    ws = torch.zeros(drs.la_bidirectional_workspace_bytes(4, 16, 1000, 64, 64, tdt), dtype=torch.uint8, device=DEV)
    y = run(inp, "head", own_aggregates=True, workspace=ws)
    assert_close(y.float().cpu().numpy(), ref(inp, "head"), RTOL[dtype], 2, f"fused bidir own aggregates {dtype}")
    assert drs.lookback_timeouts(ws) > 0


def test_fused_deterministic():
    """The folds run in a fixed order: two calls give the same bits."""
    inp = wl.la_inputs(8, 8, 2000, 64, 64, dtype="bf16", mode="head", seed=5)
    a = run(inp, "head").clone()
    b = run(inp, "head")
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(8, 8, 2085, 64, 64), (32, 8, 600, 32, 64)])
def test_long_segment_plans_compose(shape):
    """Plans with segments of more than four chunks (33 chunks in 7 segments; 256
    units of 10 chunks in 2 segments) take the composition: the same bar."""
    B, H, T, Dk, Dv = shape
    inp = wl.la_inputs(B, H, T, Dk, Dv, dtype="bf16", mode="head", seed=T)
    y = run(inp, "head")
    assert_close(y.float().cpu().numpy(), ref(inp, "head"), RTOL["bf16"], 2, f"bidir {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["none", "head"])
def test_composed_matches_oracle(dtype, mode):
    inp = wl.la_inputs(2, 3, 1300, 64, 64, dtype=dtype, mode=mode, seed=17)
    y = run(inp, mode, compose=True)
    assert_close(y.float().cpu().numpy(), ref(inp, mode), RTOL[dtype], 2, f"composed bidir {dtype} {mode}")


def test_fused_and_composed_agree_at_workload():
    """bidir_retention_bf16 at full size: the fused kernel and the composition, both
    against the oracle on every (b, h) unit."""
    cfg = wl.LA_CONFIGS["bidir_retention_bf16"]
    inp = wl.la_config_inputs(cfg)
    r = ref(inp, cfg.mode)
    for compose in (False, True):
        y = run(inp, cfg.mode, compose=compose)
        yy = y.float().cpu().numpy()
        assert_close(yy, r, RTOL["bf16"], 2, f"bidir_retention_bf16 compose={compose}")
        record_margin(f"bidir_retention_bf16 compose={compose}", y=worst_ratio(yy, r, RTOL["bf16"], 2))


def test_concurrent_fused_calls_on_two_streams():
    """Two fused calls whose workgroups together exceed what the GPU holds at once, on
    two streams (default priority) with their own workspaces.  A segment waits on
    later segments too; one whose workgroup cannot start while the other call's
    waiting workgroups hold the compute units makes the wait run out, and the wave then
    computes the aggregate itself.  Either way both results match the oracle."""
    B, H, T, D = 8, 8, 2048, 64
    inp = wl.la_inputs(B, H, T, D, D, dtype="bf16", mode="head", seed=909)
    q, k, v, g = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["decay"])
    r = ref(inp, "head")
    need = drs.la_bidirectional_workspace_bytes(B, H, T, D, D, torch.bfloat16)
    wss = [torch.zeros(need, dtype=torch.uint8, device=DEV) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for it in range(3):
        print(f"two-stream fused bidir, round {it}", flush=True)
        outs = []
        torch.cuda.synchronize()
        for st, ws in zip(streams, wss):
            with torch.cuda.stream(st):
                outs.append(drs.la_bidirectional(q, k, v, g, "head", workspace=ws, stream=st))
        torch.cuda.synchronize()
        for i, y in enumerate(outs):
            assert_close(y.float().cpu().numpy(), r, RTOL["bf16"], 2, f"stream {i}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 64, 65])
def test_fused_short_sequences_forced_chunked(dtype, T):
    """Short sequences forced onto the chunked kernels take the fused kernel with one
    segment (T <= 64: a single, possibly partial chunk; 65: a second chunk of one row)."""
    inp = wl.la_inputs(2, 3, T, 32, 64, dtype=dtype, mode="head", seed=980 + T)
    y = run(inp, "head", force="chunked")
    assert_close(y.float().cpu().numpy(), ref(inp, "head"), RTOL[dtype], 2, f"fused bidir forced T={T} {dtype}")
