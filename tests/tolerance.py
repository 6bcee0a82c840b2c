"""Parity bar between the HIP path and the fp64 oracle.

An element x passes iff  |x - ref| <= rtol * (|ref| + rms(ref over its slice)),
where the slice is the block the element belongs to: one (b,h) [T,Dv] output,
one (b,h) [Dk,Dv] state, one (b,h) [Dk] key sum, one b's [T,C] WKV output, one
plane-and-batch [C] row of the WKV state.  rtol is 1e-5 for fp32 inputs and
2e-2 for bf16 inputs with fp32 accumulation.  The rms term keeps outputs that
cross zero from failing on a meaningless relative error; the |ref| term keeps
large elements to a true relative bound.
"""
import numpy as np

RTOL = {"f32": 1e-5, "bf16": 2e-2}


def excess(x, ref, rtol, slice_ndim):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    axes = tuple(range(ref.ndim - slice_ndim, ref.ndim))
    rms = np.sqrt(np.mean(ref ** 2, axis=axes, keepdims=True))
    bound = rtol * (np.abs(ref) + rms)
    return np.abs(x - ref) - bound, np.abs(x - ref), rms


def assert_close(x, ref, rtol, slice_ndim=2, what=""):
    ex, err, rms = excess(x, ref, rtol, slice_ndim)
    if not np.all(np.isfinite(np.asarray(x, np.float64))):
        raise AssertionError(f"{what}: non-finite values in the HIP result")
    bad = ex > 0
    if bad.any():
        i = np.unravel_index(np.argmax(ex), ex.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements outside rtol={rtol}; worst at {i}: "
            f"got {np.asarray(x, np.float64)[i]:.8g}, want {np.asarray(ref)[i]:.8g}, "
            f"err {err[i]:.3e}")


def worst_ratio(x, ref, rtol, slice_ndim=2):
    """Largest |x - ref| / bound over all elements: below 1 passes, and the
    distance to 1 is the margin left under the bar."""
    ex, err, rms = excess(x, ref, rtol, slice_ndim)
    bound = rtol * (np.abs(np.asarray(ref, np.float64)) + rms)
    return float(np.max(err / np.maximum(bound, 1e-300)))


def record_margin(name, **ratios):
    """Append one parity record (worst error / bar per output) to
    gpurun_out/parity_margins.jsonl (a run artefact, not committed), and
    return the line."""
    import json
    import os
    from pathlib import Path
    out = Path(__file__).resolve().parent.parent / "gpurun_out"
    os.makedirs(out, exist_ok=True)
    line = json.dumps({"case": name, **{k: round(v, 5) for k, v in ratios.items()}})
    with open(out / "parity_margins.jsonl", "a") as f:
        f.write(line + "\n")
    print(line)
    return line


def rel_frobenius(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))
