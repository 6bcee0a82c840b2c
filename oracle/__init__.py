"""fp64 CPU oracle for the decayed recurrences -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never does; the two share no code.

The arithmetic lives in ``oracle.c`` (plain sequential C, double precision,
one independent unit per OpenMP iteration).  This module only converts the
inputs to contiguous float64 arrays, calls the C routines through ctypes and
returns numpy arrays.

Parity status: ``la`` (every decay mode), ``la_bidirectional``, ``la_backward``,
``wkv``, ``wkv_backward``, ``ema`` and ``ema_bidirectional`` are pinned by the CPU tests
(``tests/test_oracle_la.py``, ``tests/test_oracle_wkv.py``,
``tests/test_oracle_ema.py``) against the worked examples printed on the
tensortonic exercise page, the parallel (quadratic) forms, a prefix scan built
from the published associative operator, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "_lib" / "liboracle.so"

DECAY_MODES = {"none": 0, "head": 1, "step": 2, "elem": 3}

_lib = None


def build() -> Path:
    """Compile ``oracle.c`` into ``oracle/_lib/liboracle.so`` with gcc."""
    _LIB.parent.mkdir(parents=True, exist_ok=True)
    tmp = _LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-o", str(tmp), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB.exists() or _LIB.stat().st_mtime < (_HERE / "oracle.c").stat().st_mtime:
        build()   # missing, or older than its source
    lib = ctypes.CDLL(str(_LIB))
    dp = ctypes.POINTER(ctypes.c_double)
    L, I = ctypes.c_long, ctypes.c_int
    lib.oracle_la.argtypes = [dp, dp, dp, dp, I, dp, dp, dp, dp, dp,
                              L, L, L, L, L, I, I, I]
    lib.oracle_la.restype = None
    lib.oracle_wkv.argtypes = [dp, dp, dp, dp, dp, dp, dp, L, L, L, I]
    lib.oracle_wkv.restype = None
    lib.oracle_ema.argtypes = [dp, dp, dp, dp, dp, L, L, L, I, I]
    lib.oracle_ema.restype = None
    lib.oracle_la_backward.argtypes = [dp, dp, dp, dp, I, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                       L, L, L, L, L, I, I, I]
    lib.oracle_la_backward.restype = None
    lib.oracle_wkv_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, L, L, L, I]
    lib.oracle_wkv_backward.restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    """Cores this process may use: the affinity mask, capped by OMP_NUM_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _f64(x):
    """Exact conversion to a contiguous float64 numpy array (bf16/fp32 -> fp64 is exact)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def la(q, k, v, decay=None, mode="none", state_in=None, cum_k_in=None,
       reverse=False, normalize=False, threads=None):
    """Causal decayed linear attention in fp64.

    q, k: [B,H,T,Dk]; v: [B,H,T,Dv]; decay: None, [H] (mode 'head'), [B,H,T]
    (mode 'step') or [B,H,T,Dk] (mode 'elem': one factor per key channel);
    state_in [B,H,Dk,Dv]; cum_k_in [B,H,Dk].
    Returns (y [B,H,T,Dv], state_out [B,H,Dk,Dv], cum_k_out [B,H,Dk] or None).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, H, T, Dk) and v.shape == (B, H, T, Dv)
    m = DECAY_MODES[mode]
    g = _f64(decay)
    if m == 0:
        g = None
    elif m == 1:
        assert g is not None and g.shape == (H,)
    elif m == 2:
        assert g is not None and g.shape == (B, H, T)
    else:
        assert g is not None and g.shape == (B, H, T, Dk)
    s0 = _f64(state_in)
    if s0 is not None:
        assert s0.shape == (B, H, Dk, Dv)
    z0 = _f64(cum_k_in)
    if z0 is not None:
        assert z0.shape == (B, H, Dk)
    y = np.empty((B, H, T, Dv), np.float64)
    s1 = np.empty((B, H, Dk, Dv), np.float64)
    z1 = np.empty((B, H, Dk), np.float64) if normalize else None
    lib.oracle_la(_ptr(q), _ptr(k), _ptr(v), _ptr(g), m, _ptr(s0), _ptr(z0),
                  _ptr(y), _ptr(s1), _ptr(z1), B, H, T, Dk, Dv,
                  int(bool(reverse)), int(bool(normalize)),
                  int(threads or default_threads()))
    return y, s1, z1


def wkv(w, u, k, v, state_in=None, threads=None):
    """RWKV-4 WKV recurrence in fp64.

    w, u: [C]; k, v: [B,T,C]; state_in: [3,B,C] planes (aa, bb, pp) or None.
    Returns (y [B,T,C], state_out [3,B,C]).
    """
    lib = _load()
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    B, T, C = k.shape
    assert v.shape == (B, T, C) and w.shape == (C,) and u.shape == (C,)
    s0 = _f64(state_in)
    if s0 is not None:
        assert s0.shape == (3, B, C)
    y = np.empty((B, T, C), np.float64)
    s1 = np.empty((3, B, C), np.float64)
    lib.oracle_wkv(_ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(s0), _ptr(y), _ptr(s1),
                   B, T, C, int(threads or default_threads()))
    return y, s1


def ema(x, f, state_in=None, reverse=False, threads=None):
    """Gated element-wise EMA in fp64: out_t = f_t * out_{t-1} + x_t.

    x, f: [B,T,C]; state_in: [B,C] or None (zero).  reverse visits t = T-1 .. 0.
    Returns (y [B,T,C], state_out [B,C]).
    """
    lib = _load()
    x, f = _f64(x), _f64(f)
    B, T, C = x.shape
    assert f.shape == (B, T, C)
    s0 = _f64(state_in)
    if s0 is not None:
        assert s0.shape == (B, C)
    y = np.empty((B, T, C), np.float64)
    s1 = np.empty((B, C), np.float64)
    lib.oracle_ema(_ptr(x), _ptr(f), _ptr(s0), _ptr(y), _ptr(s1), B, T, C,
                   int(bool(reverse)), int(threads or default_threads()))
    return y, s1


def la_bidirectional(q, k, v, decay=None, mode="none", normalize=False, threads=None):
    """Bidirectional linear attention: the forward and the reverse call, summed.

    RetNet issue #21 builds a bidirectional encoder by combining a call with
    reverse=False and one with reverse=True; the combination read here is the sum
    of the two outputs (each includes the current token, so the diagonal term
    appears twice).  No carried state: both directions start from zero.
    Returns y [B,H,T,Dv].
    """
    yf, _, _ = la(q, k, v, decay, mode, reverse=False, normalize=normalize, threads=threads)
    yr, _, _ = la(q, k, v, decay, mode, reverse=True, normalize=normalize, threads=threads)
    return yf + yr


def ema_bidirectional(x, f, threads=None):
    """Bidirectional gated EMA: the forward and the reverse scan from zero, summed
    (the O(TC) bidirectional encoder of RetNet issue #21).  Returns y [B,T,C]."""
    yf, _ = ema(x, f, reverse=False, threads=threads)
    yr, _ = ema(x, f, reverse=True, threads=threads)
    return yf + yr


def la_backward(q, k, v, dy, decay=None, mode="none", state_in=None, dstate_out=None,
                reverse=False, threads=None, normalize=False, cum_k_in=None, dcum_k_out=None):
    """Gradients of L = sum_t dy_t . y_t + <dstate_out, S_final> (+ <dcum_k_out,
    z_final> when normalising) for the causal decayed linear attention of ``la``,
    in fp64.

    Returns (dq, dk, dv, ddecay, dstate_in), and with normalize=True also
    dcum_k_in [B,H,Dk] as a sixth element: ddecay has the shape of ``decay``
    (mode 'head': the per-step gradients summed over batch and time; None for
    mode 'none'); dstate_in [B,H,Dk,Dv].
    """
    lib = _load()
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, H, T, Dk) and v.shape == (B, H, T, Dv) and dy.shape == (B, H, T, Dv)
    assert normalize or (cum_k_in is None and dcum_k_out is None)
    m = DECAY_MODES[mode]
    g = None if m == 0 else _f64(decay)
    s0 = _f64(state_in)
    dsf = _f64(dstate_out)
    z0 = _f64(cum_k_in)
    dzf = _f64(dcum_k_out)
    dq = np.empty((B, H, T, Dk))
    dk = np.empty((B, H, T, Dk))
    dv = np.empty((B, H, T, Dv))
    dgs = np.empty((B, H, T, Dk) if m == 3 else (B, H, T))
    ds0 = np.empty((B, H, Dk, Dv))
    dz0 = np.empty((B, H, Dk))
    lib.oracle_la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), m, _ptr(s0), _ptr(z0), _ptr(dy), _ptr(dsf),
                           _ptr(dzf), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgs), _ptr(ds0), _ptr(dz0),
                           B, H, T, Dk, Dv, int(bool(normalize)), int(bool(reverse)),
                           int(threads or default_threads()))
    if m == 0:
        dg = None
    elif m == 1:
        dg = dgs.sum(axis=(0, 2))
    else:
        dg = dgs
    if normalize:
        return dq, dk, dv, dg, ds0, dz0
    return dq, dk, dv, dg, ds0


def wkv_backward(w, u, k, v, dy, state_in=None, threads=None, return_dstate=False):
    """Gradients of L = sum_t dy_t . y_t for the WKV recurrence of ``wkv``, in fp64
    (linear form; exact while the exponents stay far from fp64's range).

    Returns (dw [C], du [C], dk [B,T,C], dv [B,T,C]); dw and du are summed over
    the batch.  With return_dstate also the gradient of the carried state given,
    [3,B,C] planes (d aa, d bb, d pp); zeros when state_in is None.
    """
    lib = _load()
    w, u, k, v, dy = _f64(w), _f64(u), _f64(k), _f64(v), _f64(dy)
    B, T, C = k.shape
    assert v.shape == (B, T, C) and dy.shape == (B, T, C) and w.shape == (C,) and u.shape == (C,)
    s0 = _f64(state_in)
    dwb = np.empty((B, C))
    dub = np.empty((B, C))
    dk = np.empty((B, T, C))
    dv = np.empty((B, T, C))
    ds = np.empty((3, B, C)) if return_dstate else None
    lib.oracle_wkv_backward(_ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(s0), _ptr(dy), _ptr(dwb), _ptr(dub),
                            _ptr(dk), _ptr(dv), _ptr(ds), B, T, C, int(threads or default_threads()))
    if return_dstate:
        return dwb.sum(axis=0), dub.sum(axis=0), dk, dv, ds
    return dwb.sum(axis=0), dub.sum(axis=0), dk, dv
