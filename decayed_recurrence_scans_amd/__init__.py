"""decayed_recurrence_scans_amd -- Python binding of libdrs (MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in ``include/drs.h``: device
pointers of PyTorch tensors and torch's current HIP stream go in, status codes
come out (raised as :class:`DrsError`).  PyTorch is used only to allocate
device memory for outputs that the caller does not pass; every step of the
computation runs in the HIP kernels of ``libdrs.so``.  There is no fallback:
if the library is missing or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

__all__ = [
    "la_forward", "la_forward_noalloc", "la_workspace_bytes", "wkv_forward", "wkv_workspace_bytes", "ema_forward",
    "ema_workspace_bytes", "la_bidirectional", "la_bidirectional_workspace_bytes",
    "ema_bidirectional", "ema_bidirectional_workspace_bytes", "la_backward", "la_backward_workspace_bytes",
    "wkv_backward", "wkv_backward_workspace_bytes",
    "status_string", "version",
    "library_path", "load_library", "DrsError",
    "DRS_F32", "DRS_BF16", "DRS_DECAY_NONE", "DRS_DECAY_HEAD", "DRS_DECAY_STEP", "DRS_DECAY_ELEM",
    "DRS_REVERSE", "DRS_NORMALIZE", "DRS_FORCE_SEQ", "DRS_FORCE_SCAN", "DRS_FORCE_CHAIN",
    "DRS_FORCE_RECURRENT", "DRS_FORCE_CHUNKED", "DRS_LA_OWN_AGGREGATES", "DRS_WKV_OWN_AGGREGATES", "DRS_LA_COMPOSE",
    "DRS_FORCE_ROWS", "DRS_MAX_GROUP", "la_forward_group", "la_forward_group_workspace_bytes", "LAProblem",
    "lookback_timeouts",
]

# mirrors of include/drs.h
DRS_OK, DRS_ERR_INVALID, DRS_ERR_UNSUPPORTED, DRS_ERR_WORKSPACE, DRS_ERR_DEVICE, DRS_ERR_SCRATCH = range(6)
DRS_NOALLOC_SCRATCH_BYTES = 64 << 20
DRS_F32, DRS_BF16 = 0, 1
DRS_DECAY_NONE, DRS_DECAY_HEAD, DRS_DECAY_STEP, DRS_DECAY_ELEM = 0, 1, 2, 3
DRS_REVERSE = 0x1
DRS_NORMALIZE = 0x2
DRS_FORCE_SEQ = 0x100
DRS_FORCE_SCAN = 0x200
DRS_FORCE_CHAIN = 0x400
DRS_FORCE_RECURRENT = 0x800
DRS_FORCE_CHUNKED = 0x1000
DRS_LA_OWN_AGGREGATES = 0x2000
DRS_WKV_OWN_AGGREGATES = 0x4000
DRS_FORCE_ROWS = 0x8000
DRS_LA_COMPOSE = 0x10000
DRS_MAX_GROUP = 4

_MODES = {"none": DRS_DECAY_NONE, "head": DRS_DECAY_HEAD, "step": DRS_DECAY_STEP, "elem": DRS_DECAY_ELEM}
_LA_FORCE = {None: 0, "recurrent": DRS_FORCE_RECURRENT, "chunked": DRS_FORCE_CHUNKED}
_PKG = Path(__file__).resolve().parent
_LIB_PATH = _PKG / "_lib" / "libdrs.so"
_lib = None


class DrsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> Path:
    return _LIB_PATH


def load_library():
    """Load libdrs.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(
            f"libdrs.so not found at {_LIB_PATH}; build it first "
            "(python -m decayed_recurrence_scans_amd._build)")
    lib = ctypes.CDLL(str(_LIB_PATH))
    vp, fp, I, U, S = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.la_forward.argtypes = [vp, vp, vp, I, fp, I, fp, fp, vp, fp, fp, I, I, I, I, I, I, U, vp, S, vp]
    lib.la_forward.restype = I
    lib.la_forward_noalloc.argtypes = [vp, vp, vp, I, fp, I, fp, fp, vp, fp, fp, I, I, I, I, I, I, U, vp]
    lib.la_forward_noalloc.restype = I
    lib.la_forward_group_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, U]
    lib.la_forward_group_workspace_bytes.restype = S
    lib.la_forward_group.argtypes = [ctypes.POINTER(LAProblem), I, I, I, I, I, I, I, I, vp, S, vp]
    lib.la_forward_group.restype = I
    lib.la_workspace_bytes.argtypes = [I, I, I, I, I, I, I, U]
    lib.la_workspace_bytes.restype = S
    lib.wkv_forward.argtypes = [fp, fp, fp, fp, fp, fp, fp, I, I, I, U, vp, S, vp]
    lib.wkv_forward.restype = I
    lib.wkv_workspace_bytes.argtypes = [I, I, I, U]
    lib.wkv_workspace_bytes.restype = S
    lib.ema_forward.argtypes = [vp, vp, I, fp, vp, fp, I, I, I, U, vp, S, vp]
    lib.ema_forward.restype = I
    lib.ema_workspace_bytes.argtypes = [I, I, I, I, U]
    lib.ema_workspace_bytes.restype = S
    lib.la_bidirectional.argtypes = [vp, vp, vp, I, fp, I, vp, I, I, I, I, I, I, U, vp, S, vp]
    lib.la_bidirectional.restype = I
    lib.la_bidirectional_workspace_bytes.argtypes = [I, I, I, I, I, I, I, U]
    lib.la_bidirectional_workspace_bytes.restype = S
    lib.ema_bidirectional.argtypes = [vp, vp, I, vp, I, I, I, U, vp, S, vp]
    lib.ema_bidirectional.restype = I
    lib.ema_bidirectional_workspace_bytes.argtypes = [I, I, I, I, U]
    lib.ema_bidirectional_workspace_bytes.restype = S
    lib.la_backward.argtypes = [vp, vp, vp, I, fp, I, fp, fp, fp, vp, fp, fp, vp, vp, vp, fp, fp, fp,
                                I, I, I, I, I, I, U, vp, S, vp]
    lib.la_backward.restype = I
    lib.la_backward_workspace_bytes.argtypes = [I, I, I, I, I, I, I, U]
    lib.la_backward_workspace_bytes.restype = S
    lib.wkv_backward.argtypes = [fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, I, I, I, U, vp, S, vp]
    lib.wkv_backward.restype = I
    lib.wkv_backward_workspace_bytes.argtypes = [I, I, I, U]
    lib.wkv_backward_workspace_bytes.restype = S
    lib.drs_status_string.argtypes = [I]
    lib.drs_status_string.restype = ctypes.c_char_p
    lib.drs_version.argtypes = []
    lib.drs_version.restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().drs_status_string(int(status)).decode()


def version() -> int:
    return load_library().drs_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# Zero-filled workspaces, one per (device, stream), shared by la_forward and
# wkv_forward: calls on one stream are ordered, and every launch leaves the
# look-back counters (the first 256 bytes) re-armed for the next one.
_ws_cache = {}


class LAProblem(ctypes.Structure):
    """``drs_la_problem`` of the C ABI (one problem of ``la_forward_group``)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("decay", ctypes.c_void_p), ("mode", ctypes.c_int), ("state_in", ctypes.c_void_p),
                ("cum_k_in", ctypes.c_void_p), ("y", ctypes.c_void_p), ("state_out", ctypes.c_void_p),
                ("cum_k_out", ctypes.c_void_p), ("flags", ctypes.c_uint)]


def _workspace(nbytes, device, stream):
    handle = (stream or torch.cuda.current_stream()).cuda_stream
    key = (device.index, handle)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def lookback_timeouts(workspace=None) -> int:
    """Look-back waits that ran out (counter 3 of the workspace, and words 35, 19, 51
    for the further problems of a group call), summed over the cached workspaces or read from
    the one given.  For linear attention this
    counts the earlier segments' aggregates that a wave computed itself
    (after its wait ran out, or all of them with own_aggregates=True); for the
    WKV and EMA chained kernels, waits that gave up.  Synchronises the device."""
    bufs = [workspace] if workspace is not None else list(_ws_cache.values())
    # word 3 of each problem's counters (la_forward_group: problem i's start at word 0, 32, 16, 48)
    return sum(int(b[:256].view(torch.int32)[[3, 35, 19, 51]].sum().item()) for b in bufs)


def la_workspace_bytes(B, H, T, Dk, Dv, dtype=torch.bfloat16, chunk=0, force=None) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    return int(load_library().la_workspace_bytes(int(B), int(H), int(T), int(Dk), int(Dv), dt,
                                                 int(chunk), _LA_FORCE[force]))


def _check_decay(decay, m, B, H, T, Dk):
    decay = _dev(decay, "decay", torch.float32)
    if decay is not None:
        want = {DRS_DECAY_HEAD: (H,), DRS_DECAY_STEP: (B, H, T), DRS_DECAY_ELEM: (B, H, T, Dk)}.get(m)
        if want is not None and tuple(decay.shape) != want:
            raise ValueError(f"decay must have shape {want}")
    return decay


def la_forward(q, k, v, decay=None, mode="none", state_in=None, cum_k_in=None, *,
               reverse=False, normalize=False, chunk=0, y=None, state_out=None,
               cum_k_out=None, return_state=True, workspace=None, stream=None, force=None,
               own_aggregates=False):
    """Causal decayed linear attention (``la_forward`` of the C ABI).

    q, k [B,H,T,Dk], v [B,H,T,Dv] (float32 or bfloat16, same dtype); decay fp32
    [H] (mode 'head'), [B,H,T] (mode 'step') or [B,H,T,Dk] (mode 'elem');
    state_in fp32 [B,H,Dk,Dv]; cum_k_in fp32 [B,H,Dk] (with normalize).  Outputs
    not passed in are allocated; state_out / cum_k_out may be the very tensors
    passed as state_in / cum_k_in (in-place update, e.g. a decode step).
    force: None, 'recurrent' or 'chunked' pins the kernel path.  own_aggregates: every
    time segment of the chunked kernel computes the earlier segments' aggregates
    itself instead of waiting for them (DRS_LA_OWN_AGGREGATES; slow, for tests).  workspace: a zero-filled uint8 GPU tensor of at least
    la_workspace_bytes(...) bytes, or None for a cached one per (device, stream).
    Returns (y, state_out, cum_k_out); the last two are None when not requested.
    """
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dt = DRS_BF16 if q.dtype == torch.bfloat16 else DRS_F32
    q = _dev(q, "q")
    k = _dev(k, "k", q.dtype)
    v = _dev(v, "v", q.dtype)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, T, Dk) or tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("shape mismatch between q, k and v")
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    decay = _check_decay(decay, m, B, H, T, Dk)
    state_in = _dev(state_in, "state_in", torch.float32)
    cum_k_in = _dev(cum_k_in, "cum_k_in", torch.float32)
    if y is None:
        y = torch.empty((B, H, T, Dv), dtype=q.dtype, device=q.device)
    y = _dev(y, "y", q.dtype)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    state_out = _dev(state_out, "state_out", torch.float32)
    if cum_k_out is None and return_state and normalize:
        cum_k_out = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    cum_k_out = _dev(cum_k_out, "cum_k_out", torch.float32)
    flags = (DRS_REVERSE if reverse else 0) | (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    flags |= DRS_LA_OWN_AGGREGATES if own_aggregates else 0
    lib = load_library()
    need = int(lib.la_workspace_bytes(B, H, T, Dk, Dv, dt, int(chunk), flags))
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_forward(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(decay), m, _ptr(state_in), _ptr(cum_k_in),
        _ptr(y), _ptr(state_out), _ptr(cum_k_out), B, H, T, Dk, Dv, int(chunk), flags,
        _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "la_forward")
    return y, state_out, cum_k_out


def la_forward_group_workspace_bytes(count, B, H, T, Dk, Dv, dtype=torch.bfloat16, chunk=0, normalize=False) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    return int(load_library().la_forward_group_workspace_bytes(int(count), int(B), int(H), int(T), int(Dk), int(Dv),
                                                               dt, int(chunk), DRS_NORMALIZE if normalize else 0))


def la_forward_group(problems, *, chunk=0, workspace=None, stream=None):
    """``la_forward_group`` of the C ABI: up to DRS_MAX_GROUP la_forward problems of
    one shape in one call (one launch when they share the chunked kernel).

    problems: dicts with q, k, v and optionally decay, mode, state_in, cum_k_in,
    reverse, normalize, y, state_out, cum_k_out, return_state (as la_forward takes
    them).  workspace: a uint8 GPU tensor of at least la_forward_group_workspace_bytes
    bytes whose first 256 bytes are zero before first use (it may be la_forward's), or
    None for the cached one per (device, stream).  Returns a list of (y, state_out,
    cum_k_out), one per problem.
    """
    if not 1 <= len(problems) <= DRS_MAX_GROUP:
        raise ValueError(f"1 to {DRS_MAX_GROUP} problems")
    q0 = problems[0]["q"]
    if q0.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dt = DRS_BF16 if q0.dtype == torch.bfloat16 else DRS_F32
    B, H, T, Dk = q0.shape
    Dv = problems[0]["v"].shape[-1]
    arr = (LAProblem * len(problems))()
    outs, keep, union = [], [], 0
    for i, pr in enumerate(problems):
        q = _dev(pr["q"], "q", q0.dtype)
        k = _dev(pr["k"], "k", q0.dtype)
        v = _dev(pr["v"], "v", q0.dtype)
        if tuple(q.shape) != (B, H, T, Dk) or tuple(k.shape) != (B, H, T, Dk) or tuple(v.shape) != (B, H, T, Dv):
            raise ValueError("every problem of a group has the same shapes")
        mode = pr.get("mode", "none")
        m = _MODES[mode] if isinstance(mode, str) else int(mode)
        decay = _check_decay(pr.get("decay"), m, B, H, T, Dk)
        normalize = bool(pr.get("normalize", False))
        ret = pr.get("return_state", True)
        state_in = _dev(pr.get("state_in"), "state_in", torch.float32)
        cum_k_in = _dev(pr.get("cum_k_in"), "cum_k_in", torch.float32)
        y = pr.get("y")
        y = _dev(torch.empty((B, H, T, Dv), dtype=q.dtype, device=q.device) if y is None else y, "y", q.dtype)
        so = pr.get("state_out")
        if so is None and ret:
            so = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
        so = _dev(so, "state_out", torch.float32)
        zo = pr.get("cum_k_out")
        if zo is None and ret and normalize:
            zo = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
        zo = _dev(zo, "cum_k_out", torch.float32)
        flags = (DRS_REVERSE if pr.get("reverse") else 0) | (DRS_NORMALIZE if normalize else 0)
        union |= flags
        addr = lambda t: None if t is None else t.data_ptr()
        arr[i] = LAProblem(addr(q), addr(k), addr(v), addr(decay), m, addr(state_in), addr(cum_k_in), addr(y),
                           addr(so), addr(zo), flags)
        keep += [q, k, v, decay, state_in, cum_k_in]
        outs.append((y, so, zo))
    lib = load_library()
    n = len(problems)
    stream = stream or torch.cuda.current_stream()
    handle = stream.cuda_stream
    need = int(lib.la_forward_group_workspace_bytes(n, B, H, T, Dk, Dv, dt, int(chunk), union))
    if workspace is None and need:
        workspace = _workspace(need, q0.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_forward_group(arr, n, dt, B, H, T, Dk, Dv, int(chunk), _ptr(workspace), wbytes,
                              ctypes.c_void_p(handle))
    if st != DRS_OK:
        raise DrsError(st, "la_forward_group")
    return outs


def la_forward_noalloc(q, k, v, decay=None, mode="none", state_in=None, cum_k_in=None, *, y,
                       state_out=None, cum_k_out=None, reverse=False, normalize=False, chunk=0,
                       stream=None, force=None):
    """``la_forward_noalloc`` of the C ABI: la_forward with the library's static
    scratch instead of a workspace, for callers that cannot allocate.  Every output
    is the caller's (y is required; state_out / cum_k_out are written when given),
    so this function allocates nothing either.  Calls overlapping on one GPU race."""
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dt = DRS_BF16 if q.dtype == torch.bfloat16 else DRS_F32
    q = _dev(q, "q")
    k = _dev(k, "k", q.dtype)
    v = _dev(v, "v", q.dtype)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, T, Dk) or tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("shape mismatch between q, k and v")
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    decay = _check_decay(decay, m, B, H, T, Dk)
    y = _dev(y, "y", q.dtype)
    if tuple(y.shape) != (B, H, T, Dv):
        raise ValueError("y must have shape [B,H,T,Dv]")
    args = [_dev(t, n, torch.float32) for t, n in ((state_in, "state_in"), (cum_k_in, "cum_k_in"),
                                                    (state_out, "state_out"), (cum_k_out, "cum_k_out"))]
    flags = (DRS_REVERSE if reverse else 0) | (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    st = load_library().la_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(decay), m, _ptr(args[0]), _ptr(args[1]), _ptr(y),
        _ptr(args[2]), _ptr(args[3]), B, H, T, Dk, Dv, int(chunk), flags, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "la_forward_noalloc")
    return y, args[2], args[3]


def wkv_workspace_bytes(B, T, C, flags=0) -> int:
    return int(load_library().wkv_workspace_bytes(int(B), int(T), int(C), int(flags)))


def wkv_forward(w, u, k, v, state_in=None, *, force=None, y=None, state_out=None,
                return_state=True, workspace=None, stream=None, own_aggregates=False):
    """RWKV-4 WKV (``wkv_forward`` of the C ABI), fp32.

    w, u [C]; k, v [B,T,C]; state_in [3,B,C] planes (aa, bb, pp) or None.
    force: None, 'seq', 'scan', 'chain' or 'rows' (the row-owning sweep, never
    chosen by itself; C % 4 == 0).  own_aggregates: in the chained kernel and the
    row-owning sweep every time block computes the earlier blocks' aggregates itself
    instead of waiting for them (DRS_WKV_OWN_AGGREGATES; slow, for tests).  workspace: a
    uint8 GPU tensor of at least wkv_workspace_bytes(...) bytes whose first 256
    bytes are zero before its first use, or None for the cached one per (device,
    stream).  Returns (y, state_out).
    """
    w = _dev(w, "w", torch.float32)
    u = _dev(u, "u", torch.float32)
    k = _dev(k, "k", torch.float32)
    v = _dev(v, "v", torch.float32)
    B, T, C = k.shape
    if tuple(v.shape) != (B, T, C) or tuple(w.shape) != (C,) or tuple(u.shape) != (C,):
        raise ValueError("shape mismatch between w, u, k and v")
    state_in = _dev(state_in, "state_in", torch.float32)
    flags = {None: 0, "seq": DRS_FORCE_SEQ, "scan": DRS_FORCE_SCAN, "chain": DRS_FORCE_CHAIN,
             "rows": DRS_FORCE_ROWS}[force]
    flags |= DRS_WKV_OWN_AGGREGATES if own_aggregates else 0
    if y is None:
        y = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    y = _dev(y, "y", torch.float32)
    if state_out is None and return_state:
        state_out = torch.empty((3, B, C), dtype=torch.float32, device=k.device)
    state_out = _dev(state_out, "state_out", torch.float32)
    need = wkv_workspace_bytes(B, T, C, flags)
    if workspace is None and need:
        workspace = _workspace(need, k.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().wkv_forward(
        _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in), _ptr(y), _ptr(state_out),
        B, T, C, flags, _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "wkv_forward")
    return y, state_out


def ema_workspace_bytes(B, T, C, dtype=torch.float32, reverse=False) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    return int(load_library().ema_workspace_bytes(int(B), int(T), int(C), dt,
                                                  DRS_REVERSE if reverse else 0))


def ema_forward(x, f, state_in=None, *, reverse=False, y=None, state_out=None,
                return_state=True, workspace=None, stream=None):
    """Gated element-wise EMA y_t = f_t * y_{t-1} + x_t (``ema_forward`` of the C ABI).

    x, f [B,T,C] (float32 or bfloat16, same dtype); state_in fp32 [B,C] or None.
    workspace: a uint8 GPU tensor of at least ema_workspace_bytes(...) bytes whose
    first 256 bytes are zero before its first use, or None for the cached one.
    Returns (y, state_out).
    """
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    dt = DRS_BF16 if x.dtype == torch.bfloat16 else DRS_F32
    x = _dev(x, "x")
    f = _dev(f, "f", x.dtype)
    B, T, C = x.shape
    if tuple(f.shape) != (B, T, C):
        raise ValueError("shape mismatch between x and f")
    state_in = _dev(state_in, "state_in", torch.float32)
    if y is None:
        y = torch.empty((B, T, C), dtype=x.dtype, device=x.device)
    y = _dev(y, "y", x.dtype)
    if state_out is None and return_state:
        state_out = torch.empty((B, C), dtype=torch.float32, device=x.device)
    state_out = _dev(state_out, "state_out", torch.float32)
    flags = DRS_REVERSE if reverse else 0
    lib = load_library()
    need = int(lib.ema_workspace_bytes(B, T, C, dt, flags))
    if workspace is None and need:
        workspace = _workspace(need, x.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ema_forward(_ptr(x), _ptr(f), dt, _ptr(state_in), _ptr(y), _ptr(state_out),
                         B, T, C, flags, _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "ema_forward")
    return y, state_out


def la_bidirectional_workspace_bytes(B, H, T, Dk, Dv, dtype=torch.bfloat16, chunk=0, normalize=False,
                                     force=None) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    flags = (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    return int(load_library().la_bidirectional_workspace_bytes(int(B), int(H), int(T), int(Dk), int(Dv),
                                                               dt, int(chunk), flags))


def la_bidirectional(q, k, v, decay=None, mode="none", *, normalize=False, chunk=0, y=None,
                     workspace=None, stream=None, force=None, compose=False, own_aggregates=False):
    """Forward plus reverse linear attention from zero state (``la_bidirectional``).

    Arguments as la_forward without states.  compose: the two scans and a sum
    instead of the fused kernel (DRS_LA_COMPOSE).  own_aggregates: the fused or
    chunked kernels compute the other segments' aggregates themselves (slow, for
    tests).  workspace: a uint8 GPU tensor of at least
    la_bidirectional_workspace_bytes(...) bytes whose first 256 bytes are zero
    before its first use, or None for the cached one.  Returns y.
    """
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dt = DRS_BF16 if q.dtype == torch.bfloat16 else DRS_F32
    q = _dev(q, "q")
    k = _dev(k, "k", q.dtype)
    v = _dev(v, "v", q.dtype)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, T, Dk) or tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("shape mismatch between q, k and v")
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    decay = _check_decay(decay, m, B, H, T, Dk)
    if y is None:
        y = torch.empty((B, H, T, Dv), dtype=q.dtype, device=q.device)
    y = _dev(y, "y", q.dtype)
    flags = (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    flags |= (DRS_LA_COMPOSE if compose else 0) | (DRS_LA_OWN_AGGREGATES if own_aggregates else 0)
    lib = load_library()
    need = int(lib.la_bidirectional_workspace_bytes(B, H, T, Dk, Dv, dt, int(chunk), flags))
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_bidirectional(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(decay), m, _ptr(y), B, H, T, Dk, Dv,
                              int(chunk), flags, _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "la_bidirectional")
    return y


def ema_bidirectional_workspace_bytes(B, T, C, dtype=torch.float32) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    return int(load_library().ema_bidirectional_workspace_bytes(int(B), int(T), int(C), dt, 0))


def ema_bidirectional(x, f, *, y=None, workspace=None, stream=None):
    """Forward plus reverse gated EMA from zero (``ema_bidirectional``).  Returns y."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    dt = DRS_BF16 if x.dtype == torch.bfloat16 else DRS_F32
    x = _dev(x, "x")
    f = _dev(f, "f", x.dtype)
    B, T, C = x.shape
    if tuple(f.shape) != (B, T, C):
        raise ValueError("shape mismatch between x and f")
    if y is None:
        y = torch.empty((B, T, C), dtype=x.dtype, device=x.device)
    y = _dev(y, "y", x.dtype)
    lib = load_library()
    need = int(lib.ema_bidirectional_workspace_bytes(B, T, C, dt, 0))
    if workspace is None and need:
        workspace = _workspace(need, x.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ema_bidirectional(_ptr(x), _ptr(f), dt, _ptr(y), B, T, C, 0, _ptr(workspace), wbytes,
                               _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "ema_bidirectional")
    return y


def la_backward_workspace_bytes(B, H, T, Dk, Dv, dtype=torch.bfloat16, chunk=0, reverse=False, force=None,
                                normalize=False) -> int:
    dt = DRS_BF16 if dtype == torch.bfloat16 else DRS_F32
    flags = (DRS_REVERSE if reverse else 0) | (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    return int(load_library().la_backward_workspace_bytes(int(B), int(H), int(T), int(Dk), int(Dv), dt,
                                                          int(chunk), flags))


def la_backward(q, k, v, dy, decay=None, mode="none", state_in=None, state_out=None, dstate_out=None, *,
                reverse=False, normalize=False, cum_k_in=None, dcum_k_out=None, chunk=0, need_ddecay=True,
                need_dstate_in=True, dq=None, dk=None, dv=None, workspace=None, stream=None, force=None):
    """Gradients of sum_t dy_t . y_t + <dstate_out, S_final> (+ <dcum_k_out, z_final>
    when normalising) for la_forward (``la_backward`` of the C ABI).

    q, k, v, decay, state_in, cum_k_in, reverse, normalize, chunk: as given to
    la_forward; state_out: that call's final state (needed on the chunked path for
    the decay gradient when dstate_out is given); dy [B,H,T,Dv] in q's dtype;
    dstate_out fp32 [B,H,Dk,Dv] or None; dcum_k_out fp32 [B,H,Dk] or None.
    Returns (dq, dk, dv, ddecay, dstate_in), and with normalize=True also
    dcum_k_in [B,H,Dk] (None when not needed) as a sixth element: ddecay has
    decay's shape (None for mode 'none' or need_ddecay=False), dstate_in fp32
    [B,H,Dk,Dv] (None when not needed).  workspace: a uint8 GPU tensor of at
    least la_backward_workspace_bytes(...) bytes whose first 256 bytes are zero
    before its first use, or None for the cached one.
    """
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q must be float32 or bfloat16")
    dt = DRS_BF16 if q.dtype == torch.bfloat16 else DRS_F32
    q = _dev(q, "q")
    k = _dev(k, "k", q.dtype)
    v = _dev(v, "v", q.dtype)
    dy = _dev(dy, "dy", q.dtype)
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, T, Dk) or tuple(v.shape[:3]) != (B, H, T) or tuple(dy.shape) != tuple(v.shape):
        raise ValueError("shape mismatch between q, k, v and dy")
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    decay = _check_decay(decay, m, B, H, T, Dk)
    state_in = _dev(state_in, "state_in", torch.float32)
    cum_k_in = _dev(cum_k_in, "cum_k_in", torch.float32)
    state_out = _dev(state_out, "state_out", torch.float32)
    dstate_out = _dev(dstate_out, "dstate_out", torch.float32)
    dcum_k_out = _dev(dcum_k_out, "dcum_k_out", torch.float32)
    dq = _dev(dq if dq is not None else torch.empty_like(q), "dq", q.dtype)
    dk = _dev(dk if dk is not None else torch.empty_like(k), "dk", q.dtype)
    dv = _dev(dv if dv is not None else torch.empty_like(v), "dv", q.dtype)
    ddecay = torch.empty_like(decay) if (need_ddecay and decay is not None) else None
    dstate_in = (torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
                 if need_dstate_in else None)
    dcum_k_in = (torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
                 if (normalize and need_dstate_in) else None)
    flags = (DRS_REVERSE if reverse else 0) | (DRS_NORMALIZE if normalize else 0) | _LA_FORCE[force]
    lib = load_library()
    need = int(lib.la_backward_workspace_bytes(B, H, T, Dk, Dv, dt, int(chunk), flags))
    if workspace is None and need:
        workspace = _workspace(need, q.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_backward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(decay), m, _ptr(state_in), _ptr(cum_k_in),
                         _ptr(state_out), _ptr(dy), _ptr(dstate_out), _ptr(dcum_k_out), _ptr(dq), _ptr(dk),
                         _ptr(dv), _ptr(ddecay), _ptr(dstate_in), _ptr(dcum_k_in), B, H, T, Dk, Dv, int(chunk),
                         flags, _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "la_backward")
    if normalize:
        return dq, dk, dv, ddecay, dstate_in, dcum_k_in
    return dq, dk, dv, ddecay, dstate_in


def wkv_backward_workspace_bytes(B, T, C) -> int:
    return int(load_library().wkv_backward_workspace_bytes(int(B), int(T), int(C), 0))


def wkv_backward(w, u, k, v, dy, state_in=None, *, need_dw=True, need_du=True, dk=None, dv=None,
                 need_dstate_in=False, workspace=None, stream=None):
    """Gradients of sum_t dy_t y_t for wkv_forward (``wkv_backward`` of the C ABI).

    dy [B,T,C] (the outputs are recomputed).  Returns (dw [C], du [C], dk, dv),
    and with need_dstate_in also the gradient of state_in, [3,B,C] planes (d aa,
    d bb, d pp; zeros for state_in None); dw / du are None when not requested.
    workspace: a uint8 GPU tensor of at least wkv_backward_workspace_bytes(B, T, C)
    bytes, or None for the cached one.
    """
    w = _dev(w, "w", torch.float32)
    u = _dev(u, "u", torch.float32)
    k = _dev(k, "k", torch.float32)
    v = _dev(v, "v", torch.float32)
    dy = _dev(dy, "dy", torch.float32)
    B, T, C = k.shape
    for name, t in (("v", v), ("dy", dy)):
        if tuple(t.shape) != (B, T, C):
            raise ValueError(f"{name} must have shape {(B, T, C)}")
    if tuple(w.shape) != (C,) or tuple(u.shape) != (C,):
        raise ValueError("w and u must have shape (C,)")
    state_in = _dev(state_in, "state_in", torch.float32)
    dk = _dev(dk if dk is not None else torch.empty_like(k), "dk", torch.float32)
    dv = _dev(dv if dv is not None else torch.empty_like(v), "dv", torch.float32)
    dw = torch.empty_like(w) if need_dw else None
    du = torch.empty_like(u) if need_du else None
    ds = torch.empty((3, B, C), dtype=torch.float32, device=k.device) if need_dstate_in else None
    need = wkv_backward_workspace_bytes(B, T, C)
    if workspace is None:
        workspace = _workspace(need, k.device, stream)
    workspace = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    st = load_library().wkv_backward(_ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state_in), _ptr(dy),
                                     _ptr(dw), _ptr(du), _ptr(dk), _ptr(dv), _ptr(ds), B, T, C, 0,
                                     _ptr(workspace), wbytes, _stream(stream))
    if st != DRS_OK:
        raise DrsError(st, "wkv_backward")
    if need_dstate_in:
        return dw, du, dk, dv, ds
    return dw, du, dk, dv
