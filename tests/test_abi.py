"""The C ABI library builds, loads, exports every declared symbol, and rejects
bad arguments on the host -- all without a GPU (no call here launches work:
each one fails validation before any HIP call)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

import decayed_recurrence_scans_amd as drs

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "drs.h"


@pytest.fixture(scope="module")
def lib():
    if not drs.library_path().exists():
        from decayed_recurrence_scans_amd import _build
        _build.build()
    return drs.load_library()


def declared_functions():
    text = HEADER.read_text()
    return re.findall(r"DRS_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_constants_match_the_binding():
    """Every flag the header defines has the same value in the Python binding, and
    no two flags share a bit."""
    defs = dict(re.findall(r"#define\s+(DRS_[A-Z_]+)\s+(0x[0-9a-fA-F]+)u", HEADER.read_text()))
    assert "DRS_LA_OWN_AGGREGATES" in defs and len(defs) >= 8
    seen = 0
    for name, val in defs.items():
        v = int(val, 16)
        assert getattr(drs, name) == v, name
        assert v & (v - 1) == 0 and not (seen & v), name
        seen |= v


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) >= {"la_forward", "la_workspace_bytes", "wkv_forward", "wkv_workspace_bytes",
                          "ema_forward", "ema_workspace_bytes", "la_bidirectional",
                          "la_bidirectional_workspace_bytes", "ema_bidirectional",
                          "ema_bidirectional_workspace_bytes", "la_backward", "la_backward_workspace_bytes",
                          "wkv_backward", "wkv_backward_workspace_bytes",
                          "drs_status_string", "drs_version"}


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(drs.library_path())],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    for code in range(6):
        assert drs.status_string(code) != "unknown status"
    assert drs.status_string(99) == "unknown status"
    assert drs.version() >= 100


# a fake, 16-byte aligned, never dereferenced address
P = ctypes.c_void_p(0x1000)
P2 = ctypes.c_void_p(0x2000)
P3 = ctypes.c_void_p(0x3000)
P4 = ctypes.c_void_p(0x4000)
N = None


WS = ctypes.c_void_p(0x100000)


# T = 300 takes the chunked path, which needs a workspace: every case below must
# fail validation (none may reach a launch).
def la(lib, q=P, k=P2, v=P3, dt=1, decay=N, mode=0, s_in=N, z_in=N, y=P4, s_out=N, z_out=N,
       B=2, H=2, T=300, Dk=64, Dv=64, chunk=0, flags=0, ws=WS, wsb=1 << 40):
    return lib.la_forward(q, k, v, dt, decay, mode, s_in, z_in, y, s_out, z_out,
                          B, H, T, Dk, Dv, chunk, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=N), drs.DRS_ERR_INVALID),
    (dict(y=N), drs.DRS_ERR_INVALID),
    (dict(B=0), drs.DRS_ERR_INVALID),
    (dict(H=-1), drs.DRS_ERR_INVALID),
    (dict(T=0), drs.DRS_ERR_INVALID),
    (dict(dt=7), drs.DRS_ERR_INVALID),
    (dict(mode=1), drs.DRS_ERR_INVALID),                       # HEAD without decay
    (dict(mode=0, decay=ctypes.c_void_p(0x5000)), drs.DRS_ERR_INVALID),
    (dict(mode=4, decay=ctypes.c_void_p(0x5000)), drs.DRS_ERR_INVALID),
    (dict(mode=3), drs.DRS_ERR_INVALID),                       # ELEM without decay
    (dict(flags=0x8), drs.DRS_ERR_INVALID),
    (dict(z_in=ctypes.c_void_p(0x5000)), drs.DRS_ERR_INVALID),  # cum_k without NORMALIZE
    (dict(flags=drs.DRS_LA_OWN_AGGREGATES, ws=N), drs.DRS_ERR_WORKSPACE),   # a known flag: checks go on
    (dict(flags=drs.DRS_FORCE_RECURRENT | drs.DRS_FORCE_CHUNKED), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_SEQ), drs.DRS_ERR_INVALID),        # a WKV flag
    (dict(mode=3, decay=ctypes.c_void_p(0x5000), dt=0, flags=drs.DRS_FORCE_CHUNKED),
     drs.DRS_ERR_UNSUPPORTED),                                  # per-channel factors, chunked: bf16 only
    (dict(mode=3, decay=ctypes.c_void_p(0x5000), z_in=ctypes.c_void_p(0x6000),
          flags=drs.DRS_FORCE_CHUNKED | drs.DRS_NORMALIZE), drs.DRS_ERR_UNSUPPORTED),
    (dict(mode=3, decay=ctypes.c_void_p(0x5004), flags=drs.DRS_FORCE_CHUNKED),
     drs.DRS_ERR_UNSUPPORTED),                                  # chunked factors need 16-byte alignment
    (dict(mode=3, decay=ctypes.c_void_p(0x5000), ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(T=1 << 24, Dv=128, flags=drs.DRS_FORCE_RECURRENT), drs.DRS_ERR_UNSUPPORTED),   # y over 2^31 B
    (dict(T=4, Dk=24), drs.DRS_ERR_UNSUPPORTED),                 # step-by-step path, bad Dk
    (dict(T=4, chunk=48), drs.DRS_ERR_UNSUPPORTED),
    (dict(y=P), drs.DRS_ERR_INVALID),                           # y aliases q
    (dict(q=ctypes.c_void_p(0x1008)), drs.DRS_ERR_INVALID),     # misaligned
    (dict(Dk=24), drs.DRS_ERR_UNSUPPORTED),
    (dict(Dv=256), drs.DRS_ERR_UNSUPPORTED),
    (dict(chunk=48), drs.DRS_ERR_UNSUPPORTED),
    (dict(ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(wsb=100), drs.DRS_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100008)), drs.DRS_ERR_INVALID),   # misaligned workspace
])
def test_la_forward_rejects(lib, kw, want):
    assert la(lib, **kw) == want


def la_na(lib, q=P, k=P2, v=P3, dt=1, decay=N, mode=0, s_in=N, z_in=N, y=P4, s_out=N, z_out=N,
          B=2, H=2, T=300, Dk=64, Dv=64, chunk=0, flags=0):
    return lib.la_forward_noalloc(q, k, v, dt, decay, mode, s_in, z_in, y, s_out, z_out,
                                  B, H, T, Dk, Dv, chunk, flags, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=N), drs.DRS_ERR_INVALID),
    (dict(B=0), drs.DRS_ERR_INVALID),
    (dict(mode=1), drs.DRS_ERR_INVALID),
    (dict(flags=0x8), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_SEQ), drs.DRS_ERR_INVALID),
    (dict(y=P), drs.DRS_ERR_INVALID),
    (dict(q=ctypes.c_void_p(0x1008)), drs.DRS_ERR_INVALID),
    (dict(Dk=24), drs.DRS_ERR_UNSUPPORTED),
    (dict(chunk=48), drs.DRS_ERR_UNSUPPORTED),
    # more scratch than the static buffer: 4096 units of Dk = Dv = 128 (one segment
    # each, 8 slots of 8.7 KB per unit: 285 MB), and per-key-channel factors at 1024 units
    (dict(B=64, H=64, T=4096, Dk=128, Dv=128), drs.DRS_ERR_SCRATCH),
    (dict(B=32, H=32, T=4096, Dk=128, Dv=128, mode=3, decay=ctypes.c_void_p(0x5000)), drs.DRS_ERR_SCRATCH),
])
def test_la_forward_noalloc_rejects(lib, kw, want):
    """Argument checks of la_forward, then the static scratch's limit; all before
    any HIP call."""
    assert la_na(lib, **kw) == want


def test_noalloc_limit_matches_the_workspace_query(lib):
    """The limit is the header's, and the scratch need of a call is the workspace
    query's figure for its path (an upper bound): the workloads fit."""
    text = HEADER.read_text()
    assert re.search(r"#define\s+DRS_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)64 << 20\)", text)
    assert drs.DRS_NOALLOC_SCRATCH_BYTES == 64 << 20
    for shape in [(8, 8, 2048, 64, 64), (4, 16, 16384, 128, 128), (4, 16, 4096, 128, 128)]:
        assert 0 < lib.la_workspace_bytes(*shape, 1, 0, 0) <= drs.DRS_NOALLOC_SCRATCH_BYTES
    assert lib.la_workspace_bytes(64, 64, 4096, 128, 128, 1, 0, 0) > drs.DRS_NOALLOC_SCRATCH_BYTES


def la_bi(lib, q=P, k=P2, v=P3, dt=1, decay=N, mode=0, y=P4, B=2, H=2, T=300, Dk=64, Dv=64, chunk=0,
          flags=0, ws=WS, wsb=1 << 40):
    return lib.la_bidirectional(q, k, v, dt, decay, mode, y, B, H, T, Dk, Dv, chunk, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=N), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_REVERSE), drs.DRS_ERR_INVALID),
    (dict(flags=0x8), drs.DRS_ERR_INVALID),
    (dict(y=P2), drs.DRS_ERR_INVALID),
    (dict(Dv=48), drs.DRS_ERR_UNSUPPORTED),
    (dict(ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(T=4, ws=N), drs.DRS_ERR_WORKSPACE),                     # the second output needs room
    (dict(T=4, wsb=1024), drs.DRS_ERR_WORKSPACE),
])
def test_la_bidirectional_rejects(lib, kw, want):
    assert la_bi(lib, **kw) == want


def ema_bi(lib, x=P, f=P2, dt=0, y=ctypes.c_void_p(0x6000), B=2, T=8, C=64, flags=0, ws=N, wsb=0):
    return lib.ema_bidirectional(x, f, dt, y, B, T, C, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=N), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_REVERSE), drs.DRS_ERR_INVALID),
    (dict(y=P), drs.DRS_ERR_INVALID),
    (dict(ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x7000), wsb=256 + 2 * 8 * 64 * 4 - 4), drs.DRS_ERR_WORKSPACE),
])
def test_ema_bidirectional_rejects(lib, kw, want):
    assert ema_bi(lib, **kw) == want


def test_bidirectional_workspace_queries(lib):
    import torch
    la_ws = drs.la_workspace_bytes(8, 8, 2048, 64, 64)
    y_bytes = 8 * 8 * 2048 * 64 * 2
    assert drs.la_bidirectional_workspace_bytes(8, 8, 2048, 64, 64) == la_ws + y_bytes
    # short sequences: no scan workspace, the second output after the 256 counter bytes
    assert drs.la_bidirectional_workspace_bytes(2, 2, 4, 64, 64) == 256 + 2 * 2 * 4 * 64 * 2
    assert drs.ema_workspace_bytes(8, 2048, 4096, torch.bfloat16) == 0      # walk kernel: none
    # enough channels: the fused kernel, block summaries of both directions only
    assert drs.ema_bidirectional_workspace_bytes(8, 2048, 4096, torch.bfloat16) == 256 + 8 * 64 * 16 * 5 * 64 * 4
    n = drs.ema_workspace_bytes(1, 3000, 300, torch.bfloat16)
    assert drs.ema_bidirectional_workspace_bytes(1, 3000, 300, torch.bfloat16) == n + 3000 * 300 * 2
    assert lib.ema_bidirectional_workspace_bytes(1, 8, 8, 0, drs.DRS_REVERSE) == 0
    assert lib.la_bidirectional_workspace_bytes(1, 1, 8, 64, 48, 1, 0, 0) == 0


P5, P6, P7, P8 = (ctypes.c_void_p(a) for a in (0x8000, 0x9000, 0xa000, 0xb000))


def la_bwd(lib, q=P, k=P2, v=P3, dt=1, decay=N, mode=0, s_in=N, z_in=N, s_out=N, dy=P4, dsf=N, dzf=N, dq=P5,
           dk=P6, dv=P7, ddec=N, ds0=N, dz0=N, B=2, H=2, T=300, Dk=64, Dv=64, chunk=0, flags=0, ws=WS,
           wsb=1 << 40):
    return lib.la_backward(q, k, v, dt, decay, mode, s_in, z_in, s_out, dy, dsf, dzf, dq, dk, dv, ddec, ds0, dz0,
                           B, H, T, Dk, Dv, chunk, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(dy=N), drs.DRS_ERR_INVALID),
    (dict(dv=N), drs.DRS_ERR_INVALID),
    (dict(T=0), drs.DRS_ERR_INVALID),
    (dict(ddec=P8), drs.DRS_ERR_INVALID),                        # no factors to differentiate
    (dict(mode=1, decay=P8, ddec=ctypes.c_void_p(0xc000), dsf=ctypes.c_void_p(0xd000)),
     drs.DRS_ERR_INVALID),                                       # decay gradient needs the final state
    (dict(dq=P), drs.DRS_ERR_INVALID),                           # output aliases an input
    (dict(dk=P5), drs.DRS_ERR_INVALID),                          # two outputs alias
    (dict(dq=ctypes.c_void_p(0x8008)), drs.DRS_ERR_INVALID),     # misaligned
    (dict(flags=drs.DRS_FORCE_RECURRENT | drs.DRS_FORCE_CHUNKED), drs.DRS_ERR_INVALID),
    (dict(z_in=ctypes.c_void_p(0xe000)), drs.DRS_ERR_INVALID),  # key sum without DRS_NORMALIZE
    (dict(dz0=ctypes.c_void_p(0xe000)), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_NORMALIZE, dz0=P), drs.DRS_ERR_INVALID),    # output aliases an input
    (dict(flags=drs.DRS_NORMALIZE, ws=N), drs.DRS_ERR_WORKSPACE),   # normalised: the step-by-step path
    (dict(flags=drs.DRS_NORMALIZE, z_in=ctypes.c_void_p(0xe000), dzf=ctypes.c_void_p(0xf000), ws=N),
     drs.DRS_ERR_WORKSPACE),
    (dict(mode=3, decay=P8, ddec=ctypes.c_void_p(0xc000), ws=N), drs.DRS_ERR_WORKSPACE),   # per channel
    # the step-by-step path recomputes the final state: no state_out needed
    (dict(mode=1, decay=P8, ddec=ctypes.c_void_p(0xc000), dsf=ctypes.c_void_p(0xd000),
          flags=drs.DRS_FORCE_RECURRENT, ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(flags=drs.DRS_NORMALIZE, Dv=48), drs.DRS_ERR_UNSUPPORTED),
    (dict(Dk=48), drs.DRS_ERR_UNSUPPORTED),
    (dict(ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(wsb=4096), drs.DRS_ERR_WORKSPACE),
])
def test_la_backward_rejects(lib, kw, want):
    assert la_bwd(lib, **kw) == want


def test_la_backward_workspace_query(lib):
    n = drs.la_backward_workspace_bytes(8, 8, 2048, 64, 64)
    assert n > drs.la_workspace_bytes(8, 8, 2048, 64, 64) and n % 256 == 0
    assert drs.la_backward_workspace_bytes(2, 2, 8, 64, 64) > 256        # helpers even without scan scratch
    assert lib.la_backward_workspace_bytes(2, 2, 8, 64, 40, 1, 0, 0) == 0
    # the normalised backward stores dy / den and the denominator gradient per step
    units, T, Dk, Dv = 4 * 16, 4096, 128, 128
    norm = drs.la_backward_workspace_bytes(4, 16, T, Dk, Dv, normalize=True)
    assert norm >= units * T * (Dk + Dv + 1) * 4 and norm % 256 == 0


def wkv_bwd(lib, w=P, u=P2, k=P3, v=P4, s_in=N, dy=P6, dw=N, du=N, dk=P7, dv=P8, ds=N, B=2, T=8, C=64,
            flags=0, ws=WS, wsb=1 << 40):
    return lib.wkv_backward(w, u, k, v, s_in, dy, dw, du, dk, dv, ds, B, T, C, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(dy=N), drs.DRS_ERR_INVALID),
    (dict(dk=N), drs.DRS_ERR_INVALID),
    (dict(C=0), drs.DRS_ERR_INVALID),
    (dict(flags=1), drs.DRS_ERR_INVALID),
    (dict(dk=P3), drs.DRS_ERR_INVALID),                           # output aliases an input
    (dict(dv=P7), drs.DRS_ERR_INVALID),                           # two outputs alias
    (dict(dw=ctypes.c_void_p(0xc000), du=ctypes.c_void_p(0xc000)), drs.DRS_ERR_INVALID),
    (dict(ds=P7), drs.DRS_ERR_INVALID),                           # state gradient aliases dk
    (dict(ds=ctypes.c_void_p(0xd000), s_in=ctypes.c_void_p(0xd000)), drs.DRS_ERR_INVALID),   # ... the state
    (dict(ds=ctypes.c_void_p(0xd002)), drs.DRS_ERR_INVALID),     # misaligned
    (dict(k=ctypes.c_void_p(0x3002)), drs.DRS_ERR_INVALID),
    (dict(B=70000), drs.DRS_ERR_UNSUPPORTED),
    (dict(T=1 << 20, C=1024), drs.DRS_ERR_UNSUPPORTED),          # a batch row over 2^31 bytes
    (dict(ws=N), drs.DRS_ERR_WORKSPACE),
    (dict(wsb=1024), drs.DRS_ERR_WORKSPACE),
])
def test_wkv_backward_rejects(lib, kw, want):
    assert wkv_bwd(lib, **kw) == want


def test_wkv_backward_workspace_query(lib):
    n = drs.wkv_backward_workspace_bytes(8, 1024, 4096)
    assert n == 256 + 8 * (1024 // 64) * 6 * 4096 * 8 + 2 * 8 * 4096 * 4   # checkpoints, partials
    assert lib.wkv_backward_workspace_bytes(8, 10, 10, 1) == 0
    assert lib.wkv_backward_workspace_bytes(0, 10, 10, 0) == 0


def wkv(lib, w=P, u=P2, k=P3, v=P4, s_in=N, y=ctypes.c_void_p(0x6000), s_out=N, B=2, T=8, C=64,
        flags=0, ws=N, wsb=0):
    return lib.wkv_forward(w, u, k, v, s_in, y, s_out, B, T, C, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(w=N), drs.DRS_ERR_INVALID),
    (dict(y=N), drs.DRS_ERR_INVALID),
    (dict(B=0), drs.DRS_ERR_INVALID),
    (dict(T=0), drs.DRS_ERR_INVALID),
    (dict(C=-3), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_SEQ | drs.DRS_FORCE_SCAN), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_SCAN | drs.DRS_FORCE_CHAIN), drs.DRS_ERR_INVALID),
    (dict(flags=0x4), drs.DRS_ERR_INVALID),
    (dict(y=P3), drs.DRS_ERR_INVALID),                          # y aliases k
    (dict(k=ctypes.c_void_p(0x3002)), drs.DRS_ERR_INVALID),     # misaligned float
    (dict(flags=drs.DRS_FORCE_SCAN), drs.DRS_ERR_WORKSPACE),    # no workspace
    (dict(flags=drs.DRS_FORCE_SCAN, ws=ctypes.c_void_p(0x7000), wsb=16), drs.DRS_ERR_WORKSPACE),
    (dict(flags=drs.DRS_FORCE_CHAIN), drs.DRS_ERR_WORKSPACE),   # no workspace
    (dict(T=300), drs.DRS_ERR_WORKSPACE),                       # default: chained path needs one
    (dict(flags=drs.DRS_FORCE_CHAIN, ws=ctypes.c_void_p(0x7008), wsb=1 << 20), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_CHAIN, T=100000, C=64), drs.DRS_ERR_UNSUPPORTED),   # too many time blocks
    (dict(B=70000), drs.DRS_ERR_UNSUPPORTED),
    (dict(flags=drs.DRS_FORCE_ROWS | drs.DRS_FORCE_CHAIN), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_FORCE_ROWS), drs.DRS_ERR_WORKSPACE),    # no workspace
    (dict(flags=drs.DRS_FORCE_ROWS, C=66), drs.DRS_ERR_UNSUPPORTED),               # C % 4 != 0
    (dict(flags=drs.DRS_FORCE_ROWS, k=ctypes.c_void_p(0x3004)), drs.DRS_ERR_UNSUPPORTED),   # 16-byte pieces
    (dict(flags=drs.DRS_FORCE_ROWS, s_in=ctypes.c_void_p(0x8000), s_out=ctypes.c_void_p(0x8000)),
     drs.DRS_ERR_UNSUPPORTED),                                  # state updated in place
])
def test_wkv_forward_rejects(lib, kw, want):
    assert wkv(lib, **kw) == want


def ema(lib, x=P, f=P2, dt=0, s_in=N, y=ctypes.c_void_p(0x6000), s_out=N, B=2, T=8, C=64, flags=0,
        ws=N, wsb=0):
    return lib.ema_forward(x, f, dt, s_in, y, s_out, B, T, C, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=N), drs.DRS_ERR_INVALID),
    (dict(y=N), drs.DRS_ERR_INVALID),
    (dict(B=0), drs.DRS_ERR_INVALID),
    (dict(T=-1), drs.DRS_ERR_INVALID),
    (dict(dt=7), drs.DRS_ERR_INVALID),
    (dict(flags=drs.DRS_NORMALIZE), drs.DRS_ERR_INVALID),      # only DRS_REVERSE is a flag here
    (dict(y=P), drs.DRS_ERR_INVALID),                           # y aliases x
    (dict(f=ctypes.c_void_p(0x2002)), drs.DRS_ERR_INVALID),     # misaligned fp32
    (dict(T=1 << 20, C=1 << 10), drs.DRS_ERR_UNSUPPORTED),       # a batch row over 2^31 bytes
    (dict(T=3000, C=64), drs.DRS_ERR_WORKSPACE),               # look-back kernel needs a workspace
    (dict(T=3000, C=64, ws=ctypes.c_void_p(0x7008), wsb=1 << 20), drs.DRS_ERR_INVALID),
])
def test_ema_forward_rejects(lib, kw, want):
    assert ema(lib, **kw) == want


def test_ema_workspace_query(lib):
    import torch
    assert drs.ema_workspace_bytes(8, 2048, 4096, torch.bfloat16) == 0          # walk kernel
    n = drs.ema_workspace_bytes(1, 3000, 300, torch.float32)
    assert n > 256 and n % 256 == 0
    assert drs.ema_workspace_bytes(1, 3000, 300, torch.bfloat16, reverse=True) == n
    assert lib.ema_workspace_bytes(0, 10, 10, 0, 0) == 0
    assert lib.ema_workspace_bytes(1, 10, 10, 0, drs.DRS_NORMALIZE) == 0


def test_la_workspace_query(lib):
    n = drs.la_workspace_bytes(8, 8, 2048, 64, 64)
    assert n > 0 and n % 256 == 0
    assert drs.la_workspace_bytes(8, 8, 2048, 64, 48) == 0               # unsupported Dv
    assert lib.la_workspace_bytes(0, 8, 2048, 64, 64, 1, 0, 0) == 0
    # longer sequences use more segments, so at least as much workspace
    assert drs.la_workspace_bytes(4, 16, 16384, 128, 128) >= drs.la_workspace_bytes(4, 16, 4096, 128, 128)
    # the step-by-step path (T <= 16, or forced) needs none; forcing the chunked one does
    assert drs.la_workspace_bytes(64, 16, 1, 128, 128) == 0
    assert drs.la_workspace_bytes(2, 2, 16, 64, 64) == 0
    assert drs.la_workspace_bytes(2, 2, 17, 64, 64) > 0
    assert drs.la_workspace_bytes(2, 2, 300, 64, 64, force="recurrent") == 0
    assert drs.la_workspace_bytes(2, 2, 8, 64, 64, force="chunked") > 0


def test_wkv_workspace_query(lib):
    # the WKV workload (B=8, T=1024, C=4096) runs the chained single pass
    chain = drs.wkv_workspace_bytes(8, 1024, 4096, drs.DRS_FORCE_CHAIN)
    assert chain > 256 and drs.wkv_workspace_bytes(8, 1024, 4096) == chain
    assert drs.wkv_workspace_bytes(8, 1024, 4096, drs.DRS_FORCE_SEQ) == 0
    n = drs.wkv_workspace_bytes(8, 1024, 4096, drs.DRS_FORCE_SCAN)
    assert n > 256 and (n - 256) % (3 * 8 * 4096 * 4) == 0            # counters, then slots
    assert drs.wkv_workspace_bytes(4, 64, 512) == 0                        # short: sequential
    # very long, few channels: too many time blocks for the chain, two-pass scan
    small = drs.wkv_workspace_bytes(1, 65536, 1024)
    assert small > 256 and (small - 256) % (3 * 1024 * 4) == 0
    assert drs.wkv_workspace_bytes(1, 65536, 1024, drs.DRS_FORCE_CHAIN) == 0   # unsupported: 0
    # fewer than 512 channel groups: the chain while its workgroups fit one round
    # (64 groups x 4 blocks), the two-pass scan beyond it (64 groups x 16 blocks)
    one = drs.wkv_workspace_bytes(1, 1024, 4096)
    assert one == drs.wkv_workspace_bytes(1, 1024, 4096, drs.DRS_FORCE_CHAIN) > 256
    many = drs.wkv_workspace_bytes(2, 4096, 4096)
    assert many == drs.wkv_workspace_bytes(2, 4096, 4096, drs.DRS_FORCE_SCAN) > 256
    assert (many - 256) % (3 * 2 * 4096 * 4) == 0
    assert drs.wkv_workspace_bytes(0, 10, 10) == 0
    assert drs.wkv_workspace_bytes(8, 10, 10, 0x4) == 0                    # unknown flag
    # the row-owning sweep: counters, a flag per (group, span, wave), 8 KB of states per flag
    rows = drs.wkv_workspace_bytes(8, 1024, 4096, drs.DRS_FORCE_ROWS)
    assert rows > 256 and rows % 256 == 0
    assert drs.wkv_workspace_bytes(8, 1024, 4094, drs.DRS_FORCE_ROWS) == 0    # C % 4 != 0
    assert drs.wkv_workspace_bytes(8, 2048, 4096, drs.DRS_FORCE_ROWS) > rows


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        drs.la_forward(x, x, x)
    with pytest.raises(ValueError):
        drs.wkv_forward(torch.zeros(4), torch.zeros(4), torch.zeros(1, 2, 4), torch.zeros(1, 2, 4))


def test_la_forward_group_rejects_and_sizes(lib):
    import ctypes as C
    n = drs.la_forward_group_workspace_bytes(2, 8, 8, 2048, 64, 64)
    one = drs.la_workspace_bytes(8, 8, 2048, 64, 64)
    # the shared 256 bytes of counters, then each problem's flags and aggregates
    assert n == 256 + 2 * ((one - 256 + 255) // 256 * 256) and n % 256 == 0
    assert drs.la_forward_group_workspace_bytes(1, 8, 8, 2048, 64, 64) >= one
    assert lib.la_forward_group_workspace_bytes(0, 8, 8, 2048, 64, 64, 1, 0, 0) == 0
    assert lib.la_forward_group_workspace_bytes(5, 8, 8, 2048, 64, 64, 1, 0, 0) == 0
    probs = (drs.LAProblem * 2)()
    for i in range(2):
        probs[i] = drs.LAProblem(0x1000, 0x2000, 0x3000, None, 0, None, None, 0x6000 + 0x1000 * i, None, None, 0)
    ws = C.c_void_p(0x100000)
    assert lib.la_forward_group(None, 2, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
    assert lib.la_forward_group(probs, 0, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
    assert lib.la_forward_group(probs, 5, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
    assert lib.la_forward_group(probs, 2, 1, 2, 2, 300, 64, 64, 0, None, 0, None) == drs.DRS_ERR_WORKSPACE
    assert lib.la_forward_group(probs, 2, 1, 2, 2, 300, 64, 64, 0, ws, 4096, None) == drs.DRS_ERR_WORKSPACE
    probs[1].y = 0x1000                          # one problem's output is another's input
    assert lib.la_forward_group(probs, 2, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
    probs[1].y = 0x6000                          # two problems write the same output
    assert lib.la_forward_group(probs, 2, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
    probs[1].y = 0x7000
    probs[1].mode = 9                            # an invalid problem: nothing launched
    assert lib.la_forward_group(probs, 2, 1, 2, 2, 300, 64, 64, 0, ws, 1 << 30, None) == drs.DRS_ERR_INVALID
