"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer run (CPU only).

Every library source is compiled host-only (no device code) with the sanitizers
on the host pass, the fp64 oracle with the same clang and sanitizers, and the
two are linked with ``tests/sanitizer_driver.cpp``, which runs every oracle
routine on small random inputs and drives the C ABI's argument checks and
workspace queries (small, ragged, huge and invalid sizes).  No call in the
driver reaches a kernel launch.  Any memory error, undefined behaviour (signed
overflow in a size computation, say) or failed check ends the run non-zero.
"""
import os
import shutil
import struct
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

from decayed_recurrence_scans_amd import _build

ROOT = Path(__file__).resolve().parent.parent
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# the sanitizers apply to the host pass only (there is no device pass here)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stderr[-3000:]}"


def empty_offload_bundle(path):
    """A well-formed offload bundle holding only an empty host entry: what the host
    pass embeds in place of the device code it would otherwise register (this build
    launches nothing, so it needs no code object)."""
    triple = b"host-x86_64-unknown-linux-gnu"
    head = b"__CLANG_OFFLOAD_BUNDLE__" + struct.pack("<Q", 1)
    off = len(head) + 24 + len(triple)
    path.write_bytes(head + struct.pack("<QQQ", off, 0, len(triple)) + triple)
    return path


def test_sanitized_host_build_and_run(tmp_path):
    if not (Path(HIPCC).exists() and Path(CLANG).exists()):
        pytest.skip("ROCm toolchain not installed")
    inc = ["-I", str(ROOT / "include"), "-I", str(_build.CSRC)]
    fb = empty_offload_bundle(tmp_path / "empty.hipfb")
    common = [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17", "-Xclang", "-fcuda-include-gpubinary",
              "-Xclang", str(fb), *HOST_SAN, *inc]
    jobs = [common + ["-c", str(_build.CSRC / s), "-o", str(tmp_path / (Path(s).stem + ".o"))]
            for s in _build.SOURCES]
    jobs.append(common + ["-c", str(ROOT / "tests" / "sanitizer_driver.cpp"), "-o", str(tmp_path / "driver.o")])
    jobs.append([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", "-c", str(ROOT / "oracle" / "oracle.c"),
                 "-o", str(tmp_path / "oracle.o")])
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, jobs))
    exe = tmp_path / "driver"
    objs = sorted(str(p) for p in tmp_path.glob("*.o"))
    _run([HIPCC, "--offload-host-only", *HOST_SAN, *objs, "-o", str(exe), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "sanitizer driver ok" in r.stdout
