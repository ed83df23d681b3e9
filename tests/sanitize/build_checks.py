"""Build the host-sanitizer check program: the library's sources and
host_checks.cpp compiled into one executable with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code (the GPU code is not instrumented).
Output: _build/sanitize/host_checks (rebuilt when a source is newer)."""

from __future__ import annotations

import glob
import importlib.util
import os
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
EXE = os.path.join(OUT, "host_checks")
DRIVER = os.path.join(HERE, "host_checks.cpp")
# host code only: -fno-gpu-sanitize keeps the device code uninstrumented
SAN = ["-fsanitize=address,undefined", "-fno-gpu-sanitize", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _library_build():
    spec = importlib.util.spec_from_file_location(
        "sk_build_for_sanitize", os.path.join(ROOT, "gemm_sk_repack_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _inputs(B):
    return ([os.path.join(B.CSRC, s) for s in B.SOURCES] + [DRIVER]
            + glob.glob(os.path.join(B.CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h")))


def ensure_built() -> str:
    B = _library_build()
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [DRIVER]
    if os.path.exists(EXE) and os.path.getmtime(EXE) >= max(os.path.getmtime(p) for p in _inputs(B)):
        return EXE
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(OUT, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    cmds = [[B.HIPCC, *B.CFLAGS, *SAN, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(B._run, cmds))
    B._run([B.HIPCC, f"--offload-arch={B.ARCH}", *SAN, *objs, "-o", EXE + ".tmp"])
    os.replace(EXE + ".tmp", EXE)
    return EXE
