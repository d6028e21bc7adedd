"""Build the HIP library libqsa.so in-tree for gfx950 (hipcc, no JIT cache).

Every translation unit under csrc/ is compiled to an object in _build/ and linked
into sparse_attention_ragged_amd/libqsa.so. All device code is compiled with
packed-fp32 instruction selection disabled.

``ensure_built()`` is what the package calls on import: it rebuilds only when the
library is missing or was built from other sources (a sha256 of every source, the
public header, this file's compiler flags and the target is stored beside the
library), under a file lock so that concurrent processes build once. ``build()``
always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import fcntl
import glob
import hashlib
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqsa.so")
STAMP = LIB + ".sha256"
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + INCLUDE, "-I" + CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]


def _log(msg: str):
    print("[libqsa] " + msg, file=sys.stderr, flush=True)


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def source_digest() -> str:
    """sha256 over every file the library is built from (names and bytes), the flags
    and the target architecture."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h")))
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.relpath(f, ROOT).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    h.update(repr((COMMON[:5], DEVICE, ARCH)).encode())
    return h.hexdigest()


def _jobs() -> int:
    env = os.environ.get("MAX_JOBS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 4)
    return max(1, min(n, 16))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip"] + COMMON + DEVICE + ["-c", src, "-o", obj]
    else:
        cmd = [hipcc()] + COMMON + ["-c", src, "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature: drop that warning
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    _log("compiled %s (%.1f s)" % (os.path.basename(src), time.time() - t0))
    return obj


def build(jobs: int = 0) -> str:
    """Compile every csrc/*.hip and csrc/*.cpp and link libqsa.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    digest = source_digest()
    srcs = sources()
    t0 = time.time()
    _log("building %s for %s from %d sources (%d jobs)" % (os.path.basename(LIB), ARCH, len(srcs),
                                                          jobs or _jobs()))
    # longest translation units first, so that they do not start last
    order = sorted(srcs, key=lambda s: -os.path.getsize(s))
    with cf.ThreadPoolExecutor(max_workers=jobs or _jobs()) as ex:
        objs = dict(zip(order, ex.map(_compile, order)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + [objs[s] for s in srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    _log("built %s in %.1f s" % (LIB, time.time() - t0))
    return LIB


def is_current() -> bool:
    """The library exists and was built from the sources as they are now."""
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_digest()


def ensure_built() -> str:
    """Build libqsa.so unless it is current; concurrent callers build it once."""
    if is_current():
        return LIB
    os.makedirs(BUILD, exist_ok=True)
    with open(os.path.join(BUILD, ".lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        try:
            if not is_current():
                build()
        finally:
            fcntl.flock(lock, fcntl.LOCK_UN)
    return LIB


if __name__ == "__main__":
    print(build())
