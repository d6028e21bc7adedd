"""Host code under address and undefined-behaviour sanitizers (CPU only, no GPU).

* The C ABI's argument checks and launch planning (csrc/qsa_api.cpp, qsa_plan.cpp,
  qsa_support.cpp: pure C++, no HIP) are built with g++ -fsanitize=address,undefined
  against stub launchers (tests/host/stub_launchers.cpp) and driven by a deterministic
  fuzz of edge-value descriptors (tests/host/abi_fuzz.cpp): no sanitizer report, and no
  call refuses the workspace its *_workspace_size query reported.
* The fp64 oracle (oracle/qsa_oracle.c) is built with the same sanitizers and every
  oracle pin runs against it, in a child process with the ASan runtime preloaded.
* The set-up itself is checked: a planted heap overflow and a planted signed overflow in
  a throwaway library make the same child process fail.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_ragged_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_fuzz")
    srcs = [os.path.join(CSRC, f) for f in ("qsa_api.cpp", "qsa_plan.cpp", "qsa_support.cpp")]
    srcs += [os.path.join(ROOT, "tests", "host", f) for f in ("stub_launchers.cpp", "abi_fuzz.cpp")]
    b = _run(["g++", "-std=c++17"] + SAN + ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + srcs + ["-o", exe])
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([exe, "400000"])
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "failures 0" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


PIN_RUNNER = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, oracle_pins as P
    lib = oracle.load(sys.argv[1])
    if len(sys.argv) > 2:      # the set-up check: call the planted function
        import ctypes
        bad = ctypes.CDLL(sys.argv[2])
        bad.planted.restype = ctypes.c_int
        bad.planted.argtypes = [ctypes.c_int]
        print("planted returned", bad.planted(int(sys.argv[3])))
    for pin in P.ALL_PINS:
        pin(lib)
    print("pins ok", len(P.ALL_PINS))
""")


def _sanitized_oracle(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    b = _run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"] + SAN +
             ["-o", so, os.path.join(ROOT, "oracle", "qsa_oracle.c"), "-lm"])
    assert b.returncode == 0, b.stderr[-4000:]
    runner = tmp_path / "run_pins.py"
    runner.write_text(PIN_RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests")))
    env = dict(os.environ, LD_PRELOAD=_asan_runtime() or "", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    return so, str(runner), env


def test_oracle_pins_under_sanitizers(tmp_path):
    if _asan_runtime() is None:
        pytest.skip("no ASan runtime for gcc")
    so, runner, env = _sanitized_oracle(tmp_path)
    r = _run([sys.executable, runner, so], env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "pins ok" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


@pytest.mark.parametrize("mode,reports", [(0, ("heap-buffer-overflow", "insufficient space for an object")),
                                          (1, ("signed integer overflow",))])
def test_sanitizer_setup_detects_planted_errors(tmp_path, mode, reports):
    """The child-process set-up does report errors: a library with a planted heap
    overflow (mode 0) or signed overflow (mode 1), built with the same flags, fails it."""
    if _asan_runtime() is None:
        pytest.skip("no ASan runtime for gcc")
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent("""
        #include <limits.h>
        #include <stdlib.h>
        int planted(int mode)
        {
            volatile int big = INT_MAX;
            if (mode == 1)
                return big + 1;              /* signed overflow */
            int *a = malloc(4 * sizeof(int));
            volatile int i = 4;
            int v = a[i];                    /* one past the end */
            free(a);
            return v;
        }
    """))
    bad = str(tmp_path / "libplanted.so")
    b = _run(["gcc", "-std=c11", "-fPIC", "-shared"] + SAN + ["-o", bad, str(src)])
    assert b.returncode == 0, b.stderr[-4000:]
    so, runner, env = _sanitized_oracle(tmp_path)
    r = _run([sys.executable, runner, so, bad, str(mode)], env=env)
    out = r.stdout + r.stderr
    assert r.returncode != 0 and any(x in out for x in reports), (r.returncode, out[-3000:])
    assert "pins ok" not in r.stdout
