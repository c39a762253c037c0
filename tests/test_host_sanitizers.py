"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds made here, in a temporary folder, and the existing CPU tests run
against them in a child process with the matching sanitizer runtime
preloaded:

* the oracle (g++, ``-fsanitize=address,undefined``), under the oracle pins
  of ``test_oracle_pins.py``: every index of the pack/unpack, act-quant,
  lookup-table, product and epilogue loops on the pins' shapes;
* libsherry with its host code instrumented (hipcc, sanitizer flags for the
  host pass only; the gfx950 device code is built as usual and never runs
  here), under ``test_abi_host.py``: argument validation, planning over
  2000 seeded shapes, the workspace and scratch limits, the no-allocation
  entry point's checks, and sizes at the int64 extremes.

Each sanitizer set-up first has to catch a planted heap overflow in a
one-function library of its own, so a run that silently lost its
instrumentation fails instead of passing.  Errors abort the child
(``-fno-sanitize-recover=all``, ``halt_on_error``).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"     # the compiler whose ASan runtime hipcc's host pass uses
CSRC = os.path.join(ROOT, "bit_weight_amd", "csrc")

PLANTED = r"""
#include <cstdlib>
extern "C" int planted_overflow(int n) {
  int* a = static_cast<int*>(std::malloc(sizeof(int) * n));
  for (int i = 0; i < n; ++i) a[i] = i;
  int v = a[n];                     // one past the end
  std::free(a);
  return v;
}
"""
PLANTED_RUN = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); "
               "print('not caught', L.planted_overflow(8), flush=True)")


def _gcc_asan_runtime():
    try:
        path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _env(preload: str, **extra) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""),
               PYTHONDONTWRITEBYTECODE="1")
    env.update(extra)
    return env


def _run(cmd, env, timeout=900):
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def _assert_planted_overflow_is_caught(compile_cmd, lib, env):
    subprocess.check_call(compile_cmd)
    res = _run([sys.executable, "-c", PLANTED_RUN, lib], env, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode != 0 and "heap-buffer-overflow" in out, out[-2000:]
    assert "not caught" not in res.stdout


def _assert_clean(res):
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in res.stdout, out[-2000:]


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    runtime = _gcc_asan_runtime()
    if runtime is None or shutil.which("g++") is None:
        pytest.skip("g++ with libasan is not available")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    env = _env(runtime, SHERRY_ORACLE_LIBDIR=str(tmp_path))

    planted_src = tmp_path / "planted.cpp"
    planted_src.write_text(PLANTED)
    planted = str(tmp_path / "libplanted.so")
    _assert_planted_overflow_is_caught(
        ["g++", "-O1", *san, "-shared", "-fPIC", str(planted_src), "-o", planted], planted, env)

    # the oracle's own flags (no fast math, no contraction) plus the sanitizers
    base = ["-std=c++17", "-O1", "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC", *san]
    src = os.path.join(ROOT, "oracle", "sherry_oracle.cpp")
    subprocess.check_call(["g++", *base, src, "-o", str(tmp_path / "liboracle.so")])
    subprocess.check_call(["g++", *base, "-fopenmp", src, "-o", str(tmp_path / "liboracle_omp.so")])

    res = _run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-m", "not gpu",
                "-p", "no:cacheprovider"], env)
    _assert_clean(res)


def test_abi_host_validation_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    runtime = _clang_asan_runtime()
    if runtime is None or not os.path.exists(HIPCC) or not os.path.exists(CLANGXX):
        pytest.skip("hipcc and the clang ASan runtime are not available")
    lib = str(tmp_path / "libsherry_san.so")
    env = _env(runtime, SHERRY_LIB=lib)

    planted_src = tmp_path / "planted.cpp"
    planted_src.write_text(PLANTED)
    planted = str(tmp_path / "libplanted.so")
    _assert_planted_overflow_is_caught(
        [CLANGXX, "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
         str(planted_src), "-o", planted], planted, env)

    # host pass instrumented; device pass as in the product build
    sys.path.insert(0, ROOT)
    from bit_weight_amd import build as product_build
    flags = [f for f in product_build.FLAGS if f not in ("-O3",)] + ["-O1", "-g"]
    host_san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for src in product_build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags, *host_san, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, f"{src}: {out[-3000:]}"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])

    res = _run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q", "-m", "not gpu",
                "-p", "no:cacheprovider"], env)
    _assert_clean(res)
