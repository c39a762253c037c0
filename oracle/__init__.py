"""CPU oracle for the Sherry 3:4-sparse ternary matmul -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and no
product code path falls back to it.

The arithmetic lives in ``sherry_oracle.cpp`` (plain single-threaded C++17);
this module compiles it with g++ and wraps it with ctypes over numpy arrays.
Every function restates the page "Sherry框架：三元量化与3:4稀疏优化LLM推理"
(pnsm.cn): §3.1 for the quantizer, §2.1 for the 5-bit code, §2.2 for the
lookup table and the integer add tree with one float multiply.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sherry_oracle.cpp")
# SHERRY_ORACLE_LIBDIR names a folder holding other builds of both
# libraries (the sanitizer builds of the CPU tests); by default this one
_LIBDIR = os.environ.get("SHERRY_ORACLE_LIBDIR") or _HERE
_LIB = os.path.join(_LIBDIR, "liboracle.so")
# the same source built with OpenMP: only the int32 product runs on several
# threads (its outputs are independent sums, so the values are identical)
_LIB_OMP = os.path.join(_LIBDIR, "liboracle_omp.so")
CXXFLAGS = ["-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off",
            "-shared", "-fPIC"]
OMP_FLAGS = ["-fopenmp"]

_libs = {}


def _compile(out: str, extra) -> None:
    tmp = out + ".tmp"
    subprocess.check_call(["g++", *CXXFLAGS, *extra, _SRC, "-o", tmp])
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` (single-threaded) and
    ``oracle/liboracle_omp.so`` (the same source with OpenMP) with g++."""
    if force or not os.path.exists(_LIB):
        _compile(_LIB, [])
    if force or not os.path.exists(_LIB_OMP):
        _compile(_LIB_OMP, OMP_FLAGS)
    return _LIB


def _load(parallel: bool = False):
    path = _LIB_OMP if parallel else _LIB
    if path not in _libs:
        if not os.path.exists(path):
            _compile(path, OMP_FLAGS if parallel else [])
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        sigs = {
            "oracle_pattern": [ci, vp],
            "oracle_decode_code": [ci, vp],
            "oracle_encode_block": [vp],
            "oracle_quantize": [vp, i64, i64, vp, vp],
            "oracle_pack": [vp, i64, i64, vp],
            "oracle_packed_bytes": [i64, i64],
            "oracle_packed2_bytes": [i64, i64],
            "oracle_unpack": [vp, i64, i64, vp],
            "oracle_pack2": [vp, i64, i64, vp],
            "oracle_unpack2": [vp, i64, i64, vp],
            "oracle_act_quant": [vp, i64, i64, vp, vp],
            "oracle_lut": [vp, i64, i64, vp],
            "oracle_gemm_i32": [vp, vp, i64, i64, i64, vp],
            "oracle_epilogue": [vp, vp, vp, i64, i64, vp],
            "oracle_threads": [],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = i64 if name.endswith("_bytes") else ci
        _libs[path] = lib
    return _libs[path]


def threads(parallel: bool = True) -> int:
    """Threads the int32 product uses in the plain (1) or OpenMP build."""
    return int(_load(parallel).oracle_threads())


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def pattern(p: int) -> np.ndarray:
    """Canonical pattern p (0..15): exactly 3 nonzeros, first nonzero +1."""
    out = np.zeros(4, np.int8)
    _check(_load().oracle_pattern(p, _p(out)), "pattern")
    return out


def decode_code(c: int) -> np.ndarray:
    """The 4-weight block for 5-bit code c = 2*p + s (0..31)."""
    out = np.zeros(4, np.int8)
    _check(_load().oracle_decode_code(c, _p(out)), "decode_code")
    return out


def encode_block(t) -> int:
    """5-bit code of an exactly-3-nonzero ternary block, or -1."""
    a = np.ascontiguousarray(np.asarray(t, dtype=np.int8).reshape(4))
    return int(_load().oracle_encode_block(_p(a)))


def quantize(W: np.ndarray):
    """[Sherry §3.1] W fp32 [N,K] -> (T int8 [N,K] in {-1,0,1}, alpha fp32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    T = np.empty((N, K), np.int8)
    alpha = np.empty(N, np.float32)
    _check(_load().oracle_quantize(_p(W), N, K, _p(T), _p(alpha)), "quantize")
    return T, alpha


def packed_bytes(N: int, K: int) -> int:
    """Bytes of the 5-bit layout of an [N,K] matrix, padded to 64 x 128 tiles."""
    return int(_load().oracle_packed_bytes(N, K))


def packed2_bytes(N: int, K: int) -> int:
    """Bytes of the 2-bit layout of an [N,K] matrix, padded to 64 x 128 tiles."""
    return int(_load().oracle_packed2_bytes(N, K))


def pack(T: np.ndarray) -> np.ndarray:
    """Dense T -> packed bytes in the tiled 5-bit layout (padding: code 0)."""
    T = np.ascontiguousarray(T, dtype=np.int8)
    N, K = T.shape
    out = np.empty(packed_bytes(N, K), np.uint8)
    _check(_load().oracle_pack(_p(T), N, K, _p(out)), "pack")
    return out


def unpack(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed bytes -> dense T int8 [N,K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == packed_bytes(N, K)
    T = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack(_p(packed), N, K, _p(T)), "unpack")
    return T


def pack2(T: np.ndarray) -> np.ndarray:
    """Dense ternary T -> the 2-bit baseline format (padded like pack)."""
    T = np.ascontiguousarray(T, dtype=np.int8)
    N, K = T.shape
    out = np.empty(packed2_bytes(N, K), np.uint8)
    _check(_load().oracle_pack2(_p(T), N, K, _p(out)), "pack2")
    return out


def unpack2(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """2-bit baseline bytes -> dense T int8 [N,K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == packed2_bytes(N, K)
    T = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack2(_p(packed), N, K, _p(T)), "unpack2")
    return T


def act_quant(x: np.ndarray):
    """x fp32 [M,K] -> (q int8 [M,K], s fp32 [M]), per-token symmetric."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _check(_load().oracle_act_quant(_p(x), M, K, _p(q), _p(s)), "act_quant")
    return q, s


def lut(q: np.ndarray) -> np.ndarray:
    """[Sherry §2.2] q int8 [M,K] -> L int32 [M, K/4, 16]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    L = np.empty((M, K // 4, 16), np.int32)
    _check(_load().oracle_lut(_p(q), M, K, _p(L)), "lut")
    return L


def gemm_i32(q: np.ndarray, T: np.ndarray, parallel: bool = False) -> np.ndarray:
    """acc[m,n] = sum_k q[m,k] * T[n,k] (plain triple loop, int64 -> int32).
    parallel=True runs the same source's OpenMP build (weight rows spread over
    the host cores; identical values)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    T = np.ascontiguousarray(T, dtype=np.int8)
    M, K = q.shape
    N, K2 = T.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(_load(parallel).oracle_gemm_i32(_p(q), _p(T), M, N, K, _p(acc)), "gemm_i32")
    return acc


def epilogue(acc: np.ndarray, s_x: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """[Sherry §2.2 step 4] y = ((float)acc * s_x[m]) * alpha[n], fp32."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _check(_load().oracle_epilogue(_p(acc), _p(s_x), _p(alpha), M, N, _p(y)),
           "epilogue")
    return y


def gemm(q, s_x, T, alpha, parallel: bool = False):
    """Full product: int32 accumulators and the fp32 output."""
    acc = gemm_i32(q, T, parallel)
    return acc, epilogue(acc, s_x, alpha)
