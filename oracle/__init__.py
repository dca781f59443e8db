"""CPU oracle for the ternary-weight linear layer (test infrastructure only).

Only the test-suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The GPU library never imports,
links or calls it, and the two share no code.

``ternary_oracle.c`` holds the definitions (plain fp64 loops, own fp16/bf16
decoders); this module builds it with gcc and wraps it with ctypes + numpy.
``dense.py`` is a second, independent brute-force evaluation for tiny shapes.
Sources followed (titles/sections; see the C file for details):
  trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1, §4.2;
  m.nxbn.cn/news/169761 (7B ternary checkpoint into vLLM) §2.2, §3.2, §4.2;
  m.xxqk.cn/news/593501 (Bonsai 2 27B into vLLM) §4.3.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ternary_oracle.c"
_LIB = _HERE / "libternary_oracle.so"
_lib = None

GCC_FLAGS = ["-O2", "-fopenmp", "-shared", "-fPIC", "-ffp-contract=off", "-std=c11", "-Wall"]


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (host only)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.check_call(["gcc", *GCC_FLAGS, str(_SRC), "-o", str(tmp), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes view of one build of the C oracle (the default build or a test copy)."""

    def __init__(self, path: Path | str):
        lib = ctypes.CDLL(str(path))
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ternary_oracle_version.restype = ctypes.c_int
        lib.ternary_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ternary_oracle_f16_to_f64.restype = ctypes.c_double
        lib.ternary_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ternary_oracle_bf16_to_f64.restype = ctypes.c_double
        for nm in ("ternary_oracle_code_table", "ternary_oracle_code_eq",
                   "ternary_oracle_code_bits"):
            getattr(lib, nm).argtypes = [ctypes.c_int]
            getattr(lib, nm).restype = ctypes.c_int
        lib.ternary_oracle_unpack.argtypes = [p, i64, i64, p]
        lib.ternary_oracle_unpack.restype = None
        lib.ternary_oracle_pack.argtypes = [p, i64, i64, p]
        lib.ternary_oracle_pack.restype = i64
        lib.ternary_oracle_linear.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, p, p,
                                              ctypes.c_int]
        lib.ternary_oracle_linear.restype = ctypes.c_int
        lib.ternary_oracle_linear_at.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64,
                                                 p, p, i64, p, p, ctypes.c_int]
        lib.ternary_oracle_linear_at.restype = ctypes.c_int
        lib.ternary_oracle_count_reserved.argtypes = [p, i64]
        lib.ternary_oracle_count_reserved.restype = i64
        self.lib = lib
        self.path = str(path)

    def f16_to_f64(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.ternary_oracle_f16_to_f64
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def bf16_to_f64(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.ternary_oracle_bf16_to_f64
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def code_value(self, c: int, form: str = "table") -> int:
        return {"table": self.lib.ternary_oracle_code_table,
                "eq": self.lib.ternary_oracle_code_eq,
                "bits": self.lib.ternary_oracle_code_bits}[form](int(c))

    def unpack(self, packed: np.ndarray, K: int | None = None) -> np.ndarray:
        """bytes [N, K/4] -> int8 [N, K]."""
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        if p.ndim == 1:
            p = p.reshape(1, -1)
        N = p.shape[0]
        K = p.shape[1] * 4 if K is None else K
        q = np.empty((N, K), dtype=np.int8)
        self.lib.ternary_oracle_unpack(_ptr(p), N, K, _ptr(q))
        return q

    def pack(self, q: np.ndarray):
        """int8 [N, K] -> (bytes [N, K/4], invalid_count)."""
        qq = np.ascontiguousarray(q, dtype=np.int8)
        if qq.ndim == 1:
            qq = qq.reshape(1, -1)
        N, K = qq.shape
        if K % 4:
            raise ValueError("K must be a multiple of 4")
        out = np.empty((N, K // 4), dtype=np.uint8)
        inv = self.lib.ternary_oracle_pack(_ptr(qq), N, K, _ptr(out))
        return out, int(inv)

    def count_reserved(self, packed: np.ndarray) -> int:
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        return int(self.lib.ternary_oracle_count_reserved(_ptr(p), p.size))

    def linear(self, x_bits, packed, scale_bits, group_size: int, dtype: str = "bf16",
               nthreads: int | None = None, return_threads: bool = False):
        """fp64 y [M, N] and per-element bound B [M, N] (B = sum_k |x| |s|)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        M, K = x.shape
        N = p.shape[0]
        if p.shape[1] * 4 != K:
            raise ValueError("packed shape does not match K")
        y = np.empty((M, N), dtype=np.float64)
        b = np.empty((M, N), dtype=np.float64)
        nt = default_threads() if nthreads is None else nthreads
        used = self.lib.ternary_oracle_linear(_ptr(x), 1 if dtype == "fp16" else 0, M, N, K,
                                              _ptr(p), _ptr(s), int(group_size), _ptr(y),
                                              _ptr(b), nt)
        if used < 0:
            raise ValueError("oracle rejected the arguments")
        return (y, b, used) if return_threads else (y, b)

    def linear_at(self, x_bits, packed, scale_bits, group_size: int, ms, ns,
                  dtype: str = "bf16", nthreads: int | None = None):
        """fp64 y and bound at the listed (m, n) outputs only."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        M, K = x.shape
        N = p.shape[0]
        y = np.empty(ms.shape, dtype=np.float64)
        b = np.empty(ms.shape, dtype=np.float64)
        nt = default_threads() if nthreads is None else nthreads
        used = self.lib.ternary_oracle_linear_at(_ptr(x), 1 if dtype == "fp16" else 0, M, N, K,
                                                 _ptr(p), _ptr(s), int(group_size), _ptr(ms),
                                                 _ptr(ns), ms.size, _ptr(y), _ptr(b), nt)
        if used < 0:
            raise ValueError("oracle rejected the arguments")
        return y, b


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def default() -> Oracle:
    """The oracle built from ternary_oracle.c (built on first use)."""
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=True)
        _lib = Oracle(_LIB)
    return _lib


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def code_value(c, form="table"):
    return default().code_value(c, form)


def unpack(packed, K=None):
    return default().unpack(packed, K)


def pack(q):
    return default().pack(q)


def count_reserved(packed):
    return default().count_reserved(packed)


def linear(*a, **kw):
    return default().linear(*a, **kw)


def linear_at(*a, **kw):
    return default().linear_at(*a, **kw)


def within_bound(y_dev: np.ndarray, y_ref: np.ndarray, bound: np.ndarray,
                 rel: float = 1e-3, abs_: float = 1e-6) -> np.ndarray:
    """Element-wise acceptance |y_dev - y_ref| <= rel * B + abs_."""
    return np.abs(np.asarray(y_dev, np.float64) - y_ref) <= rel * bound + abs_
