"""CPU oracle of the ternary-weight matmul (float64, plain loops in C).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never calls it, and it shares no code with the HIP path.

The arithmetic lives in ``tern_oracle.c`` (see its header for the passages of
the pages it follows); this module compiles it with gcc (no fast-math) and
wraps it with ctypes over numpy arrays.  Calls release the GIL, so the
optional ``threads`` argument splits output columns over Python threads; each
output element is still computed by the same plain loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tern_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

KIND = {"f16": 0, "bf16": 1, "f32": 2}

_lock = threading.Lock()
_lib_cache = {}


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle into a shared library (gcc -O2, IEEE semantics)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp, c_int, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = dbl
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_code_value.argtypes = [ctypes.c_uint]
    lib.oracle_code_value.restype = c_int
    lib.oracle_unpack.argtypes = [vp, vp, i64, i64]
    lib.oracle_unpack.restype = c_int
    lib.oracle_pack.argtypes = [vp, vp, i64, i64]
    lib.oracle_pack.restype = c_int
    lib.oracle_matmul_cols.argtypes = [vp, c_int, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp]
    lib.oracle_matmul_cols.restype = c_int
    lib.oracle_matmul_at.argtypes = [vp, c_int, vp, vp, i64, i64, i64, i64, vp, vp, i64, vp, vp]
    lib.oracle_matmul_at.restype = c_int
    lib.oracle_decode_array.argtypes = [vp, c_int, i64, vp]
    lib.oracle_decode_array.restype = None
    lib.oracle_round_array.argtypes = [vp, c_int, i64, vp]
    lib.oracle_round_array.restype = None
    lib.oracle_ulp_array.argtypes = [vp, c_int, i64, vp]
    lib.oracle_ulp_array.restype = None
    lib.oracle_dequant.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_dequant.restype = c_int
    lib.oracle_block_map.argtypes = [vp, i64, i64, i64, vp]
    lib.oracle_block_map.restype = c_int
    lib.oracle_quantize_scales.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_quantize_scales.restype = c_int
    lib.oracle_matmul_s8_cols.argtypes = [vp, c_int, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp]
    lib.oracle_matmul_s8_cols.restype = c_int
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it first if it is not there)."""
    path = path or LIBRARY
    with _lock:
        if path in _lib_cache:
            return _lib_cache[path]
        if path == LIBRARY and not os.path.exists(path):
            build()
        lib = _bind(ctypes.CDLL(path))
        _lib_cache[path] = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


class Oracle:
    """Thin numpy wrapper over one compiled oracle library."""

    def __init__(self, path: Optional[str] = None):
        self.lib = load(path)

    # --- formats -------------------------------------------------------
    def decode(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        want = np.uint32 if dtype == "f32" else np.uint16
        b = np.ascontiguousarray(np.asarray(bits).view(want) if np.asarray(bits).dtype != want
                                 else np.asarray(bits))
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode_array(_ptr(b), KIND[dtype], b.size, _ptr(out))
        return out

    def round(self, v: np.ndarray, dtype: str) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty_like(v)
        self.lib.oracle_round_array(_ptr(v), KIND[dtype], v.size, _ptr(out))
        return out

    def ulp(self, v: np.ndarray, dtype: str) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty_like(v)
        self.lib.oracle_ulp_array(_ptr(v), KIND[dtype], v.size, _ptr(out))
        return out

    # --- the code ---------------------------------------------------------
    def code_value(self, code: int) -> int:
        return int(self.lib.oracle_code_value(code))

    def unpack(self, packed: np.ndarray, N: int, K: int) -> np.ndarray:
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        assert p.size == N * (K // 4)
        T = np.empty((N, K), dtype=np.int8)
        if self.lib.oracle_unpack(_ptr(p), _ptr(T), N, K) != 0:
            raise ValueError("oracle_unpack: bad shape")
        return T

    def pack(self, T: np.ndarray) -> np.ndarray:
        T = np.ascontiguousarray(T, dtype=np.int8)
        N, K = T.shape
        P = np.empty((N, K // 4), dtype=np.uint8)
        if self.lib.oracle_pack(_ptr(T), _ptr(P), N, K) != 0:
            raise ValueError("oracle_pack: bad shape")
        return P

    # --- the matmul -------------------------------------------------------
    def matmul(self, x_bits: np.ndarray, x_dtype: str, packed: np.ndarray,
               scale_bits: np.ndarray, M: int, N: int, K: int, group: int = 128,
               threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """Full Y[M,N] and error scale B[M,N], both float64."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        assert x.size == M * K and p.size == N * (K // 4) and s.size == N * (K // group)
        Y = np.zeros((M, N), dtype=np.float64)
        B = np.zeros((M, N), dtype=np.float64)
        kind = KIND[x_dtype]
        threads = max(1, min(int(threads), N)) if N > 0 else 1
        bounds = [N * i // threads for i in range(threads + 1)]
        errs = []

        def run(a, b):
            rc = self.lib.oracle_matmul_cols(_ptr(x), kind, _ptr(p), _ptr(s), M, N, K, group,
                                             a, b, _ptr(Y), _ptr(B))
            if rc != 0:
                errs.append(rc)

        if threads == 1:
            run(0, N)
        else:
            ts = [threading.Thread(target=run, args=(bounds[i], bounds[i + 1]))
                  for i in range(threads)]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
        if errs:
            raise ValueError("oracle_matmul: bad arguments")
        return Y, B

    def matmul_at(self, x_bits: np.ndarray, x_dtype: str, packed: np.ndarray,
                  scale_bits: np.ndarray, M: int, N: int, K: int, ms: np.ndarray,
                  ns: np.ndarray, group: int = 128) -> Tuple[np.ndarray, np.ndarray]:
        """Y and B at the outputs (ms[i], ns[i]) only."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        Y = np.zeros(ms.shape, dtype=np.float64)
        B = np.zeros(ms.shape, dtype=np.float64)
        rc = self.lib.oracle_matmul_at(_ptr(x), KIND[x_dtype], _ptr(p), _ptr(s), M, N, K, group,
                                       _ptr(ms), _ptr(ns), ms.size, _ptr(Y), _ptr(B))
        if rc != 0:
            raise ValueError("oracle_matmul_at: bad arguments")
        return Y, B

    # --- the comparison route, block map, int8 scales ---------------------
    def dequant(self, packed: np.ndarray, scale_bits: np.ndarray, N: int, K: int,
                group: int = 128) -> np.ndarray:
        """Dense W[N,K] = t * s in float64."""
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        W = np.empty((N, K), dtype=np.float64)
        if self.lib.oracle_dequant(_ptr(p), _ptr(s), N, K, group, _ptr(W)) != 0:
            raise ValueError("oracle_dequant: bad shape")
        return W

    def block_map(self, packed: np.ndarray, N: int, K: int, group: int = 128) -> np.ndarray:
        """uint32 [N, ceil(K/group/32)]: bit g%32 of word g/32 set if block g has a nonzero weight."""
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        words = (K // group + 31) // 32
        out = np.empty((N, words), dtype=np.uint32)
        if self.lib.oracle_block_map(_ptr(p), N, K, group, _ptr(out)) != 0:
            raise ValueError("oracle_block_map: bad shape")
        return out

    def quantize_scales(self, scale_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """(q int8 [N, groups], r float32 [N]) with s ~ q * r (per-row absmax / 127)."""
        s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
        N, groups = s.shape
        q = np.empty((N, groups), dtype=np.int8)
        r = np.empty(N, dtype=np.float32)
        self.lib.oracle_quantize_scales(_ptr(s), N, groups, _ptr(q), _ptr(r))
        return q, r

    def matmul_s8(self, x_bits: np.ndarray, x_dtype: str, packed: np.ndarray, q: np.ndarray,
                  r_f32: np.ndarray, M: int, N: int, K: int, group: int = 128,
                  threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """Y and B with effective scales q[n,g] * r[n] (r given as float32)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        qq = np.ascontiguousarray(q, dtype=np.int8)
        rb = np.ascontiguousarray(np.asarray(r_f32, dtype=np.float32)).view(np.uint32)
        Y = np.zeros((M, N), dtype=np.float64)
        B = np.zeros((M, N), dtype=np.float64)
        kind = KIND[x_dtype]
        threads = max(1, min(int(threads), N)) if N > 0 else 1
        bounds = [N * i // threads for i in range(threads + 1)]
        errs = []

        def run(a, b):
            if self.lib.oracle_matmul_s8_cols(_ptr(x), kind, _ptr(p), _ptr(qq), _ptr(rb), M, N, K,
                                              group, a, b, _ptr(Y), _ptr(B)) != 0:
                errs.append(1)

        ts = [threading.Thread(target=run, args=(bounds[i], bounds[i + 1])) for i in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        if errs:
            raise ValueError("oracle_matmul_s8: bad arguments")
        return Y, B

    # --- the pass criterion -------------------------------------------------
    def tolerance(self, Y: np.ndarray, B: np.ndarray, y_dtype: str,
                  rel: float = 2e-3) -> np.ndarray:
        """Allowed |Y_gpu - Y_oracle|: rel * B plus one ulp of the output type at Y."""
        return rel * B + self.ulp(Y, y_dtype)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
