"""CPU oracle for blockwise absmax quantization (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package.  The library under ``dequantization_block_absmax_amd`` never does; the
two share no code.  The arithmetic lives in ``bq_oracle.c`` (plain scalar C, built with
``-ffp-contract=off`` and no fast-math); this module only builds it and marshals numpy
arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bq_oracle.c")
LIB = os.path.join(HERE, "libbq_oracle.so")

F32, F16, BF16 = 0, 1, 2
Q4, Q8 = 0, 1

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

_lock = threading.Lock()
_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compiles the oracle (or a variant of its source) into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i64, i32, fp, u8p = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                             ctypes.c_void_p)
    sig = {
        "bqo_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "bqo_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "bqo_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "bqo_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "bqo_nearest": (ctypes.c_int, [ctypes.c_float, fp, ctypes.c_int]),
        "bqo_zero_code": (ctypes.c_int, [fp, ctypes.c_int]),
        "bqo_guard_scale": (ctypes.c_float, [ctypes.c_float]),
        "bqo_normalize": (ctypes.c_float, [ctypes.c_float, ctypes.c_float]),
        "bqo_nested_mean": (ctypes.c_float, [fp, i64]),
        "bqo_pairwise_sum": (ctypes.c_double, [fp, i64]),
        "bqo_quantize_blockwise": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, fp, ctypes.c_int,
                                                  fp, u8p]),
        "bqo_dequantize_blockwise": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, fp, ctypes.c_int,
                                                    fp, u8p]),
        "bqo_linear_blockwise": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, i64, i32, fp, ctypes.c_int,
                                                fp, u8p, vp]),
        "bqo_gemm_blockwise": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, i64, i32, fp, ctypes.c_int,
                                              fp, u8p, vp]),
        "bqo_quantize_nested": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, fp, ctypes.c_int, fp,
                                               ctypes.c_int, i32, fp, u8p, fp, fp, u8p]),
        "bqo_dequantize_nested": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, fp, ctypes.c_int,
                                                 fp, ctypes.c_int, i32, u8p, fp, ctypes.c_float,
                                                 u8p]),
        "bqo_dequant_q32": (ctypes.c_int, [u8p, ctypes.c_int, i64, i32, ctypes.c_int, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Loads the oracle library; builds it first when missing or older than its source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            _lib = _declare(ctypes.CDLL(LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def dtype_code(dt) -> int:
    dt = np.dtype(dt) if not isinstance(dt, str) else dt
    if dt in ("float32", np.dtype(np.float32)):
        return F32
    if dt in ("float16", np.dtype(np.float16)):
        return F16
    if dt in ("bfloat16",):
        return BF16
    raise ValueError(dt)


class Oracle:
    """numpy-facing wrapper.  16-bit inputs and outputs are passed as uint16 bit patterns
    together with an explicit dtype code (F16 or BF16); fp32 data as float32 arrays."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    # scalar helpers --------------------------------------------------------------------
    def nearest(self, y: float, table: np.ndarray) -> int:
        t = np.ascontiguousarray(table, dtype=np.float32)
        return self.lib.bqo_nearest(float(np.float32(y)), _ptr(t), len(t))

    def zero_code(self, table: np.ndarray) -> int:
        t = np.ascontiguousarray(table, dtype=np.float32)
        return self.lib.bqo_zero_code(_ptr(t), len(t))

    def normalize(self, x: float, a: float) -> np.float32:
        return np.float32(self.lib.bqo_normalize(float(np.float32(x)), float(np.float32(a))))

    def nested_mean(self, absmax: np.ndarray) -> np.float32:
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        return np.float32(self.lib.bqo_nested_mean(_ptr(a), len(a)))

    def pairwise_sum(self, a: np.ndarray) -> float:
        a = np.ascontiguousarray(a, dtype=np.float32)
        return self.lib.bqo_pairwise_sum(_ptr(a), len(a))

    def f32_to_bf16(self, x: float) -> int:
        return self.lib.bqo_f32_to_bf16(float(np.float32(x)))

    def f32_to_f16(self, x: float) -> int:
        return self.lib.bqo_f32_to_f16(float(np.float32(x)))

    def bf16_to_f32(self, b: int) -> np.float32:
        return np.float32(self.lib.bqo_bf16_to_f32(int(b)))

    def f16_to_f32(self, h: int) -> np.float32:
        return np.float32(self.lib.bqo_f16_to_f32(int(h)))

    # array entry points ----------------------------------------------------------------
    @staticmethod
    def packed_bytes(n: int, K: int) -> int:
        return n if K == 256 else (n + 1) // 2

    def quantize_blockwise(self, x: np.ndarray, dtype: int, blocksize: int, table: np.ndarray):
        x = np.ascontiguousarray(x)
        n = x.size
        t = np.ascontiguousarray(table, dtype=np.float32)
        nb = -(-n // blocksize)
        absmax = np.zeros(max(nb, 1), np.float32)
        packed = np.zeros(max(self.packed_bytes(n, len(t)), 1), np.uint8)
        rc = self.lib.bqo_quantize_blockwise(_ptr(x), dtype, n, blocksize, _ptr(t), len(t),
                                             _ptr(absmax), _ptr(packed))
        if rc != 0:
            raise ValueError("oracle quantize_blockwise rejected its arguments (%d)" % rc)
        return absmax[:nb], packed[:self.packed_bytes(n, len(t))]

    def dequantize_blockwise(self, packed: np.ndarray, absmax: np.ndarray, n: int, dtype: int,
                             blocksize: int, table: np.ndarray) -> np.ndarray:
        t = np.ascontiguousarray(table, dtype=np.float32)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        rc = self.lib.bqo_dequantize_blockwise(_ptr(out), dtype, n, blocksize, _ptr(t), len(t),
                                               _ptr(a), _ptr(p))
        if rc != 0:
            raise ValueError("oracle dequantize_blockwise rejected its arguments (%d)" % rc)
        return out[:n]

    def linear_blockwise(self, x: np.ndarray, dtype: int, M: int, K: int, N: int, blocksize: int,
                         table: np.ndarray, absmax: np.ndarray, packed: np.ndarray) -> np.ndarray:
        """y (M x N, binary64) = x (M x K, raw elements of `dtype`) . deq(W)^T, W the N x K
        tensor quantized blockwise over its flat index (packed codes + absmax)."""
        xx = np.ascontiguousarray(x)
        t = np.ascontiguousarray(table, dtype=np.float32)
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        y = np.zeros(max(M * N, 1), np.float64)
        rc = self.lib.bqo_linear_blockwise(_ptr(xx), dtype, M, K, N, blocksize, _ptr(t), len(t), _ptr(a),
                                           _ptr(p), _ptr(y))
        if rc != 0:
            raise ValueError("oracle linear_blockwise rejected its arguments (%d)" % rc)
        return y[:M * N].reshape(M, N)

    def gemm_blockwise(self, x: np.ndarray, dtype: int, M: int, K: int, N: int, blocksize: int,
                       table: np.ndarray, absmax: np.ndarray, packed: np.ndarray) -> np.ndarray:
        """y (M x N, binary64) = x (M x K, raw fp16/bf16 elements) . W16^T, W16 the 16-bit
        dequantized weights of the N x K tensor quantized blockwise over its flat index."""
        xx = np.ascontiguousarray(x)
        t = np.ascontiguousarray(table, dtype=np.float32)
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        y = np.zeros(max(M * N, 1), np.float64)
        rc = self.lib.bqo_gemm_blockwise(_ptr(xx), dtype, M, K, N, blocksize, _ptr(t), len(t), _ptr(a),
                                         _ptr(p), _ptr(y))
        if rc != 0:
            raise ValueError("oracle gemm_blockwise rejected its arguments (%d)" % rc)
        return y[:M * N].reshape(M, N)

    def quantize_nested(self, x: np.ndarray, dtype: int, blocksize: int, table: np.ndarray,
                        table2: np.ndarray, blocksize2: int = 256):
        x = np.ascontiguousarray(x)
        n = x.size
        t = np.ascontiguousarray(table, dtype=np.float32)
        t2 = np.ascontiguousarray(table2, dtype=np.float32)
        nb = -(-n // blocksize)
        ng = -(-nb // blocksize2)
        absmax = np.zeros(max(nb, 1), np.float32)
        q2 = np.zeros(max(nb, 1), np.uint8)
        absmax2 = np.zeros(max(ng, 1), np.float32)
        mean = np.zeros(1, np.float32)
        packed = np.zeros(max(self.packed_bytes(n, len(t)), 1), np.uint8)
        rc = self.lib.bqo_quantize_nested(_ptr(x), dtype, n, blocksize, _ptr(t), len(t), _ptr(t2),
                                          len(t2), blocksize2, _ptr(absmax), _ptr(q2),
                                          _ptr(absmax2), _ptr(mean), _ptr(packed))
        if rc != 0:
            raise ValueError("oracle quantize_nested rejected its arguments (%d)" % rc)
        return dict(absmax=absmax[:nb], q2=q2[:nb], absmax2=absmax2[:ng], mean=mean[0],
                    packed=packed[:self.packed_bytes(n, len(t))])

    def dequantize_nested(self, packed, q2, absmax2, mean, n: int, dtype: int, blocksize: int,
                          table, table2, blocksize2: int = 256) -> np.ndarray:
        t = np.ascontiguousarray(table, dtype=np.float32)
        t2 = np.ascontiguousarray(table2, dtype=np.float32)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        q = np.ascontiguousarray(q2, dtype=np.uint8)
        a2 = np.ascontiguousarray(absmax2, dtype=np.float32)
        rc = self.lib.bqo_dequantize_nested(_ptr(out), dtype, n, blocksize, _ptr(t), len(t),
                                            _ptr(t2), len(t2), blocksize2, _ptr(q), _ptr(a2),
                                            float(np.float32(mean)), _ptr(p))
        if rc != 0:
            raise ValueError("oracle dequantize_nested rejected its arguments (%d)" % rc)
        return out[:n]

    def dequant_q32(self, blocks: np.ndarray, n: int, row_len: int, fmt: int,
                    dtype: int = BF16) -> np.ndarray:
        b = np.ascontiguousarray(blocks, dtype=np.uint8)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        rc = self.lib.bqo_dequant_q32(_ptr(b), dtype, n, row_len, fmt, _ptr(out))
        if rc != 0:
            raise ValueError("oracle dequant_q32 rejected its arguments (%d)" % rc)
        return out[:n]


def unpack_codes(packed: np.ndarray, n: int, K: int) -> np.ndarray:
    """Codes from packed bytes (layout of the oracle's pack step: high nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    if K == 256:
        return p[:n].copy()
    codes = np.empty(2 * p.size, np.uint8)
    codes[0::2] = p >> 4
    codes[1::2] = p & 0x0F
    return codes[:n]
