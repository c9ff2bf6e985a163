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
        "bqo_prepare_table": (ctypes.c_int, [fp, ctypes.c_int, fp]),
        "bqo_nested_groups": (ctypes.c_int, [fp, i64, ctypes.c_float, fp, ctypes.c_int, i32, i64, i64, u8p, fp]),
        "bqo_nested_stats": (ctypes.c_int, [fp, i64, fp, ctypes.c_int, i32, u8p, fp, fp]),
        "iqo_vector_error": (ctypes.c_float, [ctypes.c_float] * 4),
        "iqo_iq2xs_encode_block": (ctypes.c_int, [fp, ctypes.c_uint16, u8p, u8p]),
        "iqo_iq2xs_quantize": (ctypes.c_int64, [vp, ctypes.c_int, i64, u8p, vp, u8p, i64, i64]),
        "iqo_iq2xs_dequantize": (ctypes.c_int, [u8p, u8p, i64, ctypes.c_int, vp]),
        "iqo_iq1s_scale": (ctypes.c_uint16, [ctypes.c_float]),
        "iqo_iq1s_encode_block": (None, [fp, u8p, u8p]),
        "iqo_iq1s_quantize": (ctypes.c_int, [vp, ctypes.c_int, i64, u8p, u8p, i64, i64]),
        "iqo_iq1s_dequantize": (ctypes.c_int, [u8p, u8p, i64, ctypes.c_int, vp]),
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

    def prepare_table(self, table: np.ndarray):
        """The table as the oracle uses it (-0.0 read as +0.0), or None when it breaks R7."""
        t = np.ascontiguousarray(table, dtype=np.float32)
        out = np.zeros(max(t.size, 1), np.float32)
        if self.lib.bqo_prepare_table(_ptr(t), t.size, _ptr(out)) != 0:
            return None
        return out[:t.size]

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

    # IQ2_XS-style superblocks ------------------------------------------------------------
    IQ2XS_BLOCK, IQ2XS_BYTES = 256, 74

    @staticmethod
    def _iq_grid(grid: np.ndarray) -> np.ndarray:
        g = np.ascontiguousarray(grid, dtype=np.uint8).reshape(-1)
        if g.size != 512 * 8:
            raise ValueError("the grid holds 512 entries of 8 bytes")
        return g

    def iq2xs_vector_error(self, xn: float, dot: float, qn: float, s: float) -> np.float32:
        return np.float32(self.lib.iqo_vector_error(*(float(np.float32(v)) for v in (xn, dot, qn, s))))

    def iq2xs_encode_block(self, x: np.ndarray, d_bits: int, grid: np.ndarray):
        """One superblock of 256 binary32 values -> (74 payload bytes, rejected flag)."""
        xx = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        if xx.size != 256:
            raise ValueError("a superblock holds 256 values")
        g = self._iq_grid(grid)
        out = np.zeros(self.IQ2XS_BYTES, np.uint8)
        rej = self.lib.iqo_iq2xs_encode_block(_ptr(xx), int(d_bits), _ptr(g), _ptr(out))
        return out, rej

    def iq2xs_quantize(self, x: np.ndarray, dtype: int, grid: np.ndarray, scales: np.ndarray):
        """x: n raw elements of `dtype` (n a multiple of 256); scales: n/256 binary16 bit
        patterns.  Returns (payload bytes, number of rejected scales)."""
        xx = np.ascontiguousarray(x).reshape(-1)
        n, nb = xx.size, xx.size // self.IQ2XS_BLOCK
        g = self._iq_grid(grid)
        sc = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
        if sc.size != nb:
            raise ValueError("one scale per superblock")
        out = np.zeros(max(nb * self.IQ2XS_BYTES, 1), np.uint8)
        rej = self.lib.iqo_iq2xs_quantize(_ptr(xx), dtype, n, _ptr(g), _ptr(sc), _ptr(out), 0, nb)
        if rej < 0:
            raise ValueError("oracle iq2xs_quantize rejected its arguments")
        return out[:nb * self.IQ2XS_BYTES], int(rej)

    def iq2xs_dequantize(self, blocks: np.ndarray, grid: np.ndarray, n: int, dtype: int = F32) -> np.ndarray:
        b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
        g = self._iq_grid(grid)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        if self.lib.iqo_iq2xs_dequantize(_ptr(b), _ptr(g), n, dtype, _ptr(out)) != 0:
            raise ValueError("oracle iq2xs_dequantize rejected its arguments")
        return out[:n]

    # IQ1_S-style superblocks ------------------------------------------------------------
    IQ1S_BYTES = 50

    @staticmethod
    def _iq1_grid(grid: np.ndarray) -> np.ndarray:
        g = np.ascontiguousarray(grid, dtype=np.int8).reshape(-1)
        if g.size != 2048 * 8:
            raise ValueError("the grid holds 2048 entries of 8 signed bytes")
        return g

    def iq1s_scale(self, amax: float) -> int:
        return int(self.lib.iqo_iq1s_scale(float(np.float32(amax))))

    def iq1s_encode_block(self, x: np.ndarray, grid: np.ndarray) -> np.ndarray:
        xx = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        if xx.size != 256:
            raise ValueError("a superblock holds 256 values")
        out = np.zeros(self.IQ1S_BYTES, np.uint8)
        self.lib.iqo_iq1s_encode_block(_ptr(xx), _ptr(self._iq1_grid(grid)), _ptr(out))
        return out

    def iq1s_quantize(self, x: np.ndarray, dtype: int, grid: np.ndarray) -> np.ndarray:
        xx = np.ascontiguousarray(x).reshape(-1)
        n, nb = xx.size, xx.size // 256
        out = np.zeros(max(nb * self.IQ1S_BYTES, 1), np.uint8)
        if self.lib.iqo_iq1s_quantize(_ptr(xx), dtype, n, _ptr(self._iq1_grid(grid)), _ptr(out), 0, nb) != 0:
            raise ValueError("oracle iq1s_quantize rejected its arguments")
        return out[:nb * self.IQ1S_BYTES]

    def iq1s_dequantize(self, blocks: np.ndarray, grid: np.ndarray, n: int, dtype: int = F32) -> np.ndarray:
        b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        if self.lib.iqo_iq1s_dequantize(_ptr(b), _ptr(self._iq1_grid(grid)), n, dtype, _ptr(out)) != 0:
            raise ValueError("oracle iq1s_dequantize rejected its arguments")
        return out[:n]


def default_threads() -> int:
    """Host threads for the range-split entry points: the CPU count, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def _ranges(units: int, parts: int):
    """[lo, hi) ranges splitting 0..units into at most `parts` contiguous pieces."""
    parts = max(1, min(parts, units))
    step = -(-units // parts)
    return [(lo, min(units, lo + step)) for lo in range(0, units, step)]


def _run_all(jobs, threads: int):
    """Runs the callables in `jobs` on `threads` host threads (ctypes releases the GIL during a
    call into the C oracle) and raises if any returns a nonzero status."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        codes = list(ex.map(lambda f: f(), jobs))
    bad = [c for c in codes if c != 0]
    if bad:
        raise ValueError("oracle rejected its arguments (%d)" % bad[0])


class ParallelOracle(Oracle):
    """The same C functions, called on contiguous ranges of whole blocks (groups, rows) from
    several host threads.  Blocks are independent in every step except the nested mean, which
    stays one call over the whole absmax array, so the outputs are bit-identical to one call
    over everything; this class only splits index ranges and points each call at its slice
    of the input and output arrays (no arithmetic of the method happens here)."""

    def __init__(self, threads: int | None = None, lib: ctypes.CDLL | None = None):
        super().__init__(lib)
        self.threads = threads or default_threads()

    def _parts(self, units: int):
        return _ranges(units, 4 * self.threads)

    def quantize_blockwise(self, x: np.ndarray, dtype: int, blocksize: int, table: np.ndarray):
        x = np.ascontiguousarray(x).reshape(-1)
        n = x.size
        t = np.ascontiguousarray(table, dtype=np.float32)
        K = t.size
        nb = -(-n // blocksize)
        absmax = np.zeros(max(nb, 1), np.float32)
        packed = np.zeros(max(self.packed_bytes(n, K), 1), np.uint8)
        lib = self.lib

        def job(b0, b1):
            e0, e1 = b0 * blocksize, min(n, b1 * blocksize)  # e0 is even: 4-bit bytes start at e0 / 2
            p0 = e0 if K == 256 else e0 // 2
            return lambda: lib.bqo_quantize_blockwise(_ptr(x) + e0 * x.itemsize, dtype, e1 - e0, blocksize,
                                                      _ptr(t), K, _ptr(absmax) + 4 * b0, _ptr(packed) + p0)
        _run_all([job(b0, b1) for b0, b1 in self._parts(nb)], self.threads)
        return absmax[:nb], packed[:self.packed_bytes(n, K)]

    def dequantize_blockwise(self, packed: np.ndarray, absmax: np.ndarray, n: int, dtype: int,
                             blocksize: int, table: np.ndarray) -> np.ndarray:
        t = np.ascontiguousarray(table, dtype=np.float32)
        K = t.size
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        lib = self.lib
        nb = -(-n // blocksize)

        def job(b0, b1):
            e0, e1 = b0 * blocksize, min(n, b1 * blocksize)
            p0 = e0 if K == 256 else e0 // 2
            return lambda: lib.bqo_dequantize_blockwise(_ptr(out) + e0 * out.itemsize, dtype, e1 - e0, blocksize,
                                                        _ptr(t), K, _ptr(a) + 4 * b0, _ptr(p) + p0)
        _run_all([job(b0, b1) for b0, b1 in self._parts(nb)], self.threads)
        return out[:n]

    def iq2xs_quantize(self, x: np.ndarray, dtype: int, grid: np.ndarray, scales: np.ndarray):
        xx = np.ascontiguousarray(x).reshape(-1)
        n, nb = xx.size, xx.size // self.IQ2XS_BLOCK
        g = self._iq_grid(grid)
        sc = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
        if sc.size != nb:
            raise ValueError("one scale per superblock")
        out = np.zeros(max(nb * self.IQ2XS_BYTES, 1), np.uint8)
        lib, counts = self.lib, []

        def job(b0, b1):
            def run():
                counts.append(lib.iqo_iq2xs_quantize(_ptr(xx), dtype, n, _ptr(g), _ptr(sc), _ptr(out), b0, b1))
                return 0 if counts[-1] >= 0 else -1
            return run
        _run_all([job(b0, b1) for b0, b1 in self._parts(nb)], self.threads)
        if any(c < 0 for c in counts):
            raise ValueError("oracle iq2xs_quantize rejected its arguments")
        return out[:nb * self.IQ2XS_BYTES], int(sum(counts))

    def iq1s_quantize(self, x: np.ndarray, dtype: int, grid: np.ndarray) -> np.ndarray:
        xx = np.ascontiguousarray(x).reshape(-1)
        n, nb = xx.size, xx.size // 256
        g = self._iq1_grid(grid)
        out = np.zeros(max(nb * self.IQ1S_BYTES, 1), np.uint8)
        lib = self.lib

        def job(b0, b1):
            return lambda: lib.iqo_iq1s_quantize(_ptr(xx), dtype, n, _ptr(g), _ptr(out), b0, b1)
        _run_all([job(b0, b1) for b0, b1 in self._parts(nb)], self.threads)
        return out[:nb * self.IQ1S_BYTES]

    def nested_stats(self, absmax: np.ndarray, table2: np.ndarray, blocksize2: int = 256):
        """mean (one call over the whole array), then q2 / absmax2 over ranges of groups."""
        a = np.ascontiguousarray(absmax, dtype=np.float32)
        nb = a.size
        t2 = np.ascontiguousarray(table2, dtype=np.float32)
        ng = -(-nb // blocksize2)
        q2 = np.zeros(max(nb, 1), np.uint8)
        absmax2 = np.zeros(max(ng, 1), np.float32)
        mean = self.nested_mean(a)
        lib = self.lib

        def job(g0, g1):
            return lambda: lib.bqo_nested_groups(_ptr(a), nb, float(mean), _ptr(t2), t2.size, blocksize2, g0, g1,
                                                 _ptr(q2), _ptr(absmax2))
        _run_all([job(g0, g1) for g0, g1 in self._parts(ng)], self.threads)
        return q2[:nb], absmax2[:ng], mean

    def quantize_nested(self, x: np.ndarray, dtype: int, blocksize: int, table: np.ndarray,
                        table2: np.ndarray, blocksize2: int = 256):
        if self.prepare_table(table2) is None or np.asarray(table2).size != 256:
            raise ValueError("oracle quantize_nested rejected its arguments (-1)")
        absmax, packed = self.quantize_blockwise(x, dtype, blocksize, table)
        q2, absmax2, mean = self.nested_stats(absmax, table2, blocksize2)
        return dict(absmax=absmax, q2=q2, absmax2=absmax2, mean=mean, packed=packed)

    def dequantize_nested(self, packed, q2, absmax2, mean, n: int, dtype: int, blocksize: int,
                          table, table2, blocksize2: int = 256) -> np.ndarray:
        t = np.ascontiguousarray(table, dtype=np.float32)
        t2 = np.ascontiguousarray(table2, dtype=np.float32)
        K = t.size
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        p = np.ascontiguousarray(packed, dtype=np.uint8)
        q = np.ascontiguousarray(q2, dtype=np.uint8)
        a2 = np.ascontiguousarray(absmax2, dtype=np.float32)
        lib = self.lib
        nb = -(-n // blocksize)
        ng = -(-nb // blocksize2)

        def job(g0, g1):  # whole groups: block b0 = g0 * B2 starts absmax2 slice g0
            b0, b1 = g0 * blocksize2, min(nb, g1 * blocksize2)
            e0, e1 = b0 * blocksize, min(n, b1 * blocksize)
            p0 = e0 if K == 256 else e0 // 2
            return lambda: lib.bqo_dequantize_nested(_ptr(out) + e0 * out.itemsize, dtype, e1 - e0, blocksize,
                                                     _ptr(t), K, _ptr(t2), t2.size, blocksize2, _ptr(q) + b0,
                                                     _ptr(a2) + 4 * g0, float(np.float32(mean)), _ptr(p) + p0)
        _run_all([job(g0, g1) for g0, g1 in self._parts(ng)], self.threads)
        return out[:n]

    def dequant_q32(self, blocks: np.ndarray, n: int, row_len: int, fmt: int,
                    dtype: int = BF16) -> np.ndarray:
        b = np.ascontiguousarray(blocks, dtype=np.uint8)
        out = np.zeros(max(n, 1), np.float32 if dtype == F32 else np.uint16)
        bs = 18 if fmt == Q4 else 34
        lib = self.lib
        rows = n // row_len if row_len > 0 else 0

        def job(r0, r1):  # whole rows
            e0, e1 = r0 * row_len, r1 * row_len
            return lambda: lib.bqo_dequant_q32(_ptr(b) + e0 // 32 * bs, dtype, e1 - e0, row_len, fmt,
                                               _ptr(out) + e0 * out.itemsize)
        if rows == 0 or n % row_len != 0:
            return super().dequant_q32(blocks, n, row_len, fmt, dtype)
        _run_all([job(r0, r1) for r0, r1 in self._parts(rows)], self.threads)
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
