"""Python binding of libbq (blockwise absmax quantization for MI355X / gfx950).

Argument marshalling only: every function here has the name of a C entry point of
include/bq.h and forwards to it through ctypes.  Device buffers are passed as torch tensors
(their data_ptr is used) or raw integer addresses; PyTorch only provides device memory and
streams.  No computation happens in Python, and there is no fallback: importing this
package raises if libbq.so has not been built (``python dequantization_block_absmax_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbq.so")

BQ_F32, BQ_F16, BQ_BF16 = 0, 1, 2
BQ_Q32_Q4, BQ_Q32_Q8 = 0, 1
(BQ_OK, BQ_ERR_NULL, BQ_ERR_DTYPE, BQ_ERR_SIZE, BQ_ERR_BLOCKSIZE, BQ_ERR_TABLE, BQ_ERR_ALIGNMENT,
 BQ_ERR_FORMAT, BQ_ERR_WORKSPACE, BQ_ERR_HIP) = range(10)

EXPORTS = ("bq_quantize_blockwise", "bq_dequantize_blockwise", "bq_quantize_nested",
           "bq_dequantize_nested", "bq_dequant_q32", "bq_iq2xs_quantize", "bq_iq2xs_dequantize",
           "bq_iq1s_quantize", "bq_iq1s_dequantize", "bq_nested_workspace_bytes", "bq_status_string",
           "bq_debug_nearest_codes", "bq_last_hip_error", "bq_linear_blockwise", "bq_gemm_blockwise",
           "bq_debug_time_next_kernel", "bq_quantize_nested_noalloc")


class BQError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = "%s: %s (status %d)" % (where, status_string(status), status)
        if status == BQ_ERR_HIP:
            msg += ", hipError_t %d" % _lib.bq_last_hip_error()
        super().__init__(msg)
        self.status = status


class bq_code_table(ctypes.Structure):
    _fields_ = [("entries", ctypes.POINTER(ctypes.c_float)), ("size", ctypes.c_int32)]


class bq_nested_stats(ctypes.Structure):
    _fields_ = [("qabsmax", ctypes.c_void_p), ("absmax2", ctypes.c_void_p), ("mean", ctypes.c_void_p),
                ("table", ctypes.POINTER(bq_code_table)), ("blocksize2", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbq.so is not built (run: python dequantization_block_absmax_amd/build.py)")
    # One HIP runtime per process: PyTorch ships its own libamdhip64 (same soname as ROCm's,
    # linked under another file name).  Loading torch first makes libbq bind to that
    # runtime; loading libbq first would bring in a second runtime that sees no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    tp = ctypes.POINTER(bq_code_table)
    sp = ctypes.POINTER(bq_nested_stats)
    sig = {
        "bq_quantize_blockwise": [vp, st, i64, i32, tp, vp, vp, vp],
        "bq_dequantize_blockwise": [vp, st, i64, i32, tp, vp, vp, vp],
        "bq_quantize_nested": [vp, st, i64, i32, tp, sp, vp, vp],
        "bq_quantize_nested_noalloc": [vp, st, i64, i32, tp, sp, vp, vp],
        "bq_dequantize_nested": [vp, st, i64, i32, tp, sp, vp, vp],
        "bq_dequant_q32": [vp, st, i64, i32, st, vp, vp],
        "bq_iq2xs_quantize": [vp, st, i64, i64, vp, vp, vp, vp, vp],
        "bq_iq2xs_dequantize": [vp, vp, i64, i64, st, vp, vp],
        "bq_iq1s_quantize": [vp, st, i64, i64, vp, vp, vp],
        "bq_iq1s_dequantize": [vp, vp, i64, i64, st, vp, vp],
        "bq_linear_blockwise": [vp, st, i64, i64, i64, i32, tp, vp, vp, vp, vp],
        "bq_gemm_blockwise": [vp, st, i64, i64, i64, i32, tp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = st
    lib.bq_nested_workspace_bytes.argtypes = [i64, i32, i32]
    lib.bq_nested_workspace_bytes.restype = ctypes.c_size_t
    lib.bq_debug_nearest_codes.argtypes = [tp, vp, i64, vp, vp, vp]
    lib.bq_debug_nearest_codes.restype = st
    lib.bq_debug_time_next_kernel.argtypes = [vp, vp]
    lib.bq_debug_time_next_kernel.restype = st
    lib.bq_last_hip_error.argtypes = []
    lib.bq_last_hip_error.restype = st
    lib.bq_status_string.argtypes = [st]
    lib.bq_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.bq_status_string(int(status)).decode()


def _addr(x) -> int | None:
    """Device address of a tensor, or an int address as given (None/0 -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream) -> int | None:
    """Raw hipStream_t: a torch stream, an int handle, or None for torch's current stream."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def dtype_code(dt) -> int:
    """bq_dtype of a torch dtype (or an int code, returned unchanged)."""
    if isinstance(dt, int):
        return dt
    import torch
    return {torch.float32: BQ_F32, torch.float16: BQ_F16, torch.bfloat16: BQ_BF16}[dt]


def code_table(entries) -> bq_code_table:
    """A bq_code_table over a host copy of `entries` (kept alive by the returned struct)."""
    arr = np.ascontiguousarray(np.asarray(entries, dtype=np.float32))
    t = bq_code_table(arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(arr.size))
    t._keep = arr
    return t


def _table_ptr(table):
    if table is None:
        return None
    if not isinstance(table, bq_code_table):
        table = code_table(table)
    return ctypes.pointer(table)


def nested_stats(qabsmax, absmax2, mean, table, blocksize2: int = 256, workspace=None,
                 workspace_bytes: int | None = None) -> bq_nested_stats:
    t = table if isinstance(table, bq_code_table) or table is None else code_table(table)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    s = bq_nested_stats(_addr(qabsmax), _addr(absmax2), _addr(mean),
                        ctypes.pointer(t) if t is not None else None, int(blocksize2), _addr(workspace),
                        int(workspace_bytes))
    s._keep = t
    return s


# ---- entry points (same names as the C ABI; each returns the bq_status) -----------------

def bq_quantize_blockwise(inp, dtype, n: int, blocksize: int, table, absmax, packed, stream=None) -> int:
    return _lib.bq_quantize_blockwise(_addr(inp), dtype_code(dtype), int(n), int(blocksize), _table_ptr(table),
                                      _addr(absmax), _addr(packed), _stream(stream))


def bq_dequantize_blockwise(out, dtype, n: int, blocksize: int, table, absmax, packed, stream=None) -> int:
    return _lib.bq_dequantize_blockwise(_addr(out), dtype_code(dtype), int(n), int(blocksize),
                                        _table_ptr(table), _addr(absmax), _addr(packed), _stream(stream))


def bq_quantize_nested(inp, dtype, n: int, blocksize: int, table, stats: bq_nested_stats | None, packed,
                       stream=None) -> int:
    return _lib.bq_quantize_nested(_addr(inp), dtype_code(dtype), int(n), int(blocksize), _table_ptr(table),
                                   ctypes.pointer(stats) if stats is not None else None, _addr(packed),
                                   _stream(stream))


def bq_quantize_nested_noalloc(inp, dtype, n: int, blocksize: int, table, stats: bq_nested_stats | None, packed,
                               stream=None) -> int:
    return _lib.bq_quantize_nested_noalloc(_addr(inp), dtype_code(dtype), int(n), int(blocksize), _table_ptr(table),
                                           ctypes.pointer(stats) if stats is not None else None, _addr(packed),
                                           _stream(stream))


def bq_dequantize_nested(out, dtype, n: int, blocksize: int, table, stats: bq_nested_stats | None, packed,
                         stream=None) -> int:
    return _lib.bq_dequantize_nested(_addr(out), dtype_code(dtype), int(n), int(blocksize), _table_ptr(table),
                                     ctypes.pointer(stats) if stats is not None else None, _addr(packed),
                                     _stream(stream))


def bq_dequant_q32(blocks, dtype, n: int, row_len: int, fmt: int, out, stream=None) -> int:
    return _lib.bq_dequant_q32(_addr(blocks), dtype_code(dtype), int(n), int(row_len), int(fmt), _addr(out),
                               _stream(stream))


def bq_iq2xs_quantize(x, dtype, n: int, row_len: int, grid, scales, blocks, rejected, stream=None) -> int:
    return _lib.bq_iq2xs_quantize(_addr(x), dtype_code(dtype), int(n), int(row_len), _addr(grid), _addr(scales),
                                  _addr(blocks), _addr(rejected), _stream(stream))


def bq_iq2xs_dequantize(blocks, grid, n: int, row_len: int, dtype, out, stream=None) -> int:
    return _lib.bq_iq2xs_dequantize(_addr(blocks), _addr(grid), int(n), int(row_len), dtype_code(dtype), _addr(out),
                                    _stream(stream))


def bq_iq1s_quantize(x, dtype, n: int, row_len: int, grid, blocks, stream=None) -> int:
    return _lib.bq_iq1s_quantize(_addr(x), dtype_code(dtype), int(n), int(row_len), _addr(grid), _addr(blocks),
                                 _stream(stream))


def bq_iq1s_dequantize(blocks, grid, n: int, row_len: int, dtype, out, stream=None) -> int:
    return _lib.bq_iq1s_dequantize(_addr(blocks), _addr(grid), int(n), int(row_len), dtype_code(dtype), _addr(out),
                                   _stream(stream))


def bq_linear_blockwise(x, dtype, M: int, K: int, N: int, blocksize: int, table, absmax, packed, y,
                        stream=None) -> int:
    return _lib.bq_linear_blockwise(_addr(x), dtype_code(dtype), int(M), int(K), int(N), int(blocksize),
                                    _table_ptr(table), _addr(absmax), _addr(packed), _addr(y), _stream(stream))


def bq_gemm_blockwise(x, dtype, M: int, K: int, N: int, blocksize: int, table, absmax, packed, y,
                      stream=None) -> int:
    return _lib.bq_gemm_blockwise(_addr(x), dtype_code(dtype), int(M), int(K), int(N), int(blocksize),
                                  _table_ptr(table), _addr(absmax), _addr(packed), _addr(y), _stream(stream))


def bq_nested_workspace_bytes(n: int, blocksize: int, blocksize2: int = 256) -> int:
    return int(_lib.bq_nested_workspace_bytes(int(n), int(blocksize), int(blocksize2)))


def bq_debug_nearest_codes(table, y: np.ndarray):
    """Host replay of the kernels' nearest-code search: returns (status, codes, mode, compares)."""
    yy = np.ascontiguousarray(y, dtype=np.float32)
    codes = np.zeros(max(yy.size, 1), np.int32)
    mode, cmp = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = _lib.bq_debug_nearest_codes(_table_ptr(table), yy.ctypes.data, yy.size, codes.ctypes.data,
                                     ctypes.addressof(mode), ctypes.addressof(cmp))
    return st, codes[:yy.size], mode.value, cmp.value


def _event(e) -> int | None:
    """Raw hipEvent_t of a torch.cuda.Event (created on first use), an int handle, or None."""
    if e is None or isinstance(e, int):
        return e or None
    if not e.cuda_event:
        e.record()  # torch creates the event on its first record
    return e.cuda_event or None


def bq_debug_time_next_kernel(start, stop) -> int:
    """Arms events for the next kernel the library launches on this thread (the data kernel of a
    nested quantize, or the only kernel of other calls): `stop` takes its end time, `start` is a
    marker just before it.  Either may be None."""
    return _lib.bq_debug_time_next_kernel(_event(start), _event(stop))


def bq_last_hip_error() -> int:
    return int(_lib.bq_last_hip_error())


def bq_status_string(status: int) -> str:
    return status_string(status)


def check(status: int, where: str = "bq") -> None:
    if status != BQ_OK:
        raise BQError(status, where)


# ---- sizes --------------------------------------------------------------------------------

def num_blocks(n: int, blocksize: int) -> int:
    return -(-int(n) // int(blocksize))


def packed_bytes(n: int, table_size: int) -> int:
    return int(n) if table_size == 256 else (int(n) + 1) // 2
