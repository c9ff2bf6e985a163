"""Helpers of the GPU parity tests: run the library through its C ABI on torch device buffers,
and run the oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth

TORCH_DT = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}
ORACLE_DT = {"float32": oracle.F32, "float16": oracle.F16, "bfloat16": oracle.BF16}
BQ_DT = {"float32": bq.BQ_F32, "float16": bq.BQ_F16, "bfloat16": bq.BQ_BF16}


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor as raw bits (uint16 for 16-bit types, float32 kept)."""
    c = t.detach().cpu().contiguous()
    if c.dtype in (torch.float16, torch.bfloat16):
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def oracle_input(x: torch.Tensor) -> np.ndarray:
    return host_bits(x)


def alloc(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)


def gpu_quantize(x: torch.Tensor, dtype: str, blocksize: int, table, stream=None):
    n = x.numel()
    K = len(table)
    nb = bq.num_blocks(n, blocksize)
    absmax = torch.full((max(nb, 1),), float("nan"), dtype=torch.float32, device=x.device)
    packed = torch.full((max(bq.packed_bytes(n, K), 16),), 0xAB, dtype=torch.uint8, device=x.device)
    bq.check(bq.bq_quantize_blockwise(x, BQ_DT[dtype], n, blocksize, table, absmax, packed, stream),
             "quantize")
    return absmax, packed


def gpu_dequantize(packed: torch.Tensor, absmax: torch.Tensor, n: int, dtype: str, blocksize: int, table,
                   stream=None) -> torch.Tensor:
    out = torch.full((max(n, 8),), 7, dtype=TORCH_DT[dtype], device=packed.device)
    bq.check(bq.bq_dequantize_blockwise(out, BQ_DT[dtype], n, blocksize, table, absmax, packed, stream),
             "dequantize")
    return out


def assert_f32_bits_equal(got: np.ndarray, expect: np.ndarray, what: str):
    """Bitwise equality of binary32 arrays; NaNs must be NaN on both sides."""
    got = np.asarray(got, np.float32)
    expect = np.asarray(expect, np.float32)
    assert got.shape == expect.shape, what
    gn, en = np.isnan(got), np.isnan(expect)
    assert np.array_equal(gn, en), "%s: NaN positions differ" % what
    gb, eb = got.view(np.uint32), expect.view(np.uint32)
    bad = np.nonzero((gb != eb) & ~gn)[0]
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %r expected %r" % (
        what, bad.size, bad[0], got[bad[0]], expect[bad[0]])


def assert_bytes_equal(got: np.ndarray, expect: np.ndarray, what: str):
    got = np.asarray(got)
    expect = np.asarray(expect)
    assert got.shape == expect.shape, "%s: shape %s vs %s" % (what, got.shape, expect.shape)
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %r expected %r" % (
        what, bad.size, bad[0], got[bad[0]], expect[bad[0]])


def assert_out_equal(got: torch.Tensor, expect: np.ndarray, n: int, dtype: str, what: str):
    g = host_bits(got)[:n]
    if dtype == "float32":
        assert_f32_bits_equal(g, expect, what)
    else:
        assert_bytes_equal(g, expect, what)


def check_blockwise(o: oracle.Oracle, x: torch.Tensor, dtype: str, blocksize: int, table, what: str,
                    out_dtypes=None):
    """Quantize + dequantize on the GPU and compare every output with the oracle."""
    n = x.numel()
    K = len(table)
    absmax, packed = gpu_quantize(x, dtype, blocksize, table)
    xin = oracle_input(x)
    oa, op = o.quantize_blockwise(xin, ORACLE_DT[dtype], blocksize, table)
    assert_f32_bits_equal(absmax.cpu().numpy()[:oa.size], oa, what + " absmax")
    assert_bytes_equal(packed.cpu().numpy()[:op.size], op, what + " packed")
    for odt in (out_dtypes or [dtype]):
        out = gpu_dequantize(packed, absmax, n, odt, blocksize, table)
        ref = o.dequantize_blockwise(op, oa, n, ORACLE_DT[odt], blocksize, table)
        assert_out_equal(out, ref, n, odt, what + " dequant->" + odt)
    return absmax, packed


def check_linear_against_oracle(o: oracle.Oracle, y: np.ndarray, x: torch.Tensor, dtype: str, N: int, B: int,
                                table, absmax, packed, tag: str):
    """bq_linear_blockwise output y (M x N, host) within the bound its C ABI states of the
    oracle's binary64 sum: |y - y_oracle| <= (K/1024 + 64) * 2^-24 * sum_k |x w|."""
    M, K = x.shape
    ref = o.linear_blockwise(host_bits(x), ORACLE_DT[dtype], M, K, N, B, table, absmax, packed)
    wdeq = o.dequantize_blockwise(packed, absmax, N * K, oracle.F32, B, table).astype(np.float64).reshape(N, K)
    mag = np.abs(x.float().cpu().numpy().astype(np.float64)) @ np.abs(wdeq).T
    tol = (K / 1024 + 64) * 2.0 ** -24 * mag
    err = np.abs(y.astype(np.float64) - ref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (tag, [(int(m), int(n), float(y[m, n]), float(ref[m, n]), float(tol[m, n]))
                                 for m, n in bad[:5]])


def bits_to_float64(bits: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])
    return t.float().numpy().astype(np.float64)


def check_gemm_against_oracle(o: oracle.Oracle, y: np.ndarray, x: torch.Tensor, dtype: str, N: int, B: int,
                              table, absmax, packed, tag: str):
    """bq_gemm_blockwise output y (M x N, host) within the bound its C ABI states of the
    oracle's binary64 sum over the 16-bit weights: |y - y_oracle| <= (K + 64) * 2^-24 * sum_k |x w16|."""
    M, K = x.shape
    ref = o.gemm_blockwise(host_bits(x), ORACLE_DT[dtype], M, K, N, B, table, absmax, packed)
    w16 = bits_to_float64(o.dequantize_blockwise(packed, absmax, N * K, ORACLE_DT[dtype], B, table), dtype)
    mag = np.abs(x.float().cpu().numpy().astype(np.float64)) @ np.abs(w16.reshape(N, K)).T
    tol = (K + 64) * 2.0 ** -24 * mag
    err = np.abs(y.astype(np.float64) - ref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (tag, [(int(m), int(n), float(y[m, n]), float(ref[m, n]), float(tol[m, n]))
                                 for m, n in bad[:5]])
