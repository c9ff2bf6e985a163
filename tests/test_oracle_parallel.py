"""The range-split oracle (oracle.ParallelOracle) gives the same bytes as one call of the C
oracle over the whole input: blocks (and statistics groups, and GGUF rows) are independent,
and the nested mean stays one call over the whole absmax array.  Ragged sizes put partial
blocks, odd element counts and partial groups at the ends of the ranges."""
import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(scope="module")
def pair():
    return oracle.Oracle(), oracle.ParallelOracle(threads=5)


def _bits(x):
    return np.atleast_1d(np.asarray(x)).view(np.uint8)


@pytest.mark.parametrize("dtype,B,K,n", [("bfloat16", 64, 16, 77_777), ("float16", 4096, 256, 100_003),
                                         ("float32", 32, 16, 12_345), ("float32", 256, 256, 1_001)])
def test_blockwise_same_bytes(pair, dtype, B, K, n):
    o, po = pair
    code = {"float32": oracle.F32, "float16": oracle.F16, "bfloat16": oracle.BF16}[dtype]
    x = synth.blockwise_input(n, dtype, 9, std=1.0, p_out=0.01, p_nf=0.001)
    xb = x.view(torch.int16).numpy().view(np.uint16) if dtype != "float32" else x.numpy()
    table = synth.table16() if K == 16 else synth.table256()
    a, p = o.quantize_blockwise(xb, code, B, table)
    a2, p2 = po.quantize_blockwise(xb, code, B, table)
    assert np.array_equal(_bits(a), _bits(a2)) and np.array_equal(p, p2)
    for odt in (oracle.F32, oracle.F16, oracle.BF16):
        d = o.dequantize_blockwise(p, a, n, odt, B, table)
        d2 = po.dequantize_blockwise(p, a, n, odt, B, table)
        assert np.array_equal(_bits(d), _bits(d2))


@pytest.mark.parametrize("B,B2,n", [(64, 256, 64 * 256 * 5 + 64 * 3 + 7), (32, 2048, 32 * 2048 * 2 + 99)])
def test_nested_same_bytes(pair, B, B2, n):
    o, po = pair
    x = synth.blockwise_input(n, "bfloat16", 10, std=0.02, p_out=0.001, p_nf=0.001)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    t16, t256 = synth.table16(), synth.table256()
    r = o.quantize_nested(xb, oracle.BF16, B, t16, t256, B2)
    r2 = po.quantize_nested(xb, oracle.BF16, B, t16, t256, B2)
    for k in r:
        assert np.array_equal(_bits(r[k]), _bits(r2[k])), k
    d = o.dequantize_nested(r["packed"], r["q2"], r["absmax2"], r["mean"], n, oracle.BF16, B, t16, t256, B2)
    d2 = po.dequantize_nested(r["packed"], r["q2"], r["absmax2"], r["mean"], n, oracle.BF16, B, t16, t256, B2)
    assert np.array_equal(d, d2)


@pytest.mark.parametrize("fmt", [oracle.Q4, oracle.Q8])
def test_q32_same_bytes(pair, fmt):
    o, po = pair
    rows, cols = 37, 448
    blocks = synth.q32_blocks(rows * cols // 32, "q4" if fmt == oracle.Q4 else "q8", seed=3).numpy()
    a = o.dequant_q32(blocks, rows * cols, cols, fmt, oracle.BF16)
    b = po.dequant_q32(blocks, rows * cols, cols, fmt, oracle.BF16)
    assert np.array_equal(a, b)
