"""GPU parity of the fused dequantize + linear (bq_linear_blockwise) against the oracle.

The GPU sums in binary32 in an order of its own, so each output is compared with the bound
the C ABI states: |y - y_oracle| <= (K/1024 + 64) * 2^-24 * sum_k |x[m][k] w[n][k]|, where
y_oracle is the oracle's binary64 sum (its own error, at most K * 2^-53 of the same sum, is
far inside the bound) and the sum of magnitudes comes from the oracle's binary32 dequantized
weights.  Weights are quantized by the oracle from seeded values, and the codes and block
maxima it produced are the inputs of both sides."""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import BQ_DT, ORACLE_DT, TORCH_DT, check_linear_against_oracle, host_bits

pytestmark = pytest.mark.gpu

DTYPES = ["float32", "float16", "bfloat16"]
TABLES = {16: synth.table16(), 256: synth.table256()}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def quantized_weights(o, N, K, B, table, seed):
    """N x K weights ~ N(0, 0.02) with a few outliers and one all-zero block, quantized by
    the oracle over the flat index."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(N * K) * 0.02).astype(np.float32)
    w[rng.integers(0, N * K, size=max(1, N * K // 997))] *= 40.0
    if N * K >= 2 * B:
        w[B:2 * B] = 0.0
    return o.quantize_blockwise(w, oracle.F32, B, table)


def activations(M, K, dtype, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(TORCH_DT[dtype])


def run_gpu(dev, x, dtype, N, B, table, absmax, packed):
    M, K = x.shape
    xd = x.to(dev).contiguous()
    a = torch.from_numpy(np.ascontiguousarray(absmax)).to(dev)
    p = torch.zeros(max(packed.size, 16), dtype=torch.uint8)
    p[:packed.size] = torch.from_numpy(np.ascontiguousarray(packed))
    p = p.to(dev)
    y = torch.full((M, max(N, 1)), float("nan"), dtype=torch.float32, device=dev)
    bq.check(bq.bq_linear_blockwise(xd, BQ_DT[dtype], M, K, N, B, bq.code_table(table), a, p, y), "linear")
    torch.cuda.synchronize()
    return y.cpu().numpy()[:, :N]


SHAPES = [  # (K, N, B): one-chunk, ragged chunk, several chunks per wave, partial row groups
    (16, 1, 32), (48, 9, 32), (1024, 8, 64), (1040, 17, 128), (3072, 5, 2048), (4112, 37, 4096),
    (9216, 11, 256),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K_table", [16, 256])
def test_linear_small_shapes(dev, o, dtype, K_table):
    table = TABLES[K_table]
    for i, (K, N, B) in enumerate(SHAPES):
        absmax, packed = quantized_weights(o, N, K, B, table, seed=100 + i)
        for M in (1, 2, 3, 4):
            x = activations(M, K, dtype, seed=200 + 10 * i + M)
            y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
            check_linear_against_oracle(o, y, x, dtype, N, B, table, absmax, packed,
                                 "%s K=%d N=%d B=%d M=%d table=%d" % (dtype, K, N, B, M, K_table))


def test_linear_exact_when_all_terms_exact(dev, o):
    """With the hand-worked dyadic table, power-of-two block maxima and small integer
    activations every product and partial sum is exact in binary32, so any summation order
    gives the oracle's value exactly."""
    table = np.float32([-1, -0.875, -0.75, -0.625, -0.5, -0.375, -0.25, -0.125, 0, 0.125, 0.25, 0.375,
                        0.5, 0.625, 0.75, 1])
    M, N, K, B = 4, 19, 2048, 64
    q = (np.arange(N)[:, None] * 5 + np.arange(K)[None, :] * 3) % 16
    flat = q.reshape(-1)
    packed = ((flat[0::2] << 4) | flat[1::2]).astype(np.uint8)
    absmax = np.ldexp(np.float32(1), (np.arange(N * K // B) % 5) - 2).astype(np.float32)
    x = torch.from_numpy(((np.arange(M * K).reshape(M, K) * 7) % 11 - 5).astype(np.float32)).to(torch.bfloat16)
    y = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    ref = o.linear_blockwise(host_bits(x), oracle.BF16, M, K, N, B, table, absmax, packed)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("K_table,M", [(16, 4), (256, 1)])
def test_linear_decode_shape_sampled_rows(dev, o, K_table, M):
    """The 14336 x 4096 weight of the benchmark (bf16 activations, B = 64), every output
    computed on the GPU; the oracle checks 40 sampled rows (first, last and random), and then
    every row.  The codes are seeded random bytes and the block maxima seeded log-normal
    values: the fused product reads them as given, whatever quantizer made them."""
    table = TABLES[K_table]
    N, K, B = 14336, 4096, 64
    rng = np.random.default_rng(7)
    packed = rng.integers(0, 256, size=N * K // 2 if K_table == 16 else N * K, dtype=np.uint8)
    absmax = (0.02 * np.exp(rng.standard_normal(N * K // B))).astype(np.float32)
    x = activations(M, K, "bfloat16", seed=8)
    y = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    assert np.all(np.isfinite(y))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(9).integers(0, N, 38)]))
    per_row = K // 2 if K_table == 16 else K
    sub_packed = np.concatenate([packed[r * per_row:(r + 1) * per_row] for r in rows])
    sub_absmax = np.concatenate([absmax[r * (K // B):(r + 1) * (K // B)] for r in rows])
    check_linear_against_oracle(o, y[:, rows], x, "bfloat16", len(rows), B, table, sub_absmax, sub_packed,
                         "decode shape table=%d M=%d" % (K_table, M))
    check_linear_against_oracle(o, y, x, "bfloat16", N, B, table, absmax, packed,
                                "decode shape, every row, table=%d M=%d" % (K_table, M))


# Tall weights with 4-bit codes at M = 3 or 4 take the matrix-core form (at least 32 weight
# rows per CU: 8192 on MI355X's 256 CUs; K a multiple of 64 up to 4096; blocks of 64 or more):
# a ragged last tile and run of tiles, waves and lane blocks past K, blocks longer than a row.
# (8200, 1040, 64) has K % 64 != 0 and takes the vector form.
MATRIX_CORE_SHAPES = [(8195, 4096, 64), (8200, 1088, 256), (8193, 64, 64), (8196, 3008, 4096), (8200, 1040, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_linear_matrix_core_form(dev, o, dtype):
    """Seeded random codes and log-normal block maxima (the product reads them as given), every
    output checked against the oracle within the stated bound."""
    table = TABLES[16]
    for i, (N, K, B) in enumerate(MATRIX_CORE_SHAPES):
        rng = np.random.default_rng(300 + i)
        packed = rng.integers(0, 256, size=N * K // 2, dtype=np.uint8)
        absmax = (0.02 * np.exp(rng.standard_normal(-(-N * K // B)))).astype(np.float32)
        for M in (3, 4):
            x = activations(M, K, dtype, seed=400 + 10 * i + M)
            y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
            check_linear_against_oracle(o, y, x, dtype, N, B, table, absmax, packed,
                                        "%s N=%d K=%d B=%d M=%d" % (dtype, N, K, B, M))


@pytest.mark.parametrize("M", [3, 4])
def test_linear_matrix_core_exact(dev, o, M):
    """The dyadic case of test_linear_exact_when_all_terms_exact on a weight tall enough for the
    matrix-core form: every product and partial sum is exact, so the result must equal the
    oracle's exactly (a lane, row or block mixed up in the matrix layout changes it)."""
    table = np.float32([-1, -0.875, -0.75, -0.625, -0.5, -0.375, -0.25, -0.125, 0, 0.125, 0.25, 0.375,
                        0.5, 0.625, 0.75, 1])
    N, K, B = 8196, 2048, 64
    q = (np.arange(N)[:, None] * 5 + np.arange(K)[None, :] * 3 + np.arange(N)[:, None] // 7) % 16
    flat = q.reshape(-1)
    packed = ((flat[0::2] << 4) | flat[1::2]).astype(np.uint8)
    absmax = np.ldexp(np.float32(1), (np.arange(N * K // B) % 5) - 2).astype(np.float32)
    x = torch.from_numpy(((np.arange(M * K).reshape(M, K) * 7) % 11 - 5).astype(np.float32)).to(torch.bfloat16)
    y = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    ref = o.linear_blockwise(host_bits(x), oracle.BF16, M, K, N, B, table, absmax, packed)
    assert np.array_equal(y.astype(np.float64), ref)
