"""GPU parity of the fused dequantize + GEMM on the matrix cores (bq_gemm_blockwise) against
the oracle.

The weights are the 16-bit values the dequantize writes, so every product is exact in
binary32 and only the accumulation order differs from the oracle's binary64 sum: each output
is compared with the bound the C ABI states, |y - y_oracle| <= (K + 64) * 2^-24 * sum_k
|x[m][k] w16[n][k]|, with the magnitudes from the oracle's own 16-bit weights.  Weights are
quantized by the oracle from seeded values; those codes and block maxima are the inputs of
both sides."""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import BQ_DT, ORACLE_DT, TORCH_DT, bits_to_float64, check_gemm_against_oracle, host_bits

pytestmark = pytest.mark.gpu

DTYPES = ["bfloat16", "float16"]
TABLES = {16: synth.table16(), 256: synth.table256()}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def quantized_weights(o, N, K, B, table, seed):
    """N x K weights ~ N(0, 0.02) with a few outliers and one all-zero block, quantized by the
    oracle over the flat index."""
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
    bq.check(bq.bq_gemm_blockwise(xd, BQ_DT[dtype], M, K, N, B, bq.code_table(table), a, p, y), "gemm")
    torch.cuda.synchronize()
    return y.cpu().numpy()[:, :N]


SHAPES = [  # (M, K, N, B): single tiles, ragged rows and columns, several chunks per wave; from
    # M = 129 the LDS-tiled kernel, with an odd number of 64-k steps (K = 192, 320)
    (1, 64, 1, 32), (5, 128, 33, 64), (32, 256, 64, 128), (33, 512, 65, 32), (64, 1024, 100, 256),
    (70, 192, 130, 4096), (129, 2048, 37, 1024), (257, 192, 131, 64), (300, 320, 260, 512),
    (200, 256, 100, 32),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K_table", [16, 256])
def test_gemm_small_shapes(dev, o, dtype, K_table):
    table = TABLES[K_table]
    for i, (M, K, N, B) in enumerate(SHAPES):
        absmax, packed = quantized_weights(o, N, K, B, table, seed=300 + i)
        x = activations(M, K, dtype, seed=400 + i)
        y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
        check_gemm_against_oracle(o, y, x, dtype, N, B, table, absmax, packed,
                             "%s M=%d K=%d N=%d B=%d table=%d" % (dtype, M, K, N, B, K_table))


def test_gemm_exact_when_all_terms_exact(dev, o):
    """Hand-worked dyadic table, power-of-two block maxima and small integer activations:
    every weight is exact in 16 bits and every partial sum exact in binary32, so any order of
    summation gives the oracle's value exactly, for both 16-bit types."""
    table = np.float32([-1, -0.875, -0.75, -0.625, -0.5, -0.375, -0.25, -0.125, 0, 0.125, 0.25, 0.375,
                        0.5, 0.625, 0.75, 1])
    N, K, B = 70, 1024, 64
    q = (np.arange(N)[:, None] * 5 + np.arange(K)[None, :] * 3) % 16
    flat = q.reshape(-1)
    packed = ((flat[0::2] << 4) | flat[1::2]).astype(np.uint8)
    absmax = np.ldexp(np.float32(1), (np.arange(N * K // B) % 5) - 2).astype(np.float32)
    for M in (40, 150):  # the register-tiled kernel, then the LDS-tiled one
        xi = ((np.arange(M * K).reshape(M, K) * 7) % 11 - 5).astype(np.float32)
        for dtype in DTYPES:
            x = torch.from_numpy(xi).to(TORCH_DT[dtype])
            y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
            ref = o.gemm_blockwise(host_bits(x), ORACLE_DT[dtype], M, K, N, B, table, absmax, packed)
            assert np.array_equal(y.astype(np.float64), ref), (dtype, M)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K_table", [16, 256])
def test_gemm_weights_match_the_16_bit_dequantize(dev, o, dtype, K_table):
    """Activation rows that are unit vectors pick single weights: y[m][n] = w16[n][k_m], one
    exact product, so y must equal the 16-bit weights the oracle's dequantize writes, bit for
    bit (this checks the rounding of each weight, which a summation bound cannot see)."""
    table = TABLES[K_table]
    N, K, B = 96, 512, 64
    absmax, packed = quantized_weights(o, N, K, B, table, seed=500 + K_table)
    w16 = bits_to_float64(o.dequantize_blockwise(packed, absmax, N * K, ORACLE_DT[dtype], B, table), dtype)
    # 13 rows (register-tiled kernel), then 171 (LDS-tiled kernel: every third k)
    for ks in (np.array([0, 1, 7, 63, 64, 65, 200, 255, 256, 333, 448, 510, 511]), np.arange(0, K, 3)):
        xf = np.zeros((len(ks), K), np.float32)
        xf[np.arange(len(ks)), ks] = 1.0
        x = torch.from_numpy(xf).to(TORCH_DT[dtype])
        y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
        assert np.array_equal(y.astype(np.float64), w16.reshape(N, K)[:, ks].T), len(ks)


@pytest.mark.parametrize("K_table,M", [(16, 64), (256, 200), (16, 1024), (256, 1024)])
def test_gemm_prefill_shape_sampled_rows(dev, o, K_table, M):
    """A 14336 x 4096 weight (bf16 activations, B = 64), every output computed on the GPU; the
    oracle checks 24 sampled weight rows (first, last and random) for every activation row.
    Codes are seeded random bytes and block maxima seeded log-normal values.  A second call
    must give the same bits."""
    table = TABLES[K_table]
    N, K, B = 14336, 4096, 64
    rng = np.random.default_rng(11)
    packed = rng.integers(0, 256, size=N * K // 2 if K_table == 16 else N * K, dtype=np.uint8)
    absmax = (0.02 * np.exp(rng.standard_normal(N * K // B))).astype(np.float32)
    x = activations(M, K, "bfloat16", seed=12)
    y = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    assert np.all(np.isfinite(y))
    y2 = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(13).integers(0, N, 22)]))
    per_row = K // 2 if K_table == 16 else K
    sub_packed = np.concatenate([packed[r * per_row:(r + 1) * per_row] for r in rows])
    sub_absmax = np.concatenate([absmax[r * (K // B):(r + 1) * (K // B)] for r in rows])
    check_gemm_against_oracle(o, y[:, rows], x, "bfloat16", len(rows), B, table, sub_absmax, sub_packed,
                         "prefill shape table=%d M=%d" % (K_table, M))


# Grids of 256-row tiles take the big-tile kernel (on MI355X's 256 CUs): 256 x 128 tiles when
# 192 to 256 of them cover the output, else 256 x 256 tiles when at least 128 do.  300 x 12200
# gives 2 x 96 tiles of 256 x 128 (44 rows in the last tile row, 40 columns in the last tile
# column); 1100 x 12290 gives 5 x 49 tiles of 256 x 256 (76 rows, 2 columns); K = 320 is an
# odd number of 64-k steps.


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("K_table", [16, 256])
@pytest.mark.parametrize("M,N,B", [(300, 12200, 32), (300, 12200, 64), (1100, 12290, 32), (1100, 12290, 64)])
def test_gemm_big_tiles_ragged(dev, o, dtype, K_table, M, N, B):
    """Seeded random codes and log-normal block maxima; the oracle checks about 30 sampled weight
    rows (tile edges, the last row and random ones) for every activation row; a second call
    gives the same bits."""
    table = TABLES[K_table]
    K = 320
    rng = np.random.default_rng(21 + K_table)
    packed = rng.integers(0, 256, size=N * K // 2 if K_table == 16 else N * K, dtype=np.uint8)
    absmax = (0.02 * np.exp(rng.standard_normal(-(-N * K // B)))).astype(np.float32)
    x = activations(M, K, dtype, seed=22)
    y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
    y2 = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    edges = [0, 63, 64, 127, 128, 255, 256, N - 41, N - 40, N - 3, N - 2, N - 1]
    rows = np.unique(np.concatenate([edges, np.random.default_rng(23).integers(0, N, 18)]))
    per_row = K // 2 if K_table == 16 else K
    sub_packed = np.concatenate([packed[r * per_row:(r + 1) * per_row] for r in rows])
    sub_absmax = np.concatenate([absmax[r * (K // B):(r + 1) * (K // B)] for r in rows])
    check_gemm_against_oracle(o, y[:, rows], x, dtype, len(rows), B, table, sub_absmax, sub_packed,
                              "big tiles %s table=%d" % (dtype, K_table))


@pytest.mark.parametrize("K_table", [16, 256])
def test_gemm_big_tiles_blocks_across_rows(dev, o, K_table):
    """Blocks of 256 over rows of K = 64 (each block spans four weight rows, so the scale of a
    staged chunk is not the scale of its row's first chunk) on a grid of 3 x 43 tiles of
    256 x 256 (520 x 11000: ragged in both directions); every output against the oracle."""
    table = TABLES[K_table]
    M, N, K, B = 520, 11000, 64, 256
    rng = np.random.default_rng(31 + K_table)
    packed = rng.integers(0, 256, size=N * K // 2 if K_table == 16 else N * K, dtype=np.uint8)
    absmax = (0.02 * np.exp(rng.standard_normal(-(-N * K // B)))).astype(np.float32)
    x = activations(M, K, "bfloat16", seed=32)
    y = run_gpu(dev, x, "bfloat16", N, B, table, absmax, packed)
    check_gemm_against_oracle(o, y, x, "bfloat16", N, B, table, absmax, packed,
                              "blocks across rows table=%d" % K_table)


@pytest.mark.parametrize("K_table", [16, 256])
@pytest.mark.parametrize("M,N", [(500, 12250), (1030, 9860)])
def test_gemm_big_tiles_exact(dev, o, K_table, M, N):
    """A dyadic table (k / 8 for k = -8 .. 7, or k / 128 for k = -128 .. 127, each exact in both
    16-bit types), power-of-two block maxima and small integer activations on a grid the
    big-tile kernel takes (500 x 12250: 2 x 96 tiles of 256 x 128; 1030 x 9860: 5 x 39 tiles of
    256 x 256): every weight and partial sum is exact,
    so sampled weight rows must equal the oracle's values exactly (a row, column or k mixed up
    in the fragment or staging layout changes them)."""
    half = K_table // 2
    table = (np.arange(-half, half) / half).astype(np.float32)
    K, B = 128, 64
    q = (np.arange(N)[:, None] * 5 + np.arange(K)[None, :] * 3 + np.arange(N)[:, None] // 9) % K_table
    if K_table == 16:  # two codes per byte, the first in the high nibble
        q = q.reshape(-1)
        packed = ((q[0::2] << 4) | q[1::2]).astype(np.uint8)
    else:
        packed = q.reshape(-1).astype(np.uint8)
    per_row = K // 2 if K_table == 16 else K
    absmax = np.ldexp(np.float32(1), (np.arange(N * K // B) % 5) - 2).astype(np.float32)
    xi = ((np.arange(M * K).reshape(M, K) * 7 + np.arange(M)[:, None] // 13) % 11 - 5).astype(np.float32)
    edges = [0, 31, 32, 63, 64, 127, 128, 255, 256, N - 1]
    rows = np.unique(np.concatenate([edges, np.random.default_rng(24).integers(0, N, 30)]))
    sub_packed = np.concatenate([packed[r * per_row:(r + 1) * per_row] for r in rows])
    sub_absmax = np.concatenate([absmax[r * (K // B):(r + 1) * (K // B)] for r in rows])
    for dtype in ("bfloat16", "float16"):
        x = torch.from_numpy(xi).to(TORCH_DT[dtype])
        y = run_gpu(dev, x, dtype, N, B, table, absmax, packed)
        ref = o.gemm_blockwise(host_bits(x), ORACLE_DT[dtype], M, K, len(rows), B, table, sub_absmax, sub_packed)
        assert np.array_equal(y[:, rows].astype(np.float64), ref), dtype
