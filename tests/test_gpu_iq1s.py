"""GPU parity of the IQ1_S-style encoder and its decoder (bq_iq1s_quantize /
bq_iq1s_dequantize through the C ABI) against the CPU oracle, byte for byte.

Inputs follow the blockwise recipe (normal weights, 1% outliers at 50x, 0.1% NaN / +-inf) plus
special superblocks: all zero, integers (exact arithmetic and ties), a vector whose squares
overflow binary32, one whose shifted dots overflow as well, binary32 subnormals, and a block
whose scale saturates binary16.  The grid is a seeded 2048-entry ternary grid, or arbitrary
signed bytes."""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import BQ_DT, ORACLE_DT, TORCH_DT, host_bits

pytestmark = pytest.mark.gpu

DTYPES = ["float32", "float16", "bfloat16"]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def po():
    return oracle.ParallelOracle()


def gpu_encode(x: torch.Tensor, dtype: str, row_len: int, grid: torch.Tensor) -> torch.Tensor:
    n = x.numel()
    nb = n // 256
    blocks = torch.full((max(nb * 50, 16),), 0xAB, dtype=torch.uint8, device=x.device)
    bq.check(bq.bq_iq1s_quantize(x, BQ_DT[dtype], n, row_len, grid, blocks), "iq1s quantize")
    torch.cuda.synchronize()
    return blocks[:nb * 50]


def gpu_decode(blocks: torch.Tensor, grid: torch.Tensor, n: int, row_len: int, dtype: str) -> torch.Tensor:
    out = torch.full((max(n, 8),), 7, dtype=TORCH_DT[dtype], device=blocks.device)
    bq.check(bq.bq_iq1s_dequantize(blocks, grid, n, row_len, BQ_DT[dtype], out), "iq1s dequantize")
    torch.cuda.synchronize()
    return out[:n]


def special_input(n: int, dtype: str, seed: int, dev) -> torch.Tensor:
    """The blockwise recipe plus special superblocks 0-5 (each superblock is 256 elements)."""
    x = synth.blockwise_input(n, dtype, seed, std=0.02, p_out=0.01, p_nf=0.001, device=dev)
    f = x.to(torch.float32)
    f[0:256] = 0.0
    if n // 256 > 5:
        f[256:512] = torch.arange(256, device=dev, dtype=torch.float32) % 41 - 20
        if dtype != "float16":
            f[512 + 8:512 + 16] = 3.0e19
            f[768 + 16:768 + 24] = 1.0e37
            f[768 + 17] = -1.0e37
            f[1024:1280] = f[1024:1280] * 2.0 ** -130
            f[1280:1536] = f[1280:1536] * 1.0e12  # the scale saturates binary16
    return f.to(TORCH_DT[dtype])


def check_encode(po, x, dtype, row_len, grid_np, dev, sample=None):
    grid = torch.from_numpy(grid_np.reshape(-1)).to(dev)
    got = gpu_encode(x, dtype, row_len, grid).cpu().numpy().reshape(-1, 50)
    xb = host_bits(x)
    if sample is None:
        want = po.iq1s_quantize(xb, ORACLE_DT[dtype], grid_np).reshape(-1, 50)
        idx = np.arange(got.shape[0])
    else:
        idx = sample
        want = po.iq1s_quantize(xb.reshape(-1, 256)[idx].reshape(-1), ORACLE_DT[dtype], grid_np).reshape(-1, 50)
        got = got[idx]
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "superblocks differ: %s (first: got %s want %s)" % (
        idx[bad[:8]].tolist(), got[bad[0]].tolist(), want[bad[0]].tolist())


@pytest.mark.parametrize("dtype", DTYPES)
def test_encode_parity(dev, po, dtype):
    x = special_input(8 * 2048, dtype, 51, dev)
    check_encode(po, x, dtype, 2048, synth.iq1s_grid(), dev)


@pytest.mark.parametrize("std", [0.001, 1.0, 300.0])
def test_encode_magnitudes(dev, po, std):
    x = synth.blockwise_input(16 * 256, "bfloat16", 52, std=std, device=dev)
    check_encode(po, x, "bfloat16", 256, synth.iq1s_grid(9), dev)


def test_encode_arbitrary_grid(dev, po):
    """A grid of arbitrary signed bytes (duplicates included)."""
    g = synth.u64(11, 8, 0, 2048 * 8).numpy().astype(np.uint64)
    grid = (g >> np.uint64(56)).astype(np.uint8).view(np.int8).reshape(2048, 8)
    grid[900] = grid[7]
    x = special_input(8 * 256, "float32", 53, dev)
    check_encode(po, x, "float32", 1024, grid, dev)


def test_encode_full_size_sampled(dev, po):
    """The 4096 x 14336 bf16 weight in one call; 384 superblocks (the first, the last and a
    seeded sample) compared with the oracle one by one."""
    rows, cols = 4096, 14336
    x = synth.blockwise_input(rows * cols, "bfloat16", 54, std=0.02, p_out=0.01, p_nf=0.0001, device=dev)
    nb = x.numel() // 256
    rng = np.random.default_rng(54)
    idx = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, 382)]))
    check_encode(po, x, "bfloat16", cols, synth.iq1s_grid(), dev, sample=idx)


@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_parity(dev, po, dtype):
    """Decoding the oracle's payloads and random bytes (any d, NaN and infinities included),
    with the ternary grid and with arbitrary signed bytes."""
    x = special_input(8 * 256, "float32", 55, dev)
    rnd = (synth.u64(12, 9, 0, 24 * 50).numpy().astype(np.uint64) >> np.uint64(56)).astype(np.uint8)
    g = synth.u64(13, 8, 0, 2048 * 8).numpy().astype(np.uint64)
    for grid_np in (synth.iq1s_grid(), (g >> np.uint64(56)).astype(np.uint8).view(np.int8).reshape(2048, 8)):
        payload = np.concatenate([po.iq1s_quantize(host_bits(x), oracle.F32, grid_np), rnd])
        n = payload.size // 50 * 256
        grid = torch.from_numpy(grid_np.reshape(-1)).to(dev)
        got = host_bits(gpu_decode(torch.from_numpy(payload).to(dev), grid, n, 512, dtype))
        want = po.iq1s_dequantize(payload, grid_np, n, ORACLE_DT[dtype])
        if dtype == "float32":
            gn, wn = np.isnan(got), np.isnan(want)
            assert np.array_equal(gn, wn)
            assert np.array_equal(got.view(np.uint32)[~gn], want.view(np.uint32)[~wn])
        else:
            isnan = lambda b: (b & 0x7FFF) > (0x7C00 if dtype == "float16" else 0x7F80)  # noqa: E731
            assert np.array_equal(isnan(got), isnan(want))
            ok = ~isnan(want)
            bad = np.nonzero(got[ok] != want[ok])[0]
            assert bad.size == 0, (bad[:8], got[ok][bad[:8]], want[ok][bad[:8]])
