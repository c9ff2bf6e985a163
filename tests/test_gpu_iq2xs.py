"""GPU parity of the IQ2_XS-style search encoder and its decoder (bq_iq2xs_quantize /
bq_iq2xs_dequantize through the C ABI) against the CPU oracle, byte for byte.

Inputs follow the blockwise recipe (normal weights, 1% outliers at 50x, 0.1% NaN / +-inf),
with caller scales from synth.iq2xs_scales, the special scales (+-0, NaN, +-inf, negative,
subnormal, the largest binary16) and special superblocks (all zero, elements whose squares or
products overflow binary32, binary32 subnormals, integer data with exact ties).  The grid is a
seeded 512-entry grid over the IQ2_XS byte alphabet {8, 25, 43}, or arbitrary bytes."""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import BQ_DT, ORACLE_DT, TORCH_DT, host_bits

pytestmark = pytest.mark.gpu

DTYPES = ["float32", "float16", "bfloat16"]
SPECIAL_SCALES = [0x0000, 0x8000, 0x7E00, 0x7C00, 0xFC00, 0xBC00, 0x8001, 0x0001, 0x7BFF]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def po():
    return oracle.ParallelOracle()


def gpu_encode(x: torch.Tensor, dtype: str, row_len: int, grid: torch.Tensor, scales: torch.Tensor):
    n = x.numel()
    nb = n // 256
    blocks = torch.full((max(nb * 74, 16),), 0xAB, dtype=torch.uint8, device=x.device)
    rejected = torch.zeros(1, dtype=torch.int32, device=x.device)
    bq.check(bq.bq_iq2xs_quantize(x, BQ_DT[dtype], n, row_len, grid, scales, blocks, rejected), "iq2xs quantize")
    torch.cuda.synchronize()
    return blocks[:nb * 74], int(rejected.item())


def gpu_decode(blocks: torch.Tensor, grid: torch.Tensor, n: int, row_len: int, dtype: str) -> torch.Tensor:
    out = torch.full((max(n, 8),), 7, dtype=TORCH_DT[dtype], device=blocks.device)
    bq.check(bq.bq_iq2xs_dequantize(blocks, grid, n, row_len, BQ_DT[dtype], out), "iq2xs dequantize")
    torch.cuda.synchronize()
    return out[:n]


def special_input(n: int, dtype: str, seed: int, dev) -> torch.Tensor:
    """The blockwise recipe plus special superblocks 0-4 (each superblock is 256 elements):
    all zero; integers in [-20, 20] (exact arithmetic, ties); a vector whose squares overflow
    binary32; a vector whose products with the grid overflow too (one negative element, odd
    parity); binary32 subnormals.  The overflowing cases need binary32's range (not fp16)."""
    x = synth.blockwise_input(n, dtype, seed, std=0.02, p_out=0.01, p_nf=0.001, device=dev)
    f = x.to(torch.float32)
    f[0:256] = 0.0
    if n // 256 > 4:
        f[256:512] = torch.arange(256, device=dev, dtype=torch.float32) % 41 - 20
        if dtype != "float16":
            f[512 + 8:512 + 16] = 3.0e19
            f[768 + 16:768 + 24] = 1.0e37
            f[768 + 16] = -1.0e37
            f[1024:1280] = f[1024:1280] * 2.0 ** -130
    return f.to(TORCH_DT[dtype])


def scales_for(x: torch.Tensor, seed: int) -> torch.Tensor:
    """synth.iq2xs_scales, with d = 8 for the integer superblock, d = 1 for the overflowing
    ones, d = 2^-7 for the subnormal one, then the special scales every third superblock."""
    s = synth.iq2xs_scales(x)
    nb = s.numel()
    as16 = lambda bits: int(np.uint16(bits).view(np.int16))  # noqa: E731
    if nb > 4:
        s[1], s[2], s[3], s[4] = as16(0x4800), as16(0x3C00), as16(0x3C00), as16(0x2000)
    for i, bits in enumerate(SPECIAL_SCALES):
        k = 5 + 3 * i
        if k < nb:
            s[k] = as16(bits)
    return s


def check_encode(po, x, dtype, row_len, grid_np, scales, dev, sample=None):
    grid = torch.from_numpy(grid_np.reshape(-1)).to(dev)
    blocks, rej = gpu_encode(x, dtype, row_len, grid, scales)
    xb = host_bits(x)
    sb = scales.cpu().numpy().view(np.uint16)
    got = blocks.cpu().numpy().reshape(-1, 74)
    if sample is None:
        want, want_rej = po.iq2xs_quantize(xb, ORACLE_DT[dtype], grid_np, sb)
        assert rej == want_rej, (rej, want_rej)
        want = want.reshape(-1, 74)
        idx = np.arange(got.shape[0])
    else:
        idx = sample
        xs = xb.reshape(-1, 256)[idx].reshape(-1)
        want, _ = po.iq2xs_quantize(xs, ORACLE_DT[dtype], grid_np, sb[idx])
        want = want.reshape(-1, 74)
        got = got[idx]
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "superblocks differ: %s (first: got %s want %s)" % (
        idx[bad[:8]].tolist(), got[bad[0]].tolist(), want[bad[0]].tolist())
    return blocks


@pytest.mark.parametrize("dtype", DTYPES)
def test_encode_parity(dev, po, dtype):
    rows, row_len = 12, 4096
    x = special_input(rows * row_len, dtype, 31, dev)
    check_encode(po, x, dtype, row_len, synth.iq2xs_grid(), scales_for(x, 31), dev)


@pytest.mark.parametrize("ratio", [0.3, 0.8, 2.5])
def test_encode_scale_ranges(dev, po, ratio):
    """Scales from too small to too large move the chosen local scales across all 16 values."""
    x = synth.blockwise_input(32 * 256, "bfloat16", 32, std=1.0, device=dev)
    check_encode(po, x, "bfloat16", 256, synth.iq2xs_grid(7), synth.iq2xs_scales(x, ratio), dev)


def test_encode_arbitrary_grid(dev, po):
    """A grid of arbitrary bytes (zeros and duplicate entries included)."""
    g = synth.u64(9, 8, 0, 4096).numpy().astype(np.uint64)
    grid = (g >> np.uint64(56)).astype(np.uint8).reshape(512, 8)
    grid[100] = grid[3]
    grid[7] = 0
    x = special_input(16 * 256, "float32", 33, dev)
    check_encode(po, x, "float32", 1024, grid, scales_for(x, 33), dev)


def test_encode_one_superblock_per_row(dev, po):
    x = synth.blockwise_input(3 * 256, "float16", 34, std=0.05, device=dev)
    check_encode(po, x, "float16", 256, synth.iq2xs_grid(), synth.iq2xs_scales(x), dev)


def test_encode_full_size_sampled(dev, po):
    """The 4096 x 14336 bf16 weight (229,376 superblocks) encoded in one call; 768 superblocks
    (the first, the last and a seeded sample) compared with the oracle one by one."""
    rows, cols = 4096, 14336
    x = synth.blockwise_input(rows * cols, "bfloat16", 35, std=0.02, p_out=0.01, p_nf=0.0001, device=dev)
    scales = synth.iq2xs_scales(x)
    nb = x.numel() // 256
    rng = np.random.default_rng(35)
    idx = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, 766)]))
    check_encode(po, x, "bfloat16", cols, synth.iq2xs_grid(), scales, dev, sample=idx)


@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_parity(dev, po, dtype):
    """Decoding the oracle's payloads and random bytes (any d, NaN and infinities included)."""
    grid_np = synth.iq2xs_grid()
    x = special_input(8 * 256, "float32", 36, dev)
    enc, _ = po.iq2xs_quantize(host_bits(x), oracle.F32, grid_np, scales_for(x, 36).cpu().numpy().view(np.uint16))
    rnd = (synth.u64(10, 9, 0, 24 * 74).numpy().astype(np.uint64) >> np.uint64(56)).astype(np.uint8)
    payload = np.concatenate([enc, rnd])
    n = payload.size // 74 * 256
    grid = torch.from_numpy(grid_np.reshape(-1)).to(dev)
    got = host_bits(gpu_decode(torch.from_numpy(payload).to(dev), grid, n, 512, dtype))
    want = po.iq2xs_dequantize(payload, grid_np, n, ORACLE_DT[dtype])
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


def test_rejected_counter_accumulates(dev, po):
    """*rejected counts rejected superblocks and is only ever incremented."""
    x = synth.blockwise_input(8 * 256, "bfloat16", 37, std=0.02, device=dev)
    s = synth.iq2xs_scales(x)
    s[1] = int(np.uint16(0x7E00).view(np.int16))
    s[6] = int(np.uint16(0xC000).view(np.int16))
    grid = torch.from_numpy(synth.iq2xs_grid().reshape(-1)).to(dev)
    blocks = torch.empty(8 * 74, dtype=torch.uint8, device=dev)
    rejected = torch.full((1,), 5, dtype=torch.int32, device=dev)
    for _ in range(2):
        bq.check(bq.bq_iq2xs_quantize(x, bq.BQ_BF16, x.numel(), 2048, grid, s, blocks, rejected), "iq2xs")
    torch.cuda.synchronize()
    assert int(rejected.item()) == 5 + 2 * 2
    got = blocks.cpu().numpy().reshape(8, 74)
    assert not got[1].any() and not got[6].any()
