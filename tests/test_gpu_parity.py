"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for bit.

Every output is compared in full with the oracle: small and ragged shapes (several
8192-element tiles and tails, every dtype, table size and block size) and the five full-size
benchmark workloads.  At the full sizes the oracle runs on contiguous ranges of whole blocks
(groups, rows) from several host threads (oracle.ParallelOracle), which gives the same bytes
as one call over the whole input."""
import json
import os

import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import (BQ_DT, ORACLE_DT, TORCH_DT, assert_bytes_equal, assert_f32_bits_equal,
                         assert_out_equal, check_blockwise, gpu_dequantize, gpu_quantize, host_bits,
                         oracle_input)

pytestmark = pytest.mark.gpu

BLOCKSIZES = [32, 64, 128, 256, 512, 1024, 2048, 4096]
DTYPES = ["float32", "float16", "bfloat16"]
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.fixture(scope="module")
def po():
    return oracle.ParallelOracle()


def _sync():
    torch.cuda.synchronize()


# ---- hand-worked golden examples ---------------------------------------------------------

def test_golden_examples_on_gpu(dev, o):
    g = json.load(open(os.path.join(GOLDEN, "blockwise_4bit_dyadic.json")))
    table = np.float32([float(v) for v in g["table"]])
    for ex in g["examples"]:
        vals = [float.fromhex(v) if v.startswith(("0x", "-0x")) else float(v) for v in ex["x"]]
        x = torch.tensor(np.float32(vals), device=dev)
        absmax, packed = gpu_quantize(x, "float32", ex["blocksize"], table)
        nbytes = (len(vals) + 1) // 2
        assert packed.cpu().numpy()[:nbytes].tobytes().hex() == ex["packed_hex"].replace(" ", ""), ex["name"]
        assert absmax.cpu().numpy()[0] == np.float32(float(ex["absmax"][0])), ex["name"]
        out = gpu_dequantize(packed, absmax, len(vals), "float32", ex["blocksize"], table)
        expect = np.float32([float(v) for v in ex["dequant_f32"]])
        assert_f32_bits_equal(out.cpu().numpy()[:len(vals)], expect, ex["name"])


def test_golden_q32_on_gpu(dev):
    g = json.load(open(os.path.join(GOLDEN, "dequant_rounding_gguf_nested.json")))["q32"]
    for blk_hex, vals in zip(g["q4_blocks_hex"], g["q4_values"]):
        blocks = torch.tensor(np.frombuffer(bytes.fromhex(blk_hex), np.uint8).copy(), device=dev)
        blocks = torch.cat([blocks, torch.zeros(14, dtype=torch.uint8, device=dev)])
        out = torch.empty(32, dtype=torch.float32, device=dev)
        bq.check(bq.bq_dequant_q32(blocks, bq.BQ_F32, 32, 32, bq.BQ_Q32_Q4, out))
        assert_f32_bits_equal(out.cpu().numpy(), np.float32([float(v) for v in vals]), blk_hex)
    for d_hex, codes, vals in zip(g["q8_blocks_hex"], g["q8_codes"], g["q8_values"]):
        raw = np.concatenate([np.frombuffer(bytes.fromhex(d_hex), np.uint8), np.int8(codes).view(np.uint8)])
        blocks = torch.tensor(np.concatenate([raw, np.zeros(14, np.uint8)]), device=dev)
        out = torch.empty(32, dtype=torch.bfloat16, device=dev)
        bq.check(bq.bq_dequant_q32(blocks, bq.BQ_BF16, 32, 32, bq.BQ_Q32_Q8, out))
        expect = torch.tensor([float(v) for v in vals]).to(torch.bfloat16)
        assert torch.equal(out.cpu(), expect), d_hex


# ---- small and ragged shapes, all dtypes, tables and block sizes --------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [16, 256])
def test_ragged_shapes(dev, o, dtype, K):
    table = synth.table16() if K == 16 else synth.table256()
    seed = 100 + K + DTYPES.index(dtype)
    for B in BLOCKSIZES:
        for n in (1, 31, 33, B - 1, B + 1, 3 * B + 5, 8192 + 17, 3 * 8192 + B + 3):
            x = synth.blockwise_input(n, dtype, seed + n, std=1.0, p_out=0.01, p_nf=0.003, device=dev)
            check_blockwise(o, x, dtype, B, table, "%s K=%d B=%d n=%d" % (dtype, K, B, n))


@pytest.mark.parametrize("dtype", DTYPES)
def test_cross_dtype_outputs(dev, o, dtype):
    """Dequantize into every output dtype from the same codes."""
    x = synth.blockwise_input(3 * 8192 + 77, dtype, 7, std=3.0, p_out=0.01, p_nf=0.001, device=dev)
    for table in (synth.table16(), synth.table256()):
        check_blockwise(o, x, dtype, 128, table, "cross " + dtype, out_dtypes=DTYPES)


# ---- special values ----------------------------------------------------------------------

def _special_blocks(dtype: str, B: int) -> torch.Tensor:
    rng = np.random.default_rng(5)
    blocks = []
    tiny32 = np.float32(2.0**-140)
    if dtype == "float32":
        scales = [1.0, 2.0**-130, 2.0**-70, 2.0**-64, 2.0**-63, 2.0**64, 2.0**65, 2.0**100, 3e38]
    elif dtype == "bfloat16":
        scales = [1.0, 2.0**-130, 2.0**-70, 2.0**-64, 2.0**64, 2.0**100, 3e38]
    else:
        scales = [1.0, 2.0**-20, 6e-5, 2.0**-24, 60000.0]
    for s in scales:
        blocks.append(rng.normal(0, 1, B) * s)
    blocks.append(np.zeros(B))
    blocks.append(-np.zeros(B))
    blocks.append(np.full(B, np.nan))
    blocks.append(np.where(np.arange(B) % 2 == 0, np.inf, -np.inf))
    blocks.append(np.where(np.arange(B) % 3 == 0, np.nan, rng.normal(0, 1, B)))
    b = rng.normal(0, 1, B)
    b[[0, B // 2, B - 1]] = [np.inf, -np.inf, np.nan]
    blocks.append(b)
    if dtype == "float32":
        blocks.append(rng.normal(0, 1, B) * float(tiny32))  # subnormal inputs
        blocks.append(np.float32(np.arange(B) - B // 2) * np.float32(2.0**-149))
    if dtype == "bfloat16":
        blocks.append(np.float32(np.arange(B) - B // 2) * np.float32(2.0**-133))
    if dtype == "float16":
        blocks.append(np.float32(np.arange(B) - B // 2) * np.float32(2.0**-24))
    arr = np.concatenate(blocks).astype(np.float64)
    t = torch.tensor(arr, dtype=torch.float64).to(torch.float32).to(TORCH_DT[dtype])
    return t


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B", [32, 256, 4096])
def test_special_values(dev, o, dtype, B):
    x = _special_blocks(dtype, B).to(dev)
    for table in (synth.table16(), synth.table256()):
        check_blockwise(o, x, dtype, B, table, "special %s B=%d K=%d" % (dtype, B, len(table)),
                        out_dtypes=DTYPES)


def test_dequant_of_arbitrary_codes_and_absmax(dev, o):
    """Every code value, absmax values including NaN, +-Inf, 0, huge and subnormal."""
    rng = np.random.default_rng(9)
    n = 8192 * 2 + 3
    for table, B in ((synth.table16(), 64), (synth.table256(), 32)):
        K = len(table)
        nb = -(-n // B)
        absmax = np.abs(rng.normal(0, 2, nb)).astype(np.float32)
        absmax[:8] = [np.nan, np.inf, -np.inf, 0.0, -0.0, 3e38, 1e-40, 70000.0]
        packed = rng.integers(0, 256, (n + 1) // 2 if K == 16 else n).astype(np.uint8)
        pd = torch.tensor(np.concatenate([packed, np.zeros(16, np.uint8)]), device=dev)
        ad = torch.tensor(absmax, device=dev)
        for odt in DTYPES:
            out = gpu_dequantize(pd, ad, n, odt, B, table)
            ref = o.dequantize_blockwise(packed, absmax, n, ORACLE_DT[odt], B, table)
            assert_out_equal(out, ref, n, odt, "arbitrary codes K=%d -> %s" % (K, odt))


# ---- every search mode ---------------------------------------------------------------------

SEARCH_TABLES = {
    "hand16": np.float32([-1, -0.875, -0.75, -0.625, -0.5, -0.375, -0.25, -0.125, 0, 0.125, 0.25, 0.375,
                          0.5, 0.625, 0.75, 1]),
    "dyadic256": synth.dyadic_table(256),
    "nf4_like": np.float32(np.sort(np.concatenate([[-1, 0, 1], np.linspace(-0.7, 0.72, 13)]))),
    "tiny_entries": np.float32(np.sort(np.concatenate([[-1, 0, 1, 2.0**-20, -2.0**-20, 2.0**-19],
                                                       np.linspace(0.1, 0.9, 10)]))),
    "clustered256": np.float32(np.sort(np.concatenate([np.linspace(-1, 0.45, 56),
                                                       0.5 + np.arange(200) * 2.0**-23 * 8]))),
    "dense_top16": np.float32(np.concatenate([np.linspace(-1, 0.9, 12), [0.93, 0.96, 0.98, 1.0]])),
    # binary16 buckets with thresholds in the binary16 subnormal range
    "subnormal16": np.float32(np.sort(np.concatenate([
        s * np.concatenate([np.arange(1, 17) * 2.0**-19, np.geomspace(2.0**-14, 1.0, 112)]) for s in (-1, 1)]))),
}


@pytest.mark.parametrize("name", sorted(SEARCH_TABLES))
def test_search_modes(dev, o, name):
    table = SEARCH_TABLES[name]
    st, _, mode, cmp = bq.bq_debug_nearest_codes(table, np.float32([0.0]))
    assert st == bq.BQ_OK
    x = synth.blockwise_input(4 * 8192 + 100, "float32", 11, std=1.0, p_out=0.01, p_nf=0.001, device=dev)
    # values clustered around the dense region hit the many-threshold buckets
    xc = x.clone()
    xc[::3] = 0.5 + (xc[::3] * 1e-4)
    # blocks whose maximum is 1 and whose other values are tiny: y down to the binary16
    # subnormal range and below
    xt = x.clone()
    xt[::64] = 1.0
    xt[1::2] = xt[1::2] * (2.0 ** -18)
    xt[3::4] = xt[3::4] * (2.0 ** -6)
    for B in (64, 4096):
        check_blockwise(o, x, "float32", B, table, "%s mode=%d cmp=%d B=%d" % (name, mode, cmp, B))
        check_blockwise(o, xc, "float32", B, table, "%s clustered B=%d" % (name, B))
        check_blockwise(o, xt, "float32", B, table, "%s tiny B=%d" % (name, B))


# ---- determinism and stream semantics ------------------------------------------------------

def test_determinism_across_runs_and_streams(dev):
    x = synth.blockwise_input(1 << 20, "bfloat16", 3, std=0.02, p_out=0.001, p_nf=0.0001, device=dev)
    t16 = synth.table16()
    a0, p0 = gpu_quantize(x, "bfloat16", 64, t16)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a1, p1 = gpu_quantize(x, "bfloat16", 64, t16, stream=s)
    s.synchronize()
    _sync()
    assert torch.equal(p0, p1) and torch.equal(a0.view(torch.int32), a1.view(torch.int32))
    o0 = gpu_dequantize(p0, a0, x.numel(), "bfloat16", 64, t16)
    o1 = gpu_dequantize(p0, a0, x.numel(), "bfloat16", 64, t16)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def test_runs_on_the_callers_stream(dev, o):
    """The input is produced on a side stream behind a long device-side delay; the quantizer
    is enqueued on that stream at once and must see the produced values, not stale ones."""
    n = 1 << 22
    t16 = synth.table16()
    src = synth.blockwise_input(n, "bfloat16", 21, std=1.0, device=dev)
    x = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    absmax = torch.zeros(n // 64, dtype=torch.float32, device=dev)
    packed = torch.zeros(n // 2, dtype=torch.uint8, device=dev)
    _sync()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # a device-side delay before the producer runs
        x.copy_(src)
        bq.check(bq.bq_quantize_blockwise(x, bq.BQ_BF16, n, 64, t16, absmax, packed, s))
    s.synchronize()
    oa, op = o.quantize_blockwise(host_bits(src), oracle.BF16, 64, t16)
    assert_f32_bits_equal(absmax.cpu().numpy(), oa, "stream absmax")
    assert_bytes_equal(packed.cpu().numpy(), op, "stream packed")


# ---- nested statistics ---------------------------------------------------------------------

def gpu_nested(x: torch.Tensor, dtype: str, B: int, t16, t256, B2=256, out_dtype=None):
    n = x.numel()
    dev = x.device
    nb = bq.num_blocks(n, B)
    ng = bq.num_blocks(nb, B2)
    ws_bytes = bq.bq_nested_workspace_bytes(n, B, B2)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    q2 = torch.full((max(nb, 16),), 0xCD, dtype=torch.uint8, device=dev)
    absmax2 = torch.full((max(ng, 1),), float("nan"), dtype=torch.float32, device=dev)
    mean = torch.full((4,), float("nan"), dtype=torch.float32, device=dev)
    packed = torch.full((max(bq.packed_bytes(n, len(t16)), 16),), 0xAB, dtype=torch.uint8, device=dev)
    stats = bq.nested_stats(q2, absmax2, mean, t256, B2, ws, ws_bytes)
    bq.check(bq.bq_quantize_nested(x, BQ_DT[dtype], n, B, t16, stats, packed), "quantize_nested")
    out = torch.empty(max(n, 8), dtype=TORCH_DT[out_dtype or dtype], device=dev)
    bq.check(bq.bq_dequantize_nested(out, BQ_DT[out_dtype or dtype], n, B, t16, stats, packed), "dequantize_nested")
    return dict(absmax=workspace_absmax(ws, nb, dtype), q2=q2[:nb], absmax2=absmax2[:ng], mean=mean[0],
                packed=packed, out=out)


def workspace_absmax(ws: torch.Tensor, nb: int, dtype: str) -> torch.Tensor:
    """The block maxima the nested quantize leaves at the start of its workspace, widened to
    binary32: stored as binary32 for fp32 input and as the input's 16-bit type otherwise."""
    if dtype == "float32":
        return ws[:nb * 4].view(torch.float32)
    return ws[:nb * 2].view(TORCH_DT[dtype]).float()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,B2", [(64, 256), (32, 32), (128, 64), (4096, 256), (256, 4096), (512, 32), (1024, 64),
                                  (2048, 128), (32, 512), (64, 1024), (128, 2048)])
def test_nested_full_parity(dev, o, dtype, B, B2):
    t16, t256 = synth.table16(), synth.table256()
    for n in (B * B2 * 3 + B * 7 + 5, 777, B * B2):
        x = synth.blockwise_input(n, dtype, 31 + n, std=0.02, p_out=0.001, p_nf=0.001, device=dev)
        r = gpu_nested(x, dtype, B, t16, t256, B2)
        ref = o.quantize_nested(oracle_input(x), ORACLE_DT[dtype], B, t16, t256, B2)
        what = "nested %s B=%d B2=%d n=%d" % (dtype, B, B2, n)
        assert_f32_bits_equal(r["absmax"].cpu().numpy(), ref["absmax"], what + " absmax")
        assert np.float32(r["mean"].item()).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), \
            what + " mean"
        assert_bytes_equal(r["q2"].cpu().numpy(), ref["q2"], what + " q2")
        assert_f32_bits_equal(r["absmax2"].cpu().numpy(), ref["absmax2"], what + " absmax2")
        assert_bytes_equal(r["packed"].cpu().numpy()[:ref["packed"].size], ref["packed"], what + " packed")
        out_ref = o.dequantize_nested(ref["packed"], ref["q2"], ref["absmax2"], ref["mean"], n, ORACLE_DT[dtype],
                                      B, t16, t256, B2)
        assert_out_equal(r["out"], out_ref, n, dtype, what + " dequant")


def test_nested_mean_tree_shapes(dev, o):
    """Block counts around powers of two and the per-wave partial-sum runs, with magnitudes
    spread over many binades so that any other summation order would change the mean."""
    t16, t256 = synth.table16(), synth.table256()
    rng = np.random.default_rng(77)
    # the last two give 11,995 and 32,961 per-wave partial sums: several ragged 2048-runs
    for nb in (1, 2, 255, 256, 257, 1023, 1024, 1025, 65536 + 1, 262144 + 256 * 3 + 1, 2999 * 256 - 77,
               2 * 4096 * 256 + 12345):
        heads = np.float32(np.abs(rng.normal(0, 1, nb)) * 2.0 ** rng.integers(-30, 30, nb))
        x = np.zeros(nb * 32, np.float32)
        x[::32] = heads
        xd = torch.tensor(x, device=dev)
        r = gpu_nested(xd, "float32", 32, t16, t256, 256)
        m_ref = o.nested_mean(heads)
        assert np.float32(r["mean"].item()).view(np.uint32) == np.float32(m_ref).view(np.uint32), nb


def test_nested_mean_many_runs(dev, o):
    """2^33 + 3 * 2^23 fp16 elements in blocks of 32: 4,206,592 per-wave partial sums, so 2054
    runs of 2048 remain and the separate mean kernel finishes the tree.  Only block heads
    are nonzero, so the oracle needs just the 2^28 + 3 * 2^18 block maxima; sampled groups of
    q2 / absmax2 are checked one by one."""
    B, B2 = 32, 256
    n = (1 << 33) + 3 * (1 << 23)
    nb = n // B
    rng = np.random.default_rng(5)
    heads = (np.abs(rng.normal(0, 1, nb)) * 2.0 ** rng.integers(-12, 12, nb)).astype(np.float16)
    heads_f32 = heads.astype(np.float32)
    x = torch.zeros(n, dtype=torch.float16, device=dev)
    x[::B] = torch.from_numpy(heads).to(dev)
    t16, t256 = synth.table16(), synth.table256()
    ng = nb // B2
    ws_bytes = bq.bq_nested_workspace_bytes(n, B, B2)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    q2 = torch.empty(nb, dtype=torch.uint8, device=dev)
    absmax2 = torch.empty(ng, dtype=torch.float32, device=dev)
    mean = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    packed = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    stats = bq.nested_stats(q2, absmax2, mean, t256, B2, ws, ws_bytes)
    bq.check(bq.bq_quantize_nested(x, BQ_DT["float16"], n, B, t16, stats, packed), "quantize_nested")
    del x, packed
    m_ref = o.nested_mean(heads_f32)
    assert np.float32(mean.item()).view(np.uint32) == np.float32(m_ref).view(np.uint32)
    table = np.float32(t256)
    for g in (0, 1, ng // 2, ng - 1):
        d = (heads_f32[g * B2:(g + 1) * B2] - m_ref).astype(np.float32)
        a2 = np.float32(np.abs(d).max())
        assert np.float32(absmax2[g].item()).view(np.uint32) == a2.view(np.uint32), g
        want = [o.nearest(o.normalize(v, a2), table) for v in d]
        assert q2[g * B2:(g + 1) * B2].cpu().numpy().tolist() == want, g


# ---- the five benchmark workloads ----------------------------------------------------------

def test_fp32_2pow19_4bit_blocksize64(dev, o):
    x = synth.blockwise_input(524288, "float32", 1, std=1.0, device=dev)
    check_blockwise(o, x, "float32", 64, synth.table16(), "fp32 2^19 B=64")


def test_fp16_2pow23plus1_4bit_all_blocksizes(dev, po):
    x = synth.blockwise_input(8388609, "float16", 2, std=1.0, p_out=1e-3, p_nf=1e-4, device=dev)
    for B in BLOCKSIZES:
        check_blockwise(po, x, "float16", B, synth.table16(), "fp16 2^23+1 B=%d" % B)


def test_bf16_2pow26_8bit_blocksize4096(dev, po):
    """bf16, n = 2^26 (128 MiB), 8-bit codes, B = 4096: every absmax, code byte and
    dequantized element against the oracle."""
    n, B = 67108864, 4096
    t256 = synth.table256()
    x = synth.blockwise_input(n, "bfloat16", 3, std=0.02, device=dev)
    absmax, packed = gpu_quantize(x, "bfloat16", B, t256)
    out = gpu_dequantize(packed, absmax, n, "bfloat16", B, t256)
    xb = host_bits(x)
    what = "bf16 2^26 8-bit B=4096"
    oa, op = po.quantize_blockwise(xb, oracle.BF16, B, t256)
    assert_f32_bits_equal(absmax.cpu().numpy()[:oa.size], oa, what + " absmax")
    assert_bytes_equal(packed.cpu().numpy()[:op.size], op, what + " codes")
    ref = po.dequantize_blockwise(op, oa, n, oracle.BF16, B, t256)
    assert_bytes_equal(host_bits(out)[:n], ref, what + " dequant")


# ---- 8-bit codes, several tiles per workgroup ----------------------------------------------

# 3,075 tiles of 8192 elements, the last one partial: several times more workgroups than the
# device holds at once, with 8-bit codes.
N_MANY = 3 * (1 << 23) + 3 * 8192 + 77


@pytest.mark.parametrize("dtype,B", [("bfloat16", 4096), ("float32", 64), ("float16", 256), ("float16", 2048)])
def test_8bit_several_tiles_per_workgroup(dev, po, dtype, B):
    n = N_MANY
    t256 = synth.table256()
    x = synth.blockwise_input(n, dtype, 41, std=0.02, p_out=1e-4, p_nf=1e-5, device=dev)
    absmax, packed = gpu_quantize(x, dtype, B, t256)
    out = gpu_dequantize(packed, absmax, n, dtype, B, t256)
    xb = host_bits(x)
    what = "8-bit %s n=%d B=%d" % (dtype, n, B)
    oa, op = po.quantize_blockwise(xb, ORACLE_DT[dtype], B, t256)
    assert_f32_bits_equal(absmax.cpu().numpy()[:oa.size], oa, what + " absmax")
    assert_bytes_equal(packed.cpu().numpy()[:op.size], op, what + " codes")
    ref = po.dequantize_blockwise(op, oa, n, ORACLE_DT[dtype], B, t256)
    assert_out_equal(out, ref, n, dtype, what + " dequant")


def test_8bit_nested_several_tiles_per_workgroup(dev, po):
    """The nested statistics over 8-bit data codes at N_MANY elements, every output in full."""
    n, B, B2 = N_MANY, 64, 256
    t256 = synth.table256()
    x = synth.blockwise_input(n, "bfloat16", 43, std=0.02, p_out=1e-4, p_nf=1e-5, device=dev)
    r = gpu_nested(x, "bfloat16", B, t256, t256, B2)
    check_nested_full(po, r, host_bits(x), "bfloat16", n, B, t256, t256, B2, "nested 8-bit bf16 n=%d" % n)


def check_nested_full(po, r, xb, dtype, n, B, t_data, t_stats, B2, what):
    """Every output of a nested quantize + dequantize on the GPU against the oracle."""
    ref = po.quantize_nested(xb, ORACLE_DT[dtype], B, t_data, t_stats, B2)
    assert_f32_bits_equal(r["absmax"].cpu().numpy(), ref["absmax"], what + " absmax")
    assert np.float32(r["mean"].item()).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), what + " mean"
    assert_bytes_equal(r["q2"].cpu().numpy(), ref["q2"], what + " q2")
    assert_f32_bits_equal(r["absmax2"].cpu().numpy(), ref["absmax2"], what + " absmax2")
    assert_bytes_equal(r["packed"].cpu().numpy()[:ref["packed"].size], ref["packed"], what + " packed")
    out_ref = po.dequantize_nested(ref["packed"], ref["q2"], ref["absmax2"], ref["mean"], n, ORACLE_DT[dtype], B,
                                   t_data, t_stats, B2)
    assert_out_equal(r["out"], out_ref, n, dtype, what + " dequant")


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_q32_partial_tile_and_offset(dev, o, fmt):
    """Whole tiles (128 blocks) go through LDS with 16-byte loads; a partial last tile and a block
    array that is not 16-byte aligned (it starts one 18- or 34-byte block into a buffer) take
    the 2-byte-load path.  Both must give the same values."""
    bs = 18 if fmt == "q4" else 34
    f = bq.BQ_Q32_Q4 if fmt == "q4" else bq.BQ_Q32_Q8
    of = oracle.Q4 if fmt == "q4" else oracle.Q8
    nblk = 256 * 5 + 77
    buf = synth.q32_blocks(nblk + 1, fmt, seed=9, device=dev)
    for start in (0, 1):  # in blocks: the second view is only 2-byte aligned
        blocks = buf[start * bs:(start + nblk) * bs]
        n = nblk * 32
        for odt in ("bfloat16", "float32"):
            out = torch.empty(n, dtype=TORCH_DT[odt], device=dev)
            bq.check(bq.bq_dequant_q32(blocks, BQ_DT[odt], n, 32, f, out))
            ref = o.dequant_q32(blocks.cpu().numpy(), n, 32, of, ORACLE_DT[odt])
            assert_out_equal(out, ref, n, odt, "q32 %s start=%d %s" % (fmt, start, odt))


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_gguf_4096x14336(dev, o, fmt):
    rows, cols = 4096, 14336
    n = rows * cols
    blocks = synth.q32_blocks(n // 32, fmt, seed=4, device=dev)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    f = bq.BQ_Q32_Q4 if fmt == "q4" else bq.BQ_Q32_Q8
    bq.check(bq.bq_dequant_q32(blocks, bq.BQ_BF16, n, cols, f, out))
    ref = o.dequant_q32(blocks.cpu().numpy(), n, cols, oracle.Q4 if fmt == "q4" else oracle.Q8, oracle.BF16)
    assert_bytes_equal(host_bits(out), ref, "gguf 4096x14336 " + fmt)
    for odt in ("float32", "float16"):  # other output types on a slice of rows
        m = 64 * cols
        out2 = torch.empty(m, dtype=TORCH_DT[odt], device=dev)
        bq.check(bq.bq_dequant_q32(blocks, BQ_DT[odt], m, cols, f, out2))
        ref2 = o.dequant_q32(blocks[:m // 32 * (18 if fmt == "q4" else 34)].cpu().numpy(), m, cols,
                             oracle.Q4 if fmt == "q4" else oracle.Q8, ORACLE_DT[odt])
        assert_out_equal(out2, ref2, m, odt, "gguf 4096x14336 %s -> %s" % (fmt, odt))


def test_bf16_2pow29_4bit_nested(dev, po):
    """bf16, n = 2^29 (1 GiB), 4-bit codes, B = 64, nested statistics in groups of 256: every
    absmax, code byte, q2, absmax2, the mean and every dequantized element against the oracle."""
    n, B, B2 = 536870912, 64, 256
    t16, t256 = synth.table16(), synth.table256()
    x = synth.blockwise_input(n, "bfloat16", 5, std=0.02, device=dev)
    r = gpu_nested(x, "bfloat16", B, t16, t256, B2)
    _sync()
    xb = host_bits(x)
    del x
    check_nested_full(po, r, xb, "bfloat16", n, B, t16, t256, B2, "bf16 2^29 nested")


# ---- GGUF blocks with special scales, and a table with a -0.0 entry ----------------------

@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_q32_special_scales(dev, o, fmt):
    """Blocks whose fp16 scale is NaN (either sign), +-Inf, +-0, negative, subnormal or the
    largest finite value, in whole and partial tiles, against the oracle.  A NaN result is
    compared as a NaN (its sign and payload are not defined by IEEE 754 for 0 * Inf, and a NaN
    scale's sign may be dropped by the multiply); every other element bit for bit."""
    bs = 18 if fmt == "q4" else 34
    f = bq.BQ_Q32_Q4 if fmt == "q4" else bq.BQ_Q32_Q8
    of = oracle.Q4 if fmt == "q4" else oracle.Q8
    nblk = 128 * 3 + 21
    blocks = synth.q32_blocks(nblk, fmt, seed=12).cpu().numpy().copy()
    scales = [0x7E00, 0xFE00, 0x7C01, 0x7C00, 0xFC00, 0x0000, 0x8000, 0xBC00, 0x8001, 0x0001, 0x7BFF, 0xFBFF,
              0xC500, 0x83FF]
    rng = np.random.default_rng(3)
    for b in range(nblk):  # every fourth block takes a special scale, the rest random signs
        d = scales[(b // 4) % len(scales)] if b % 4 == 0 else int(blocks[b * bs]) | (int(blocks[b * bs + 1]) << 8)
        if b % 4 == 2:
            d |= 0x8000 * int(rng.integers(0, 2))
        blocks[b * bs] = d & 0xFF
        blocks[b * bs + 1] = d >> 8
    if fmt == "q4":  # make sure q - 8 == 0 meets an infinite scale: byte 0x88 in some blocks
        blocks[np.arange(0, nblk, 4) * bs + 2] = 0x88
    dblk = torch.tensor(blocks, device=dev)
    n = nblk * 32
    for odt in DTYPES:
        out = torch.empty(n, dtype=TORCH_DT[odt], device=dev)
        bq.check(bq.bq_dequant_q32(dblk, BQ_DT[odt], n, 32, f, out))
        ref = o.dequant_q32(blocks, n, 32, of, ORACLE_DT[odt])
        got = host_bits(out)[:n]
        what = "q32 %s special scales -> %s" % (fmt, odt)
        if odt == "float32":
            assert_f32_bits_equal(got, ref, what)
        else:
            exp_mask = 0x7F80 if odt == "bfloat16" else 0x7C00
            g_nan = ((got & exp_mask) == exp_mask) & ((got & ~np.uint16(0x8000 | exp_mask)) != 0)
            r_nan = ((ref & exp_mask) == exp_mask) & ((ref & ~np.uint16(0x8000 | exp_mask)) != 0)
            assert np.array_equal(g_nan, r_nan), what + ": NaN positions differ"
            assert_bytes_equal(got[~r_nan], ref[~r_nan], what)


def test_negative_zero_table_entry(dev, o):
    """A table whose zero entry is written as -0.0 quantizes and dequantizes exactly like the
    oracle, which reads it as +0.0: zero blocks and elements near zero dequantize to +0.0."""
    base = synth.table16().copy()
    t = base.copy()
    t[base == 0] = np.float32(-0.0)
    assert np.signbit(t[base == 0]).all()
    x = synth.blockwise_input(3 * 8192 + 77, "bfloat16", 19, std=1.0, p_out=0.01, p_nf=0.001, device=dev)
    x[:4096] = 0  # zero blocks
    x[8192:8192 + 64:2] = 0
    for B in (32, 64, 4096):
        absmax, packed = check_blockwise(o, x, "bfloat16", B, t, "-0.0 entry B=%d" % B, out_dtypes=DTYPES)
        out = gpu_dequantize(packed, absmax, x.numel(), "float32", B, t)
        assert not np.signbit(out[:4096].cpu().numpy()).any(), "a zero block dequantized to -0.0"
    z = torch.zeros(8192 * 2, dtype=torch.float32, device=dev)
    check_blockwise(o, z, "float32", 64, synth.dyadic_table(256), "zeros, dyadic 256 table")
    d = synth.dyadic_table(256).copy()
    d[128] = np.float32(-0.0)
    check_blockwise(o, z, "float32", 64, d, "zeros, dyadic 256 table with -0.0", out_dtypes=DTYPES)


def test_data_kernel_timing_hook(dev, o):
    """Events armed with bq_debug_time_next_kernel bracket the data kernel of the next nested
    quantize only (a positive elapsed time, shorter than the whole call), are forgotten after
    it, and leave the outputs unchanged; a start armed on one call and a stop on the next span
    both calls' armed kernels."""
    n, B = 1 << 22, 64
    t16, t256 = synth.table16(), synth.table256()
    x = synth.blockwise_input(n, "bfloat16", 17, std=0.02, device=dev)
    r0 = gpu_nested(x, "bfloat16", B, t16, t256)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bq.check(bq.bq_debug_time_next_kernel(e0, e1))
    c0.record()
    r1 = gpu_nested(x, "bfloat16", B, t16, t256)
    c1.record()
    torch.cuda.synchronize()
    k_ms, call_ms = e0.elapsed_time(e1), c0.elapsed_time(c1)
    assert 0 < k_ms < call_ms, (k_ms, call_ms)
    for k in ("absmax", "q2", "absmax2", "packed", "out"):
        assert torch.equal(r0[k].view(torch.uint8), r1[k].view(torch.uint8)), k
    # disarmed after one use: a later call records nothing into the events
    e1.record()
    torch.cuda.synchronize()
    gpu_nested(x, "bfloat16", B, t16, t256)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) >= k_ms
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bq.check(bq.bq_debug_time_next_kernel(s0, None))
    gpu_nested(x, "bfloat16", B, t16, t256)
    bq.check(bq.bq_debug_time_next_kernel(None, s1))
    r2 = gpu_nested(x, "bfloat16", B, t16, t256)
    torch.cuda.synchronize()
    assert s0.elapsed_time(s1) > k_ms
    for k in ("absmax", "q2", "absmax2", "packed", "out"):
        assert torch.equal(r0[k].view(torch.uint8), r2[k].view(torch.uint8)), k
