"""bq_quantize_nested_noalloc (the library's own scratch memory in place of a caller workspace)
against bq_quantize_nested on the same inputs, bit for bit, on two calls in a row, the second
with a smaller input, so the second call runs on scratch that still holds the first call's
contents.  Both go through the C ABI."""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _outputs(dev, n, B, B2, K):
    nb = bq.num_blocks(n, B)
    return dict(q2=torch.full((nb,), 0xCD, dtype=torch.uint8, device=dev),
                a2=torch.full((bq.num_blocks(nb, B2),), float("nan"), dtype=torch.float32, device=dev),
                mean=torch.full((1,), float("nan"), dtype=torch.float32, device=dev),
                packed=torch.full((max(bq.packed_bytes(n, K), 16),), 0xAB, dtype=torch.uint8, device=dev))


def _run(fn, x, dtype, n, B, table, table2, B2, out, ws=None):
    stats = bq.nested_stats(out["q2"], out["a2"], out["mean"], table2, B2, ws)
    bq.check(fn(x, dtype, n, B, table, stats, out["packed"]), fn.__name__)


CASES = [  # (dtype, n, B, B2, table size): the second of each pair is smaller than the first
    [("bfloat16", (1 << 24) + 4099, 64, 256, 16), ("bfloat16", 3 * 8192 + 77, 64, 256, 16)],
    [("float32", (1 << 22) + 33, 32, 2048, 256), ("float16", 100_001, 4096, 32, 16)],
]


@pytest.mark.parametrize("pair", CASES, ids=["bf16_large_then_small", "f32_then_f16"])
def test_noalloc_matches_workspace_entry_point(dev, pair):
    t16, t256 = synth.table16(), synth.table256()
    for i, (dtype, n, B, B2, K) in enumerate(pair):
        tdt = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}[dtype]
        code = {"float32": bq.BQ_F32, "float16": bq.BQ_F16, "bfloat16": bq.BQ_BF16}[dtype]
        table = t16 if K == 16 else t256
        x = synth.blockwise_input(n, dtype, 70 + i, std=0.02, p_out=1e-3, p_nf=1e-4, device=dev).to(tdt)
        ws = torch.empty(bq.bq_nested_workspace_bytes(n, B, B2), dtype=torch.uint8, device=dev)
        want, got = _outputs(dev, n, B, B2, K), _outputs(dev, n, B, B2, K)
        _run(bq.bq_quantize_nested, x, code, n, B, table, t256, B2, want, ws)
        _run(bq.bq_quantize_nested_noalloc, x, code, n, B, table, t256, B2, got)
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(got[k].view(torch.uint8), want[k].view(torch.uint8)), (dtype, n, k)
        if n < 200_000:  # and the smaller case against the oracle too
            xb = x.cpu().view(torch.int16).numpy().view(np.uint16) if dtype != "float32" else x.cpu().numpy()
            ref = oracle.Oracle().quantize_nested(xb, {"float32": oracle.F32, "float16": oracle.F16,
                                                       "bfloat16": oracle.BF16}[dtype], B, table, t256, B2)
            assert np.array_equal(got["q2"].cpu().numpy(), ref["q2"])
            assert np.array_equal(got["a2"].cpu().numpy().view(np.uint32), ref["absmax2"].view(np.uint32))
            assert got["mean"].cpu().numpy().view(np.uint32)[0] == np.float32(ref["mean"]).view(np.uint32)
            assert np.array_equal(got["packed"].cpu().numpy()[:ref["packed"].size], ref["packed"])


def test_noalloc_refuses_inputs_beyond_its_scratch(dev):
    x = torch.empty(16, dtype=torch.bfloat16, device=dev)
    out = _outputs(dev, 1024, 64, 256, 16)
    stats = bq.nested_stats(out["q2"], out["a2"], out["mean"], synth.table256(), 256, None)
    # n = 2^30 would need a 70 MiB workspace; the check happens before anything is enqueued
    assert bq.bq_quantize_nested_noalloc(x, bq.BQ_BF16, 1 << 30, 64, synth.table16(), stats,
                                         out["packed"]) == bq.BQ_ERR_WORKSPACE
