"""The C ABI under HIP graph capture and on a two-stream copy/quantize pipeline, against the
oracle.

Every call enqueues kernels only (no allocation, no host synchronization, no per-call
host-to-device copy), so a sequence of calls can be captured once and replayed ("Respect the
current CUDA stream in blockwise quantization", bitsandbytes PR 2052, Limitations: its graph
capture failed on a per-call code-map copy).  Each replay is compared with the oracle (bit
for bit for quantize / dequantize / GGUF outputs, within the stated bound for the fused
linear and GEMM, which must also repeat the eager bits), with eager work and
synchronizations between replays.  The pipeline's outputs are compared with the oracle run
over the whole host array.
"""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import oracle
import synth
from gpu_helpers import (assert_bytes_equal, assert_f32_bits_equal, check_gemm_against_oracle,
                         check_linear_against_oracle, host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def po():
    return oracle.ParallelOracle()


def test_graph_replay_matches_oracle(dev, po):
    n, B, B2 = (1 << 22) + 4099, 64, 256
    t16_np, t256_np = synth.table16(), synth.table256()
    t16, t256 = bq.code_table(t16_np), bq.code_table(t256_np)
    x = synth.blockwise_input(n, "bfloat16", 41, std=0.02, p_out=1e-3, p_nf=1e-4, device=dev)
    nb = bq.num_blocks(n, B)
    ng = bq.num_blocks(nb, B2)
    rows, cols = 64, 14336
    m = rows * cols
    q4 = synth.q32_blocks(m // 32, "q4", seed=42, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(43)
    # fused linear: seeded codes and block maxima of an 8200 x 4096 weight, tall enough for the
    # matrix-core form at three rows (32 rows per CU on MI355X)
    Ml, Kl, Nl = 3, 4096, 8200
    wpk = torch.randint(0, 256, (Nl * Kl // 2,), dtype=torch.uint8, device=dev, generator=gen)
    wam = 0.01 + 0.02 * torch.rand(Nl * Kl // B, device=dev, generator=gen)
    xl = torch.randn(Ml, Kl, device=dev, generator=gen).to(torch.bfloat16)
    Mg, Ng = 40, 1000  # fused GEMM on the first 1000 rows of that weight
    xg = torch.randn(Mg, Kl, device=dev, generator=gen).to(torch.bfloat16)
    # fused GEMM in its 256 x 256 tile form: 8-bit codes, 1024 x 12288 outputs (4 x 48 tiles), K = 128
    Mw, Kw, Nw = 1024, 128, 12288
    wpk8 = torch.randint(0, 256, (Nw * Kw,), dtype=torch.uint8, device=dev, generator=gen)
    wam8 = 0.01 + 0.02 * torch.rand(Nw * Kw // B, device=dev, generator=gen)
    xw = torch.randn(Mw, Kw, device=dev, generator=gen).to(torch.bfloat16)
    wrows = np.unique(np.concatenate([[0, 127, 128, 255, 256, Nw - 1], np.random.default_rng(44).integers(0, Nw, 12)]))

    # the oracle's outputs for the same inputs
    xb = host_bits(x)
    ref = po.quantize_nested(xb, oracle.BF16, B, t16_np, t256_np, B2)
    ref_out = po.dequantize_nested(ref["packed"], ref["q2"], ref["absmax2"], ref["mean"], n, oracle.BF16, B, t16_np,
                                   t256_np, B2)
    ref_out4 = po.dequant_q32(q4.cpu().numpy(), m, cols, oracle.Q4, oracle.BF16)
    wpk_h, wam_h = wpk.cpu().numpy(), wam.cpu().numpy()
    wpk8_h, wam8_h = wpk8.cpu().numpy(), wam8.cpu().numpy()
    wpk8_rows = np.concatenate([wpk8_h[r * Kw:(r + 1) * Kw] for r in wrows])
    wam8_rows = np.concatenate([wam8_h[r * (Kw // B):(r + 1) * (Kw // B)] for r in wrows])

    def buffers():
        ws_bytes = bq.bq_nested_workspace_bytes(n, B, B2)
        return dict(packed=torch.zeros(bq.packed_bytes(n, 16), dtype=torch.uint8, device=dev),
                    q2=torch.zeros(nb, dtype=torch.uint8, device=dev),
                    a2=torch.zeros(ng, dtype=torch.float32, device=dev),
                    mean=torch.zeros(1, dtype=torch.float32, device=dev),
                    ws=torch.zeros(ws_bytes, dtype=torch.uint8, device=dev),
                    out=torch.zeros(n, dtype=torch.bfloat16, device=dev),
                    out4=torch.zeros(m, dtype=torch.bfloat16, device=dev),
                    y=torch.zeros(Ml, Nl, dtype=torch.float32, device=dev),
                    yg=torch.zeros(Mg, Ng, dtype=torch.float32, device=dev),
                    yw=torch.zeros(Mw, Nw, dtype=torch.float32, device=dev))

    def run(b, stream=None):
        st = bq.nested_stats(b["q2"], b["a2"], b["mean"], t256, B2, b["ws"])
        bq.check(bq.bq_quantize_nested(x, bq.BQ_BF16, n, B, t16, st, b["packed"], stream), "quantize_nested")
        bq.check(bq.bq_dequantize_nested(b["out"], bq.BQ_BF16, n, B, t16, st, b["packed"], stream),
                 "dequantize_nested")
        bq.check(bq.bq_dequant_q32(q4, bq.BQ_BF16, m, cols, bq.BQ_Q32_Q4, b["out4"], stream), "dequant_q32")
        bq.check(bq.bq_linear_blockwise(xl, bq.BQ_BF16, Ml, Kl, Nl, B, t16, wam, wpk, b["y"], stream), "linear")
        bq.check(bq.bq_gemm_blockwise(xg, bq.BQ_BF16, Mg, Kl, Ng, B, t16, wam, wpk, b["yg"], stream), "gemm")
        bq.check(bq.bq_gemm_blockwise(xw, bq.BQ_BF16, Mw, Kw, Nw, B, t256, wam8, wpk8, b["yw"], stream), "gemm wide")

    def check_against_oracle(b, what):
        assert_bytes_equal(b["packed"].cpu().numpy(), ref["packed"], what + " packed")
        assert_bytes_equal(b["q2"].cpu().numpy(), ref["q2"], what + " q2")
        assert_f32_bits_equal(b["a2"].cpu().numpy(), ref["absmax2"], what + " absmax2")
        assert_f32_bits_equal(b["mean"].cpu().numpy(), np.float32([ref["mean"]]), what + " mean")
        assert_bytes_equal(host_bits(b["out"]), ref_out, what + " nested dequant")
        assert_bytes_equal(host_bits(b["out4"]), ref_out4, what + " q32")
        check_linear_against_oracle(po, b["y"].cpu().numpy(), xl.cpu(), "bfloat16", Nl, B, t16_np, wam_h, wpk_h,
                                    what + " linear")
        check_gemm_against_oracle(po, b["yg"].cpu().numpy(), xg.cpu(), "bfloat16", Ng, B, t16_np,
                                  wam_h[:Ng * Kl // B], wpk_h[:Ng * Kl // 2], what + " gemm")
        check_gemm_against_oracle(po, b["yw"].cpu().numpy()[:, wrows], xw.cpu(), "bfloat16", len(wrows), B, t256_np,
                                  wam8_rows, wpk8_rows, what + " gemm wide (sampled rows)")

    eager = buffers()
    run(eager)
    torch.cuda.synchronize()
    check_against_oracle(eager, "eager")
    y_eager, yg_eager, yw_eager = eager["y"].clone(), eager["yg"].clone(), eager["yw"].clone()

    g = buffers()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(g)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(g)  # calls pick up torch's current (capturing) stream
    for replay in range(4):
        for k in g:  # clear the outputs eagerly between replays
            g[k].zero_()
        run(eager)   # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check_against_oracle(g, "replay %d" % replay)
        # the fused products are not unique, but every call gives the same bits
        assert torch.equal(g["y"].view(torch.int32), y_eager.view(torch.int32)), replay
        assert torch.equal(g["yg"].view(torch.int32), yg_eager.view(torch.int32)), replay
        assert torch.equal(g["yw"].view(torch.int32), yw_eager.view(torch.int32)), replay


def test_two_stream_copy_quantize_pipeline(dev, po):
    """Host chunks are copied on one stream (pinned memory) while the previous chunk is
    quantized on another; events order each quantize after its copy.  Every absmax and code
    byte equals the oracle's over the whole host array."""
    chunk, nchunks, B = 1 << 22, 6, 256
    t16_np = synth.table16()
    t16 = bq.code_table(t16_np)
    host = synth.blockwise_input(chunk * nchunks, "float16", 43, std=1.0, p_out=1e-3).view(torch.int16)
    host = host.pin_memory()
    dev_in = [torch.empty(chunk, dtype=torch.int16, device=dev) for _ in range(2)]
    nb = chunk // B
    absmax = torch.empty(nchunks, nb, dtype=torch.float32, device=dev)
    packed = torch.empty(nchunks, chunk // 2, dtype=torch.uint8, device=dev)
    copy_s, work_s = torch.cuda.Stream(), torch.cuda.Stream()
    copied = [torch.cuda.Event() for _ in range(nchunks)]
    used = [torch.cuda.Event() for _ in range(nchunks)]
    for c in range(nchunks):
        buf = dev_in[c % 2]
        if c >= 2:
            copy_s.wait_event(used[c - 2])  # the buffer's previous chunk is quantized
        with torch.cuda.stream(copy_s):
            buf.copy_(host[c * chunk:(c + 1) * chunk], non_blocking=True)
            copied[c].record(copy_s)
        work_s.wait_event(copied[c])
        bq.check(bq.bq_quantize_blockwise(buf, bq.BQ_F16, chunk, B, t16, absmax[c], packed[c], work_s))
        used[c].record(work_s)
    torch.cuda.synchronize()
    oa, op = po.quantize_blockwise(host.numpy().view(np.uint16), oracle.F16, B, t16_np)
    assert_f32_bits_equal(absmax.cpu().numpy().reshape(-1), oa, "pipeline absmax")
    assert_bytes_equal(packed.cpu().numpy().reshape(-1), op, "pipeline codes")
