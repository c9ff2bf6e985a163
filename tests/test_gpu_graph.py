"""The C ABI under HIP graph capture and on a two-stream copy/quantize pipeline.

Every call enqueues kernels only (no allocation, no host synchronization, no per-call
host-to-device copy), so a sequence of calls can be captured once and replayed ("Respect the
current CUDA stream in blockwise quantization", bitsandbytes PR 2052, Limitations: its graph
capture failed on a per-call code-map copy).  Each replay is checked bit for bit against the
eager results, with eager work and synchronizations between replays.
"""
import numpy as np
import pytest
import torch

import dequantization_block_absmax_amd as bq
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def test_graph_replay_matches_eager(dev):
    n, B, B2 = (1 << 22) + 4099, 64, 256
    t16, t256 = bq.code_table(synth.table16()), bq.code_table(synth.table256())
    x = synth.blockwise_input(n, "bfloat16", 41, std=0.02, p_out=1e-3, p_nf=1e-4, device=dev)
    nb = bq.num_blocks(n, B)
    ng = bq.num_blocks(nb, B2)
    rows, cols = 64, 14336
    m = rows * cols
    q4 = synth.q32_blocks(m // 32, "q4", seed=42, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(43)
    Ml, Kl, Nl = 3, 4096, 1000  # fused linear: seeded codes and block maxima of a 1000 x 4096 weight
    wpk = torch.randint(0, 256, (Nl * Kl // 2,), dtype=torch.uint8, device=dev, generator=gen)
    wam = 0.01 + 0.02 * torch.rand(Nl * Kl // B, device=dev, generator=gen)
    xl = torch.randn(Ml, Kl, device=dev, generator=gen).to(torch.bfloat16)
    Mg = 40  # fused GEMM on the same weight
    xg = torch.randn(Mg, Kl, device=dev, generator=gen).to(torch.bfloat16)

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
                    yg=torch.zeros(Mg, Nl, dtype=torch.float32, device=dev))

    def run(b, stream=None):
        st = bq.nested_stats(b["q2"], b["a2"], b["mean"], t256, B2, b["ws"])
        bq.check(bq.bq_quantize_nested(x, bq.BQ_BF16, n, B, t16, st, b["packed"], stream), "quantize_nested")
        bq.check(bq.bq_dequantize_nested(b["out"], bq.BQ_BF16, n, B, t16, st, b["packed"], stream),
                 "dequantize_nested")
        bq.check(bq.bq_dequant_q32(q4, bq.BQ_BF16, m, cols, bq.BQ_Q32_Q4, b["out4"], stream), "dequant_q32")
        bq.check(bq.bq_linear_blockwise(xl, bq.BQ_BF16, Ml, Kl, Nl, B, t16, wam, wpk, b["y"], stream), "linear")
        bq.check(bq.bq_gemm_blockwise(xg, bq.BQ_BF16, Mg, Kl, Nl, B, t16, wam, wpk, b["yg"], stream), "gemm")

    eager = buffers()
    run(eager)
    torch.cuda.synchronize()
    keys = ("packed", "q2", "a2", "mean", "out", "out4", "y", "yg")
    want = {k: eager[k].clone() for k in keys}

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
        for k in keys:  # clear the outputs eagerly between replays
            g[k].zero_()
        run(eager)      # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(g[k].view(torch.uint8), want[k].view(torch.uint8)), (replay, k)


def test_two_stream_copy_quantize_pipeline(dev):
    """Host chunks are copied on one stream (pinned memory) while the previous chunk is
    quantized on another; events order each quantize after its copy.  The result equals one
    quantize call per chunk on the default stream."""
    chunk, nchunks, B = 1 << 22, 6, 256
    t16 = bq.code_table(synth.table16())
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
    full = host.to(dev).view(torch.float16)
    for c in range(nchunks):
        a = torch.empty(nb, dtype=torch.float32, device=dev)
        p = torch.empty(chunk // 2, dtype=torch.uint8, device=dev)
        bq.check(bq.bq_quantize_blockwise(full[c * chunk:(c + 1) * chunk], bq.BQ_F16, chunk, B, t16, a, p))
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), absmax[c].view(torch.int32)), c
        assert torch.equal(p, packed[c]), c
