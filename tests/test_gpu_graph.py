"""ternary_linear captured in a HIP graph: every replay equals the eager result.

Replays are interleaved with other eager work and synchronisations, and each
replay's outputs are compared bit-exactly with the eager outputs (the kernels
are deterministic and record no memset nodes).  A stream is warmed up (one
eager call per shape) before capturing on it: a split-K GEMM's workspace is
allocated then, and capturing on a stream that never ran the call reports
TERNARY_ERR_WORKSPACE instead of allocating.  A workspace replaced by a larger
one stays allocated, so a graph captured before the replacement still replays
correctly.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


def test_graph_replays_match_eager(tl):
    import torch
    say("graph capture of GEMV (per-channel, grouped), few-token GEMM and GEMM launches")
    rng = np.random.default_rng(31)
    specs = [(1, 1000, 4096, -1), (4, 700, 2048, 128), (96, 300, 1024, 128), (1, 64, 132, -1),
             (16, 640, 4096, -1), (12, 320, 8192, 128)]
    cases = []
    for M, N, K, g in specs:
        codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
        packed, _ = oracle.pack(codes)
        scale = synth.draw_scales(rng, N, K, g)
        x = synth.draw_x(rng, M, K)
        dev = (to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16), g)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        cases.append((x, packed, scale, g, dev, out))
    eager = []
    for x, packed, scale, g, (xd, pd, sd, _), out in cases:
        y = tl.linear(xd, pd, sd, g)
        torch.cuda.synchronize()
        y_ref, bound = oracle.linear(x, packed, scale, g)
        check_within(widen(bits_of(y), "bf16"), y_ref, bound, "eager before capture",
                     out_rounding="bf16" if x.shape[1] < 256 else None)
        eager.append(y)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):  # warm-up on the capture stream (its split-K workspace)
        for _, _, _, g, (xd, pd, sd, _), out in cases:
            tl.linear(xd, pd, sd, g, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _, _, _, g, (xd, pd, sd, _), out in cases:
            tl.linear(xd, pd, sd, g, out=out)

    other_x = torch.randn(8, 4096, device="cuda:0").bfloat16()
    for rep in range(4):
        for _, _, _, _, _, out in cases:
            out.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (_, _, _, _, _, out) in enumerate(cases):
            assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), (rep, i)
        # eager work between replays, on the same stream
        xd, pd, sd, g = cases[0][4]
        tl.linear(other_x[:1], pd, sd, g)
        tl.linear(other_x, pd, sd, g)
        torch.cuda.synchronize()


def _split_case(rng, M, N, K):
    import torch
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, -1)
    x = synth.draw_x(rng, M, K)
    return (x, packed, scale), (to_dev(x, torch.bfloat16), to_dev(packed, None),
                                to_dev(scale, torch.float16))


def test_capture_on_cold_stream_reports_workspace(tl):
    # a split-K GEMM (32 tiles, K split 8 ways) captured on a stream that never
    # ran it: nothing may be allocated under capture, so the call reports
    # TERNARY_ERR_WORKSPACE and records no launch
    import torch
    say("capture of a split-K GEMM on a cold stream")
    _, (xd, pd, sd) = _split_case(np.random.default_rng(5), 2048, 512, 4096)
    cold = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(graph, stream=cold):
        try:
            tl.linear(xd, pd, sd, -1)
        except tl.TernaryError as e:
            status = e.status
    assert status == -9
    del graph


def test_graph_survives_workspace_regrow(tl):
    # capture a split-K call after warming its stream, then grow the stream's
    # workspace with a larger split-K call: the graph keeps the buffer it was
    # captured with (retired, not freed), so every replay still equals eager
    import torch
    say("graph replay after the workspace grows")
    rng = np.random.default_rng(6)
    (x, packed, scale), (xd, pd, sd) = _split_case(rng, 256, 512, 2048)      # 2 MB of partials
    _, (xd2, pd2, sd2) = _split_case(rng, 2048, 512, 4096)                   # 32 MB
    side = torch.cuda.Stream()
    out = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda:0")
    with torch.cuda.stream(side):
        eager = tl.linear(xd, pd, sd, -1)
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, -1)
    check_within(widen(bits_of(eager), "bf16"), y_ref, bound, "eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        tl.linear(xd, pd, sd, -1, out=out)
    for rep in range(3):
        with torch.cuda.stream(side):
            tl.linear(xd2, pd2, sd2, -1)   # grows the workspace on the first pass
        torch.cuda.synchronize()
        out.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
    del graph
