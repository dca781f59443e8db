"""ternary_linear captured in a HIP graph: every replay equals the eager result.

Replays are interleaved with other eager work and synchronisations, and each
replay's outputs are compared bit-exactly with the eager outputs (the kernels
are deterministic and record no memset nodes).
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
    say("graph capture of GEMV (per-channel, grouped) and GEMM launches")
    rng = np.random.default_rng(31)
    specs = [(1, 1000, 4096, -1), (4, 700, 2048, 128), (96, 300, 1024, 128), (1, 64, 132, -1)]
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

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
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
