"""ternary_linear_batch_noalloc (the allocation-free entry point) through the C
ABI, against ternary_linear_batch on the same inputs: the same bits, and both
within the stated bound of the oracle, |y - y_ref| <= 1e-3 * sum_k |x_k| s + 1e-6.

Two calls in a row, the second smaller (the static scratch keeps the first
call's partials; the second must not depend on them), a batch mixing decode,
few-token (K-sliced) and prefill problems, a grouped launch with a work-balanced
K split, a batch whose split-K partials exceed the static buffer (rejected
with nothing enqueued), and a capture on a stream that never ran the call (the
allocation-free call needs no warm-up).
"""

import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen

pytestmark = pytest.mark.gpu

SCRATCH_ERR = -10


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


def _problems(specs, seed):
    import torch
    rng = np.random.default_rng(seed)
    out = []
    for M, N, K, g in specs:
        packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
        scale = synth.draw_scales(rng, N, K, g)
        x = synth.draw_x(rng, M, K, "bf16")
        dev = (to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16))
        out.append((M, N, K, g, x, packed, scale, dev))
    return out


def _call(tl, probs, noalloc, stream=None):
    """One batch call through the C ABI; returns (status, outputs)."""
    import torch
    arr = (tl.Problem * len(probs))()
    outs = []
    for i, (M, N, K, g, _, _, _, (xd, pd, sd)) in enumerate(probs):
        y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda:0")
        outs.append(y)
        arr[i] = tl.Problem(xd.data_ptr(), pd.data_ptr(), sd.data_ptr(), y.data_ptr(), M, N, K, g)
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    fn = tl.lib().ternary_linear_batch_noalloc if noalloc else tl.lib().ternary_linear_batch
    st = fn(arr, len(probs), 0, ctypes.c_void_p(s))
    return st, outs


def _tile_samples(rng, M, N):
    ms, ns = [], []
    for m0 in range(0, M, 128):
        for n0 in range(0, N, 256):
            ms.append(rng.integers(m0, min(M, m0 + 128), 2))
            ns.append(rng.integers(n0, min(N, n0 + 256), 2))
    return np.concatenate(ms + [np.array([0, M - 1])]), np.concatenate(ns + [np.array([N - 1, 0])])


def _check(tl, probs, tag):
    import torch
    st_a, ya = _call(tl, probs, noalloc=False)
    st_b, yb = _call(tl, probs, noalloc=True)
    torch.cuda.synchronize()
    assert st_a == 0 and st_b == 0, (st_a, st_b)
    for i, ((M, N, K, g, x, packed, scale, _), a, b) in enumerate(zip(probs, ya, yb)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{tag} problem {i}: bits differ"
        yv = widen(bits_of(b), "bf16")
        if M * N * K <= (1 << 28):
            y_ref, bound = oracle.linear(x, packed, scale, g)
            check_within(yv, y_ref, bound, f"{tag} problem {i}")
        else:
            rng = np.random.default_rng(i)
            ms, ns = _tile_samples(rng, M, N)
            y_ref, bound = oracle.linear_at(x, packed, scale, g, ms, ns)
            check_within(yv[ms, ns], y_ref, bound, f"{tag} problem {i} (tile samples)")


def test_noalloc_two_calls_second_smaller(tl):
    # k-shaped problem at 2048 tokens: 32 output tiles, K split 8 ways (32 MB
    # of partials), then a 4-tile problem split 4 ways (2 MB)
    say("noalloc: split-K call, then a smaller one")
    _check(tl, _problems([(2048, 512, 4096, -1)], 1), "first")
    _check(tl, _problems([(256, 512, 2048, -1)], 2), "second")


def test_noalloc_mixed_batch(tl):
    say("noalloc: decode + grouped prefill + 128x128 GEMM + few-token GEMM in one batch")
    specs = [(1, 4096, 4096, -1), (1, 512, 4096, -1), (256, 300, 2048, 128), (100, 200, 1152, 128),
             (300, 260, 1024, -1), (16, 640, 4096, -1), (12, 320, 8192, 128)]
    _check(tl, _problems(specs, 3), "mixed")


def test_noalloc_balanced_split(tl):
    # the 7B-shaped layer at 32 tokens: one grouped launch whose down
    # projection's K range is sliced for balance (2.6 MB of partials, within
    # the static buffer): the same plan and bits as the allocating call
    say("noalloc: grouped launch with a work-balanced K split")
    specs = [(32, s.N, s.K, -1) for s in synth.CONFIGS[2].shapes]
    _check(tl, _problems(specs, 6), "balanced")


def test_noalloc_rejects_oversize(tl):
    # two problems whose 240 tiles split 2 and 3 ways need 74 MB of partials,
    # more than the static buffer: rejected, and nothing runs
    import torch
    say("noalloc: batch needing more scratch than the static buffer")
    probs = _problems([(2048, 2048, 2048, -1), (2048, 1792, 2048, -1)], 4)
    st, outs = _call(tl, probs, noalloc=True)
    torch.cuda.synchronize()
    assert st == SCRATCH_ERR
    for y in outs:
        assert torch.all(y == 7.0), "a rejected call wrote its output"


def test_noalloc_captures_without_warmup(tl):
    # a graph captured on a stream that never ran the call, replayed several
    # times with eager work in between: every replay equals the eager result
    import torch
    say("noalloc: capture on a fresh stream")
    probs = _problems([(2048, 512, 4096, -1), (1, 4096, 4096, -1), (16, 640, 4096, -1)], 5)
    st, eager = _call(tl, probs, noalloc=True)
    torch.cuda.synchronize()
    assert st == 0
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    arr = (tl.Problem * len(probs))()
    outs = []
    for i, (M, N, K, gs, _, _, _, (xd, pd, sd)) in enumerate(probs):
        y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda:0")
        outs.append(y)
        arr[i] = tl.Problem(xd.data_ptr(), pd.data_ptr(), sd.data_ptr(), y.data_ptr(), M, N, K, gs)
    with torch.cuda.graph(g, stream=side):
        st = tl.lib().ternary_linear_batch_noalloc(
            arr, len(probs), 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    for rep in range(3):
        for y in outs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        _call(tl, probs[:1], noalloc=False)   # other work on the GPU between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep} problem {i}"
