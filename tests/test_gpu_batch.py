"""ternary_linear_batch: one fused decode launch, or one grouped prefill
GEMM launch, for several projections.

Each output must lie within the bound of the oracle, and a batch must give
the same bits every time it runs.  Batched and single calls may differ in the
last bits (the batch plans its K split over all of its problems), so each is
checked against the oracle on its own.
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


def _problems(rng, specs, dtype="bf16"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    out = []
    for M, N, K, g in specs:
        codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
        packed, _ = oracle.pack(codes)
        scale = synth.draw_scales(rng, N, K, g)
        x = synth.draw_x(rng, M, K, dtype)
        out.append((x, packed, scale, g,
                    (to_dev(x, tdt), to_dev(packed, None), to_dev(scale, torch.float16), g)))
    return out


def _run_and_check(tl, probs, dtype="bf16", samples=None):
    import torch
    singles = [tl.linear(*d) for *_, d in probs]
    outs = tl.linear_batch([(d[0], d[1], d[2], d[3], None) for *_, d in probs])
    again = tl.linear_batch([(d[0], d[1], d[2], d[3], None) for *_, d in probs])
    torch.cuda.synchronize()
    for i, ((x, packed, scale, g, _), a, b, c) in enumerate(zip(probs, singles, outs, again)):
        assert torch.equal(b.view(torch.int16), c.view(torch.int16)), f"problem {i} not repeatable"
        yv = widen(bits_of(b), dtype)
        ya = widen(bits_of(a), dtype)
        if samples is None:
            y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
            rounding = dtype if x.shape[1] < 256 else None
            check_within(yv, y_ref, bound, f"batch problem {i}", out_rounding=rounding)
            check_within(ya, y_ref, bound, f"single problem {i}", out_rounding=rounding)
        else:
            rng = np.random.default_rng(i)
            M, N = yv.shape
            ms, ns = rng.integers(0, M, samples), rng.integers(0, N, samples)
            y_ref, bound = oracle.linear_at(x, packed, scale, g, ms, ns, dtype=dtype)
            check_within(yv[ms, ns], y_ref, bound, f"batch problem {i}")
            check_within(ya[ms, ns], y_ref, bound, f"single problem {i}")


@pytest.mark.parametrize("M", [1, 8, 16])
def test_batch_7b_decode_layer(tl, M):
    # every output of the fused decode launch (at 16 tokens: the fused
    # few-token GEMM launch, the down projection K-sliced) against the oracle
    say(f"batch of the 7 decode projections, M={M}")
    specs = [(M, s.N, s.K, -1) for s in synth.CONFIGS[2].shapes]
    _run_and_check(tl, _problems(np.random.default_rng(40 + M), specs))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_batch_mixed(tl, dtype):
    say(f"mixed batch (GEMV + GEMM + plain kernel) {dtype}")
    specs = [(1, 300, 1024, 128), (3, 65, 2304, -1), (8, 129, 9216, 128), (64, 100, 512, 128),
             (2, 40, 132, -1), (5, 1, 128, 128), (1, 2000, 640, -1)]
    _run_and_check(tl, _problems(np.random.default_rng(41), specs, dtype), dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_batch_few_token_mixed(tl, dtype):
    # 9 .. 32 tokens in one batch: three scale modes and two token tiles
    # (16 and 32: one few-token launch per pair present), a K-sliced problem, a group
    # size the few-token GEMM does not take and groups of 128 past 16 tokens
    # (GEMM)
    say(f"few-token batch {dtype}")
    specs = [(16, 640, 4096, -1), (12, 320, 8192, 128), (9, 1000, 1024, 128),
             (10, 200, 1024, 64), (24, 300, 2048, -1), (17, 520, 6144, -1),
             (32, 130, 4352, 256), (20, 100, 1024, 128)]
    _run_and_check(tl, _problems(np.random.default_rng(45), specs, dtype), dtype=dtype)


def test_batch_big_k_chunked(tl):
    say("batch with chunked activations (M=8, K=18944; M=4, K=25600)")
    specs = [(8, 200, 18944, -1), (4, 100, 25600, 128), (8, 64, 5120, 128)]
    _run_and_check(tl, _problems(np.random.default_rng(42), specs), samples=600)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_batch_grouped_prefill(tl, dtype):
    # Per-channel prefill problems of one grouped GEMM launch: 256 + 6 + 16 +
    # 15 + 9 tiles of 256 x 128, so no K range is split; different K, ragged M
    # and N, a problem that shares another's activations (as q/k/v do), plus a
    # group-scaled problem that runs on its own.
    import torch
    say(f"grouped prefill batch {dtype}")
    specs = [(2048, 4096, 512, -1), (300, 520, 1024, -1), (2048, 256, 256, -1),
             (300, 1100, 2048, -1), (256, 300, 512, 128)]
    rng = np.random.default_rng(43)
    probs = _problems(rng, specs, dtype)
    x1, d1 = probs[1][0], probs[1][4]
    codes = synth.draw_codes(rng, 700, 1024, 0.3, 0.3)
    packed, _ = oracle.pack(codes)
    scale = synth.draw_scales(rng, 700, 1024, -1)
    probs.append((x1, packed, scale, -1,
                  (d1[0], to_dev(packed, None), to_dev(scale, torch.float16), -1)))
    _run_and_check(tl, probs, dtype=dtype)


def test_batch_grouped_prefill_split(tl):
    # Small per-channel prefill problems (32 + 9 + 15 tiles): each problem
    # whose K allows it is split (its own partial tiles and reduce launch),
    # the K = 256 one is not.
    say("grouped prefill batch with split K")
    specs = [(512, 2048, 1024, -1), (300, 520, 4096, -1), (300, 1100, 2048, -1),
             (256, 300, 256, -1)]
    _run_and_check(tl, _problems(np.random.default_rng(44), specs))


def test_batch_rejects_alias_on_device(tl):
    import torch
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda:0")
    p = torch.zeros((16, 64), dtype=torch.uint8, device="cuda:0")
    s = torch.ones((16, 2), dtype=torch.float16, device="cuda:0")
    y = torch.empty((1, 16), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(tl.TernaryError) as e:
        tl.linear_batch([(x, p, s, 128, y), (x, p, s, 128, y)])
    assert e.value.status == -6


@pytest.mark.parametrize("cfg,M", [(2, 32), (4, 256)])
def test_batch_balanced_split(tl, cfg, M):
    # Grouped GEMM launches whose tiles cover the compute units but whose one
    # long-K problem runs far longer per tile than the rest: the 7B-shaped
    # layer at 32 tokens (368 tiles of K = 4096, 32 down tiles of K = 18944)
    # and the 27B-class group-128 pair at 256 tokens (up K = 5120, down
    # K = 25600).  The long problem's K range is sliced over workgroups and
    # reduced in slice order; 1500 sampled outputs per problem.
    c = synth.CONFIGS[cfg]
    say(f"balanced K slices in a grouped launch: {c.name}, M={M}")
    specs = [(M, s.N, s.K, c.group_size) for s in c.shapes]
    _run_and_check(tl, _problems(np.random.default_rng(46 + M), specs), samples=1500)
