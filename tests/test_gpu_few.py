"""The few-token streaming GEMM (TERNARY_PATH_FEW) against the oracle.

The kernel serves 1 <= M <= 32 with x shared in LDS by the eight 16-channel
blocks of a workgroup ([xxqk] m.xxqk.cn/news/593501 §4.3 for the layer); it is
held to the layer's bound |y - y_ref| <= 1e-3 * sum_k |x_k| s(n,k) + 1e-6 on
every output it writes, on row-major and tiled codes, with the same bits on
both layouts.  Shapes cover 8-, 16- and 32-token tiles, ragged channel blocks,
parts of unequal length, every K-part count (1, 2, 4) and the three scale
modes it takes (per channel, groups of 128 and 256).
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen
from oracle import layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def _run(tl, M, N, K, g, dtype, seed):
    import torch
    rng = np.random.default_rng(seed)
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, dtype)
    xd, sd = to_dev(x, _tdt(dtype)), to_dev(scale, torch.float16)
    pd = to_dev(packed, None)
    y_r = tl.linear(xd, pd, sd, g, path="few")
    y_t = tl.linear(xd, to_dev(layout.tile(packed, N, K), None), sd, g, path="few",
                    layout="tiled")
    torch.cuda.synchronize()
    return x, packed, scale, y_r, y_t


# (M, N, K, g, dtype): 8-token tiles (M <= 8, up to 4 K parts) and 16-token
# tiles (2 parts at these N), ragged N, K of 1 .. 74 slabs
CASES = [
    (1, 1000, 4096, -1, "bf16"),
    (2, 40, 256, -1, "bf16"),
    (3, 77, 1280, 128, "bf16"),
    (5, 130, 2048, 256, "fp16"),
    (8, 512, 4096, -1, "bf16"),
    (8, 33, 18944, -1, "bf16"),
    (8, 100, 4864, 128, "fp16"),
    (9, 200, 2048, -1, "bf16"),
    (12, 61, 1024, 128, "bf16"),
    (16, 1024, 5120, 128, "bf16"),
    (16, 96, 1024, -1, "fp16"),
    (16, 50, 7936, 256, "bf16"),
    # groups of 128, whose scales come a round of four slabs at a time: K
    # ranges that end inside a round (the last round's DMA starts early),
    # one block split over K parts and slices
    (10, 40, 1792, 128, "fp16"),
    (16, 16, 6400, 128, "bf16"),
    (4, 23, 25600, 128, "bf16"),
    # 32-token tiles (one K part; per channel and groups of 256): ragged M
    # and N, a K long enough to slice over workgroups
    (17, 300, 2048, -1, "bf16"),
    (24, 130, 4096, 256, "fp16"),
    (31, 1000, 1024, -1, "fp16"),
    (32, 64, 18944, -1, "bf16"),
    (32, 520, 5120, 256, "bf16"),
]


@pytest.mark.parametrize("M,N,K,g,dtype", CASES)
def test_few_matches_oracle(tl, M, N, K, g, dtype):
    say(f"few M={M} N={N} K={K} g={g} {dtype}")
    x, packed, scale, y_r, y_t = _run(tl, M, N, K, g, dtype, M * 7919 + N * 31 + K + g)
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    check_within(widen(bits_of(y_r), dtype), y_ref, bound, f"few rows M={M} N={N} K={K} g={g}")
    assert np.array_equal(bits_of(y_r), bits_of(y_t)), "tiled and row-major codes differ"


@pytest.mark.parametrize("M,g", [(8, -1), (16, 128)])
def test_few_one_part(tl, M, g):
    # enough channel blocks that each workgroup holds 8 blocks of one part
    # (K long enough that rounding y to bf16 stays inside the bound)
    say(f"few one part M={M} g={g}")
    N, K = 40960, 1024
    x, packed, scale, y_r, y_t = _run(tl, M, N, K, g, "bf16", 11 + M)
    y_ref, bound = oracle.linear(x, packed, scale, g)
    check_within(widen(bits_of(y_r), "bf16"), y_ref, bound, "few one part")
    assert np.array_equal(bits_of(y_r), bits_of(y_t))


def test_few_reserved_codes_read_as_zero(tl):
    import torch
    say("few reserved codes")
    rng = np.random.default_rng(5)
    M, N, K = 6, 64, 1024
    packed = synth.draw_bytes(rng, N, K)              # includes code 11
    assert oracle.count_reserved(packed) > 0
    scale = synth.draw_scales(rng, N, K, 128)
    x = synth.draw_x(rng, M, K)
    y = tl.linear(to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16),
                  128, path="few")
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, 128)
    check_within(widen(bits_of(y), "bf16"), y_ref, bound, "few reserved")


@pytest.mark.parametrize("si", [0, 1])
def test_few_27b_shapes_sampled(tl, si):
    # the 27B group-128 projections at 16 tokens: every token of 64 sampled
    # channels against the oracle, and tiled == row-major on all outputs
    import torch
    case = synth.make_case(4, si, 16)
    N, K = case.codes.shape
    say(f"few 27B {case.shape.name} M=16")
    pd = tl.pack(to_dev(case.codes, None))
    xd, sd = to_dev(case.x, torch.bfloat16), to_dev(case.scale, torch.float16)
    y_r = tl.linear(xd, pd, sd, 128, path="few")
    y_t = tl.linear(xd, tl.tile(pd), sd, 128, path="few", layout="tiled")
    torch.cuda.synchronize()
    assert torch.equal(y_r.view(torch.int16), y_t.view(torch.int16))
    rows = np.sort(np.random.default_rng(si).choice(N, size=64, replace=False))
    packed, _ = oracle.pack(case.codes[rows])
    y_ref, bound = oracle.linear(case.x, packed, case.scale[rows], 128)
    check_within(widen(bits_of(y_r), "bf16")[:, rows], y_ref, bound, f"few 27B {case.shape.name}")
