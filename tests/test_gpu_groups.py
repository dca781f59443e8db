"""Group sizes other than 128 (32, 64, 256) on every kernel path, against the
CPU oracle, to the stated bound |y - y_ref| <= 1e-3 * sum_k |x_k| s(n,k) + 1e-6.

The pages meet checkpoints grouped by 64 (m.xxqk.cn/news/593501 §4.2, §5.2)
and list 32 and 256 beside the usual 128 (yangyitao.com vLLM book, chapter 13,
§13.3.3).  Each path gets its own cases: the streaming decode GEMV (M <= 2),
the M <= 8 GEMV (M * columns-per-token <= 16), the pipelined GEMM (groups of
64/128/256 with an even number of groups per row; small, mid and split-K
configurations), the 128x128 GEMM (every group size, K % 256 != 0 or an odd
number of groups per row), the plain kernel, and a batch that mixes group
sizes.
"""

import zlib

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


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def _case(M, N, K, g, dtype, raw=False, tag=""):
    rng = np.random.default_rng(zlib.crc32(repr((tag, M, N, K, g, dtype, raw)).encode()))
    if raw:
        packed = synth.draw_bytes(rng, N, K)
    else:
        packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, dtype)
    return packed, scale, x


DECODE_KERNELS = ["gemv_f4", "gemv_b16"]


def _check(tl, M, N, K, g, dtype="bf16", path="auto", expect=None, raw=False, tag=""):
    import torch
    what = f"{tag} M={M} N={N} K={K} g={g} {dtype} path={path} raw={raw}"
    say(what)
    if expect is not None:
        assert tl.select_path(M, N, K, g) == expect, what
    packed, scale, x = _case(M, N, K, g, dtype, raw, tag)
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    try:
        y = tl.linear(to_dev(x, _tdt(dtype)), to_dev(packed, None), to_dev(scale, torch.float16),
                      g, path=path)
    except tl.TernaryError as e:
        if e.status == -8 and path in DECODE_KERNELS:
            pytest.skip(f"{path} does not take {what}")
        raise
    torch.cuda.synchronize()
    check_within(widen(bits_of(y), dtype), y_ref, bound, what)


# streaming decode GEMV: M <= 2 (8, 4 or 2 columns per token)
STREAM = [
    (1, 100, 4096, 32), (2, 45, 2560, 32), (1, 33, 16384, 32), (2, 7, 1152, 32),
    (1, 100, 4096, 64), (2, 77, 6272, 64), (1, 40, 20480, 64), (1, 600, 3200, 64),
    (1, 100, 4096, 256), (2, 45, 10240, 256), (1, 48, 30720, 256), (2, 19, 5376, 256),
]


@pytest.mark.parametrize("path", ["auto", *DECODE_KERNELS])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,g", STREAM)
def test_groups_stream_gemv(tl, M, N, K, g, dtype, path):
    _check(tl, M, N, K, g, dtype, path=path, expect="gemv", tag="stream")


# M <= 8 GEMV beyond the streaming kernel (groups of 64 up to M = 4, of 256 up
# to M = 8), and the streaming kernel's longest parts (M <= 2, K up to 65536:
# 20 and 32 slabs per wave, run as one-shot chunks)
# (the fp4 x fp8 kernel also takes groups of 32 and 64 up to M = 8 with bf16
# activations, in two to four matrix passes)
GEMV = [(3, 257, 4096, 64), (4, 100, 1536, 64), (4, 33, 8192, 64),
        (3, 100, 2048, 256), (5, 64, 4096, 256), (8, 48, 5120, 256), (7, 1030, 1280, 256),
        (1, 40, 40960, 256), (2, 9, 65536, 256), (8, 70, 2048, 64), (6, 33, 4096, 32),
        (8, 100, 1024, 32), (8, 64, 3072, 128)]


@pytest.mark.parametrize("path", ["auto", *DECODE_KERNELS])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,g", GEMV)
def test_groups_small_m_gemv(tl, M, N, K, g, dtype, path):
    expect = "gemv" if tl.select_path(M, N, K, g) == "gemv" else None
    if path == "auto" and expect is None:
        pytest.skip("not a decode shape for both dtypes")
    _check(tl, M, N, K, g, dtype, path=path, expect=expect, tag="gemv")


# pipelined GEMM: few tokens (8-stage small configuration), mid, ragged M and
# N, and a long K whose few tiles split K (fp32 partials + reduce)
BIG = [(16, 300, 2048, 64), (16, 300, 2048, 256), (64, 257, 1536, 64), (64, 257, 1536, 256),
       (256, 300, 2048, 64), (256, 300, 2048, 256), (130, 129, 1024, 64),
       (200, 260, 3072, 256), (64, 256, 18944, 64), (40, 512, 8192, 256)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,g", BIG)
def test_groups_pipelined_gemm(tl, M, N, K, g, dtype):
    # the GEMM forced (up to 16 tokens for groups of 128, 32 for groups of
    # 256, the automatic path takes the few-token GEMM, which
    # tests/test_gpu_few.py covers)
    few_m = {128: 16, 256: 32}.get(g, 0)
    auto = "few" if M <= few_m and K % 256 == 0 else "gemm"
    assert tl.select_path(M, N, K, g) == auto
    _check(tl, M, N, K, g, dtype, path="gemm", tag="big")


# 128x128 GEMM: groups of 32 (every M > 2 that the GEMV does not take),
# K % 256 != 0, and an odd number of 256-groups per row
SQUARE = [(9, 100, 256, 32), (130, 129, 1024, 32), (64, 300, 4096, 32), (20, 70, 1152, 64),
          (100, 200, 1280, 256), (33, 65, 768, 256), (5, 100, 640, 64)]


@pytest.mark.parametrize("M,N,K,g", SQUARE)
def test_groups_square_gemm(tl, M, N, K, g):
    _check(tl, M, N, K, g, "bf16", expect="gemm", tag="square")


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("path", ["gemv", "gemm", "simple", *DECODE_KERNELS])
def test_groups_forced_paths(tl, g, path):
    M = 2 if path.startswith("gemv") else 5
    _check(tl, M, 200, 1536, g, "bf16", path=path, tag="forced")


@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_groups_raw_bytes(tl, g):
    # uniform random bytes: code 11 reads as 0 on every path
    for M, path in ((1, "auto"), (2, "auto"), (4, "gemm"), (300, "auto")):
        _check(tl, M, 96, 2048, g, "bf16", path=path, raw=True, tag="raw")


def test_groups_simple_only_shapes(tl):
    # K % 128 != 0: only the plain kernel takes these
    _check(tl, 3, 70, 160, 32, "bf16", expect="simple", tag="simple")
    _check(tl, 1, 9, 192, 64, "fp16", expect="simple", tag="simple")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_groups_mixed_batch(tl, dtype):
    """One ternary_linear_batch with decode problems of four scale modes (one
    fused launch each) and prefill problems of two group sizes (one grouped
    GEMM launch each)."""
    import torch
    say(f"mixed-group batch {dtype}")
    specs = [(1, 300, 4096, 32), (1, 200, 2048, 64), (1, 100, 4096, 128), (1, 50, 1024, -1),
             (2, 64, 2048, 256), (256, 300, 2048, 64), (256, 260, 1536, 256),
             (64, 100, 1024, 32)]
    probs, refs = [], []
    for i, (M, N, K, g) in enumerate(specs):
        packed, scale, x = _case(M, N, K, g, dtype, tag=f"batch{i}")
        refs.append(oracle.linear(x, packed, scale, g, dtype=dtype))
        probs.append((to_dev(x, _tdt(dtype)), to_dev(packed, None), to_dev(scale, torch.float16),
                      g, None))
    outs = tl.linear_batch(probs)
    torch.cuda.synchronize()
    for (M, N, K, g), y, (y_ref, bound) in zip(specs, outs, refs):
        check_within(widen(bits_of(y), dtype), y_ref, bound, f"batch M={M} N={N} K={K} g={g}")
