"""The zero-skipping pipelined GEMM (TERNARY_PATH_GEMM_ZSKIP) against the
plain pipelined GEMM and the oracle.

A wave skips the decode and MFMAs of a step whose channels x 64 K are all
zero codes (00 or 11) ([trdm] trdm.cn
"三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §6).  The skipped
products are zeros, so the result must be the same bits as TERNARY_PATH_GEMM
(same kernel configuration, same K split) and within the layer's bound of the
oracle.  Inputs: block-sparse codes (zero blocks of 256 x 256, 64 x 256 and
16 x 64, about half the blocks), i.i.d. codes, all-zero codes, and raw random bytes.
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


def _block_sparse(rng, N, K, bn, bk, p_zero=0.5):
    """i.i.d. codes with whole bn x bk blocks set to 0 (probability p_zero)."""
    codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
    zero = rng.random(((N + bn - 1) // bn, (K + bk - 1) // bk)) < p_zero
    mask = np.repeat(np.repeat(zero, bn, axis=0), bk, axis=1)[:N, :K]
    codes[mask] = 0
    return codes


def _compare(tl, x, packed, scale, g, dtype, tag, N, K):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    xd, pd, sd = to_dev(x, tdt), to_dev(packed, None), to_dev(scale, torch.float16)
    y0 = tl.linear(xd, pd, sd, g, path="gemm")
    y1 = tl.linear(xd, pd, sd, g, path="gemm_zskip")
    yt = tl.linear(xd, to_dev(layout.tile(packed, N, K), None), sd, g, path="gemm_zskip",
                   layout="tiled")
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(y0), bits_of(y1)), f"{tag}: zero skipping changed the bits"
    assert np.array_equal(bits_of(y1), bits_of(yt)), f"{tag}: tiled and row-major codes differ"
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    check_within(widen(bits_of(y1), dtype), y_ref, bound, tag)
    return y1


@pytest.mark.parametrize("M,N,K,g,bn,bk,dtype", [
    (300, 1100, 2048, -1, 64, 256, "bf16"),
    (64, 700, 4096, 128, 64, 256, "bf16"),
    (256, 520, 1024, 256, 16, 64, "fp16"),
    (16, 1030, 2048, -1, 16, 64, "bf16"),
    (130, 300, 1536, 64, 64, 256, "bf16"),
    (2048, 512, 512, -1, 64, 256, "bf16"),
    (512, 1024, 2048, 128, 256, 256, "bf16"),
    (300, 768, 1024, -1, 256, 256, "fp16"),
])
def test_zskip_block_sparse(tl, M, N, K, g, bn, bk, dtype):
    say(f"zskip block-sparse M={M} N={N} K={K} g={g} blocks {bn}x{bk} {dtype}")
    rng = np.random.default_rng(M * 31 + N + K)
    codes = _block_sparse(rng, N, K, bn, bk)
    packed, _ = oracle.pack(codes)
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, dtype)
    _compare(tl, x, packed, scale, g, dtype, "block-sparse", N, K)


def test_zskip_dense_and_raw(tl):
    # i.i.d. codes (nothing to skip) and raw random bytes (code 11 included)
    say("zskip i.i.d. codes and raw bytes")
    rng = np.random.default_rng(9)
    N, K, M = 500, 2048, 96
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.25, 0.25))
    scale = synth.draw_scales(rng, N, K, 128)
    x = synth.draw_x(rng, M, K)
    _compare(tl, x, packed, scale, 128, "bf16", "iid", N, K)
    raw = synth.draw_bytes(rng, N, K)
    _compare(tl, x, raw, scale, 128, "bf16", "raw bytes", N, K)


def test_zskip_all_zero(tl):
    # only codes 00 and 11: every step skipped, y = 0 exactly
    say("zskip all-zero codes")
    rng = np.random.default_rng(10)
    N, K, M = 300, 1024, 64
    packed = np.where(rng.random((N, K // 4)) < 0.5, 0x00, 0xFF).astype(np.uint8)
    scale = synth.draw_scales(rng, N, K, -1)
    x = synth.draw_x(rng, M, K)
    y = _compare(tl, x, packed, scale, -1, "bf16", "all zero", N, K)
    assert not np.any(bits_of(y) & 0x7FFF)
