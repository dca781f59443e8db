"""Edge cases of the fp4 x fp8 decode kernel's activation split.

That kernel feeds each activation to the matrix cores as a sum of e4m3 pieces
with power-of-two scales per 32 elements (two pieces for bf16, three for fp16).
The split is exact for every element within 2^13 of its block's largest; the
tests below drive it where it is hardest: full-width significands (the sum
must come out exact), wide dynamic range inside a block, the extremes of the
activation formats, zero blocks and signed zeros.  The bar is the stated one,
|y - y_ref| <= 1e-3 * sum_k |x_k| s(n,k) + 1e-6 against the fp64 oracle, and
bit-exact where the exact result is representable.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen

pytestmark = pytest.mark.gpu

PATH = "gemv_f4"


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


def _to_bits(v, dtype):
    return synth.f64_to_bf16_bits(v) if dtype == "bf16" else synth.f64_to_f16_bits(v)


def _run(tl, x_bits, packed, scale_bits, g, dtype):
    import torch
    y = tl.linear(to_dev(x_bits, _tdt(dtype)), to_dev(packed, None),
                  to_dev(scale_bits, torch.float16), g, path=PATH)
    torch.cuda.synchronize()
    return bits_of(y)


@pytest.mark.parametrize("dtype,M", [("bf16", 1), ("bf16", 3), ("bf16", 8), ("fp16", 1),
                                     ("fp16", 5)])
@pytest.mark.parametrize("g", [-1, 128])
def test_split_is_exact(tl, dtype, M, g):
    """Full-width significands (8 bits bf16, 11 bits fp16) in a few binades,
    codes +-1, power-of-two scales: the exact y is a short dyadic number whose
    fp32 partial sums are exact, so y must equal its rounding bit for bit.
    Any piece lost in the split would change it."""
    say(f"f4 split exactness {dtype} M={M} g={g}")
    rng = np.random.default_rng(11 + M + (g > 0))
    N, K = 64, 256
    sig = 8 if dtype == "bf16" else 11
    span = 6 if dtype == "bf16" else 3          # binades of |x|
    mant = rng.integers(2 ** (sig - 1), 2 ** sig, size=(M, K))
    ex = rng.integers(-span, 1, size=(M, K))
    xv = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0) * np.ldexp(mant.astype(np.float64), ex - sig)
    x = _to_bits(xv, dtype)
    assert np.array_equal(widen(x, dtype), xv)
    codes = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    packed, _ = oracle.pack(codes)
    ng = 1 if g == -1 else K // g
    sv = np.ldexp(1.0, rng.integers(-6, -2, size=(N, ng)))
    s = _to_bits(sv if g > 0 else sv[:, 0], "fp16")
    sfull = np.repeat(sv, K // ng, axis=1)
    exact = xv @ (codes * sfull).T                 # every term exact, sum exact in fp64
    got = _run(tl, x, packed, s, g, dtype)
    assert np.array_equal(got, _to_bits(exact, dtype)), "split lost bits"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("g", [-1, 128, 64, 32])
def test_wide_dynamic_range_blocks(tl, dtype, g):
    """|x| log-uniform over 30 binades (bf16) or 30 (fp16, down to its
    subnormals), so most 32-element blocks hold elements far below their
    largest: those are rounded in the split, within the bound."""
    say(f"f4 dynamic range {dtype} g={g}")
    rng = np.random.default_rng(21 + (g > 0) * g)
    M, N, K = 2, 96, 2048
    lo, hi = (-20, 10) if dtype == "bf16" else (-24, 6)
    xv = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0) * np.exp2(rng.uniform(lo, hi, (M, K)))
    x = _to_bits(xv, dtype)
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    y = widen(_run(tl, x, packed, scale, g, dtype), dtype)
    check_within(y, y_ref, bound, f"dynamic range {dtype} g={g}")


def test_extreme_magnitudes_bf16(tl):
    """Blocks of huge (2^100), tiny normal (2^-120) and subnormal bf16
    activations, alone and mixed inside one block, zero blocks and -0.0."""
    say("f4 extreme magnitudes bf16")
    rng = np.random.default_rng(31)
    M, N, K = 1, 80, 1024
    xv = rng.standard_normal(K)
    xv[0:32] *= 2.0 ** 100                 # a huge block
    xv[32:64] *= 2.0 ** -120               # a tiny block
    xv[64:96] = np.ldexp(rng.integers(1, 127, 32).astype(np.float64), -133)  # subnormal bf16
    xv[96:128] = 0.0                       # a zero block
    xv[128:160] = -0.0
    xv[160] = 2.0 ** 90                    # one huge element beside small ones
    xv[192:224] = 0.0
    xv[200] = -3.0                         # a single nonzero in a block
    x = synth.f64_to_bf16_bits(xv[None, :])
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    for g in (-1, 128):
        scale = synth.draw_scales(rng, N, K, g)
        y_ref, bound = oracle.linear(x, packed, scale, g)
        y = widen(_run(tl, x, packed, scale, g, "bf16"), "bf16")
        assert np.all(np.isfinite(y))
        check_within(y, y_ref, bound, f"extremes g={g}")


def test_extreme_magnitudes_fp16(tl):
    """fp16 activations at their largest finite value, their smallest
    subnormal and in between, inside one block and across blocks."""
    say("f4 extreme magnitudes fp16")
    rng = np.random.default_rng(41)
    M, N, K = 1, 64, 512
    xv = rng.standard_normal(K)
    xv[0:32] = np.where(rng.random(32) < 0.5, -65504.0, 65504.0)
    xv[32:64] = np.ldexp(rng.integers(1, 1024, 32).astype(np.float64), -24)  # subnormals
    xv[64] = 60000.0                       # beside small ones in one block
    xv[65:96] = np.ldexp(1.0, -24)
    xv[96:128] = 0.0
    x = synth.f64_to_f16_bits(xv[None, :])
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    for g in (-1, 128):
        scale = synth.draw_scales(rng, N, K, g)
        y_ref, bound = oracle.linear(x, packed, scale, g, dtype="fp16")
        y = widen(_run(tl, x, packed, scale, g, "fp16"), "fp16")
        assert np.all(np.isfinite(y))
        check_within(y, y_ref, bound, f"fp16 extremes g={g}")


def test_agrees_with_16bit_kernel_within_bound(tl):
    """The two decode kernels on the same 7B-shaped problem: each within the
    bound of the oracle (they sum in different orders, so not bitwise)."""
    say("f4 vs b16 decode kernels")
    import torch
    case = synth.make_case(2, 4, 1)       # gate 18944 x 4096 at M = 1
    packed, _ = oracle.pack(case.codes)
    y_ref, bound = oracle.linear(case.x, packed, case.scale, -1)
    for path in ("gemv_f4", "gemv_b16"):
        y = tl.linear(to_dev(case.x, torch.bfloat16), to_dev(packed, None),
                      to_dev(case.scale, torch.float16), -1, path=path)
        torch.cuda.synchronize()
        check_within(widen(bits_of(y), "bf16"), y_ref, bound, path)


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("offset", [0, 1])
def test_group_scales_any_alignment(tl, g, offset):
    """Group scales are staged two to a 4-byte load when the scale array is
    4-byte aligned, one per 2-byte load otherwise: both against the oracle,
    with tiled and row-major codes, on a ragged block and more than one
    chunk of slabs."""
    import torch
    say(f"f4 group scales g={g} offset={offset}")
    M, N, K = 1, 45, 3072
    rng = np.random.default_rng(977 + g + offset)
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, "bf16")
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype="bf16")
    sbuf = torch.zeros(scale.size + 8, dtype=torch.float16, device="cuda:0")
    sd = sbuf[offset:offset + scale.size].view(scale.shape)
    sd.copy_(to_dev(scale, torch.float16))
    xd = to_dev(x, torch.bfloat16)
    pd = to_dev(packed, None)
    for lay, codes in (("rows", pd), ("tiled", tl.tile(pd))):
        y = tl.linear(xd, codes, sd, g, path=PATH, layout=lay)
        torch.cuda.synchronize()
        check_within(widen(bits_of(y), "bf16"), y_ref, bound, f"f4 g={g} offset={offset} {lay}")
