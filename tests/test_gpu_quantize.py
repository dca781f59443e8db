"""GPU quantizer (ternary_quantize) against the CPU oracle, bit-exact: the
codes and fp16 scales are integer decisions, taken in both places from the
exact values of the 16-bit weights."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen
from oracle import quantize as OQ

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


def _run(tl, wbits, g, dt):
    import torch
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    packed, scale = tl.quantize(to_dev(wbits, tdt), g)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), bits_of(scale)


def _check(tl, wbits, g, dt):
    q_ref, s_ref = OQ.quantize(wbits, g, dt)
    p_ref, inv = oracle.pack(q_ref)
    assert inv == 0
    p_dev, s_dev = _run(tl, wbits, g, dt)
    assert np.array_equal(s_dev.reshape(s_ref.shape), s_ref), "scales differ"
    assert np.array_equal(p_dev, p_ref), "codes differ"


# Shapes span several 256-lane passes of a row, ragged row lengths (K not a
# multiple of 1024) and a single 4-weight row.
SHAPES = [(1, 4), (3, 36), (1, 64), (7, 1028), (33, 4096), (129, 3072), (64, 18944)]


CASES = [(N, K, g) for N, K in SHAPES for g in (-1, 32, 64, 128, 256) if g == -1 or K % g == 0]


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("N,K,g", CASES)
def test_quantize_matches_oracle(tl, N, K, g, dt):
    say(f"quantize N={N} K={K} g={g} {dt}")
    rng = np.random.default_rng(N * 31 + K + (g if g > 0 else 7))
    _check(tl, synth.draw_weights(rng, N, K, 0.02, dt), g, dt)


@pytest.mark.parametrize("g", [-1, 32, 128])
def test_quantize_edge_values(tl, g):
    """Zero groups, exact ties at s/2, the next value above s/2, subnormal
    fp16 scales (bf16 weights below fp16's normal range) and negative zeros."""
    say(f"quantize edge values g={g}")
    N, K = 6, 256
    w = np.random.default_rng(9).standard_normal((N, K)) * 0.02
    w[0] = 0.0                                   # an all-zero row
    w[1, :32] = 0.0                              # an all-zero first group
    w[2, :] = 0.0
    w[2, 0], w[2, 1], w[2, 2] = 1.0, 0.5, -0.5   # ties -> 0
    w[2, 3], w[2, 4] = 0.50390625, -0.50390625   # next bf16 above 1/2 -> +-1
    w[3] = w[3] * 1e-4                           # scales below fp16's normal range
    w[4, :] = 0.0
    w[4, 0], w[4, 1], w[4, 2] = 255 * 2.0 ** -28, 2.0 ** -21, -(2.0 ** -21)
    wb = synth.f64_to_bf16_bits(w)
    wb[5, ::3] = 0x8000                          # -0.0
    _check(tl, wb, g, "bf16")


def test_quantize_deterministic_and_layer_input(tl):
    """Two calls give identical bytes, and the layer on the quantizer's output
    matches the oracle layer on the oracle's codes and scales."""
    import torch
    say("quantize -> linear")
    rng = np.random.default_rng(77)
    N, K, g = 512, 4096, 128
    wb = synth.draw_weights(rng, N, K, 0.02, "bf16")
    a = _run(tl, wb, g, "bf16")
    b = _run(tl, wb, g, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q_ref, s_ref = OQ.quantize(wb, g, "bf16")
    p_ref, _ = oracle.pack(q_ref)
    x = synth.draw_x(rng, 4, K)
    y_ref, bound = oracle.linear(x, p_ref, s_ref, g)
    packed, scale = tl.quantize(to_dev(wb, torch.bfloat16), g)
    y = tl.linear(to_dev(x, torch.bfloat16), packed, scale, g)
    torch.cuda.synchronize()
    check_within(widen(bits_of(y), "bf16"), y_ref, bound, "linear(quantize(w))")


def test_quantize_empty_rows(tl):
    import torch
    say("quantize N=0")
    w = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda:0")
    packed, scale = tl.quantize(w, 64)
    torch.cuda.synchronize()
    assert packed.shape == (0, 32) and scale.shape == (0, 2)
