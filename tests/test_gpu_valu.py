"""The vector-ALU decode GEMV (TERNARY_PATH_GEMV_VALU) against the oracle.

That kernel adds +x, -x or nothing per code in fp32 and reduces across lanes
(m.nxbn.cn/news/169761 §4.1); it exists to be timed against the matrix-core
decode kernels, and is held to the same bound,
|y - y_ref| <= 1e-3 * sum_k |x_k| s(n,k) + 1e-6, on every output.
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


@pytest.mark.parametrize("N,K,g,dtype", [
    (1000, 4096, -1, "bf16"), (77, 256, -1, "fp16"), (130, 18944, -1, "bf16"),
    (50, 1024, 64, "bf16"), (33, 2048, 128, "fp16"), (40, 768, 256, "bf16"),
    (17, 65536, -1, "bf16"), (16, 4352, 128, "bf16"),
])
def test_valu_matches_oracle(tl, N, K, g, dtype):
    import torch
    say(f"valu gemv N={N} K={K} g={g} {dtype}")
    rng = np.random.default_rng(N * 13 + K)
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, 1, K, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    y = tl.linear(to_dev(x, tdt), to_dev(packed, None), to_dev(scale, torch.float16), g,
                  path="gemv_valu")
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    check_within(widen(bits_of(y), dtype), y_ref, bound, "valu")


def test_valu_reserved_codes_read_as_zero(tl):
    import torch
    say("valu gemv reserved codes")
    rng = np.random.default_rng(5)
    N, K = 64, 1024
    packed = synth.draw_bytes(rng, N, K)              # includes code 11
    assert oracle.count_reserved(packed) > 0
    scale = synth.draw_scales(rng, N, K, -1)
    x = synth.draw_x(rng, 1, K)
    y = tl.linear(to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16),
                  -1, path="gemv_valu")
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, -1)
    check_within(widen(bits_of(y), "bf16"), y_ref, bound, "valu reserved")


@pytest.mark.parametrize("si", [0, 4, 6])
def test_valu_7b_shapes_full(tl, si):
    # q, gate and down of the 7B layer at M = 1, every output compared
    import torch
    case = synth.make_case(2, si, 1)
    say(f"valu gemv 7B {case.shape.name}")
    packed, _ = oracle.pack(case.codes)
    y = tl.linear(to_dev(case.x, torch.bfloat16), to_dev(packed, None),
                  to_dev(case.scale, torch.float16), -1, path="gemv_valu")
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(case.x, packed, case.scale, -1)
    check_within(widen(bits_of(y), "bf16"), y_ref, bound, f"valu 7B {case.shape.name}")
