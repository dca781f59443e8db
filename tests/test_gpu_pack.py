"""GPU pack/unpack against the CPU oracle, bit-exact (integer work)."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


def _pack_dev(tl, codes, with_count=True):
    import torch
    q = to_dev(codes, None)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0") if with_count else None
    p = tl.pack(q, cnt)
    torch.cuda.synchronize()
    return p.cpu().numpy(), (int(cnt.item()) if with_count else None)


@pytest.mark.parametrize("N,K", [(1, 4), (3, 4), (1, 60), (1, 64), (7, 100), (33, 256),
                                 (129, 1028), (512, 4096)])
def test_pack_matches_oracle(tl, N, K):
    say(f"pack N={N} K={K}")
    rng = np.random.default_rng(N * 7919 + K)
    codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
    ref, inv = oracle.pack(codes)
    got, cnt = _pack_dev(tl, codes)
    assert inv == 0 and cnt == 0
    assert np.array_equal(got, ref)


def test_pack_counts_invalid(tl):
    say("pack invalid values")
    rng = np.random.default_rng(5)
    codes = rng.integers(-128, 128, size=(37, 132)).astype(np.int8)
    ref, inv = oracle.pack(codes)
    got, cnt = _pack_dev(tl, codes)
    assert cnt == inv and inv > 0
    assert np.array_equal(got, ref)
    got2, _ = _pack_dev(tl, codes, with_count=False)
    assert np.array_equal(got2, ref)


@pytest.mark.parametrize("N,K", [(1, 4), (5, 36), (64, 1024), (300, 4100)])
def test_unpack_random_bytes(tl, N, K):
    say(f"unpack random bytes N={N} K={K}")
    import torch
    rng = np.random.default_rng(N + K)
    b = synth.draw_bytes(rng, N, K)
    assert oracle.count_reserved(b) > 0 or b.size < 4
    ref = oracle.unpack(b)
    got = tl.unpack(to_dev(b, None))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_unpack_all_256_bytes(tl):
    say("unpack exhaustive bytes")
    import torch
    b = np.arange(256, dtype=np.uint8).reshape(4, 64)
    got = tl.unpack(to_dev(b, None))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.unpack(b))


def test_roundtrip_full_size(tl):
    say("pack/unpack 18944x4096")
    import torch
    codes = synth.draw_codes(np.random.default_rng(99), 18944, 4096, 0.3, 0.3)
    q = to_dev(codes, None)
    p = tl.pack(q)
    back = tl.unpack(p)
    torch.cuda.synchronize()
    ref, _ = oracle.pack(codes)
    assert np.array_equal(p.cpu().numpy(), ref)
    assert torch.equal(back, q)


def test_int8_view_of_packed(tl):
    say("unpack of an int8-typed packed tensor")
    import torch
    rng = np.random.default_rng(3)
    b = synth.draw_bytes(rng, 16, 256)
    dev = to_dev(b, None).view(torch.int8)
    got = tl.unpack(dev)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.unpack(b))
