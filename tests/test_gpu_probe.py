"""The measurement probes of include/ternary_probe.h on the GPU: the copy moves
exactly its bytes, the read runs over ragged sizes, and the MFMA loop computes
what its register operands define (so the flops it is credited with are
really issued)."""

import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_ternary_linear_amd as tl
    tl.lib()
    return tl


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (16 * 1001, 7), (1 << 20, 64),
                                       ((1 << 22) + 48, 300)])
def test_probe_copy_exact(tl, nbytes, wg):
    import torch
    say(f"probe copy bytes={nbytes} wg={wg}")
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    tl.probe_copy(src, dst, wg)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("nbytes,wg", [(16, 1), (16 * 1001, 7), ((1 << 22) + 48, 300)])
def test_probe_read_runs(tl, nbytes, wg, nt):
    import torch
    say(f"probe read bytes={nbytes} wg={wg} nontemporal={nt}")
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    tl.probe_read(src, sink, wg, nontemporal=nt)
    torch.cuda.synchronize()


def _wave_total():
    """Sum over a wave's 64 outputs of one loop iteration: four chains
    (a,b), (b,a), (a,a), (b,b) of 16x16x32 products.  Lane l supplies A row
    l % 16 and B column l % 16, both for k = 8 (l // 16) + e, e = 0..7; element
    e of operand a has value 2^-7 (1 + ((l + e) & 7) / 8), and operand b is a
    with its four 32-bit words reversed."""
    def aval(l, e):
        return 2.0 ** -7 * (1 + ((l + e) & 7) / 8)

    def bval(l, e):
        return 2.0 ** -7 * (1 + ((l + 2 * (3 - e // 2) + e % 2) & 7) / 8)

    def total(P, Q):
        s = 0.0
        for k in range(32):
            rows = sum(P(i + 16 * (k // 8), k % 8) for i in range(16))
            cols = sum(Q(j + 16 * (k // 8), k % 8) for j in range(16))
            s += rows * cols
        return s

    return total(aval, bval) + total(bval, aval) + total(aval, aval) + total(bval, bval)


@pytest.mark.parametrize("wg,iters", [(1, 1), (3, 5), (256, 64)])
def test_probe_mfma_values(tl, wg, iters):
    import torch
    say(f"probe mfma wg={wg} iters={iters}")
    out = tl.probe_mfma(wg, iters)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(wg * 4, 64).sum(axis=1)
    # every product and partial sum is a small multiple of 2^-20: exact in fp32
    assert np.all(got == iters * _wave_total()), (got[:4], iters * _wave_total())
    assert tl.probe_mfma_flops(wg, iters) == wg * 4 * iters * 4 * 2 * 16 * 16 * 32
