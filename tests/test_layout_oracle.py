"""The oracle's tiled code layout (oracle/layout.py) against positions worked
out by hand (tests/golden/tiled_positions.txt) and the invariants any byte
permutation with zero padding must keep.  The layout is the GPU library's own
storage order for the codes of the row-major packing (trdm.cn
"三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战" §3.1); these tests pin the
oracle's copy of it, which the GPU tests then hold the library to."""

from pathlib import Path

import numpy as np
import pytest

import oracle
from oracle import layout

GOLDEN = Path(__file__).resolve().parent / "golden" / "tiled_positions.txt"


def golden_positions():
    out = []
    for ln in GOLDEN.read_text().splitlines():
        ln = ln.split("#", 1)[0].strip()
        if ln:
            N, K, n, j, off = map(int, ln.split())
            out.append((N, K, n, j, off))
    return out


def test_golden_has_cases():
    assert len(golden_positions()) >= 12


@pytest.mark.parametrize("case", golden_positions())
def test_hand_worked_positions(case):
    N, K, n, j, off = case
    packed = np.zeros((N, K // 4), dtype=np.uint8)
    packed[n, j] = 0xA5
    t = layout.tile(packed, N, K)
    assert np.flatnonzero(t).tolist() == [off]
    assert t[off] == 0xA5
    assert np.array_equal(layout.untile(t, N, K), packed)


@pytest.mark.parametrize("N,K,total", [(17, 260, 4096), (16, 256, 1024), (1, 4, 1024),
                                       (0, 256, 0), (16, 0, 0), (4096, 4096, 4 << 20),
                                       (18944, 4096, 18944 * 1024), (33, 1028, 3 * 5 * 1024)])
def test_size(N, K, total):
    assert layout.geometry(N, K)[2] == total


@pytest.mark.parametrize("N,K", [(1, 4), (15, 252), (17, 260), (33, 1028), (64, 512), (16, 768),
                                 (40, 132)])
def test_permutation_with_zero_padding(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    packed = rng.integers(1, 256, size=(N, K // 4), dtype=np.uint8)   # no zero bytes
    t = layout.tile(packed, N, K)
    # every byte of the packing appears once, all others are padding zeros
    assert np.count_nonzero(t) == packed.size
    assert np.array_equal(np.sort(t[t != 0]), np.sort(packed.ravel()))
    assert np.array_equal(layout.untile(t, N, K), packed)


def test_block_holds_its_rows_and_columns():
    # block (b, s) holds exactly rows 16b..16b+15, bytes 64s..64s+63
    N, K = 40, 1028
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)
    t = layout.tile(packed, N, K)
    bands, slabs, _ = layout.geometry(N, K)
    for b in range(bands):
        for s in range(slabs):
            blk = t[(b * slabs + s) * 1024:(b * slabs + s + 1) * 1024]
            rows = packed[16 * b:16 * b + 16, 64 * s:64 * s + 64]
            got = [blk[g * 256 + r * 16: g * 256 + r * 16 + 16] for r in range(rows.shape[0])
                   for g in range(4)]
            want = [np.pad(rows[r, 16 * g:16 * g + 16], (0, 16 - rows[r, 16 * g:16 * g + 16].size))
                    for r in range(rows.shape[0]) for g in range(4)]
            for a, w in zip(got, want):
                assert np.array_equal(a, w)


def test_linear_is_layout_independent():
    # the layer's result depends only on the codes: the oracle evaluated on
    # the round trip of a tiled buffer is the oracle on the row-major codes
    rng = np.random.default_rng(9)
    N, K = 21, 384
    import synth
    codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
    packed, _ = oracle.pack(codes)
    scale = synth.draw_scales(rng, N, K, 128)
    x = synth.draw_x(rng, 2, K)
    back = layout.untile(layout.tile(packed, N, K), N, K)
    y0, b0 = oracle.linear(x, packed, scale, 128)
    y1, b1 = oracle.linear(x, back, scale, 128)
    assert np.array_equal(y0, y1) and np.array_equal(b0, b1)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        layout.geometry(4, 6)
    with pytest.raises(ValueError):
        layout.tile(np.zeros((4, 3), np.uint8), 4, 16)
    with pytest.raises(ValueError):
        layout.untile(np.zeros(100, np.uint8), 4, 16)
