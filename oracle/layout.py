"""Tiled code layout of the GPU library, written out from its definition
(test infrastructure only; the GPU library never imports this).

The layout is the library's own, not the pages': the bytes of the row-major
packing ([N, K/4], trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
§3.1) regrouped into blocks of 16 rows x 64 bytes (256 codes).  Rows are
padded to a multiple of 16 and K to a multiple of 256 with zero bytes (code
00); block (b, s) covers rows 16b .. 16b+15 and bytes 64s .. 64s+63 of each
row and is stored as 1024 consecutive bytes: its four quarters g = 0..3 (bytes
64s+16g .. 64s+16g+15 of each row) in order, each quarter its 16 rows in
order, each row's 16 bytes in order.  Blocks are stored band by band (all
slabs s of band b, then band b+1).

The functions below follow that description block by block with plain
slicing, no reshapes that would hide the order.
"""

from __future__ import annotations

import numpy as np

ROWS, SLAB_BYTES, QUARTER = 16, 64, 16


def geometry(N: int, K: int):
    """(row bands, slabs, total bytes) of the tiled layout of an [N, K] matrix."""
    if N < 0 or K < 0 or K % 4:
        raise ValueError("N >= 0, K >= 0, K % 4 == 0")
    bands = -(-N // ROWS)
    slabs = -(-K // 256)
    return bands, slabs, bands * slabs * ROWS * SLAB_BYTES


def tile(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Row-major codes uint8 [N, K/4] -> tiled bytes, uint8 [total]."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.shape != (N, K // 4):
        raise ValueError(f"packed must be [{N}, {K // 4}]")
    bands, slabs, total = geometry(N, K)
    padded = np.zeros((bands * ROWS, slabs * SLAB_BYTES), dtype=np.uint8)
    padded[:N, :K // 4] = packed
    out = np.zeros(total, dtype=np.uint8)
    pos = 0
    for b in range(bands):
        for s in range(slabs):
            for g in range(4):
                c0 = s * SLAB_BYTES + g * QUARTER
                for r in range(ROWS):
                    out[pos:pos + QUARTER] = padded[b * ROWS + r, c0:c0 + QUARTER]
                    pos += QUARTER
    assert pos == total
    return out


def untile(tiled: np.ndarray, N: int, K: int) -> np.ndarray:
    """Tiled bytes -> row-major codes uint8 [N, K/4] (padding is not read)."""
    tiled = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    bands, slabs, total = geometry(N, K)
    if tiled.size != total:
        raise ValueError(f"tiled must hold {total} bytes")
    padded = np.zeros((bands * ROWS, slabs * SLAB_BYTES), dtype=np.uint8)
    pos = 0
    for b in range(bands):
        for s in range(slabs):
            for g in range(4):
                c0 = s * SLAB_BYTES + g * QUARTER
                for r in range(ROWS):
                    padded[b * ROWS + r, c0:c0 + QUARTER] = tiled[pos:pos + QUARTER]
                    pos += QUARTER
    return padded[:N, :K // 4].copy()
