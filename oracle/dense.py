"""Second, independent evaluation of the ternary linear layer (test infrastructure).

Used only to cross-check the C oracle on tiny shapes.  It shares nothing with
``ternary_oracle.c``: the 2-bit fields are read by integer division, the code
is decoded with the comparison form (c == 1) - (c == 2) that the 7B-checkpoint
page (m.nxbn.cn/news/169761, §2.2) states, fp16/bf16 are widened through
numpy's own float16/float32 types, and the product is a dense fp64 matmul
y = x @ (Q * S)^T, the dequantise-then-matmul definition of the Bonsai page
(m.xxqk.cn/news/593501, §4.3).
"""

from __future__ import annotations

import numpy as np


def fields(packed: np.ndarray) -> np.ndarray:
    """bytes [N, B] -> 2-bit fields [N, 4B], least significant pair first."""
    b = np.asarray(packed, dtype=np.int64)
    per = [(b // (4 ** i)) % 4 for i in range(4)]
    return np.stack(per, axis=-1).reshape(b.shape[0], -1)


def decode(packed: np.ndarray) -> np.ndarray:
    c = fields(packed)
    return (c == 1).astype(np.int64) - (c == 2).astype(np.int64)


def widen_f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def widen_bf16(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def full_scale(scale_bits, N: int, K: int, group_size: int) -> np.ndarray:
    s = widen_f16(scale_bits)
    if group_size == -1:
        return np.broadcast_to(s.reshape(N, 1), (N, K)).copy()
    return np.repeat(s.reshape(N, K // group_size), group_size, axis=1)


def linear(x_bits, packed, scale_bits, group_size: int, dtype: str = "bf16"):
    """(y, bound) with y = x @ (Q*S)^T and bound = |x| @ |S|^T, dense fp64."""
    x = widen_f16(x_bits) if dtype == "fp16" else widen_bf16(x_bits)
    q = decode(packed).astype(np.float64)
    N, K = q.shape
    s = full_scale(scale_bits, N, K, group_size)
    y = x @ (q * s).T
    bound = np.abs(x) @ np.abs(s).T
    return y, bound
