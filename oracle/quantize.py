"""Oracle of the ternary quantizer (test infrastructure only: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it).

The rule is the symmetric linear quantizer of the yangyitao.com vLLM book,
chapter 13 ("量化：精度与速度的工程平衡"), §13.1.3: w_q = round(w / s) with
s = max|w| divided by the largest code, on the ternary code range
{-1, 0, +1} (largest code 1), one s per output channel or per group of g
consecutive K weights (§13.3).  Readings where the pages leave the step open:

  * s is stored as fp16 (the layer's scale format), rounded to nearest even,
    and the codes are rounded against that stored s, so that q * s is what
    the layer computes with;
  * round() is round-half-to-even (numpy's rint), so |w| == s/2 gives 0;
  * a group whose s is 0 gets codes 0 (w / 0 is undefined).

Everything is evaluated in fp64 from the exact values of the 16-bit inputs.
"""

from __future__ import annotations

import numpy as np

from .dense import widen_bf16, widen_f16


def quantize(w_bits, group_size: int, dtype: str = "bf16"):
    """16-bit weight bit patterns [N, K] -> (q int8 [N, K], scale fp16 bits
    [N] or [N, K // group_size])."""
    w = widen_bf16(w_bits) if dtype == "bf16" else widen_f16(w_bits)
    N, K = w.shape
    g = K if group_size == -1 else group_size
    if K % g:
        raise ValueError("K must be a multiple of the group size")
    blocks = w.reshape(N, K // g, g)
    s = np.abs(blocks).max(axis=2)              # s = max|w| / 1 (§13.1.3)
    s16 = s.astype(np.float16)                  # stored scale, nearest even
    sd = s16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = blocks / sd[:, :, None]             # w / s
    q = np.clip(np.rint(t), -1, 1)              # round, on the code range
    q = np.where((sd == 0)[:, :, None], 0.0, q)
    q = q.reshape(N, K).astype(np.int8)
    sbits = s16.view(np.uint16)
    return q, (sbits.reshape(N) if group_size == -1 else sbits)


def dequantize(q, scale_bits, group_size: int) -> np.ndarray:
    """q * s in fp64 (the weights the layer computes with)."""
    q = np.asarray(q, dtype=np.float64)
    N, K = q.shape
    s = widen_f16(scale_bits).reshape(N, -1)
    g = K if group_size == -1 else group_size
    return q * np.repeat(s, g, axis=1)
