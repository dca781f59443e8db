"""Host <-> device marshalling and the parity check used by the GPU tests."""

from __future__ import annotations

import sys

import numpy as np

import oracle


def say(msg: str) -> None:
    """Name the case before a GPU step, so a failing run says which one."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(dtype).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def bits_of(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def half_ulp(y_ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of y_ref in the output dtype (normal range)."""
    frac_bits = 7 if dtype == "bf16" else 10
    _, e = np.frexp(np.abs(y_ref))
    return np.where(y_ref == 0, 0.0, np.ldexp(0.5, e - 1 - frac_bits))


def check_within(y_dev: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str,
                 rel: float = 1e-3, abs_: float = 1e-6, out_rounding: str | None = None) -> float:
    """Assert |y_dev - y_ref| <= rel*B + abs_ everywhere; return the worst ratio.

    ``out_rounding`` (a dtype name) adds half an output ULP of y_ref to the
    limit.  Only edge cases with very short K use it: there |y| can approach
    B = sum|x|s, and rounding the result to bf16 alone (up to 2^-9 |y|) then
    exceeds 1e-3 B, whatever the kernel does.
    """
    err = np.abs(y_dev - y_ref)
    lim = rel * bound + abs_
    if out_rounding is not None:
        lim = lim + half_ulp(y_ref, out_rounding)
    ok = err <= lim
    if not ok.all():
        idx = np.argwhere(~ok)[:8]
        detail = [(tuple(int(v) for v in i), float(y_dev[tuple(i)]), float(y_ref[tuple(i)]),
                   float(lim[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int((~ok).sum())}/{ok.size} outside the bound; "
                             f"(index, gpu, ref, limit): {detail}")
    return float((err / lim).max()) if err.size else 0.0
