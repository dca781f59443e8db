"""Pins that tie the quantizer oracle (oracle/quantize.py) to facts fixed
outside it: the yangyitao.com vLLM book, chapter 13 (§13.1.3 the symmetric
rule w_q = round(w / s), s = max|w| / largest code; §13.1.4 the error bound
s/2 of rounding to nearest) with the ternary code range {-1, 0, +1}, plus
closed forms and invariants.

Each pin takes the quantizer module (the real one, or a deliberately broken
copy in the mutation test) and raises AssertionError on disagreement.
"""

from __future__ import annotations

import numpy as np

from oracle import dense
from synth import f64_to_bf16_bits, f64_to_f16_bits

GROUPS = (-1, 32, 64, 128, 256)


def _bits(v, dtype):
    return f64_to_bf16_bits(v) if dtype == "bf16" else f64_to_f16_bits(v)


def _widen(b, dtype):
    return dense.widen_bf16(b) if dtype == "bf16" else dense.widen_f16(b)


def _groups(a, g):
    N, K = a.shape
    g = K if g == -1 else g
    return a.reshape(N, K // g, g)


def pin_quantize_exact_ternary(Q):
    """w = c * q with each group holding a nonzero: the quantizer returns q
    and s = c exactly (c exact in bf16 and fp16)."""
    rng = np.random.default_rng(21)
    N, K = 5, 512
    for g in GROUPS:
        q0 = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        gq = _groups(q0, g)
        gq[:, :, 0] = 1                                    # every group has a nonzero
        G = gq.shape[1]
        c = np.ldexp(1.0 + rng.integers(0, 8, size=(N, G)) / 8.0, rng.integers(-9, 3, size=(N, G)))
        w = (gq * c[:, :, None]).reshape(N, K)
        for dt in ("bf16", "fp16"):
            q, s = Q.quantize(_bits(w, dt), g, dt)
            assert np.array_equal(q, q0), (g, dt)
            assert np.array_equal(dense.widen_f16(s).reshape(N, G), c), (g, dt)


def pin_quantize_error_bound(Q):
    """|w - q s| <= s/2 for every weight (§13.1.4), q in {-1, 0, +1}, and s
    within fp16 rounding of the group's max |w| (it scales the largest
    weight to a code of magnitude 1)."""
    rng = np.random.default_rng(22)
    for dt in ("bf16", "fp16"):
        for g in GROUPS:
            w = _bits(rng.standard_normal((7, 1024)) * 0.03, dt)
            q, s = Q.quantize(w, g, dt)
            assert set(np.unique(q)) <= {-1, 0, 1}
            wd = _widen(w, dt)
            err = np.abs(wd - Q.dequantize(q, s, g))
            sd = dense.widen_f16(s).reshape(7, -1)
            half = np.repeat(sd, 1024 // sd.shape[1], axis=1) / 2
            assert np.all(err <= half), (g, dt)
            mx = np.abs(_groups(wd, g)).max(axis=2)
            assert np.all(np.abs(sd - mx) <= mx * 2.0 ** -11), (g, dt)
            # the largest weight of each group maps to +-1
            amax = np.abs(_groups(wd, g)).argmax(axis=2)
            qg = _groups(q, g)
            picked = np.take_along_axis(qg, amax[:, :, None], axis=2)[:, :, 0]
            assert np.all(np.abs(picked) == 1), (g, dt)


def pin_quantize_ties_to_even(Q):
    """round(w/s) at w = +-s/2 gives 0 (ties to even); the next representable
    weight above s/2 gives +-1."""
    N, K, g = 2, 64, 32
    for dt in ("bf16", "fp16"):
        w = np.zeros((N, K))
        w[:, 0] = 1.0                      # s = 1 in both groups
        w[:, 32] = -1.0
        w[0, 1], w[0, 2], w[1, 33] = 0.5, -0.5, 0.5
        up = 0.5 + (2.0 ** -8 if dt == "bf16" else 2.0 ** -11)  # next value above 1/2
        w[1, 3], w[1, 4] = up, -up
        q, s = Q.quantize(_bits(w, dt), g, dt)
        assert np.all(dense.widen_f16(s) == 1.0)
        assert q[0, 1] == 0 and q[0, 2] == 0 and q[1, 33] == 0, dt
        assert q[1, 3] == 1 and q[1, 4] == -1, dt
        assert q[0, 0] == 1 and q[0, 32] == -1


def pin_quantize_zero_groups(Q):
    """An all-zero group gets s = 0 and codes 0; its neighbours are untouched."""
    rng = np.random.default_rng(23)
    for g in (32, 64, 128, 256):
        w = rng.standard_normal((3, 512)) * 0.02
        w[1, g:2 * g] = 0.0
        q, s = Q.quantize(_bits(w, "bf16"), g, "bf16")
        assert np.all(s.reshape(3, -1)[1, 1] == 0) and np.all(q[1, g:2 * g] == 0), g
        w2 = w.copy()
        w2[1, g:2 * g] = 0.0
        w2[0, :] = 0.0
        q2, s2 = Q.quantize(_bits(w2, "bf16"), g, "bf16")
        assert np.all(q2[0] == 0) and np.all(s2.reshape(3, -1)[0] == 0)
        assert np.array_equal(q2[1:], q[1:]) and np.array_equal(s2.reshape(3, -1)[1:],
                                                                s.reshape(3, -1)[1:])


def pin_quantize_group_locality(Q):
    """Changing one weight changes only its own group's scale and codes."""
    rng = np.random.default_rng(24)
    for g in GROUPS:
        w = rng.standard_normal((4, 512)) * 0.02
        q, s = Q.quantize(_bits(w, "bf16"), g, "bf16")
        w2 = w.copy()
        w2[2, 300] = 0.5                    # becomes that group's max
        q2, s2 = Q.quantize(_bits(w2, "bf16"), g, "bf16")
        G = 512 // (512 if g == -1 else g)
        gi = 300 // (512 if g == -1 else g)
        sg, sg2 = s.reshape(4, G), s2.reshape(4, G)
        mask = np.ones((4, G), bool)
        mask[2, gi] = False
        assert np.array_equal(sg[mask], sg2[mask]) and sg[2, gi] != sg2[2, gi], g
        lo, hi = gi * (512 // G), (gi + 1) * (512 // G)
        qm = np.ones((4, 512), bool)
        qm[2, lo:hi] = False
        assert np.array_equal(q[qm], q2[qm]), g
        assert q2[2, 300] == 1


def pin_quantize_symmetry_and_scaling(Q):
    """quantize(-w) = (-q, s); quantize(2w) = (q, 2s) (powers of two are exact)."""
    rng = np.random.default_rng(25)
    for g in GROUPS:
        w = rng.standard_normal((3, 256)) * 0.05
        q, s = Q.quantize(_bits(w, "fp16"), g, "fp16")
        qn, sn = Q.quantize(_bits(-w, "fp16"), g, "fp16")
        assert np.array_equal(qn, -q) and np.array_equal(sn, s), g
        q2, s2 = Q.quantize(_bits(2 * w, "fp16"), g, "fp16")
        assert np.array_equal(q2, q), g
        assert np.array_equal(dense.widen_f16(s2), 2 * dense.widen_f16(s)), g


def pin_quantize_brute_force(Q):
    """Tiny shapes: every code is the nearest point of {-s, 0, +s} to w (ties
    to 0), every s the fp16 value nearest the group's max |w|, found by
    scanning all finite fp16 values."""
    rng = np.random.default_rng(26)
    allf16 = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    for g in (-1, 32, 64):
        w = rng.standard_normal((2, 128)) * 0.1
        wb = _bits(w, "bf16")
        wd = dense.widen_bf16(wb)
        q, s = Q.quantize(wb, g, "bf16")
        sd = dense.widen_f16(s).reshape(2, -1)
        mx = np.abs(_groups(wd, g)).max(axis=2)
        for (i, j), m in np.ndenumerate(mx):
            d = np.abs(allf16 - m)
            best = allf16[d == d.min()]
            assert sd[i, j] in best, (g, i, j)
        full = np.repeat(sd, 128 // sd.shape[1], axis=1)
        for (i, k), v in np.ndenumerate(wd):
            cands = np.array([-full[i, k], 0.0, full[i, k]])
            d = np.abs(cands - v)
            ok = np.flatnonzero(d == d.min())
            want = 0 if 1 in ok else int(ok[0]) - 1
            assert q[i, k] == want, (g, i, k, v, full[i, k])


def pin_quantize_subnormal_scale(Q):
    """bf16 weights below fp16's normal range: s is the subnormal fp16 value
    nearest max|w|, and the codes are rounded against that stored s.  With
    max|w| = 255 * 2^-28, s rounds up to 2^-20, so w = 2^-21 sits exactly at
    s/2 and gives 0 (ties to even), although it exceeds max|w| / 2."""
    m, half = 255 * 2.0 ** -28, 2.0 ** -21
    w = np.zeros((2, 32))
    w[:, 0] = m
    w[0, 1], w[0, 2] = half, -half
    w[1, 1], w[1, 2] = 9 * 2.0 ** -24, -7 * 2.0 ** -24     # just above, below s/2
    q, s = Q.quantize(_bits(w, "bf16"), 32, "bf16")
    assert np.array_equal(dense.widen_bf16(_bits(w, "bf16")), w)      # w exact in bf16
    assert np.all(dense.widen_f16(s) == 2.0 ** -20), dense.widen_f16(s)
    assert q[0, 0] == 1 and q[0, 1] == 0 and q[0, 2] == 0
    assert q[1, 0] == 1 and q[1, 1] == 1 and q[1, 2] == 0


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
