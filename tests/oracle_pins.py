"""Pins that tie the CPU oracle to facts fixed outside the oracle itself.

Each pin takes an ``oracle.Oracle`` (the real build, or a deliberately broken
copy in the mutation test) and raises AssertionError when the oracle disagrees
with the pages or with the mathematics:

  * values printed on the pages (the worked byte, the code table, the bit
    order), stored under tests/golden/ with their citations;
  * closed forms with exactly representable inputs (all-zero, all +1, all -1,
    one-hot codes; per-channel all +1);
  * invariants (power-of-two scale doubling, equal group scales equal the
    per-channel result, row permutation, batching);
  * library routines (numpy's float16 and float32 widening);
  * an independent dense brute force (oracle/dense.py) on tiny shapes.
"""

from __future__ import annotations

from pathlib import Path

import numpy as np

from oracle import dense
from synth import f64_to_bf16_bits, f64_to_f16_bits

GOLDEN = Path(__file__).resolve().parent / "golden"


def golden_bytes():
    rows = []
    for line in (GOLDEN / "unpack_bytes.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        parts = line.split()
        rows.append((int(parts[0], 16), [int(v) for v in parts[1:5]]))
    return rows


# ---------------------------------------------------------------- format pins

def pin_golden_unpack(o):
    for byte, vals in golden_bytes():
        got = o.unpack(np.array([[byte]], np.uint8))[0].tolist()
        assert got == vals, f"unpack(0x{byte:02x}) = {got}, pages give {vals}"


def pin_golden_pack(o):
    for byte, vals in golden_bytes():
        if any(((byte >> (2 * i)) & 3) == 3 for i in range(4)):
            continue  # reserved fields are never produced by pack
        got, inv = o.pack(np.array([vals], np.int8))
        assert inv == 0
        assert int(got[0, 0]) == byte, f"pack({vals}) = 0x{int(got[0, 0]):02x}, expected 0x{byte:02x}"


def pin_code_forms(o):
    # The three written forms of the code map agree with the table on the page.
    table = {0: 0, 1: 1, 2: -1, 3: 0}  # trdm §3.1: 00->0, 01->+1, 10->-1, 11->0
    for c in range(4):
        for form in ("table", "eq", "bits"):
            assert o.code_value(c, form) == table[c], (c, form)


def pin_all_bytes_vs_dense(o):
    allb = np.arange(256, dtype=np.uint8).reshape(16, 16)
    got = o.unpack(allb)
    ref = dense.decode(allb)
    assert np.array_equal(got.astype(np.int64), ref)


def pin_pack_roundtrip(o):
    rng = np.random.default_rng(1234)
    q = rng.integers(-1, 2, size=(7, 52)).astype(np.int8)
    p, inv = o.pack(q)
    assert inv == 0
    assert np.array_equal(o.unpack(p), q)
    # bytes without reserved fields survive unpack -> pack unchanged
    b = rng.integers(0, 256, size=(5, 24), dtype=np.uint8)
    fields = dense.fields(b)
    clean = b.copy()
    clean[(fields == 3).reshape(5, 24, 4).any(axis=-1)] = 0x55
    p2, inv2 = o.pack(o.unpack(clean))
    assert inv2 == 0 and np.array_equal(p2, clean)
    # reserved fields are read as 0, so they come back as 00
    p3, _ = o.pack(o.unpack(np.array([[0xff, 0xe4]], np.uint8)))
    assert p3.tolist() == [[0x00, 0x24]]


def pin_pack_invalid(o):
    q = np.array([[1, 2, -1, -3, 0, 5, 1, 1]], np.int8)
    p, inv = o.pack(q)
    assert inv == 3
    assert o.unpack(p).tolist() == [[1, 0, -1, 0, 0, 0, 1, 1]]


def pin_reserved_census(o):
    assert o.count_reserved(np.array([0xff, 0x03, 0x00, 0xe4], np.uint8)) == 6


# ---------------------------------------------------------------- number formats

def pin_f16_decoder(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decoder(o):
    bits = np.arange(65536, dtype=np.uint32)
    got = o.bf16_to_f64(bits.astype(np.uint16))
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen quietly
        ref = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- linear: closed forms

def _pack_const(o, N, K, v):
    p, _ = o.pack(np.full((N, K), v, np.int8))
    return p


def _ints_bf16(rng, M, K, lo=-8, hi=9):
    xi = rng.integers(lo, hi, size=(M, K)).astype(np.float64)
    return xi, f64_to_bf16_bits(xi)


GROUPS = (32, 64, 128, 256)  # group sizes the GPU library takes


def pin_linear_all_zero(o):
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 256
    _, x = _ints_bf16(rng, M, K)
    for g in GROUPS:
        s = f64_to_f16_bits(rng.uniform(0.01, 0.05, size=(N, K // g)))
        for packed in (_pack_const(o, N, K, 0), np.full((N, K // 4), 0xff, np.uint8)):
            y, b = o.linear(x, packed, s, g)
            assert np.all(y == 0.0)
            assert np.all(b > 0.0)


def pin_linear_all_plus_minus(o):
    rng = np.random.default_rng(8)
    M, N, K = 3, 6, 768
    xi, x = _ints_bf16(rng, M, K)
    for g in GROUPS:
        e = rng.integers(-9, -3, size=(N, K // g))
        sv = np.ldexp(1.0, e)  # powers of two: every partial sum is exact in fp64
        s = f64_to_f16_bits(sv)
        # closed form: sum over groups of s[n,g] times the group's sum of x
        gsum = xi.reshape(M, K // g, g).sum(axis=2)          # [M, G]
        expect = gsum @ sv.T                                  # [M, N]
        y, b = o.linear(x, _pack_const(o, N, K, 1), s, g)
        assert np.array_equal(y, expect), g
        y2, _ = o.linear(x, _pack_const(o, N, K, -1), s, g)
        assert np.array_equal(y2, -expect), g
        assert np.array_equal(b, np.abs(xi).reshape(M, K // g, g).sum(axis=2) @ sv.T), g


def pin_linear_per_channel_all_plus(o):
    rng = np.random.default_rng(9)
    M, N, K = 2, 7, 100
    xi, x = _ints_bf16(rng, M, K)
    sv = np.ldexp(1.0, rng.integers(-8, -2, size=N))
    y, _ = o.linear(x, _pack_const(o, N, K, 1), f64_to_f16_bits(sv), -1)
    assert np.array_equal(y, np.outer(xi.sum(axis=1), sv))


def pin_linear_one_hot(o):
    rng = np.random.default_rng(10)
    M, N, K = 2, 4, 256
    xv = rng.standard_normal((M, K))
    x = f64_to_bf16_bits(xv)
    xd = dense.widen_bf16(x)
    for g in GROUPS:
        s = f64_to_f16_bits(rng.uniform(0.005, 0.05, size=(N, K // g)))
        sd = dense.widen_f16(s)
        for k0, sign in ((0, 1), (31, -1), (32, 1), (131, -1), (255, 1)):
            q = np.zeros((N, K), np.int8)
            q[:, k0] = sign
            p, _ = o.pack(q)
            y, _ = o.linear(x, p, s, g)
            # only the scale of the group holding k0 may enter
            assert np.array_equal(y, sign * np.outer(xd[:, k0], sd[:, k0 // g])), (g, k0)


# ---------------------------------------------------------------- linear: invariants

def _random_case(rng, M, N, K, g, dtype="bf16"):
    q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    sv = rng.uniform(0.005, 0.05, size=(N,) if g == -1 else (N, K // g))
    xv = rng.standard_normal((M, K))
    x = f64_to_bf16_bits(xv) if dtype == "bf16" else f64_to_f16_bits(xv)
    return q, f64_to_f16_bits(sv), x


def pin_scale_doubling(o):
    rng = np.random.default_rng(11)
    q, s, x = _random_case(rng, 3, 9, 256, 128)
    p, _ = o.pack(q)
    y1, _ = o.linear(x, p, s, 128)
    s2 = f64_to_f16_bits(2.0 * dense.widen_f16(s))
    y2, _ = o.linear(x, p, s2, 128)
    assert np.array_equal(y2, 2.0 * y1)


def pin_equal_groups_equal_per_channel(o):
    rng = np.random.default_rng(12)
    q, sc, x = _random_case(rng, 2, 5, 512, -1)
    p, _ = o.pack(q)
    yc, bc = o.linear(x, p, sc, -1)
    for g in GROUPS:
        sg = np.repeat(sc.reshape(5, 1), 512 // g, axis=1)
        yg, bg = o.linear(x, p, sg, g)
        assert np.array_equal(yg, yc) and np.array_equal(bg, bc), g


def pin_nested_groups(o):
    """Scales equal on both halves of every 2g-group give the 2g result: the
    group index must be k // g, not some other split of the row."""
    rng = np.random.default_rng(17)
    q, _, x = _random_case(rng, 3, 6, 1024, -1)
    p, _ = o.pack(q)
    for g in GROUPS[:-1]:
        s2 = f64_to_f16_bits(rng.uniform(0.005, 0.05, size=(6, 1024 // (2 * g))))
        s1 = np.repeat(s2, 2, axis=1)
        y1, b1 = o.linear(x, p, s1, g)
        y2, b2 = o.linear(x, p, s2, 2 * g)
        assert np.array_equal(y1, y2) and np.array_equal(b1, b2), g
        # and a different scale on one half changes exactly that half's share
        s1b = s1.copy()
        s1b[:, 1] = f64_to_f16_bits(2.0 * dense.widen_f16(s1[:, 1]))
        y3, _ = o.linear(x, p, s1b, g)
        qd = q.astype(np.float64)
        xd = dense.widen_bf16(x)
        share = xd[:, g:2 * g] @ (qd[:, g:2 * g] * dense.widen_f16(s1[:, 1])[:, None]).T
        assert np.allclose(y3 - y1, share, rtol=0, atol=1e-12 * (1 + np.abs(b1).max())), g


def pin_row_permutation(o):
    rng = np.random.default_rng(13)
    q, s, x = _random_case(rng, 3, 8, 256, 128)
    p, _ = o.pack(q)
    perm = rng.permutation(8)
    y, _ = o.linear(x, p, s, 128)
    yp, _ = o.linear(x, p[perm], s[perm], 128)
    assert np.array_equal(yp, y[:, perm])


def pin_batching(o):
    rng = np.random.default_rng(14)
    q, s, x = _random_case(rng, 4, 6, 384, 128)
    p, _ = o.pack(q)
    y, _ = o.linear(x, p, s, 128)
    for m in range(4):
        ym, _ = o.linear(x[m:m + 1], p, s, 128)
        assert np.array_equal(ym[0], y[m])


def pin_sampled_matches_full(o):
    rng = np.random.default_rng(15)
    q, s, x = _random_case(rng, 3, 10, 256, 128)
    p, _ = o.pack(q)
    y, b = o.linear(x, p, s, 128)
    ms = rng.integers(0, 3, size=20)
    ns = rng.integers(0, 10, size=20)
    ys, bs = o.linear_at(x, p, s, 128, ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(bs, b[ms, ns])


# ---------------------------------------------------------------- brute force

def pin_dense_brute_force(o):
    rng = np.random.default_rng(16)
    for M, N, K in ((1, 1, 4), (2, 3, 128), (4, 16, 256), (3, 5, 132), (2, 4, 96)):
        for g in (-1, 32, 64, 128, 256):
            if g > 0 and K % g:
                continue
            for dtype in ("bf16", "fp16"):
                for raw in (False, True):
                    _, s, x = _random_case(rng, M, N, K, g, dtype)
                    if raw:
                        p = rng.integers(0, 256, size=(N, K // 4), dtype=np.uint8)
                    else:
                        p, _ = o.pack(rng.integers(-1, 2, size=(N, K)).astype(np.int8))
                    y, b = o.linear(x, p, s, g, dtype=dtype)
                    yd, bd = dense.linear(x, p, s, g, dtype=dtype)
                    scale = np.maximum(bd, 1e-300)
                    assert np.all(np.abs(y - yd) <= 1e-12 * scale), (M, N, K, g, dtype, raw)
                    assert np.all(np.abs(b - bd) <= 1e-12 * scale)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
