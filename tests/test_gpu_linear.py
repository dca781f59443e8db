"""GPU ternary_linear against the CPU oracle.

Bar: |y_gpu - y_ref| <= 1e-3 * sum_k |x_k| * s(n,k) + 1e-6 for every output
(the stated tolerance; y_ref and the bound are fp64 from the oracle).  The
oracle packs the codes itself; the GPU side packs the same codes with its own
kernel, and the bytes are compared bit-exactly first.
"""

import zlib

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


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def _case(rng, M, N, K, g, dtype, raw=False, p0=0.4):
    pm = (1.0 - p0) / 2
    if raw:
        packed = synth.draw_bytes(rng, N, K)
        codes = None
    else:
        codes = synth.draw_codes(rng, N, K, pm, pm)
        packed, _ = oracle.pack(codes)
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, dtype)
    return codes, packed, scale, x


DECODE_KERNELS = ["gemv_f4", "gemv_b16"]


def _run(tl, x, packed, scale, g, dtype, path="auto", codes=None):
    """Run one linear call; a forced decode kernel that does not take the
    shape (TERNARY_ERR_PATH) skips the test."""
    import torch
    if codes is not None:
        p_dev = tl.pack(to_dev(codes, None))
        torch.cuda.synchronize()
        assert np.array_equal(p_dev.cpu().numpy(), packed), "GPU pack differs from the oracle"
    else:
        p_dev = to_dev(packed, None)
    try:
        y = tl.linear(to_dev(x, _tdt(dtype)), p_dev, to_dev(scale, torch.float16), g, path=path)
    except tl.TernaryError as e:
        if e.status == -8 and path in DECODE_KERNELS:
            pytest.skip(f"{path} does not take M={x.shape[0]} K={x.shape[1]} g={g} {dtype}")
        raise
    torch.cuda.synchronize()
    return widen(bits_of(y), dtype)


SMALL = [
    # (M, N, K, group) -- several tiles and a ragged tail in N (and M for GEMM)
    (1, 16, 128, 128), (1, 100, 384, 128), (1, 300, 1024, -1), (2, 33, 256, -1),
    (3, 257, 4096, 128), (5, 64, 2048, -1), (8, 100, 18944, -1), (8, 48, 5120, 128),
    (1, 1, 128, 128), (7, 1030, 640, 128),
    (9, 100, 256, 128), (16, 130, 1024, -1), (64, 257, 384, 128), (130, 129, 1024, -1),
    (256, 64, 512, 128), (200, 300, 2048, -1),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,g", SMALL)
def test_linear_auto_small(tl, M, N, K, g, dtype):
    say(f"linear auto M={M} N={N} K={K} g={g} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr((M, N, K, g, dtype)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, g, dtype)
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    y = _run(tl, x, packed, scale, g, dtype, codes=codes)
    check_within(y, y_ref, bound, f"auto M={M} N={N} K={K} g={g} {dtype}")


# Decode shapes for both decode kernels: K split over up to 8
# waves, parts of uneven length, parts longer than the one-shot length (run
# with a window, per-channel: several window steps, the last one partial; in
# one-shot chunks of near-equal length, grouped), a half slab at
# the end of K, ragged N (a last block of 4 rows), tiny N, and workgroups
# whose last waves hold no block.
STREAM = [
    (1, 40, 20480, 128), (1, 50, 18944, -1), (2, 45, 10240, -1), (2, 77, 6272, 128),
    (1, 4100, 4096, -1), (2, 19, 5248, 128), (1, 600, 3200, 128), (2, 1, 8192, -1),
    (1, 48, 30720, 128), (1, 33, 32768, -1), (2, 20, 16384, 128), (1, 7, 31872, 128),
    # 3..8 tokens (instances of 4 and 8 tokens; parts longer than the one-shot
    # length run as one-shot chunks in turn)
    (3, 100, 4096, -1), (4, 77, 18944, -1), (5, 50, 6272, 128), (8, 4100, 4096, -1),
    (7, 33, 30720, 128), (8, 20, 1024, -1), (6, 40, 5120, -1), (8, 9, 65536, 128),
]


@pytest.mark.parametrize("kernel", DECODE_KERNELS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,g", STREAM)
def test_linear_stream_decode(tl, M, N, K, g, dtype, kernel):
    say(f"linear decode {kernel} M={M} N={N} K={K} g={g} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr(("stream", M, N, K, g, dtype)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, g, dtype)
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    y = _run(tl, x, packed, scale, g, dtype, path=kernel, codes=codes)
    check_within(y, y_ref, bound, f"{kernel} M={M} N={N} K={K} g={g} {dtype}")


@pytest.mark.parametrize("path", ["gemv", "gemm", "simple", *DECODE_KERNELS])
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("g", [128, -1])
def test_forced_paths_agree_with_oracle(tl, path, M, g):
    say(f"linear forced {path} M={M} g={g}")
    rng = np.random.default_rng(1000 + M * 10 + (g > 0))
    N, K = 200, 1536
    codes, packed, scale, x = _case(rng, M, N, K, g, "bf16")
    y_ref, bound = oracle.linear(x, packed, scale, g)
    y = _run(tl, x, packed, scale, g, "bf16", path=path, codes=codes)
    check_within(y, y_ref, bound, f"{path} M={M} g={g}")


@pytest.mark.parametrize("M,N,K", [(1, 5, 132), (3, 300, 4), (2, 70, 1000), (40, 33, 36)])
def test_simple_path_odd_K(tl, M, N, K):
    say(f"linear odd K M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    codes, packed, scale, x = _case(rng, M, N, K, -1, "bf16")
    assert tl.select_path(M, N, K, -1) == "simple"
    y_ref, bound = oracle.linear(x, packed, scale, -1)
    y = _run(tl, x, packed, scale, -1, "bf16", codes=codes)
    # K as small as 4: |y| may reach B, so the bf16 rounding of y is allowed for
    check_within(y, y_ref, bound, f"odd K M={M} N={N} K={K}", out_rounding="bf16")


@pytest.mark.parametrize("path", ["gemv", "gemm", "simple", *DECODE_KERNELS])
@pytest.mark.parametrize("g", [128, -1])
def test_reserved_codes_read_as_zero(tl, path, g):
    say(f"linear random bytes (with 11 codes) {path} g={g}")
    rng = np.random.default_rng(77 + (g > 0))
    M = 3 if path != "gemm" else 40
    _, packed, scale, x = _case(rng, M, 150, 1024, g, "bf16", raw=True)
    assert oracle.count_reserved(packed) > 0
    y_ref, bound = oracle.linear(x, packed, scale, g)
    y = _run(tl, x, packed, scale, g, "bf16", path=path)
    check_within(y, y_ref, bound, f"raw bytes {path} g={g}")


@pytest.mark.parametrize("path", ["gemv", "gemm", "simple", *DECODE_KERNELS])
def test_closed_form_exact(tl, path):
    # All +1 codes, integer activations and power-of-two scales: every partial
    # sum is exact in fp32, so y is exact and must match bit for bit.
    say(f"linear closed form all +1 {path}")
    rng = np.random.default_rng(4)
    M, N, K, g = (20 if path == "gemm" else 4), 48, 512, 128
    xi = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
    x = synth.f64_to_bf16_bits(xi)
    sv = np.ldexp(1.0, rng.integers(-8, -3, size=(N, K // g)))
    s = synth.f64_to_f16_bits(sv)
    packed, _ = oracle.pack(np.ones((N, K), np.int8))
    expect = xi.reshape(M, K // g, g).sum(axis=2) @ sv.T
    y = _run(tl, x, packed, s, g, "bf16", path=path)
    # the exact result is a short dyadic number; bf16 rounding of it is exact
    # only if it fits 8 significant bits, so compare against its bf16 rounding
    assert np.array_equal(y, widen(synth.f64_to_bf16_bits(expect), "bf16"))
    neg, _ = oracle.pack(-np.ones((N, K), np.int8))
    y2 = _run(tl, x, neg, s, g, "bf16", path=path)
    assert np.array_equal(y2, -widen(synth.f64_to_bf16_bits(expect), "bf16"))
    zero = np.zeros((N, K // 4), np.uint8)
    y3 = _run(tl, x, zero, s, g, "bf16", path=path)
    assert np.all(y3 == 0.0)


# y = x0 + x1 exactly (two +1 codes, unit scales), with x1 putting y on a tie
# of the output format, just above or below one, or on none; the expected
# patterns follow from round-to-nearest, ties to even (u = 1 ULP at 1.0):
#   1 + u/2 -> 1 (tie, even down)    1 + 3u/2 -> 1 + 2u (tie, even up)
#   1 + 3u/4 -> 1 + u (above half)   1 + u/4 -> 1 (below half)
#   the two ties negated             2 + u -> 2 (tie at the next binade)
ROUNDING = {  # dtype: (fraction bits, expected output bit patterns)
    "bf16": (7, [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80, 0xBF82, 0x4000, 0x3F80]),
    "fp16": (10, [0x3C00, 0x3C02, 0x3C01, 0x3C00, 0xBC00, 0xBC02, 0x4000, 0x3C00]),
}


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("path", ["gemv", "gemm", "simple", *DECODE_KERNELS])
def test_output_rounding_ties_to_even(tl, path, dtype):
    say(f"linear output rounding {path} {dtype}")
    import torch
    fb, expect = ROUNDING[dtype]
    u = 2.0 ** -fb
    pairs = [(1.0, u / 2), (1.0, 3 * u / 2), (1.0, 3 * u / 4), (1.0, u / 4), (-1.0, -u / 2),
             (-1.0, -3 * u / 2), (2.0, u), (1.0, 0.0)]
    reps = 1 if path.startswith("gemv") else 8      # 8 tokens (GEMV) or 64 (GEMM tiles)
    N, K = 20, 256
    xv = np.zeros((8 * reps, K))
    xv[:, 0] = [a for a, _ in pairs] * reps
    xv[:, 1] = [b for _, b in pairs] * reps
    to_bits = synth.f64_to_bf16_bits if dtype == "bf16" else synth.f64_to_f16_bits
    x = to_bits(xv)
    assert np.array_equal(widen(x, dtype), xv)  # every activation is exact
    codes = np.zeros((N, K), np.int8)
    codes[:, :2] = 1
    packed, _ = oracle.pack(codes)
    scale = synth.f64_to_f16_bits(np.ones(N))
    y = tl.linear(to_dev(x, _tdt(dtype)), to_dev(packed, None), to_dev(scale, torch.float16),
                  -1, path=path)
    torch.cuda.synchronize()
    got = bits_of(y)
    want = np.repeat(np.array(expect * reps, np.uint16)[:, None], N, axis=1)
    assert np.array_equal(got, want), [hex(v) for v in got[:8, 0]]


def test_deterministic(tl):
    say("linear determinism")
    import torch
    rng = np.random.default_rng(8)
    for M in (1, 8, 300):
        codes, packed, scale, x = _case(rng, M, 513, 2048, 128, "bf16")
        xd, pd, sd = to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16)
        a = tl.linear(xd, pd, sd, 128)
        b = tl.linear(xd, pd, sd, 128)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_and_out_argument(tl):
    say("linear M=0 and out=")
    import torch
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    p = torch.zeros((10, 64), dtype=torch.uint8, device="cuda:0")
    s = torch.ones((10, 2), dtype=torch.float16, device="cuda:0")
    y = tl.linear(x, p, s)
    assert tuple(y.shape) == (0, 10)
    rng = np.random.default_rng(9)
    codes, packed, scale, xb = _case(rng, 2, 10, 256, 128, "bf16")
    out = torch.full((2, 10), 7.0, dtype=torch.bfloat16, device="cuda:0")
    r = tl.linear(to_dev(xb, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16),
                  out=out)
    torch.cuda.synchronize()
    assert r.data_ptr() == out.data_ptr()
    y_ref, bound = oracle.linear(xb, packed, scale, 128)
    check_within(widen(bits_of(out), "bf16"), y_ref, bound, "out=")


def test_rejects_through_binding(tl):
    say("binding error paths")
    import torch
    p = torch.zeros((10, 64), dtype=torch.uint8, device="cuda:0")
    s = torch.ones((10, 2), dtype=torch.float16, device="cuda:0")
    x9 = torch.zeros((9, 256), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(tl.TernaryError) as e:
        tl.linear(x9, p, s, path="gemv")
    assert e.value.status == -8
    buf = torch.zeros(4096, dtype=torch.bfloat16, device="cuda:0")
    x = buf[:512].view(2, 256)
    out = buf[:20].view(2, 10)  # output overlapping the activations
    with pytest.raises(tl.TernaryError) as e:
        tl.linear(x, p, s, out=out)
    assert e.value.status == -6


# ---------------------------------------------------------------- full-size configs

FULL = [(c, si, M) for c, cfg in sorted(synth.CONFIGS.items())
        for si in range(len(cfg.shapes)) for M in cfg.Ms]


def _tile_indices(rng, M, N, tn=256, tm=128, per_tile=2):
    """per_tile random outputs in every tn x tm output tile of the GEMM (channel
    tiles of 256 and token tiles of 128 are the largest any configuration
    uses, so every tile and every split-K slice of a tile is represented), plus
    the corners and the centre."""
    ms, ns = [], []
    for m0 in range(0, M, tm):
        for n0 in range(0, N, tn):
            ms.append(rng.integers(m0, min(M, m0 + tm), size=per_tile))
            ns.append(rng.integers(n0, min(N, n0 + tn), size=per_tile))
    edge_m = np.array([0, M - 1, 0, M - 1, M // 2])
    edge_n = np.array([0, 0, N - 1, N - 1, N // 2])
    return np.concatenate(ms + [edge_m]), np.concatenate(ns + [edge_n])


@pytest.mark.parametrize("cfg,si,M", FULL, ids=[f"c{c}-{synth.CONFIGS[c].shapes[s].name}-M{m}"
                                                for c, s, m in FULL])
def test_full_size(tl, cfg, si, M):
    """Every config case at its full size on the automatic path: all outputs
    against the oracle for M <= 64 (the oracle evaluates those in seconds),
    outputs sampled by output tile beyond."""
    import torch
    case = synth.make_case(cfg, si, M)
    shp = case.shape
    g = case.group_size
    say(f"full config {cfg} {shp.name} N={shp.N} K={shp.K} M={M} g={g} "
        f"path={tl.select_path(M, shp.N, shp.K, g)}")
    packed, _ = oracle.pack(case.codes)
    p_dev = tl.pack(to_dev(case.codes, None))
    y = tl.linear(to_dev(case.x, torch.bfloat16), p_dev, to_dev(case.scale, torch.float16), g)
    torch.cuda.synchronize()
    assert np.array_equal(p_dev.cpu().numpy(), packed)
    yv = widen(bits_of(y), "bf16")
    assert np.all(np.isfinite(yv))
    if M <= 64:
        y_ref, bound = oracle.linear(case.x, packed, case.scale, g)
        check_within(yv, y_ref, bound, f"config {cfg} {shp.name} M={M} (all outputs)")
    else:
        rng = np.random.default_rng(cfg * 100 + si * 10 + M)
        ms, ns = _tile_indices(rng, M, shp.N)
        y_ref, bound = oracle.linear_at(case.x, packed, case.scale, g, ms, ns)
        check_within(yv[ms, ns], y_ref, bound, f"config {cfg} {shp.name} M={M} (tile samples)")


# Prefill shapes, per-channel, M >= 256, N >= 1024.  K % 256 == 0 runs the
# DMA-pipelined kernel: ragged token and channel tiles, N % 4 != 0 (element
# stores instead of 8-byte stores), exact tile multiples, and M = 2048 (eight
# token tiles: the XCD-ordered tile walk).  K = 640 and K = 128 run the
# 128 x 128 kernel.
BIG = [(300, 1100, 768), (260, 1030, 256), (512, 1024, 1280), (257, 1027, 512),
       (2048, 1040, 256), (300, 1100, 640), (257, 1027, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", BIG)
def test_linear_gemm_large_tiles(tl, M, N, K, dtype):
    say(f"linear large-tile gemm M={M} N={N} K={K} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr(("big", M, N, K, dtype)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, -1, dtype)
    assert tl.select_path(M, N, K, -1) == "gemm"
    y_ref, bound = oracle.linear(x, packed, scale, -1, dtype=dtype)
    y = _run(tl, x, packed, scale, -1, dtype, codes=codes)
    check_within(y, y_ref, bound, f"big M={M} N={N} K={K} {dtype}",
                 out_rounding=dtype if K < 256 else None)


# Prefill shapes with too few 256x128 tiles for the CUs: the K range is split
# over several workgroups (8, 4 and 16 slices here) that store fp32 partial
# tiles, and a second kernel adds them in slice order.  Ragged tiles, tile
# counts that do and do not split over the 8 XCDs, both dtypes; every call is
# repeated (once on another stream, with its own workspace) to check that the
# result is bit-identical.
SPLIT = [(256, 256, 4096), (300, 520, 2048), (512, 1024, 8192)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", SPLIT)
def test_linear_gemm_split_k(tl, M, N, K, dtype):
    import torch
    say(f"linear split-K gemm M={M} N={N} K={K} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr(("splitk", M, N, K, dtype)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, -1, dtype)
    y_ref, bound = oracle.linear(x, packed, scale, -1, dtype=dtype)
    xd, pd, sd = to_dev(x, _tdt(dtype)), to_dev(packed, None), to_dev(scale, torch.float16)
    y1 = tl.linear(xd, pd, sd, -1)
    y2 = tl.linear(xd, pd, sd, -1)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y3 = tl.linear(xd, pd, sd, -1)
    side.synchronize()
    torch.cuda.synchronize()
    b1, b2, b3 = (bits_of(t) for t in (y1, y2, y3))
    assert np.array_equal(b1, b2) and np.array_equal(b1, b3), "split-K result not repeatable"
    check_within(widen(b1, dtype), y_ref, bound, f"split-K M={M} N={N} K={K} {dtype}")


def test_workspace_shutdown_and_regrow(tl):
    # ternary_shutdown frees the per-stream workspaces after their streams
    # drain; the next split-K call allocates again, and a larger problem grows
    # the workspace; every result keeps its bits.
    import torch
    say("workspace shutdown / regrow")
    rng = np.random.default_rng(7)
    small = _case(rng, 256, 256, 4096, -1, "bf16")
    large = _case(rng, 512, 1024, 8192, -1, "bf16")
    dev = [(to_dev(x, torch.bfloat16), to_dev(p, None), to_dev(s, torch.float16))
           for (_, p, s, x) in (small, large)]
    first = [bits_of(tl.linear(*d, -1)) for d in dev]
    tl.shutdown()
    again_small = bits_of(tl.linear(*dev[0], -1))
    again_large = bits_of(tl.linear(*dev[1], -1))  # grows the fresh workspace
    tl.shutdown()
    tl.shutdown()  # nothing left to free: still fine
    last = bits_of(tl.linear(*dev[1], -1))
    torch.cuda.synchronize()
    assert np.array_equal(first[0], again_small)
    assert np.array_equal(first[1], again_large) and np.array_equal(first[1], last)
    y_ref, bound = oracle.linear(small[3], small[1], small[2], -1, dtype="bf16")
    check_within(widen(first[0], "bf16"), y_ref, bound, "workspace small")


# Group-128 prefill shapes on the pipelined kernel (K % 256 == 0): the group
# sums fold with the two scales of each 4-step round.  Ragged tiles, config 1
# at M=64, config 4's down shape at M=16 (K split over many slices), a split
# small problem, both dtypes.  A scale array that is only 2-byte aligned runs
# the 128x128 kernel instead and must give the same bound.
GROUPED_BIG = [(300, 1100, 768), (64, 3072, 1024), (256, 300, 2048), (16, 5120, 25600),
               (130, 257, 256)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", GROUPED_BIG)
def test_linear_gemm_grouped_pipelined(tl, M, N, K, dtype):
    import torch
    say(f"linear grouped pipelined gemm M={M} N={N} K={K} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr(("gbig", M, N, K, dtype)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, 128, dtype)
    y_ref, bound = oracle.linear(x, packed, scale, 128, dtype=dtype)
    xd, pd = to_dev(x, _tdt(dtype)), to_dev(packed, None)
    sd = to_dev(scale, torch.float16)
    y1 = tl.linear(xd, pd, sd, 128, path="gemm")
    y2 = tl.linear(xd, pd, sd, 128, path="gemm")
    # the same scales at an address that is 2 (mod 4) bytes aligned
    buf = torch.empty(scale.size + 1, dtype=torch.float16, device="cuda:0")
    buf[1:] = sd.reshape(-1)
    sd_odd = buf[1:].view(sd.shape)
    y3 = tl.linear(xd, pd, sd_odd, 128, path="gemm")
    torch.cuda.synchronize()
    b1, b2 = bits_of(y1), bits_of(y2)
    assert np.array_equal(b1, b2), "not repeatable"
    check_within(widen(b1, dtype), y_ref, bound, f"grouped M={M} N={N} K={K} {dtype}")
    check_within(widen(bits_of(y3), dtype), y_ref, bound,
                 f"grouped (2-byte aligned scales) M={M} N={N} K={K} {dtype}")


# Few-token prefill shapes on the pipelined kernel: 16-token (M <= 16) and
# 32-token (M <= 32) tiles of 128 channels 8 stages deep (K % 512 == 0), and
# 64-token tiles (32 < M <= 64, or K % 512 != 0), both scale modes, ragged
# tiles; the GEMM path forced at M = 1 and 8.
SMALLM = [(9, 300, 2048, -1), (32, 1100, 1024, -1), (48, 520, 768, -1), (1, 700, 4096, -1),
          (8, 700, 5120, 128), (33, 200, 1536, 128), (20, 260, 768, 128),
          (13, 300, 1536, 128), (16, 1030, 2048, -1), (24, 129, 2048, 128)]


@pytest.mark.parametrize("M,N,K,g", SMALLM)
def test_linear_gemm_few_tokens(tl, M, N, K, g):
    say(f"linear few-token gemm M={M} N={N} K={K} g={g}")
    rng = np.random.default_rng(zlib.crc32(repr(("fewtok", M, N, K, g)).encode()))
    codes, packed, scale, x = _case(rng, M, N, K, g, "bf16")
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype="bf16")
    y = _run(tl, x, packed, scale, g, "bf16", path="gemm")
    check_within(y, y_ref, bound, f"few-token gemm M={M} N={N} K={K} g={g}")


# Shapes with many more workgroups than the device holds at once (80 slabs
# per block: 10 per wave in the 16-bit kernel, 20 in the fp4 x fp8 kernel,
# run in chunks), every output compared.  Raw random bytes
# (reserved code 11 included) stand in for packed codes.
RING = [(1, 16384, 20480, 128), (1, 16384, 20480, -1), (2, 32768, 10240, -1)]


@pytest.mark.parametrize("kernel", DECODE_KERNELS)
@pytest.mark.parametrize("M,N,K,g", RING)
def test_stream_full_ring(tl, M, N, K, g, kernel):
    say(f"decode full ring {kernel} M={M} N={N} K={K} g={g}")
    rng = np.random.default_rng(zlib.crc32(repr(("ring", M, N, K, g)).encode()))
    packed = synth.draw_bytes(rng, N, K)
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, "bf16")
    yv = _run(tl, x, packed, scale, g, "bf16", path=kernel)
    y_ref, bound = oracle.linear(x, packed, scale, g)
    check_within(yv, y_ref, bound, f"ring {kernel} M={M} N={N} K={K} g={g}")


def test_ternary_linear_entry_point_through_ctypes(tl):
    # the C entry point ternary_linear itself (the binding calls ternary_linear_ex)
    import ctypes
    import torch
    say("ternary_linear through ctypes")
    rng = np.random.default_rng(12)
    for M, N, K, g in ((1, 300, 4096, -1), (3, 200, 2048, 128), (100, 130, 1024, -1)):
        codes, packed, scale, x = _case(rng, M, N, K, g, "bf16")
        xd, pd, sd = to_dev(x, torch.bfloat16), to_dev(packed, None), to_dev(scale, torch.float16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        st = tl.lib().ternary_linear(xd.data_ptr(), 0, M, N, K, pd.data_ptr(), sd.data_ptr(), g,
                                     y.data_ptr(),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == 0
        y_ref, bound = oracle.linear(x, packed, scale, g)
        check_within(widen(bits_of(y), "bf16"), y_ref, bound, f"ternary_linear M={M}")


@pytest.mark.parametrize("kernel,K", [("gemv_b16", 65536), ("gemv_f4", 16384)])
def test_scale_offsets_past_2GiB(tl, kernel, K):
    # groups of 32: 2 GiB of scales, so the last rows' scale offsets pass 2^31
    # bytes; those rows hold +1 / -1 codes with power-of-two scales and x = 1,
    # every other row zero codes and zero scales, so y is exact
    import torch
    say(f"scale offsets past 2 GiB {kernel} K={K}")
    g, ngroups = 32, K // 32
    N = (1 << 31) // (ngroups * 2) + 48
    packed = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda:0")
    scale = torch.zeros((N, ngroups), dtype=torch.float16, device="cuda:0")
    packed[N - 1] = 0x55                  # codes +1
    packed[N - 2] = 0xAA                  # codes -1
    packed[N - 40] = 0x55
    scale[N - 1] = 2.0 ** -4
    scale[N - 2] = 2.0 ** -3
    scale[N - 40] = 2.0 ** -5
    x = torch.ones((1, K), dtype=torch.bfloat16, device="cuda:0")
    y = tl.linear(x, packed, scale, g, path=kernel)
    torch.cuda.synchronize()
    yv = y.float().cpu().numpy()[0]
    assert yv[N - 1] == K * 2.0 ** -4 and yv[N - 2] == -K * 2.0 ** -3 and yv[N - 40] == K * 2.0 ** -5
    mask = np.ones(N, bool)
    mask[[N - 1, N - 2, N - 40]] = False
    assert np.all(yv[mask] == 0.0)
    del packed, scale
    torch.cuda.empty_cache()
