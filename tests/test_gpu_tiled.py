"""The library's tiled code layout on the GPU.

ternary_tile / ternary_untile must reproduce the oracle's layout
(oracle/layout.py, pinned by hand-worked positions) bit for bit.  Every path
that reads tiled codes (both decode GEMVs, the pipelined GEMM, the plain
kernel) is held to the oracle's result on the row-major codes, within
the layer's bound, and a forced path must give the same bits on tiled and on
row-major codes: the layouts differ only in where a kernel finds a byte.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_of, check_within, say, to_dev, widen
from oracle import layout

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


@pytest.mark.parametrize("N,K", [(1, 4), (15, 252), (17, 260), (33, 1028), (64, 512),
                                 (4101, 4096), (300, 18944), (5, 65536)])
def test_tile_and_untile_match_oracle(tl, N, K):
    import torch
    say(f"tile/untile N={N} K={K}")
    rng = np.random.default_rng(N + K)
    packed = synth.draw_bytes(rng, N, K)
    want = layout.tile(packed, N, K)
    got = tl.tile(to_dev(packed, None))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().reshape(-1), want)
    back = tl.untile(to_dev(want, None), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), packed)


def test_tile_overwrites_padding(tl):
    # padding bytes are written (as 0), whatever the output held before
    import torch
    say("tile padding")
    N, K = 17, 260
    packed = synth.draw_bytes(np.random.default_rng(1), N, K)
    out = torch.full((tl.tiled_bytes(N, K),), 0xFF, dtype=torch.uint8, device="cuda:0")
    assert tl.lib().ternary_tile(to_dev(packed, None).data_ptr(), N, K, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), layout.tile(packed, N, K))


# (M, N, K, group, dtype, path): shapes every tiled path takes, with ragged N
# (N % 16 != 0) and K not a multiple of 256 where the path allows it
CASES = [
    (1, 1000, 4096, -1, "bf16", "gemv_f4"),
    (3, 77, 384, 128, "bf16", "gemv_f4"),     # K = 1.5 slabs: half a slab of padding
    (8, 130, 2048, -1, "bf16", "gemv_f4"),
    (2, 50, 1024, 32, "bf16", "gemv_f4"),
    (4, 33, 512, 64, "bf16", "gemv_f4"),
    (5, 40, 768, 256, "bf16", "gemv_f4"),
    (1, 100, 1024, -1, "fp16", "gemv_f4"),
    (2, 61, 1280, 128, "fp16", "gemv_f4"),
    (64, 300, 1024, -1, "bf16", "gemm"),
    (300, 130, 2048, 128, "bf16", "gemm"),
    (17, 64, 512, 64, "bf16", "gemm"),
    (96, 520, 4096, 256, "fp16", "gemm"),
    (1, 200, 4096, -1, "bf16", "gemv_b16"),
    (8, 100, 18944, -1, "bf16", "gemv_b16"),  # the 7B down shape at M = 8 (the F4 LDS is too small)
    (2, 45, 384, 128, "fp16", "gemv_b16"),
    (4, 33, 1024, 64, "bf16", "gemv_b16"),
    (3, 33, 260, -1, "bf16", "simple"),
    (10, 17, 160, 32, "bf16", "simple"),
    (2, 70, 512, 128, "fp16", "simple"),
]


@pytest.mark.parametrize("M,N,K,g,dtype,path", CASES)
def test_tiled_path_matches_oracle_and_rows(tl, M, N, K, g, dtype, path):
    import torch
    say(f"tiled linear {path} M={M} N={N} K={K} g={g} {dtype}")
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
    packed, _ = oracle.pack(codes)
    tiled = layout.tile(packed, N, K)
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K, dtype)
    xd, sd = to_dev(x, _tdt(dtype)), to_dev(scale, torch.float16)
    y_t = tl.linear(xd, to_dev(tiled, None), sd, g, path=path, layout="tiled")
    y_r = tl.linear(xd, to_dev(packed, None), sd, g, path=path)
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, g, dtype=dtype)
    check_within(widen(bits_of(y_t), dtype), y_ref, bound, f"tiled {path}",
                 out_rounding=dtype if K < 256 else None)
    assert np.array_equal(bits_of(y_t), bits_of(y_r)), "tiled and row-major codes differ"


@pytest.mark.parametrize("M,N,K,g", [(1, 40, 4096, -1), (4, 33, 260, -1), (64, 100, 1024, 128),
                                     (9, 48, 384, 128), (2, 20, 4096, 32)])
def test_tiled_auto_path(tl, M, N, K, g):
    # the automatic choice takes a path that reads tiled codes for every shape
    import torch
    say(f"tiled linear auto M={M} N={N} K={K} g={g}")
    rng = np.random.default_rng(M + N + K)
    packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
    scale = synth.draw_scales(rng, N, K, g)
    x = synth.draw_x(rng, M, K)
    y = tl.linear(to_dev(x, torch.bfloat16), to_dev(layout.tile(packed, N, K), None),
                  to_dev(scale, torch.float16), g, layout="tiled")
    torch.cuda.synchronize()
    y_ref, bound = oracle.linear(x, packed, scale, g)
    check_within(widen(bits_of(y), "bf16"), y_ref, bound, "tiled auto",
                 out_rounding="bf16" if K < 256 else None)


def test_tiled_rejects_row_major_only_paths(tl):
    import torch
    say("tiled forced-path rejections")
    s = torch.ones(16, dtype=torch.float16, device="cuda:0")
    x2 = torch.zeros((64, 384), dtype=torch.bfloat16, device="cuda:0")
    t2 = torch.zeros(tl.tiled_bytes(16, 384), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(tl.TernaryError) as e:
        tl.linear(x2, t2, s, -1, path="gemm", layout="tiled")
    assert e.value.status == -8


def _layer(tl, cfg, M):
    """The projections of a config with device row-major and tiled codes."""
    import torch
    out = []
    for si, shp in enumerate(synth.CONFIGS[cfg].shapes):
        case = synth.make_case(cfg, si, M)
        pd = tl.pack(to_dev(case.codes, None))
        out.append((case, to_dev(case.x, torch.bfloat16), pd, tl.tile(pd),
                    to_dev(case.scale, torch.float16)))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [1, 8])
def test_7b_layer_batch_tiled_equals_rows(tl, M):
    # the fused decode launch at the 7B layer's full size: tiled codes give
    # the bits row-major codes give (both launches plan the same parts), and
    # mixing layouts in one batch changes nothing
    import torch
    say(f"7B layer batch tiled vs rows M={M}")
    lay = _layer(tl, 2, M)
    g = synth.CONFIGS[2].group_size
    rows = tl.linear_batch([(x, p, s, g, None) for _, x, p, _, s in lay])
    tiled = tl.linear_batch([(x, t, s, g, None, "tiled") for _, x, _, t, s in lay])
    mixed = tl.linear_batch([(x, t if i % 2 else p, s, g, None, "tiled" if i % 2 else "rows")
                             for i, (_, x, p, t, s) in enumerate(lay)])
    torch.cuda.synchronize()
    for i, (a, b, c) in enumerate(zip(rows, tiled, mixed)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i
        assert torch.equal(a.view(torch.int16), c.view(torch.int16)), i
    # and the tiled outputs against the oracle on sampled channels
    rng = np.random.default_rng(M)
    for i, ((case, *_), y) in enumerate(zip(lay, tiled)):
        N = case.codes.shape[0]
        rows_ = np.sort(rng.choice(N, size=min(N, 48), replace=False))
        packed, _ = oracle.pack(case.codes[rows_])
        sc = case.scale[rows_]
        y_ref, bound = oracle.linear(case.x, packed, sc, g)
        check_within(widen(bits_of(y), "bf16")[:, rows_], y_ref, bound, f"7B tiled {i}")


def test_prefill_batch_tiled_equals_rows(tl):
    # the grouped GEMM launch (split K over several workgroups at these
    # sizes): tiled and row-major codes give the same bits
    import torch
    say("prefill batch tiled vs rows")
    rng = np.random.default_rng(77)
    specs = [(256, 512, 2048, -1), (256, 1024, 4096, -1), (128, 640, 1024, 128)]
    probs = []
    for M, N, K, g in specs:
        packed, _ = oracle.pack(synth.draw_codes(rng, N, K, 0.3, 0.3))
        scale = synth.draw_scales(rng, N, K, g)
        x = synth.draw_x(rng, M, K)
        pd = to_dev(packed, None)
        probs.append((x, packed, scale, g, to_dev(x, torch.bfloat16), pd, tl.tile(pd),
                      to_dev(scale, torch.float16)))
    rows = tl.linear_batch([(xd, pd, sd, g, None) for _, _, _, g, xd, pd, _, sd in probs])
    tiled = tl.linear_batch([(xd, td, sd, g, None, "tiled") for _, _, _, g, xd, _, td, sd in probs])
    noalloc = tl.linear_batch([(xd, td, sd, g, None, "tiled") for _, _, _, g, xd, _, td, sd in probs],
                              noalloc=True)
    torch.cuda.synchronize()
    for i, (a, b, c) in enumerate(zip(rows, tiled, noalloc)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i
        assert torch.equal(a.view(torch.int16), c.view(torch.int16)), i
    for i, ((x, packed, scale, g, *_), y) in enumerate(zip(probs, tiled)):
        y_ref, bound = oracle.linear(x, packed, scale, g)
        check_within(widen(bits_of(y), "bf16"), y_ref, bound, f"prefill tiled {i}")


def test_tiled_graph_replays(tl):
    import torch
    say("tiled batch under graph capture")
    lay = _layer(tl, 2, 1)
    g = synth.CONFIGS[2].group_size
    outs = [torch.empty((1, c.codes.shape[0]), dtype=torch.bfloat16, device="cuda:0")
            for c, *_ in lay]
    probs = [(x, t, s, g, o, "tiled") for (_, x, _, t, s), o in zip(lay, outs)]
    eager = [y.clone() for y in tl.linear_batch(probs)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        tl.linear_batch(probs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        tl.linear_batch(probs)
    for rep in range(3):
        for o in outs:
            o.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), (rep, i)
    del graph
