"""The C-ABI library without a GPU: it loads, exports what include/ternary.h
and include/ternary_probe.h declare, and rejects invalid arguments on the
host before any launch.

None of these calls reach the device: every case fails host-side validation
(or is an M == 0 / N == 0 no-op), so the pointers passed are never used.
"""

import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "ternary.h"
PROBE_HEADER = ROOT / "include" / "ternary_probe.h"


@pytest.fixture(scope="module")
def tl():
    import gemm_ternary_linear_amd as tl
    if not tl.LIB_PATH.exists():
        from gemm_ternary_linear_amd import build
        build.build()
    return tl


def declared_functions(headers=(HEADER, PROBE_HEADER)):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"\b(ternary_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_expected(tl):
    assert declared_functions((HEADER,)) == sorted(tl.EXPORTS)
    assert declared_functions((PROBE_HEADER,)) == sorted(tl.PROBE_EXPORTS)


def test_library_exports_every_declared_symbol(tl):
    L, P = tl.lib(), tl.probe_lib()
    for name in declared_functions((HEADER,)):
        assert hasattr(L, name), name
    for name in declared_functions((PROBE_HEADER,)):
        assert hasattr(P, name), name
        assert not hasattr(L, name), f"{name} is a probe: not in the layer's library"


def test_exported_symbols_in_dynamic_table(tl):
    import subprocess
    for path, header in ((tl.LIB_PATH, HEADER), (tl.PROBE_LIB_PATH, PROBE_HEADER)):
        out = subprocess.run(["nm", "-D", "--defined-only", str(path)],
                             capture_output=True, text=True, check=True).stdout
        names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
        for name in declared_functions((header,)):
            assert name in names, (path.name, name)


def test_no_oracle_linkage(tl):
    import subprocess
    out = subprocess.run(["nm", "-D", str(tl.LIB_PATH)], capture_output=True, text=True,
                         check=True).stdout
    assert "oracle" not in out
    ldd = subprocess.run(["ldd", str(tl.LIB_PATH)], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


def test_versions_and_strings(tl):
    assert tl.abi_version() == 7
    assert tl.gemv_max_m() == 8
    for st in range(0, -11, -1):
        s = tl.status_string(st)
        assert s and s != "unknown status"
    assert tl.status_string(-99) == "unknown status"


FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced


def _lin(tl, x=FAKE, dtype=0, M=1, N=16, K=128, p=FAKE * 2, s=FAKE * 3, g=128, y=FAKE * 4, path=0):
    return tl.lib().ternary_linear_ex(x, dtype, M, N, K, p, s, g, y, path, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), -4),
    (dict(g=16), -3),
    (dict(g=512), -3),
    (dict(g=96), -3),
    (dict(g=0), -3),
    (dict(K=0), -2),
    (dict(K=130, g=-1), -2),
    (dict(K=132), -2),           # grouped needs K % group == 0
    (dict(K=160, g=64), -2),
    (dict(K=384, g=256), -2),
    (dict(M=-1), -2),
    (dict(N=-5), -2),
    (dict(M=1 << 25), -2),
    (dict(x=0), -1),
    (dict(p=0), -1),
    (dict(s=0), -1),
    (dict(y=0), -1),
    (dict(x=FAKE + 8), -5),
    (dict(y=FAKE * 4 + 2), -5),
    (dict(p=FAKE * 2 + 1), -5),
    (dict(s=FAKE * 3 + 1), -5),
    (dict(y=FAKE), -6),                       # y == x
    (dict(y=FAKE * 2 + 16), -6),              # y inside packed
    (dict(path=9), -8),
    (dict(M=9, path=1), -8),                  # GEMV takes M <= 8 only
    (dict(K=132, g=-1, path=1), -8),          # fast kernels need K % 128 == 0
    (dict(K=132, g=-1, path=2), -8),
    (dict(M=3, K=256, g=32, path=5), -8),     # 16-bit decode kernel: g = 32 leaves 2 tokens
    (dict(M=5, K=256, g=64, path=5), -8),     # g = 64 leaves 4
    (dict(M=9, path=4), -8),                  # fp4 x fp8 decode kernel: M <= 8
    (dict(K=132, g=-1, path=4), -8),
    (dict(M=9, path=5), -8),
    (dict(path=6), -8),                       # VALU decode kernel: K % 256 == 0
    (dict(M=2, K=256, g=-1, path=6), -8),     # M == 1 only
    (dict(K=256, g=32, path=6), -8),          # groups of 64, 128, 256 only
    (dict(path=7), -8),                       # few-token GEMM: K % 256 == 0
    (dict(path=8), -8),                       # zero-skipping GEMM: K % 256 == 0
    (dict(path=9), -8),
    (dict(M=64, K=384, g=128, path=8), -8),
    (dict(M=64, K=512, g=32, path=8), -8),    # the pipelined kernel's group sizes only
    (dict(M=64, K=512, g=128, s=FAKE * 3 + 2, path=8), -8),
    (dict(M=33, K=256, g=-1, path=7), -8),    # M <= 32
    (dict(M=17, K=1024, g=128, path=7), -8),  # group-128 scales: M <= 16
    (dict(M=9, K=768, g=128, path=7), -8),    # and K >= 1024
    (dict(K=256, g=64, path=7), -8),          # per channel, groups of 128 or 256
    (dict(K=256, g=32, path=7), -8),
    (dict(K=256, g=128, s=FAKE * 3 + 2, path=7), -8),  # group-128 scales 4-byte aligned
    (dict(M=1, K=65792, g=-1, path=7, p=FAKE * 16, s=FAKE * 64, y=FAKE * 128), -8),
    # fp4 x fp8 kernel: 8 tokens of K = 65536 do not fit its LDS (x is 1 MB here)
    (dict(M=8, N=16, K=65536, g=-1, path=4, p=FAKE * 64, s=FAKE * 128, y=FAKE * 256), -8),
    # fp16 activations at g = 64 and M = 5 take 8 matrix passes there (at most 4)
    (dict(M=5, K=256, g=64, dtype=1, path=4), -8),
    # the GEMV takes K <= 65536
    (dict(M=1, K=65664, g=-1, path=1, p=FAKE * 16, s=FAKE * 64, y=FAKE * 128), -8),
    (dict(K=160, g=32, path=2), -8),          # fast kernels need K % 128 == 0
])
def test_linear_rejects(tl, kw, status):
    assert _lin(tl, **kw) == status


@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(M=0, x=0, y=0), dict(N=0, p=0, s=0)])
def test_linear_empty_is_noop(tl, kw):
    assert _lin(tl, **kw) == 0


def test_pack_unpack_reject(tl):
    L = tl.lib()
    assert L.ternary_pack(FAKE, 4, 6, FAKE * 2, None, None) == -2
    assert L.ternary_pack(FAKE, -1, 8, FAKE * 2, None, None) == -2
    assert L.ternary_pack(0, 4, 8, FAKE * 2, None, None) == -1
    assert L.ternary_pack(FAKE + 1, 4, 8, FAKE * 2, None, None) == -5
    assert L.ternary_pack(FAKE, 4, 8, FAKE * 2, FAKE * 3 + 2, None) == -5
    assert L.ternary_pack(FAKE, 4, 64, FAKE + 16, None, None) == -6
    assert L.ternary_pack(FAKE, 0, 64, 0, None, None) == 0
    assert L.ternary_unpack(FAKE, 4, 6, FAKE * 2, None) == -2
    assert L.ternary_unpack(0, 4, 8, FAKE * 2, None) == -1
    assert L.ternary_unpack(FAKE, 4, 8, FAKE * 2 + 4, None) == -5
    assert L.ternary_unpack(FAKE, 4, 64, FAKE - 16, None) == -6
    assert L.ternary_unpack(FAKE, 4, 0, 0, None) == 0


def test_quantize_reject(tl):
    L = tl.lib()
    W, P, S = FAKE, FAKE * 4, FAKE * 8
    assert L.ternary_quantize(W, 2, 4, 128, 64, P, S, None) == -4      # dtype
    assert L.ternary_quantize(W, 0, 4, 128, 48, P, S, None) == -3      # group size
    assert L.ternary_quantize(W, 0, 4, 6, -1, P, S, None) == -2        # K % 4
    assert L.ternary_quantize(W, 0, 4, 96, 64, P, S, None) == -2       # K % g
    assert L.ternary_quantize(W, 0, -1, 128, 64, P, S, None) == -2
    assert L.ternary_quantize(0, 0, 4, 128, 64, P, S, None) == -1
    assert L.ternary_quantize(W, 0, 4, 128, 64, 0, S, None) == -1
    assert L.ternary_quantize(W, 0, 4, 128, 64, P, 0, None) == -1
    assert L.ternary_quantize(W + 8, 0, 4, 128, 64, P, S, None) == -5
    assert L.ternary_quantize(W, 0, 4, 128, 64, P + 4, S, None) == -5
    assert L.ternary_quantize(W, 0, 4, 128, 64, P, S + 1, None) == -5
    assert L.ternary_quantize(W, 1, 4, 128, 64, W + 512, S, None) == -6   # packed inside w
    assert L.ternary_quantize(W, 0, 4, 128, 64, P, W + 16, None) == -6    # scale inside w
    assert L.ternary_quantize(W, 0, 4, 128, 64, P, P + 2, None) == -6     # scale inside packed
    assert L.ternary_quantize(W, 0, 0, 128, 64, 0, 0, None) == 0          # N == 0: no-op


@pytest.mark.parametrize("M,K,g,path", [
    (1, 4096, -1, "gemv"), (8, 4096, 128, "gemv"), (9, 4096, 128, "few"),
    # 9 .. 32 tokens: the few-token GEMM where it takes the shape (K % 256 == 0,
    # per channel or groups of 256, groups of 128 up to 16 tokens), else the GEMM
    (16, 4096, -1, "few"), (12, 4352, 256, "few"), (17, 4096, -1, "few"),
    (32, 18944, -1, "few"), (24, 4352, 256, "few"), (33, 4096, -1, "gemm"),
    (16, 4096, 128, "few"), (17, 4096, 128, "gemm"), (12, 768, 128, "gemm"), (12, 1024, 128, "few"),
    (9, 4096, 64, "gemm"), (9, 384, 128, "gemm"), (16, 65792, -1, "gemm"),
    (2048, 18944, -1, "gemm"), (1, 132, -1, "simple"), (64, 100, -1, "simple"),
    # long K up to 65536 stays on the GEMV at every M <= 8 (measured faster)
    (8, 18944, -1, "gemv"), (4, 25600, 128, "gemv"), (3, 18944, -1, "gemv"),
    (8, 16256, 128, "gemv"), (8, 65536, -1, "gemv"), (1, 65664, -1, "gemm"),
    (0, 128, 128, "gemv"),
    # other group sizes: the GEMV takes M * columns-per-token <= 16
    (2, 4096, 32, "gemv"), (3, 4096, 32, "gemm"), (4, 4096, 64, "gemv"), (5, 4096, 64, "gemm"),
    (8, 4096, 256, "gemv"), (1, 16384, 32, "gemv"), (1, 32768, 32, "gemv"),
    (64, 4096, 256, "gemm"), (1, 160, 32, "simple"),
])
def test_select_path(tl, M, K, g, path):
    if M == 0:
        assert tl.select_path(M, 16, K, g) in ("gemv", "few", "gemm", "simple")
    else:
        assert tl.select_path(M, 16, K, g) == path


def test_select_path_rejects(tl):
    L = tl.lib()
    assert L.ternary_select_path(1, 16, 130, -1) == -2
    assert L.ternary_select_path(1, 16, 256, 16) == -3
    assert L.ternary_select_path(1, 16, 256, 512) == -3
    assert L.ternary_select_path(1, 16, 384, 256) == -2


def _prob(tl, x, p, s, y, M=1, N=16, K=128, g=128):
    return tl.Problem(x, p, s, y, M, N, K, g)


def test_batch_rejects(tl):
    L = tl.lib()
    P = tl.Problem
    ok1 = _prob(tl, FAKE, FAKE * 2, FAKE * 3, FAKE * 4)
    ok2 = _prob(tl, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8)
    arr = (P * 2)(ok1, ok2)
    assert L.ternary_linear_batch(None, 1, 0, None) == -1
    assert L.ternary_linear_batch(arr, 0, 0, None) == -2
    assert L.ternary_linear_batch(arr, 9, 0, None) == -2
    assert L.ternary_linear_batch(arr, 2, 5, None) == -4
    # second output overlaps the first problem's activations
    bad = (P * 2)(ok1, _prob(tl, FAKE * 5, FAKE * 6, FAKE * 7, FAKE + 64))
    assert L.ternary_linear_batch(bad, 2, 0, None) == -6
    # two outputs overlap each other
    bad2 = (P * 2)(ok1, _prob(tl, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 4 + 16))
    assert L.ternary_linear_batch(bad2, 2, 0, None) == -6
    # an invalid member fails the whole batch with its own status
    bad3 = (P * 2)(ok1, _prob(tl, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, K=130, g=-1))
    assert L.ternary_linear_batch(bad3, 2, 0, None) == -2
    bad4 = (P * 2)(ok1, _prob(tl, FAKE * 5, 0, FAKE * 7, FAKE * 8))
    assert L.ternary_linear_batch(bad4, 2, 0, None) == -1
    # all members empty: success without any launch
    empty = (P * 2)(_prob(tl, 0, 0, 0, 0, M=0), _prob(tl, 0, 0, 0, 0, N=0))
    assert L.ternary_linear_batch(empty, 2, 0, None) == 0


def test_probe_rejects(tl):
    L = tl.probe_lib()
    A, B = 1 << 20, 1 << 21   # 16-byte aligned, never dereferenced
    SHAPE, NULL, ALIGN, ALIAS = -2, -1, -5, -6
    assert L.ternary_probe_read(A, 17, 64, A, None) == SHAPE
    assert L.ternary_probe_read(A, -16, 64, A, None) == SHAPE
    assert L.ternary_probe_read(A, 1024, 0, A, None) == SHAPE
    assert L.ternary_probe_read(A, 1024, 65537, A, None) == SHAPE
    assert L.ternary_probe_read(A, 0, 64, None, None) == 0
    assert L.ternary_probe_read(None, 1024, 64, A, None) == NULL
    assert L.ternary_probe_read(A + 4, 1024, 64, A, None) == ALIGN
    assert L.ternary_probe_read_nt(A, 17, 64, A, None) == SHAPE
    assert L.ternary_probe_read_nt(A, 1024, 65537, A, None) == SHAPE
    assert L.ternary_probe_read_nt(A, 0, 64, None, None) == 0
    assert L.ternary_probe_read_nt(None, 1024, 64, A, None) == NULL
    assert L.ternary_probe_read_nt(A + 4, 1024, 64, A, None) == ALIGN
    assert L.ternary_probe_copy(A, B, 24, 64, None) == SHAPE
    assert L.ternary_probe_copy(A, None, 1024, 64, None) == NULL
    assert L.ternary_probe_copy(A, B + 8, 1024, 64, None) == ALIGN
    assert L.ternary_probe_copy(A, A + 512, 1024, 64, None) == ALIAS
    assert L.ternary_probe_copy(A, B, 0, 64, None) == 0
    assert L.ternary_probe_mfma(0, 4, A, None) == SHAPE
    assert L.ternary_probe_mfma(64, 0, A, None) == SHAPE
    assert L.ternary_probe_mfma(64, (1 << 20) + 1, A, None) == SHAPE
    assert L.ternary_probe_mfma(64, 4, None, None) == NULL
    assert L.ternary_probe_mfma(64, 4, A + 2, None) == ALIGN


def test_binding_unpack_rejects_wrong_K(tl):
    # K must be the row length the packed bytes hold; a larger K would read
    # past the buffer, a smaller one would return a wrong flat prefix
    import torch
    p = torch.zeros((3, 16), dtype=torch.uint8)
    for K in (60, 68, 128, 4):
        with pytest.raises(ValueError, match="does not match the packed rows"):
            tl.unpack(p, K)


def _lint(tl, x=FAKE, dtype=0, M=1, N=16, K=256, p=FAKE * 2, s=FAKE * 3, g=-1, y=FAKE * 4, path=0):
    return tl.lib().ternary_linear_tiled(x, dtype, M, N, K, p, s, g, y, path, None)


def test_tiled_bytes(tl):
    L = tl.lib()
    assert L.ternary_tiled_bytes(17, 260) == 4096
    assert L.ternary_tiled_bytes(16, 256) == 1024
    assert L.ternary_tiled_bytes(1, 4) == 1024
    assert L.ternary_tiled_bytes(0, 256) == 0
    assert L.ternary_tiled_bytes(18944, 4096) == 18944 * 1024
    assert L.ternary_tiled_bytes(3, 6) == -2
    assert L.ternary_tiled_bytes(-1, 4) == -2
    assert L.ternary_tiled_bytes(1 << 25, 4) == -2
    assert L.ternary_tiled_bytes(1 << 24, 1 << 24) == -2     # above 2^40 bytes


def test_tile_untile_reject(tl):
    L = tl.lib()
    for fn in (L.ternary_tile, L.ternary_untile):
        assert fn(FAKE, 4, 6, FAKE * 4, None) == -2
        assert fn(FAKE, -1, 8, FAKE * 4, None) == -2
        assert fn(0, 4, 8, FAKE * 4, None) == -1
        assert fn(FAKE, 4, 8, 0, None) == -1
        assert fn(FAKE + 4, 4, 8, FAKE * 4, None) == -5
        assert fn(FAKE, 4, 8, FAKE * 4 + 8, None) == -5
        assert fn(FAKE, 0, 8, 0, None) == 0
    # the tiled buffer (1 KB here) overlaps the row-major one (8 bytes)
    assert L.ternary_tile(FAKE, 4, 8, FAKE - 512, None) == -6        # (packed, ..., tiled)
    assert L.ternary_tile(FAKE + 1008, 4, 8, FAKE, None) == -6
    assert L.ternary_untile(FAKE - 512, 4, 8, FAKE, None) == -6      # (tiled, ..., packed)
    assert L.ternary_untile(FAKE, 4, 8, FAKE + 1008, None) == -6


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), -4),
    (dict(g=16), -3),
    (dict(K=130), -2),
    (dict(x=0), -1),
    (dict(p=0), -1),
    (dict(p=FAKE * 2 + 4), -5),
    # y overlaps the tiled codes beyond the row-major size (16 x 256 -> 1 KB
    # either way; 17 rows -> 2 KB tiled against 1088 bytes row-major)
    (dict(N=17, y=FAKE * 2 + 1536), -6),
    (dict(M=64, K=384, path=2), -8),           # tiled GEMM needs K % 256 == 0
    (dict(M=64, K=512, g=32, path=2), -8),     # and group sizes 64, 128, 256
    (dict(M=9, path=4), -8),
    (dict(path=6), -8),
])
def test_linear_tiled_rejects(tl, kw, status):
    assert _lint(tl, **kw) == status


def test_linear_tiled_empty_is_noop(tl):
    assert _lint(tl, M=0) == 0
    assert _lint(tl, N=0, p=0, s=0) == 0


def test_batch_rejects_unknown_layout(tl):
    L = tl.lib()
    P = tl.Problem
    ok = P(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, 16, 128, 128, 0)
    bad = P(FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, 1, 16, 128, 128, 2)
    assert L.ternary_linear_batch((P * 2)(ok, bad), 2, 0, None) == -2
    # a tiled member's codes count with their tiled size in the overlap checks
    t = P(FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, 1, 17, 256, -1, 1)
    clash = P(FAKE, FAKE * 2, FAKE * 3, FAKE * 6 + 1536, 1, 16, 128, 128, 0)
    assert L.ternary_linear_batch((P * 2)(t, clash), 2, 0, None) == -6
