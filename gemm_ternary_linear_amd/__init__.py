"""Ternary-weight linear layer for MI355X (gfx950): thin binding over libternary.so.

    y = x @ (q * s)^T,  q in {-1, 0, +1} packed 4 codes per byte (2 bits each,
    00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0, first weight in the lowest bits),
    s an fp16 scale per output channel or per group of 32, 64, 128 or 256
    consecutive K weights.

The format is the one stated on trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
(§3.1) and m.nxbn.cn/news/169761 (§2.2); the layer's interface (x, weight,
scale) -> y follows m.nxbn.cn/news/169761 §5.2.

Everything here only marshals arguments: shapes, dtypes and the current HIP
stream are read from torch tensors and passed to the C ABI of
``include/ternary.h``.  Every step of the computation runs in the HIP kernels.
If the library is not built this module raises on first use; there is no
CPU fallback.
"""

from __future__ import annotations

import ctypes
from pathlib import Path

import torch

__all__ = [
    "TernaryError", "lib", "pack", "unpack", "linear", "linear_batch", "select_path", "gemv_max_m",
    "PATHS", "BF16", "FP16", "abi_version", "shutdown", "LIB_PATH", "probe_read", "probe_copy",
    "probe_mfma", "probe_mfma_flops", "probe_lib", "PROBE_LIB_PATH", "quantize",
    "linear_batch_noalloc", "tile", "untile",
    "tiled_bytes", "LAYOUTS",
]

LIB_PATH = Path(__file__).resolve().parent / "libternary.so"
# Measurement probes (include/ternary_probe.h) live in a library of their own.
PROBE_LIB_PATH = Path(__file__).resolve().parent / "libternary_probe.so"

BF16, FP16 = 0, 1
PATHS = {"auto": 0, "gemv": 1, "gemm": 2, "simple": 3, "gemv_f4": 4, "gemv_b16": 5,
         "gemv_valu": 6, "few": 7, "gemm_zskip": 8}
LAYOUTS = {"rows": 0, "tiled": 1}

# Every symbol include/ternary.h declares.
EXPORTS = (
    "ternary_pack", "ternary_unpack", "ternary_linear", "ternary_linear_ex",
    "ternary_linear_batch", "ternary_select_path", "ternary_gemv_max_m",
    "ternary_status_string", "ternary_abi_version", "ternary_shutdown", "ternary_quantize",
    "ternary_linear_batch_noalloc", "ternary_tile", "ternary_untile", "ternary_tiled_bytes",
    "ternary_linear_tiled",
)
# Every symbol include/ternary_probe.h declares (measurement probes).
PROBE_EXPORTS = ("ternary_probe_read", "ternary_probe_read_nt", "ternary_probe_copy",
                 "ternary_probe_mfma")
MAX_BATCH = 8
PROBE_THREADS = 256


class Problem(ctypes.Structure):
    """ternary_problem of include/ternary.h."""
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("group_size", ctypes.c_int64),
                ("layout", ctypes.c_int64)]

_lib = None


class TernaryError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(str(LIB_PATH))
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.ternary_pack.argtypes = [p, i64, i64, p, p, p]
    L.ternary_unpack.argtypes = [p, i64, i64, p, p]
    L.ternary_linear.argtypes = [p, i32, i64, i64, i64, p, p, i64, p, p]
    L.ternary_linear_ex.argtypes = [p, i32, i64, i64, i64, p, p, i64, p, i32, p]
    L.ternary_linear_tiled.argtypes = [p, i32, i64, i64, i64, p, p, i64, p, i32, p]
    L.ternary_tile.argtypes = [p, i64, i64, p, p]
    L.ternary_untile.argtypes = [p, i64, i64, p, p]
    L.ternary_tiled_bytes.argtypes = [i64, i64]
    L.ternary_tiled_bytes.restype = i64
    L.ternary_linear_batch.argtypes = [p, i32, i32, p]
    L.ternary_linear_batch_noalloc.argtypes = [p, i32, i32, p]
    L.ternary_quantize.argtypes = [p, i32, i64, i64, i64, p, p, p]
    L.ternary_select_path.argtypes = [i64, i64, i64, i64]
    L.ternary_status_string.argtypes = [i32]
    L.ternary_status_string.restype = ctypes.c_char_p
    for nm in ("ternary_pack", "ternary_unpack", "ternary_linear", "ternary_linear_ex",
               "ternary_linear_batch", "ternary_select_path", "ternary_gemv_max_m",
               "ternary_abi_version", "ternary_shutdown", "ternary_quantize",
               "ternary_linear_batch_noalloc", "ternary_linear_tiled", "ternary_tile",
               "ternary_untile"):
        getattr(L, nm).restype = i32
    _lib = L
    return L


_probe_lib = None


def probe_lib() -> ctypes.CDLL:
    """The measurement-probe library (bench and its tests only); raises if it
    has not been built."""
    global _probe_lib
    if _probe_lib is not None:
        return _probe_lib
    if not PROBE_LIB_PATH.exists():
        raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build the HIP libraries first")
    L = ctypes.CDLL(str(PROBE_LIB_PATH))
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.ternary_probe_read.argtypes = [p, i64, i32, p, p]
    L.ternary_probe_read_nt.argtypes = [p, i64, i32, p, p]
    L.ternary_probe_copy.argtypes = [p, p, i64, i32, p]
    L.ternary_probe_mfma.argtypes = [i32, i32, p, p]
    for nm in PROBE_EXPORTS:
        getattr(L, nm).restype = i32
    _probe_lib = L
    return L


def status_string(status: int) -> str:
    return lib().ternary_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().ternary_abi_version())


def shutdown() -> None:
    """Free the library's per-stream workspaces (ternary_shutdown)."""
    _check(int(lib().ternary_shutdown()), "ternary_shutdown")


def gemv_max_m() -> int:
    return int(lib().ternary_gemv_max_m())


def select_path(M: int, N: int, K: int, group_size: int) -> str:
    r = int(lib().ternary_select_path(M, N, K, group_size))
    if r < 0:
        raise TernaryError(r, "ternary_select_path")
    return {v: k for k, v in PATHS.items()}[r]


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    """The current HIP stream of t's device (what torch would launch on)."""
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise TernaryError(status, where)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pack(q: torch.Tensor, invalid_count: torch.Tensor | None = None) -> torch.Tensor:
    """int8 [N, K] in {-1,0,1} -> uint8 [N, K/4].  Values outside {-1,0,1} are
    written as 0 and, if ``invalid_count`` (int32 device scalar) is given,
    added to it."""
    _dev(q, "q")
    if q.dtype != torch.int8 or q.dim() != 2:
        raise ValueError("q must be a 2-D int8 tensor")
    N, K = q.shape
    out = torch.empty((N, K // 4), dtype=torch.uint8, device=q.device)
    cnt = None
    if invalid_count is not None:
        _dev(invalid_count, "invalid_count")
        if invalid_count.dtype != torch.int32 or invalid_count.numel() != 1:
            raise ValueError("invalid_count must be a one-element int32 tensor")
        cnt = invalid_count.data_ptr()
    _check(lib().ternary_pack(q.data_ptr(), N, K, out.data_ptr(), cnt, _stream(q)), "ternary_pack")
    return out


def unpack(packed: torch.Tensor, K: int | None = None) -> torch.Tensor:
    """uint8 (or int8 reinterpreted) [N, K/4] -> int8 [N, K].  ``K``, if given,
    must be the row length the packed bytes hold (4 codes per byte)."""
    if packed.dtype == torch.int8:
        packed = packed.view(torch.uint8)
    if packed.dtype != torch.uint8 or packed.dim() != 2:
        raise ValueError("packed must be a 2-D uint8/int8 tensor")
    N = packed.shape[0]
    if K is not None and K != packed.shape[1] * 4:
        raise ValueError(f"K={K} does not match the packed rows ({packed.shape[1]} bytes hold "
                         f"K={packed.shape[1] * 4})")
    K = packed.shape[1] * 4
    _dev(packed, "packed")
    out = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _check(lib().ternary_unpack(packed.data_ptr(), N, K, out.data_ptr(), _stream(packed)),
           "ternary_unpack")
    return out


_ACT = {torch.bfloat16: BF16, torch.float16: FP16}


def tiled_bytes(N: int, K: int) -> int:
    """Bytes of the tiled layout of an [N, K] code matrix (ternary_tiled_bytes)."""
    r = int(lib().ternary_tiled_bytes(N, K))
    if r < 0:
        raise TernaryError(r, "ternary_tiled_bytes")
    return r


def tile(packed: torch.Tensor) -> torch.Tensor:
    """Row-major codes uint8 [N, K/4] -> the library's tiled layout, a uint8
    tensor [ceil(N/16), ceil(K/256), 1024] (one kilobyte per block of 16 rows x
    256 codes; include/ternary.h gives the byte order)."""
    if packed.dtype == torch.int8:
        packed = packed.view(torch.uint8)
    if packed.dtype != torch.uint8 or packed.dim() != 2:
        raise ValueError("packed must be a 2-D uint8/int8 tensor")
    _dev(packed, "packed")
    N, K = packed.shape[0], packed.shape[1] * 4
    out = torch.empty(((N + 15) // 16, (K + 255) // 256, 1024), dtype=torch.uint8,
                      device=packed.device)
    assert out.numel() == tiled_bytes(N, K)
    _check(lib().ternary_tile(packed.data_ptr(), N, K, out.data_ptr(), _stream(packed)),
           "ternary_tile")
    return out


def untile(tiled: torch.Tensor, N: int, K: int) -> torch.Tensor:
    """The inverse of tile(): tiled codes of an [N, K] matrix -> uint8 [N, K/4]."""
    _dev(tiled, "tiled")
    if tiled.dtype != torch.uint8 or tiled.numel() != tiled_bytes(N, K):
        raise ValueError(f"tiled must be uint8 with {tiled_bytes(N, K)} bytes for N={N}, K={K}")
    out = torch.empty((N, K // 4), dtype=torch.uint8, device=tiled.device)
    _check(lib().ternary_untile(tiled.data_ptr(), N, K, out.data_ptr(), _stream(tiled)),
           "ternary_untile")
    return out


def quantize(w: torch.Tensor, group_size: int = 128):
    """bf16/fp16 weights [N, K] -> (packed uint8 [N, K/4], fp16 scales [N] or
    [N, K/group_size]) by ternary_quantize: per group s = max|w| (fp16),
    q = round(w / s) in {-1, 0, +1}."""
    _dev(w, "w")
    dt = _ACT.get(w.dtype)
    if dt is None or w.dim() != 2:
        raise ValueError("w must be a 2-D bfloat16 or float16 tensor")
    N, K = w.shape
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    sshape = (N,) if group_size == -1 else (N, K // group_size if group_size > 0 else 0)
    scale = torch.empty(sshape, dtype=torch.float16, device=w.device)
    _check(int(lib().ternary_quantize(w.data_ptr(), dt, N, K, group_size, packed.data_ptr(),
                                      scale.data_ptr(), _stream(w))), "ternary_quantize")
    return packed, scale


def _check_problem(x, packed, scale, group_size, out, layout="rows"):
    """Shapes/dtypes of one problem checked against each other -> (dt, M, N, K, g, packed, out).
    Row-major codes are [N, K/4]; tiled ones any uint8 tensor of tiled_bytes(N, K)
    bytes, N then being taken from the scale's first dimension."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {tuple(LAYOUTS)}")
    dt = _ACT.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bfloat16 or float16")
    if packed.dtype == torch.int8:
        packed = packed.view(torch.uint8)
    xs, ps, ss = x.shape, packed.shape, scale.shape
    if len(xs) != 2:
        raise ValueError("x must be 2-D [M, K] (flatten leading dimensions first)")
    if scale.dtype != torch.float16:
        raise ValueError("scale must be float16")
    M, K = xs
    if layout == "tiled":
        if packed.dtype != torch.uint8 or not len(ss):
            raise ValueError("tiled codes must be a uint8 tensor; scale gives N")
        N = ss[0]
        if packed.numel() != tiled_bytes(N, K):
            raise ValueError(f"tiled codes hold {packed.numel()} bytes, N={N}, K={K} needs "
                             f"{tiled_bytes(N, K)}")
    else:
        if packed.dtype != torch.uint8 or len(ps) != 2:
            raise ValueError("packed must be a 2-D uint8/int8 tensor")
        N = ps[0]
        if ps[1] * 4 != K:
            raise ValueError(f"packed has {ps[1]} bytes per row, K={K} needs {K // 4}")
    if group_size is None:
        group_size = -1 if len(ss) == 1 else (K // ss[1] if ss[1] else 0)
    if group_size == -1:
        ok = tuple(ss) == (N,)
    else:
        ok = len(ss) == 2 and group_size > 0 and ss[0] == N and ss[1] * group_size == K
    if not ok:
        raise ValueError(f"scale shape {tuple(ss)} does not match N={N}, K={K}, "
                         f"group_size={group_size}")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be contiguous, match x's dtype and have shape [M, N]")
    for t in (x, packed, scale, out):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    return dt, M, N, K, group_size, packed, out


def linear(x: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
           group_size: int | None = None, path: str = "auto",
           out: torch.Tensor | None = None, layout: str = "rows") -> torch.Tensor:
    """y [M, N] = x [M, K] @ (q * s)^T in x's dtype (bf16 or fp16).

    ``scale`` is fp16 [N] (per channel) or [N, K/group_size]; ``group_size`` is
    inferred from its shape when not given.  ``path`` forces a kernel
    ("gemv", "gemm", "simple", "gemv_f4", "gemv_b16"); "auto" picks by M.
    ``layout`` is "rows" (packed [N, K/4]) or "tiled" (packed from tile()).
    Shapes are checked here against each other, so the sizes passed to the C
    ABI match the tensors.
    """
    dt, M, N, K, group_size, packed, out = _check_problem(x, packed, scale, group_size, out,
                                                          layout)
    fn = lib().ternary_linear_tiled if layout == "tiled" else lib().ternary_linear_ex
    st = fn(x.data_ptr(), dt, M, N, K, packed.data_ptr(), scale.data_ptr(), group_size,
            out.data_ptr(), PATHS[path], _stream(x))
    if st:
        raise TernaryError(st, "ternary_linear_tiled" if layout == "tiled" else "ternary_linear")
    return out


def linear_batch(problems, noalloc: bool = False) -> list:
    """Several projections in as few launches as possible (one for all decode
    shapes).  ``problems`` is a sequence of (x, packed, scale, group_size, out)
    tuples, optionally with a sixth element, the layout ("rows" or "tiled");
    group_size and out may be None; returns the outputs.  With
    ``noalloc`` the call goes to ternary_linear_batch_noalloc (split-K scratch
    in the library's static array; no device memory is allocated by the
    library; the outputs are allocated here unless given)."""
    n = len(problems)
    if not 1 <= n <= MAX_BATCH:
        raise ValueError(f"1..{MAX_BATCH} problems per batch")
    arr = (Problem * n)()
    outs = []
    dts = set()
    for i, prob in enumerate(problems):
        x, packed, scale, g, out = prob[:5]
        layout = prob[5] if len(prob) > 5 else "rows"
        dt, M, N, K, g, packed, out = _check_problem(x, packed, scale, g, out, layout)
        dts.add(dt)
        arr[i] = Problem(x.data_ptr(), packed.data_ptr(), scale.data_ptr(), out.data_ptr(),
                         M, N, K, g, LAYOUTS[layout])
        outs.append(out)
    if len(dts) != 1:
        raise ValueError("all problems of a batch share one activation dtype")
    fn = lib().ternary_linear_batch_noalloc if noalloc else lib().ternary_linear_batch
    st = fn(arr, n, dts.pop(), _stream(problems[0][0]))
    if st:
        raise TernaryError(st, "ternary_linear_batch_noalloc" if noalloc else "ternary_linear_batch")
    return outs


def linear_batch_noalloc(problems) -> list:
    """linear_batch through ternary_linear_batch_noalloc."""
    return linear_batch(problems, noalloc=True)


# ---------------------------------------------------------------- probes

def probe_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int,
               nontemporal: bool = False) -> None:
    """Read all bytes of ``buf`` once (ternary_probe_read, or
    ternary_probe_read_nt with non-temporal loads); ``sink`` is a one-element
    int32 device tensor."""
    _dev(buf, "buf")
    _dev(sink, "sink")
    nbytes = buf.numel() * buf.element_size()
    name = "ternary_probe_read_nt" if nontemporal else "ternary_probe_read"
    _check(int(getattr(probe_lib(), name)(buf.data_ptr(), nbytes, workgroups, sink.data_ptr(),
                                          _stream(buf))), name)


def probe_copy(src: torch.Tensor, dst: torch.Tensor, workgroups: int) -> None:
    """Copy ``src`` into ``dst`` (same byte size) with ternary_probe_copy."""
    _dev(src, "src")
    _dev(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    _check(int(probe_lib().ternary_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                              workgroups, _stream(src))),
           "ternary_probe_copy")


def probe_mfma(workgroups: int, iters: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Run the MFMA loop probe; returns its float32 [workgroups * 256] output.
    The launch performs workgroups * 4 * iters * 4 * 16384 flops."""
    n = workgroups * PROBE_THREADS
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    elif out.dtype != torch.float32 or out.numel() < n:
        raise ValueError(f"out must be float32 with at least {n} elements")
    _dev(out, "out")
    _check(int(probe_lib().ternary_probe_mfma(workgroups, iters, out.data_ptr(), _stream(out))),
           "ternary_probe_mfma")
    return out


def probe_mfma_flops(workgroups: int, iters: int) -> int:
    return workgroups * 4 * iters * 4 * 16384
