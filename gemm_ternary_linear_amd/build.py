"""Build the gfx950 HIP libraries in-tree (hipcc, no GPU needed): libternary.so
(the layer) and libternary_probe.so (measurement probes, used by the bench and
its tests only)."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libternary.so"
PROBE_LIB = PKG / "libternary_probe.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    # packed fp32 VALU forms stay off: all fp32 math is emitted as scalar ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemv_f4.hip", "gemv_stream.hip", "gemv_valu.hip",
           "gemm_few.hip", "gemm.hip", "simple.hip", "noalloc.hip", "workspace.hip", "quantize.hip"]
PROBE_SOURCES = ["probe.hip"]


def _compile(src: str) -> Path:
    obj = BUILD / (Path(src).stem + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out: Path) -> None:
    tmp = out.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4, 8)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB.name}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
