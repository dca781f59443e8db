"""Every decode GEMV and few-token GEMM kernel instance compiles without
scratch (register spills): these kernels are short-lived bursts of waves, and per-wave
scratch set-up and traffic would cost them directly.  Compiles the decode
sources for gfx950 (device code only) with hipcc's resource-usage remarks."""

import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "gemm_ternary_linear_amd" / "csrc"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
DECODE_SOURCES = ["gemv_f4.hip", "gemv_stream.hip", "gemm_few.hip"]


def _resources(src: str, out_dir: str) -> dict:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "--cuda-device-only", "-c",
           str(CSRC / src), "-o", str(Path(out_dir) / (src + ".o")),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for ln in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs|Occupancy \[waves/SIMD\]): (\d+)", ln)
        if m and name:
            out[name][m.group(1).split()[0]] = int(m.group(2))
    return out


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_decode_kernels_use_no_scratch():
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(3) as ex:
        results = list(ex.map(lambda s: _resources(s, d), DECODE_SOURCES))
    kernels = {k: v for r in results for k, v in r.items() if "kernel" in k}
    assert any("gemv_f4_kernel" in k for k in kernels)
    assert any("gemv_stream_kernel" in k for k in kernels)
    assert any("few_kernel" in k for k in kernels)
    spills = {k: v.get("ScratchSize") for k, v in kernels.items() if v.get("ScratchSize", 0) != 0}
    assert not spills, f"kernel instances with scratch: {spills}"


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_pipelined_gemm_uses_no_scratch():
    # every instance the automatic choice can run (the zero-block-skipping
    # ones, a forced path kept for measurement, are allowed to spill: their
    # group-scaled instances do)
    with tempfile.TemporaryDirectory() as d:
        res = _resources("gemm.hip", d)
    plain = {k: v for k, v in res.items() if "gemm_dma_kernel" in k and k.endswith("Lb0EEEvNS1_8BigBatchE")}
    assert len(plain) >= 26, sorted(plain)
    spills = {k: v.get("ScratchSize") for k, v in plain.items() if v.get("ScratchSize", 0) != 0}
    assert not spills, f"pipelined GEMM instances with scratch: {spills}"
