#!/usr/bin/env python3
"""Benchmark of the ternary linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one decode pass of a 7B-shaped layer: the seven ternary
projections q, k, v, o (4096/512 x 4096), gate, up (18944 x 4096) and down
(4096 x 18944) at M = 1 token, per-channel fp16 scales, bf16 activations,
in one ternary_linear_batch call (one fused decode-GEMV launch).  The codes are
stored in the library's tiled layout (ternary_tile: blocks of 16 rows x 256
codes, one contiguous kilobyte each), the layout a deployment converts its
weights to once at load; the same figures with row-major codes (the pages'
[N, K/4] packing) are reported beside (rows_codes, prefill.rows_value).
Weights rotate over enough copies (>= 1 GiB) that no step finds them in the
256 MB Infinity Cache; inputs are resident in HBM before timing starts.

Printed (one JSON line on stdout):
  value        decode throughput: algorithmic bytes of all timed launches /
               wall time of the timed region (HIP events, synchronised);
  roofline     the decode GEMV kernel (one launch per step): algorithmic bytes
               per launch / its mean launch duration (HIP events on the launch
               stream around the timed replay), against 8 TB/s; `traffic` = HBM bytes per launch from rocprofv3
               FETCH_SIZE/WRITE_SIZE counters (profiles/), or null when the
               kernels changed since those were taken;
  prefill      the same seven projections at M = 2048 tokens (GEMM path), one
               ternary_linear_batch call per step (one grouped GEMM launch):
               TFLOP/s and its own roofline against 2.5 PFLOP/s bf16 MFMA, with
               seven separate calls per step and per-projection launches beside;
  configs      every other (config, shape, M) of the five workloads: per-launch time on
               the automatic path as GB/s and TFLOP/s with both roofline fractions;
  crossover    forced GEMV and GEMM launch times for every swept case the GEMV takes,
               and for config 4 at each M (where the GEMV -> GEMM crossover lies);
  pack         ternary_pack / ternary_unpack throughput on the 18944 x 4096 weight;
  cpu_baseline the CPU oracle (fp64, OpenMP) on the full decode layer at
               M = 1 on this host's cores, same algorithmic bytes.
Algorithmic bytes per launch: N*K/4 (codes) + scales (2N, or N*K/64 grouped)
+ 2*M*K (x) + 2*M*N (y).  Flops per launch: 2*M*N*K.

    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR
digests two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE)
into profiles/gemv_f4_7b_decode_m1_counters.txt (the fused decode launch)
and profiles/gemm_dma_7b_prefill_m2048_counters.txt (the grouped prefill
launch).
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 1 << 30          # weight bytes cycled per rotation (> 256 MB MALL)
COPY_PROBE_BYTES = 512 << 20    # known-size copy kernel used to calibrate counters
COUNTERS = {
    # kernel family -> (file, kernel-name substring, what the launch is)
    "decode": (ROOT / "profiles" / "gemv_f4_7b_decode_m1_counters.txt", "gemv_f4_kernel",
               "the fused decode GEMV launch (all 7 projections of the 7B layer at M=1, "
               "tiled codes)"),
    "prefill": (ROOT / "profiles" / "gemm_dma_7b_prefill_m2048_counters.txt", "gemm_dma_kernel",
                "the grouped prefill GEMM launch (all 7 projections of the 7B layer at "
                "M=2048, tiled codes)"),
}
DECODE_CFG, PREFILL_CFG = 2, 3
PROBE_ITERS = {512: 8192, 1024: 4096, 2048: 2048}   # MFMA loop probe: workgroups -> iters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(N, K, M, g):
    return N * K // 4 + (2 * N if g == -1 else N * K // 64) + 2 * M * K + 2 * M * N


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted((ROOT / "gemm_ternary_linear_amd" / "csrc").glob("*")):
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- device setup

def to_dev(a, dtype=None):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(dtype).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


class Layer:
    """The projections of one config, packed on the GPU (row-major codes, or
    the library's tiled layout), with rotated copies."""

    def __init__(self, tl, cfg_index, M, copies=None, layout="rows"):
        import torch
        import synth
        self.cfg = synth.CONFIGS[cfg_index]
        self.M = M
        self.layout = layout
        self.path = "auto"
        self.g = self.cfg.group_size
        self.shapes = list(self.cfg.shapes)
        self.cases = []
        self.x, self.packed, self.scale, self.y = [], [], [], []
        for si, shp in enumerate(self.shapes):
            case = synth.make_case(cfg_index, si, M)
            q = to_dev(case.codes)
            p = tl.pack(q)
            del q
            if layout == "tiled":
                p = tl.tile(p)
            self.cases.append(case)
            self.packed.append([p])
            self.scale.append([to_dev(case.scale, torch.float16)])
            self.x.append(to_dev(case.x, torch.bfloat16))
            self.y.append(torch.empty((M, shp.N), dtype=torch.bfloat16, device="cuda:0"))
        self.layer_weight_bytes = sum(s.N * s.K // 4 for s in self.shapes)
        R = copies if copies is not None else max(1, math.ceil(ROTATE_BYTES / self.layer_weight_bytes))
        for j in range(len(self.shapes)):
            for _ in range(R - 1):
                self.packed[j].append(self.packed[j][0].clone())
                self.scale[j].append(self.scale[j][0].clone())
        self.copies = R
        torch.cuda.synchronize()

    def launch(self, tl, j, r):
        tl.linear(self.x[j], self.packed[j][r % self.copies], self.scale[j][r % self.copies],
                  self.g, out=self.y[j], layout=self.layout, path=self.path)

    def step(self, tl, r):
        """All projections of the layer in one ternary_linear_batch call."""
        c = r % self.copies
        tl.linear_batch([(self.x[j], self.packed[j][c], self.scale[j][c], self.g, self.y[j],
                          self.layout) for j in range(len(self.shapes))])

    def step_separate(self, tl, r):
        """The same projections as one ternary_linear call each."""
        for j in range(len(self.shapes)):
            self.launch(tl, j, r)

    def bytes_per_launch(self, j):
        s = self.shapes[j]
        return alg_bytes(s.N, s.K, self.M, self.g)

    def flops_per_launch(self, j):
        s = self.shapes[j]
        return 2 * self.M * s.N * s.K


SETTLE_S = 0.05  # --settle-ms


def settle(replay):
    """Run `replay` untimed, synchronising after each call, until SETTLE_S
    seconds have passed.  Under continuous load the device's clocks take some
    tens of milliseconds to settle (the fused decode step measures about 20 us
    over the first few milliseconds from idle and 17.6 us from about 40 ms on),
    so every graph-timed figure is taken after this."""
    import time
    import torch
    t_end = time.perf_counter() + SETTLE_S
    while True:
        replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


def time_region(tl, layer, steps, warmup, separate=False):
    """Wall time of `steps` back-to-back eager steps (events around the region)."""
    import torch
    step = layer.step_separate if separate else layer.step
    for w in range(warmup):
        step(tl, w)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(tl, warmup + i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e-3


_CAPTURE_STREAM = None


def capture_stream():
    """One side stream for every graph capture here: the library keeps a
    split-K workspace per stream and allocates nothing under capture, so each
    capture is preceded by eager calls on this same stream."""
    global _CAPTURE_STREAM
    import torch
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    return _CAPTURE_STREAM


def time_graph_region(tl, layer, steps, warmup, separate=False):
    """Wall time of exactly `steps` steps replayed from one captured HIP graph.

    The graph holds `steps` consecutive steps (weights rotating over the
    copies); it is replayed untimed for SETTLE_S seconds (settle()), then once
    inside the timed region.
    """
    import torch
    step = layer.step_separate if separate else layer.step
    side = capture_stream()
    with torch.cuda.stream(side):  # warm-up on the capture stream (split-K workspaces)
        for w in range(warmup):
            step(tl, w)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(steps):
            step(tl, warmup + i)
    settle(g.replay)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) * 1e-3


def time_per_shape(tl, layer, launches=64, reps=3):
    """Mean duration (s) of one launch of each projection: a graph of
    `launches` back-to-back launches of that projection (rotating copies),
    replayed `reps` times between events on the launch stream, after settle()."""
    import torch
    out = []
    side = capture_stream()
    for j in range(len(layer.shapes)):
        with torch.cuda.stream(side):  # a split-K shape's workspace exists before capture
            layer.launch(tl, j, 0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(launches):
                layer.launch(tl, j, i)
        settle(g.replay)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1) * 1e-3 / (launches * reps))
        del g
    return out


def time_launches(tl, layer, steps):
    """Per-launch durations (s) from an event pair around every launch."""
    import torch
    n = len(layer.shapes)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        for j in range(n):
            evs[i][j][0].record()
            layer.launch(tl, j, 7919 + i)
            evs[i][j][1].record()
    torch.cuda.synchronize()
    return [[a.elapsed_time(b) * 1e-3 for (a, b) in row] for row in evs]


# ---------------------------------------------------------------- counters

def read_counter_csv(d: Path):
    rows = []
    for f in sorted(Path(d).rglob("*counter_collection.csv")):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_pmc(fetch_dir: str, write_dir: str) -> None:
    """Digest two counter runs into one counters file per kernel family: the
    largest-grid dispatch of the family is the fused (decode) or grouped
    (prefill) launch of the layer's seven projections."""
    per = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_counter_csv(Path(d))
        if not rows:
            raise SystemExit(f"no counter_collection.csv under {d}")
        disp = {}
        for r in rows:
            if r.get("Counter_Name") != name:
                continue
            key = r["Dispatch_Id"]
            disp.setdefault(key, [r["Kernel_Name"], int(r.get("Grid_Size", 0)), 0.0])
            disp[key][2] += float(r["Counter_Value"])
        per[name] = disp
    probe = {}
    for name, disp in per.items():
        v = [c for k, _, c in disp.values() if "neg_kernel" in k]
        if not v:
            raise SystemExit(f"{name}: no copy-probe dispatch")
        probe[name] = sum(v) / len(v)
    k_fetch = COPY_PROBE_BYTES / (probe["FETCH_SIZE"] * 1024.0)
    k_write = COPY_PROBE_BYTES / (probe["WRITE_SIZE"] * 1024.0)
    for fam, (path, sub, what) in COUNTERS.items():
        got = {}
        for name, disp in per.items():
            grids = [gs for k, gs, _ in disp.values() if sub in k]
            if not grids:
                raise SystemExit(f"{name}: no {sub} dispatch")
            top = max(grids)
            v = [c for k, gs, c in disp.values() if sub in k and gs == top]
            got[name] = (sum(v) / len(v), len(v), top)
        (f_k, nf, grid), (w_k, nw, _) = got["FETCH_SIZE"], got["WRITE_SIZE"]
        traffic = f_k * 1024.0 * k_fetch + w_k * 1024.0 * k_write
        lines = [
            f"# HBM traffic of {what}",
            "# from two rocprofv3 --pmc runs of bench.py:",
            "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o bench -- \\",
            "#       python3 bench.py --no-cpu --no-sweep --no-rows --steps 10 --warmup 2 --prefill-steps 1 --prefill-warmup 2 --settle-ms 0",
            "#   (the same with --pmc WRITE_SIZE into <W>), then",
            "#   python3 bench.py --summarize-pmc <F> <W>",
            "# Counters read KiB per dispatch (summed over instances); each is scaled by what",
            f"# it reads for a copy kernel of known size (torch.neg over {COPY_PROBE_BYTES >> 20} MiB",
            "# fp32: reads and writes that many bytes).",
            f"source_hash {kernel_source_hash()}",
            f"grid_threads {grid}",
            f"dispatches_fetch {nf}",
            f"dispatches_write {nw}",
            f"fetch_kib_mean {f_k:.3f}",
            f"write_kib_mean {w_k:.3f}",
            f"probe_fetch_kib {probe['FETCH_SIZE']:.3f}",
            f"probe_write_kib {probe['WRITE_SIZE']:.3f}",
            f"fetch_scale {k_fetch:.5f}",
            f"write_scale {k_write:.5f}",
            f"traffic_bytes_per_launch {traffic:.1f}",
        ]
        path.parent.mkdir(exist_ok=True)
        path.write_text("\n".join(lines) + "\n")
        print("\n".join(lines))


MFMA_FILE = ROOT / "profiles" / "gemm_dma_7b_prefill_m2048_mfma.txt"
MFMA_PASSES = (
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
     "SQ_INSTS_VALU_MFMA_MOPS_BF16"),
    ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_INSTS_VALU"),
)


def summarize_mfma(*dirs) -> None:
    """Digest the MFMA/LDS counter runs of bench.py for the grouped prefill GEMM
    launch (largest-grid gemm_dma_kernel dispatch) beside the MFMA loop probe
    (probe_mfma_kernel, whose matrix cores are busy for its whole duration and
    whose flop count is known), which calibrates the counters."""
    vals = {}
    for d in dirs:
        for r in read_counter_csv(Path(d)):
            key = (r["Kernel_Name"], int(r.get("Grid_Size", 0)), r["Dispatch_Id"])
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
            vals[key][r["Counter_Name"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no counter_collection.csv under {dirs}")

    def family(sub):
        keys = [k for k in vals if sub in k[0]]
        if not keys:
            raise SystemExit(f"no {sub} dispatch")
        top = max(k[1] for k in keys)
        keys = [k for k in keys if k[1] == top]
        mean = {}
        for c in {c for k in keys for c in vals[k]}:
            v = [vals[k][c] for k in keys if c in vals[k]]
            mean[c] = (sum(v) / len(v), len(v))
        return top, mean

    g_grid, g = family("gemm_dma_kernel")
    p_grid, pr = family("probe_mfma_kernel")
    lines = [
        "# MFMA and LDS counters of the grouped prefill GEMM launch (all 7 projections of the",
        "# 7B layer at M=2048, one gemm_dma_kernel dispatch) beside the MFMA loop probe",
        "# (probe_mfma_kernel: 4 waves per SIMD, four independent bf16 MFMA chains each,",
        "# no memory traffic), from rocprofv3 --pmc runs of bench.py, one per counter set:",
    ]
    for cs in MFMA_PASSES:
        lines.append(f"#   rocprofv3 --pmc {' '.join(cs)} --output-format csv -d <D> -o bench -- \\")
        lines.append("#       python3 bench.py --no-cpu --no-sweep --no-rows --steps 10 --warmup 2 "
                     "--prefill-steps 1 --prefill-warmup 2 --settle-ms 0")
    lines += [
        "#   python3 bench.py --summarize-mfma <D1> <D2>",
        "# Values are per dispatch (summed over counter instances), mean over the dispatches",
        "# of that launch shape.  mfma_busy_per_gui = SQ_VALU_MFMA_BUSY_CYCLES /",
        "# GRBM_GUI_ACTIVE; mfma_busy_vs_probe divides it by the probe's, i.e. the share of",
        "# the launch's duration in which the matrix cores are as busy as in the probe.",
        "# mfma_flops = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 (checked on the probe, whose",
        "# flops are known).",
        f"source_hash {kernel_source_hash()}",
        f"gemm_grid_threads {g_grid}",
        f"probe_grid_threads {p_grid}",
    ]
    for c in sorted(set(g) | set(pr)):
        gv = g.get(c, (float("nan"), 0))
        pv = pr.get(c, (float("nan"), 0))
        lines.append(f"{c:<32} gemm {gv[0]:>18.1f} (n={gv[1]})   probe {pv[0]:>18.1f} (n={pv[1]})")

    def get(m, c):
        return m[c][0] if c in m else float("nan")

    rg = get(g, "SQ_VALU_MFMA_BUSY_CYCLES") / get(g, "GRBM_GUI_ACTIVE")
    rp = get(pr, "SQ_VALU_MFMA_BUSY_CYCLES") / get(pr, "GRBM_GUI_ACTIVE")
    wg = p_grid // 256
    probe_flops = wg * 4 * 4 * 16384 * PROBE_ITERS.get(wg, 0)
    lines += [
        f"gemm_mfma_busy_per_gui {rg:.4f}",
        f"probe_mfma_busy_per_gui {rp:.4f}",
        f"gemm_mfma_busy_vs_probe {rg / rp:.4f}",
        f"gemm_mfma_flops {512 * get(g, 'SQ_INSTS_VALU_MFMA_MOPS_BF16'):.6e}",
        f"probe_mfma_flops {512 * get(pr, 'SQ_INSTS_VALU_MFMA_MOPS_BF16'):.6e}",
        f"probe_flops_issued {probe_flops:.6e}",
        f"gemm_lds_bank_conflict_per_active "
        f"{get(g, 'SQ_LDS_BANK_CONFLICT') / get(g, 'SQ_LDS_IDX_ACTIVE'):.4f}",
    ]
    MFMA_FILE.parent.mkdir(exist_ok=True)
    MFMA_FILE.write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


VALU_FILE = ROOT / "profiles" / "gemv_f4_7b_decode_m1_valu.txt"
VALU_PASS = ("VALUBusy", "MfmaUtil", "SQ_INSTS_VALU", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY",
             "SQ_ACTIVE_INST_ANY", "SQ_BUSY_CYCLES")


def summarize_valu(d: str) -> None:
    """Digest one --pmc run of bench.py for the fused decode launch (the
    largest-grid gemv_f4_kernel dispatch): how busy its vector ALUs and
    matrix cores are, and how much of a wave's life goes to waiting."""
    vals = {}
    for r in read_counter_csv(Path(d)):
        key = (r["Kernel_Name"], int(r.get("Grid_Size", 0)), r["Dispatch_Id"])
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
        vals[key][r["Counter_Name"]] += float(r["Counter_Value"])
    keys = [k for k in vals if "gemv_f4_kernel" in k[0]]
    if not keys:
        raise SystemExit(f"no gemv_f4_kernel dispatch under {d}")
    top = max(k[1] for k in keys)
    keys = [k for k in keys if k[1] == top]
    mean = {}
    for c in {c for k in keys for c in vals[k]}:
        v = [vals[k][c] for k in keys if c in vals[k]]
        mean[c] = (sum(v) / len(v), len(v))
    lines = [
        "# Vector-ALU and matrix-core activity of the fused decode GEMV launch (all 7",
        "# projections of the 7B layer at M=1, tiled codes, the largest gemv_f4_kernel dispatch), from",
        "#   rocprofv3 --pmc " + " ".join(VALU_PASS) + " --output-format csv -d <D> -o bench -- \\",
        "#       python3 bench.py --no-cpu --no-sweep --no-rows --steps 10 --warmup 2 "
        "--prefill-steps 1 --prefill-warmup 2 --settle-ms 0",
        "#   python3 bench.py --summarize-valu <D>",
        "# VALUBusy and MfmaUtil are rocprofv3's derived percentages of the launch's GPU time;",
        "# wait_share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of the waves' lifetime spent",
        "# waiting on memory), issue_share = SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES.",
        f"source_hash {kernel_source_hash()}",
        f"grid_threads {top}",
    ]
    for c in sorted(mean):
        lines.append(f"{c:<24} {mean[c][0]:>16.4f} (n={mean[c][1]})")

    def get(c):
        return mean[c][0] if c in mean else float("nan")

    lines += [f"wait_share {get('SQ_WAIT_INST_ANY') / get('SQ_WAVE_CYCLES'):.4f}",
              f"issue_share {get('SQ_ACTIVE_INST_ANY') / get('SQ_WAVE_CYCLES'):.4f}"]
    VALU_FILE.parent.mkdir(exist_ok=True)
    VALU_FILE.write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


TRACE_FILE = ROOT / "profiles" / "kernels_7b_decode_prefill_trace.txt"


def summarize_trace(d: str) -> None:
    """Digest a rocprofv3 --kernel-trace --stats run of this script."""
    d = Path(d)
    stats = []
    for f in sorted(d.rglob("*kernel_stats.csv")):
        with open(f, newline="") as fh:
            stats += list(csv.DictReader(fh))
    trace = []
    for f in sorted(d.rglob("*kernel_trace.csv")):
        with open(f, newline="") as fh:
            trace += list(csv.DictReader(fh))
    if not stats or not trace:
        raise SystemExit(f"no kernel_stats/kernel_trace csv under {d}")
    lines = [
        "# rocprofv3 kernel trace of `python3 bench.py --no-cpu --no-sweep --no-rows` (7B decode layer",
        "# at M=1 as one fused ternary_linear_batch launch per step, per-projection launches,",
        "# the 7B prefill layer at M=2048, and the probe kernels), made by:",
        "#   rocprofv3 --kernel-trace --stats --output-format csv -d <D> -o bench -- \\",
        "#       python3 bench.py --no-cpu --no-sweep --no-rows",
        "#   python3 bench.py --summarize-trace <D>",
        f"source_hash {kernel_source_hash()}",
        "",
        "## kernel stats (all dispatches of the run)",
        f"{'calls':>6} {'mean_us':>10} {'min_us':>9} {'max_us':>9}  kernel",
    ]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        nm = r["Name"].replace("(anonymous namespace)::", "")
        short = nm.split("(")[0].replace("void ", "")
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.3f} "
                     f"{float(r['MinNs']) / 1e3:>9.3f} {float(r['MaxNs']) / 1e3:>9.3f}  {short[:90]}")
    lines += ["", "## ternary and probe kernels by launch shape (grid threads x workgroup threads)",
              f"{'calls':>6} {'median_us':>10} {'mean_us':>9}  kernel grid"]
    groups = {}
    for r in trace:
        k = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        if "ternary" not in k and "probe_" not in k:
            continue
        short = k.split("(")[0].replace("void ", "").replace("ternary::", "")
        key = (short, int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1),
               int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for (short, gs, ws), v in sorted(groups.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        v.sort()
        lines.append(f"{len(v):>6} {v[len(v) // 2] / 1e3:>10.3f} {sum(v) / len(v) / 1e3:>9.3f}  "
                     f"{short[:60]} grid={gs} wg={ws}")
    TRACE_FILE.parent.mkdir(exist_ok=True)
    TRACE_FILE.write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


def stored_traffic(family):
    """Traffic per launch from the committed counters of a kernel family
    ("decode", "prefill"), if they were taken on these kernel sources."""
    path = COUNTERS[family][0]
    if not path.exists():
        return None
    kv = {}
    for ln in path.read_text().splitlines():
        if ln and not ln.startswith("#"):
            k, v = ln.split(None, 1)
            kv[k] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def stored_mfma():
    """MFMA busy share of the grouped prefill launch (relative to the MFMA loop
    probe) from the committed counters, if taken on these kernel sources."""
    if not MFMA_FILE.exists():
        return None
    kv = {}
    for ln in MFMA_FILE.read_text().splitlines():
        if ln and not ln.startswith("#"):
            k, v = ln.split(None, 1)
            kv[k] = v.strip()
    if kv.get("source_hash") != kernel_source_hash() or "gemm_mfma_busy_vs_probe" not in kv:
        return None
    return float(kv["gemm_mfma_busy_vs_probe"])


# ---------------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        for ln in Path("/proc/cpuinfo").read_text().splitlines():
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_decode(layer):
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    packed = [oracle.pack(c.codes)[0] for c in layer.cases]
    times, used = [], 0
    for _ in range(3):
        t = 0.0
        for j, c in enumerate(layer.cases):
            t0 = time.perf_counter()
            _, _, used = oracle.linear(c.x, packed[j], c.scale, layer.g, nthreads=threads,
                                       return_threads=True)
            t += time.perf_counter() - t0
        times.append(t)
    t = sorted(times)[1]
    total = sum(layer.bytes_per_launch(j) for j in range(len(layer.shapes)))
    return {"value": round(total / t / 1e9, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "full 7B decode layer (7 projections, M=1, per-channel), fp64 oracle, "
                      "median of 3 runs",
            "seconds_per_layer": round(t, 4)}


def cpu_baseline_prefill(layer, tokens=8):
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    t, used, flops = 0.0, 0, 0
    for j, c in enumerate(layer.cases):
        packed = oracle.pack(c.codes)[0]
        t0 = time.perf_counter()
        _, _, used = oracle.linear(c.x[:tokens], packed, c.scale, layer.g, nthreads=threads,
                                   return_threads=True)
        t += time.perf_counter() - t0
        flops += 2 * tokens * c.shape.N * c.shape.K
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"first {tokens} of the 2048 tokens through all 7 projections, fp64 oracle"}


# ---------------------------------------------------------------- main

def bench_pack(tl):
    import torch
    import synth
    import numpy as np
    N, K = 18944, 4096
    codes = synth.draw_codes(np.random.default_rng(5), N, K, 0.3, 0.3)
    q = to_dev(codes)
    p = tl.pack(q)
    u = tl.unpack(p)
    torch.cuda.synchronize()
    reps = 20
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    for _ in range(reps):
        tl.pack(q)
    e[1].record()
    e[2].record()
    for _ in range(reps):
        tl.unpack(p)
    e[3].record()
    torch.cuda.synchronize()
    nbytes = N * K + N * K // 4
    tp = e[0].elapsed_time(e[1]) * 1e-3 / reps
    tu = e[2].elapsed_time(e[3]) * 1e-3 / reps
    ok = bool(torch.equal(u, q))
    return {"shape": [N, K], "pack_GBps": round(nbytes / tp / 1e9, 1),
            "unpack_GBps": round(nbytes / tu / 1e9, 1), "roundtrip_exact": ok}


def measure_zero_skip(tl, launches=16, reps=3):
    """The zero-skipping pipelined GEMM (path gemm_zskip) against the plain one
    on the 7B gate projection (18944 x 4096) at 2048 tokens, tiled codes: i.i.d.
    codes (the prefill layer's distribution) and the same codes with about half
    of their 64 x 256 or 256 x 256 blocks zeroed.  Mean us per launch of each path, from a
    graph of `launches` launches replayed `reps` times after settle()."""
    import numpy as np
    import torch
    import synth
    N, K, M = 18944, 4096, 2048
    rng = np.random.default_rng(2024)
    codes = synth.draw_codes(rng, N, K, 0.3, 0.3)
    inputs = [("iid", codes)]
    out = {"shape": f"{N}x{K}, M={M}, per-channel, tiled codes"}
    for bn in (64, 256):  # half of the bn x 256 blocks zero (256: the tile height)
        zero = rng.random((N // bn, K // 256)) < 0.5
        sparse = codes.copy()
        sparse[np.repeat(np.repeat(zero, bn, axis=0), 256, axis=1)] = 0
        inputs.append((f"zero_blocks_{bn}x256", sparse))
        out[f"zero_fraction_{bn}x256"] = round(float(zero.mean()), 4)
    scale = to_dev(synth.draw_scales(rng, N, K, -1), torch.float16)
    x = to_dev(synth.draw_x(rng, M, K), torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    side = capture_stream()
    for name, c in inputs:
        t = tl.tile(tl.pack(to_dev(c)))
        res = {}
        for path in ("gemm", "gemm_zskip"):
            def call():
                tl.linear(x, t, scale, -1, out=y, path=path, layout="tiled")
            with torch.cuda.stream(side):
                call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(launches):
                    call()
            settle(g.replay)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[path + "_us"] = round(e0.elapsed_time(e1) * 1e3 / (launches * reps), 2)
            del g
        out[name] = res
        del t
    torch.cuda.empty_cache()
    return out


def sweep_configs(tl, min_rotate=ROTATE_BYTES, max_copies=4096):
    """Every (config, shape, M) of the five workloads that the headline lines do
    not already time (codes in the tiled layout): per-launch time on the automatic path, as GB/s and
    TFLOP/s with both roofline fractions; for every case the GEMV takes, and
    for config 4 at each M, also the forced GEMV and GEMM paths, to place the
    GEMV -> GEMM crossover.

    Timing: the weights of the shape's first case (drawn as for that case; x
    per M from the M's own generator) are copied R times into one allocation,
    R * weight bytes >= 1 GiB where R <= max_copies, and a HIP graph of R
    launches (one per copy), captured after a warm-up on its capture stream,
    is replayed between events on the stream it replays on, after settle()."""
    import torch
    import numpy as np
    import synth
    out, cross = {}, {}
    cap = torch.cuda.Stream()

    def graph_us(fn, R):
        with torch.cuda.stream(cap):
            for r in range(2):
                fn(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for r in range(R):
                fn(r)
        settle(g.replay)
        best = None
        for _ in range(2):
            # the replay runs on the current stream: the events go there too
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / R
            best = t if best is None else min(best, t)
        del g
        return best

    for ci in (0, 1, 2, 4):
        cfg = synth.CONFIGS[ci]
        out[str(ci)] = {}
        for si, shp in enumerate(cfg.shapes):
            ms = [m for m in cfg.Ms if not (ci == 2 and m == 1)]  # M=1 is the headline
            if not ms:
                continue
            case = synth.make_case(ci, si, cfg.Ms[0])
            q = to_dev(case.codes)
            p1 = tl.tile(tl.pack(q))
            del q
            s1 = to_dev(case.scale, torch.float16)
            wbytes = p1.numel() + 2 * s1.numel()
            R = int(min(max_copies, max(1, math.ceil(min_rotate / wbytes))))
            P = p1.unsqueeze(0).expand(R, *p1.shape).contiguous()
            S = s1.unsqueeze(0).expand(R, *s1.shape).contiguous()
            del p1, s1
            res = {}
            for M in ms:
                rng = synth.rng_for(ci, si, M)
                x = to_dev(synth.draw_x(rng, M, shp.K, "bf16"), torch.bfloat16)
                y = torch.empty((M, shp.N), dtype=torch.bfloat16, device="cuda:0")
                b, f = alg_bytes(shp.N, shp.K, M, cfg.group_size), 2 * M * shp.N * shp.K

                def run(path):
                    return graph_us(lambda r: tl.linear(x, P[r], S[r], cfg.group_size,
                                                        path=path, out=y, layout="tiled"), R)

                t = run("auto")
                res[str(M)] = {"path": tl.select_path(M, shp.N, shp.K, cfg.group_size),
                               "us": round(t * 1e6, 3), "GBps": round(b / t / 1e9, 1),
                               "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4),
                               "TFLOPs": round(f / t / 1e12, 2),
                               "mfma_frac": round(f / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "copies": R}
                if ci == 4 or M <= tl.gemv_max_m():
                    c = {"gemm_us": round(run("gemm") * 1e6, 3)}
                    if M <= tl.gemv_max_m():
                        c["gemv_us"] = round(run("gemv") * 1e6, 3)
                    cross.setdefault(f"{ci}:{shp.name}", {})[str(M)] = c
                del x, y
            out[str(ci)][shp.name] = res
            del P, S
            torch.cuda.empty_cache()
            log(f"[bench] config {ci} {shp.name}: {res}")
    return out, cross


# Launch sets profiled on their own (one rocprofv3 run each): config, M, and
# whether the step is one fused batch call or one call per projection.
WORKLOADS = {
    "27b_m16": (4, 16, False), "27b_m64": (4, 64, False), "27b_m256": (4, 256, False),
    "7b_decode_single_m1": (2, 1, False), "7b_decode_fused_m8": (2, 8, True),
    "7b_fused_m16": (2, 16, True), "7b_fused_m32": (2, 32, True),
}
WORKLOAD_REPS = 6


def run_workload(tl, name):
    """Run one launch set of WORKLOADS (tiled codes): the copy probe, then
    WORKLOAD_REPS launches of each projection (or fused steps), after one
    untimed launch each."""
    import torch
    cfg, M, fused = WORKLOADS[name]
    layer = Layer(tl, cfg, M, layout="tiled")
    copy_probe()
    if cfg == 4 or M >= 16:  # MFMA reference for the matrix-core launches' busy counters
        buf = torch.empty(2048 * tl.PROBE_THREADS, dtype=torch.float32, device="cuda:0")
        tl.probe_mfma(2048, PROBE_ITERS[2048], buf)
        torch.cuda.synchronize()
        del buf
    if fused:
        for i in range(WORKLOAD_REPS + 1):
            layer.step(tl, i)
    else:
        for j in range(len(layer.shapes)):
            for i in range(WORKLOAD_REPS + 1):
                layer.launch(tl, j, i)
    torch.cuda.synchronize()
    print(json.dumps({"workload": name, "shapes": [s.name for s in layer.shapes], "M": M,
                      "fused": fused, "reps": WORKLOAD_REPS + 1}))


def summarize_workload(name: str, dirs) -> None:
    """Digest the counter runs of one WORKLOADS entry: per (kernel, grid)
    group of dispatches, in launch order, the mean of each counter; FETCH_SIZE
    and WRITE_SIZE scaled to bytes by the copy probe and set against the
    algorithmic bytes of the projection the group runs."""
    import synth
    cfg, M, fused = WORKLOADS[name]
    shapes = list(synth.CONFIGS[cfg].shapes)
    g = synth.CONFIGS[cfg].group_size
    groups, probe, mprobe = {}, {}, {}
    for d in dirs:
        per = {}
        for r in read_counter_csv(Path(d)):
            key = r["Dispatch_Id"]
            per.setdefault(key, [r["Kernel_Name"], int(r.get("Grid_Size", 0)), {}])
            c = r["Counter_Name"]
            per[key][2][c] = per[key][2].get(c, 0.0) + float(r["Counter_Value"])
        n_main = 0
        for key in sorted(per, key=int):
            kname, grid, vals = per[key]
            if "neg_kernel" in kname:
                for c, v in vals.items():
                    probe.setdefault(c, []).append(v)
                continue
            if "probe_mfma_kernel" in kname:
                for c, v in vals.items():
                    mprobe.setdefault(c, []).append(v)
                continue
            short = kname.replace("(anonymous namespace)::", "").replace("ternary::", "")
            short = re.sub(r"^void ", "", short)
            short = re.sub(r"\(.*$", "", short)
            if not re.search(r"gemv|gemm|simple|few", short):
                continue  # the layer's pack / tile kernels
            # launches run projection by projection, WORKLOAD_REPS + 1 each; a
            # split-K or K-slice reduce belongs to the launch before it
            if "split_reduce" in short or "few_reduce" in short:
                idx = max(n_main - 1, 0) // (WORKLOAD_REPS + 1)
            else:
                idx = n_main // (WORKLOAD_REPS + 1)
                n_main += 1
            label = "fused step" if fused else (shapes[idx].name if idx < len(shapes) else "?")
            grp = groups.setdefault((label, short, grid), {})
            for c, v in vals.items():
                grp.setdefault(c, []).append(v)
    mean = lambda v: sum(v) / len(v)
    k_fetch = COPY_PROBE_BYTES / (mean(probe["FETCH_SIZE"]) * 1024.0)
    k_write = COPY_PROBE_BYTES / (mean(probe["WRITE_SIZE"]) * 1024.0)
    by_name = {s.name: s for s in shapes}
    tot = sum(alg_bytes(s.N, s.K, M, g) for s in shapes)
    lines = [f"# Counters of the launch set '{name}' (config {cfg}, M={M}, tiled codes, "
             f"{'one fused batch call per step' if fused else 'one call per projection'}),",
             "# one rocprofv3 --pmc run per counter set, each of",
             f"#   python3 bench.py --workload {name}",
             "# e.g. rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o bench -- "
             f"python3 bench.py --workload {name}",
             "# (likewise WRITE_SIZE, and for GEMM launches SQ_VALU_MFMA_BUSY_CYCLES "
             "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES), then",
             f"#   python3 bench.py --summarize-workload {name} <F> <W> [<MFMA>]",
             "# Per (kernel, grid) group in launch order: dispatches, mean KiB per dispatch",
             "# mfma_busy_vs_probe: SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE of the group over",
             "# that of the MFMA loop probe (probe_mfma_kernel, run in the same process).",
             "# (summed over instances); traffic = FETCH*fetch_scale + WRITE*write_scale in",
             f"# bytes, the scales from a copy kernel of known size (torch.neg over "
             f"{COPY_PROBE_BYTES >> 20} MiB fp32).",
             f"source_hash {kernel_source_hash()}",
             f"fetch_scale {k_fetch:.5f}", f"write_scale {k_write:.5f}"]
    if fused:
        lines.append(f"alg_bytes_per_step {tot}")
    for k, v in groups.items():
        label, short, grid = k
        n = len(next(iter(v.values())))
        row = [f"[{label}] {short[:70]} grid={grid} n={n}"]
        if "FETCH_SIZE" in v and "WRITE_SIZE" in v:
            f_k, w_k = mean(v["FETCH_SIZE"]), mean(v["WRITE_SIZE"])
            t = f_k * 1024 * k_fetch + w_k * 1024 * k_write
            row.append(f"fetch_kib {f_k:.1f} write_kib {w_k:.1f} traffic_bytes {t:.0f}")
            if label in by_name and "reduce" not in short:
                a = alg_bytes(by_name[label].N, by_name[label].K, M, g)
                row.append(f"alg_bytes {a} traffic/alg {t / a:.3f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v and "GRBM_GUI_ACTIVE" in v:
            busy = mean(v["SQ_VALU_MFMA_BUSY_CYCLES"]) / mean(v["GRBM_GUI_ACTIVE"])
            row.append(f"mfma_busy_per_gui {busy:.3f}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mprobe:
                pb = mean(mprobe["SQ_VALU_MFMA_BUSY_CYCLES"]) / mean(mprobe["GRBM_GUI_ACTIVE"])
                row.append(f"mfma_busy_vs_probe {busy / pb:.3f}")
        lines.append("  ".join(row))
    fam = ("gemv_f4" if M == 1 else "gemv_stream" if M <= 8
           else "gemm_few" if M <= (16 if g == 128 else 32) else "gemm_dma")
    path = ROOT / "profiles" / f"{fam}_{name}_counters.txt"
    path.parent.mkdir(exist_ok=True)
    path.write_text("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_probe():
    """A plain read+write kernel of known size, for counter calibration."""
    import torch
    n = COPY_PROBE_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(2):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def measure_ceilings(tl, layer_bytes, steps):
    """Achievable rates of this device, from the probe kernels of
    include/ternary_probe.h, each at its best launch size from a short list:

    - read_1GiB: one 16-byte-load streaming read of 1 GiB;
    - read_layer_size: `steps` reads of `layer_bytes` each (the decode layer's
      algorithmic bytes), rotating over 1 GiB and replayed from one HIP graph,
      timed like the decode step; read_gate_size: the same at the 18944 x 4096
      projection's bytes (a lone launch of that size);
      both reads with plain and with non-temporal loads (the policy of the
      decode kernels' code loads), the faster one reported, the plain one beside;
    - copy_512MiB: a 512 MiB -> 512 MiB copy (reads plus writes);
    - mfma_loop: four independent bf16 MFMA chains per wave on register
      operands, 1.1e12 flops per launch; cold (the first launches) and
      sustained (after 10 untimed launches)."""
    import torch

    def ev_time(fn, reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(r)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    big = torch.ones(ROTATE_BYTES // 4, dtype=torch.int32, device="cuda:0")
    best = {}
    for nt in (False, True):
        best[nt] = (0.0, None)
        for wg in (1024, 2048, 4096, 8192):
            tl.probe_read(big, sink, wg, nontemporal=nt)
            t = ev_time(lambda r: tl.probe_read(big, sink, wg, nontemporal=nt), 5)
            best[nt] = max(best[nt], (ROTATE_BYTES / t / 1e9, wg), key=lambda b: b[0])
    nt = best[True][0] > best[False][0]
    out["read_1GiB"] = {"GBps": round(best[nt][0], 1), "workgroups": best[nt][1],
                        "loads": "non-temporal" if nt else "plain",
                        "plain_GBps": round(best[False][0], 1),
                        "frac": round(best[nt][0] / HBM_PEAK_GBPS, 4)}

    def graph_read(nbytes):
        """Best streaming read of `nbytes` per launch, `steps` launches rotating
        over 1 GiB in one HIP graph, plain and non-temporal loads."""
        chunk = nbytes // 16 * 4               # int32 elements, 16-byte multiple
        nchunk = big.numel() // chunk
        views = [big[i * chunk:(i + 1) * chunk] for i in range(nchunk)]
        best = {}
        for nt in (False, True):
            best[nt] = (0.0, None)
            for wg in (512, 1024, 2048):
                tl.probe_read(views[0], sink, wg, nontemporal=nt)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(steps):
                        tl.probe_read(views[i % nchunk], sink, wg, nontemporal=nt)
                settle(g.replay)
                t = ev_time(lambda r: g.replay(), 1) / steps
                del g
                best[nt] = max(best[nt], (chunk * 4 / t / 1e9, wg), key=lambda b: b[0])
        nt = best[True][0] > best[False][0]
        return {"GBps": round(best[nt][0], 1), "workgroups": best[nt][1],
                "loads": "non-temporal" if nt else "plain",
                "plain_GBps": round(best[False][0], 1),
                "bytes": chunk * 4, "us": round(chunk * 4 / best[nt][0] / 1e3, 3),
                "frac": round(best[nt][0] / HBM_PEAK_GBPS, 4)}

    out["read_layer_size"] = graph_read(layer_bytes)
    # the 18944 x 4096 projection's bytes at one token: the ceiling of a lone
    # launch of that size, which pays the ramp-up and drain once per launch
    out["read_gate_size"] = graph_read(alg_bytes(18944, 4096, 1, -1))

    half = big.numel() // 2
    src, dst = big[:half], big[half:]
    best = (0.0, None)
    for wg in (1024, 2048, 4096):
        tl.probe_copy(src, dst, wg)
        t = ev_time(lambda r: tl.probe_copy(src, dst, wg), 5)
        best = max(best, (2 * half * 4 / t / 1e9, wg), key=lambda b: b[0])
    out["copy_512MiB"] = {"GBps": round(best[0], 1), "workgroups": best[1],
                          "frac": round(best[0] / HBM_PEAK_GBPS, 4)}
    del src, dst, big

    mf = {}
    for wg, iters in PROBE_ITERS.items():
        buf = torch.empty(wg * tl.PROBE_THREADS, dtype=torch.float32, device="cuda:0")
        flops = tl.probe_mfma_flops(wg, iters)
        torch.cuda.synchronize()
        cold = ev_time(lambda r: tl.probe_mfma(wg, iters, buf), 2)
        for _ in range(10):
            tl.probe_mfma(wg, iters, buf)
        warm = ev_time(lambda r: tl.probe_mfma(wg, iters, buf), 10)
        mf[wg] = (flops / warm / 1e12, flops / cold / 1e12, wg, iters)
        del buf
    sus, cold, wg, iters = max(mf.values(), key=lambda v: v[0])
    out["mfma_loop"] = {"TFLOPs_sustained": round(sus, 1), "TFLOPs_cold": round(cold, 1),
                        "workgroups": wg, "iters": iters,
                        "frac": round(sus / MFMA_BF16_PEAK_TFLOPS, 4)}
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=60,
                    help="untimed prefill steps first (clocks settle under sustained MFMA load)")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed graph replays before each graph-timed figure (clocks settle)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-config sweep (configs 0, 1, 2 at M=8, 4) and the zero-skip timing")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the row-major-codes figures reported beside the tiled ones "
                         "(profiled runs: only tiled launches then)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "LDS_DIR"))
    ap.add_argument("--summarize-valu", metavar="VALU_DIR")
    ap.add_argument("--detail", type=str, default=None, help="write per-shape results here")
    ap.add_argument("--workload", choices=sorted(WORKLOADS),
                    help="run one launch set for counter collection (no timing)")
    ap.add_argument("--summarize-workload", nargs="+", metavar="NAME_AND_DIRS",
                    help="NAME DIR [DIR ...]: digest counter runs of --workload NAME")
    args = ap.parse_args()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle_ms) / 1e3

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_valu:
        summarize_valu(args.summarize_valu)
        return
    if args.summarize_workload:
        summarize_workload(args.summarize_workload[0], args.summarize_workload[1:])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(a sharded layer would split the N rows of each projection across GPUs; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_ternary_linear_amd as tl
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    tl.lib()
    if args.workload:
        run_workload(tl, args.workload)
        return

    log("[bench] building the decode layer (config 2, M=1, tiled codes)")
    dec = Layer(tl, DECODE_CFG, 1, layout="tiled")
    paths = {s.name: tl.select_path(1, s.N, s.K, dec.g) for s in dec.shapes}
    log(f"[bench] decode paths {paths}, {dec.copies} rotated copies")
    copy_probe()

    t_eager = time_region(tl, dec, args.steps, args.warmup)
    t_region = time_graph_region(tl, dec, args.steps, args.warmup)
    t_sep = time_graph_region(tl, dec, args.steps, args.warmup, separate=True)
    step_bytes = sum(dec.bytes_per_launch(j) for j in range(len(dec.shapes)))
    value = step_bytes * args.steps / t_region / 1e9
    eager_value = step_bytes * args.steps / t_eager / 1e9
    sep_value = step_bytes * args.steps / t_sep / 1e9
    log(f"[bench] decode: graph replay {t_region * 1e3:.3f} ms for {args.steps} steps "
        f"= {value:.1f} GB/s; eager {eager_value:.1f} GB/s; seven separate launches "
        f"{sep_value:.1f} GB/s")

    # The step is one fused GEMV launch: its mean duration is the region time
    # over the steps (HIP events on the launch stream around the graph replay).
    mean_dur = t_region / args.steps
    achieved = step_bytes / mean_dur / 1e9
    dur = time_per_shape(tl, dec)
    shapes_out = {}
    for j, s in enumerate(dec.shapes):
        b = dec.bytes_per_launch(j)
        shapes_out[s.name] = {"N": s.N, "K": s.K, "us": round(dur[j] * 1e6, 3),
                              "GBps": round(b / dur[j] / 1e9, 1),
                              "frac": round(b / dur[j] / 1e9 / HBM_PEAK_GBPS, 4)}
    traffic = stored_traffic("decode")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic is None else round(traffic, 1),
                "kernel": "gemv_f4_kernel<bf16, per-channel, M=1>: one fused launch of the "
                          "7 projections, tiled codes",
                "alg_bytes_per_launch": step_bytes,
                "mean_launch_us": round(mean_dur * 1e6, 3)}
    log(f"[bench] decode per-launch {shapes_out}")
    rotated = dec.copies
    del dec
    torch.cuda.empty_cache()
    rows_dec = None
    if not args.no_rows:
        # the same layer with row-major codes (the pages' [N, K/4] packing)
        dr = Layer(tl, DECODE_CFG, 1, layout="rows")
        t_rows = time_graph_region(tl, dr, args.steps, args.warmup)
        dur_r = time_per_shape(tl, dr)
        rows_dec = {"value": round(step_bytes * args.steps / t_rows / 1e9, 1),
                    "frac_of_hbm_peak": round(step_bytes * args.steps / t_rows / 1e9
                                              / HBM_PEAK_GBPS, 4),
                    "mean_launch_us": round(t_rows / args.steps * 1e6, 3),
                    "shapes_us": {s.name: round(dur_r[j] * 1e6, 3)
                                  for j, s in enumerate(dr.shapes)}}
        log(f"[bench] decode with row-major codes {rows_dec}")
        # the vector-ALU decode GEMV (add/sub per code, cross-lane reduction)
        # on the same projections, one launch each
        dr.path = "gemv_valu"
        dur_v = time_per_shape(tl, dr)
        rows_dec["valu_gemv_us"] = {s.name: round(dur_v[j] * 1e6, 3)
                                    for j, s in enumerate(dr.shapes)}
        rows_dec["valu_gemv_sum_us"] = round(sum(dur_v) * 1e6, 3)
        rows_dec["f4_gemv_sum_us"] = round(sum(dur_r) * 1e6, 3)
        log(f"[bench] VALU decode GEMV per launch {rows_dec['valu_gemv_us']}")
        del dr
        torch.cuda.empty_cache()

    log("[bench] building the prefill layer (config 3, M=2048, tiled codes)")
    pre = Layer(tl, PREFILL_CFG, 2048, copies=2, layout="tiled")
    pre_flops = sum(pre.flops_per_launch(j) for j in range(len(pre.shapes)))
    # One step = one ternary_linear_batch call = one grouped GEMM launch (the
    # layer has enough tiles that no K range is split): events on the launch
    # stream around the steps give the launch's mean duration.
    t_pre = time_region(tl, pre, args.prefill_steps, args.prefill_warmup)
    pre_value = pre_flops * args.prefill_steps / t_pre / 1e12
    t_pre_sep = time_region(tl, pre, args.prefill_steps, args.prefill_warmup, separate=True)
    pre_sep_value = pre_flops * args.prefill_steps / t_pre_sep / 1e12
    per_p = time_launches(tl, pre, args.prefill_steps)
    dur_p = [sum(per_p[i][j] for i in range(args.prefill_steps)) / args.prefill_steps
             for j in range(len(pre.shapes))]
    pre_shapes = {}
    for j, s in enumerate(pre.shapes):
        f = pre.flops_per_launch(j)
        pre_shapes[s.name] = {"N": s.N, "K": s.K, "us": round(dur_p[j] * 1e6, 2),
                              "TFLOPs": round(f / dur_p[j] / 1e12, 1),
                              "frac": round(f / dur_p[j] / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    mean_pre = t_pre / args.prefill_steps
    ach_p = pre_flops / mean_pre / 1e12
    traffic_p = stored_traffic("prefill")
    prefill = {
        "metric": "ternary_linear TFLOP/s at M=2048 (7B prefill layer, per-channel)",
        "value": round(pre_value, 1), "unit": "TFLOP/s",
        "frac_of_mfma_peak": round(pre_value / MFMA_BF16_PEAK_TFLOPS, 4),
        "ms_per_layer": round(mean_pre * 1e3, 4),
        "timing": f"eager, {args.prefill_warmup} untimed steps first (sustained clocks), one "
                  "ternary_linear_batch call per step (one grouped GEMM launch); seven separate "
                  "calls per step and per-projection launches beside",
        "separate_launches_value": round(pre_sep_value, 1),
        "path": tl.select_path(2048, 4096, 4096, -1),
        "roofline": {"bound": "mfma", "achieved": round(ach_p, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach_p / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if traffic_p is None else round(traffic_p, 1),
                     "mfma_busy_vs_probe": stored_mfma(),
                     "kernel": "gemm_dma_kernel<bf16, per-channel>: one grouped launch of the "
                               "7 projections, tiled codes",
                     "alg_flops_per_launch": pre_flops,
                     "alg_bytes_per_launch": sum(pre.bytes_per_launch(j)
                                                 for j in range(len(pre.shapes))),
                     "mean_launch_us": round(mean_pre * 1e6, 2)},
        "shapes": pre_shapes,
    }
    log(f"[bench] prefill {pre_value:.1f} TFLOP/s (separate calls {pre_sep_value:.1f}) "
        f"{pre_shapes}")
    if not args.no_rows:
        pr = Layer(tl, PREFILL_CFG, 2048, copies=2, layout="rows")
        t_pr = time_region(tl, pr, args.prefill_steps, args.prefill_warmup)
        prefill["rows_value"] = round(pre_flops * args.prefill_steps / t_pr / 1e12, 1)
        log(f"[bench] prefill with row-major codes {prefill['rows_value']} TFLOP/s")
        del pr
        torch.cuda.empty_cache()
    pack = bench_pack(tl)
    log(f"[bench] pack {pack}")
    ceilings = measure_ceilings(tl, step_bytes, min(args.steps, 200))
    for sh in shapes_out.values():  # lone launches of the gate shape against its read
        if (sh["N"], sh["K"]) == (18944, 4096):
            sh["frac_of_measured_read"] = round(ceilings["read_gate_size"]["us"] / sh["us"], 4)
    log(f"[bench] ceilings {ceilings}")
    roofline["frac_of_measured_read"] = round(
        achieved / ceilings["read_layer_size"]["GBps"], 4)
    prefill["roofline"]["frac_of_mfma_loop"] = round(
        ach_p / ceilings["mfma_loop"]["TFLOPs_sustained"], 4)
    configs, crossover = (None, None) if args.no_sweep else sweep_configs(tl)
    zero_skip = None if args.no_sweep else measure_zero_skip(tl)
    log(f"[bench] zero skip {zero_skip}")

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu_dec = Layer.__new__(Layer)
        import synth
        cpu_dec.cfg = synth.CONFIGS[DECODE_CFG]
        cpu_dec.M, cpu_dec.g, cpu_dec.shapes = 1, cpu_dec.cfg.group_size, list(cpu_dec.cfg.shapes)
        cpu_dec.cases = [synth.make_case(DECODE_CFG, si, 1) for si in range(len(cpu_dec.shapes))]
        cpu = cpu_baseline_decode(cpu_dec)
        prefill["cpu_baseline"] = cpu_baseline_prefill(pre)
        log(f"[bench] cpu {cpu} {prefill['cpu_baseline']}")

    out = {
        "metric": "ternary_linear HBM GB/s + %peak at M=1; TFLOP/s + %MFMA peak at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_region / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7B-shaped decode layer: 7 ternary projections "
                               "(q,k,v,o 4096|512x4096; gate,up 18944x4096; down 4096x18944), "
                               "M=1, per-channel fp16 scales, bf16 x",
                   "M": 1, "global_batch": 1, "rotated_copies": rotated, "parallelism": "none",
                   "layout": "tiled codes (ternary_tile: 16-row x 256-code blocks of 1 KB); "
                             "row-major codes under rows_codes"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "timing": f"one HIP-graph replay of the K steps (one fused launch each), after "
                  f"{args.warmup} eager steps and {args.settle_ms:g} ms of untimed replays "
                  "(clocks settle); eager launches and seven separate launches per step "
                  "reported beside",
        "eager_value": round(eager_value, 1),
        "separate_launches_value": round(sep_value, 1),
        "rows_codes": rows_dec,
        "roofline": roofline,
        "decode_shapes": shapes_out,
        "prefill": prefill,
        "configs": configs,
        "crossover": crossover,
        "zero_skip": zero_skip,
        "pack": pack,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "kernels_hash": kernel_source_hash(),
    }
    if args.detail:
        Path(args.detail).write_text(json.dumps(out, indent=1))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
