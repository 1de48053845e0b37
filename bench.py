#!/usr/bin/env python3
"""Benchmark of the mixer hot path on one MI355X.

One step = one pass of the 3x3 Latin-square stack ("Placement Is Free, Composition Is Not",
sec. 1 and sec. 3.2; Table 3 lists the per-layer prefill cost of each variant at 2K/8K/32K):
nine causal-prefill layers, rows [full, sliding, differential], [sliding, differential,
full], [differential, full, sliding], at B=1, H=16 (16 heads of head_dim 128, Table 2),
L=8192, sliding window 1024, lambda 0.8, each layer with its own seeded bf16 q/k/v already
resident in HBM. The nine launches go back to back on one stream through
``mixer_stack_prefill``.

Reported (one JSON line):
  value           useful attention TFLOP/s of the whole step (4*d flops per visible
                  query-key pair, summed over the nine layers, / step time);
  per_position    each of the nine layers' median time, in schedule order;
  per_variant     per-layer kernel time and useful TFLOP/s of each variant at L=8K, from HIP
                  events recorded between the launches in a second pass of K steps, and the
                  fraction of the dense bf16 MFMA peak; the executed rate counts the matrix
                  instructions of the kernel's own tile schedule (masked keys of whole tiles,
                  the differential's second value product); the matrix-pipe busy share and
                  effective clock come from the committed SQ counter summary while it matches
                  the kernel source;
  roofline        the same for the kernel that takes most of the step time, with its HBM
                  traffic and matrix-pipe busy share from the committed counter summaries;
  sweep           the lengths of Table 3 (sec. 4.2) for one layer type at a time, launched
                  back to back: full at L=2K, 8K and 32K, the differential at 8K and 32K (on
                  by default; --no-sweep skips it);
  memory          peak device memory of one isolated layer at L = 2K, 8K, 32K: q, k, v and
                  out, and the drop in free device memory across the launches (0: the
                  library allocates nothing);
  arms            step time of the same nine layers in the other depth orders of Table 7
                  (periodic, block) and as the all-full reference;
  mfma_ceiling    the bf16 matrix-core rate the chip sustains under its power cap on
                  random operands (nothing but MFMAs), with the stack value's share of it
                  (each variant's share is in per_variant);
  gqa             one layer per variant at the model's grouped-head shape (16 heads over
                  4 KV heads, Table 2), timed with HIP events;
  cpu_baseline    the fp64 oracle on the same nine layers, every row (host cores, with
                  the thread count it used and the CPU model).

Timing starts at the working clock: the GPU lowers its clock while the host draws the
inputs, so 0.3 s of untimed stack steps (--settle) run before the W warm-up steps, and the
timed region is exactly the K steps after those.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle SECONDS]
       [--no-cpu-baseline] [--no-gqa] [--no-extras] [--copy-calibration] [--no-sweep]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Dense bf16 MFMA peak of MI355X: 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
VARIANT_NAMES = ("full", "sliding", "differential")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
SQ_FILE = os.path.join(ROOT, "profiles", "sq_busy.txt")
# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.
N_XCD, N_CU, N_SIMD = 8, 256, 1024
MFMA_FLOPS = 32 * 32 * 16 * 2    # one v_mfma_f32_32x32x16_bf16 (scores, value products)
MFMA16_FLOPS = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_bf16 (the differential's row sums)
# Sources of the bf16 kernel the bench times (a traffic summary is valid only for them).
KERNEL_SOURCES = [os.path.join(ROOT, "heterogeneous_attention_mixer_amd", "csrc", f)
                  for f in ("attn_prefill_dma.hip", "device_common.h", "kernels.h")]
# The d=128 bf16 kernel of each variant: its name as reported, and a substring of its
# mangled symbol in profiler output.
KERNELS = {"full": ("prefill_phase_kernel<128, full>", "prefill_phase_kernelILi128ELi0E"),
           "sliding": ("prefill_dma_kernel<128, sliding>", "prefill_dma_kernelILi128ELi1E"),
           "differential": ("prefill_phase_kernel<128, differential>",
                            "prefill_phase_kernelILi128ELi2E")}


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    does not write back and invalidate the caches, which a default event (and so a
    torch.cuda.Event) does at every record, slowing the work that follows (measured: per-layer
    torch events cost a step of the stack 1.1 %, these 0.4 %). ``cuda_event`` is the raw
    handle, which the library's runners record."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        h = ctypes.c_void_p()
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                    self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value

    def record(self):
        """Record on the current torch stream."""
        import ctypes

        import torch
        s = torch.cuda.current_stream().cuda_stream
        if TimingEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event),
                                           ctypes.c_void_p(s)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to ``end`` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        if TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms),
                                                ctypes.c_void_p(self.cuda_event),
                                                ctypes.c_void_p(end.cuda_event)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        import ctypes
        if TimingEvent._hip is not None and getattr(self, "cuda_event", None):
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def full_takes_phase_kernel(B: int, H: int, L: int, n_cu: int = N_CU) -> bool:
    """Whether a full causal layer runs the phase-separated kernel (256-row workgroups): when
    its grid holds more than one of them per CU, as the launcher decides."""
    return B * H * ((L + 255) // 256) > n_cu


def visible_pairs(variant: str, L: int, window: int) -> int:
    """Visible (query, key) pairs of one head: causal L(L+1)/2; sliding keeps W per row
    once the row index reaches W."""
    if variant == "sliding" and window < L:
        return window * (window + 1) // 2 + (L - window) * window
    return L * (L + 1) // 2


def useful_flops(variant: str, B: int, H: int, L: int, d: int, window: int) -> int:
    """4*d flops per visible pair: 2*d for the scores (the differential's two half-width
    maps together also cost 2*d) and 2*d for the weighted sum of values."""
    return 4 * d * B * H * visible_pairs(variant, L, window)


def executed_mfma_split(variant: str, B: int, H: int, L: int, d: int, window: int,
                        n_cu: int = N_CU):
    """Matrix instructions one launch of the bf16 kernel issues, as (32x32x16, 16x16x32)
    counts, from the same tile schedule the kernels follow: whole 64-key tiles, 32 query rows
    per wave, masked keys computed like visible ones.

    Full and sliding (128 query rows per workgroup, 4 row blocks): per wave, the scores of
    its first tile in the prologue, then per iteration the next tile's scores and the
    previous tile's value product (the first iteration's value product multiplies zero
    probabilities), the last iteration only the value product, and the value product of the
    last tile after the loop. With at most one workgroup per CU the key split runs (two
    waves per row block, alternate tiles); otherwise one wave per row block. A wave skips
    the first scores of a tile no row of it sees and the last value product of a tile past
    its rows, where the kernel does (see the kernel's prologue and tail). Full causal in the
    key split with an even number of 64-row query tiles pairs tile p with tile n-1-p in one
    workgroup, and a wave of the light tile ends its loop early (see the kernel's loop).
    Phase-separated kernel, the differential (8 waves: 4 row blocks x 2 maps, 128 rows) and
    full causal on grids of more than one 256-row workgroup per CU (8 waves: 8 row blocks):
    per wave hi + 2 matrix phases of the scores (half-width for the differential) and the
    value product each (the first value product multiplies zeros, the last scores are
    discarded), and four 16x16x32 row-sum instructions per exponential pass: one
    per vector phase after the first (hi), and one for the first tile, taken once its rows
    have a reference (its own vector phase takes none). Passes taken again because a tile's
    sum exceeds 2^8 depend on the data and are not counted (none on the bench's inputs)."""
    bm, bn = 128, 64
    nq = (L + bm - 1) // bm
    qk = 2 * (d // 16)          # one tile's scores: 2 key blocks x d/16 steps
    pv = 2 * 2 * (d // 32)      # one tile's value product: 4 key groups x d/32 channel blocks
    slide = variant == "sliding"
    total = 0
    if variant == "differential" or (variant == "full" and
                                     full_takes_phase_kernel(B, H, L, n_cu)):
        rows, qk_phase = (128, 2 * (d // 32)) if variant == "differential" else (256, qk)
        small = 0
        for qt in range((L + rows - 1) // rows):
            hi = (min(qt * rows + rows, L) - 1) // bn
            total += 8 * (hi + 2) * (qk_phase + pv)
            small += 8 * (hi + 1) * 4
        return B * H * total, B * H * small
    spl = 2 if B * H * nq <= n_cu else 1
    nt64 = (L + bn - 1) // bn
    if variant == "full" and spl == 2 and nt64 % 2 == 0:
        # Paired 64-row query tiles p and nt64-1-p in one workgroup (row blocks 0, 1 and 2, 3),
        # two waves per row block; a wave's loop ends with the last of its tiles its rows see
        # (at least one iteration).
        for p in range(nt64 // 2):
            th = nt64 - 1 - p
            n_it = (min(th * bn + bn, L) - 1) // bn // 2 + 1
            for rb in range(4):
                qw = p * bn + 32 * rb if rb < 2 else th * bn + 32 * (rb - 2)
                for half in range(2):
                    jl = (qw + 31) // bn
                    n_run = min(n_it, (jl - half) // 2 + 1 if jl >= half else 1)
                    see_first = half == 0 or half * bn <= qw + 31
                    tail = (2 * (n_run - 1) + half) * bn <= qw + 31
                    total += (qk if see_first else 0) + (n_run - 1) * (qk + pv) + pv + \
                        (pv if tail else 0)
        return B * H * total, 0
    for qt in range(nq):
        q0 = qt * bm
        hi = (min(q0 + bm, L) - 1) // bn
        lo = max(0, q0 - window + 1) // bn if slide else 0
        n_it = (hi - lo) // spl + 1
        for rb in range(4):
            qw = q0 + 32 * rb
            for half in range(spl):
                j0 = lo + half
                see_first = ((half == 0 or j0 * bn <= qw + 31) and
                             (not slide or j0 * bn + bn - 1 >= qw - window + 1))
                jl = lo + spl * (n_it - 1) + half
                tail = jl * bn <= qw + 31
                total += (qk if see_first else 0) + (n_it - 1) * (qk + pv) + pv + \
                    (pv if tail else 0)
    return B * H * total, 0


def executed_mfmas(variant: str, B: int, H: int, L: int, d: int, window: int,
                   n_cu: int = N_CU) -> int:
    """Matrix instructions of one launch (what SQ_INSTS_MFMA counts); see
    executed_mfma_split."""
    return sum(executed_mfma_split(variant, B, H, L, d, window, n_cu))


def executed_flops(variant: str, B: int, H: int, L: int, d: int, window: int,
                   n_cu: int = N_CU) -> int:
    """Flops of the matrix instructions of one launch; see executed_mfma_split."""
    n32, n16 = executed_mfma_split(variant, B, H, L, d, window, n_cu)
    return n32 * MFMA_FLOPS + n16 * MFMA16_FLOPS


def launch_threads(variant: str, B: int, H: int, L: int, n_cu: int = N_CU) -> int:
    """Work-items in one launch of the d=128 bf16 kernel (the Grid_Size profilers report).
    Full and sliding on the pipelined kernel: one workgroup per (b*h, 128-row query tile), of
    256 work-items, 512 with the key split (grids of at most one workgroup per CU). The
    phase-separated kernel (the differential with 128-row units, full causal with 256-row
    units on grids of more than one of them per CU): 512-item workgroups, one per unit, or,
    with more units than CUs, the persistent launch of one per CU."""
    if variant == "differential" or (variant == "full" and
                                     full_takes_phase_kernel(B, H, L, n_cu)):
        rows = 128 if variant == "differential" else 256
        return min(B * H * ((L + rows - 1) // rows), n_cu) * 512
    wgs = B * H * ((L + 127) // 128)
    return wgs * 512 if wgs <= n_cu else wgs * 256


def _stack_dispatch(variant: str, row: dict) -> bool:
    """Whether a profiler row can belong to a launch of the stack workload (B=1 H=16
    L=8192), by its grid. The persistent launches of the phase-separated kernel have one
    workgroup per CU at every length, so the counter runs time the stack alone
    (--no-sweep --no-gqa --no-extras); this keeps out the launches a grid does tell apart.
    Rows without a Grid_Size column are taken as they are."""
    g = row.get("Grid_Size")
    if not g:
        return True
    from heterogeneous_attention_mixer_amd import synth
    cfg = synth.LATIN_STACK
    return int(g) == launch_threads(variant, cfg["B"], cfg["H"], cfg["L"])


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed: what the compiler
    sees. String literals in these sources hold no comment markers."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the kernel's code (comments and layout excluded), keying the counter file."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(variant: str):
    """HBM bytes per launch of ``variant`` from the committed counter summary, or None when
    there is none or the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    key = f"{variant}_hbm_bytes_per_launch"
    return float(kv[key]) if key in kv else None


def _read_kv(path):
    kv = {}
    if not os.path.exists(path):
        return kv
    with open(path) as f:
        for line in f:
            line = line.strip()
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def read_sq(variant: str):
    """Matrix-pipe busy fraction and MFMA count per launch of ``variant`` from the committed
    SQ counter summary, or None when there is none or the kernel source changed since the
    counters were taken."""
    kv = _read_kv(SQ_FILE)
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return {"mfma_busy": float(kv[f"{variant}_mfma_busy"]),
                "sq_insts_mfma": int(float(kv[f"{variant}_sq_insts_mfma"])),
                "effective_clock_ghz": float(kv[f"{variant}_effective_clock_ghz"])}
    except KeyError:
        return None


def write_sq(csv_path: str, command: str) -> str:
    """Turn one rocprofv3 --pmc run (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, GRBM_GUI_ACTIVE,
    with --kernel-trace) over the bench's stack into SQ_FILE, keyed to the kernel source
    hash: per d=128 bf16 variant the matrix pipe's busy share of the dispatch's cycles
    (busy cycles per SIMD over GUI-active cycles per XCD), the MFMA count per launch, and the
    effective clock (GUI-active cycles per XCD over the dispatch's duration)."""
    import csv
    vals = {}
    dur = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            key = next((v for v, (_, tag) in KERNELS.items() if tag in name), None)
            if key is None or not _stack_dispatch(key, r):
                continue
            did = r.get("Dispatch_Id", "")
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], {})[did] = float(
                r["Counter_Value"])
            if "End_Timestamp" in r and "Start_Timestamp" in r:
                dur.setdefault(key, {})[did] = (int(r["End_Timestamp"]) -
                                                int(r["Start_Timestamp"]))
    lines = ["# Matrix-pipe busy share, MFMA count and effective clock per launch of the d=128",
             "# bf16 kernel of each variant at B=1 H=16 L=8192 (Latin stack workload), from one",
             "# rocprofv3 --pmc run with --kernel-trace, averaged over the stack's launches.",
             "# mfma_busy = (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8 XCDs);",
             "# effective_clock_ghz = (GRBM_GUI_ACTIVE / 8) / dispatch duration.",
             f"# command: {command}",
             f"kernel_source_sha256_16 = {kernel_source_hash()}"]
    for v in VARIANT_NAMES:
        c = vals.get(v, {})
        need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")
        if not all(n in c for n in need):
            continue
        ids = sorted(set.intersection(*(set(c[n]) for n in need)))
        busy = [c["SQ_VALU_MFMA_BUSY_CYCLES"][i] / N_SIMD / (c["GRBM_GUI_ACTIVE"][i] / N_XCD)
                for i in ids]
        insts = [c["SQ_INSTS_MFMA"][i] for i in ids]
        clk = [c["GRBM_GUI_ACTIVE"][i] / N_XCD / dur[v][i]
               for i in ids if dur.get(v, {}).get(i)]
        lines.append(f"{v}_mfma_busy = {sum(busy) / len(busy):.4f}")
        lines.append(f"{v}_sq_insts_mfma = {sum(insts) / len(insts):.0f}")
        if clk:
            lines.append(f"{v}_effective_clock_ghz = {sum(clk) / len(clk):.4f}")
        lines.append(f"{v}_dispatches = {len(ids)}")
    os.makedirs(os.path.dirname(SQ_FILE), exist_ok=True)
    with open(SQ_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    return SQ_FILE


def cpu_model() -> str:
    """The host CPU's model name as the kernel reports it (Linux), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


COPY_BYTES = 256 * 1024 * 1024  # the --copy-calibration copy: reads and writes this much


def write_traffic(fetch_csv: str, write_csv: str, command: str) -> str:
    """Turn two rocprofv3 --pmc counter files (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch, of ``bench.py --copy-calibration``) into HBM bytes per launch of each d=128
    bf16 variant. Each counter is scaled so that the plain device copy of COPY_BYTES reads
    (or writes) exactly COPY_BYTES. Writes TRAFFIC_FILE, keyed to the kernel source hash."""
    import csv

    def per_kernel(path, counter):
        out = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = next((v for v, (_, tag) in KERNELS.items() if tag in name),
                           "copy" if "copyBuffer" in name else None)
                if key == "copy" or (key and _stack_dispatch(key, r)):
                    out.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in out.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no copy-kernel calibration in the counter files")
    fscale = COPY_BYTES / fetch["copy"]
    wscale = COPY_BYTES / write["copy"]
    lines = ["# HBM bytes per launch of the d=128 bf16 kernel of each variant at B=1 H=16 L=8192",
             "# (Latin stack workload), from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE,",
             "# each scaled by what it reads for a plain 256 MiB device copy.",
             f"# command: {command}",
             f"kernel_source_sha256_16 = {kernel_source_hash()}",
             f"fetch_scale = {fscale:.4f}",
             f"write_scale = {wscale:.4f}"]
    for v in VARIANT_NAMES:
        if v in fetch and v in write:
            lines.append(f"{v}_fetch_bytes_per_launch = {fetch[v] * fscale:.0f}")
            lines.append(f"{v}_write_bytes_per_launch = {write[v] * wscale:.0f}")
            lines.append(f"{v}_hbm_bytes_per_launch = "
                         f"{fetch[v] * fscale + write[v] * wscale:.0f}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    return TRAFFIC_FILE


def cpu_baseline(host_layers, sched, cfg, rows_per_head: int):
    """The fp64 oracle, as it stands, on the layers of one step (every layer of the stack;
    every query row, or a seeded sample of ``rows_per_head`` rows per head when that is
    positive). Returns the cpu_baseline object."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    rng = np.random.default_rng(12345)
    L, d, B, H = cfg["L"], cfg["d"], cfg["B"], cfg["H"]
    flops = 0
    elapsed = 0.0
    for layer, inp in enumerate(host_layers):
        variant = VARIANT_NAMES[sched[layer]]
        if 0 < rows_per_head < L:
            rows = np.sort(rng.choice(L, size=rows_per_head, replace=False))
        else:
            rows = None
        t0 = time.perf_counter()
        oracle.prefill_rows(inp.q, inp.k, inp.v, variant, cfg["window"], cfg["lam"], rows)
        elapsed += time.perf_counter() - t0
        for i in (range(L) if rows is None else rows.tolist()):
            lo = max(0, i - cfg["window"] + 1) if variant == "sliding" else 0
            flops += 4 * d * B * H * (i - lo + 1)
    what = ("every query row" if not 0 < rows_per_head < L
            else f"{rows_per_head} seeded query rows per head")
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"{what} of all {len(host_layers)} layers of one step of the stack "
                   f"(full, sliding W={cfg['window']}, differential lambda={cfg['lam']}), "
                   f"B={B} H={H} L={L} d={d}, fp64 loops; {flops / 1e9:.1f} GFLOP in "
                   f"{elapsed:.1f} s"),
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle rows per head per layer for the CPU baseline (0 = all)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy first (for HBM counter scaling)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed launches before the warm-up steps (and before "
                         "each sweep point), so that timing starts at the working clock")
    ap.add_argument("--no-gqa", action="store_true",
                    help="skip the grouped-head layers (profiling runs whose per-kernel "
                         "averages must cover the stack's launches only)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the memory and placement-arm sections (profiling runs, as "
                         "for --no-gqa)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the single-type layers at the lengths of Table 3 (full at "
                         "L=2K/8K/32K, differential at L=8K/32K), which run by default; for "
                         "profiling runs")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write the HBM traffic summary from two rocprofv3 "
                         "counter files and exit")
    ap.add_argument("--traffic-command", default="",
                    help="with --write-traffic or --write-sq: the profiling command, recorded "
                         "in the file")
    ap.add_argument("--write-sq", metavar="COUNTER_CSV",
                    help="host only: write the matrix-pipe busy summary from one rocprofv3 "
                         "counter file (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, "
                         "GRBM_GUI_ACTIVE, with --kernel-trace) and exit")
    args = ap.parse_args(argv)

    if args.write_traffic:
        print(write_traffic(args.write_traffic[0], args.write_traffic[1],
                            args.traffic_command))
        return 0
    if args.write_sq:
        print(write_sq(args.write_sq, args.traffic_command))
        return 0

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported (the layer "
              "would shard over batch and heads with no exchange, which is not implemented)",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        return 2

    import torch

    from heterogeneous_attention_mixer_amd import build as mbuild
    from heterogeneous_attention_mixer_amd import mixer, synth
    if mbuild.needs_build():
        mbuild.build()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    mixer.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = dict(synth.LATIN_STACK)
    B, H, L, d, W, lam = cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["window"], cfg["lam"]
    base = [VARIANT_NAMES.index(x) for x in cfg["base"]]
    sched = mixer.mixer_latin_build(base)
    n_layers = len(sched)

    if args.copy_calibration:
        n = 256 * 1024 * 1024
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Inputs: layer l drawn from seed seed0 + l, copied to HBM before any timing.
    host_layers, qs, ks, vs = [], [], [], []
    for layer in range(n_layers):
        inp = synth.make_qkv(cfg["seed0"] + layer, B, H, L, d, "bf16")
        host_layers.append(inp)
        t = [torch.from_numpy(b).view(torch.bfloat16).to(dev)
             for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
        qs.append(t[0])
        ks.append(t[1])
        vs.append(t[2])
    outs = [torch.empty_like(q) for q in qs]
    # Grouped key/value heads at the model's attention shape (Table 2, sec. 4.1: 16 heads
    # over 4 KV heads): one layer per variant, inputs from seed seed0 + variant number.
    g = synth.GQA
    gqa_inputs = []
    for vi, variant in enumerate(VARIANT_NAMES if not args.no_gqa else ()):
        inp = synth.make_qkv_gqa(g["seed0"] + vi, g["B"], g["H"], g["Hkv"], g["L"], g["d"])
        gqa_inputs.append([torch.from_numpy(b).view(torch.bfloat16).to(dev)
                           for b in (inp.q_bits, inp.k_bits, inp.v_bits)])
    torch.cuda.synchronize()

    def settle(fn, seconds):
        # The GPU lowers its clock while the host prepares inputs and needs tens of
        # milliseconds of load to come back: untimed launches until `seconds` have passed.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()

    def step(events=None):
        mixer.mixer_stack_prefill(3, sched, qs, ks, vs, outs, W, lam, events=events)

    gc.collect()
    settle(step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps, bracketed by two HIP events that the library records on the
    # launch stream right before the first layer and right after the last (so no host time
    # before the first launch is counted, and no event sits between the layers). A second,
    # instrumented pass of K steps then records an event around every layer for the
    # per-layer figures. The events are fence-free HIP events (TimingEvent); each record
    # still costs the stream about a microsecond.
    K = args.steps
    start = TimingEvent()
    end = TimingEvent()
    layer_events = [[TimingEvent() for _ in range(n_layers + 1)]
                    for _ in range(K)]

    def timed_pass():
        for i in range(K):
            evs = [None] * (n_layers + 1)
            if i == 0:
                evs[0] = start
            if i == K - 1:
                evs[n_layers] = end
            step(evs)
        torch.cuda.synchronize()

    # One untimed pass of the timed loop itself first. The first pass of a freshly set-up
    # loop runs every kernel a few % slower than all later ones, measured with and without
    # per-layer events and after clock settling or a continuous burst alike (the cause lies
    # outside the kernels); the timed pass measures the steady state.
    timed_pass()
    # A full collection of Python's cyclic garbage takes milliseconds in a process that has
    # torch loaded, and the argument arrays each step builds can trigger one: the collector
    # is held off until the device has finished (the collection itself runs before the clock
    # settling: measured, the kernels ran 6 % slower in a timed region that followed it).
    gc.disable()
    try:
        t_wall = time.perf_counter()
        timed_pass()
        t_wall = time.perf_counter() - t_wall
    finally:
        gc.enable()
    ms_per_step = start.elapsed_time(end) / K

    total_flops = sum(useful_flops(VARIANT_NAMES[v], B, H, L, d, W) for v in sched)
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    # The instrumented pass.
    for i in range(K):
        step(layer_events[i])
    torch.cuda.synchronize()
    per_launch = {name: [] for name in VARIANT_NAMES}
    for evs in layer_events:
        for layer in range(n_layers):
            per_launch[VARIANT_NAMES[sched[layer]]].append(
                evs[layer].elapsed_time(evs[layer + 1]))
    # Each depth of the stack on its own (median over the instrumented steps): a layer's cost
    # next to neighbours of other types.
    per_position = []
    for layer in range(n_layers):
        ts = sorted(evs[layer].elapsed_time(evs[layer + 1]) for evs in layer_events)
        per_position.append({"variant": VARIANT_NAMES[sched[layer]],
                             "ms_median": round(ts[len(ts) // 2], 5)})
    per_variant = {}
    for name, ts in per_launch.items():
        if not ts:
            continue
        ms = sum(ts) / len(ts)
        fl = useful_flops(name, B, H, L, d, W)
        ex = executed_flops(name, B, H, L, d, W)
        srt = sorted(ts)
        per_variant[name] = {
            "ms_per_launch": round(ms, 5),
            "ms_median": round(srt[len(srt) // 2], 5),
            "ms_min": round(srt[0], 5),
            "launches": len(ts),
            "useful_tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "executed_tflops": round(ex / (ms * 1e-3) / 1e12, 2),
            "executed_per_useful": round(ex / fl, 4),
            "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "useful_gflop_per_launch": round(fl / 1e9, 3),
        }
        sq = read_sq(name)
        if sq:
            per_variant[name]["mfma_busy"] = sq["mfma_busy"]
            per_variant[name]["effective_clock_ghz"] = sq["effective_clock_ghz"]
    dominant = max(per_variant, key=lambda n: per_variant[n]["ms_per_launch"]
                   * per_variant[n]["launches"])
    dom = per_variant[dominant]
    achieved = dom["useful_tflops"]
    roofline = {
        "bound": "mfma",
        "kernel": f"{KERNELS[dominant][0]} (bf16)",
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": read_traffic(dominant),
        "mfma_busy": (read_sq(dominant) or {}).get("mfma_busy"),
    }

    # Peak device memory of one isolated layer (Table 3's memory column): the high-water mark
    # of torch's allocator from before the layer's q/k/v/out exist until all three variants
    # have run on them, and the drop in the device's free memory across the launches (which
    # would show any allocation made inside the library).
    def layer_memory(Lx):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base_alloc = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        t = [torch.empty(B, H, Lx, d, dtype=torch.bfloat16, device=dev).normal_()
             for _ in range(4)]
        torch.cuda.synchronize()
        io = torch.cuda.memory_allocated(dev) - base_alloc
        free0 = torch.cuda.mem_get_info(dev)[0]
        for variant in VARIANT_NAMES:
            mixer.mixer_prefill_async(t[0], t[1], t[2], t[3], variant,
                                      W if variant == "sliding" else 0,
                                      lam if variant == "differential" else 0.0)
        torch.cuda.synchronize()
        res = {"io_bytes": int(io),
               "high_water_bytes": int(torch.cuda.max_memory_allocated(dev) - base_alloc),
               "device_free_drop_bytes": int(free0 - torch.cuda.mem_get_info(dev)[0])}
        del t
        return res

    memory = (None if args.no_extras
              else {f"L{Lx}": layer_memory(Lx) for Lx in (2048, 8192, 32768)})

    # The placement arms of Table 7 (sec. 6.1) over the three types built here: the same
    # nine layers (same inputs per depth) in other orders, and the all-full reference.
    arm_orders = {
        "latin": sched,
        "periodic": base * 3,
        "block": [x for x in base for _ in range(3)],
        "homo_full": [0] * n_layers,
    }
    # Round-robin over the arms, one step of each per round with events around it, so every
    # arm sees the same clock state (the chip's clock drifts with load and time).
    if args.no_extras:
        arm_orders = {}
    else:
        settle(step, args.settle)
    rounds = 10
    # Events around every layer (recorded by the library on the launch stream).
    arm_ev = {arm: [[TimingEvent() for _ in range(n_layers + 1)]
                    for _ in range(rounds)] for arm in arm_orders}
    for arm, order in arm_orders.items():
        mixer.mixer_layers_prefill(order, qs, ks, vs, outs, W, lam)
    for r in range(rounds):
        for arm, order in arm_orders.items():
            mixer.mixer_layers_prefill(order, qs, ks, vs, outs, W, lam, events=arm_ev[arm][r])
    torch.cuda.synchronize()
    arms = {}
    for arm, order in arm_orders.items():
        ms = sum(evs[0].elapsed_time(evs[-1]) for evs in arm_ev[arm]) / rounds
        fl = sum(useful_flops(VARIANT_NAMES[v], B, H, L, d, W) for v in order)
        pos = []
        for layer in range(n_layers):
            ts = sorted(evs[layer].elapsed_time(evs[layer + 1]) for evs in arm_ev[arm])
            pos.append(round(ts[len(ts) // 2], 5))
        arms[arm] = {"order": "".join("FSD"[v] for v in order), "ms_per_step": round(ms, 5),
                     "useful_tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                     "ms_median_per_layer": pos}

    # The matrix-core ceiling under the power cap (a measurement aid): the same bf16 MFMA on
    # random operands and nothing else, every SIMD busy, so that the prefill kernels can also
    # be rated against the rate this chip sustains rather than only the 2.4 GHz figure.
    ceiling = None
    if not args.no_extras:
        import numpy as np
        mc = synth.MFMA_CEILING
        bits = synth.make_mfma_fragments(mc["seed"], mc["nsets"])
        frags = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        sink = torch.empty(mc["blocks"] * mixer.CEILING_SINK_PER_BLOCK, dtype=torch.float32,
                           device=dev)

        def run_ceiling():
            mixer.mixer_mfma_ceiling_async(frags, sink, mc["blocks"], mc["iters"])
        settle(run_ceiling, args.settle)
        reps = 5
        e0 = TimingEvent()
        e1 = TimingEvent()
        run_ceiling()  # the start event behind one launch, as for the grouped-head layers
        e0.record()
        for _ in range(reps):
            run_ceiling()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = mc["blocks"] * 16 * mc["iters"] * 32 * 32 * 16 * 2
        ct = fl / (ms * 1e-3) / 1e12
        ceiling = {"tflops": round(ct, 2), "frac_of_bf16_peak": round(ct / PEAK_BF16_TFLOPS, 4),
                   "ms_per_launch": round(ms, 5),
                   "launch": (f"{mc['blocks']} workgroups x 4 waves, each wave 4 chains of "
                              f"{mc['iters']} v_mfma_f32_32x32x16_bf16 on seeded N(0,1) bf16 "
                              f"operands")}
        for pv in per_variant.values():
            pv["frac_of_measured_ceiling"] = round(pv["useful_tflops"] / ct, 4)
        roofline["measured_ceiling_tflops"] = ceiling["tflops"]
        roofline["frac_of_measured_ceiling"] = round(achieved / ct, 4)
        del frags, sink

    # The grouped-head layers, right after the stack (the chip is at its working clock).
    gqa = {}
    for vi, variant in enumerate(VARIANT_NAMES if not args.no_gqa else ()):
        Wg = g["window"] if variant == "sliding" else 0
        lg = g["lam"] if variant == "differential" else 0.0
        t = gqa_inputs[vi]
        o = torch.empty_like(t[0])
        for _ in range(5):
            mixer.mixer_prefill_gqa_async(*t, o, variant, Wg, lg)
        torch.cuda.synchronize()
        reps = 20
        e0 = TimingEvent()
        e1 = TimingEvent()
        # The start event goes in behind one more launch: the timed launches then follow each
        # other on the device while the host enqueues them, and the host's time before the
        # first of them is not counted.
        mixer.mixer_prefill_gqa_async(*t, o, variant, Wg, lg)
        e0.record()
        for _ in range(reps):
            mixer.mixer_prefill_gqa_async(*t, o, variant, Wg, lg)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = useful_flops(variant, g["B"], g["H"], g["L"], g["d"], Wg)
        gqa[variant] = {
            "ms_per_launch": round(ms, 5),
            "useful_tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del o
    del gqa_inputs

    sweep = None
    if not args.no_sweep:
        sweep = {}
        # Each layer alone, back to back (the same workload as the stack's layers at
        # L=8192, without the neighbours of other types).
        for name, variant, Ls in (("full", "full", (2048, 8192, 32768)),
                                  ("differential", "differential", (8192, 32768))):
            for Lx in Ls:
                inp = synth.make_qkv(3 if variant == "full" else 4, B, H, Lx, d, "bf16")
                t = [torch.from_numpy(b).view(torch.bfloat16).to(dev)
                     for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
                o = torch.empty_like(t[0])
                settle(lambda: mixer.mixer_prefill_async(*t, o, variant, 0, lam),
                       args.settle)
                # One call of the layers runner enqueues every repetition, and the library
                # records the events around them on the launch stream, so that a short kernel
                # (34 us at L=2048) waits neither for the Python binding's per-call work
                # between launches nor for its argument setup before the first.
                reps = 10 if Lx <= 8192 else 3
                e0 = TimingEvent()
                e1 = TimingEvent()
                # events only before the first launch and after the last; an untimed pass
                # with the same events first, as for the stack
                for _ in range(2):
                    mixer.mixer_layers_prefill([variant] * reps, [t[0]] * reps,
                                               [t[1]] * reps, [t[2]] * reps, [o] * reps, 0,
                                               lam, events=[e0] + [None] * (reps - 1) + [e1])
                    torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                fl = useful_flops(variant, B, H, Lx, d, 0)
                ex = executed_flops(variant, B, H, Lx, d, 0)
                sweep[f"{name}_L{Lx}"] = {
                    "ms_per_launch": round(ms, 5),
                    "useful_tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                    "executed_per_useful": round(ex / fl, 4),
                    "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                               4)}
                del t, o

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_layers, sched, cfg, args.cpu_rows)

    line = {
        "metric": "prefill attention TFLOP/s per variant at L=8K; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v rounded to bf16, fresh per layer",
        "config": {
            "workload": (f"3x3 Latin-square stack of causal-prefill layers, rows "
                         f"[full,sliding,differential],[sliding,differential,full],"
                         f"[differential,full,sliding]; B={B} H={H} L={L} d={d} "
                         f"window={W} lambda={lam}"),
            "B": B, "H": H, "L": L, "d": d, "window": W, "lambda": lam,
            "layers": n_layers, "useful_gflop_per_step": round(total_flops / 1e9, 2),
        },
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "per_variant": per_variant,
        "per_position": per_position,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": round(t_wall, 4),
    }
    line["memory"] = memory
    line["arms"] = arms or None
    line["mfma_ceiling"] = ceiling
    if ceiling:
        # The stack's rate as a share of the rate the same chip sustains on matrix work
        # alone: steadier across GPUs than the raw value, whose spread is the power cap's.
        ceiling["stack_value_frac"] = round(value / ceiling["tflops"], 4)
    line["gqa"] = None if args.no_gqa else {
        "config": (f"one layer per variant, B={g['B']} H={g['H']} Hkv={g['Hkv']} "
                   f"L={g['L']} d={g['d']} window={g['window']} lambda={g['lam']}"),
        "per_variant": gqa,
    }
    if sweep is not None:
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
