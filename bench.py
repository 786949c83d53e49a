#!/usr/bin/env python3
"""W4A16 GEMM throughput on one MI355X: Llama-3-8B layer shapes at M = 1, 16 and 2048.

One step = the four projection GEMMs of a Llama-3-8B layer (QKV 4096x6144, O 4096x4096,
gate_up 4096x28672, down 14336x4096; g = 128, asymmetric uint4 codes, fp16 scales, fp16
activations and output) at each of M = 1, 16 and 2048: twelve mpgemm_w4a16 calls.  Weights
are pre-packed and resident in HBM; each call reads a different copy from a rotating pool
larger than the 256 MB Infinity Cache, so weight bytes come from HBM, not from a cache that
the previous call warmed.

Prints one JSON line: value = whole-step TFLOP/s (2*M*N*K summed over the twelve GEMMs,
divided by the step time), plus HBM GB/s of algorithmic bytes, the roofline of the dominant
kernel, per-config GEMM lines and the CPU oracle timed on bounded samples (cpu_baseline).

Timing.
  * The timed steps launch every GEMM from Python (the host enqueues a step in about an
    eighth of the GPU's time for it).  Kernel durations come from hipEvents recorded,
    inside the timed steps, on the stream the library launches on, around each run of
    consecutive launches of one kernel (the four GEMMs of one M, or fewer where the
    selector changes kernel), divided by the launches in it.  Every event is created
    before the timed region (creating them inside it let single stalls of 40-70 ms into
    the 20-step window on some boxes), with hipEventDisableSystemFence: a default event's
    system-scope release made the kernel after it wait for a cache writeback.  `roofline` uses them for the dominant kernel; it also carries the
    average launch duration of the same kernel in the committed rocprofv3 kernel trace
    (profiles/w4a16_llama3_8b_m1_16_2048_kernel_trace.txt, written by --trace-summary from
    a trace of this same command) while the kernel sources still hash to the digest it
    records, and the fraction that figure gives.
  * Every other GEMM time ("cold per launch") replays one HIP graph of launches that each
    read a different copy of the weights, with at least 1.2 GB between two reads of the same
    copy, so no launch is served by the Infinity Cache; the time per launch includes the
    graph's launch-to-launch gap.
  * `peaks` are measured in the run by the probes of libmpgemm_probes.so: the cold stream
    read time of a buffer of each GEMM's byte count (the floor for any kernel that must
    read those bytes) and the MFMA loop rate on non-zero data under the power limit.
    Every GEMM line reports its fraction of the published peak (`frac`: 8 TB/s, 2.5 PF)
    and of the measured one (`frac_measured`).
  * `traffic` is the HBM bytes per launch that rocprofv3's FETCH_SIZE and WRITE_SIZE
    counters read for the dominant kernel, scaled by what the same counters read for a
    plain 1 GiB copy (--copy-calibration); it is taken from the summary file under
    profiles/ and reported only while the kernel sources still hash to the digest recorded
    there, else null.

Per-config lines (`configs`): every GEMM of the workloads the metric is quoted on, timed
cold per launch: Llama-3-8B decode (M = 1, 8, 16) and prefill (M = 512, 2048, 8192),
Llama-3-70B with bf16 activations (M = 1, 64, 4096) and Qwen3-32B with 64-deep groups and
symmetric codes (M = 1, 2, 4, 16, 128, 1024, 8192).  Other code formats at the Llama-3-8B
(or, for FP8, Qwen3-8B) shapes, the small-prefill pass at M = 128..512 and decode attention
over 8-bit and FP8 KV caches follow.  None of these is part of `value`.

cpu_baseline: the CPU oracle as it stands (scalar dequantization, then an fp64 GEMM
parallel over rows), per Llama-3-8B shape: M = 1 in full on one thread (its rows give
nothing to parallelize), and M = 2048 on a 32-row sample over all host threads, scaled by
2048 / 32 (rows are independent; labelled as extrapolated).
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA
MS = (1, 16, 2048)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "w4a16_llama3_8b_m1_16_2048_hbm_traffic.txt")
TRACE_FILE = os.path.join(PROFILES, "w4a16_llama3_8b_m1_16_2048_kernel_trace.txt")
COLD_BYTES = 1.2e9              # distinct weight bytes between two reads of one copy


def kernel_source_digest():
    """sha256 (16 hex digits) over the HIP sources and the build flags of the library's GEMM
    path (everything but the attention kernels and the probes, which the GEMM profiles do
    not cover)."""
    pkg = os.path.join(ROOT, "weight_only_quantized_mpgemm_amd")
    csrc = os.path.join(pkg, "csrc")
    h = hashlib.sha256()
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
             if f.endswith((".hip", ".hpp")) and f not in ("attention.hip", "probes.hip")] + \
        [os.path.join(pkg, "build.py")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _summary_rows(path):
    """(digest, rows) of a summary file under profiles/: rows are whitespace-split lines
    outside comments and headers."""
    if not os.path.exists(path):
        return None, []
    digest, rows = None, []
    with open(path) as fh:
        for line in fh:
            if line.startswith("# source_digest:"):
                digest = line.split(":", 1)[1].strip()
            elif line.strip() and not line.startswith("#"):
                rows.append(line.split())
    return digest, rows


def load_traffic():
    """{(kernel, M, K, N): scaled HBM bytes per launch} from the counter summary, or {} when
    the file is absent or was taken from other kernel sources."""
    digest, rows = _summary_rows(TRAFFIC_FILE)
    if digest != kernel_source_digest():
        return {}
    return {(f[0], int(f[1]), int(f[2]), int(f[3])): float(f[6]) for f in rows
            if f[0] != "kernel" and len(f) >= 7}


def load_trace():
    """{kernel: average launch us over the timed steps} from the committed kernel trace
    summary, or {} when absent or taken from other kernel sources."""
    digest, rows = _summary_rows(TRACE_FILE)
    if digest != kernel_source_digest():
        return {}
    out = {}
    for f in rows:
        if len(f) == 3 and f[0] != "kernel":
            try:
                out[f[0]] = float(f[2])
            except ValueError:
                pass
    return out


def gemm_bytes(M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one W4A16 GEMM: packed codes, scales, zeros, X and Y."""
    cells = -(-K // g) * N
    return K * N // 2 + cells * 2 + (0 if symmetric else cells // 2) + M * K * 2 + M * N * 2


def gemm_bytes_w8(M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one W8A16 GEMM: 8-bit codes, scales, byte zeros, X and Y."""
    cells = -(-K // g) * N
    return K * N + cells * 2 + (0 if symmetric else cells) + M * K * 2 + M * N * 2


def gemm_bytes_lowbit(bits, M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one 2- or 3-bit GEMM: b-bit codes, scales, 4-bit zeros, X, Y."""
    cells = -(-K // g) * N
    return K * N * bits // 8 + cells * 2 + (0 if symmetric else cells // 2) + M * K * 2 + M * N * 2


def gemm_flops(M, K, N):
    return 2 * M * N * K


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ rocprofv3 summary --

def launches_of_call(mp, M, K, N):
    """GEMM kernel launches of one mpgemm_w4a16 call the selector makes at this shape on
    MI355X's 256 compute units (two where the 256 x 256 tile runs its last round's columns
    as 256 x 128 tiles)."""
    cfg = mp.select_config(M, N, K, 128, __import__("torch").float16)
    if cfg < 12:
        return 1
    return mp.prefill_launches(M, N, K, cfg, 256)[0]


def trace_summary(csv_path, out_path, steps, warmup, cmd):
    """Writes the kernel-trace summary bench.py's roofline reads: the GEMM kernels'
    dispatches of the timed steps (12 per step, after `warmup` steps) of a rocprofv3
    --kernel-trace run of `python3 bench.py --steps S --warmup W ...`."""
    import weight_only_quantized_mpgemm_amd as mp
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gemm = [r for r in rows if "decode_kernel" in r["Kernel_Name"] or
            "prefill_x32_kernel" in r["Kernel_Name"]]
    calls = [(M, K, N) for M in MS for K, N, _ in LLAMA_SHAPES]
    per_step = sum(launches_of_call(mp, M, K, N) for M, K, N in calls)
    first = warmup * per_step
    timed = gemm[first:first + steps * per_step]
    assert len(timed) == steps * per_step, (len(gemm), first, steps)
    per_kernel, per_gemm = {}, {}
    i = 0
    for _ in range(steps):
        for M, K, N in calls:
            n = launches_of_call(mp, M, K, N)
            rs = timed[i:i + n]
            i += n
            name = mp.config_name(mp.select_config(M, N, K, 128, __import__("torch").float16))
            # a call of two launches (the 256 x 256 tile's last round as 256 x 128 tiles):
            # first start to last end, one call
            d = (int(rs[-1]["End_Timestamp"]) - int(rs[0]["Start_Timestamp"])) / 1000.0
            per_kernel.setdefault(name, []).append(d)
            per_gemm.setdefault((name, M, K, N), []).append(d)
    stats = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        stats.setdefault(r["Kernel_Name"], []).append(d)
    with open(out_path, "w") as fh:
        fh.write("# rocprofv3 kernel trace of the Llama-3-8B W4A16 step (M=1,16,2048; 12 GEMMs)\n")
        fh.write(f"# command: {cmd}\n")
        fh.write(f"# source_digest: {kernel_source_digest()}\n")
        fh.write(f"# timed steps only ({steps} steps after {warmup} warmup); durations = "
                 "End-Start per dispatch\n\n")
        fh.write("## per kernel (the figure bench.py's roofline uses: average launch duration; a "
                 "call that runs two launches counts once, first start to last end)\n")
        fh.write(f"{'kernel':24s} {'launches':>9s} {'avg_us':>10s}\n")
        for k, v in sorted(per_kernel.items()):
            fh.write(f"{k:24s} {len(v):9d} {sum(v) / len(v):10.3f}\n")
        fh.write("\n## per GEMM (TB/s and TFLOP/s of algorithmic bytes and flops)\n")
        fh.write("# kernel M K N n avg_us min_us TFLOP/s TB/s\n")
        for (k, M, K, N), v in sorted(per_gemm.items(), key=lambda x: (x[0][1], x[0][2], x[0][3])):
            a = sum(v) / len(v)
            fh.write(f"# {k:22s} {M:5d} {K:6d} {N:6d} {len(v):4d} {a:9.2f} {min(v):8.2f} "
                     f"{gemm_flops(M, K, N) / a / 1e6:8.1f} {gemm_bytes(M, K, N, 128) / a / 1e6:7.2f}\n")
        fh.write("\n## rocprofv3 kernel statistics (every dispatch of the run)\n")
        for k, v in sorted(stats.items(), key=lambda x: -sum(x[1]))[:24]:
            fh.write(f"# {k[:70]:70s} calls={len(v):6d} avg_us={sum(v) / len(v):10.3f} "
                     f"min_us={min(v):10.3f} max_us={max(v):10.3f}\n")
    print(f"wrote {out_path}")


def _pmc_dispatches(csv_path, counter):
    """[(kernel name, value)] per dispatch, in dispatch order, of one counter in a rocprofv3
    --pmc CSV (values summed over the rows of a dispatch)."""
    rows = list(csv.DictReader(open(csv_path)))
    per = {}
    for r in rows:
        if r.get("Counter_Name", counter) != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        per[d] = (name, per[d][1] + val) if d in per else (name, val)
    return [per[d] for d in sorted(per)]


def traffic_summary(fetch_csv, write_csv, out_path, steps, warmup, cmds):
    """Writes the HBM traffic summary bench.py's roofline reads, from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE) of `python3 bench.py --copy-calibration --steps S
    --warmup W --no-peaks --no-configs --no-variants --no-cpu-baseline`: counter KiB per
    dispatch of the timed steps' GEMM kernels, scaled by what the counters read for the
    1 GiB calibration copy (the first copy-kernel dispatch)."""
    import torch
    import weight_only_quantized_mpgemm_amd as mp
    calls = [(M, K, N) for M in MS for K, N, _ in LLAMA_SHAPES]
    tables, factors = [], []
    for path, counter, true_kib in ((fetch_csv, "FETCH_SIZE", 1 << 20),
                                    (write_csv, "WRITE_SIZE", 1 << 20)):
        disp = _pmc_dispatches(path, counter)
        cal = next(v for n, v in disp if "copyBuffer" in n or "copy" in n.lower())
        factors.append(true_kib / cal)
        gemm = [v for n, v in disp if "decode_kernel" in n or "prefill_x32_kernel" in n]
        per_step = sum(launches_of_call(mp, M, K, N) for M, K, N in calls)
        first = warmup * per_step
        timed = gemm[first:first + steps * per_step]
        assert len(timed) == steps * per_step, (counter, len(gemm))
        t, i = {}, 0
        for _ in range(steps):
            for c in calls:
                n = launches_of_call(mp, *c)
                t.setdefault(c, []).append(sum(timed[i:i + n]))    # the call's launches
                i += n
        tables.append({k: sum(v) / len(v) for k, v in t.items()})
        tables[-1]["_cal"] = cal
    with open(out_path, "w") as fh:
        fh.write("# HBM traffic per launch of the W4A16 kernels, Llama-3-8B step (M=1,16,2048)\n")
        fh.write(f"# command (fetch): {cmds[0]}\n# command (write): {cmds[1]}\n")
        fh.write("# calibration: first copy-kernel dispatch = the 1 GiB device copy "
                 "(--copy-calibration):\n")
        fh.write(f"#   FETCH_SIZE {tables[0]['_cal']:.1f} KiB -> factor {factors[0]:.4f}; "
                 f"WRITE_SIZE {tables[1]['_cal']:.1f} KiB -> factor {factors[1]:.4f}\n")
        fh.write(f"# bytes = (FETCH_SIZE * fetch factor + WRITE_SIZE * write factor) * 1024, "
                 f"averaged over the {steps} timed steps\n")
        fh.write(f"# source_digest: {kernel_source_digest()}\n")
        fh.write("# ratio = counted bytes / algorithmic bytes (codes + scales + zeros + X + Y)\n")
        fh.write(f"{'kernel':24s} {'M':>6s} {'K':>6s} {'N':>6s} {'fetch_kib':>12s} "
                 f"{'write_kib':>12s} {'bytes':>14s} {'algorithmic':>14s} {'ratio':>7s}\n")
        for M, K, N in calls:
            name = mp.config_name(mp.select_config(M, N, K, 128, torch.float16))
            fk, wk = tables[0][(M, K, N)], tables[1][(M, K, N)]
            by = (fk * factors[0] + wk * factors[1]) * 1024
            alg = gemm_bytes(M, K, N, 128)
            fh.write(f"{name:24s} {M:6d} {K:6d} {N:6d} {fk:12.1f} {wk:12.1f} {by:14.0f} "
                     f"{alg:14d} {by / alg:7.3f}\n")
    print(f"wrote {out_path}")


# ------------------------------------------------------------------------ CPU baseline --

def cpu_baseline_per_shape(gpu_us):
    """The oracle on the Llama-3-8B shapes: M = 1 in full on one thread (the oracle runs
    rows in parallel, so one row takes one thread whatever the host has), M = 2048 on a
    32-row sample over all host threads and on a 2-row sample on one thread (each scaled to
    2048 rows and labelled extrapolated)."""
    import oracle
    import workloads
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1))
    rows, total_s, total_flops = [], 0.0, 0
    for K, N, label in LLAMA_SHAPES:
        for M, rows_run, th in ((1, 1, 1), (2048, 32, threads), (2048, 2, 1)):
            case = workloads.make_case(workloads.LLAMA3_8B_DECODE, rows_run, K, N)
            _, secs = oracle.timed_w4a16(case["x"], case["codes"], case["scales"], case["zeros"],
                                         128, "f16", th)
            if not (th == 1 and rows_run < M):      # the 1-thread sample: reported only
                total_s += secs
                total_flops += gemm_flops(rows_run, K, N)
            t_full = secs * M / rows_run
            g = gpu_us.get((M, K, N))
            rows.append({"M": M, "K": K, "N": N, "layer": label, "threads": th,
                         "rows_timed": rows_run, "seconds": round(secs, 3),
                         "seconds_full_M": round(t_full, 3),
                         "extrapolated": rows_run != M,
                         "gflops": round(gemm_flops(M, K, N) / t_full / 1e9, 3),
                         "gpu_us": g, "speedup_gpu": round(t_full / (g * 1e-6)) if g else None})
            log(f"cpu oracle {label} M={M} ({rows_run} rows, {th} threads): {secs:.2f} s")
    summary = {"value": total_flops / total_s / 1e12, "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": "Llama-3-8B qkv/o_proj/gate_up/down: M=1 in full (1 thread) and a "
                         f"32-row sample of M=2048 ({threads} threads); dequantize + fp64 "
                         f"GEMM; {total_s:.1f} s"}
    return summary, rows


# ------------------------------------------------------------------- cold-weight pools --

LLAMA_SHAPES = ((4096, 6144, "qkv"), (4096, 4096, "o_proj"), (4096, 28672, "gate_up"),
                (14336, 4096, "down"))


@dataclasses.dataclass
class Spec:
    """One GEMM of a per-config line."""
    M: int
    K: int
    N: int
    label: str
    g: int = 128
    sym: bool = False
    act: str = "f16"            # "f16" or "bf16"
    code: str = "w4"            # "w4", "w8", "fp8", "w2", "w3"
    scale_lo: float = 0.005
    scale_hi: float = 0.02


# Counter runs: the Llama-3-8B decode GEMMs (M = 1 and 16) and prefill GEMMs (M = 2048), each
# launched once as a warm-up (left out of the summary) and then COUNTER_REPS times over
# rotating cold weight copies, one shape after another, so the dispatch order names the shape.
COUNTER_SHAPES = [(M, K, N) for M in (1, 16, 2048) for K, N, _ in LLAMA_SHAPES]
COUNTER_REPS = 4
COUNTERS = ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_WAIT_INST_ANY",
            "SQ_VALU_MFMA_BUSY_CYCLES", "FETCH_SIZE", "GRBM_GUI_ACTIVE")


def counters_workload(lib_path):
    """The launches a counter run profiles (see COUNTER_SHAPES), after the 1 GiB calibration
    copy.  lib_path: another build of libmpgemm.so (e.g. of an earlier commit) to profile
    instead of the in-tree one; exports it lacks are left out of the binding."""
    import torch
    import weight_only_quantized_mpgemm_amd as mp
    if lib_path:
        mp.LIB_PATH = os.path.abspath(lib_path)
        have = ctypes.CDLL(mp.LIB_PATH)
        for name in [n for n in mp.SIGNATURES if not hasattr(have, n)]:
            mp.SIGNATURES.pop(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.ones(1 << 29, dtype=torch.int16, device=dev)       # 1 GiB calibration copy
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    pools = {}
    # after every call, a marker (a fill of int16 zeros, a kernel nothing else launches here):
    # the summary adds up the kernels between two markers as one call (a call can run two
    # launches, e.g. the 256 x 256 tile's last round as 256 x 128 tiles)
    mark = torch.empty(1, dtype=torch.int16, device=dev)
    for M, K, N in COUNTER_SHAPES:
        if (K, N) not in pools:
            pools[(K, N)] = make_pool(mp, torch, dev, Spec(M=1, K=K, N=N, label="counters"))
        pool = pools[(K, N)]
        x = torch.randn(M, K, device=dev).half()
        y = torch.empty(M, N, device=dev, dtype=torch.float16)
        mark.fill_(7)
        torch.cuda.synchronize()
        for i in range(1 + COUNTER_REPS):
            mp.w4a16(x, pool[i % len(pool)], out=y)
            torch.cuda.synchronize()
            mark.fill_(7)
            torch.cuda.synchronize()
        log(f"counters: M={M} K={K} N={N} x {COUNTER_REPS}")


def _pmc_table(csv_path):
    """{dispatch id: (kernel name, start ns, end ns, {counter: value summed over rows})}."""
    out = {}
    for r in csv.DictReader(open(csv_path)):
        d = int(r["Dispatch_Id"])
        name, cnt = r["Kernel_Name"], r["Counter_Name"]
        if d not in out:
            out[d] = (name, int(r["Start_Timestamp"]), int(r["End_Timestamp"]), {})
        c = out[d][3]
        c[cnt] = c.get(cnt, 0.0) + float(r["Counter_Value"])
    return out


def counters_summary(runs, out_path):
    """Per-shape counter table of one or more `--counters` runs: runs = [(label, csv, cmd)]."""
    lines = ["# rocprofv3 counters of the W4A16 GEMM kernels, Llama-3-8B shapes (fp16, g = 128,",
             "# asymmetric), cold weights; averages over the timed launches of each shape",
             "# dur: End - Start of the dispatch under counter collection (short kernels run slower",
             "# than in a graph replay); clock = GRBM_GUI_ACTIVE / 8 XCDs / dur, shown from 50 us on",
             "# (the counter also runs outside the dispatch, which dominates short ones); MFMA busy =",
             "# SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024 SIMDs); VALU = SQ_INSTS_VALU",
             "# in millions; wait/wave = SQ_WAIT_INST_ANY * 4 cycles / SQ_WAVES;",
             "# VALU/wave = SQ_INSTS_VALU / SQ_WAVES; fetch = FETCH_SIZE KiB scaled by the 1 GiB copy's",
             "# reading, against the algorithmic bytes (codes + scales + zeros + X + Y)",
             f"# source_digest (current sources): {kernel_source_digest()}"]
    for label, path, cmd in runs:
        table = _pmc_table(path)
        ids = sorted(table)
        cal = next(d for d in ids if "copy" in table[d][0].lower())
        factor = (1 << 20) / table[cal][3]["FETCH_SIZE"]
        # calls: the GEMM kernels between two markers (int16 fills), in order
        calls, cur, started = [], [], False
        for d in ids[ids.index(cal) + 1:]:
            name = table[d][0]
            if "FillFunctor<short>" in name:
                if started and cur:
                    calls.append(cur)
                cur, started = [], True
            elif started and ("decode_kernel" in name or "prefill_x32_kernel" in name):
                cur.append(d)
        per = 1 + COUNTER_REPS
        assert len(calls) == per * len(COUNTER_SHAPES), (label, len(calls))
        lines += ["", f"## {label}", f"# command: {cmd}", f"# FETCH_SIZE calibration factor {factor:.4f}",
                  "# kernel                  M      K      N   dur_us  clk_GHz  mfma_busy  waves"
                  "   VALU/wave  VALU_M  wait_cyc/wave  fetch_MB  fetch/alg"]
        for i, (M, K, N) in enumerate(COUNTER_SHAPES):
            cs = calls[i * per + 1:(i + 1) * per]
            ds = [d for c in cs for d in c]
            avg = {c: sum(table[d][3].get(c, 0.0) for d in ds) / len(cs) for c in COUNTERS}
            # a call's duration: its kernels' durations added (counter collection serializes
            # the launches of a call with gaps of its own between them)
            dur = sum(table[d][2] - table[d][1] for d in ds) / len(cs)             # ns
            gui = avg["GRBM_GUI_ACTIVE"] / 8
            clk = gui / dur
            mfma = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024) if gui else 0.0
            waves = avg["SQ_WAVES"]
            fetch = avg["FETCH_SIZE"] * factor * 1024
            alg = gemm_bytes(M, K, N, 128)
            kname = "prefill_x32" if "prefill" in table[ds[0]][0] else "decode"
            clk_s = f"{clk:8.3f}" if dur >= 50e3 else f"{'-':>8s}"
            lines.append(f"  {kname:20s} {M:5d} {K:6d} {N:6d} {dur / 1e3:8.2f} {clk_s} "
                         f"{mfma:10.3f} {waves:6.0f} {avg['SQ_INSTS_VALU'] / waves:11.1f} "
                         f"{avg['SQ_INSTS_VALU'] / 1e6:7.3f} "
                         f"{avg['SQ_WAIT_INST_ANY'] * 4 / waves:14.0f} {fetch / 1e6:9.2f} "
                         f"{fetch / alg:9.3f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out_path}")


def make_pool(mp, torch, dev, spec, min_copies=3):
    """Packed-weight copies of one shape, random codes and zeros with valid fp16 scales in
    [scale_lo, scale_hi], enough of them that COLD_BYTES pass between two reads of a copy.
    (Timing does not depend on the values; the codes are uniform like real ones.)"""
    K, N, g = spec.K, spec.N, spec.g
    lib = mp.lib()
    if spec.code == "w4":
        cb = lib.mpgemm_packed_code_bytes(K, N)
        mb = lib.mpgemm_packed_meta_bytes(K, N, g, int(spec.sym))
        bits, fp8 = 4, None
    elif spec.code in ("w8", "fp8"):
        cb = lib.mpgemm_packed_code_bytes_w8(K, N)
        mb = lib.mpgemm_packed_meta_bytes_w8(K, N, g, int(spec.sym or spec.code == "fp8"))
        bits, fp8 = 8, ("e4m3" if spec.code == "fp8" else None)
    else:
        b = int(spec.code[1])
        cb = lib.mpgemm_packed_code_bytes_lowbit(b, K, N)
        mb = lib.mpgemm_packed_meta_bytes(K, N, g, int(spec.sym))
        bits, fp8 = b, None
    Kp, Np = -(-K // 128) * 128, -(-N // 16) * 16     # the packed planes' padded shape
    cells = (Kp // g) * Np
    copies = max(min_copies, math.ceil(COLD_BYTES / (cb + mb)) + 1)
    pool = []
    for _ in range(copies):
        codes = torch.randint(0, 256, (cb,), dtype=torch.uint8, device=dev)
        if fp8:
            codes &= 0xF7          # finite E4M3 codes (no all-ones exponent and mantissa)
        meta = torch.randint(0, 256, (mb,), dtype=torch.uint8, device=dev)
        sc = meta[:cells * 2].view(torch.float16)
        sc.uniform_(spec.scale_lo, spec.scale_hi)
        pool.append(mp.PackedWeights(codes, meta, K, N, g, spec.sym, bits, fp8))
    return pool


class TimingEvent:
    """A HIP event made with hipEventDisableSystemFence, for the timed steps' run
    boundaries: recording it skips the system-scope release (a cache writeback) that a
    default event performs, which the next kernel would otherwise wait for.  The events
    only time work that torch.cuda.synchronize() has already waited for."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self.ev = ctypes.c_void_p()
        st = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                      self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream):
        st = TimingEvent._hip.hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_ms(self, later):
        ms = ctypes.c_float()
        st = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, later.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.ev:
            TimingEvent._hip.hipEventDestroy(self.ev)


def time_cold(torch, stream, launch, n):
    """Average time (s) of one launch in a HIP graph of n launches (launch(i) for each),
    replayed once after a warm replay."""
    for i in range(min(n, 2)):
        launch(i)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(n):
            launch(i)
    gr.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    gr.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del gr
    return e0.elapsed_time(e1) * 1e-3 / n


# -------------------------------------------------------------------------- peaks -------

def measure_peaks(torch, dev, stream):
    """Cold stream-read floors at byte counts from 4 MiB to 1 GiB, and the MFMA loop rates,
    from libmpgemm_probes.so."""
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_quantized_mpgemm_amd", "libmpgemm_probes.so"))
    lib.mpgemm_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mpgemm_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    pool_bytes = 3 << 30
    pool = torch.randint(0, 255, (pool_bytes,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    def cur():
        # read at call time: under graph capture torch runs on its capture stream
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    reads = []
    for mib in (4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 512, 1024):
        nbytes = mib << 20
        slots = pool_bytes // nbytes
        n = max(4, min(slots, 64))
        best = None
        for chunk, unroll in ((16, 4), (32, 8), (64, 8)):
            def launch(i, nbytes=nbytes, chunk=chunk, unroll=unroll, slots=slots):
                off = (i % slots) * nbytes
                st = lib.mpgemm_probe_hbm_read(ctypes.c_void_p(pool.data_ptr() + off), nbytes,
                                               chunk, unroll, ctypes.c_void_p(sink.data_ptr()),
                                               cur())
                assert st == 0, st
            t = time_cold(torch, stream, launch, n)
            if best is None or t < best[0]:
                best = (t, chunk, unroll)
        reads.append({"MiB": mib, "us": round(best[0] * 1e6, 2),
                      "tbps": round(nbytes / best[0] / 1e12, 3), "chunk_kib": best[1],
                      "unroll": best[2]})
    del pool
    msink = torch.zeros(512 * 256, dtype=torch.float32, device=dev)
    names = {0: "32x32x16_f16", 1: "16x16x32_f16", 2: "32x32x16_bf16", 3: "16x16x32_bf16"}
    mfma = {}
    for kind in range(4):
        iters, blocks = 4000, 512

        def launch(i, kind=kind):
            assert lib.mpgemm_probe_mfma(kind, iters, blocks, ctypes.c_void_p(msink.data_ptr()),
                                         cur()) == 0
        t = time_cold(torch, stream, launch, 4)
        mfma[names[kind]] = round(blocks * 4 * iters * 4 * 32768 / t / 1e12, 1)
    torch.cuda.empty_cache()
    return {"hbm_read_floor": reads, "mfma_tflops": mfma,
            "method": "cold stream reads (best of 3 probe shapes; every launch reads bytes not "
                      "read within 1 GiB) and four independent in-place MFMA chains per wave "
                      "on non-zero data, 2 waves per SIMD"}


def floor_us(peaks, nbytes):
    """Stream-read time of nbytes (linear between the measured sizes, proportional above)."""
    pts = [(r["MiB"] * 2**20, r["us"]) for r in peaks["hbm_read_floor"]]
    if nbytes <= pts[0][0]:
        return pts[0][1]
    for (a, ta), (b, tb) in zip(pts, pts[1:]):
        if nbytes <= b:
            return ta + (tb - ta) * (nbytes - a) / (b - a)
    return pts[-1][1] * nbytes / pts[-1][0]


def gemm_line(spec, t, peaks, kernel, bytes_fn=None):
    """One GEMM's record: time, rates, and fractions of the published and measured peaks."""
    M, K, N = spec.M, spec.K, spec.N
    by = (bytes_fn or (lambda: gemm_bytes(M, K, N, spec.g, spec.sym)))()
    fl = gemm_flops(M, K, N)
    bound = "hbm" if fl / by < 315 else "mfma"
    rec = {"M": M, "K": K, "N": N, "layer": spec.label, "kernel": kernel,
           "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
           "gbps": round(by / t / 1e9, 1), "bound": bound}
    if bound == "hbm":
        rec["frac"] = round(by / t / 1e9 / HBM_PEAK_GBPS, 4)
        if peaks:
            rec["frac_measured"] = round(floor_us(peaks, by) * 1e-6 / t, 4)
    else:
        rec["frac"] = round(fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
        if peaks:
            pk = max(v for k, v in peaks["mfma_tflops"].items() if k.endswith(spec.act))
            rec["frac_measured"] = round(fl / t / 1e12 / pk, 4)
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pool-gb", type=float, default=1.5,
                    help="size of the rotating pool of packed weight copies (timed steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the probe measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config lines (counter runs use this)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other code formats, small-M prefill and attention passes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy, whose HBM "
                         "counter readings scale the counter-based traffic figures")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "OUT"),
                    help="summarize a rocprofv3 kernel trace of this command's timed steps "
                         "(with the same --steps/--warmup) into OUT, then exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "command with --copy-calibration into OUT, then exit")
    ap.add_argument("--counters", action="store_true",
                    help="run only the counter workload (the Llama-3-8B GEMMs at M = 1, 16 and "
                         "2048, cold) for a rocprofv3 --pmc run, then exit")
    ap.add_argument("--lib", default="",
                    help="with --counters: profile this build of libmpgemm.so instead")
    ap.add_argument("--counters-summary", nargs="+", metavar="LABEL=CSV",
                    help="summarize --counters runs (LABEL=CSV, one per run; --trace-command "
                         "gives their commands separated by '|') into the last argument, "
                         "then exit")
    ap.add_argument("--trace-command", default="",
                    help="the profiled command(s), recorded in a summary ('|' between the "
                         "fetch and write commands of --traffic-summary)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would "
              "run its own shard of N or K independently); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.trace_summary[1], args.steps, args.warmup,
                      args.trace_command)
        return
    if args.traffic_summary:
        cmds = (args.trace_command.split("|") + ["", ""])[:2]
        traffic_summary(*args.traffic_summary, args.steps, args.warmup, [c.strip() for c in cmds])
        return
    if args.counters_summary:
        *pairs, out = args.counters_summary
        cmds = [c.strip() for c in args.trace_command.split("|")] + [""] * len(pairs)
        counters_summary([(p.split("=", 1)[0], p.split("=", 1)[1], cmds[i])
                          for i, p in enumerate(pairs)], out)
        return
    if args.counters:
        counters_workload(args.lib)
        return

    import numpy as np
    import torch

    import weight_only_quantized_mpgemm_amd as mp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)       # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
    wl = workloads.LLAMA3_8B_DECODE
    shapes = wl.shapes
    g = wl.group

    # ---- the timed step: one seeded layer, replicated into a rotating pool ----
    layer = []
    for K, N, label in shapes:
        codes, scales, zeros = workloads.weights(K, N, g, False, wl.scale_lo, wl.scale_hi,
                                                 workloads.seed_for("bench", 0, K, N))
        packed = mp.pack_weights(torch.from_numpy(codes).to(dev),
                                 torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.float16),
                                 torch.from_numpy(zeros).to(dev), g)
        layer.append(packed)
    torch.cuda.synchronize()
    layer_bytes = sum(p.nbytes for p in layer)
    copies = max(3 * len(MS), int(np.ceil(args.pool_gb * 1e9 / layer_bytes)))
    pool = [layer] + [[mp.PackedWeights(p.codes.clone(), p.meta.clone(), p.K, p.N, p.group,
                                        p.symmetric) for p in layer] for _ in range(copies - 1)]
    torch.cuda.synchronize()
    log(f"weight pool: {copies} copies x {layer_bytes / 1e6:.1f} MB")

    xs, ys = {}, {}
    for M in MS:
        for K in sorted({k for k, _, _ in shapes}):
            bits = workloads.activations(M, K, "f16", workloads.seed_for("bench-x", M, K, 0))
            xs[(M, K)] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)
        for N in sorted({n for _, n, _ in shapes}):
            ys[(M, N)] = torch.empty((M, N), dtype=torch.float16, device=dev)

    calls = [(M, K, N, label) for M in MS for K, N, label in shapes]
    cfg_of = {c: mp.select_config(c[0], c[2], c[1], g, torch.float16) for c in calls}
    # runs of consecutive launches of one kernel at one M within a step: (kernel, [calls])
    runs = []
    for c in calls:
        name = mp.config_name(cfg_of[c])
        if runs and runs[-1][0] == name and runs[-1][1][-1][0] == c[0]:
            runs[-1][1].append(c)
        else:
            runs.append((name, [c]))
    shape_idx = {(K, N): j for j, (K, N, _) in enumerate(shapes)}

    def step(s, evs=None):
        for r, (_, rcalls) in enumerate(runs):
            if evs is not None:
                evs[r].record(stream)
            for M, K, N, label in rcalls:
                c = (s * len(MS) + MS.index(M)) % copies
                mp.w4a16(xs[(M, K)], pool[c][shape_idx[(K, N)]], out=ys[(M, N)])
        if evs is not None:
            evs[-1].record(stream)

    for s in range(args.warmup):
        step(s)
    # every event exists before the timed region (creating one can reach into the driver)
    run_events = [[TimingEvent() for _ in range(len(runs) + 1)]
                  for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, run_events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    step_s = elapsed / args.steps
    step_flops = sum(gemm_flops(M, K, N) for M, K, N, _ in calls)
    step_bytes = sum(gemm_bytes(M, K, N, g) for M, K, N, _ in calls)

    # per kernel: total event time over the timed steps, launches, flops and bytes
    per_cfg = {}
    for r, (name, rcalls) in enumerate(runs):
        t = sum(evs[r].elapsed_ms(evs[r + 1]) * 1e-3 for evs in run_events)
        agg = per_cfg.setdefault(name, {"t": 0.0, "flops": 0, "bytes": 0, "n": 0, "calls": [],
                                        "bound": "hbm" if rcalls[0][0] <= 64 else "mfma"})
        agg["t"] += t
        agg["n"] += len(rcalls) * args.steps
        agg["flops"] += sum(gemm_flops(M, K, N) for M, K, N, _ in rcalls) * args.steps
        agg["bytes"] += sum(gemm_bytes(M, K, N, g) for M, K, N, _ in rcalls) * args.steps
        agg["calls"] += rcalls

    traffic = load_traffic()
    trace = load_trace()

    def roofline(cfg):
        a = per_cfg[cfg]
        avg_launch_s = a["t"] / a["n"]
        tr = [traffic.get((cfg, M, K, N)) for M, K, N, _ in a["calls"]]
        tr = round(sum(tr) / len(tr)) if tr and None not in tr else None
        per_launch = (a["flops"] if a["bound"] == "mfma" else a["bytes"]) / a["n"]
        common = {"kernel": cfg, "launches_per_step": a["n"] // args.steps,
                  "avg_launch_us": round(avg_launch_s * 1e6, 3),
                  "algorithmic_bytes_per_launch": round(a["bytes"] / a["n"]),
                  "algorithmic_flops_per_launch": round(a["flops"] / a["n"])}
        prof = trace.get(cfg)
        if a["bound"] == "mfma":
            ach = a["flops"] / a["t"] / 1e12
            out = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                   "traffic": tr, **common}
            if prof:
                out["avg_launch_us_profile"] = prof
                out["frac_profile"] = round(per_launch / (prof * 1e-6) / 1e12 /
                                            MFMA_F16_PEAK_TFLOPS, 4)
            return out
        ach = a["bytes"] / a["t"] / 1e9
        out = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
               "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": tr, **common}
        if prof:
            out["avg_launch_us_profile"] = prof
            out["frac_profile"] = round(per_launch / (prof * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        return out

    dominant = max(per_cfg, key=lambda k: per_cfg[k]["t"])
    rl = {"roofline": roofline(dominant), "roofline_by_kernel": {k: roofline(k) for k in per_cfg}}
    log(f"step {step_s * 1e3:.3f} ms, {step_flops / step_s / 1e12:.1f} TFLOP/s")
    del pool, layer
    torch.cuda.empty_cache()

    # ---- measured peaks ----
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(torch, dev, stream)
        log(f"peaks: read {[(r['MiB'], r['tbps']) for r in peaks['hbm_read_floor']]} "
            f"mfma {peaks['mfma_tflops']}")

    def cold_pass(specs, gemm_fn, bytes_fn=None):
        """Cold per-launch timing of each spec; one pool per distinct (K, N, code)."""
        rows, cur = [], None
        for sp in specs:
            key = (sp.K, sp.N, sp.code, sp.g, sp.sym)
            if cur is None or cur[0] != key:
                cur = None
                torch.cuda.empty_cache()
                cur = (key, make_pool(mp, torch, dev, sp))
            cpool = cur[1]
            dt = torch.float16 if sp.act == "f16" else torch.bfloat16
            x = torch.randn(sp.M, sp.K, device=dev).to(dt)
            y = torch.empty(sp.M, sp.N, device=dev, dtype=dt)
            n = len(cpool)

            def launch(i):
                gemm_fn(x, cpool[i % n], out=y)
            t = time_cold(torch, stream, launch, n)
            kern = mp.config_name(mp.select_config(sp.M, sp.N, sp.K, sp.g, dt))
            bf = (lambda sp=sp: bytes_fn(sp)) if bytes_fn else None
            rows.append(gemm_line(sp, t, peaks, kern, bf))
            del x, y
        del cur
        torch.cuda.empty_cache()
        return rows

    # ---- per-config lines: every GEMM of the workloads, cold per launch ----
    configs = {}
    if not args.no_configs:
        L8 = LLAMA_SHAPES
        L70 = workloads.LLAMA3_70B.shapes
        Q32 = workloads.QWEN3_32B.shapes
        sets = {
            "llama3_8b_w4a16_g128_decode": [Spec(M, K, N, lab) for K, N, lab in L8
                                            for M in (1, 8, 16)],
            "llama3_8b_w4a16_g128_prefill": [Spec(M, K, N, lab) for K, N, lab in L8
                                             for M in (512, 2048, 8192)],
            "llama3_70b_w4a16_g128_bf16": [Spec(M, K, N, lab, act="bf16") for K, N, lab in L70
                                           for M in (1, 64, 4096)],
            "qwen3_32b_w4a16_g64_sym": [Spec(M, K, N, lab, g=64, sym=True, scale_lo=0.002,
                                             scale_hi=0.01) for K, N, lab in Q32
                                        for M in (1, 2, 4, 16, 128, 1024, 8192)],
        }
        for name, specs in sets.items():
            configs[name] = cold_pass(specs, mp.w4a16)
            log(f"{name}: " + ", ".join(f"{r['M']}x{r['K']}x{r['N']} {r['us']}us "
                                        f"{r['frac']:.2f}" for r in configs[name]))

    # ---- other code formats, small prefill, attention ----
    variants = {}
    if not args.no_variants:
        variants["w4a16_small_m_per_gemm"] = cold_pass(
            [Spec(M, K, N, lab) for M in (128, 256, 512) for K, N, lab in LLAMA_SHAPES], mp.w4a16)
        variants["w8a16_per_gemm"] = cold_pass(
            [Spec(M, K, N, lab, code="w8", scale_lo=0.005 / 16, scale_hi=0.02 / 16)
             for K, N, lab in LLAMA_SHAPES for M in MS], mp.w8a16,
            lambda sp: gemm_bytes_w8(sp.M, sp.K, sp.N, sp.g))
        variants["wfp8a16_qwen3_8b_per_gemm"] = cold_pass(
            [Spec(M, K, N, lab, sym=True, act="bf16", code="fp8", scale_lo=0.005 / 64,
                  scale_hi=0.02 / 64) for K, N, lab in workloads.QWEN3_8B_SHAPES for M in MS],
            mp.wfp8a16, lambda sp: gemm_bytes_w8(sp.M, sp.K, sp.N, sp.g, symmetric=True))
        for bits in (2, 3):
            variants[f"w{bits}a16_per_gemm"] = cold_pass(
                [Spec(M, K, N, lab, code=f"w{bits}", scale_lo=0.01, scale_hi=0.05)
                 for K, N, lab in LLAMA_SHAPES for M in MS], mp.wlowbit_a16,
                lambda sp, b=bits: gemm_bytes_lowbit(b, sp.M, sp.K, sp.N, sp.g))
        variants["attention_kv8_decode"] = attention_pass(args, dev, stream, None, torch, mp)
        variants["attention_kvfp8_decode"] = attention_pass(args, dev, stream, "e4m3", torch, mp)

    out = {
        "metric": "W4A16 GEMM TFLOP/s and HBM GB/s (% roofline), Llama-3-8B shapes M=1/16/2048",
        "value": round(step_flops / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b W4A16 g128 asym fp16: qkv 4096x6144, o_proj "
                               "4096x4096, gate_up 4096x28672, down 14336x4096 at "
                               "M=1,16,2048 (12 GEMMs per step)",
                   "weight_pool_copies": copies, "group": g, "launch": "eager"},
        "hbm_gbps": round(step_bytes / step_s / 1e9, 1),
        **rl,
        "peaks": peaks,
        "configs": configs,
        **variants,
        "kernel_source_digest": kernel_source_digest(),
    }
    if not args.no_cpu_baseline:
        gpu_us = {}
        for r in configs.get("llama3_8b_w4a16_g128_decode", []) + \
                configs.get("llama3_8b_w4a16_g128_prefill", []):
            gpu_us[(r["M"], r["K"], r["N"])] = r["us"]
        out["cpu_baseline"], out["cpu_baseline_per_shape"] = cpu_baseline_per_shape(gpu_us)
    print(json.dumps(out), flush=True)


def attention_pass(args, dev, stream, fp8, torch, mp):
    """Decode attention (mpgemm_attention_decode_kv8, or _kvfp8 for an FP8 format) at batch x
    context 1 x 8192, 16 x 2048, 64 x 2048 and 128 x 4096, cold per launch: one HIP graph of
    calls over block tables that each point at blocks no other call of the graph reads, at
    least 1.2 GB of them."""
    Hq, Hkv, D = 32, 8, 128
    bb = mp.kv_block_bytes(Hkv, D)
    nblocks = int(max(args.pool_gb, 2.5) * 1e9 // bb)
    cache = torch.randint(0, 256, (nblocks * bb,), dtype=torch.uint8, device=dev)
    if fp8:
        cache &= 0xF7          # finite E4M3 and E5M2 codes (no all-ones exponent / NaN)
    blk = cache.view(nblocks, Hkv, bb // Hkv)
    blk[:, :, 128 * D:128 * D + 256].view(torch.float16).fill_(0.01)

    def call(q, table, lens, T, scale, o):
        if fp8:
            mp.attention_decode_kvfp8(q, cache, table, lens, Hkv, T, scale, fp8, out=o)
        else:
            mp.attention_decode_kv8(q, cache, table, lens, Hkv, T, scale, out=o)

    res = []
    for B, T in ((1, 8192), (16, 2048), (64, 2048), (128, 4096)):
        nb = (T + 63) // 64
        ntab = nblocks // (B * nb)
        if ntab < 2:
            continue
        reps = max(2, min(ntab, math.ceil(COLD_BYTES / (B * nb * bb)) + 1))
        tables = [torch.arange(r * B * nb, (r + 1) * B * nb, dtype=torch.int32, device=dev)
                  .view(B, nb) for r in range(reps)]
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        q = torch.randn(B, Hq, D, device=dev).to(torch.float16)
        o = torch.empty_like(q)
        scale = 1.0 / D ** 0.5
        t = time_cold(torch, stream, lambda i: call(q, tables[i], lens, T, scale, o), reps)
        per_tok = 2 * D + 4 + (0 if fp8 else 2)
        by = B * Hkv * T * per_tok + 2 * B * Hq * D * 2 + B * nb * 4
        res.append({"B": B, "context": T, "heads": [Hq, Hkv, D], "us": round(t * 1e6, 2),
                    "gbps": round(by / t / 1e9, 1), "bound": "hbm",
                    "frac": round(by / t / 1e9 / HBM_PEAK_GBPS, 4)})
    del cache, blk
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
