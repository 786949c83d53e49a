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
kernel, a per-GEMM breakdown and the CPU oracle timed on a bounded sample (cpu_baseline).

The timed steps launch every GEMM from Python (--graph instead captures each M's four
GEMMs per weight copy as a HIP graph and replays it; measured, that is no faster here,
because a replay starts later after the preceding event than an eager launch does).
Kernel durations come from hipEvents recorded, inside the timed steps, on the stream the
library launches on, around each run of consecutive launches of one kernel (the four GEMMs
of one M), divided by the launches in it; host launch gaps of a few microseconds still
inflate the 6-20 us decode kernels there.  The per-GEMM breakdown is a separate pass after
the timed steps: ten back-to-back launches per GEMM replayed from one HIP graph between
one pair of events, which keeps host gaps out.  `traffic` is the HBM bytes per
launch that rocprofv3's FETCH_SIZE and WRITE_SIZE counters read for the dominant kernel,
scaled by what the same counters read for a plain 1 GiB copy (--copy-calibration); it is
taken from the summary file under profiles/ and reported only while the kernel sources
still hash to the digest recorded there, else null.

`w4a16_small_m_per_gemm` repeats the per-GEMM pass at M = 128, 256 and 512 (grids of fewer
tiles than compute units, where the tiled kernels split K), against the MFMA roofline.
`w8a16_per_gemm` repeats the per-GEMM pass with 8-bit weights (mpgemm_w8a16, same shapes,
its own rotating pool), each GEMM against the HBM roofline (M <= 64; bytes count one byte
per code and per zero) or the fp16 MFMA roofline.  `wfp8a16_qwen3_8b_per_gemm` does the
same with FP8 (E4M3) weights at the Qwen3-8B projection shapes (QKV 4096x6144, O 4096x4096,
gate_up 4096x24576, down 12288x4096) and bf16 activations (mpgemm_wfp8a16; one byte per
code, no zeros).  `w2a16_per_gemm` and `w3a16_per_gemm` do it with 2-bit and 3-bit weights
(mpgemm_wlowbit_a16) at the Llama-3-8B shapes for M = 1 and 16, against the HBM roofline,
and M = 2048 (the codes rewritten in the 4-bit layout, then the tiled kernel) against the
fp16 MFMA roofline.
`attention_kv8_decode` times mpgemm_attention_decode_kv8 (Llama-3-8B heads, one query token
per sequence, batch x context 1 x 8192, 16 x 2048, 64 x 2048, 128 x 4096) against the HBM
roofline (bytes: K and V codes, scales and zeros, Q, O, the block table);
`attention_kvfp8_decode` does the same over an E4M3 cache (mpgemm_attention_decode_kvfp8;
no zeros).  None of these is part of `value`.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
MS = (1, 16, 2048)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a16_llama3_8b_m1_16_2048_hbm_traffic.txt")


def kernel_source_digest():
    """sha256 (16 hex digits) over the HIP sources and the build flags of the library's GEMM
    path (everything but the attention kernels, which the GEMM profiles do not cover)."""
    pkg = os.path.join(ROOT, "weight_only_quantized_mpgemm_amd")
    csrc = os.path.join(pkg, "csrc")
    h = hashlib.sha256()
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
             if f.endswith((".hip", ".hpp")) and f != "attention.hip"] + \
        [os.path.join(pkg, "build.py")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """{(kernel, M, K, N): scaled HBM bytes per launch} from the counter summary, or {} when
    the file is absent or was taken from other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    table, digest = {}, None
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("# source_digest:"):
                digest = line.split(":", 1)[1].strip()
            elif line.strip() and not line.startswith("#"):
                f = line.split()
                if f[0] == "kernel":
                    continue
                table[(f[0], int(f[1]), int(f[2]), int(f[3]))] = float(f[6])
    return table if digest == kernel_source_digest() else {}


def gemm_bytes(M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one W4A16 GEMM: packed codes, scales, zeros, X and Y."""
    cells = (K // g) * N
    return K * N // 2 + cells * 2 + (0 if symmetric else cells // 2) + M * K * 2 + M * N * 2


def gemm_bytes_w8(M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one W8A16 GEMM: 8-bit codes, scales, byte zeros, X and Y."""
    cells = (K // g) * N
    return K * N + cells * 2 + (0 if symmetric else cells) + M * K * 2 + M * N * 2


def gemm_bytes_lowbit(bits, M, K, N, g, symmetric=False):
    """Algorithmic HBM bytes of one 2- or 3-bit GEMM: b-bit codes, scales, 4-bit zeros, X, Y."""
    cells = (K // g) * N
    return K * N * bits // 8 + cells * 2 + (0 if symmetric else cells // 2) + M * K * 2 + M * N * 2


def gemm_flops(M, K, N):
    return 2 * M * N * K


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(shapes, group, m_rows=32):
    """The oracle, as it stands, on M = m_rows rows of every shape (full N)."""
    import oracle
    import workloads
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1))
    total_s, flops = 0.0, 0
    for K, N, label in shapes:
        case = workloads.make_case(workloads.LLAMA3_8B_DECODE, m_rows, K, N)
        _, secs = oracle.timed_w4a16(case["x"], case["codes"], case["scales"], case["zeros"],
                                     group, "f16", threads)
        total_s += secs
        flops += gemm_flops(m_rows, K, N)
        log(f"cpu oracle {label} M={m_rows}: {secs:.2f} s")
    return {"value": flops / total_s / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"M={m_rows} rows x all four Llama-3-8B shapes (full K, N), "
                      f"dequantize + fp64 GEMM, {total_s:.1f} s"}


def attention_pass(args, dev, stream, fp8):
    """Times decode attention (mpgemm_attention_decode_kv8, or _kvfp8 for an FP8 format) at
    batch x context 1 x 8192, 16 x 2048, 64 x 2048 and 128 x 4096 under a HIP graph."""
    import torch
    import weight_only_quantized_mpgemm_amd as mp
    Hq, Hkv, D = 32, 8, 128
    bb = mp.kv_block_bytes(Hkv, D)
    # at least two block tables of the largest case (128 x 4096: 1.1 GB each)
    nblocks = int(max(args.pool_gb, 2.5) * 1e9 // bb)
    cache = torch.randint(0, 256, (nblocks * bb,), dtype=torch.uint8, device=dev)
    if fp8:
        cache &= 0xF7          # finite E4M3 and E5M2 codes (no all-ones exponent / NaN)
    # valid fp16 scales (0.01) in every block's scale fields
    blk = cache.view(nblocks, Hkv, bb // Hkv)
    blk[:, :, 128 * D:128 * D + 256].view(torch.float16).fill_(0.01)

    def call(q, table, lens, T, scale, o):
        if fp8:
            mp.attention_decode_kvfp8(q, cache, table, lens, Hkv, T, scale, fp8, out=o)
        else:
            mp.attention_decode_kv8(q, cache, table, lens, Hkv, T, scale, out=o)

    res, reps = [], 10
    for B, T in ((1, 8192), (16, 2048), (64, 2048), (128, 4096)):
        nb = (T + 63) // 64
        ntab = min(reps, nblocks // (B * nb))
        if ntab < 2:
            continue
        tabs = [torch.arange(r * B * nb, (r + 1) * B * nb, dtype=torch.int32, device=dev)
                .view(B, nb) for r in range(ntab)]
        tables = [tabs[r % ntab] for r in range(reps)]
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        q = torch.randn(B, Hq, D, device=dev).to(torch.float16)
        o = torch.empty_like(q)
        scale = 1.0 / D ** 0.5
        for r in range(reps):               # warm (and allocate the workspace)
            call(q, tables[r], lens, T, scale, o)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for r in range(reps):
                call(q, tables[r], lens, T, scale, o)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        # codes, fp16 scales (and 8-bit zeros: none for FP8), Q and O, the block table
        per_tok = 2 * D + 4 + (0 if fp8 else 2)
        by = B * Hkv * T * per_tok + 2 * B * Hq * D * 2 + B * nb * 4
        res.append({"B": B, "context": T, "heads": [Hq, Hkv, D], "us": round(t * 1e6, 2),
                    "gbps": round(by / t / 1e9, 1), "bound": "hbm",
                    "frac": round(by / t / 1e9 / HBM_PEAK_GBPS, 4)})
        del gr
    del cache, blk
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pool-gb", type=float, default=1.5,
                    help="size of the rotating pool of packed weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from captured HIP graphs")
    ap.add_argument("--no-per-gemm", action="store_true",
                    help="skip the per-GEMM breakdown pass (counter runs use this)")
    ap.add_argument("--no-small-m", action="store_true",
                    help="skip the W4A16 pass at M = 128, 256, 512")
    ap.add_argument("--no-w8", action="store_true",
                    help="skip the W8A16 per-GEMM pass (8-bit weights, same shapes)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8-weight per-GEMM pass (E4M3, Qwen3-8B shapes)")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the attention-decode passes (8-bit and FP8 KV caches)")
    ap.add_argument("--no-lowbit", action="store_true",
                    help="skip the 2-bit and 3-bit per-GEMM passes (Llama-3-8B shapes, M=1,16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy, whose HBM "
                         "counter readings scale the counter-based traffic figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would "
              "run its own shard of N or K independently); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import weight_only_quantized_mpgemm_amd as mp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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

    # ---- packed weights: one seeded layer, replicated into a rotating pool ----
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
    stream = torch.cuda.current_stream(dev)
    # runs of consecutive launches of one kernel at one M within a step: (kernel, [calls])
    runs, run_starts = [], set()
    for i, c in enumerate(calls):
        name = mp.config_name(cfg_of[c])
        if runs and runs[-1][0] == name and runs[-1][1][-1][0] == c[0]:
            runs[-1][1].append(c)
        else:
            runs.append((name, [c]))
            run_starts.add(i)
    run_events = []
    shape_idx = {(K, N): j for j, (K, N, _) in enumerate(shapes)}

    def launch_m(M, c):
        for K, N, _ in shapes:
            mp.w4a16(xs[(M, K)], pool[c][shape_idx[(K, N)]], out=ys[(M, N)])

    # One graph per (M, weight copy): the four launches of one M are one run of one kernel.
    use_graphs = args.graph and all(
        sum(1 for _, rc in runs if rc[0][0] == M) == 1 for M in MS)
    graphs = {}
    if use_graphs:
        for M in MS:
            launch_m(M, 0)                     # load the library and kernels before capture
        torch.cuda.synchronize()
        for c in range(copies):
            for M in MS:
                g_ = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_):
                    launch_m(M, c)
                graphs[(M, c)] = g_
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} graphs")

    def step(s, record):
        evs = []
        for i, (M, K, N, label) in enumerate(calls):
            c = (s * len(MS) + MS.index(M)) % copies
            if record and i in run_starts:
                evs.append(torch.cuda.Event(enable_timing=True))
                evs[-1].record(stream)
            if use_graphs:
                if shape_idx[(K, N)] == 0:
                    graphs[(M, c)].replay()
            else:
                mp.w4a16(xs[(M, K)], pool[c][shape_idx[(K, N)]], out=ys[(M, N)])
        if record:
            evs.append(torch.cuda.Event(enable_timing=True))
            evs[-1].record(stream)
            run_events.append(evs)

    for s in range(args.warmup):
        step(s, record=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    step_s = elapsed / args.steps
    step_flops = sum(gemm_flops(M, K, N) for M, K, N, _ in calls)
    step_bytes = sum(gemm_bytes(M, K, N, g) for M, K, N, _ in calls)

    # per kernel: total event time over the timed steps, launches, flops and bytes
    per_cfg = {}
    for r, (name, rcalls) in enumerate(runs):
        t = sum(evs[r].elapsed_time(evs[r + 1]) * 1e-3 for evs in run_events)
        agg = per_cfg.setdefault(name, {"t": 0.0, "flops": 0, "bytes": 0, "n": 0, "calls": [],
                                        "bound": "hbm" if rcalls[0][0] <= 64 else "mfma"})
        agg["t"] += t
        agg["n"] += len(rcalls) * args.steps
        agg["flops"] += sum(gemm_flops(M, K, N) for M, K, N, _ in rcalls) * args.steps
        agg["bytes"] += sum(gemm_bytes(M, K, N, g) for M, K, N, _ in rcalls) * args.steps
        agg["calls"] += rcalls

    traffic = load_traffic()

    def roofline(cfg):
        a = per_cfg[cfg]
        avg_launch_s = a["t"] / a["n"]
        tr = [traffic.get((cfg, M, K, N)) for M, K, N, _ in a["calls"]]
        tr = round(sum(tr) / len(tr)) if tr and None not in tr else None
        common = {"kernel": cfg, "launches_per_step": a["n"] // args.steps,
                  "avg_launch_us": round(avg_launch_s * 1e6, 3),
                  "algorithmic_bytes_per_launch": round(a["bytes"] / a["n"]),
                  "algorithmic_flops_per_launch": round(a["flops"] / a["n"])}
        if a["bound"] == "mfma":
            ach = a["flops"] / a["t"] / 1e12
            return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": tr, **common}
        ach = a["bytes"] / a["t"] / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": tr,
                **common}

    per_call = []
    if not args.no_per_gemm:
        reps = 10
        for ci, c in enumerate(calls):
            M, K, N, label = c
            j = shape_idx[(K, N)]
            def launch_reps():
                for r in range(reps):
                    mp.w4a16(xs[(M, K)], pool[(ci * reps + r) % copies][j], out=ys[(M, N)])
            launch_reps()                     # warm, then capture the ten launches
            torch.cuda.synchronize()
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_):
                launch_reps()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g_.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            fl, by = gemm_flops(M, K, N), gemm_bytes(M, K, N, g)
            bound = "hbm" if M <= 64 else "mfma"
            frac = (by / t / 1e9 / HBM_PEAK_GBPS) if bound == "hbm" else \
                (fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS)
            per_call.append({"M": M, "K": K, "N": N, "layer": label,
                             "kernel": mp.config_name(cfg_of[c]), "us": round(t * 1e6, 2),
                             "tflops": round(fl / t / 1e12, 2), "gbps": round(by / t / 1e9, 1),
                             "bound": bound, "frac": round(frac, 4)})

    # Other code formats: a per-GEMM pass like the one above, each on its own rotating pool
    # of packed copies; reported beside the W4A16 step, not part of `value`.
    del pool
    torch.cuda.empty_cache()

    def variant_pass(layer, shape_list, gemm, bytes_fn, act_dtype, ms=MS):
        torch.cuda.synchronize()
        nbytes = sum(p.nbytes for p in layer)
        ncopies = max(3, int(np.ceil(args.pool_gb * 1e9 / nbytes)))
        vpool = [layer] + [[dataclasses.replace(p, codes=p.codes.clone(), meta=p.meta.clone())
                            for p in layer] for _ in range(ncopies - 1)]
        vx = {(M, K): torch.randn(M, K, device=dev).to(act_dtype)
              for M in ms for K, _, _ in shape_list}
        vy = {(M, N): torch.empty(M, N, device=dev, dtype=act_dtype)
              for M in ms for _, N, _ in shape_list}
        torch.cuda.synchronize()
        rows, reps = [], 10
        for ci, (M, (K, N, label)) in enumerate((M, sh) for M in ms for sh in shape_list):
            j = [sh[:2] for sh in shape_list].index((K, N))
            def launch_reps():
                for r in range(reps):
                    gemm(vx[(M, K)], vpool[(ci * reps + r) % ncopies][j], out=vy[(M, N)])
            launch_reps()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                launch_reps()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            fl, by = gemm_flops(M, K, N), bytes_fn(M, K, N, g)
            bound = "hbm" if M <= 64 else "mfma"
            frac = (by / t / 1e9 / HBM_PEAK_GBPS) if bound == "hbm" else \
                (fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS)
            rows.append({"M": M, "K": K, "N": N, "layer": label,
                         "kernel": mp.config_name(mp.select_config(M, N, K, g, act_dtype)),
                         "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
                         "gbps": round(by / t / 1e9, 1), "bound": bound,
                         "frac": round(frac, 4)})
        del vpool, vx, vy
        torch.cuda.empty_cache()
        return rows

    def dev_f16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)

    # W4A16 at small prefill batches (M = 128, 256, 512): grids of fewer tiles than CUs,
    # where the tiled kernels split K.
    small = []
    if not args.no_small_m:
        small = variant_pass(layer, shapes, mp.w4a16, gemm_bytes, torch.float16,
                             ms=(128, 256, 512))

    # W8A16 (8-bit weights, asymmetric) at the Llama-3-8B shapes, fp16 activations.
    w8 = []
    if not args.no_w8:
        layer8 = []
        for K, N, label in shapes:
            codes, scales, zeros = workloads.weights_w8(K, N, g, False, wl.scale_lo, wl.scale_hi,
                                                        workloads.seed_for("bench-w8", 0, K, N))
            layer8.append(mp.pack_weights_w8(torch.from_numpy(codes).to(dev), dev_f16(scales),
                                             torch.from_numpy(zeros).to(dev), g))
        w8 = variant_pass(layer8, shapes, mp.w8a16, gemm_bytes_w8, torch.float16)
        del layer8

    # FP8 (E4M3) weights at the Qwen3-8B shapes, bf16 activations.
    fp8 = []
    if not args.no_fp8:
        wl8 = workloads.QWEN3_8B_FP8
        layerf = []
        for K, N, label in wl8.shapes:
            codes, scales = workloads.weights_fp8(K, N, g, "e4m3", wl8.scale_lo, wl8.scale_hi,
                                                  workloads.seed_for("bench-fp8", 0, K, N))
            layerf.append(mp.pack_weights_fp8(torch.from_numpy(codes).to(dev), dev_f16(scales),
                                              g, "e4m3"))
        fp8 = variant_pass(layerf, wl8.shapes, mp.wfp8a16,
                           lambda M, K, N, g_: gemm_bytes_w8(M, K, N, g_, symmetric=True),
                           torch.bfloat16)
        del layerf

    # 2-bit and 3-bit weights (asymmetric, g = 128) at the Llama-3-8B shapes, decode M only.
    lowbit = {}
    if not args.no_lowbit:
        for bits in (2, 3):
            layerb = []
            for K, N, label in shapes:
                rng = np.random.default_rng(workloads.seed_for(f"bench-w{bits}", 0, K, N))
                codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
                zeros = rng.integers(0, 1 << bits, (K // g, N), dtype=np.uint8)
                scales = rng.uniform(0.01, 0.05, (K // g, N)).astype(np.float16).view(np.uint16)
                layerb.append(mp.pack_weights_lowbit(bits, torch.from_numpy(codes).to(dev),
                                                     dev_f16(scales),
                                                     torch.from_numpy(zeros).to(dev), g))
            lowbit[f"w{bits}a16_per_gemm"] = variant_pass(
                layerb, shapes, mp.wlowbit_a16,
                lambda M, K, N, g_, b=bits: gemm_bytes_lowbit(b, M, K, N, g_), torch.float16,
                ms=(1, 16, 2048))
            del layerb

    # Decode attention over the packed 8-bit and FP8 (E4M3) KV caches (Llama-3-8B heads: 32
    # query, 8 KV, 128 wide), one query token per sequence.  Calls rotate through block
    # tables that point into a pool of blocks larger than the Infinity Cache, so KV bytes
    # come from HBM.
    attn, attn_fp8 = [], []
    if not args.no_attention:
        attn = attention_pass(args, dev, stream, None)
        attn_fp8 = attention_pass(args, dev, stream, "e4m3")

    dominant = max(per_cfg, key=lambda k: per_cfg[k]["t"])
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
                   "weight_pool_copies": copies, "group": g,
                   "launch": "hip_graph" if use_graphs else "eager"},
        "hbm_gbps": round(step_bytes / step_s / 1e9, 1),
        "roofline": roofline(dominant),
        "roofline_by_kernel": {k: roofline(k) for k in per_cfg},
        "per_gemm": per_call,
        "w4a16_small_m_per_gemm": small,
        "w8a16_per_gemm": w8,
        "wfp8a16_qwen3_8b_per_gemm": fp8,
        **lowbit,
        "attention_kv8_decode": attn,
        "attention_kvfp8_decode": attn_fp8,
        "kernel_source_digest": kernel_source_digest(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes, g)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
