"""Builds libmpgemm.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m weight_only_quantized_mpgemm_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection
switched off (those forms are avoided on this hardware) and floating-point contraction off
(the dequantization relies on an exact add followed by a single rounding multiply).  The
compiler's per-kernel resource report is checked: a kernel that spills to scratch memory
fails the build (a spill in these register-resident pipelines costs far more than it
saves, and nothing else would show it).  The generated code of the kernels that issue
MFMAs through inline asm is checked too: no accumulator may be read sooner than 32 wait
states after the MFMA that writes it (the compiler cannot enforce that for asm).
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmpgemm.so")
SOURCES = ["api.hip", "pack.hip", "gemm_decode.hip", "gemm_prefill_x32.hip", "gemm_prefill_x32_w8.hip", "gemm_prefill_x32_fp8.hip",
           "attention.hip"]
HEADERS = ["device.hpp", "kernels.hpp", "prefill_x32.hpp"]
# Peak microkernels (include/mpgemm_probes.h): a library of their own, apart from the GEMM
# path, for the measured roofline denominators.
PROBE_SOURCES = ["probes.hip"]
PROBE_LIB = os.path.join(PKG, "libmpgemm_probes.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def scratch_users(report: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) for every kernel the resource report shows using scratch."""
    out, name = [], None
    for line in report.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


# Sources whose kernels issue MFMAs through inline asm: the compiler does not know those
# instructions' result latency, so the build checks the generated code instead.
ASM_MFMA_SOURCES = ["gemm_prefill_x32.hip", "gemm_prefill_x32_w8.hip",
                    "gemm_prefill_x32_fp8.hip"]
MIN_RESULT_WAIT = 32     # wait states between an MFMA and the first read of its result


def acc_read_hazards(asm: str, min_wait: int = MIN_RESULT_WAIT) -> list[tuple[str, int]]:
    """(kernel, distance) for every kernel in which some MFMA's accumulator result is read
    (v_accvgpr_read / v_accvgpr_mov) fewer than `min_wait` wait states after the MFMA, in
    straight-line order; distance = instructions in between plus s_nop wait states."""
    out = []
    for name in re.findall(r"\n([A-Za-z_][\w.$]*):[^\n]*\n", asm):
        if "kernel" not in name:
            continue
        start = asm.index("\n" + name + ":")
        end = asm.find(".Lfunc_end", start)
        lines = [ln.strip() for ln in asm[start:end].split("\n")[1:]]
        lines = [ln for ln in lines if ln and not ln.startswith((";", "."))]
        worst = None
        for k, ln in enumerate(lines):
            if not ln.startswith("v_mfma"):
                continue
            dst = ln.split()[1].rstrip(",")
            m = re.match(r"a\[(\d+):(\d+)\]", dst)
            if not m:
                continue
            lo, hi = int(m.group(1)), int(m.group(2))
            states = 0
            for j in range(k + 1, min(k + 128, len(lines))):
                ln2 = lines[j]
                if ln2.startswith("s_nop"):
                    states += int(ln2.split()[1]) + 1
                    continue
                if ln2.startswith(("v_accvgpr_read", "v_accvgpr_mov")):
                    srcs = re.findall(r"a(\d+)", ln2.split(",", 1)[1])
                    if any(lo <= int(a) <= hi for a in srcs):
                        d = j - k - 1 + states
                        worst = d if worst is None else min(worst, d)
                        break
                if ln2.startswith("v_mfma") and ln2.split()[1].rstrip(",") == dst:
                    break
        if worst is not None and worst < min_wait:
            out.append((name, worst))
    return out


def _path_lines(asm: str, name: str) -> list[str]:
    start = asm.index("\n" + name + ":")
    end = asm.find(".Lfunc_end", start)
    out = []
    for ln in asm[start:end].split("\n")[1:]:
        ln = ln.strip()
        if re.match(r"\.LBB\w+:", ln):
            out.append(ln.split()[0])
        elif ln and not ln.startswith((".", ";")):
            out.append(ln)
    return out


def stage_wait_violations(seq: list[str], mb: int) -> list[tuple]:
    """Walks one execution path of a ring-buffered kernel: the k-th group of `mb` LDS-DMA
    loads (buffer_load ... lds) carries stage k; the b-th s_barrier (b = 0: the prologue's)
    must find stage b's group complete, i.e. the s_waitcnt right before it must leave in
    flight no more loads than were issued after that group's last part (vmcnt counts a
    wave's loads in issue order).  Returns (barrier, loads after, vmcnt) per violation."""
    loads, nlds, bars, bad, prev = [], 0, 0, [], None
    for ln in seq:
        if ln.startswith("buffer_load"):
            if " lds" in ln:
                loads.append(nlds // mb)
                nlds += 1
            else:
                loads.append(None)
        elif ln.startswith("s_barrier"):
            nv = 63                                   # no wait right before: anything in flight
            m = re.match(r"s_waitcnt (0x[0-9a-fA-F]+|\d+)$", prev or "")
            if m:
                imm = int(m.group(1), 0)
                nv = (imm & 15) | (((imm >> 14) & 3) << 4)
            elif (prev or "").startswith("s_waitcnt"):
                v = re.search(r"vmcnt\((\d+)\)", prev)
                nv = int(v.group(1)) if v else 63
            idx = [k for k, t in enumerate(loads) if t == bars]
            if len(idx) < mb:
                bad.append((bars, -1, nv))
            elif len(loads) - 1 - idx[-1] < nv:
                bad.append((bars, len(loads) - 1 - idx[-1], nv))
            bars += 1
        prev = ln
    return bad


def ring_shape(name: str) -> tuple[int, int | None]:
    """(ring stages, DMA loads per wave and stage) of a 32x32x16 tiled kernel, from its
    template arguments <ACT, SYM, G, NWS, SH, CODE, RAG, MA>: tiles whose live row blocks
    MA fill less than the tile (one row of tiles; not the 256 x 256 tile), with four weight
    register sets, keep only those rows in an eight-stage ring, the others all rows in four
    stages."""
    args = re.search(r"prefill_x32_kernelI((?:L[ib]\d+E){8})E", name)
    if args is None:                     # no template arguments: a four-stage ring
        return 4, None
    vals = [int(v) for v in re.findall(r"L[ib](\d+)E", args.group(1))]
    nws, sh, ma = vals[3], vals[4], vals[7]
    mb = {1: 8, 2: 4, 3: 8}[sh]
    if sh != 3 and ma < mb and nws == 4:
        return 8, ma
    return 4, mb


def ring_wait_violations(asm: str) -> list[tuple[str, str, list]]:
    """Checks every 32x32x16 tiled kernel's stage waits along the paths a launch takes:
    prologue, then the stage loop once and twice, then (four-weight-set kernels) the
    four-stage tail after one pass of the loop or in place of it."""
    out = []
    for name in re.findall(r"\n([A-Za-z_][\w.$]*):[^\n]*\n", asm):
        if "prefill_x32_kernel" not in name:
            continue
        lines = _path_lines(asm, name)
        lab = {ln[:-1]: i for i, ln in enumerate(lines) if re.match(r"\.LBB\w+:$", ln)}
        b0 = next(i for i, ln in enumerate(lines) if ln.startswith("s_barrier"))
        # DMA loads per stage and wave: the prologue issues all stages of the ring but one
        xs, dmb = ring_shape(name)
        mb = sum(1 for ln in lines[:b0] if ln.startswith("buffer_load") and " lds" in ln) // (xs - 1)
        if dmb is not None and mb != dmb:
            out.append((name, "prologue", [(-1, mb, dmb)]))
            continue
        br = next(i for i in range(b0, len(lines)) if lines[i].startswith("s_cbranch"))
        skip = lines[br].split()[1]
        top = next(i for i in range(br + 1, len(lines)) if re.match(r"\.LBB\w+:$", lines[i]))
        back = next(i for i in range(top, len(lines))
                    if lines[i].startswith("s_cbranch") and lines[i].split()[1] == lines[top][:-1])
        prologue, loop = lines[:br], lines[top + 1:back]
        paths = {"loop once": prologue + loop, "loop twice": prologue + loop + loop}
        j = next(i for i in range(back + 1, len(lines)) if lines[i].startswith("s_cbranch"))
        tl = next(i for i in range(j + 1, len(lines)) if re.match(r"\.LBB\w+:$", lines[i]))
        after = lines[tl + 1:lab.get(lines[j].split()[1], tl + 1)]
        if any(ln.startswith("s_barrier") for ln in after):          # a four-stage tail
            tail = lines[j + 1:tl] + after
            sk = lines[lab[skip] + 1:]
            k = next(i for i, ln in enumerate(sk) if ln.startswith(("s_branch", "s_cbranch")))
            paths["loop and tail"] = prologue + loop + tail
            paths["tail only"] = prologue + sk[:k] + tail
        for path, seq in paths.items():
            bad = stage_wait_violations(seq, mb)
            if bad:
                out.append((name, path, bad))
    return out


# A vector ALU write of a register that an MFMA then reads (as A, B or C) needs two wait
# states in between.  The compiler inserts them for instructions it emits itself, but it does
# not know what an inline asm statement writes; the build checks every kernel instead.
MIN_VALU_TO_MFMA_WAIT = 2


def _regs(tok: str) -> set[tuple[str, int]]:
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(line: str) -> list[str]:
    parts = line.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def valu_mfma_hazards(asm: str, min_wait: int = MIN_VALU_TO_MFMA_WAIT) -> list[tuple]:
    """(kernel, VALU instruction, distance) for every vector ALU write of a VGPR or AGPR
    that some MFMA reads fewer than `min_wait` wait states later, along every branch path;
    distance = instructions in between plus s_nop wait states."""
    out = []
    for name in re.findall(r"\n([A-Za-z_][\w.$]*):[^\n]*\n", asm):
        if "kernel" not in name:
            continue
        lines = _path_lines(asm, name)
        lab = {ln[:-1]: i for i, ln in enumerate(lines) if re.match(r"\.LBB\w+:$", ln)}
        for k, ln in enumerate(lines):
            if not ln.startswith("v_") or ln.startswith(("v_mfma", "v_smfmac")):
                continue
            ops = _operands(ln)
            dst = _regs(ops[0]) if ops else set()
            if not dst:
                continue
            stack = [(k + 1, 0)]
            while stack:
                j, states = stack.pop()
                while j < len(lines) and states < min_wait:
                    ln2 = lines[j]
                    if ln2.endswith(":"):
                        j += 1
                        continue
                    if ln2.startswith(("v_mfma", "v_smfmac")):
                        if dst & set().union(*map(_regs, _operands(ln2)[1:])):
                            out.append((name, ln, states))
                            break
                    if ln2.startswith("s_nop"):
                        states += int(ln2.split()[1], 0) + 1
                        j += 1
                        continue
                    if ln2.startswith("s_endpgm"):
                        break
                    if ln2.startswith("s_branch"):
                        j, states = lab[ln2.split()[1]] + 1, states + 1
                        continue
                    if ln2.startswith("s_cbranch"):
                        stack.append((lab[ln2.split()[1]] + 1, states + 1))
                    if ops and ln2.startswith("v_") and dst & _regs(_operands(ln2)[0]) and \
                            not ln2.startswith(("v_mfma", "v_smfmac")):
                        break                                     # overwritten first
                    states += 1
                    j += 1
    return out


def _check_asm_mfma(src: str, extra: list[str]) -> None:
    asm_path = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *FLAGS, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o",
           asm_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stderr}")
    asm = open(asm_path).read()
    bad = valu_mfma_hazards(asm)
    if bad:
        raise RuntimeError(f"{src}: MFMA operands read too soon after a vector ALU write "
                           f"(wait states): {len(bad)} cases, first {bad[:3]}")
    if src not in ASM_MFMA_SOURCES:
        return
    bad = acc_read_hazards(asm)
    if bad:
        raise RuntimeError(f"{src}: MFMA results read too early (wait states): {bad}")
    if "prefill_x32" in src:
        bad = ring_wait_violations(asm)
        if bad:
            raise RuntimeError(f"{src}: a stage wait can pass before its DMA landed: {bad[:4]}")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    spills = scratch_users(res.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {spills}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compiles every source (always; no staleness shortcuts) and links libmpgemm.so and
    libmpgemm_probes.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs) + 2) as ex:
        checks = [ex.submit(_check_asm_mfma, s, extra) for s in srcs]
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra), srcs)))
        for c in checks:
            c.result()
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
