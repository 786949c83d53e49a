"""Seeded synthetic inputs for the W4A16 GEMM, and the workload shape tables.

This module is the only thing the HIP path's tests and the oracle share.  It draws random
numbers and casts them to storage formats; it holds none of the method's arithmetic (no
dequantization, no packing, no products).

Recipe (every array is drawn from numpy's PCG64 with a per-case seed):
  codes  uint8 [K, N]        uniform integers in [0, 15]
  zeros  uint8 [K/g, N]      uniform integers in [0, 15]; None for symmetric codes (zero 8)
  scales fp16  [K/g, N]      uniform in [lo, hi] drawn as float64, rounded to fp16 (RNE)
  X      fp16|bf16 [M, K]    standard normal drawn as float32, rounded to the activation
                             format (RNE; bf16 through torch's float32 -> bfloat16 cast)
8-bit codes (W8A16): codes and zeros uniform integers in [0, 255] (None: symmetric, zero
128), scales as above with the range divided by 16, so dequantized weights keep the 4-bit
workloads' magnitudes.
FP8 codes: 64 * standard normal (float32), clipped to the format's largest finite value and
cast to float8_e4m3fn / float8_e5m2 by torch (round to nearest even), taken as bytes; scales
as above with the range divided by 64 (so weights are about normal with the scale's
spread).  The FP8 workload has the shapes of the Qwen3-8B projections and bf16 activations.
KV cache (attention decode): K and V codes uniform in [0, 255], zeros uniform in
[100, 155], scales uniform in [0.005, 0.02] (values about uniform in [-2.5, 2.5]); FP8 KV
codes cast as FP8 weights are, with scales uniform in [1/128, 1/32] (values about normal,
standard deviation 0.5 to 2); queries
standard normal in the activation format; heads and head size of Llama-3-8B (32 query
heads, 8 KV heads, 128) unless a case says otherwise.
Shapes are those of the layers the workloads are named after (Llama-3-8B, Llama-3-70B,
Qwen3-32B projection matrices).  No dataset or checkpoint is read.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

BASE_SEED = 20250821


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    group: int
    symmetric: bool
    scale_lo: float
    scale_hi: float
    dtype: str                      # activation / output format: "f16" or "bf16"
    ms: tuple
    shapes: tuple                   # ((K, N, label), ...)


TINY = Workload("tiny", 128, False, 0.005, 0.02, "f16", (4,), ((256, 256, "tiny"),))

LLAMA3_8B_SHAPES = ((4096, 6144, "qkv"), (4096, 4096, "o_proj"),
                    (4096, 28672, "gate_up"), (14336, 4096, "down"))
LLAMA3_8B_DECODE = Workload("llama3_8b_decode", 128, False, 0.005, 0.02, "f16",
                            (1, 8, 16), LLAMA3_8B_SHAPES)
LLAMA3_8B_PREFILL = Workload("llama3_8b_prefill", 128, False, 0.005, 0.02, "f16",
                             (512, 2048, 8192), LLAMA3_8B_SHAPES)
LLAMA3_70B = Workload("llama3_70b", 128, False, 0.005, 0.02, "bf16", (1, 64, 4096),
                      ((8192, 10240, "qkv"), (8192, 8192, "o_proj"),
                       (8192, 57344, "gate_up"), (28672, 8192, "down")))
QWEN3_32B = Workload("qwen3_32b", 64, True, 0.002, 0.01, "f16",
                     (1, 2, 4, 16, 128, 1024, 8192),
                     ((5120, 10240, "qkv"), (8192, 5120, "o_proj"),
                      (5120, 51200, "gate_up"), (25600, 5120, "down")))

QWEN3_8B_SHAPES = ((4096, 6144, "qkv"), (4096, 4096, "o_proj"),
                   (4096, 24576, "gate_up"), (12288, 4096, "down"))
QWEN3_8B_FP8 = Workload("qwen3_8b_fp8", 128, True, 0.005, 0.02, "bf16", (1, 16, 2048),
                        QWEN3_8B_SHAPES)

ALL_WORKLOADS = (TINY, LLAMA3_8B_DECODE, LLAMA3_8B_PREFILL, LLAMA3_70B, QWEN3_32B,
                 QWEN3_8B_FP8)


def seed_for(tag: str, M: int, K: int, N: int) -> int:
    return BASE_SEED + zlib.crc32(f"{tag}:{M}:{K}:{N}".encode()) % 1_000_003


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(M: int, K: int, dtype: str, seed: int) -> np.ndarray:
    """X bits [M, K] in the activation format."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _to_bf16_bits(x)
    raise ValueError(dtype)


def weights(K: int, N: int, group: int, symmetric: bool, scale_lo: float, scale_hi: float,
            seed: int):
    """(codes uint8 [K,N], scales fp16 bits [K/g,N], zeros uint8 [K/g,N] or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, size=(K // group, N)).astype(np.float16)
    zeros = None if symmetric else rng.integers(0, 16, size=(K // group, N), dtype=np.uint8)
    return codes, scales.view(np.uint16), zeros


def device_case(M: int, K: int, N: int, group: int, seed: int, device):
    """Inputs too large to draw on the host quickly, drawn on `device` by torch's seeded
    generator with the recipe of `weights` / `activations` (codes and zeros uniform in
    0..15, scales uniform in [0.005, 0.02] rounded to fp16, X standard normal rounded to
    fp16): (x fp16 [M,K], codes uint8 [K,N], scales fp16 [K/g,N], zeros uint8 [K/g,N])."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    codes = torch.randint(0, 16, (K, N), dtype=torch.uint8, device=device, generator=gen)
    scales = (torch.rand((K // group, N), device=device, generator=gen) * 0.015 + 0.005).half()
    zeros = torch.randint(0, 16, (K // group, N), dtype=torch.uint8, device=device, generator=gen)
    x = torch.randn((M, K), device=device, generator=gen, dtype=torch.float16)
    return x, codes, scales, zeros


def weights_w8(K: int, N: int, group: int, symmetric: bool, scale_lo: float, scale_hi: float,
               seed: int):
    """8-bit codes: (codes uint8 [K,N] in 0..255, scales fp16 bits [K/g,N] drawn in
    [scale_lo/16, scale_hi/16], zeros uint8 [K/g,N] in 0..255 or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(scale_lo / 16, scale_hi / 16, size=(K // group, N)).astype(np.float16)
    zeros = None if symmetric else rng.integers(0, 256, size=(K // group, N), dtype=np.uint8)
    return codes, scales.view(np.uint16), zeros


def make_case_w8(wl: Workload, M: int, K: int, N: int, seed: int | None = None):
    """All inputs of one W8A16 GEMM with workload `wl`'s group, symmetry, scale range
    (divided by 16) and activation format."""
    if seed is None:
        seed = seed_for(wl.name + "-w8", M, K, N)
    codes, scales, zeros = weights_w8(K, N, wl.group, wl.symmetric, wl.scale_lo, wl.scale_hi,
                                      seed)
    x = activations(M, K, wl.dtype, seed + 1)
    return dict(x=x, codes=codes, scales=scales, zeros=zeros, group=wl.group,
                symmetric=wl.symmetric, dtype=wl.dtype, M=M, K=K, N=N, seed=seed)


FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def to_fp8_bits(v32: np.ndarray, fmt: str) -> np.ndarray:
    """float32 values (within the format's finite range) cast to FP8 bytes by torch."""
    import torch
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.to(dt).view(torch.uint8).numpy()


def weights_fp8(K: int, N: int, group: int, fmt: str, scale_lo: float, scale_hi: float,
                seed: int):
    """FP8 codes: (codes uint8 [K,N] FP8 bytes, scales fp16 bits [K/g,N])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = np.clip(rng.standard_normal((K, N), dtype=np.float32) * 64, -FP8_MAX[fmt], FP8_MAX[fmt])
    scales = rng.uniform(scale_lo / 64, scale_hi / 64, size=(K // group, N)).astype(np.float16)
    return to_fp8_bits(v, fmt), scales.view(np.uint16)


def make_case_fp8(wl: Workload, M: int, K: int, N: int, fmt: str = "e4m3",
                  seed: int | None = None):
    """All inputs of one FP8-weight GEMM with workload `wl`'s group, scale range (divided
    by 64) and activation format."""
    if seed is None:
        seed = seed_for(wl.name + "-" + fmt, M, K, N)
    codes, scales = weights_fp8(K, N, wl.group, fmt, wl.scale_lo, wl.scale_hi, seed)
    x = activations(M, K, wl.dtype, seed + 1)
    return dict(x=x, codes=codes, scales=scales, zeros=None, group=wl.group, fmt=fmt,
                symmetric=True, dtype=wl.dtype, M=M, K=K, N=N, seed=seed)


def kv_cache(B: int, T: int, Hkv: int, D: int, seed: int):
    """(kc, ks, kz, vc, vs, vz): codes [B, T, Hkv, D], scales (fp16 bits) and zeros
    [B, T, Hkv] of an 8-bit KV cache in user form."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kc = rng.integers(0, 256, (B, T, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (B, T, Hkv, D), dtype=np.uint8)
    ks = rng.uniform(0.005, 0.02, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    vs = rng.uniform(0.005, 0.02, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    kz = rng.integers(100, 156, (B, T, Hkv), dtype=np.uint8)
    vz = rng.integers(100, 156, (B, T, Hkv), dtype=np.uint8)
    return kc, ks, kz, vc, vs, vz


def kv_cache_fp8(B: int, T: int, Hkv: int, D: int, fmt: str, seed: int):
    """(kc, ks, None, vc, vs, None): FP8 codes [B, T, Hkv, D] and scales (fp16 bits)
    [B, T, Hkv] of an FP8 KV cache in user form (no zero points)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lim = FP8_MAX[fmt]
    kc = to_fp8_bits(np.clip(64 * rng.standard_normal((B, T, Hkv, D), dtype=np.float32), -lim, lim), fmt)
    vc = to_fp8_bits(np.clip(64 * rng.standard_normal((B, T, Hkv, D), dtype=np.float32), -lim, lim), fmt)
    ks = rng.uniform(1 / 128, 1 / 32, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    vs = rng.uniform(1 / 128, 1 / 32, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    return kc, ks, None, vc, vs, None


def queries(B: int, Hq: int, D: int, dtype: str, seed: int) -> np.ndarray:
    """Query bits [B, Hq, D] in the activation format."""
    return activations(B * Hq, D, dtype, seed).reshape(B, Hq, D)


def make_case(wl: Workload, M: int, K: int, N: int, seed: int | None = None):
    """All inputs of one GEMM of workload `wl` at (M, K, N)."""
    if seed is None:
        seed = seed_for(wl.name, M, K, N)
    codes, scales, zeros = weights(K, N, wl.group, wl.symmetric, wl.scale_lo, wl.scale_hi,
                                   seed)
    x = activations(M, K, wl.dtype, seed + 1)
    return dict(x=x, codes=codes, scales=scales, zeros=zeros, group=wl.group,
                symmetric=wl.symmetric, dtype=wl.dtype, M=M, K=K, N=N, seed=seed)
