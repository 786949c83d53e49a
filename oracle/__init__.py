"""CPU oracle for the W4A16 mixed-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``weight_only_quantized_mpgemm_amd``) never
imports it, and this package never imports the product path: the two share no code.

The arithmetic lives in ``mpgemm_oracle.c`` (plain scalar C, fp64); this module builds it
with gcc, loads it with ctypes and exposes numpy-level wrappers.  What each function
computes, with its citation of "LMDeploy Accelerates Mixed-Precision LLM Inference with
TurboMind" (arXiv 2508.15601), is stated in the C source.

Parity status: every function is pinned by CPU tests against values fixed independently
of this code (see tests/test_oracle.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mpgemm_oracle.c")
_LIB_PATH = os.environ.get("MPGEMM_ORACLE_LIB") or os.path.join(_HERE, "libmpgemm_oracle.so")

F16 = 0
BF16 = 1

_lib = None


def build(force: bool = True, src: str = _SRC, out: str | None = None) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over output rows)."""
    out = out or _LIB_PATH
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i = ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_dequant.argtypes = [u8p, u16p, u8p, i, i, i, i, u16p]
    lib.oracle_dequant.restype = None
    lib.oracle_gemm.argtypes = [u16p, u16p, i, i, i, i, u16p, i]
    lib.oracle_gemm.restype = None
    lib.oracle_packed_code_bytes.argtypes = [i, i]
    lib.oracle_packed_code_bytes.restype = ctypes.c_size_t
    lib.oracle_packed_meta_bytes.argtypes = [i, i, i, i]
    lib.oracle_packed_meta_bytes.restype = ctypes.c_size_t
    lib.oracle_pack.argtypes = [u8p, u16p, u8p, i, i, i, u8p, u8p]
    lib.oracle_pack.restype = None
    lib.oracle_unpack.argtypes = [u8p, u8p, i, i, i, i, u8p, u16p, u8p]
    lib.oracle_unpack.restype = None
    lib.oracle_dequant_w8.argtypes = [u8p, u16p, u8p, i, i, i, i, u16p]
    lib.oracle_dequant_w8.restype = None
    lib.oracle_packed_code_bytes_w8.argtypes = [i, i]
    lib.oracle_packed_code_bytes_w8.restype = ctypes.c_size_t
    lib.oracle_packed_meta_bytes_w8.argtypes = [i, i, i, i]
    lib.oracle_packed_meta_bytes_w8.restype = ctypes.c_size_t
    lib.oracle_pack_w8.argtypes = [u8p, u16p, u8p, i, i, i, u8p, u8p]
    lib.oracle_pack_w8.restype = None
    lib.oracle_unpack_w8.argtypes = [u8p, u8p, i, i, i, i, u8p, u16p, u8p]
    lib.oracle_unpack_w8.restype = None
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e5m2_to_f64.restype = ctypes.c_double
    lib.oracle_dequant_fp8.argtypes = [u8p, u16p, i, i, i, i, i, u16p]
    lib.oracle_dequant_fp8.restype = None
    lib.oracle_padded_k.argtypes = [i]
    lib.oracle_padded_k.restype = i
    lib.oracle_padded_n.argtypes = [i]
    lib.oracle_padded_n.restype = i
    lib.oracle_dequant_lowbit.argtypes = [i, u8p, u16p, u8p, i, i, i, i, u16p]
    lib.oracle_dequant_lowbit.restype = None
    lib.oracle_packed_code_bytes_lowbit.argtypes = [i, i, i]
    lib.oracle_packed_code_bytes_lowbit.restype = ctypes.c_size_t
    lib.oracle_pack_lowbit.argtypes = [i, u8p, u16p, u8p, i, i, i, u8p, u8p]
    lib.oracle_pack_lowbit.restype = None
    lib.oracle_unpack_lowbit.argtypes = [i, u8p, u8p, i, i, i, i, u8p, u16p, u8p]
    lib.oracle_unpack_lowbit.restype = None
    lib.oracle_attention_decode_kv8.argtypes = [u16p, u8p, u16p, u8p, u8p, u16p, u8p,
                                                ctypes.POINTER(ctypes.c_int), i, i, i, i, i,
                                                ctypes.c_float, i, u16p]
    lib.oracle_attention_decode_kv8.restype = None
    lib.oracle_attention_decode_kvfp8.argtypes = [u16p, u8p, u16p, u8p, u16p,
                                                  ctypes.POINTER(ctypes.c_int), i, i, i, i, i,
                                                  ctypes.c_float, i, i, u16p]
    lib.oracle_attention_decode_kvfp8.restype = None
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_kv_block_bytes.argtypes = [i, i]
    lib.oracle_kv_block_bytes.restype = ctypes.c_size_t
    lib.oracle_kv_pack.argtypes = [u8p, u16p, u8p, u8p, u16p, u8p, i, i, i, i, ip, u8p]
    lib.oracle_kv_pack.restype = None
    lib.oracle_kv_unpack.argtypes = [u8p, ip, i, i, i, u8p, u16p, u8p, u8p, u16p, u8p]
    lib.oracle_kv_unpack.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _dtype_code(dtype: str) -> int:
    if dtype in ("f16", "fp16", "float16"):
        return F16
    if dtype in ("bf16", "bfloat16"):
        return BF16
    raise ValueError(f"unknown activation dtype {dtype!r}")


# ---------------------------------------------------------------- number formats ----

def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_f16_to_f64(int(b)) for b in flat]).reshape(np.shape(bits))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_bf16_to_f64(int(b)) for b in flat]).reshape(np.shape(bits))


def f64_to_f16_bits(x) -> np.ndarray:
    lib = _load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    return np.array([lib.oracle_f64_to_f16(float(v)) for v in flat],
                    dtype=np.uint16).reshape(np.shape(x))


def f64_to_bf16_bits(x) -> np.ndarray:
    lib = _load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    return np.array([lib.oracle_f64_to_bf16(float(v)) for v in flat],
                    dtype=np.uint16).reshape(np.shape(x))


# ---------------------------------------------------------------- the method --------

def dequant(codes: np.ndarray, scales_bits: np.ndarray, zeros: np.ndarray | None,
            group: int, dtype: str = "f16") -> np.ndarray:
    """w[k][n] = round_act((q - z) * s); returns activation-format bits [K, N]."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert scales_bits.shape == (-(-K // group), N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == (-(-K // group), N)
        zp = _ptr(zeros, ctypes.c_uint8)
    w = np.empty((K, N), dtype=np.uint16)
    lib.oracle_dequant(_ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16), zp,
                       K, N, group, _dtype_code(dtype), _ptr(w, ctypes.c_uint16))
    return w


def gemm(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str = "f16",
         threads: int = 1) -> np.ndarray:
    """Y = round_act(X @ w) with the sum in fp64; inputs and output are format bits."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, K = x_bits.shape
    K2, N = w_bits.shape
    assert K == K2
    y = np.empty((M, N), dtype=np.uint16)
    lib.oracle_gemm(_ptr(x_bits, ctypes.c_uint16), _ptr(w_bits, ctypes.c_uint16),
                    M, N, K, _dtype_code(dtype), _ptr(y, ctypes.c_uint16), int(threads))
    return y


def w4a16(x_bits, codes, scales_bits, zeros, group, dtype="f16", threads=1):
    """The whole path: dequantize, then the GEMM."""
    return gemm(x_bits, dequant(codes, scales_bits, zeros, group, dtype), dtype, threads)


def act_bits_to_f64(bits: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """Exact values of activation-format bits, in bulk: binary16 through numpy's float16;
    bf16 as the high half of a binary32 (its definition).  Pinned against the scalar
    conversions above over every bit pattern (tests/test_oracle.py)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if _dtype_code(dtype) == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_f64(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """X @ w in float64, before the output rounding, with numpy's float64 matmul as a
    library step.  Each product of two 16-bit values is exact in float64, and any
    summation order stays within about K * 2^-53 of the sum of magnitudes of the exact
    sum: far below one unit in the last place of a 16-bit output.  For shapes whose scalar
    loop (gemm) would take minutes; pinned against gemm and an exact rational sum
    (tests/test_oracle.py)."""
    x = act_bits_to_f64(x_bits, dtype)
    w = act_bits_to_f64(w_bits, dtype)
    assert x.ndim == 2 and w.ndim == 2 and x.shape[1] == w.shape[0]
    return x @ w


def w4a16_f64(x_bits, codes, scales_bits, zeros, group, dtype="f16",
              col_chunk: int = 4096, threads: int = 0) -> np.ndarray:
    """The whole path before the output rounding: dequantize (one rounding to the
    activation format, as dequant), then gemm_f64.  Columns go in chunks of `col_chunk`,
    whose dequantizations run in up to `threads` host threads at once (0: one per core, at
    most 16); chunks are independent, so this changes nothing in the result.  Returns
    float64 [M, N]."""
    import concurrent.futures
    codes = np.asarray(codes)
    K, N = codes.shape
    x = act_bits_to_f64(x_bits, dtype)
    out = np.empty((x.shape[0], N), dtype=np.float64)
    spans = [(c0, min(N, c0 + col_chunk)) for c0 in range(0, N, col_chunk)]

    def deq(span):
        c0, c1 = span
        z = None if zeros is None else zeros[:, c0:c1]
        return dequant(codes[:, c0:c1], scales_bits[:, c0:c1], z, group, dtype)

    workers = threads or min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for (c0, c1), w in zip(spans, ex.map(deq, spans)):
            out[:, c0:c1] = x @ act_bits_to_f64(w, dtype)
    return out


def padded_shape(K: int, N: int) -> tuple[int, int]:
    """(Kp, Np): the packed planes' padded matrix for a user matrix of K x N."""
    lib = _load()
    return int(lib.oracle_padded_k(K)), int(lib.oracle_padded_n(N))


def packed_code_bytes(K: int, N: int) -> int:
    return int(_load().oracle_packed_code_bytes(K, N))


def packed_meta_bytes(K: int, N: int, group: int, symmetric: bool) -> int:
    return int(_load().oracle_packed_meta_bytes(K, N, group, int(bool(symmetric))))


def pack(codes: np.ndarray, scales_bits: np.ndarray, zeros: np.ndarray | None, group: int):
    """Layout-v1 packing; returns (packed_codes uint8, packed_meta uint8)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    rows = -(-K // group)
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert scales_bits.shape == (rows, N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == (rows, N)
        zp = _ptr(zeros, ctypes.c_uint8)
    pc = np.empty(packed_code_bytes(K, N), dtype=np.uint8)
    pm = np.empty(packed_meta_bytes(K, N, group, zeros is None), dtype=np.uint8)
    lib.oracle_pack(_ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16), zp,
                    K, N, group, _ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8))
    return pc, pm


def unpack(packed_codes: np.ndarray, packed_meta: np.ndarray, K: int, N: int, group: int,
           symmetric: bool):
    """Inverse of pack; returns (codes, scales_bits, zeros or None)."""
    lib = _load()
    pc = np.ascontiguousarray(packed_codes, dtype=np.uint8)
    pm = np.ascontiguousarray(packed_meta, dtype=np.uint8)
    codes = np.empty((K, N), dtype=np.uint8)
    rows = -(-K // group)
    scales = np.empty((rows, N), dtype=np.uint16)
    zeros = None if symmetric else np.empty((rows, N), dtype=np.uint8)
    lib.oracle_unpack(_ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8), K, N, group,
                      int(bool(symmetric)), _ptr(codes, ctypes.c_uint8),
                      _ptr(scales, ctypes.c_uint16),
                      None if zeros is None else _ptr(zeros, ctypes.c_uint8))
    return codes, scales, zeros


# ------------------------------------------------------------ 8-bit weights (W8A16) --

def dequant_w8(codes: np.ndarray, scales_bits: np.ndarray, zeros: np.ndarray | None,
               group: int, dtype: str = "f16") -> np.ndarray:
    """w[k][n] = round_act((q - z) * s), q and z 8-bit (z = 128 when zeros is None)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert scales_bits.shape == (-(-K // group), N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == (-(-K // group), N)
        zp = _ptr(zeros, ctypes.c_uint8)
    w = np.empty((K, N), dtype=np.uint16)
    lib.oracle_dequant_w8(_ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16), zp,
                          K, N, group, _dtype_code(dtype), _ptr(w, ctypes.c_uint16))
    return w


def w8a16(x_bits, codes, scales_bits, zeros, group, dtype="f16", threads=1):
    """The whole 8-bit path: dequantize, then the GEMM."""
    return gemm(x_bits, dequant_w8(codes, scales_bits, zeros, group, dtype), dtype, threads)


def packed_code_bytes_w8(K: int, N: int) -> int:
    return int(_load().oracle_packed_code_bytes_w8(K, N))


def packed_meta_bytes_w8(K: int, N: int, group: int, symmetric: bool) -> int:
    return int(_load().oracle_packed_meta_bytes_w8(K, N, group, int(bool(symmetric))))


def pack_w8(codes: np.ndarray, scales_bits: np.ndarray, zeros: np.ndarray | None, group: int):
    """8-bit layout packing; returns (packed_codes uint8, packed_meta uint8)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    rows = -(-K // group)
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert scales_bits.shape == (rows, N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == (rows, N)
        zp = _ptr(zeros, ctypes.c_uint8)
    pc = np.empty(packed_code_bytes_w8(K, N), dtype=np.uint8)
    pm = np.zeros(packed_meta_bytes_w8(K, N, group, zeros is None), dtype=np.uint8)
    lib.oracle_pack_w8(_ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16), zp,
                       K, N, group, _ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8))
    return pc, pm


def unpack_w8(packed_codes: np.ndarray, packed_meta: np.ndarray, K: int, N: int, group: int,
              symmetric: bool):
    """Inverse of pack_w8; returns (codes, scales_bits, zeros or None)."""
    lib = _load()
    pc = np.ascontiguousarray(packed_codes, dtype=np.uint8)
    pm = np.ascontiguousarray(packed_meta, dtype=np.uint8)
    codes = np.empty((K, N), dtype=np.uint8)
    rows = -(-K // group)
    scales = np.empty((rows, N), dtype=np.uint16)
    zeros = None if symmetric else np.empty((rows, N), dtype=np.uint8)
    lib.oracle_unpack_w8(_ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8), K, N, group,
                         int(bool(symmetric)), _ptr(codes, ctypes.c_uint8),
                         _ptr(scales, ctypes.c_uint16),
                         None if zeros is None else _ptr(zeros, ctypes.c_uint8))
    return codes, scales, zeros


# ------------------------------------------------------------ FP8 weights ----------

FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def fp8_to_f64(codes: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Values of OCP FP8 codes (E4M3 or E5M2)."""
    lib = _load()
    fn = lib.oracle_e5m2_to_f64 if FP8_FORMATS[fmt] else lib.oracle_e4m3_to_f64
    flat = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    return np.array([fn(int(b)) for b in flat]).reshape(np.shape(codes))


def dequant_fp8(codes: np.ndarray, scales_bits: np.ndarray, group: int, fmt: str = "e4m3",
                dtype: str = "f16") -> np.ndarray:
    """w[k][n] = round_act(fp8(q) * s); returns activation-format bits [K, N]."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert scales_bits.shape == (-(-K // group), N)
    w = np.empty((K, N), dtype=np.uint16)
    lib.oracle_dequant_fp8(_ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16),
                           K, N, group, FP8_FORMATS[fmt], _dtype_code(dtype),
                           _ptr(w, ctypes.c_uint16))
    return w


def wfp8a16(x_bits, codes, scales_bits, group, fmt="e4m3", dtype="f16", threads=1):
    """The whole FP8-weight path: dequantize, then the GEMM."""
    return gemm(x_bits, dequant_fp8(codes, scales_bits, group, fmt, dtype), dtype, threads)


# ---------------------------------------------------- 2-bit and 3-bit weights -------

def dequant_lowbit(bits: int, codes: np.ndarray, scales_bits: np.ndarray,
                   zeros: np.ndarray | None, group: int, dtype: str = "f16") -> np.ndarray:
    """w[k][n] = round_act((q - z) * s) with b-bit q, z (z = 2^(b-1) when zeros is None)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert bits in (2, 3) and scales_bits.shape == (-(-K // group), N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == scales_bits.shape
        zp = _ptr(zeros, ctypes.c_uint8)
    w = np.empty((K, N), dtype=np.uint16)
    lib.oracle_dequant_lowbit(bits, _ptr(codes, ctypes.c_uint8),
                              _ptr(scales_bits, ctypes.c_uint16), zp, K, N, group,
                              _dtype_code(dtype), _ptr(w, ctypes.c_uint16))
    return w


def wlowbit_a16(bits, x_bits, codes, scales_bits, zeros, group, dtype="f16", threads=1):
    """The whole b-bit path: dequantize, then the GEMM."""
    return gemm(x_bits, dequant_lowbit(bits, codes, scales_bits, zeros, group, dtype), dtype,
                threads)


def packed_code_bytes_lowbit(bits: int, K: int, N: int) -> int:
    return int(_load().oracle_packed_code_bytes_lowbit(bits, K, N))


def pack_lowbit(bits: int, codes: np.ndarray, scales_bits: np.ndarray,
                zeros: np.ndarray | None, group: int):
    """Sub-4-bit layout packing; returns (packed_codes uint8, packed_meta uint8)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    rows = -(-K // group)
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    assert bits in (2, 3) and scales_bits.shape == (rows, N)
    zp = None
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        assert zeros.shape == (rows, N)
        zp = _ptr(zeros, ctypes.c_uint8)
    pc = np.empty(packed_code_bytes_lowbit(bits, K, N), dtype=np.uint8)
    pm = np.empty(packed_meta_bytes(K, N, group, zeros is None), dtype=np.uint8)
    lib.oracle_pack_lowbit(bits, _ptr(codes, ctypes.c_uint8), _ptr(scales_bits, ctypes.c_uint16),
                           zp, K, N, group, _ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8))
    return pc, pm


def unpack_lowbit(bits: int, packed_codes: np.ndarray, packed_meta: np.ndarray, K: int, N: int,
                  group: int, symmetric: bool):
    """Inverse of pack_lowbit; returns (codes, scales_bits, zeros or None)."""
    lib = _load()
    pc = np.ascontiguousarray(packed_codes, dtype=np.uint8)
    pm = np.ascontiguousarray(packed_meta, dtype=np.uint8)
    rows = -(-K // group)
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty((rows, N), dtype=np.uint16)
    zeros = None if symmetric else np.empty((rows, N), dtype=np.uint8)
    lib.oracle_unpack_lowbit(bits, _ptr(pc, ctypes.c_uint8), _ptr(pm, ctypes.c_uint8), K, N,
                             group, int(bool(symmetric)), _ptr(codes, ctypes.c_uint8),
                             _ptr(scales, ctypes.c_uint16),
                             None if zeros is None else _ptr(zeros, ctypes.c_uint8))
    return codes, scales, zeros


# ------------------------------------------------ attention decode (8-bit KV) --------

def attention_decode_kv8(q_bits, kc, ks_bits, kz, vc, vs_bits, vz, lens, scale: float,
                         dtype: str = "f16") -> np.ndarray:
    """Decode attention over an 8-bit KV cache (user form; see the C source).

    q_bits [B, Hq, D]; kc, vc [B, Tmax, Hkv, D] uint8; ks_bits, vs_bits [B, Tmax, Hkv]
    fp16 bits; kz, vz [B, Tmax, Hkv] uint8; lens [B]; returns o bits [B, Hq, D].
    """
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    B, Hq, D = q_bits.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    _, Tmax, Hkv, D2 = kc.shape
    assert D2 == D and Hq % Hkv == 0
    arrs = [np.ascontiguousarray(a, dtype=t) for a, t in
            ((ks_bits, np.uint16), (kz, np.uint8), (vc, np.uint8), (vs_bits, np.uint16),
             (vz, np.uint8))]
    for a in (arrs[0], arrs[1], arrs[3], arrs[4]):
        assert a.shape == (B, Tmax, Hkv)
    assert arrs[2].shape == kc.shape
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= 0).all() and (lens <= Tmax).all()
    o = np.empty((B, Hq, D), dtype=np.uint16)
    lib.oracle_attention_decode_kv8(
        _ptr(q_bits, ctypes.c_uint16), _ptr(kc, ctypes.c_uint8), _ptr(arrs[0], ctypes.c_uint16),
        _ptr(arrs[1], ctypes.c_uint8), _ptr(arrs[2], ctypes.c_uint8),
        _ptr(arrs[3], ctypes.c_uint16), _ptr(arrs[4], ctypes.c_uint8),
        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), B, Hq, Hkv, D, Tmax,
        ctypes.c_float(scale), _dtype_code(dtype), _ptr(o, ctypes.c_uint16))
    return o


def attention_decode_kvfp8(q_bits, kc, ks_bits, vc, vs_bits, lens, scale: float,
                           fmt: str = "e4m3", dtype: str = "f16") -> np.ndarray:
    """Decode attention over an FP8 KV cache (user form as attention_decode_kv8, no
    zeros); returns o bits [B, Hq, D]."""
    lib = _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    B, Hq, D = q_bits.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    _, Tmax, Hkv, D2 = kc.shape
    assert D2 == D and Hq % Hkv == 0
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    ks_bits = np.ascontiguousarray(ks_bits, dtype=np.uint16)
    vs_bits = np.ascontiguousarray(vs_bits, dtype=np.uint16)
    assert vc.shape == kc.shape and ks_bits.shape == vs_bits.shape == (B, Tmax, Hkv)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= 0).all() and (lens <= Tmax).all()
    o = np.empty((B, Hq, D), dtype=np.uint16)
    lib.oracle_attention_decode_kvfp8(
        _ptr(q_bits, ctypes.c_uint16), _ptr(kc, ctypes.c_uint8), _ptr(ks_bits, ctypes.c_uint16),
        _ptr(vc, ctypes.c_uint8), _ptr(vs_bits, ctypes.c_uint16),
        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), B, Hq, Hkv, D, Tmax,
        ctypes.c_float(scale), FP8_FORMATS[fmt], _dtype_code(dtype), _ptr(o, ctypes.c_uint16))
    return o


def kv_block_bytes(Hkv: int, D: int) -> int:
    return int(_load().oracle_kv_block_bytes(Hkv, D))


def kv_pack(cache: np.ndarray, table_row, t0: int, kc, ks_bits, kz, vc, vs_bits, vz):
    """Writes tokens t0 .. t0+n-1 (user form [n, Hkv, D] codes, [n, Hkv] scales/zeros) of
    one sequence into `cache` (uint8, modified in place) through its block-table row."""
    lib = _load()
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    n, Hkv, D = kc.shape
    arrs = [np.ascontiguousarray(a, dtype=t) for a, t in
            ((ks_bits, np.uint16), (kz, np.uint8), (vc, np.uint8), (vs_bits, np.uint16),
             (vz, np.uint8))]
    table_row = np.ascontiguousarray(table_row, dtype=np.int32)
    assert cache.flags["C_CONTIGUOUS"] and cache.dtype == np.uint8
    assert table_row.size * 64 >= t0 + n
    assert (table_row[(t0 // 64):(t0 + n + 63) // 64] + 1).max() * kv_block_bytes(Hkv, D) <= cache.size
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_kv_pack(_ptr(kc, ctypes.c_uint8), _ptr(arrs[0], ctypes.c_uint16),
                       _ptr(arrs[1], ctypes.c_uint8), _ptr(arrs[2], ctypes.c_uint8),
                       _ptr(arrs[3], ctypes.c_uint16), _ptr(arrs[4], ctypes.c_uint8), n, t0,
                       Hkv, D, table_row.ctypes.data_as(ip), _ptr(cache, ctypes.c_uint8))


def kv_unpack(cache: np.ndarray, table_row, T: int, Hkv: int, D: int):
    """Tokens 0 .. T-1 of one sequence: (kc, ks_bits, kz, vc, vs_bits, vz) in user form."""
    lib = _load()
    table_row = np.ascontiguousarray(table_row, dtype=np.int32)
    kc = np.empty((T, Hkv, D), np.uint8)
    vc = np.empty((T, Hkv, D), np.uint8)
    ks = np.empty((T, Hkv), np.uint16)
    vs = np.empty((T, Hkv), np.uint16)
    kz = np.empty((T, Hkv), np.uint8)
    vz = np.empty((T, Hkv), np.uint8)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_kv_unpack(_ptr(np.ascontiguousarray(cache), ctypes.c_uint8),
                         table_row.ctypes.data_as(ip), T, Hkv, D, _ptr(kc, ctypes.c_uint8),
                         _ptr(ks, ctypes.c_uint16), _ptr(kz, ctypes.c_uint8),
                         _ptr(vc, ctypes.c_uint8), _ptr(vs, ctypes.c_uint16),
                         _ptr(vz, ctypes.c_uint8))
    return kc, ks, kz, vc, vs, vz


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def timed_w4a16(x_bits, codes, scales_bits, zeros, group, dtype="f16", threads=1):
    """Runs the whole oracle path and returns (Y, seconds)."""
    t0 = time.perf_counter()
    y = w4a16(x_bits, codes, scales_bits, zeros, group, dtype, threads)
    return y, time.perf_counter() - t0
