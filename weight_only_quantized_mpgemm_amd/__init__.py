"""W4A16 mixed-precision GEMM for AMD MI355X (gfx950): thin Python binding of libmpgemm.

Every step of the computation runs in the library's HIP kernels; this module only checks
tensor properties, passes ``data_ptr()`` values and torch's current HIP stream through the
C ABI declared in ``include/mpgemm.h``, and allocates outputs with torch.  There is no
fallback: if ``libmpgemm.so`` is missing or the call fails, an exception is raised.

Method: "LMDeploy Accelerates Mixed-Precision LLM Inference with TurboMind"
(arXiv 2508.15601) -- offline packing of group-quantized 4-bit weights (technique (i)) and
an online GEMM that dequantizes them in registers (I2F; Fig. 6 and Fig. 9 captions).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmpgemm.so")

F16 = 0
BF16 = 1
LAYOUT_VERSION = 1

STATUS = {
    0: "MPGEMM_OK",
    -1: "MPGEMM_ERR_INVALID_ARG",
    -2: "MPGEMM_ERR_UNSUPPORTED",
    -3: "MPGEMM_ERR_ALIGNMENT",
    -4: "MPGEMM_ERR_WORKSPACE",
    -5: "MPGEMM_ERR_HIP",
}

# Every function declared in include/mpgemm.h: name -> (restype, argtypes).
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "mpgemm_layout_version": (_i, []),
    "mpgemm_packed_code_bytes": (_sz, [_i, _i]),
    "mpgemm_packed_meta_bytes": (_sz, [_i, _i, _i, _i]),
    "mpgemm_pack_weights": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "mpgemm_unpack": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "mpgemm_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "mpgemm_w4a16": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "mpgemm_select_config": (_i, [_i, _i, _i, _i, _i]),
    "mpgemm_config_name": (ctypes.c_char_p, [_i]),
    "mpgemm_prefill_launches": (_i, [_i, _i, _i, _i, _i, _vp]),
    "mpgemm_prefill_schedule": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _i]),
    "mpgemm_w4a16_config": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _i,
                                 _vp]),
    "mpgemm_status_string": (ctypes.c_char_p, [_i]),
    "mpgemm_w4a16_noalloc": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "mpgemm_packed_code_bytes_w8": (_sz, [_i, _i]),
    "mpgemm_packed_meta_bytes_w8": (_sz, [_i, _i, _i, _i]),
    "mpgemm_pack_weights_w8": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "mpgemm_unpack_w8": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "mpgemm_w8a16": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "mpgemm_w8a16_config": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _i,
                                 _vp]),
    "mpgemm_wfp8a16": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "mpgemm_kv_block_bytes": (_sz, [_i, _i]),
    "mpgemm_kv_pack": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _vp,
                            _vp]),
    "mpgemm_attention_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "mpgemm_attention_decode_kv8": (_i, [_vp, _i, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i,
                                         ctypes.c_float, _vp, _vp, _sz, _vp]),
    "mpgemm_attention_decode_kvfp8": (_i, [_vp, _i, _i, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i,
                                           _i, ctypes.c_float, _vp, _vp, _sz, _vp]),
    "mpgemm_packed_code_bytes_lowbit": (_sz, [_i, _i, _i]),
    "mpgemm_workspace_bytes_lowbit": (_sz, [_i, _i, _i, _i, _i, _i]),
    "mpgemm_pack_weights_lowbit": (_i, [_i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "mpgemm_unpack_lowbit": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "mpgemm_wlowbit_a16": (_i, [_i, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "mpgemm_wlowbit_a16_config": (_i, [_i, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz,
                                       _i, _vp]),
    "mpgemm_wfp8a16_config": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _i,
                                   _vp]),
}

FP8_FORMATS = {"e4m3": 0, "e5m2": 1}    # mpgemm_fp8_format


class MpgemmError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = lib().mpgemm_status_string(status).decode()
        super().__init__(f"{call} failed: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmpgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m weight_only_quantized_mpgemm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, call: str) -> None:
    if status != 0:
        raise MpgemmError(status, call)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------- packed weights --

@dataclasses.dataclass
class PackedWeights:
    """Packed planes of one [K, N] weight matrix (see include/mpgemm.h): layout v1 for
    4-bit codes, the 8-bit layout for bits == 8 (integer codes, or FP8 codes when `fp8`
    names their format)."""
    codes: torch.Tensor          # uint8 [K*N/2] (4-bit) or [K*N] (8-bit)
    meta: torch.Tensor           # uint8 [(K/g)*N*2 (+ zeros: (K/g)*N/2 or (K/g)*N)]
    K: int
    N: int
    group: int
    symmetric: bool
    bits: int = 4
    fp8: str | None = None       # "e4m3" or "e5m2" for FP8 codes

    @property
    def nbytes(self) -> int:
        return self.codes.numel() + self.meta.numel()


def _group_rows(K: int, group: int) -> int:
    """Scale/zero rows of a K-deep weight: ceil(K / group) (the last group may be short)."""
    if group not in (64, 128):
        raise ValueError(f"group must be 64 or 128, got {group}")
    return -(-K // group)


def packed_code_bytes(K: int, N: int) -> int:
    return int(lib().mpgemm_packed_code_bytes(K, N))


def packed_meta_bytes(K: int, N: int, group: int, symmetric: bool) -> int:
    return int(lib().mpgemm_packed_meta_bytes(K, N, group, int(bool(symmetric))))


def empty_packed(K: int, N: int, group: int, symmetric: bool,
                 device="cuda") -> PackedWeights:
    cb = packed_code_bytes(K, N)
    mb = packed_meta_bytes(K, N, group, symmetric)
    if K * N and (cb == 0 or mb == 0):
        raise MpgemmError(-2, "empty_packed")
    return PackedWeights(torch.empty(cb, dtype=torch.uint8, device=device),
                         torch.empty(mb, dtype=torch.uint8, device=device),
                         K, N, group, bool(symmetric))


def pack_weights(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor | None,
                 group: int, out: PackedWeights | None = None) -> PackedWeights:
    """Offline packing (mpgemm_pack_weights).

    codes  uint8 [K, N] (values 0..15); scales float16 [G, N] with G = ceil(K/g); zeros
    uint8 [G, N] (values 0..15) or None for symmetric codes with zero 8.  Any N and any
    K % 8 == 0: ragged shapes are padded in the packed planes (include/mpgemm.h).
    """
    K, N = codes.shape
    _need(codes, torch.uint8, (K, N), "codes")
    rows = _group_rows(K, group)
    _need(scales, torch.float16, (rows, N), "scales")
    if zeros is not None:
        _need(zeros, torch.uint8, (rows, N), "zeros")
    if out is None:
        out = empty_packed(K, N, group, zeros is None, codes.device)
    st = lib().mpgemm_pack_weights(_ptr(codes), _ptr(scales), _ptr(zeros), K, N, group,
                                   _ptr(out.codes), _ptr(out.meta), _stream(codes.device))
    _check(st, "mpgemm_pack_weights")
    return out


def pack_weights_w8(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor | None,
                    group: int) -> PackedWeights:
    """Offline packing of 8-bit codes (mpgemm_pack_weights_w8).

    codes  uint8 [K, N] (0..255); scales float16 [ceil(K/g), N]; zeros uint8 of the same
    shape or None for symmetric codes with zero 128.
    """
    K, N = codes.shape
    _need(codes, torch.uint8, (K, N), "codes")
    rows = _group_rows(K, group)
    _need(scales, torch.float16, (rows, N), "scales")
    if zeros is not None:
        _need(zeros, torch.uint8, (rows, N), "zeros")
    cb = int(lib().mpgemm_packed_code_bytes_w8(K, N))
    mb = int(lib().mpgemm_packed_meta_bytes_w8(K, N, group, int(zeros is None)))
    if K * N and (cb == 0 or mb == 0):
        raise MpgemmError(-2, "pack_weights_w8")
    out = PackedWeights(torch.empty(cb, dtype=torch.uint8, device=codes.device),
                        torch.empty(mb, dtype=torch.uint8, device=codes.device),
                        K, N, group, zeros is None, 8)
    st = lib().mpgemm_pack_weights_w8(_ptr(codes), _ptr(scales), _ptr(zeros), K, N, group,
                                      _ptr(out.codes), _ptr(out.meta), _stream(codes.device))
    _check(st, "mpgemm_pack_weights_w8")
    return out


def pack_weights_fp8(codes: torch.Tensor, scales: torch.Tensor, group: int,
                     fmt: str = "e4m3") -> PackedWeights:
    """Offline packing of FP8 codes: the 8-bit layout with no zero plane
    (mpgemm_pack_weights_w8 with zeros == NULL).

    codes  uint8 [K, N] FP8 bit patterns (or a float8_e4m3fn / float8_e5m2 tensor, whose
    format then decides `fmt`); scales float16 [ceil(K/g), N].
    """
    if codes.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        fmt = "e4m3" if codes.dtype == torch.float8_e4m3fn else "e5m2"
        codes = codes.view(torch.uint8)
    if fmt not in FP8_FORMATS:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    out = pack_weights_w8(codes, scales, None, group)
    out.fp8 = fmt
    return out


def pack_weights_lowbit(bits: int, codes: torch.Tensor, scales: torch.Tensor,
                        zeros: torch.Tensor | None, group: int) -> PackedWeights:
    """Offline packing of 2-bit or 3-bit codes (mpgemm_pack_weights_lowbit).

    codes uint8 [K, N] (0..2^bits-1); scales float16 [ceil(K/g), N]; zeros uint8 of the
    same shape or None for symmetric codes with zero 2^(bits-1).
    """
    if bits not in (2, 3):
        raise ValueError(f"bits must be 2 or 3, got {bits}")
    K, N = codes.shape
    _need(codes, torch.uint8, (K, N), "codes")
    rows = _group_rows(K, group)
    _need(scales, torch.float16, (rows, N), "scales")
    if zeros is not None:
        _need(zeros, torch.uint8, (rows, N), "zeros")
    cb = int(lib().mpgemm_packed_code_bytes_lowbit(bits, K, N))
    mb = packed_meta_bytes(K, N, group, zeros is None)
    if K * N and (cb == 0 or mb == 0):
        raise MpgemmError(-2, "pack_weights_lowbit")
    out = PackedWeights(torch.empty(cb, dtype=torch.uint8, device=codes.device),
                        torch.empty(mb, dtype=torch.uint8, device=codes.device),
                        K, N, group, zeros is None, bits)
    st = lib().mpgemm_pack_weights_lowbit(bits, _ptr(codes), _ptr(scales), _ptr(zeros), K, N,
                                          group, _ptr(out.codes), _ptr(out.meta),
                                          _stream(codes.device))
    _check(st, "mpgemm_pack_weights_lowbit")
    return out


def unpack(packed: PackedWeights):
    """Inverse of packing (mpgemm_unpack / mpgemm_unpack_w8): (codes, scales, zeros or
    None)."""
    K, N, g = packed.K, packed.N, packed.group
    dev = packed.codes.device
    codes = torch.empty((K, N), dtype=torch.uint8, device=dev)
    scales = torch.empty((_group_rows(K, g), N), dtype=torch.float16, device=dev)
    zeros = None if packed.symmetric else torch.empty((_group_rows(K, g), N),
                                                      dtype=torch.uint8, device=dev)
    args = (_ptr(packed.codes), _ptr(packed.meta), K, N, g, int(packed.symmetric), _ptr(codes),
            _ptr(scales), _ptr(zeros), _stream(dev))
    if packed.bits in (2, 3):
        name = "mpgemm_unpack_lowbit"
        st = lib().mpgemm_unpack_lowbit(packed.bits, *args)
    else:
        name = "mpgemm_unpack_w8" if packed.bits == 8 else "mpgemm_unpack"
        st = getattr(lib(), name)(*args)
    _check(st, name)
    return codes, scales, zeros


# ------------------------------------------------------------------------- the GEMM --

def _act_code(dtype: torch.dtype) -> int:
    if dtype == torch.float16:
        return F16
    if dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"activations must be float16 or bfloat16, got {dtype}")


def select_config(M: int, N: int, K: int, group: int, dtype: torch.dtype) -> int:
    return int(lib().mpgemm_select_config(M, N, K, group, _act_code(dtype)))


def config_name(config_id: int) -> str:
    return lib().mpgemm_config_name(config_id).decode()


def prefill_schedule(M: int, N: int, K: int, config_id: int, cus: int = 256):
    """Host-side workgroup schedule of a tiled kernel: (info dict, work array [grid][4] of
    M tile, N tile, K part, split tile index or -1)."""
    info = torch.zeros(8, dtype=torch.int32)
    grid = lib().mpgemm_prefill_schedule(M, N, K, config_id, cus, info.data_ptr(), None, 0)
    _check(min(grid, 0), "mpgemm_prefill_schedule")
    work = torch.zeros(grid, 4, dtype=torch.int32)
    _check(min(0, lib().mpgemm_prefill_schedule(M, N, K, config_id, cus, info.data_ptr(),
                                                work.data_ptr(), grid)),
           "mpgemm_prefill_schedule")
    keys = ("grid", "tile_m", "tile_n", "tiles_m", "tiles_n", "full", "parts", "loop_k")
    return dict(zip(keys, info.tolist())), work


def prefill_launches(M: int, N: int, K: int, config_id: int, cus: int = 256):
    """(kernel launches, first column of the second launch or N) of one call of a tiled
    configuration, computed on the host."""
    col = ctypes.c_int(0)
    n = lib().mpgemm_prefill_launches(M, N, K, config_id, cus, ctypes.addressof(col))
    _check(min(n, 0), "mpgemm_prefill_launches")
    return n, col.value


class WorkspaceCache:
    """Device workspaces keyed by (device index, stream handle), grown on demand and never
    freed: graphs captured with an older (smaller) one keep a valid pointer.

    Split-K calls that share a workspace must not overlap in time (their arrival counters
    would race), and calls on different streams may overlap, so every stream gets a
    workspace of its own.  `alloc(device_index, nbytes)` returns a zero-filled uint8
    tensor; the GEMM kernels leave the counters zero after every call, so a buffer is
    zeroed only once."""

    def __init__(self, alloc):
        self._alloc = alloc
        self._bufs: dict[tuple[int, int], list[torch.Tensor]] = {}

    def get(self, device_index: int, stream: int, nbytes: int, capturing: bool = False):
        """The workspace of (device_index, stream) with at least `nbytes`.  Under graph
        capture nothing is allocated: a stream being captured (torch captures on a side
        stream) without a large enough workspace of its own takes one of another stream of
        the device (the eager warm-up call's).  Such a graph must then not replay while
        split-K calls run on that other stream; graphs that need that pass their own
        `workspace`."""
        if nbytes == 0:
            return None
        cached = self._bufs.setdefault((device_index, stream), [])
        if cached and cached[-1].numel() >= nbytes:
            return cached[-1]
        if capturing:
            for (dev, _), bufs in self._bufs.items():
                if dev == device_index and bufs and bufs[-1].numel() >= nbytes:
                    return bufs[-1]
            raise MpgemmError(-4, f"allocating a {nbytes}-byte workspace during graph "
                                  "capture (make one eager call of this shape first)")
        ws = self._alloc(device_index, max(nbytes, 1 << 20))
        cached.append(ws)
        return ws


def _device_index(device: torch.device) -> int:
    return device.index if device.index is not None else torch.cuda.current_device()


_WORKSPACES = WorkspaceCache(
    lambda idx, n: torch.zeros(n, dtype=torch.uint8, device=torch.device("cuda", idx)))


def workspace_for(device: torch.device, nbytes: int) -> torch.Tensor | None:
    """The cached zeroed workspace of `device` and its current stream with at least
    `nbytes` (None for 0)."""
    if nbytes == 0:
        return None
    idx = _device_index(device)
    return _WORKSPACES.get(idx, torch.cuda.current_stream(idx).cuda_stream, nbytes,
                           torch.cuda.is_current_stream_capturing())


def _gemm(kind: str, x: torch.Tensor, packed: PackedWeights, out, config, workspace):
    have = "fp8" if packed.fp8 else f"w{packed.bits}"
    if have != kind:
        raise ValueError(f"weights are packed as {have} codes, not {kind}")
    M, K = x.shape
    if K != packed.K:
        raise ValueError(f"x has K={K}, weights have K={packed.K}")
    act = _act_code(x.dtype)
    _need(x, x.dtype, (M, K), "x")
    N = packed.N
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _need(out, x.dtype, (M, N), "out")
    if kind in ("w2", "w3"):
        ws = int(lib().mpgemm_workspace_bytes_lowbit(packed.bits, M, N, K, packed.group, act))
    else:
        ws = int(lib().mpgemm_workspace_bytes(M, N, K, packed.group, act))
    if workspace is None:
        workspace = workspace_for(x.device, ws)
    else:                       # all of it: the 256 x 256 tile may split K in more than ws
        _need(workspace, torch.uint8, (workspace.numel(),), "workspace")
        ws = workspace.numel()
    if kind == "fp8":
        args = (_ptr(x), act, FP8_FORMATS[packed.fp8], _ptr(packed.codes), _ptr(packed.meta),
                M, N, K, packed.group, _ptr(out), _ptr(workspace), ws)
    elif kind in ("w2", "w3"):
        args = (packed.bits, _ptr(x), act, _ptr(packed.codes), _ptr(packed.meta), M, N, K,
                packed.group, int(packed.symmetric), _ptr(out), _ptr(workspace), ws)
    else:
        args = (_ptr(x), act, _ptr(packed.codes), _ptr(packed.meta), M, N, K, packed.group,
                int(packed.symmetric), _ptr(out), _ptr(workspace), ws)
    base = {"fp8": "mpgemm_wfp8a16", "w2": "mpgemm_wlowbit_a16", "w3": "mpgemm_wlowbit_a16"}
    name = base.get(kind, f"mpgemm_{kind}a16") + ("_config" if config else "")
    fn = getattr(lib(), name)
    st = fn(*args, int(config), _stream(x.device)) if config else fn(*args, _stream(x.device))
    _check(st, name)
    return out


def w4a16(x: torch.Tensor, packed: PackedWeights, out: torch.Tensor | None = None,
          config: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ dequant(W) (mpgemm_w4a16; mpgemm_w4a16_config when config != 0).

    x float16 or bfloat16 [M, K]; returns (or fills `out`) [M, N] in the same format.
    workspace: uint8 device tensor, zeroed before its first use (default: the device's
    cached one).
    """
    return _gemm("w4", x, packed, out, config, workspace)


def w4a16_noalloc(x: torch.Tensor, packed: PackedWeights,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ dequant(W) through mpgemm_w4a16_noalloc: no workspace, the library's static
    per-device scratch instead (see include/mpgemm.h; calls overlapping on one GPU race).
    `out` is allocated here only when it is not given."""
    if packed.bits != 4 or packed.fp8:
        raise ValueError("w4a16_noalloc takes 4-bit packed weights")
    M, K = x.shape
    if K != packed.K:
        raise ValueError(f"x has K={K}, weights have K={packed.K}")
    act = _act_code(x.dtype)
    _need(x, x.dtype, (M, K), "x")
    N = packed.N
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _need(out, x.dtype, (M, N), "out")
    st = lib().mpgemm_w4a16_noalloc(_ptr(x), act, _ptr(packed.codes), _ptr(packed.meta), M, N,
                                    K, packed.group, int(packed.symmetric), _ptr(out),
                                    _stream(x.device))
    _check(st, "mpgemm_w4a16_noalloc")
    return out


def w8a16(x: torch.Tensor, packed: PackedWeights, out: torch.Tensor | None = None,
          config: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ dequant(W8) for weights packed by pack_weights_w8 (mpgemm_w8a16; the
    _config variant when config != 0).  Arguments as for w4a16."""
    return _gemm("w8", x, packed, out, config, workspace)


def wlowbit_a16(x: torch.Tensor, packed: PackedWeights, out: torch.Tensor | None = None,
                config: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ dequant(W) for 2-bit or 3-bit weights packed by pack_weights_lowbit
    (mpgemm_wlowbit_a16; the _config variant when config != 0).  Arguments as for w4a16."""
    if packed.bits not in (2, 3):
        raise ValueError(f"weights are packed with {packed.bits}-bit codes, not 2 or 3")
    return _gemm(f"w{packed.bits}", x, packed, out, config, workspace)


def wfp8a16(x: torch.Tensor, packed: PackedWeights, out: torch.Tensor | None = None,
            config: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ (fp8(W) * s) for weights packed by pack_weights_fp8 (mpgemm_wfp8a16; the
    _config variant when config != 0).  Arguments as for w4a16."""
    return _gemm("fp8", x, packed, out, config, workspace)


# ------------------------------------------- attention decode (8-bit / FP8 KV cache) --

# Attention partials need no initialization, but must not share the GEMM workspace (whose
# split-K counters have to stay zero between calls), nor a buffer with an attention call
# that may run at the same time on another stream: a cache of their own, per stream.
_ATTN_WORKSPACES = WorkspaceCache(
    lambda idx, n: torch.empty(n, dtype=torch.uint8, device=torch.device("cuda", idx)))


def _attention_workspace(device: torch.device, nbytes: int) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    idx = _device_index(device)
    return _ATTN_WORKSPACES.get(idx, torch.cuda.current_stream(idx).cuda_stream, nbytes,
                                torch.cuda.is_current_stream_capturing())


def kv_block_bytes(Hkv: int, D: int) -> int:
    """Bytes of one 64-token cache block holding every KV head (mpgemm_kv_block_bytes)."""
    return int(lib().mpgemm_kv_block_bytes(Hkv, D))


def kv_pack(cache: torch.Tensor, table_row: torch.Tensor, t0: int, kc: torch.Tensor,
            ks: torch.Tensor, kz: torch.Tensor | None, vc: torch.Tensor, vs: torch.Tensor,
            vz: torch.Tensor | None) -> None:
    """Writes tokens t0 .. t0+n-1 of one sequence into `cache` (mpgemm_kv_pack).

    kc, vc uint8 [n, Hkv, D]; ks, vs float16 [n, Hkv]; kz, vz uint8 [n, Hkv], or both None
    for FP8 codes (no zero points); table_row int32 [table_len] (device); cache uint8
    [num_blocks * kv_block_bytes(Hkv, D)].
    """
    n, Hkv, D = kc.shape
    if (kz is None) != (vz is None):
        raise ValueError("kz and vz are given together or not at all")
    need = [(kc, torch.uint8, (n, Hkv, D), "kc"), (vc, torch.uint8, (n, Hkv, D), "vc"),
            (ks, torch.float16, (n, Hkv), "ks"), (vs, torch.float16, (n, Hkv), "vs")]
    if kz is not None:
        need += [(kz, torch.uint8, (n, Hkv), "kz"), (vz, torch.uint8, (n, Hkv), "vz")]
    for t, dt, shape, name in need:
        _need(t, dt, shape, name)
    _need(table_row, torch.int32, (table_row.numel(),), "table_row")
    bb = kv_block_bytes(Hkv, D)
    if bb == 0:
        raise MpgemmError(-2, "kv_pack")
    _need(cache, torch.uint8, (cache.numel(),), "cache")
    st = lib().mpgemm_kv_pack(_ptr(kc), _ptr(ks), _ptr(kz), _ptr(vc), _ptr(vs), _ptr(vz), n, t0,
                              Hkv, D, _ptr(table_row), table_row.numel(), cache.numel() // bb,
                              _ptr(cache), _stream(cache.device))
    _check(st, "mpgemm_kv_pack")


def attention_decode_kv8(q: torch.Tensor, cache: torch.Tensor, block_table: torch.Tensor,
                         lens: torch.Tensor, Hkv: int, max_len: int, scale: float,
                         out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step of attention over a packed 8-bit KV cache
    (mpgemm_attention_decode_kv8).  q float16/bfloat16 [B, Hq, D]; block_table int32
    [B, table_stride]; lens int32 [B] (each <= max_len); returns [B, Hq, D]."""
    return _attention(None, q, cache, block_table, lens, Hkv, max_len, scale, out, workspace)


def attention_decode_kvfp8(q: torch.Tensor, cache: torch.Tensor, block_table: torch.Tensor,
                           lens: torch.Tensor, Hkv: int, max_len: int, scale: float,
                           fp8_format: str = "e4m3", out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The same over a cache of FP8 codes ("e4m3" or "e5m2") packed without zero points
    (mpgemm_attention_decode_kvfp8)."""
    if fp8_format not in FP8_FORMATS:
        raise ValueError(f"unknown FP8 format {fp8_format!r}")
    return _attention(fp8_format, q, cache, block_table, lens, Hkv, max_len, scale, out,
                      workspace)


def _attention(fp8_format, q, cache, block_table, lens, Hkv, max_len, scale, out, workspace):
    call = "mpgemm_attention_decode_kv8" if fp8_format is None else "mpgemm_attention_decode_kvfp8"
    B, Hq, D = q.shape
    act = _act_code(q.dtype)
    _need(q, q.dtype, (B, Hq, D), "q")
    _need(block_table, torch.int32, (B, block_table.shape[1] if block_table.dim() == 2 else -1),
          "block_table")
    _need(lens, torch.int32, (B,), "lens")
    bb = kv_block_bytes(Hkv, D)
    if bb == 0:
        raise MpgemmError(-2, call)
    _need(cache, torch.uint8, (cache.numel(),), "cache")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    _need(out, q.dtype, (B, Hq, D), "out")
    ws = int(lib().mpgemm_attention_workspace_bytes(B, Hq, Hkv, D, max_len))
    if workspace is None:
        workspace = _attention_workspace(q.device, ws)
    elif ws:
        _need(workspace, torch.uint8, (workspace.numel(),), "workspace")
        ws = workspace.numel()
    rest = (_ptr(cache), cache.numel() // bb, _ptr(block_table), block_table.shape[1],
            _ptr(lens), B, Hq, Hkv, D, max_len, ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), ws, _stream(q.device))
    if fp8_format is None:
        st = lib().mpgemm_attention_decode_kv8(_ptr(q), act, *rest)
    else:
        st = lib().mpgemm_attention_decode_kvfp8(_ptr(q), act, FP8_FORMATS[fp8_format], *rest)
    _check(st, call)
    return out
