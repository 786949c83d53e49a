"""C ABI checks that need no GPU: the library loads, exports every function that
include/mpgemm.h declares, answers size queries, and rejects bad arguments before
enqueueing anything (every case here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

import weight_only_quantized_mpgemm_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpgemm.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, -1, -2, -3, -4
A = 0x10000          # a 16-byte-aligned fake device address; never dereferenced here
MIS = 0x10008        # a misaligned one


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpgemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("mpgemm_pack_weights", "mpgemm_w4a16", "mpgemm_unpack"):
        assert must in names


def test_library_exports_every_declared_function():
    lib = mp.lib()
    names = declared_functions()
    assert set(names) == set(mp.SIGNATURES), "binding and header disagree"
    for name in names:
        assert hasattr(lib, name), name


def test_layout_version_and_sizes():
    lib = mp.lib()
    assert lib.mpgemm_layout_version() == mp.LAYOUT_VERSION == 1
    assert mp.packed_code_bytes(4096, 6144) == 4096 * 6144 // 2
    assert mp.packed_meta_bytes(4096, 6144, 128, False) == 32 * 6144 * 2 + 32 * 6144 // 2
    assert mp.packed_meta_bytes(5120, 10240, 64, True) == 80 * 10240 * 2
    assert mp.packed_code_bytes(100, 16) == 0          # K % 8 != 0
    assert mp.packed_meta_bytes(256, 32, 32, False) == 0    # unsupported group
    # ragged shapes: planes of the matrix padded to Kp x Np (Np: 16s; Kp: 128s)
    assert mp.packed_code_bytes(200, 24) == 256 * 32 // 2
    assert mp.packed_meta_bytes(200, 24, 64, False) == 4 * 32 * 2 + 4 * 32 // 2
    assert mp.packed_code_bytes(384, 1) == 384 * 16 // 2
    assert mp.lib().mpgemm_packed_code_bytes_w8(136, 7) == 256 * 16
    assert mp.lib().mpgemm_packed_meta_bytes_w8(136, 7, 128, 1) == 2 * 16 * 2
    assert lib.mpgemm_workspace_bytes(1, 28672, 4096, 128, 0) == 0     # wide N: no K split


def test_status_strings():
    lib = mp.lib()
    for code, name in mp.STATUS.items():
        assert lib.mpgemm_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.mpgemm_status_string(42)


def test_selector_and_config_names():
    sel = mp.lib().mpgemm_select_config
    assert sel(1, 4096, 4096, 128, 0) == 1
    assert sel(16, 4096, 4096, 128, 0) == 1
    assert sel(16, 57344, 8192, 128, 0) == 1
    assert sel(17, 4096, 4096, 128, 0) == 2
    assert sel(32, 57344, 4096, 128, 0) == 2
    # 33..64 rows: the strip kernel only for the smallest matrices
    assert sel(33, 4096, 4096, 128, 0) == 3
    assert sel(48, 4096, 4096, 128, 0) == 3
    assert sel(33, 6144, 4096, 128, 0) == 13          # 192 workgroups against 96
    assert sel(49, 4096, 4096, 128, 1) == 13         # 4-bit, g = 128: the eight-stage ring
    assert sel(64, 4096, 4096, 128, 1) == 13
    assert sel(64, 4096, 4096, 64, 1) == 4           # g = 64: four stages
    assert sel(64, 4096, 4224, 128, 0) == 13          # N K past 4096 * 4096; 32 tiles, 16
    assert sel(33, 16384, 4096, 128, 0) == 13         # both fill all 256 units
    assert sel(64, 57344, 8192, 128, 1) == 12         # 448 tiles of 256 x 128: two rounds
    # 33..128 rows: the tile whose grid (K split on 256 units) fills more units
    assert sel(65, 4096, 4096, 128, 0) == 13          # 128 workgroups against 64
    assert sel(96, 28672, 4096, 128, 0) == 13         # 224 each, only 256 x 128 unsplit
    assert sel(128, 10240, 8192, 128, 1) == 12        # 160 each
    assert sel(128, 8192, 8192, 128, 1) == 13         # 256 each: every unit filled
    assert sel(128, 5120, 25600, 64, 0) == 13         # 160 against 80
    assert sel(128, 4096, 14336, 128, 0) == 13        # 256 against 128
    assert sel(64, 8192, 28672, 128, 1) == 12         # 256 each, K >= 16384
    assert sel(128, 8192, 28672, 128, 1) == 12
    # larger M: the 256-row tile, except where the 128-row one pads less (257..384 rows)
    assert sel(129, 4096, 4096, 128, 0) == 13
    assert sel(256, 28672, 4096, 128, 0) == 13
    assert sel(384, 6144, 4096, 128, 0) == 12
    assert sel(384, 8192, 28672, 128, 1) == 13        # long K
    assert sel(385, 6144, 4096, 128, 0) == 13
    assert sel(1024, 6144, 4096, 128, 0) == 13
    assert sel(2048, 4096, 4096, 128, 0) == 12        # M >= 2048, N < 16384, K < 8192
    assert sel(2048, 4096, 4104, 128, 0) == 12        # ragged K
    assert sel(2048, 4096, 14336, 128, 0) == 13       # long K
    # the 256 x 256 tile where its grid covers three quarters of the 256 units or more
    assert sel(2048, 6144, 4096, 128, 0) == 14        # 192 tiles
    assert sel(2048, 28672, 4096, 128, 0) == 14
    assert sel(8192, 28672, 4096, 128, 0) == 14
    assert sel(8192, 4096, 14336, 128, 0) == 14       # 512 tiles
    assert sel(256, 57344, 8192, 128, 1) == 14        # 224 tiles
    assert sel(300, 57344, 8192, 128, 1) == 12        # 257..384 rows: the 128-row tile
    assert sel(1024, 4096, 14336, 128, 0) == 13       # 64 tiles: the split 256 x 128 one
    assert sel(1024, 10240, 5120, 64, 0) == 14        # 160 tiles, one round; 320 of the others
    assert sel(768, 10240, 5120, 64, 0) == 13         # 120 tiles: under half the units
    assert sel(2048, 4096, 4096, 128, 0) == 12        # 128 tiles, but 256 x 128 fits one round
    for cid in (1, 2, 3, 4, 12, 13, 14):
        assert mp.config_name(cid)
    for cid in (7, 10, 11):
        assert mp.config_name(cid) == ""


def _gemm(X=A, dtype=0, pc=A, pm=A, M=16, N=256, K=256, g=128, sym=0, Y=A, cfg=None):
    lib = mp.lib()
    args = [ctypes.c_void_p(X), dtype, ctypes.c_void_p(pc), ctypes.c_void_p(pm), M, N, K, g,
            sym, ctypes.c_void_p(Y), None, 0]
    if cfg is None:
        return lib.mpgemm_w4a16(*args, None)
    return lib.mpgemm_w4a16_config(*args, cfg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), INVALID),
    (dict(sym=2), INVALID),
    (dict(M=-1), INVALID),
    (dict(K=100), UNSUPPORTED),
    (dict(K=384, g=256), UNSUPPORTED),
    (dict(g=32), UNSUPPORTED),
    (dict(K=260), UNSUPPORTED),                     # K % 8 != 0
    (dict(N=-1), INVALID),
    (dict(M=70000, K=65536), UNSUPPORTED),          # M*K beyond 2^31
    (dict(M=16384 - 128, K=131072), UNSUPPORTED),    # (M+128)*K at 2^31
    (dict(X=0), INVALID),
    (dict(pc=0), INVALID),
    (dict(pm=0), INVALID),
    (dict(Y=0), INVALID),
    (dict(X=MIS), ALIGN),
    (dict(Y=MIS), ALIGN),
    (dict(pc=MIS), ALIGN),
    (dict(pm=MIS), ALIGN),
    (dict(cfg=7), INVALID),
    (dict(cfg=1, M=17), UNSUPPORTED),
    (dict(cfg=4, M=65), UNSUPPORTED),
    (dict(M=0), OK),                                  # empty: a valid no-op, nothing enqueued
    (dict(N=0), OK),
    (dict(M=0, X=0, pc=0, pm=0, Y=0), OK),
])
def test_gemm_validation(kw, status):
    assert _gemm(**kw) == status


def test_pack_and_unpack_validation():
    lib = mp.lib()
    vp = ctypes.c_void_p
    assert lib.mpgemm_pack_weights(None, vp(A), None, 256, 32, 128, vp(A), vp(A), None) == INVALID
    assert lib.mpgemm_pack_weights(vp(A), vp(A), None, 204, 32, 128, vp(A), vp(A), None) == UNSUPPORTED
    assert lib.mpgemm_pack_weights(vp(A), vp(A), None, 256, 32, 96, vp(A), vp(A), None) == UNSUPPORTED
    assert lib.mpgemm_pack_weights(vp(A), vp(MIS), None, 256, 32, 128, vp(A), vp(A), None) == ALIGN
    assert lib.mpgemm_pack_weights(vp(A), vp(A), vp(MIS), 256, 32, 128, vp(A), vp(A), None) == ALIGN
    assert lib.mpgemm_pack_weights(None, None, None, 0, 32, 128, None, None, None) == OK
    # asymmetric unpack needs somewhere to put the zeros
    assert lib.mpgemm_unpack(vp(A), vp(A), 256, 32, 128, 0, vp(A), vp(A), None, None) == INVALID
    assert lib.mpgemm_unpack(vp(A), vp(A), 256, 32, 128, 3, vp(A), vp(A), vp(A), None) == INVALID
    assert lib.mpgemm_unpack(vp(A), vp(A), 256, 32, 128, 1, vp(MIS), vp(A), None, None) == ALIGN


def test_binding_rejects_cpu_tensors():
    import torch
    codes = torch.zeros((256, 32), dtype=torch.uint8)
    scales = torch.zeros((2, 32), dtype=torch.float16)
    with pytest.raises(ValueError):
        mp.pack_weights(codes, scales, None, 128)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "weight_only_quantized_mpgemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "mpgemm_oracle" not in text, f


def test_split_k_workspace_is_sized_and_required(monkeypatch):
    """A split of K over workgroups needs a workspace; without one (or with too small or a
    misaligned one) the call fails validation and enqueues nothing.  Every call here must
    fail validation: the pointers are fake."""
    lib = mp.lib()
    assert lib.mpgemm_workspace_bytes(16, 256, 256, 128, 0) == 0       # default: no split
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", "1,1,2")
    need = lib.mpgemm_workspace_bytes(16, 256, 256, 128, 0)
    # the fixed 256 KiB counter region, then 16 strip groups x 2 splits x 1 KiB of
    # partials per row block, sized for every configuration that can run M = 16 (up to 4)
    assert need == 256 * 1024 + 16 * 2 * 4 * 1024
    # large M: only the 64-row chunks of 2- and 3-bit codes run the small-M kernel
    assert lib.mpgemm_workspace_bytes(2048, 256, 256, 128, 0) == 256 * 1024 + 16 * 2 * 4 * 1024
    assert _gemm() == -4                                                # workspace NULL
    args = [ctypes.c_void_p(A), 0, ctypes.c_void_p(A), ctypes.c_void_p(A), 16, 256, 256, 128,
            0, ctypes.c_void_p(A), ctypes.c_void_p(A), 100]
    assert lib.mpgemm_w4a16(*args, None) == -4                         # far too small
    args[-1] = need
    args[-2] = ctypes.c_void_p(MIS)
    assert lib.mpgemm_w4a16(*args, None) == -4                         # misaligned


def _fp8(fmt=0, X=A, dtype=0, pc=A, pm=A, M=16, N=256, K=256, g=128, Y=A, cfg=None):
    lib = mp.lib()
    args = [ctypes.c_void_p(X), dtype, fmt, ctypes.c_void_p(pc), ctypes.c_void_p(pm), M, N, K,
            g, ctypes.c_void_p(Y), None, 0]
    if cfg is None:
        return lib.mpgemm_wfp8a16(*args, None)
    return lib.mpgemm_wfp8a16_config(*args, cfg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=2), INVALID),
    (dict(fmt=-1), INVALID),
    (dict(dtype=2), INVALID),
    (dict(K=100), UNSUPPORTED),
    (dict(X=0), INVALID),
    (dict(Y=MIS), ALIGN),
    (dict(cfg=10, M=128), INVALID),                  # no such configuration
    (dict(cfg=11, M=128, K=384), INVALID),
    (dict(cfg=12, M=128, K=4), UNSUPPORTED),
    (dict(M=0), OK),
])
def test_fp8_gemm_validation(kw, status):
    assert _fp8(**kw) == status


def test_binding_fp8_format_names_match_header():
    text = open(HEADER).read()
    assert "MPGEMM_FP8_E4M3 = 0" in text and "MPGEMM_FP8_E5M2 = 1" in text
    assert mp.FP8_FORMATS == {"e4m3": 0, "e5m2": 1}


@pytest.mark.parametrize("cfg", [5, 10, 11, 15, -1])
def test_unknown_configuration_ids_are_rejected(cfg):
    # 10 and 11 named 16x16x32 tiled kernels that the selector never chose; they are gone
    assert _gemm(M=128, K=256, cfg=cfg) == INVALID
    assert _gemm(M=128, K=200, cfg=cfg) == INVALID


def _low(bits=2, cfg=0, M=16, K=256):
    lib = mp.lib()
    vp = ctypes.c_void_p
    return lib.mpgemm_wlowbit_a16_config(bits, vp(A), 0, vp(A), vp(A), M, 256, K, 128, 0,
                                         vp(A), None, 0, cfg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=4), INVALID),
    (dict(bits=1), INVALID),
    (dict(cfg=12, M=128), WORKSPACE),        # tiled: the 4-bit rewrite needs the workspace
    (dict(cfg=13, M=128), WORKSPACE),
    (dict(cfg=10, M=128), INVALID),          # no such configuration
    (dict(cfg=1, M=17), UNSUPPORTED),
    (dict(K=12), UNSUPPORTED),
    (dict(M=0), OK),
])
def test_lowbit_gemm_validation(kw, status):
    assert _low(**kw) == status


def test_lowbit_sizes_and_pack_validation():
    lib = mp.lib()
    vp = ctypes.c_void_p
    assert lib.mpgemm_packed_code_bytes_lowbit(2, 256, 64) == 256 * 64 * 2 // 8
    assert lib.mpgemm_packed_code_bytes_lowbit(3, 200, 40) == 256 * 48 * 3 // 8
    assert lib.mpgemm_packed_code_bytes_lowbit(4, 256, 64) == 0
    assert lib.mpgemm_pack_weights_lowbit(5, vp(A), vp(A), None, 256, 32, 128, vp(A), vp(A),
                                          None) == INVALID
    assert lib.mpgemm_pack_weights_lowbit(2, None, vp(A), None, 256, 32, 128, vp(A), vp(A),
                                          None) == INVALID
    assert lib.mpgemm_unpack_lowbit(3, vp(A), vp(A), 256, 32, 128, 0, vp(A), vp(A), None,
                                    None) == INVALID


def test_kv_block_bytes_pad_heads_to_a_multiple_of_64():
    lib = mp.lib()
    assert lib.mpgemm_kv_block_bytes(8, 128) == 8 * (128 * 128 + 384)
    assert lib.mpgemm_kv_block_bytes(8, 96) == 8 * (128 * 128 + 384)
    assert lib.mpgemm_kv_block_bytes(2, 16) == 2 * (128 * 64 + 384)
    assert lib.mpgemm_kv_block_bytes(4, 192) == lib.mpgemm_kv_block_bytes(4, 176) == 4 * (128 * 192 + 384)
    for D in (0, 8, 100, 264, 512):                       # not a multiple of 16 in 16..256
        assert lib.mpgemm_kv_block_bytes(8, D) == 0
    assert lib.mpgemm_kv_block_bytes(0, 128) == 0


def test_attention_rejects_unsupported_head_sizes_before_launching():
    lib = mp.lib()
    for D in (8, 100, 272):
        for fn, extra in ((lib.mpgemm_attention_decode_kv8, ()), (lib.mpgemm_attention_decode_kvfp8, (0,))):
            args = (A, 0, *extra, A, 4, A, 1, A, 1, 8, 2, D, 64, ctypes.c_float(0.1), A, None, 0, None)
            assert fn(*args) == UNSUPPORTED
        assert lib.mpgemm_kv_pack(A, A, A, A, A, A, 1, 0, 2, D, A, 1, 4, A, None) == UNSUPPORTED


def test_lowbit_workspace_covers_the_4bit_rewrite_at_large_m():
    lib = mp.lib()
    for bits in (2, 3):
        small = lib.mpgemm_workspace_bytes_lowbit(bits, 16, 4096, 4096, 128, 0)
        assert small == lib.mpgemm_workspace_bytes(16, 4096, 4096, 128, 0)
        big = lib.mpgemm_workspace_bytes_lowbit(bits, 2048, 4096, 4096, 128, 0)
        assert big >= 256 * 1024 + 4096 * 4096 // 2
        assert lib.mpgemm_workspace_bytes_lowbit(bits, 300, 40, 200, 128, 0) >= 256 * 1024 + 256 * 48 // 2
    assert lib.mpgemm_workspace_bytes_lowbit(4, 2048, 4096, 4096, 128, 0) == 0


# ------------------------------------------------------------ probes and the binding --

PROBE_HEADER = os.path.join(ROOT, "include", "mpgemm_probes.h")


def test_probe_library_exports_every_declared_function_and_validates():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mpgemm_\w+)\s*\(", text)))
    assert names == ["mpgemm_probe_hbm_read", "mpgemm_probe_mfma"]
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_quantized_mpgemm_amd",
                                   "libmpgemm_probes.so"))
    for name in names:
        assert hasattr(lib, name), name
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    read, mfma = lib.mpgemm_probe_hbm_read, lib.mpgemm_probe_mfma
    read.argtypes = [vp, sz, ctypes.c_int, ctypes.c_int, vp, vp]
    mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    assert read(None, 1024, 64, 8, vp(A), None) == INVALID
    assert read(vp(A), 1000, 64, 8, vp(A), None) == INVALID          # not a multiple of 16
    assert read(vp(A), 1024, 0, 8, vp(A), None) == INVALID
    assert read(vp(A), 1024, 64, 5, vp(A), None) == INVALID          # unroll not 4/8/16
    assert read(vp(MIS), 1024, 64, 8, vp(A), None) == ALIGN
    assert mfma(9, 10, 1, vp(A), None) == INVALID
    assert mfma(0, 0, 1, vp(A), None) == INVALID
    assert mfma(0, 10, 1, None, None) == INVALID


def test_workspace_cache_gives_each_stream_its_own_buffer():
    """Split-K calls racing on shared arrival counters is what this prevents: two streams
    of one device never share a workspace; one stream reuses its own."""
    import torch
    made = []

    def alloc(idx, n):
        made.append((idx, n))
        return torch.zeros(n, dtype=torch.uint8)

    cache = mp.WorkspaceCache(alloc)
    a = cache.get(0, 111, 4096)
    b = cache.get(0, 222, 4096)
    assert a is not b and a.data_ptr() != b.data_ptr()
    assert cache.get(0, 111, 100) is a
    assert cache.get(1, 111, 100) is not a                 # another device
    big = cache.get(0, 111, 8 << 20)
    assert big is not a and big.numel() >= 8 << 20
    assert cache.get(0, 111, 10) is big
    assert cache.get(0, 222, 10) is b
    assert cache.get(0, 111, 0) is None
    assert int(a.sum()) == 0 and int(big.sum()) == 0
    # under capture nothing is allocated: a stream without a workspace takes another
    # stream's of the same device, if one is large enough
    assert cache.get(0, 333, 10, capturing=True).numel() >= 10
    assert cache.get(1, 333, 100, capturing=True) is not None
    with pytest.raises(mp.MpgemmError):
        cache.get(0, 333, 64 << 20, capturing=True)
    with pytest.raises(mp.MpgemmError):
        cache.get(2, 333, 10, capturing=True)
    assert [i for i, _ in made] == [0, 0, 1, 0]
