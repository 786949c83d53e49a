"""GPU parity of the 32x32x16 tiled kernels when they split the K range of their tiles
(fewer tiles than compute units; P = 2, 4 or 8 parts per tile, fp32 partials in the
workspace, added in split order by a second kernel).

Bars as for every GEMM: max|Y - Y_ref| / max|Y_ref| <= 5e-3 against the oracle, bit-exact
where every partial sum is exact; in addition the split path is deterministic, leaves the
workspace's arrival counters zero, and without a workspace the kernels run every tile
whole (the same bits as with the split turned off).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, dev_half, dev_u8, host_bits, oracle_sample, pack_case, rel_err, say

pytestmark = pytest.mark.gpu

X32, X32_TALL, X32_WIDE = 12, 13, 14
TILE = {X32: (128, 256), X32_TALL: (256, 128), X32_WIDE: (256, 256)}
COUNTER_BYTES = 256 * 1024


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def parts(M, N, K, config):
    """The split rule: fewer tiles than CUs split P ways when P tiles <= CUs, parts keep
    whole 256-deep stage blocks and at least 1024 of K, and K needs no padding."""
    bm, bn = TILE[config]
    Np, Kp = -(-N // 16) * 16, -(-K // 128) * 128
    loop = -(-Kp // 256) * 256
    tiles = -(-M // bm) * -(-Np // bn)
    r = tiles
    if K != loop or tiles >= cus():
        return 1
    for p in (8, 4, 2):
        if r * p <= cus() and loop % (256 * p) == 0 and loop // p >= 1024:
            return p
    return 1


def run(case, packed, config, env=None, monkeypatch=None):
    if env is not None:
        monkeypatch.setenv("MPGEMM_X32_SPLIT", env)
    y = mp.w4a16(dev_half(case["x"], case["dtype"]), packed, config=config)
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("M,K,N,config,P", [(130, 2048, 256, X32, 2), (130, 4096, 256, X32, 4),
                                            (130, 4096, 256, X32_TALL, 4),
                                            (130, 4096, 256, X32_WIDE, 4),
                                            (300, 8192, 512, X32_WIDE, 8),
                                            (300, 8192, 256, X32_TALL, 8),
                                            (200, 8192, 512, X32, 8)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_tiles_match_oracle(M, K, N, config, P, dtype, monkeypatch):
    assert parts(M, N, K, config) == P
    wl = workloads.LLAMA3_8B_DECODE if dtype == "f16" else workloads.QWEN3_32B
    case = workloads.make_case(wl, M, K, N)
    case["x"] = workloads.activations(M, K, dtype, case["seed"] + 1)
    case["dtype"] = dtype
    packed = pack_case(case)
    want = oracle.w4a16(case["x"], case["codes"], case["scales"], case["zeros"], case["group"],
                        dtype, threads=8)
    say(f"x32 split M={M} K={K} N={N} config={config} P={P} {dtype}")
    y = run(case, packed, config)
    assert rel_err(y, want, dtype) <= REL_TOL
    assert np.array_equal(run(case, packed, config), y)            # deterministic
    y0 = run(case, packed, config, "0", monkeypatch)                 # split turned off
    assert rel_err(y0, want, dtype) <= REL_TOL


@pytest.mark.parametrize("config", [X32, X32_TALL, X32_WIDE])
def test_split_exact_sums_bit_exact(config):
    """X in {-1, 0, 1}, s = 2^-8: every partial sum is exact in fp32 whatever the split."""
    M, K, N, g = 130, 4096, 256, 128
    assert parts(M, N, K, config) == 4
    rng = np.random.default_rng(config)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -8, dtype=np.float16).view(np.uint16)
    case = dict(x=x, codes=codes, scales=scales, zeros=zeros, group=g, dtype="f16")
    assert np.array_equal(run(case, pack_case(case), config), oracle.w4a16(x, codes, scales, zeros, g))


def test_split_8bit_and_fp8_codes():
    M, K, N = 130, 4096, 256
    assert parts(M, N, K, X32) == 4
    c8 = workloads.make_case_w8(workloads.LLAMA3_8B_DECODE, M, K, N)
    z = None if c8["zeros"] is None else dev_u8(c8["zeros"])
    p8 = mp.pack_weights_w8(dev_u8(c8["codes"]), dev_half(c8["scales"]), z, c8["group"])
    y8 = host_bits(mp.w8a16(dev_half(c8["x"], c8["dtype"]), p8, config=X32))
    want8 = oracle.w8a16(c8["x"], c8["codes"], c8["scales"], c8["zeros"], c8["group"], c8["dtype"],
                         threads=8)
    assert rel_err(y8, want8, c8["dtype"]) <= REL_TOL
    cf = workloads.make_case_fp8(workloads.QWEN3_8B_FP8, M, K, N, "e4m3")
    pf = mp.pack_weights_fp8(dev_u8(cf["codes"]), dev_half(cf["scales"]), cf["group"], "e4m3")
    yf = host_bits(mp.wfp8a16(dev_half(cf["x"], cf["dtype"]), pf, config=X32))
    wantf = oracle.wfp8a16(cf["x"], cf["codes"], cf["scales"], cf["group"], "e4m3", cf["dtype"],
                           threads=8)
    assert rel_err(yf, wantf, cf["dtype"]) <= REL_TOL


def test_llama3_8b_prefill_512_rows_splits_in_two():
    """512 x 4096 x 6144 on the 128 x 256 tile: 96 tiles, each split in two."""
    M, K, N = 512, 4096, 6144
    if cus() == 256:
        assert parts(M, N, K, X32) == 2
    case = workloads.make_case(workloads.LLAMA3_8B_DECODE, M, K, N)
    packed = pack_case(case)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 24, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 256, replace=False)]))
    y = mp.w4a16(dev_half(case["x"]), packed, config=X32)
    y = y[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
    torch.cuda.synchronize()
    assert rel_err(host_bits(y.contiguous()), oracle_sample(case, rows, cols), "f16") <= REL_TOL


def test_split_leaves_counters_zero_and_runs_whole_tiles_without_workspace(monkeypatch):
    M, K, N = 130, 4096, 256
    case = workloads.make_case(workloads.LLAMA3_8B_DECODE, M, K, N)
    packed = pack_case(case)
    need = int(mp.lib().mpgemm_workspace_bytes(M, N, K, 128, 0))
    assert need >= COUNTER_BYTES + 4 * 128 * 256 * 4
    ws = mp.workspace_for(torch.device("cuda"), need)
    for config in (X32, X32_TALL):
        run(case, packed, config)
        assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    x = dev_half(case["x"])
    for config in (X32, X32_TALL):
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        st = mp.lib().mpgemm_w4a16_config(x.data_ptr(), 0, packed.codes.data_ptr(),
                                          packed.meta.data_ptr(), M, N, K, packed.group,
                                          int(packed.symmetric), y.data_ptr(), None, 0, config,
                                          None)
        assert st == 0
        torch.cuda.synchronize()
        whole = run(case, packed, config, "0", monkeypatch)
        monkeypatch.delenv("MPGEMM_X32_SPLIT")
        assert np.array_equal(host_bits(y), whole)


def test_wide_tile_splits_only_with_room_for_its_partials(monkeypatch):
    """2048 x 14336 x 4096 on the 256 x 256 tile: 128 tiles, split in two only when the
    workspace holds 256 partials of 256 KiB; the default workspace (sized for the other
    tiles, which run whole here) gives the unsplit result bit for bit, and a larger one the
    split, both against the oracle on sampled outputs."""
    M, K, N = 2048, 14336, 4096
    if cus() == 256:
        assert parts(M, N, K, X32_WIDE) == 2
    need = COUNTER_BYTES + 128 * 2 * 256 * 256 * 4
    assert int(mp.lib().mpgemm_workspace_bytes(M, N, K, 128, 0)) < need
    case = workloads.make_case(workloads.LLAMA3_8B_DECODE, M, K, N)
    packed = pack_case(case)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 12, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 256, replace=False)]))
    want = oracle_sample(case, rows, cols)
    r_t, c_t = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    x = dev_half(case["x"])
    say("wide tile: default workspace, then a larger one, then the split turned off")
    y_def = mp.w4a16(x, packed, config=X32_WIDE)
    big = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y_split = mp.w4a16(x, packed, config=X32_WIDE, workspace=big)
    torch.cuda.synchronize()
    assert int(big[:COUNTER_BYTES].count_nonzero()) == 0
    monkeypatch.setenv("MPGEMM_X32_SPLIT", "0")
    y_whole = mp.w4a16(x, packed, config=X32_WIDE)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_def), host_bits(y_whole))
    for y in (y_def, y_split):
        got = host_bits(y[r_t][:, c_t].contiguous())
        assert rel_err(got, want, "f16") <= REL_TOL
    assert not np.array_equal(host_bits(y_split), host_bits(y_whole))   # it did split
