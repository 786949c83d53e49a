"""GPU parity of the 8-bit-weight (W8A16) path through the C ABI, against the CPU oracle.

Bars as for 4-bit codes (test_gpu_parity):
  * packing, unpacking and dequantized weights: bit-exact;
  * GEMMs whose every partial sum is exact (identity / one-hot activations, small-integer
    activations with power-of-two scales): bit-exact;
  * random inputs: max|Y - Y_ref| / max|Y_ref| <= 5e-3, Y_ref from the oracle.
Every configuration that runs 8-bit codes is forced on the cases it can run: the small-M
kernel (ids 1..4) and the 32x32x16 tiled kernel in every tile shape (12, 13, 14).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, dev_half, dev_u8, host_bits, rel_err, say

pytestmark = pytest.mark.gpu

DECODE = (1, 2, 3, 4)
TILED = (12, 13, 14)


def configs_for(M):
    return [c for c in DECODE if M <= 16 * c] + list(TILED)


def pack8(case):
    z = None if case["zeros"] is None else dev_u8(case["zeros"])
    return mp.pack_weights_w8(dev_u8(case["codes"]), dev_half(case["scales"]), z, case["group"])


def run8(case, packed, config=0, rows=None, cols=None):
    y = mp.w8a16(dev_half(case["x"], case["dtype"]), packed, config=config)
    if rows is not None:
        y = y[torch.as_tensor(rows, device=y.device)][:, torch.as_tensor(cols, device=y.device)]
    torch.cuda.synchronize()
    return host_bits(y)


def ref8(case, rows=None, cols=None):
    x, codes, scales, zeros = case["x"], case["codes"], case["scales"], case["zeros"]
    if rows is not None:
        x, codes, scales = x[rows], codes[:, cols], scales[:, cols]
        zeros = None if zeros is None else zeros[:, cols]
    return oracle.w8a16(x, codes, scales, zeros, case["group"], case["dtype"], threads=8)


# ---------------------------------------------------------------- packing ------------

@pytest.mark.parametrize("K,N,g,sym", [(256, 272, 128, False), (512, 64, 64, True),
                                       (4096, 1024, 128, False), (1024, 528, 64, False)])
def test_w8_pack_bytes_match_oracle_and_unpack_round_trips(K, N, g, sym):
    say(f"w8 pack K={K} N={N} g={g} sym={sym}")
    codes, scales, zeros = workloads.weights_w8(K, N, g, sym, 0.005, 0.02, K + N)
    case = dict(codes=codes, scales=scales, zeros=zeros, group=g)
    packed = pack8(case)
    assert packed.bits == 8 and packed.codes.numel() == K * N
    pc, pm = oracle.pack_w8(codes, scales, zeros, g)
    assert np.array_equal(packed.codes.cpu().numpy(), pc)
    assert np.array_equal(packed.meta.cpu().numpy(), pm)
    c2, s2, z2 = mp.unpack(packed)
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)
    if not sym:
        assert np.array_equal(z2.cpu().numpy(), zeros)


def test_w8_weights_are_not_accepted_by_the_4bit_gemm():
    codes, scales, zeros = workloads.weights_w8(256, 64, 128, False, 0.005, 0.02, 1)
    packed = pack8(dict(codes=codes, scales=scales, zeros=zeros, group=128))
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        mp.w4a16(x, packed)


# -------------------------------------------------------------- bit-exact cases --------

@pytest.mark.parametrize("config", TILED)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_w8_identity_activations_give_dequantized_weights_bit_exact(dtype, g, sym, config):
    K, N = 256, 272
    say(f"w8 identity dtype={dtype} g={g} sym={sym} config={config}")
    codes, scales, zeros = workloads.weights_w8(K, N, g, sym, 0.005, 0.02, 31)
    one = 0x3C00 if dtype == "f16" else 0x3F80
    eye = (np.eye(K, dtype=np.uint16) * one).astype(np.uint16)
    case = dict(x=eye, codes=codes, scales=scales, zeros=zeros, group=g, dtype=dtype)
    w = oracle.dequant_w8(codes, scales, zeros, g, dtype)
    assert np.array_equal(run8(case, pack8(case), config), w)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("config", DECODE)
def test_w8_one_hot_rows_give_weight_rows_bit_exact(dtype, config):
    K, N, g = 1024, 64, 128
    M = 16 * config - 3
    say(f"w8 one-hot dtype={dtype} config={config} M={M}")
    codes, scales, zeros = workloads.weights_w8(K, N, g, False, 0.005, 0.02, 32)
    picks = np.random.default_rng(33).choice(K, M, replace=False)
    one = 0x3C00 if dtype == "f16" else 0x3F80
    x = np.zeros((M, K), dtype=np.uint16)
    x[np.arange(M), picks] = one
    case = dict(x=x, codes=codes, scales=scales, zeros=zeros, group=g, dtype=dtype)
    w = oracle.dequant_w8(codes, scales, zeros, g, dtype)
    assert np.array_equal(run8(case, pack8(case), config), w[picks])


@pytest.mark.parametrize("M", [1, 16, 64, 200])
@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_w8_integer_activations_power_of_two_scales_bit_exact(M, g, sym):
    """X in {-1,0,1}, s = 2^-8: every partial sum is exact in fp32, so Y is unique."""
    K, N = 1024, 96
    rng = np.random.default_rng(M + g)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    zeros = None if sym else rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -8, dtype=np.float16).view(np.uint16)
    case = dict(x=x, codes=codes, scales=scales, zeros=zeros, group=g, dtype="f16")
    packed = pack8(case)
    ref = oracle.w8a16(x, codes, scales, zeros, g)
    for cfg in [0] + configs_for(M):
        say(f"w8 integer M={M} g={g} sym={sym} config={cfg}")
        assert np.array_equal(run8(case, packed, cfg), ref), cfg


# ------------------------------------------------------------------ random inputs ------

@pytest.mark.parametrize("M", [1, 5, 16, 37, 64, 128, 300])
@pytest.mark.parametrize("wl", [workloads.LLAMA3_8B_DECODE, workloads.LLAMA3_70B,
                                workloads.QWEN3_32B], ids=lambda w: w.name)
def test_w8_random_all_configs(M, wl):
    K, N = 768, 272                         # ragged last tiles along N for both tile shapes
    case = workloads.make_case_w8(wl, M, K, N)
    packed = pack8(case)
    ref = ref8(case)
    for cfg in configs_for(M):
        say(f"w8 random {wl.name} M={M} config={cfg}")
        assert rel_err(run8(case, packed, cfg), ref, case["dtype"]) <= REL_TOL, cfg


@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("K,N,label", workloads.LLAMA3_8B_SHAPES)
def test_w8_llama3_8b_full_shapes(M, K, N, label):
    case = workloads.make_case_w8(workloads.LLAMA3_8B_DECODE, M, K, N)
    packed = pack8(case)
    rng = np.random.default_rng(case["seed"])
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 12), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 192, replace=False)]))
    ref = ref8(case, rows, cols)
    cfgs = [0] + ([12, 13, 14] if M > 64 else [])
    for cfg in cfgs:
        say(f"w8 8B M={M} K={K} N={N} config={cfg}")
        assert rel_err(run8(case, packed, cfg, rows, cols), ref, "f16") <= REL_TOL, cfg


# --------------------------------------------------------------------- edge cases ------

@pytest.mark.parametrize("M", [65, 200])
def test_w8_k_a_multiple_of_128_not_256_runs_every_tiled_config(M):
    K, N = 384, 64                         # three 128-deep tiles: the two-stage loop tail
    codes, scales, zeros = workloads.weights_w8(K, N, 128, False, 0.005, 0.02, 3)
    case = dict(x=workloads.activations(M, K, "f16", 4), codes=codes, scales=scales,
                zeros=zeros, group=128, dtype="f16")
    packed = pack8(case)
    want = ref8(case)
    for cfg in (0, 12, 13, 14):
        say(f"w8 K=384 M={M} config={cfg}")
        assert rel_err(run8(case, packed, cfg), want, "f16") <= REL_TOL, cfg


def test_w8_repeated_runs_are_bitwise_identical():
    for M in (16, 256):
        case = workloads.make_case_w8(workloads.LLAMA3_8B_DECODE, M, 4096, 4096)
        packed = pack8(case)
        assert np.array_equal(run8(case, packed), run8(case, packed))
