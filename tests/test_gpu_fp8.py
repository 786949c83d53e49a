"""GPU parity of the FP8-weight path (OCP E4M3 / E5M2 codes times an fp16 group scale)
through the C ABI, against the CPU oracle.

Bars as for integer codes (test_gpu_parity):
  * packing and unpacking: bit-exact (FP8 codes are bytes in the 8-bit layout);
  * dequantized weights (identity activations, one-hot rows): bit-exact, over every finite
    code of each format;
  * GEMMs whose every partial sum is exact (small-integer weights, s = 2^-6, X in
    {-1,0,1}): bit-exact;
  * random inputs: max|Y - Y_ref| / max|Y_ref| <= 5e-3, Y_ref from the oracle;
  * NaN and infinite codes: the columns they reach are NaN / infinite on both sides.
Every configuration that runs FP8 codes is forced on the cases it can run: the small-M
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
FORMATS = ("e4m3", "e5m2")
ALL = np.arange(256, dtype=np.uint8)
FINITE = {"e4m3": ALL[(ALL & 0x7F) != 0x7F], "e5m2": ALL[(ALL & 0x7C) != 0x7C]}
ONE = {"f16": 0x3C00, "bf16": 0x3F80}


def configs_for(M):
    return [c for c in DECODE if M <= 16 * c] + list(TILED)


def pack(case):
    return mp.pack_weights_fp8(dev_u8(case["codes"]), dev_half(case["scales"]), case["group"],
                               case["fmt"])


def run(case, packed, config=0, rows=None, cols=None):
    y = mp.wfp8a16(dev_half(case["x"], case["dtype"]), packed, config=config)
    if rows is not None:
        y = y[torch.as_tensor(rows, device=y.device)][:, torch.as_tensor(cols, device=y.device)]
    torch.cuda.synchronize()
    return host_bits(y)


def ref(case, rows=None, cols=None):
    x, codes, scales = case["x"], case["codes"], case["scales"]
    if rows is not None:
        x, codes, scales = x[rows], codes[:, cols], scales[:, cols]
    return oracle.wfp8a16(x, codes, scales, case["group"], case["fmt"], case["dtype"], threads=8)


def every_code(fmt, K, N, seed):
    """Codes that walk every finite code of the format, in a seeded order."""
    fin = FINITE[fmt]
    rng = np.random.default_rng(seed)
    flat = np.concatenate([rng.permutation(fin) for _ in range(-(-K * N // fin.size))])
    return flat[:K * N].reshape(K, N).astype(np.uint8)


def scales_for(K, N, g, seed, lo=1e-3, hi=0.05):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, (K // g, N)).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- packing ------------

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("K,N,g", [(256, 272, 128), (512, 64, 64), (4096, 1024, 128)])
def test_fp8_pack_bytes_match_oracle_and_unpack_round_trips(fmt, K, N, g):
    say(f"fp8 pack {fmt} K={K} N={N} g={g}")
    codes, scales = workloads.weights_fp8(K, N, g, fmt, 0.005, 0.02, K + N)
    packed = pack(dict(codes=codes, scales=scales, group=g, fmt=fmt))
    assert packed.bits == 8 and packed.fp8 == fmt and packed.symmetric
    pc, pm = oracle.pack_w8(codes, scales, None, g)
    assert np.array_equal(packed.codes.cpu().numpy(), pc)
    assert np.array_equal(packed.meta.cpu().numpy(), pm)
    c2, s2, z2 = mp.unpack(packed)
    assert z2 is None
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)


def test_fp8_torch_float8_tensor_sets_the_format():
    codes = torch.randn(256, 32).to(torch.float8_e5m2).cuda()
    scales = torch.full((2, 32), 0.01, dtype=torch.float16, device="cuda")
    assert mp.pack_weights_fp8(codes, scales, 128).fp8 == "e5m2"


def test_fp8_and_integer_weights_are_not_interchangeable():
    codes, scales = workloads.weights_fp8(256, 64, 128, "e4m3", 0.005, 0.02, 1)
    packed = pack(dict(codes=codes, scales=scales, group=128, fmt="e4m3"))
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        mp.w8a16(x, packed)
    c8, s8, z8 = workloads.weights_w8(256, 64, 128, True, 0.005, 0.02, 1)
    p8 = mp.pack_weights_w8(dev_u8(c8), dev_half(s8), None, 128)
    with pytest.raises(ValueError):
        mp.wfp8a16(x, p8)


# -------------------------------------------------------------- bit-exact cases --------

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("config", TILED)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("g", [128, 64])
def test_fp8_identity_activations_give_dequantized_weights_bit_exact(fmt, dtype, g, config):
    K, N = 256, 272
    say(f"fp8 identity {fmt} dtype={dtype} g={g} config={config}")
    codes = every_code(fmt, K, N, 31 + g)
    scales = scales_for(K, N, g, 32 + g)
    eye = (np.eye(K, dtype=np.uint16) * ONE[dtype]).astype(np.uint16)
    case = dict(x=eye, codes=codes, scales=scales, group=g, fmt=fmt, dtype=dtype)
    # Y = W except for signed zeros: a -0 weight (code 0x80, or a product that rounds to
    # -0) summed with the +0 terms of the other rows is +0, in the oracle's GEMM as here.
    want = oracle.wfp8a16(eye, codes, scales, g, fmt, dtype, threads=8)
    w = oracle.dequant_fp8(codes, scales, g, fmt, dtype)
    assert np.all((want == w) | ((w == 0x8000) & (want == 0)))
    assert np.array_equal(run(case, pack(case), config), want)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("config", DECODE)
def test_fp8_one_hot_rows_give_weight_rows_bit_exact(fmt, dtype, config):
    K, N, g = 1024, 64, 128
    M = 16 * config - 3
    say(f"fp8 one-hot {fmt} dtype={dtype} config={config} M={M}")
    codes = every_code(fmt, K, N, 40 + config)
    scales = scales_for(K, N, g, 41)
    picks = np.random.default_rng(42).choice(K, M, replace=False)
    x = np.zeros((M, K), dtype=np.uint16)
    x[np.arange(M), picks] = ONE[dtype]
    case = dict(x=x, codes=codes, scales=scales, group=g, fmt=fmt, dtype=dtype)
    want = oracle.wfp8a16(x, codes, scales, g, fmt, dtype, threads=8)   # w[picks] but for -0
    assert np.array_equal(run(case, pack(case), config), want)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 16, 64, 200])
@pytest.mark.parametrize("g", [128, 64])
def test_fp8_integer_weights_power_of_two_scales_bit_exact(fmt, M, g):
    """Weights are small integers (exact in the format) times 2^-6, X in {-1,0,1}: every
    partial sum is exact in fp32, so Y is unique."""
    K, N = 1024, 96
    rng = np.random.default_rng(M + g)
    lim = 16 if fmt == "e4m3" else 8
    ints = rng.integers(-lim, lim + 1, (K, N)).astype(np.float32)
    codes = workloads.to_fp8_bits(ints, fmt)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    scales = np.full((K // g, N), 2.0 ** -6, dtype=np.float16).view(np.uint16)
    case = dict(x=x, codes=codes, scales=scales, group=g, fmt=fmt, dtype="f16")
    packed = pack(case)
    want = oracle.wfp8a16(x, codes, scales, g, fmt)
    for cfg in [0] + configs_for(M):
        say(f"fp8 integer {fmt} M={M} g={g} config={cfg}")
        assert np.array_equal(run(case, packed, cfg), want), cfg


# ------------------------------------------------------------------ random inputs ------

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 5, 16, 37, 64, 128, 300])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_random_all_configs(fmt, M, dtype):
    K, N = 768, 272                         # ragged last tiles along N for both tile shapes
    wl = workloads.QWEN3_8B_FP8
    case = workloads.make_case_fp8(wl, M, K, N, fmt)
    case["x"] = workloads.activations(M, K, dtype, case["seed"] + 1)
    case["dtype"] = dtype
    packed = pack(case)
    want = ref(case)
    for cfg in configs_for(M):
        say(f"fp8 random {fmt} {dtype} M={M} config={cfg}")
        assert rel_err(run(case, packed, cfg), want, dtype) <= REL_TOL, cfg


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("K,N,label", workloads.QWEN3_8B_SHAPES)
def test_fp8_qwen3_8b_full_shapes(fmt, M, K, N, label):
    case = workloads.make_case_fp8(workloads.QWEN3_8B_FP8, M, K, N, fmt)
    packed = pack(case)
    rng = np.random.default_rng(case["seed"])
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 12), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 192, replace=False)]))
    want = ref(case, rows, cols)
    cfgs = [0] + ([12, 13, 14] if M > 64 else [])
    for cfg in cfgs:
        say(f"fp8 qwen3-8b {fmt} M={M} K={K} N={N} config={cfg}")
        assert rel_err(run(case, packed, cfg, rows, cols), want, "bf16") <= REL_TOL, cfg


# --------------------------------------------------------------------- edge cases ------

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [4, 128])
def test_fp8_nan_and_infinite_codes_reach_their_columns(fmt, M):
    K, N, g = 256, 64, 128
    codes = every_code(fmt, K, N, 7)
    bad = {3: 0x7F if fmt == "e4m3" else 0x7E}          # NaN
    if fmt == "e5m2":
        bad[40] = 0x7C                                  # +infinity
    for col, code in bad.items():
        codes[17, col] = code
    scales = scales_for(K, N, g, 8)
    x = np.abs(np.random.default_rng(9).standard_normal((M, K))).astype(np.float16) \
        .view(np.uint16)                                # positive: +inf stays +inf
    case = dict(x=x, codes=codes, scales=scales, group=g, fmt=fmt, dtype="f16")
    for cfg in [0] + configs_for(M):
        say(f"fp8 nan/inf {fmt} M={M} config={cfg}")
        y = oracle.f16_bits_to_f64(run(case, pack(case), cfg))
        want = oracle.f16_bits_to_f64(ref(case))
        assert np.isnan(y[:, 3]).all() and np.isnan(want[:, 3]).all()
        if fmt == "e5m2":
            assert (y[:, 40] == np.inf).all() and (want[:, 40] == np.inf).all()
        good = [c for c in range(N) if c not in bad]
        assert np.isfinite(y[:, good]).all()
        assert rel_err(host_bits_of(y[:, good]), host_bits_of(want[:, good]), "f16") <= REL_TOL


def host_bits_of(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("M", [65, 200])
def test_fp8_k_a_multiple_of_128_not_256_runs_every_tiled_config(M):
    K, N = 384, 64                         # three 128-deep tiles: the two-stage loop tail
    case = workloads.make_case_fp8(workloads.QWEN3_8B_FP8, M, K, N, "e4m3")
    packed = pack(case)
    want = ref(case)
    for cfg in (0, 12, 13, 14):
        say(f"fp8 K=384 M={M} config={cfg}")
        assert rel_err(run(case, packed, cfg), want, "bf16") <= REL_TOL, cfg


def test_fp8_repeated_runs_are_bitwise_identical():
    for M in (16, 256):
        case = workloads.make_case_fp8(workloads.QWEN3_8B_FP8, M, 4096, 4096)
        packed = pack(case)
        assert np.array_equal(run(case, packed), run(case, packed))
