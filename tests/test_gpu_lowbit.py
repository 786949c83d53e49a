"""GPU parity of the 2-bit and 3-bit weight path through the C ABI, against the CPU oracle.

  * packing, unpacking: bit-exact (aligned and ragged shapes);
  * one-hot activation rows give dequantized weight rows bit-exact, in every small-M
    configuration (1..4), both activation formats, both group sizes;
  * small-integer activations with power-of-two scales: bit-exact, including M > 64 (the
    64-row chunks);
  * random inputs: max|Y - Y_ref| / max|Y_ref| <= 5e-3, Y_ref from the oracle, at the
    Llama-3-8B shapes too (sampled outputs).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, dev_half, dev_u8, host_bits, rel_err, say

pytestmark = pytest.mark.gpu

BITS = (2, 3)
ONE = {"f16": 0x3C00, "bf16": 0x3F80}


def configs_for(M):
    """Every configuration that runs M rows: the small-M kernel ids, and for M > 64 the two
    32x32x16 tiled ids (on the codes rewritten in the 4-bit layout)."""
    return [0] + [c for c in (1, 2, 3, 4) if M <= 16 * c] + ([12, 13, 14] if M > 64 else [])


def make(bits, K, N, g, sym, seed, lo=0.005, hi=0.05):
    rng = np.random.default_rng(seed)
    rows = -(-K // g)
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    zeros = None if sym else rng.integers(0, 1 << bits, (rows, N), dtype=np.uint8)
    scales = rng.uniform(lo, hi, (rows, N)).astype(np.float16).view(np.uint16)
    return codes, scales, zeros


def pack(bits, codes, scales, zeros, g):
    return mp.pack_weights_lowbit(bits, dev_u8(codes), dev_half(scales),
                                  None if zeros is None else dev_u8(zeros), g)


def run(x, packed, dtype, cfg=0):
    y = mp.wlowbit_a16(dev_half(x, dtype), packed, config=cfg)
    torch.cuda.synchronize()
    return host_bits(y)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N,g,sym", [(256, 272, 128, False), (512, 64, 64, True),
                                       (4096, 1024, 128, False), (200, 40, 64, False),
                                       (136, 7, 128, True)])
def test_lowbit_pack_bytes_match_oracle_and_unpack_round_trips(bits, K, N, g, sym):
    say(f"w{bits} pack K={K} N={N} g={g} sym={sym}")
    codes, scales, zeros = make(bits, K, N, g, sym, K + N + bits)
    packed = pack(bits, codes, scales, zeros, g)
    pc, pm = oracle.pack_lowbit(bits, codes, scales, zeros, g)
    assert np.array_equal(packed.codes.cpu().numpy(), pc)
    assert np.array_equal(packed.meta.cpu().numpy(), pm)
    c2, s2, z2 = mp.unpack(packed)
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)
    if not sym:
        assert np.array_equal(z2.cpu().numpy(), zeros)


def test_lowbit_weights_are_not_accepted_by_the_other_gemms():
    codes, scales, zeros = make(2, 256, 64, 128, False, 1)
    packed = pack(2, codes, scales, zeros, 128)
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        mp.w4a16(x, packed)
    with pytest.raises(mp.MpgemmError):
        mp.wlowbit_a16(torch.zeros((128, 256), dtype=torch.float16, device="cuda"), packed,
                       config=7)                     # no such configuration


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("config", (1, 2, 3, 4))
@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_lowbit_one_hot_rows_give_weight_rows_bit_exact(bits, dtype, config, g, sym):
    K, N = 1024, 64
    M = 16 * config - 3
    say(f"w{bits} one-hot dtype={dtype} config={config} g={g} sym={sym}")
    codes, scales, zeros = make(bits, K, N, g, sym, 30 + config + bits)
    picks = np.random.default_rng(33).choice(K, M, replace=False)
    x = np.zeros((M, K), dtype=np.uint16)
    x[np.arange(M), picks] = ONE[dtype]
    w = oracle.dequant_lowbit(bits, codes, scales, zeros, g, dtype)
    assert np.array_equal(run(x, pack(bits, codes, scales, zeros, g), dtype, config), w[picks])


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [1, 16, 64, 200])
@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_lowbit_integer_activations_power_of_two_scales_bit_exact(bits, M, g, sym):
    K, N = 1024, 96
    rng = np.random.default_rng(M + g + bits)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    codes, _, zeros = make(bits, K, N, g, sym, M + bits)
    scales = np.full((K // g, N), 2.0 ** -6, dtype=np.float16).view(np.uint16)
    packed = pack(bits, codes, scales, zeros, g)
    want = oracle.wlowbit_a16(bits, x, codes, scales, zeros, g)
    for cfg in configs_for(M):
        say(f"w{bits} integer M={M} g={g} sym={sym} config={cfg}")
        assert np.array_equal(run(x, packed, "f16", cfg), want), cfg


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [1, 5, 16, 37, 64, 130, 300])
@pytest.mark.parametrize("wl", [workloads.LLAMA3_8B_DECODE, workloads.LLAMA3_70B,
                                workloads.QWEN3_32B], ids=lambda w: w.name)
def test_lowbit_random_all_configs(bits, M, wl):
    K, N = 768, 272
    codes, scales, zeros = make(bits, K, N, wl.group, wl.symmetric, M * 7 + bits)
    x = workloads.activations(M, K, wl.dtype, M + bits)
    packed = pack(bits, codes, scales, zeros, wl.group)
    want = oracle.wlowbit_a16(bits, x, codes, scales, zeros, wl.group, wl.dtype, threads=8)
    for cfg in configs_for(M):
        say(f"w{bits} random {wl.name} M={M} config={cfg}")
        assert rel_err(run(x, packed, wl.dtype, cfg), want, wl.dtype) <= REL_TOL, cfg


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N", [(200, 40), (1000, 33), (4104, 100)])
@pytest.mark.parametrize("M", [3, 70])
def test_lowbit_ragged_shapes(bits, K, N, M):
    g = 64
    codes, scales, zeros = make(bits, K, N, g, False, K + N + M)
    x = workloads.activations(M, K, "bf16", K)
    packed = pack(bits, codes, scales, zeros, g)
    want = oracle.wlowbit_a16(bits, x, codes, scales, zeros, g, "bf16", threads=8)
    for cfg in configs_for(M):
        say(f"w{bits} ragged K={K} N={N} M={M} config={cfg}")
        assert rel_err(run(x, packed, "bf16", cfg), want, "bf16") <= REL_TOL, cfg


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("K,N,label", workloads.LLAMA3_8B_SHAPES)
def test_lowbit_llama3_8b_full_shapes(bits, M, K, N, label):
    codes, scales, zeros = make(bits, K, N, 128, False, K + N + M + bits)
    x = workloads.activations(M, K, "f16", K + M)
    packed = pack(bits, codes, scales, zeros, 128)
    rng = np.random.default_rng(K + N)
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 192, replace=False)]))
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 12), replace=False)]))
    want = oracle.wlowbit_a16(bits, x[rows], codes[:, cols], scales[:, cols], zeros[:, cols], 128,
                              threads=8)
    for cfg in [0] + ([12, 13] if M > 64 else []):
        say(f"w{bits} 8B M={M} K={K} N={N} config={cfg}")
        y = run(x, packed, "f16", cfg)
        assert rel_err(y[rows][:, cols], want, "f16") <= REL_TOL, cfg


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("sym", [False, True])
def test_lowbit_large_m_equals_the_4bit_gemm_of_the_same_codes_bit_for_bit(bits, sym):
    """b-bit codes are valid 4-bit codes (symmetric ones shifted onto the 4-bit zero 8): the
    tiled path must give the 4-bit GEMM's bits on the same weights."""
    M, K, N, g = 300, 1024, 272, 128
    codes, scales, zeros = make(bits, K, N, g, sym, 7 + bits)
    x = workloads.activations(M, K, "f16", 8)
    packed = pack(bits, codes, scales, zeros, g)
    shift = 8 - (1 << (bits - 1)) if sym else 0
    p4 = mp.pack_weights(dev_u8(codes + shift), dev_half(scales),
                         None if zeros is None else dev_u8(zeros), g)
    for cfg in (0, 12, 13, 14):
        y = run(x, packed, "f16", cfg)
        y4 = host_bits(mp.w4a16(dev_half(x), p4, config=cfg if cfg else 12 if M < 512 else 13))
        say(f"w{bits} vs w4 sym={sym} config={cfg}")
        assert np.array_equal(y, y4), cfg
