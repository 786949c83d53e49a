"""Pins for the CPU oracle: each test checks it against something other than itself.

Pins used (none re-types the oracle's code):
  * number formats  -- numpy's float16 and torch's bfloat16 conversions (library routines),
                       exhaustively for decode and on ties/boundaries for encode;
  * dequantization  -- closed form at power-of-two scales, sign/zero/antisymmetry
                       invariants, group/column locality, symmetric == zero 8, and exact
                       rational products rounded by Python's own binary16 packer;
  * GEMM            -- exact rational brute force (fractions) rounded once, identity and
                       one-hot activations, an integer special case against numpy int64
                       matmul, column locality;
  * packing         -- round trip, a bijection on nibble positions, the pages' nibble order
                       (tests/golden/nibble_order.txt), and the MFMA-operand view of every
                       packed word (after "isolate & shift" each 32-bit register holds the
                       (k, k+1) pair that the gfx950 16x16x32 operand lane expects).
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def py_f16_bits(x: float) -> int:
    """Python's own IEEE binary16 packer (round to nearest even)."""
    return struct.unpack("<H", struct.pack("<e", x))[0]


def exact_f16(bits) -> Fraction:
    return Fraction(float(np.uint16(bits).view(np.float16)))


# ------------------------------------------------------------------ number formats --

def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy_random_ties_and_boundaries():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000)]
    # exact midpoints between consecutive finite fp16 values (ties), both signs
    fin = np.arange(0, 0x7bff, 37, dtype=np.uint16)
    lo = fin.view(np.float16).astype(np.float64)
    hi = (fin + 1).view(np.float16).astype(np.float64)
    vals.append((lo + hi) / 2)
    vals.append(-(lo + hi) / 2)
    vals.append(np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2.0 ** -24,
                          2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * 0.999,
                          np.inf, -np.inf]))
    x = np.concatenate(vals)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16_bits(x), ref)
    assert int(oracle.f64_to_f16_bits([np.nan])[0]) & 0x7fff > 0x7c00


def test_bf16_decode_all_patterns_match_torch():
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_matches_torch_on_float32_values():
    import torch
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    # ties: float32 values exactly half way between consecutive bf16 values
    b = np.arange(0, 0x7f7f, 101, dtype=np.uint32)
    ties = ((b << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x32 = np.concatenate([x32, ties, -ties, np.array([0.0, 3.0e38, 3.4e38, 1e-40],
                                                     dtype=np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(x32.astype(np.float64)), ref)


# ------------------------------------------------------------------ dequantization --

def _all_qz(group=128):
    """16x16 grid of (q, z) laid out over one group: K = group, N = 256 columns."""
    q = np.arange(16, dtype=np.uint8)
    z = np.arange(16, dtype=np.uint8)
    qq, zz = np.meshgrid(q, z, indexing="ij")
    codes = np.tile(qq.reshape(1, 256), (group, 1))
    zeros = zz.reshape(1, 256).copy()
    return codes, zeros, qq.ravel().astype(int), zz.ravel().astype(int)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_power_of_two_scale_is_exact_closed_form(dtype):
    codes, zeros, q, z = _all_qz()
    for e in (-2, -6, -10):
        s = np.full((1, 256), 2.0 ** e, dtype=np.float16).view(np.uint16)
        w = oracle.dequant(codes, s, zeros, 128, dtype)
        val = oracle.f16_bits_to_f64(w[0]) if dtype == "f16" else oracle.bf16_bits_to_f64(w[0])
        assert np.array_equal(val, (q - z) * 2.0 ** e)


def test_dequant_sign_zero_and_antisymmetry():
    codes, zeros, q, z = _all_qz()
    rng = np.random.default_rng(3)
    s = np.full((1, 256), rng.uniform(0.005, 0.02), dtype=np.float16).view(np.uint16)
    val = oracle.f16_bits_to_f64(oracle.dequant(codes, s, zeros, 128)[0])
    assert np.array_equal(val == 0, q == z)
    assert np.array_equal(np.sign(val), np.sign(q - z))
    grid = val.reshape(16, 16)       # [q][z]
    assert np.array_equal(grid, -grid.T)


def test_dequant_rounding_matches_python_binary16_packer():
    """Exact rational product (q-z)*s, rounded once by Python's own fp16 packer."""
    rng = np.random.default_rng(4)
    K, N, g = 256, 32, 128
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(1e-6, 3.0, (K // g, N)).astype(np.float16).view(np.uint16)
    w = oracle.dequant(codes, scales, zeros, g)
    for k in range(0, K, 7):
        for n in range(N):
            exact = (int(codes[k, n]) - int(zeros[k // g, n])) * exact_f16(scales[k // g, n])
            assert float(exact) == exact           # a 5-bit x 11-bit product fits a double
            assert int(w[k, n]) == py_f16_bits(float(exact)), (k, n)


def test_dequant_symmetric_equals_zero_eight():
    rng = np.random.default_rng(5)
    K, N, g = 128, 48, 64
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.002, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    eight = np.full((K // g, N), 8, dtype=np.uint8)
    assert np.array_equal(oracle.dequant(codes, scales, None, g),
                          oracle.dequant(codes, scales, eight, g))


@pytest.mark.parametrize("g", [64, 128])
def test_dequant_group_and_column_locality(g):
    """A scale or zero belongs to rows [r*g, (r+1)*g) of its own column, nowhere else."""
    rng = np.random.default_rng(6)
    K, N = 512, 40
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, (K // g, N)).astype(np.float16).view(np.uint16)
    base = oracle.dequant(codes, scales, zeros, g)
    r, n = 2, 17
    s2 = scales.copy()
    s2[r, n] = np.float16(0.75).view(np.uint16)
    z2 = zeros.copy()
    z2[r, n] = (int(z2[r, n]) + 5) % 16
    for variant in (oracle.dequant(codes, s2, zeros, g), oracle.dequant(codes, scales, z2, g)):
        diff = variant != base
        rows, cols = np.nonzero(diff)
        assert set(cols.tolist()) == {n}
        assert rows.min() >= r * g and rows.max() < (r + 1) * g
        # every row of the group whose code differs from the zero changes
        q = codes[r * g:(r + 1) * g, n].astype(int)
        assert diff[r * g:(r + 1) * g, n].sum() >= np.count_nonzero(q != zeros[r, n]) - 1


# ------------------------------------------------------------------------ the GEMM --

def _brute_force_bits(x_bits, w_bits, to_bits):
    """Exact rational sum of products, rounded once."""
    M, K = x_bits.shape
    N = w_bits.shape[1]
    xs = [[exact_f16(b) for b in row] for row in x_bits]
    ws = [[exact_f16(b) for b in row] for row in w_bits]
    out = np.empty((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            acc = sum((xs[m][k] * ws[k][n] for k in range(K)), Fraction(0))
            assert Fraction(float(acc)) == acc     # exact in a double, so one rounding
            out[m, n] = to_bits(float(acc))
    return out


@pytest.mark.parametrize("M,K,N", [(3, 64, 5), (4, 256, 6), (1, 128, 3)])
def test_gemm_matches_exact_rational_brute_force(M, K, N):
    g = 64 if K == 64 else 128
    seed = 100 + M + K + N
    codes, scales, zeros = workloads.weights(K, N, g, False, 0.005, 0.02, seed)
    x = workloads.activations(M, K, "f16", seed + 1)
    w = oracle.dequant(codes, scales, zeros, g)
    y = oracle.gemm(x, w)
    assert np.array_equal(y, _brute_force_bits(x, w, py_f16_bits))


def test_tiny_config_columns_match_exact_rational_brute_force():
    """The tiny workload itself (M=4, K=256, N=256), eight of its columns."""
    case = workloads.make_case(workloads.TINY, 4, 256, 256)
    y = oracle.w4a16(case["x"], case["codes"], case["scales"], case["zeros"], 128)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128)
    cols = [0, 1, 15, 16, 100, 127, 128, 255]
    assert np.array_equal(y[:, cols], _brute_force_bits(case["x"], w[:, cols], py_f16_bits))


def test_gemm_bf16_matches_exact_rational_brute_force():
    import torch

    def bf16_bits(x):
        t = torch.tensor([x], dtype=torch.float64).to(torch.float32)
        assert float(t) == x                         # single rounding only
        return int(t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0])

    rng = np.random.default_rng(7)
    M, K, N = 2, 32, 4
    # small integers and power-of-two scales keep every sum exact in float32
    x = torch.tensor(rng.integers(-3, 4, (M, K)), dtype=torch.bfloat16)
    x_bits = x.view(torch.int16).numpy().view(np.uint16)
    codes = rng.integers(0, 16, (128, N), dtype=np.uint8)[:K]
    w = np.empty((K, N), dtype=np.uint16)
    for k in range(K):
        for n in range(N):
            w[k, n] = bf16_bits((int(codes[k, n]) - 8) * 2.0 ** -4)
    y = oracle.gemm(x_bits, w, "bf16")
    xv = oracle.bf16_bits_to_f64(x_bits)
    wv = oracle.bf16_bits_to_f64(w)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(xv[m, k]) * Fraction(wv[k, n]) for k in range(K))
            assert int(y[m, n]) == bf16_bits(float(exact))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_identity_activations_reproduce_dequantized_weights(dtype):
    case = workloads.make_case(workloads.TINY, 1, 256, 64, seed=11)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128, dtype)
    one = 0x3C00 if dtype == "f16" else 0x3F80
    eye = (np.eye(256, dtype=np.uint16) * one).astype(np.uint16)
    assert np.array_equal(oracle.gemm(eye, w, dtype), w)


def test_gemm_one_hot_rows_pick_single_weight_rows():
    case = workloads.make_case(workloads.TINY, 1, 256, 48, seed=12)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128)
    picks = [0, 1, 127, 128, 200, 255]
    x = np.zeros((len(picks), 256), dtype=np.uint16)
    for i, k in enumerate(picks):
        x[i, k] = 0x3C00
    assert np.array_equal(oracle.gemm(x, w), w[picks])


@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_gemm_integer_special_case_matches_int64_matmul(g, sym):
    """X in {-1,0,1}, scale 2^-6: every partial sum is exact, so Y is fixed by integers."""
    rng = np.random.default_rng(13)
    M, K, N = 5, 384, 48
    x_int = rng.integers(-1, 2, (M, K))
    x_bits = x_int.astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = None if sym else rng.integers(0, 16, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -6, dtype=np.float16).view(np.uint16)
    zfull = np.full((K, N), 8) if sym else np.repeat(zeros.astype(np.int64), g, axis=0)
    ref_int = x_int.astype(np.int64) @ (codes.astype(np.int64) - zfull)
    ref = (ref_int * 2.0 ** -6).astype(np.float16).view(np.uint16)
    y = oracle.w4a16(x_bits, codes, scales, zeros, g)
    assert np.array_equal(y, ref)


def test_gemm_column_locality():
    case = workloads.make_case(workloads.TINY, 3, 256, 32, seed=14)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128)
    y = oracle.gemm(case["x"], w)
    w2 = w.copy()
    w2[:, 5] ^= 0x0100
    y2 = oracle.gemm(case["x"], w2)
    changed = np.nonzero((y2 != y).any(axis=0))[0]
    assert set(changed.tolist()) <= {5}


def test_gemm_threads_do_not_change_result():
    case = workloads.make_case(workloads.TINY, 9, 256, 40, seed=15)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128)
    assert np.array_equal(oracle.gemm(case["x"], w, threads=1),
                          oracle.gemm(case["x"], w, threads=4))


# -------------------------------------------------- large-shape route (float64 step) --

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bulk_activation_decode_matches_scalar_conversion_every_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bulk = oracle.act_bits_to_f64(bits, dtype)
    scalar = (oracle.f16_bits_to_f64 if dtype == "f16" else oracle.bf16_bits_to_f64)(bits)
    nan = np.isnan(scalar)
    assert np.array_equal(np.isnan(bulk), nan)
    assert np.array_equal(bulk[~nan], scalar[~nan])
    assert np.array_equal(np.signbit(bulk[~nan]), np.signbit(scalar[~nan]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N", [(3, 256, 40), (7, 1024, 24), (1, 4096, 16)])
def test_gemm_f64_rounded_equals_scalar_gemm(dtype, M, K, N):
    """Rounded once to the activation format, the float64 route gives the scalar loop's
    output bit for bit (the two sums differ by far less than half an output ulp), on both
    operand orders that a transposed-operand mistake would confuse (M != N)."""
    seed = 200 + M + K + N
    codes, scales, zeros = workloads.weights(K, N, 128, False, 0.005, 0.02, seed)
    x = workloads.activations(M, K, dtype, seed + 1)
    w = oracle.dequant(codes, scales, zeros, 128, dtype)
    ref = oracle.gemm(x, w, dtype, threads=4)
    y64 = oracle.gemm_f64(x, w, dtype)
    enc = oracle.f64_to_f16_bits if dtype == "f16" else oracle.f64_to_bf16_bits
    assert np.array_equal(enc(y64), ref)
    assert np.array_equal(enc(oracle.w4a16_f64(x, codes, scales, zeros, 128, dtype,
                                               col_chunk=7)), ref)


def test_gemm_f64_within_its_bound_of_the_exact_rational_sum():
    case = workloads.make_case(workloads.TINY, 2, 256, 256, seed=16)
    w = oracle.dequant(case["codes"], case["scales"], case["zeros"], 128)
    y64 = oracle.gemm_f64(case["x"], w)
    for m in range(2):
        for n in (0, 17, 255):
            terms = [exact_f16(case["x"][m, k]) * exact_f16(w[k, n]) for k in range(256)]
            exact = sum(terms, Fraction(0))
            bound = 256 * 2.0 ** -53 * float(sum(abs(t) for t in terms))
            assert abs(Fraction(float(y64[m, n])) - exact) <= Fraction(bound)


# ------------------------------------------------------------------------- packing --

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = (s.strip() for s in line.split("=", 1))
                vals[key] = val
    return vals


def test_packed_word_nibble_order_is_the_pages_interleave():
    gold = _read_golden("nibble_order.txt")
    order = [int(v) for v in gold["order_msb_to_lsb"].split()]
    expect_word = int(gold["word_elements_equal_index"], 16)
    K, N = 128, 16
    codes = np.zeros((K, N), dtype=np.uint8)
    codes[0:8, 0] = np.arange(8)                  # elements e0..e7 of the first word
    pc, _ = oracle.pack(codes, np.zeros((1, N), np.uint16), np.zeros((1, N), np.uint8), 128)
    word = int(pc[0:4].view("<u4")[0])
    assert word == expect_word
    assert [(word >> (4 * (7 - i))) & 0xF for i in range(8)] == order


@pytest.mark.parametrize("K,N,g,sym", [(256, 64, 128, False), (384, 48, 64, True),
                                       (128, 16, 128, False), (512, 32, 64, False)])
def test_pack_unpack_round_trip(K, N, g, sym):
    rng = np.random.default_rng(K + N + g)
    codes, scales, zeros = workloads.weights(K, N, g, sym, 0.005, 0.02, int(rng.integers(1e9)))
    pc, pm = oracle.pack(codes, scales, zeros, g)
    assert pc.size == K * N // 2
    assert pm.size == (K // g) * N * 2 + (0 if sym else (K // g) * N // 2)
    c2, s2, z2 = oracle.unpack(pc, pm, K, N, g, sym)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    if not sym:
        assert np.array_equal(z2, zeros)


def test_pack_is_a_bijection_on_nibble_positions():
    """Each element lands in its own nibble; read back the element index bit by bit."""
    K, N = 256, 48
    idx = np.arange(K * N, dtype=np.int64).reshape(K, N)
    nbits = int(K * N - 1).bit_length()
    where = np.zeros(K * N, dtype=np.int64)         # element index found at each nibble
    s = np.zeros((K // 128, N), np.uint16)
    for plane in range(0, nbits, 4):
        codes = ((idx >> plane) & 0xF).astype(np.uint8)
        pc, _ = oracle.pack(codes, s, None, 128)
        nib = np.empty(pc.size * 2, dtype=np.int64)
        nib[0::2] = pc & 0xF
        nib[1::2] = pc >> 4
        where |= nib << plane
    assert np.array_equal(np.sort(where), np.arange(K * N))


@pytest.mark.parametrize("K,N", [(256, 32), (512, 64)])
def test_packed_words_match_mfma_operand_lanes(K, N):
    """[TurboMind, Fig. 6]: after isolate & shift, registers match the MMA lane layout.

    gfx950 v_mfma_f32_16x16x32_f16: operand lane l holds row l%16 and the eight
    consecutive k = 8*(l//16) .. 8*(l//16)+7 of the 32-deep step, as four 32-bit registers
    of (k, k+1) pairs.  Here lane l of a 16-column x 128-k tile reads its 16 bytes with one
    128-bit load; word t is MFMA step t; register j of the step is
    (word >> 4j) & 0x000F000F, which must hold codes (k0+2j, k0+2j+1) of column l%16.
    """
    rng = np.random.default_rng(K * N)
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    pc, _ = oracle.pack(codes, np.zeros((K // 128, N), np.uint16), None, 128)
    words = pc.view("<u4").reshape(N // 16, K // 128, 64, 4)    # [strip][ktile][lane][t]
    for strip in range(N // 16):
        for kt in range(K // 128):
            for lane in range(64):
                n = strip * 16 + lane % 16
                for t in range(4):
                    k0 = kt * 128 + 32 * t + 8 * (lane // 16)
                    w = int(words[strip, kt, lane, t])
                    for j in range(4):
                        reg = (w >> (4 * j)) & 0x000F000F
                        assert reg & 0xFFFF == codes[k0 + 2 * j, n]
                        assert reg >> 16 == codes[k0 + 2 * j + 1, n]


def test_packed_meta_is_strip_major():
    """Scales of one 16-column strip are contiguous over all groups; zeros follow them."""
    K, N, g = 256, 32, 64
    rng = np.random.default_rng(21)
    codes, scales, zeros = workloads.weights(K, N, g, False, 0.005, 0.02, 21)
    _, pm = oracle.pack(codes, scales, zeros, g)
    sc = pm[: (K // g) * N * 2].view("<u2").reshape(N // 16, K // g, 16)
    assert np.array_equal(sc, scales.reshape(K // g, N // 16, 16).transpose(1, 0, 2))
    zb = pm[(K // g) * N * 2:]
    znib = np.empty(zb.size * 2, np.uint8)
    znib[0::2] = zb & 0xF
    znib[1::2] = zb >> 4
    assert np.array_equal(znib.reshape(N // 16, K // g, 16),
                          zeros.reshape(K // g, N // 16, 16).transpose(1, 0, 2))
