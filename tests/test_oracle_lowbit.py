"""Pins for the oracle's 2-bit and 3-bit weight functions, each against something other
than the oracle itself:
  * dequantization -- the closed form (q - z) * 2^e over every (q, z) pair, exact in both
                      formats; sign/zero/antisymmetry; symmetric == the middle zero;
                      rational brute force through Python's binary16 packer; locality;
  * whole path     -- an integer special case against numpy int64 matmul;
  * packing        -- round trips (aligned and ragged); every code owns b distinct bits and
                      together they cover the plane exactly once; the MFMA-operand view:
                      the 16x16x32 A operand of lane l (row l % 16, k = 8 (l / 16) .. +7 of
                      each 32-deep step, elements 2j, 2j + 1 in the low and high half of
                      register j) read by the shift/mask extraction the header describes;
                      ragged packing equals aligned packing of the padded matrix.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle

BITS = [2, 3]


def py_f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def grid(bits, group=64):
    hi = 1 << bits
    q = np.arange(hi)
    qq, zz = np.meshgrid(q, q, indexing="ij")
    codes = np.tile(qq.reshape(1, -1).astype(np.uint8), (group, 1))
    return codes, zz.reshape(1, -1).astype(np.uint8), qq.ravel(), zz.ravel()


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_power_of_two_scale_is_exact_closed_form(bits, dtype):
    codes, zeros, q, z = grid(bits)
    for e in (0, -5, -9):
        s = np.full((1, q.size), 2.0 ** e, np.float16).view(np.uint16)
        w = oracle.dequant_lowbit(bits, codes, s, zeros, 64, dtype)
        val = oracle.f16_bits_to_f64(w) if dtype == "f16" else oracle.bf16_bits_to_f64(w)
        assert np.array_equal(val, np.tile((q - z) * 2.0 ** e, (64, 1)))


@pytest.mark.parametrize("bits", BITS)
def test_dequant_sign_zero_antisymmetry_and_symmetric_zero(bits):
    codes, zeros, q, z = grid(bits)
    s = np.full((1, q.size), 0.0123, np.float16).view(np.uint16)
    val = oracle.f16_bits_to_f64(oracle.dequant_lowbit(bits, codes, s, zeros, 64)[0])
    assert np.array_equal(val == 0, q == z)
    assert np.array_equal(np.sign(val), np.sign(q - z))
    g = val.reshape(1 << bits, 1 << bits)
    assert np.array_equal(g, -g.T)
    mid = np.full_like(zeros, 1 << (bits - 1))
    assert np.array_equal(oracle.dequant_lowbit(bits, codes, s, None, 64),
                          oracle.dequant_lowbit(bits, codes, s, mid, 64))


@pytest.mark.parametrize("bits", BITS)
def test_dequant_rounding_matches_python_binary16_packer(bits):
    rng = np.random.default_rng(60 + bits)
    K, N, g = 128, 24, 64
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 1 << bits, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(1e-5, 0.5, (K // g, N)).astype(np.float16).view(np.uint16)
    w = oracle.dequant_lowbit(bits, codes, scales, zeros, g)
    for k in range(0, K, 5):
        for n in range(N):
            exact = (int(codes[k, n]) - int(zeros[k // g, n])) * \
                Fraction(float(scales[k // g, n].view(np.float16)))
            assert int(w[k, n]) == py_f16_bits(float(exact)), (k, n)


@pytest.mark.parametrize("bits", BITS)
def test_dequant_group_and_column_locality(bits):
    rng = np.random.default_rng(62)
    K, N, g = 512, 32, 128
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 1 << bits, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    base = oracle.dequant_lowbit(bits, codes, scales, zeros, g)
    r, n = 2, 17
    s2 = scales.copy()
    s2[r, n] = np.float16(0.5).view(np.uint16)
    diff = np.argwhere(oracle.dequant_lowbit(bits, codes, s2, zeros, g) != base)
    assert len(diff) and set(diff[:, 1]) == {n}
    assert diff[:, 0].min() >= r * g and diff[:, 0].max() < (r + 1) * g


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("sym", [False, True])
def test_gemm_integer_special_case_matches_int64_matmul(bits, sym):
    rng = np.random.default_rng(63 + bits)
    M, K, N, g = 7, 512, 48, 64
    x = rng.integers(-1, 2, (M, K))
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    zeros = None if sym else rng.integers(0, 1 << bits, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -6, np.float16).view(np.uint16)
    zfull = np.full((K, N), 1 << (bits - 1)) if sym else np.repeat(zeros.astype(np.int64), g, 0)
    ref = ((x @ (codes.astype(np.int64) - zfull)) * 2.0 ** -6).astype(np.float16).view(np.uint16)
    xb = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.wlowbit_a16(bits, xb, codes, scales, zeros, g), ref)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N,g,sym", [(256, 64, 128, False), (384, 48, 64, True),
                                       (200, 40, 64, False), (8, 7, 128, True)])
def test_pack_unpack_round_trip(bits, K, N, g, sym):
    rng = np.random.default_rng(K * N + bits)
    rows = -(-K // g)
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (rows, N)).astype(np.float16).view(np.uint16)
    zeros = None if sym else rng.integers(0, 1 << bits, (rows, N), dtype=np.uint8)
    pc, pm = oracle.pack_lowbit(bits, codes, scales, zeros, g)
    Kp, Np = -(-K // 128) * 128, -(-N // 16) * 16
    assert pc.size == Kp * Np * bits // 8
    c2, s2, z2 = oracle.unpack_lowbit(bits, pc, pm, K, N, g, sym)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    if not sym:
        assert np.array_equal(z2, zeros)


@pytest.mark.parametrize("bits", BITS)
def test_every_code_owns_distinct_bits_covering_the_plane(bits):
    K, N = 128, 16
    s = np.zeros((1, N), np.uint16)
    owner = np.full(K * N * bits, -1)
    for k in range(K):
        for n in range(N):
            codes = np.zeros((K, N), np.uint8)
            codes[k, n] = (1 << bits) - 1
            pc, _ = oracle.pack_lowbit(bits, codes, s, None, 128)
            set_bits = np.nonzero(np.unpackbits(pc, bitorder="little"))[0]
            assert set_bits.size == bits
            assert (owner[set_bits] == -1).all()
            owner[set_bits] = k * N + n
    assert (owner >= 0).all()


def extract_pair(words, r, bits):
    """Low/high half codes of pair register r of one lane, by the header's recipe."""
    if bits == 2:
        src = int(words[r // 8]) >> (8 * ((r % 8) // 4))
        p = 2 * ((r % 8) % 4)
        return (src >> p) & 3, (src >> (16 + p)) & 3
    if r < 15:
        src = int(words[r // 5]) >> (9 if r % 5 >= 3 else 0)
        p = 3 * ((r % 5) % 3)
        return (src >> p) & 7, (src >> (16 + p)) & 7
    lo = sum(((int(words[c]) >> 15) & 1) << c for c in range(3))
    hi = sum(((int(words[c]) >> 31) & 1) << c for c in range(3))
    return lo, hi


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("K,N", [(128, 16), (256, 32)])
def test_packed_words_are_mfma_operand_registers(bits, K, N):
    rng = np.random.default_rng(K + N + bits)
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    s = np.zeros((K // 128, N), np.uint16)
    pc, _ = oracle.pack_lowbit(bits, codes, s, None, 128)
    words = pc.view("<u4")
    for T in range(N // 16 * K // 128):
        strip, kt = divmod(T, K // 128)
        for lane in range(64):
            lw = words[(T * 256 * bits + lane * 4 * bits) // 4:][:bits]
            n = strip * 16 + lane % 16
            for r in range(16):
                t, j = divmod(r, 4)
                k = kt * 128 + 32 * t + 8 * (lane // 16) + 2 * j
                assert extract_pair(lw, r, bits) == (codes[k, n], codes[k + 1, n]), (T, lane, r)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("K,N,g", [(200, 40, 64), (40, 20, 64), (136, 1, 128)])
def test_ragged_packing_is_aligned_packing_of_the_padded_matrix(bits, sym, K, N, g):
    rng = np.random.default_rng(K + N + g + bits)
    rows = -(-K // g)
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (rows, N)).astype(np.float16).view(np.uint16)
    zeros = None if sym else rng.integers(0, 1 << bits, (rows, N), dtype=np.uint8)
    Kp, Np = -(-K // 128) * 128, -(-N // 16) * 16
    sp = np.zeros((Kp // g, Np), np.uint16)
    sp[:rows, :N] = scales
    zp = None
    if zeros is not None:
        zp = np.zeros((Kp // g, Np), np.uint8)
        zp[:rows, :N] = zeros
    cp = np.zeros((Kp, Np), np.uint8)
    cp[:K, :N] = codes
    for k in range(K, Kp):
        cp[k, :N] = (1 << (bits - 1)) if zp is None else zp[k // g, :N]
    got = oracle.pack_lowbit(bits, codes, scales, zeros, g)
    want = oracle.pack_lowbit(bits, cp, sp, zp, g)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


@pytest.mark.parametrize("bits", BITS)
def test_only_the_low_bits_of_codes_and_zeros_are_read(bits):
    rng = np.random.default_rng(70 + bits)
    K, N, g = 256, 32, 128
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    m = (1 << bits) - 1
    assert np.array_equal(oracle.dequant_lowbit(bits, codes, scales, zeros, g),
                          oracle.dequant_lowbit(bits, codes & m, scales, zeros & m, g))
    a = oracle.pack_lowbit(bits, codes, scales, zeros, g)
    b = oracle.pack_lowbit(bits, codes & m, scales, zeros & m, g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
