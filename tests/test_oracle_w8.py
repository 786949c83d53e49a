"""Pins for the oracle's 8-bit-weight (W8A16) functions, each against something other than
the oracle itself:
  * dequantization -- closed form (q - z) * 2^e over the whole 256 x 256 (q, z) grid (exact
                      in both formats), sign/zero/antisymmetry invariants, symmetric ==
                      zero 128, group/column locality, exact rational products rounded by
                      Python's binary16 packer;
  * whole path     -- an integer special case against numpy int64 matmul (every partial
                      sum exact, so the result is unique);
  * packing        -- round trip, a bijection on byte positions, the MFMA-operand view of
                      every packed byte (the 16x16x32 operand lane l of a 16-column x 64-k
                      tile reads codes k0..k0+7 of column l % 16 as two 32-bit words), the
                      strip-major meta plane with one zero byte per element.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def py_f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def _grid(group=64):
    """All 256 x 256 (q, z) pairs over one group: K = group, N = 65536 columns."""
    q = np.arange(256)
    qq, zz = np.meshgrid(q, q, indexing="ij")
    codes = np.tile(qq.reshape(1, -1).astype(np.uint8), (group, 1))
    zeros = zz.reshape(1, -1).astype(np.uint8)
    return codes, zeros, qq.ravel(), zz.ravel()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_w8_dequant_power_of_two_scale_is_exact_closed_form(dtype):
    codes, zeros, q, z = _grid()
    for e in (-3, -8):
        s = np.full((1, q.size), 2.0 ** e, dtype=np.float16).view(np.uint16)
        w = oracle.dequant_w8(codes[:1].repeat(64, 0), s, zeros, 64, dtype)[0]
        val = oracle.f16_bits_to_f64(w) if dtype == "f16" else oracle.bf16_bits_to_f64(w)
        assert np.array_equal(val, (q - z) * 2.0 ** e)


def test_w8_dequant_sign_zero_and_antisymmetry():
    codes, zeros, q, z = _grid()
    s = np.full((1, q.size), 0.0123, dtype=np.float16).view(np.uint16)
    val = oracle.f16_bits_to_f64(oracle.dequant_w8(codes, s, zeros, 64)[0])
    assert np.array_equal(val == 0, q == z)
    assert np.array_equal(np.sign(val), np.sign(q - z))
    grid = val.reshape(256, 256)
    assert np.array_equal(grid, -grid.T)


def test_w8_dequant_rounding_matches_python_binary16_packer():
    rng = np.random.default_rng(40)
    K, N, g = 128, 24, 64
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(1e-5, 0.5, (K // g, N)).astype(np.float16).view(np.uint16)
    w = oracle.dequant_w8(codes, scales, zeros, g)
    for k in range(0, K, 5):
        for n in range(N):
            exact = (int(codes[k, n]) - int(zeros[k // g, n])) * \
                Fraction(float(scales[k // g, n].view(np.float16)))
            assert float(exact) == exact
            assert int(w[k, n]) == py_f16_bits(float(exact)), (k, n)


def test_w8_dequant_symmetric_equals_zero_128():
    rng = np.random.default_rng(41)
    K, N, g = 128, 32, 128
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    mid = np.full((K // g, N), 128, dtype=np.uint8)
    assert np.array_equal(oracle.dequant_w8(codes, scales, None, g),
                          oracle.dequant_w8(codes, scales, mid, g))


@pytest.mark.parametrize("g", [64, 128])
def test_w8_dequant_group_and_column_locality(g):
    rng = np.random.default_rng(42)
    K, N = 512, 32
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    base = oracle.dequant_w8(codes, scales, zeros, g)
    r, n = 2, 17
    s2 = scales.copy()
    s2[r, n] = np.float16(0.5).view(np.uint16)
    z2 = zeros.copy()
    z2[r, n] ^= 0x5A
    for s_, z_ in ((s2, zeros), (scales, z2)):
        w = oracle.dequant_w8(codes, s_, z_, g)
        diff = np.argwhere(w != base)
        assert diff.size and set(diff[:, 1]) == {n}
        assert diff[:, 0].min() >= r * g and diff[:, 0].max() < (r + 1) * g


@pytest.mark.parametrize("g,sym", [(128, False), (64, True)])
def test_w8_gemm_integer_special_case_matches_int64_matmul(g, sym):
    """X in {-1,0,1} and s = 2^-8: every product and partial sum is an exact multiple of
    2^-8 (at most 17 significant bits, exact in fp32 and fp64), so Y is the single
    rounding of int64 matmul * 2^-8, bit for bit, whatever the summation order."""
    rng = np.random.default_rng(43)
    M, K, N = 7, 512, 48
    x = rng.integers(-1, 2, (M, K))
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    zeros = None if sym else rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -8, dtype=np.float16).view(np.uint16)
    zfull = np.repeat(np.full((K // g, N), 128) if sym else zeros.astype(np.int64), g, axis=0)
    exact = x @ (codes.astype(np.int64) - zfull)
    # numpy's float16 cast rounds the exact sum once, to nearest even
    ref = (exact * 2.0 ** -8).astype(np.float16).view(np.uint16)
    xb = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.w8a16(xb, codes, scales, zeros, g), ref)


@pytest.mark.parametrize("K,N,g,sym", [(256, 64, 128, False), (384, 48, 64, True),
                                       (128, 16, 128, False), (512, 32, 64, False)])
def test_w8_pack_unpack_round_trip(K, N, g, sym):
    rng = np.random.default_rng(K * N + g)
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    _, scales, _ = workloads.weights(K, N, g, True, 0.001, 0.01, int(rng.integers(1e9)))
    zeros = None if sym else rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    pc, pm = oracle.pack_w8(codes, scales, zeros, g)
    assert pc.size == K * N
    assert pm.size == (K // g) * N * 2 + (0 if sym else (K // g) * N)
    c2, s2, z2 = oracle.unpack_w8(pc, pm, K, N, g, sym)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    if not sym:
        assert np.array_equal(z2, zeros)


def test_w8_pack_is_a_bijection_on_byte_positions():
    K, N = 256, 48
    idx = np.arange(K * N, dtype=np.int64).reshape(K, N)
    where = np.zeros(K * N, dtype=np.int64)
    s = np.zeros((K // 128, N), np.uint16)
    for plane in (0, 8):
        pc, _ = oracle.pack_w8(((idx >> plane) & 0xFF).astype(np.uint8), s, None, 128)
        where |= pc.astype(np.int64) << plane
    assert np.array_equal(np.sort(where), np.arange(K * N))


@pytest.mark.parametrize("K,N", [(128, 32), (512, 48)])
def test_w8_packed_bytes_match_mfma_operand_lanes(K, N):
    """gfx950 v_mfma_f32_16x16x32_f16: operand lane l holds row l % 16 and the eight
    consecutive k = 8 (l // 16) .. +7 of a 32-deep step.  Lane l of a 16-column x 64-k tile
    reads its 16 bytes with one 128-bit load; bytes 8t .. 8t+7 are step t, k ascending."""
    rng = np.random.default_rng(K + N)
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    pc, _ = oracle.pack_w8(codes, np.zeros((K // 128, N), np.uint16), None, 128)
    tiles = pc.reshape(N // 16, K // 64, 64, 16)              # [strip][ktile][lane][byte]
    for strip in range(N // 16):
        for kt in range(K // 64):
            for lane in range(64):
                n = strip * 16 + lane % 16
                for t in range(2):
                    k0 = kt * 64 + 32 * t + 8 * (lane // 16)
                    assert np.array_equal(tiles[strip, kt, lane, 8 * t:8 * t + 8],
                                          codes[k0:k0 + 8, n])


def test_w8_packed_meta_is_strip_major_with_byte_zeros():
    K, N, g = 256, 32, 64
    rng = np.random.default_rng(44)
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    zeros = rng.integers(0, 256, (K // g, N), dtype=np.uint8)
    _, pm = oracle.pack_w8(codes, scales, zeros, g)
    sc = pm[: (K // g) * N * 2].view("<u2").reshape(N // 16, K // g, 16)
    assert np.array_equal(sc, scales.reshape(K // g, N // 16, 16).transpose(1, 0, 2))
    zb = pm[(K // g) * N * 2:]
    assert np.array_equal(zb.reshape(N // 16, K // g, 16),
                          zeros.reshape(K // g, N // 16, 16).transpose(1, 0, 2))
