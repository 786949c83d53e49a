"""Pins for the oracle's ragged-shape packing (K % 128 != 0 or N % 16 != 0).

Rule under test: the planes of a K x N matrix are those of the matrix padded to Kp x Np
(Np = N rounded up to 16; Kp = K rounded up to 128), where every
padded weight dequantizes to zero: in padded rows k >= K the code is the element's zero
point (its group's zero, 0 in groups past ceil(K/g), 8 / 128 for symmetric codes); padded
columns and padded groups hold code 0, scale 0 and zero 0.

The padded matrix is built here with numpy from that rule alone, and packed by the
aligned path, whose layout is pinned elsewhere (tests/test_oracle.py, test_oracle_w8.py).
  * ragged packing == aligned packing of the padded matrix, byte for byte;
  * unpacking returns the user matrix;
  * the padded part dequantizes to exact zeros, so the GEMM of X (zero-padded to Kp) with
    the padded weights equals the GEMM of the user matrices bit for bit.
"""
import numpy as np
import pytest

import oracle

SHAPES = [(200, 40, 64), (200, 40, 128), (72, 16, 64), (128, 33, 128), (384, 7, 64), (40, 20, 64),
          (136, 1, 128), (1000, 50, 128)]


def pad_rule(K, N):
    Kp = -(-K // 128) * 128
    return Kp, -(-N // 16) * 16


def user_matrix(K, N, g, sym, bits, seed):
    rng = np.random.default_rng(seed)
    hi = 1 << bits
    rows = -(-K // g)
    codes = rng.integers(0, hi, (K, N), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.02, (rows, N)).astype(np.float16).view(np.uint16)
    zeros = None if sym else rng.integers(0, hi, (rows, N), dtype=np.uint8)
    return codes, scales, zeros


def padded_matrix(codes, scales, zeros, g, bits):
    K, N = codes.shape
    Kp, Np = pad_rule(K, N)
    rows = scales.shape[0]
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
    return cp, sp, zp


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("K,N,g", SHAPES)
def test_ragged_packing_is_aligned_packing_of_the_padded_matrix(K, N, g, sym, bits):
    codes, scales, zeros = user_matrix(K, N, g, sym, bits, K * N + g)
    cp, sp, zp = padded_matrix(codes, scales, zeros, g, bits)
    pack = oracle.pack if bits == 4 else oracle.pack_w8
    got = pack(codes, scales, zeros, g)
    want = pack(cp, sp, zp, g)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    Kp, Np = pad_rule(K, N)
    size = oracle.packed_code_bytes if bits == 4 else oracle.packed_code_bytes_w8
    assert size(K, N) == Kp * Np * bits // 8 == got[0].size
    assert oracle.padded_shape(K, N) == (Kp, Np)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("K,N,g", SHAPES)
def test_ragged_unpack_round_trips(K, N, g, sym, bits):
    codes, scales, zeros = user_matrix(K, N, g, sym, bits, K + N + g)
    pack, unpack = (oracle.pack, oracle.unpack) if bits == 4 else (oracle.pack_w8, oracle.unpack_w8)
    pc, pm = pack(codes, scales, zeros, g)
    c2, s2, z2 = unpack(pc, pm, K, N, g, sym)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    if not sym:
        assert np.array_equal(z2, zeros)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("K,N,g", SHAPES[:4])
def test_padding_dequantizes_to_zero_and_leaves_the_gemm_unchanged(K, N, g, sym, bits):
    codes, scales, zeros = user_matrix(K, N, g, sym, bits, 3 * K + N)
    cp, sp, zp = padded_matrix(codes, scales, zeros, g, bits)
    deq = oracle.dequant if bits == 4 else oracle.dequant_w8
    wp = oracle.f16_bits_to_f64(deq(cp, sp, zp, g))
    assert (wp[K:, :N] == 0).all() and (wp[:, N:] == 0).all()
    x = np.random.default_rng(K).standard_normal((5, K)).astype(np.float16).view(np.uint16)
    xp = np.zeros((5, cp.shape[0]), np.uint16)
    xp[:, :K] = x
    gemm = oracle.w4a16 if bits == 4 else oracle.w8a16
    assert np.array_equal(gemm(xp, cp, sp, zp, g)[:, :N], gemm(x, codes, scales, zeros, g))
