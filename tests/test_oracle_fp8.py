"""Pins for the oracle's FP8-weight functions (OCP E4M3 or E5M2 codes times an fp16 group
scale), each against something other than the oracle itself:
  * decoding      -- all 256 codes of each format against torch's float8_e4m3fn /
                     float8_e5m2 (library decoders), plus each format's landmark values (1,
                     the largest finite, the smallest subnormal and normal, infinities and
                     NaN codes, signed zero);
  * dequantization-- at power-of-two scales the product is exact in both activation formats;
                     random scales against exact rationals rounded by Python's binary16
                     packer; NaN and infinity propagate; scale locality (group row, column);
  * whole path    -- an integer special case against numpy int64 matmul: codes whose values
                     are small integers (all exact in the format), s = 2^-6, X in {-1,0,1},
                     so every partial sum is exact and Y is the single rounding of the
                     exact result.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(256, dtype=np.uint8)
TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FORMATS = sorted(TORCH)
# codes 0x7F / 0xFF are E4M3's NaNs; E5M2 spends exponent 31 on infinities and NaNs
FINITE = {"e4m3": ALL[(ALL & 0x7F) != 0x7F], "e5m2": ALL[(ALL & 0x7C) != 0x7C]}
INTS = {"e4m3": 16, "e5m2": 8}                 # every integer up to this is exact


def torch_fp8(codes: np.ndarray, fmt: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(TORCH[fmt])
    return t.to(torch.float64).numpy()


def fp8_code(v: float, fmt: str) -> int:
    return int(torch.tensor([v], dtype=torch.float32).to(TORCH[fmt]).view(torch.uint8)[0])


def py_f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


@pytest.mark.parametrize("fmt", FORMATS)
def test_fp8_decode_matches_torch_on_every_code(fmt):
    ours, ref = oracle.fp8_to_f64(ALL, fmt), torch_fp8(ALL, fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_landmarks():
    v = oracle.fp8_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0x7F, 0xFF, 0x80, 0xC0, 0x07,
                                    0x78], np.uint8), "e4m3")
    assert v[0] == 1.0 and v[1] == 448.0
    assert v[2] == 2.0 ** -9 and v[3] == 2.0 ** -6
    assert np.isnan(v[4]) and np.isnan(v[5])
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -2.0 and v[8] == 7 * 2.0 ** -9 and v[9] == 256.0


def test_e5m2_landmarks():
    v = oracle.fp8_to_f64(np.array([0x3C, 0x7B, 0x01, 0x04, 0x7C, 0xFC, 0x7D, 0x7F, 0xFE,
                                    0x80, 0xC0, 0x03], np.uint8), "e5m2")
    assert v[0] == 1.0 and v[1] == 57344.0
    assert v[2] == 2.0 ** -16 and v[3] == 2.0 ** -14
    assert v[4] == np.inf and v[5] == -np.inf
    assert np.isnan(v[6:9]).all()
    assert v[9] == 0.0 and np.signbit(v[9])
    assert v[10] == -2.0 and v[11] == 3 * 2.0 ** -16


def test_e5m2_is_the_high_byte_of_binary16():
    """E5M2 shares binary16's exponent bias and layout: code b is the fp16 bit pattern
    b << 8 (Python's binary16 unpacker decodes it independently)."""
    for b in FINITE["e5m2"]:
        h = struct.unpack("<e", struct.pack("<H", int(b) << 8))[0]
        assert oracle.fp8_to_f64(np.array([b], np.uint8), "e5m2")[0] == h


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_dequant_power_of_two_scale_is_exact(fmt, dtype):
    g = 64
    fin = FINITE[fmt]
    codes = np.tile(fin.reshape(1, -1), (g, 1))
    exps = (0, -4, -8) if fmt == "e4m3" else (0, -2)   # E5M2 subnormals need s >= 2^-8
    for e in exps:
        s = np.full((1, fin.size), 2.0 ** e, np.float16).view(np.uint16)
        w = oracle.dequant_fp8(codes, s, g, fmt, dtype)
        val = oracle.f16_bits_to_f64(w) if dtype == "f16" else oracle.bf16_bits_to_f64(w)
        assert np.array_equal(val, np.tile(torch_fp8(fin, fmt) * 2.0 ** e, (g, 1)))
        assert np.array_equal(np.signbit(val[0]), np.signbit(torch_fp8(fin, fmt)))


@pytest.mark.parametrize("fmt", FORMATS)
def test_fp8_dequant_nan_and_infinity_propagate(fmt):
    special = [0x7F, 0xFF] if fmt == "e4m3" else [0x7D, 0xFF, 0x7C, 0xFC]
    codes = np.array([special + [0x38 if fmt == "e4m3" else 0x3C]], np.uint8).repeat(64, 0)
    s = np.full((1, codes.shape[1]), 0.25, np.float16).view(np.uint16)
    for dtype, conv in (("f16", oracle.f16_bits_to_f64), ("bf16", oracle.bf16_bits_to_f64)):
        val = conv(oracle.dequant_fp8(codes, s, 64, fmt, dtype))
        assert np.isnan(val[:, :2]).all() and (val[:, -1] == 0.25).all()
        if fmt == "e5m2":
            assert (val[:, 2] == np.inf).all() and (val[:, 3] == -np.inf).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_fp8_dequant_rounding_matches_python_binary16_packer(fmt):
    rng = np.random.default_rng(50)
    K, N, g = 128, 24, 64
    codes = rng.choice(FINITE[fmt], (K, N)).astype(np.uint8)
    scales = rng.uniform(1e-4, 0.05, (K // g, N)).astype(np.float16).view(np.uint16)
    w = oracle.dequant_fp8(codes, scales, g, fmt)
    vals = torch_fp8(codes, fmt)
    for k in range(0, K, 3):
        for n in range(N):
            exact = Fraction(float(vals[k, n])) * Fraction(float(scales[k // g, n].view(np.float16)))
            assert float(exact) == exact
            want = py_f16_bits(float(exact)) if exact else \
                (0x8000 if np.signbit(vals[k, n]) else 0)       # -0 * s keeps its sign
            assert int(w[k, n]) == want, (k, n)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("g", [64, 128])
def test_fp8_dequant_group_and_column_locality(fmt, g):
    rng = np.random.default_rng(51)
    K, N = 512, 32
    codes = rng.choice(FINITE[fmt], (K, N)).astype(np.uint8)
    codes[codes & 0x7F == 0] = fp8_code(1.0, fmt)      # no zeros: every scale change shows
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    base = oracle.dequant_fp8(codes, scales, g, fmt)
    r, n = 2, 17
    s2 = scales.copy()
    s2[r, n] = np.float16(0.5).view(np.uint16)
    diff = np.argwhere(oracle.dequant_fp8(codes, s2, g, fmt) != base)
    assert len(diff) == g and set(diff[:, 1]) == {n}
    assert diff[:, 0].min() == r * g and diff[:, 0].max() == (r + 1) * g - 1


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("g", [64, 128])
def test_fp8_gemm_integer_special_case_matches_int64_matmul(fmt, g):
    """Weights take small integer values (all exact in the format) times s = 2^-6, X in
    {-1,0,1}: every product and partial sum is a multiple of 2^-6 below 2^13, exact in fp32
    and fp64, so Y is the single rounding of the int64 result * 2^-6."""
    rng = np.random.default_rng(52 + g)
    M, K, N = 7, 512, 48
    lim = INTS[fmt]
    ints = rng.integers(-lim, lim + 1, (K, N))
    table = {v: fp8_code(float(v), fmt) for v in range(-lim, lim + 1)}
    codes = np.vectorize(table.get)(ints).astype(np.uint8)
    assert np.array_equal(torch_fp8(codes, fmt), ints)
    x = rng.integers(-1, 2, (M, K))
    scales = np.full((K // g, N), 2.0 ** -6, np.float16).view(np.uint16)
    ref = ((x @ ints) * 2.0 ** -6).astype(np.float16).view(np.uint16)
    xb = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.wfp8a16(xb, codes, scales, g, fmt), ref)
