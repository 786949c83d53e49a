"""GPU parity of ragged shapes (N % 16 != 0, K % 128 != 0) through the C ABI, against the
CPU oracle.  The packed planes hold the matrix padded to Kp x Np with zero weights; the
kernels read activations only for k < K and store only n < N.

  * packing: bytes equal the oracle's ragged packing; unpacking returns the user matrix;
  * GEMMs: bit-exact where every partial sum is exact (X in {-1,0,1}, power-of-two
    scales), else max|Y - Y_ref| / max|Y_ref| <= 5e-3, for every configuration that can
    run the shape and every code format;
  * isolation: non-finite activations in row m + 1 never reach row m (the kernels must not
    read past the end of a row into the next one), and outputs past column N are never
    written.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, dev_half, dev_u8, host_bits, rel_err, say, tol

pytestmark = pytest.mark.gpu

# (K, N): ragged K, K % 256 == 128, ragged N (odd, < 16, not a multiple of 4), both
SHAPES = [(200, 48), (256, 40), (384, 7), (136, 1), (1000, 33), (4104, 100), (8, 16),
          (512, 4098)]


def configs(M, K, code):
    return [c for c in (1, 2, 3, 4) if M <= 16 * c] + [12, 13, 14]


def make(code, K, N, g, sym, seed):
    rng = np.random.default_rng(seed)
    rows = -(-K // g)
    if code == "w4":
        codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
        zeros = None if sym else rng.integers(0, 16, (rows, N), dtype=np.uint8)
        scales = rng.uniform(0.005, 0.02, (rows, N))
    elif code == "w8":
        codes = rng.integers(0, 256, (K, N), dtype=np.uint8)
        zeros = None if sym else rng.integers(0, 256, (rows, N), dtype=np.uint8)
        scales = rng.uniform(0.0003, 0.0012, (rows, N))
    else:
        codes = workloads.to_fp8_bits(
            np.clip(rng.standard_normal((K, N), dtype=np.float32) * 64, -448, 448), "e4m3")
        zeros = None
        scales = rng.uniform(0.0001, 0.0003, (rows, N))
    return codes, scales.astype(np.float16).view(np.uint16), zeros


def pack(code, codes, scales, zeros, g):
    c, s = dev_u8(codes), dev_half(scales)
    if code == "w4":
        return mp.pack_weights(c, s, None if zeros is None else dev_u8(zeros), g)
    if code == "w8":
        return mp.pack_weights_w8(c, s, None if zeros is None else dev_u8(zeros), g)
    return mp.pack_weights_fp8(c, s, g, "e4m3")


def gemm(code, x, packed, cfg):
    fn = {"w4": mp.w4a16, "w8": mp.w8a16, "fp8": mp.wfp8a16}[code]
    return fn(x, packed, config=cfg)


def ref(code, x, codes, scales, zeros, g, dtype):
    if code == "w4":
        return oracle.w4a16(x, codes, scales, zeros, g, dtype, threads=8)
    if code == "w8":
        return oracle.w8a16(x, codes, scales, zeros, g, dtype, threads=8)
    return oracle.wfp8a16(x, codes, scales, g, "e4m3", dtype, threads=8)


@pytest.mark.parametrize("code", ["w4", "w8", "fp8"])
@pytest.mark.parametrize("K,N", SHAPES)
def test_ragged_pack_matches_oracle_and_round_trips(code, K, N):
    g, sym = 64, code == "fp8"
    say(f"ragged pack {code} K={K} N={N}")
    codes, scales, zeros = make(code, K, N, g, sym, K * 7 + N)
    packed = pack(code, codes, scales, zeros, g)
    opack = oracle.pack if code == "w4" else oracle.pack_w8
    pc, pm = opack(codes, scales, zeros, g)
    assert np.array_equal(packed.codes.cpu().numpy(), pc)
    assert np.array_equal(packed.meta.cpu().numpy(), pm)
    c2, s2, z2 = mp.unpack(packed)
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), scales)
    if zeros is not None:
        assert np.array_equal(z2.cpu().numpy(), zeros)


@pytest.mark.parametrize("code", ["w4", "w8", "fp8"])
@pytest.mark.parametrize("M", [1, 37, 130])
@pytest.mark.parametrize("K,N", SHAPES)
def test_ragged_gemm_random_all_configs(code, M, K, N):
    g = 128 if K % 3 else 64
    sym = code == "fp8" or N % 2 == 1
    dtype = "bf16" if (K + N) % 2 else "f16"
    codes, scales, zeros = make(code, K, N, g, sym, M * 31 + K + N)
    x = workloads.activations(M, K, dtype, M + K + N)
    packed = pack(code, codes, scales, zeros, g)
    want = ref(code, x, codes, scales, zeros, g, dtype)
    for cfg in [0] + configs(M, K, code):
        say(f"ragged random {code} {dtype} M={M} K={K} N={N} g={g} sym={sym} config={cfg}")
        y = gemm(code, dev_half(x, dtype), packed, cfg)
        torch.cuda.synchronize()
        assert y.shape == (M, N)
        assert rel_err(host_bits(y), want, dtype) <= tol(dtype), cfg


@pytest.mark.parametrize("code", ["w4", "w8"])
@pytest.mark.parametrize("K,N", [(200, 40), (1000, 33), (136, 7)])
def test_ragged_gemm_integer_case_bit_exact(code, K, N):
    """X in {-1,0,1}, scales 2^-8: every partial sum is exact, so Y is unique."""
    M, g = 70, 64
    rng = np.random.default_rng(K + N)
    codes, _, zeros = make(code, K, N, g, False, K)
    scales = np.full((-(-K // g), N), 2.0 ** -8, np.float16).view(np.uint16)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    packed = pack(code, codes, scales, zeros, g)
    want = ref(code, x, codes, scales, zeros, g, "f16")
    for cfg in [0] + configs(M, K, code):
        say(f"ragged integer {code} K={K} N={N} config={cfg}")
        y = gemm(code, dev_half(x), packed, cfg)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), want), cfg


@pytest.mark.parametrize("K", [200, 4104])
@pytest.mark.parametrize("M", [6, 100])
def test_ragged_k_never_reads_the_next_row(K, M):
    """Odd rows start with infinities; even rows are finite.  A kernel that read past the
    end of an even row (into the padded k range) would turn its output into NaN."""
    N, g = 48, 128
    codes, scales, zeros = make("w4", K, N, g, False, K + M)
    x = workloads.activations(M, K, "f16", M).copy()
    x[1::2, :8] = 0x7C00                                    # +inf
    packed = pack("w4", codes, scales, zeros, g)
    want = oracle.f16_bits_to_f64(ref("w4", x, codes, scales, zeros, g, "f16"))
    for cfg in [0] + configs(M, K, "w4"):
        say(f"ragged next-row M={M} K={K} config={cfg}")
        y = gemm("w4", dev_half(x), packed, cfg)
        torch.cuda.synchronize()
        got = oracle.f16_bits_to_f64(host_bits(y))
        assert np.isfinite(got[0::2]).all(), cfg
        assert not np.isfinite(got[1::2]).any() and not np.isfinite(want[1::2]).any()
        e = np.abs(got[0::2] - want[0::2]).max() / np.abs(want[0::2]).max()
        assert e <= REL_TOL, cfg


@pytest.mark.parametrize("N", [1, 7, 33])
def test_ragged_n_writes_nothing_past_the_output(N):
    """Y is a view into a larger buffer filled with a sentinel; only the M x N window may
    change."""
    K, M, g = 256, 130, 128
    codes, scales, zeros = make("w4", K, N, g, False, N)
    x = workloads.activations(M, K, "f16", N)
    packed = pack("w4", codes, scales, zeros, g)
    want = ref("w4", x, codes, scales, zeros, g, "f16")
    for cfg in [0] + configs(M, K, "w4") + [1]:
        m = M if cfg != 1 else 16
        say(f"ragged store N={N} M={m} config={cfg}")
        buf = torch.full((m * N + 64,), 12345, dtype=torch.int16, device="cuda")
        out = buf[:m * N].view(torch.float16).view(m, N)
        mp.w4a16(dev_half(x[:m]), packed, out=out, config=cfg)
        torch.cuda.synchronize()
        assert (buf[m * N:] == 12345).all(), cfg
        got = host_bits(out)
        err = rel_err(got, want[:m], "f16")
        if err > REL_TOL:
            g64 = oracle.f16_bits_to_f64(got)
            w64 = oracle.f16_bits_to_f64(want[:m])
            bad = np.argwhere(np.abs(g64 - w64) > REL_TOL * np.abs(w64).max())
            print(f"[diag] cfg={cfg} N={N} bad rows {sorted(set(bad[:, 0].tolist()))[:40]} "
                  f"cols {sorted(set(bad[:, 1].tolist()))}", flush=True)
        assert err <= REL_TOL, cfg
