"""GPU parity at the largest shapes the C ABI accepts: (M + 128) * Kp, Kp * Np and M * Np
each just below 2^31 (the kernels address planes with 32-bit byte offsets).  Inputs are
drawn on the GPU by a seeded generator (workloads.device_case); the oracle computes
sampled rows x columns from the same input bits, to the random-input bar
(max|Y - Y_ref| / max|Y_ref| <= 5e-3)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, host_bits, rel_err, say

pytestmark = pytest.mark.gpu

LIMIT = 1 << 31


def check(M, K, N, configs, rows, cols, seed):
    assert (M + 128) * K < LIMIT and K * N < LIMIT and M * N < LIMIT
    x, codes, scales, zeros = workloads.device_case(M, K, N, 128, seed, "cuda")
    packed = mp.pack_weights(codes, scales, zeros, 128)
    rows_t = torch.as_tensor(rows, device="cuda")
    cols_t = torch.as_tensor(cols, device="cuda")
    want = oracle.w4a16(host_bits(x[rows_t]), codes[:, cols_t].cpu().numpy(),
                        host_bits(scales[:, cols_t]), zeros[:, cols_t].cpu().numpy(), 128, "f16",
                        threads=8)
    del codes
    for cfg in configs:
        say(f"limits M={M} K={K} N={N} config={cfg}")
        y = mp.w4a16(x, packed, config=cfg)
        got = host_bits(y[rows_t][:, cols_t].contiguous())
        del y
        assert rel_err(got, want, "f16") <= REL_TOL, cfg


def test_largest_m_at_k16384():
    K, N = 16384, 256
    M = LIMIT // K - 129                     # (M + 128) * K = 2^31 - 16384
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, M - 1, M - 2, M // 2], rng.choice(M, 8, replace=False)]))
    check(M, K, N, [0, 12, 13, 14], rows, np.arange(N), 11)


def test_largest_n_at_k16384():
    K, M = 16384, 3
    N = LIMIT // K - 16                      # Kp * Np = 2^31 - 16 K
    rng = np.random.default_rng(2)
    cols = np.unique(np.concatenate([[0, N - 1, N - 16], rng.choice(N, 61, replace=False)]))
    check(M, K, N, [0, 1], np.arange(M), cols, 12)


def test_longest_k():
    N = 16
    K = (LIMIT // 129 - 1) // 128 * 128      # (1 + 128) * K just below 2^31
    check(1, K, N, [0, 1], np.arange(1), np.arange(N), 13)
