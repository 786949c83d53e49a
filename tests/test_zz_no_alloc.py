"""The allocation-free entry point (mpgemm_w4a16_noalloc) against mpgemm_w4a16.

Both run the same kernels, and given the same workspace size they split K the same way, so
the allocation-free call must return mpgemm_w4a16's output bit for bit, and meet the
oracle's bar (max|Y - Y_ref| / max|Y_ref| <= 5e-3).  Each case makes two allocation-free
calls in a row on one GPU, the second on a smaller problem, so the second call runs on the
static buffer as the first call left it.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, dev_half, host_bits, pack_case, say, to_f64

pytestmark = pytest.mark.gpu

WL = {w.name: w for w in workloads.ALL_WORKLOADS}


def noalloc_via_abi(x, packed):
    """mpgemm_w4a16_noalloc called through the C ABI (ctypes), no binding logic."""
    M, K = x.shape
    y = torch.empty((M, packed.N), dtype=x.dtype, device=x.device)
    vp = ctypes.c_void_p
    st = mp.lib().mpgemm_w4a16_noalloc(
        vp(x.data_ptr()), 0 if x.dtype == torch.float16 else 1, vp(packed.codes.data_ptr()),
        vp(packed.meta.data_ptr()), M, packed.N, K, packed.group, int(packed.symmetric),
        vp(y.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
    assert st == 0, mp.lib().mpgemm_status_string(st).decode()
    return y


PAIRS = [
    # the small-M kernel splitting K over workgroups (counters and partials), then a
    # smaller one that splits too
    (("llama3_8b_decode", 16, 14336, 4096), ("llama3_8b_decode", 1, 14336, 2048)),
    # the tiled kernel with all 256 parts of a split grid (32 MiB of partials: the whole
    # buffer), then a smaller split grid
    (("llama3_70b", 256, 8192, 4096), ("llama3_8b_prefill", 130, 2048, 512)),
    # symmetric g = 64 decode split, then a tiled split
    (("qwen3_32b", 16, 25600, 5120), ("llama3_8b_prefill", 128, 4096, 1024)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][1]}x{p[0][2]}x{p[0][3]}")
def test_noalloc_matches_the_allocating_entry_point_on_two_calls(pair):
    cases, want, x, packed = [], [], [], []
    for name, M, K, N in pair:
        case = workloads.make_case(WL[name], M, K, N)
        cases.append(case)
        packed.append(pack_case(case))
        x.append(dev_half(case["x"], case["dtype"]))
        want.append(host_bits(mp.w4a16(x[-1], packed[-1])))
    say(f"noalloc {pair[0]} then {pair[1]}")
    y0 = noalloc_via_abi(x[0], packed[0])
    y1 = noalloc_via_abi(x[1], packed[1])           # second call, smaller problem
    got = [host_bits(y0), host_bits(y1)]
    for case, g, w in zip(cases, got, want):
        assert np.array_equal(g, w), (case["M"], case["K"], case["N"])
        rows = np.unique(np.linspace(0, case["M"] - 1, min(case["M"], 6)).astype(int))
        ref = oracle.w4a16_f64(case["x"][rows], case["codes"], case["scales"], case["zeros"],
                               case["group"], case["dtype"])
        yv = to_f64(g[rows], case["dtype"])
        err = float(np.abs(yv - ref).max() / np.abs(ref).max())
        assert err <= REL_TOL, err
    # the binding's wrapper takes the same path
    assert np.array_equal(host_bits(mp.w4a16_noalloc(x[1], packed[1])), want[1])
