"""GPU parity of the small-M kernel when K is split over workgroups (split-K with a
workspace: partials in fp32, the last workgroup of each column group adds them in split
order and resets its counter).

Splits are forced through MPGEMM_DECODE_SPLIT="S,NW,P" (strips per workgroup, waves per
workgroup, workgroups along K), including splits that do not divide the K tiles evenly.
Bars as in test_gpu_parity: 5e-3 relative to the oracle for random inputs; bit-exact where
every partial sum is exact (the split changes only the summation order).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import (REL_TOL, dev_half, dev_u8, host_bits, pack_case, rel_err, run, say,
                             tol)

pytestmark = pytest.mark.gpu

SPLITS_1 = ["1,1,2", "1,2,2", "2,4,2", "4,1,4", "1,1,7", "2,2,3", "4,4,4"]   # one row block
SPLITS_2 = ["1,2,3", "2,1,5"]                                                  # two row blocks


def _case(M, K, N, seed):
    return workloads.make_case(workloads.LLAMA3_8B_DECODE, M, K, N, seed=seed)


def _forced(M, K, N):
    """The forced split really splits K over workgroups (it needs a workspace)."""
    assert mp.lib().mpgemm_workspace_bytes(M, N, K, 128, 0) > 0


@pytest.mark.parametrize("split", SPLITS_1)
@pytest.mark.parametrize("M", [1, 5, 16])
def test_split_k_matches_oracle(monkeypatch, split, M):
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", split)
    K, N = 2048, 1056                         # 66 strips: ragged strip groups for S = 4
    say(f"split-K {split} M={M} K={K} N={N}")
    _forced(M, K, N)
    case = _case(M, K, N, 100 + M)
    packed = pack_case(case)
    ref = oracle.w4a16(case["x"], case["codes"], case["scales"], case["zeros"], case["group"])
    y = run(case, packed, 1)
    assert rel_err(y, ref, "f16") <= REL_TOL


@pytest.mark.parametrize("split", SPLITS_2)
def test_split_k_two_row_blocks(monkeypatch, split):
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", split)
    M, K, N = 29, 1536, 512
    say(f"split-K {split} M={M}")
    _forced(M, K, N)
    case = _case(M, K, N, 7)
    packed = pack_case(case)
    ref = oracle.w4a16(case["x"], case["codes"], case["scales"], case["zeros"], case["group"])
    assert rel_err(run(case, packed, 2), ref, "f16") <= REL_TOL


@pytest.mark.parametrize("split", ["1,1,2", "2,2,4", "4,2,3"])
def test_split_k_integer_case_bit_exact(monkeypatch, split):
    """X in {-1,0,1}, s = 2^-6: all partial sums exact, so any split gives the oracle's Y."""
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", split)
    M, K, N, g = 16, 2048, 256, 128
    rng = np.random.default_rng(77)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // g, N), dtype=np.uint8)
    scales = np.full((K // g, N), 2.0 ** -6, dtype=np.float16).view(np.uint16)
    _forced(M, K, N)
    case = dict(x=x, codes=codes, scales=scales, zeros=zeros, group=g, dtype="f16")
    packed = pack_case(case)
    say(f"split-K integer {split}")
    assert np.array_equal(run(case, packed, 1), oracle.w4a16(x, codes, scales, zeros, g))


def test_split_k_counters_reset_across_calls_and_shapes(monkeypatch):
    """Repeated and interleaved calls share the cached workspace; every call must see
    zeroed counters and give the same bits as the first call of its shape."""
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", "2,2,4")
    say("split-K repeat")
    a = _case(3, 2048, 512, 1)
    b = _case(16, 1024, 1024, 2)
    _forced(3, 2048, 512)
    _forced(16, 1024, 1024)
    pa, pb = pack_case(a), pack_case(b)
    xa, xb = dev_half(a["x"]), dev_half(b["x"])
    first_a = host_bits(mp.w4a16(xa, pa, config=1))
    first_b = host_bits(mp.w4a16(xb, pb, config=1))
    for _ in range(3):
        ya = mp.w4a16(xa, pa, config=1)
        yb = mp.w4a16(xb, pb, config=1)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(ya), first_a)
        assert np.array_equal(host_bits(yb), first_b)
    ref = oracle.w4a16(a["x"], a["codes"], a["scales"], a["zeros"], a["group"])
    assert rel_err(first_a, ref, "f16") <= REL_TOL


def test_split_k_on_two_streams_at_once():
    """Each stream gets its own cached workspace, so split-K calls that overlap on two
    streams do not share arrival counters: every result equals the one-stream result."""
    say("split-K two streams")
    a = _case(16, 14336, 4096, 3)
    b = _case(1, 14336, 2048, 4)
    _forced(16, 14336, 4096)
    _forced(1, 14336, 2048)
    pa, pb = pack_case(a), pack_case(b)
    xa, xb = dev_half(a["x"]), dev_half(b["x"])
    want_a = host_bits(mp.w4a16(xa, pa))
    want_b = host_bits(mp.w4a16(xb, pb))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for _ in range(8):
        with torch.cuda.stream(s1):
            ya = mp.w4a16(xa, pa)
        with torch.cuda.stream(s2):
            yb = mp.w4a16(xb, pb)
        outs.append((ya, yb))
    torch.cuda.synchronize()
    wa = mp.workspace_for(torch.device("cuda"), 1)
    with torch.cuda.stream(s1):
        w1 = mp.workspace_for(torch.device("cuda"), 1)
    with torch.cuda.stream(s2):
        w2 = mp.workspace_for(torch.device("cuda"), 1)
    assert len({wa.data_ptr(), w1.data_ptr(), w2.data_ptr()}) == 3
    for ya, yb in outs:
        assert np.array_equal(host_bits(ya), want_a)
        assert np.array_equal(host_bits(yb), want_b)
    ref = oracle.w4a16(b["x"], b["codes"], b["scales"], b["zeros"], b["group"], threads=8)
    assert rel_err(want_b, ref, "f16") <= REL_TOL


# Every plan shape, K split over workgroups or not, in both activation formats: each (S, NW)
# is a kernel of its own, with its own pipeline depth and instruction schedule, and bf16
# activations take another operand path (128 + q, less (128 + z) times the group's
# activation sums) than fp16.  Plans that do not fit the row blocks fall back to the
# selector's own, which is then tested once more.  M = 1 and 3 take the activations through
# LDS; 13 and 24 (one and two row blocks) per wave.
PLANS = ["1,1,1", "1,4,1", "1,8,1", "2,1,1", "2,4,1", "2,8,1", "4,2,1", "4,4,1", "4,8,1",
         "2,4,3", "4,4,2"]


@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("M", [1, 3, 13, 24])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_plan_matches_oracle(monkeypatch, plan, M, dtype):
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", plan)
    K, N = 2048, 1056
    wl = workloads.LLAMA3_8B_DECODE if dtype == "f16" else workloads.LLAMA3_70B
    say(f"plan {plan} {dtype} M={M} K={K} N={N}")
    case = workloads.make_case(wl, M, K, N, seed=300 + M)
    packed = pack_case(case)
    ref = oracle.w4a16(case["x"], case["codes"], case["scales"], case["zeros"], case["group"],
                       dtype)
    assert rel_err(run(case, packed, (M + 15) // 16), ref, dtype) <= tol(dtype)


@pytest.mark.parametrize("plan", ["1,4,1", "2,4,1", "2,1,1", "4,4,1", "4,2,2"])
@pytest.mark.parametrize("M", [1, 3, 13])
@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_plan_lowbit_matches_oracle(monkeypatch, plan, M, bits, dtype):
    monkeypatch.setenv("MPGEMM_DECODE_SPLIT", plan)
    K, N, g = 2048, 1056, 64
    say(f"plan {plan} w{bits} {dtype} M={M} K={K} N={N}")
    rng = np.random.default_rng(400 + 10 * M + bits)
    codes = rng.integers(0, 1 << bits, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 1 << bits, (K // g, N), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.05, (K // g, N)).astype(np.float16).view(np.uint16)
    x = workloads.activations(M, K, dtype, 500 + M)
    packed = mp.pack_weights_lowbit(bits, dev_u8(codes), dev_half(scales), dev_u8(zeros), g)
    want = oracle.wlowbit_a16(bits, x, codes, scales, zeros, g, dtype, threads=8)
    y = mp.wlowbit_a16(dev_half(x, dtype), packed, config=1)
    torch.cuda.synchronize()
    assert rel_err(host_bits(y), want, dtype) <= REL_TOL
