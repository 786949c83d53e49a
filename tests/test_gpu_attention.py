"""GPU parity of decode attention over the packed 8-bit and FP8 (E4M3 / E5M2) KV caches,
through the C ABI, against the CPU oracle.

  * the GPU packer writes the same cache bytes as the oracle's (pieces, scattered blocks);
  * outputs over random caches, for head groups of 1 to 16 query heads, head sizes 64 /
    128 / 256, lengths 0 .. 2000 (ragged last blocks), both activation formats, one split
    and forced splits of the block range, within the bar derived from the arithmetic:
    the oracle rounds each dequantized value x_t = (v - z) s to the activation format, the
    kernel rounds each p_t s_t instead (its matrix-core operand), each within a relative
    2^-(f+1) (f = 10 fp16, 7 bf16 fraction bits); so the two pre-rounding sums differ by at
    most 2 * 2^-(f+1) max|x| and each output rounding adds 2^-(f+1) |o| <= 2^-(f+1) max|x|:
    |O - O_ref| <= 4 * 2^-(f+1) * max|x| (fp16 1.95e-3, bf16 7.8e-3).  The bar scales with
    the values, not with |O|, which averaging over many tokens makes small;
    fp16 outputs also meet max|O - O_ref| / max|O_ref| <= 5e-3;
  * one-token contexts give the dequantized value row bit-exact (fp16: p = 1 and the
    value scale enter the matrix cores exactly);
  * tokens past each length never matter (bit-identical output with other contents);
  * table entries outside the cache are skipped without touching other sequences;
  * FP8 caches (no zero points) to the same bars: the same value bar (the kernel rounds
    p_t s_t, the oracle fp8(v) s_t, each once), bit-exact one-token rows, and bytes of the
    packed cache equal to the oracle's with zero bytes in the zero fields.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_mpgemm_amd as mp
import workloads
from test_gpu_parity import REL_TOL, host_bits, say

pytestmark = pytest.mark.gpu


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.view(dtype)


class Cache:
    """A packed cache on the GPU (and the same bytes from the oracle) for B sequences."""

    def __init__(self, kv, lens, Hkv, D, seed, spare=3):
        B = len(lens)
        self.nblk = [(L + 63) // 64 for L in lens]
        self.stride = max(max(self.nblk), 1)
        total = sum(self.nblk) + spare
        perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
        self.table = np.full((B, self.stride), -1, np.int32)
        k = 0
        for b, n in enumerate(self.nblk):
            self.table[b, :n] = perm[k:k + n]
            k += n
        bb = oracle.kv_block_bytes(Hkv, D)
        self.host = np.zeros(total * bb, np.uint8)
        self.gpu = torch.zeros(total * bb, dtype=torch.uint8, device="cuda")
        for b, L in enumerate(lens):
            if L == 0:
                continue
            # FP8 caches have no zero points: the oracle packs zero bytes, the GPU NULL
            parts = [a[b, :L] if a is not None else np.zeros((L, Hkv), np.uint8) for a in kv]
            oracle.kv_pack(self.host, self.table[b], 0, *parts)
            row = dev(self.table[b])
            for t0, t1 in ((0, min(L, 37)), (min(L, 37), L)):      # a prefill, then an append
                if t1 > t0:
                    p = [a[b, t0:t1] if a is not None else None for a in kv]
                    z = (None, None) if p[2] is None else (dev(p[2]), dev(p[5]))
                    mp.kv_pack(self.gpu, row, t0, dev(p[0]), dev(p[1].view(np.int16), torch.float16),
                               z[0], dev(p[3]), dev(p[4].view(np.int16), torch.float16), z[1])


def run(q_bits, cache, lens, Hkv, scale, dtype, max_len=None, fp8=None):
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    q = dev(q_bits.view(np.int16), tdt)
    args = (q, cache.gpu, dev(cache.table), dev(np.asarray(lens, np.int32)), Hkv,
            max(lens) if max_len is None else max_len, scale)
    if fp8 is None:
        o = mp.attention_decode_kv8(*args)
    else:
        o = mp.attention_decode_kvfp8(*args, fp8_format=fp8)
    torch.cuda.synchronize()
    return host_bits(o)


VALUE_BAR = {"f16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}


def rel(y, ref, dtype):
    conv = oracle.f16_bits_to_f64 if dtype == "f16" else oracle.bf16_bits_to_f64
    a, r = conv(y), conv(ref)
    assert np.isfinite(a).all()
    return float(np.abs(a - r).max() / max(np.abs(r).max(), 1e-30))


def within_value_bar(y, ref, kv, lens, dtype, fp8=None):
    """max|O - O_ref| <= 4 * 2^-(f+1) * max|x| over the sequences' live values."""
    conv = oracle.f16_bits_to_f64 if dtype == "f16" else oracle.bf16_bits_to_f64
    _, _, _, vc, vs, vz = kv
    table = None if fp8 is None else oracle.fp8_to_f64(np.arange(256, dtype=np.uint8), fp8)
    xmax = 0.0
    for b, L in enumerate(lens):
        if L:
            v = vc[b, :L].astype(np.float64) - vz[b, :L, :, None] if fp8 is None else table[vc[b, :L]]
            x = v * vs[b, :L].view(np.float16).astype(np.float64)[..., None]
            xmax = max(xmax, float(np.abs(x).max()))
    err = float(np.abs(conv(y) - conv(ref)).max())
    assert np.isfinite(conv(y)).all()
    return err <= VALUE_BAR[dtype] * xmax, (err, xmax)


def case(B, Hq, Hkv, D, lens, dtype, seed):
    T = max(max(lens), 1)
    kv = workloads.kv_cache(B, T, Hkv, D, seed)
    q = workloads.queries(B, Hq, D, dtype, seed + 1)
    return kv, q


@pytest.mark.parametrize("D", [64, 128])
def test_kv_pack_matches_oracle_bytes(D):
    lens, Hkv = [150, 64, 1], 2
    kv, _ = case(3, 4, Hkv, D, lens, "f16", D)
    c = Cache(kv, lens, Hkv, D, 5)
    assert np.array_equal(c.gpu.cpu().numpy(), c.host)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 1, 64), (8, 2, 256),
                                      (64, 8, 128)])
@pytest.mark.parametrize("bps", [None, "1", "3"])
def test_attention_matches_oracle(dtype, Hq, Hkv, D, bps, monkeypatch):
    if bps:
        monkeypatch.setenv("MPGEMM_ATTN_BPS", bps)
    lens = [1, 63, 64, 65, 300, 1000, 0, 129]
    kv, q = case(len(lens), Hq, Hkv, D, lens, dtype, Hq + D)
    c = Cache(kv, lens, Hkv, D, 7)
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"attention {dtype} Hq={Hq} Hkv={Hkv} D={D} bps={bps}")
    y = run(q, c, lens, Hkv, scale, dtype)
    want = oracle.attention_decode_kv8(q, *kv, lens, scale, dtype)
    assert (y[6] == 0).all() and (want[6] == 0).all()        # empty context
    ok, detail = within_value_bar(y, want, kv, lens, dtype)
    assert ok, detail
    if dtype == "f16":
        assert rel(y, want, dtype) <= REL_TOL


@pytest.mark.parametrize("bps", [None, "1"])
def test_long_context_llama3_8b_heads(bps, monkeypatch):
    if bps:
        monkeypatch.setenv("MPGEMM_ATTN_BPS", bps)
    lens = [2000, 1777, 64, 3]
    kv, q = case(4, 32, 8, 128, lens, "f16", 21)
    c = Cache(kv, lens, 8, 128, 22)
    say(f"attention long bps={bps}")
    y = run(q, c, lens, 8, 0.0883883461356163, "f16")
    want = oracle.attention_decode_kv8(q, *kv, lens, 0.0883883461356163, "f16")
    assert within_value_bar(y, want, kv, lens, "f16")[0]
    assert rel(y, want, "f16") <= REL_TOL


def test_one_token_context_gives_the_value_row_bit_exact():
    lens, Hq, Hkv, D = [1, 1, 1], 8, 2, 128
    kv, q = case(3, Hq, Hkv, D, lens, "f16", 31)
    c = Cache(kv, lens, Hkv, D, 32)
    y = run(q, c, lens, Hkv, 0.1, "f16")
    assert np.array_equal(y, oracle.attention_decode_kv8(q, *kv, lens, 0.1, "f16"))


def test_tokens_past_the_length_never_matter():
    lens, Hq, Hkv, D = [70, 5], 8, 2, 128
    kv, q = case(2, Hq, Hkv, D, [128, 128], "f16", 41)
    c1 = Cache(kv, [128, 128], Hkv, D, 42)
    y1 = run(q, c1, lens, Hkv, 0.1, "f16", max_len=128)
    kv2 = [a.copy() for a in kv]
    rng = np.random.default_rng(43)
    for b, L in enumerate(lens):
        for a in kv2:
            a[b, L:] = rng.integers(0, 256, a[b, L:].shape).astype(a.dtype)
    c2 = Cache(kv2, [128, 128], Hkv, D, 42)
    assert np.array_equal(run(q, c2, lens, Hkv, 0.1, "f16", max_len=128), y1)
    assert rel(y1, oracle.attention_decode_kv8(q, *kv, lens, 0.1, "f16"), "f16") <= REL_TOL


def test_table_entries_outside_the_cache_are_skipped():
    lens, Hq, Hkv, D = [200, 130], 8, 2, 128
    kv, q = case(2, Hq, Hkv, D, lens, "f16", 51)
    c = Cache(kv, lens, Hkv, D, 52)
    c.table[0, 1] = 10 ** 6                                  # sequence 0: a bad entry
    y = run(q, c, lens, Hkv, 0.1, "f16")
    want = oracle.attention_decode_kv8(q, *kv, lens, 0.1, "f16")
    assert np.isfinite(oracle.f16_bits_to_f64(y[0])).all()
    assert rel(y[1:], want[1:], "f16") <= REL_TOL


def test_attention_leaves_the_gemm_workspace_zero():
    """The GEMM's cached workspace holds split-K counters that must stay zero between
    calls; attention partials use a workspace of their own."""
    lens = [1000] * 4
    kv, q = case(4, 32, 8, 128, lens, "f16", 61)
    c = Cache(kv, lens, 8, 128, 62)
    ws = mp.workspace_for(torch.device("cuda"), 1 << 20)
    run(q, c, lens, 8, 0.1, "f16")
    assert int(ws[:256 * 1024].count_nonzero()) == 0          # the arrival counters


# ------------------------------------------------------------------ FP8 KV cache ----------

def case_fp8(B, Hq, Hkv, D, lens, dtype, fmt, seed):
    kv = workloads.kv_cache_fp8(B, max(max(lens), 1), Hkv, D, fmt, seed)
    return kv, workloads.queries(B, Hq, D, dtype, seed + 1)


def fp8_ref(q, kv, lens, scale, fmt, dtype):
    kc, ks, _, vc, vs, _ = kv
    return oracle.attention_decode_kvfp8(q, kc, ks, vc, vs, lens, scale, fmt, dtype)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_kvfp8_pack_matches_oracle_bytes(fmt):
    lens, Hkv, D = [150, 64, 1], 2, 128
    kv, _ = case_fp8(3, 4, Hkv, D, lens, "f16", fmt, 3)
    c = Cache(kv, lens, Hkv, D, 5)
    assert np.array_equal(c.gpu.cpu().numpy(), c.host)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 1, 64), (8, 2, 256)])
@pytest.mark.parametrize("bps", [None, "1"])
def test_kvfp8_attention_matches_oracle(fmt, dtype, Hq, Hkv, D, bps, monkeypatch):
    if bps:
        monkeypatch.setenv("MPGEMM_ATTN_BPS", bps)
    lens = [1, 63, 64, 65, 300, 1000, 0, 129]
    kv, q = case_fp8(len(lens), Hq, Hkv, D, lens, dtype, fmt, Hq + D + len(fmt))
    c = Cache(kv, lens, Hkv, D, 7)
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"attention fp8 {fmt} {dtype} Hq={Hq} Hkv={Hkv} D={D} bps={bps}")
    y = run(q, c, lens, Hkv, scale, dtype, fp8=fmt)
    want = fp8_ref(q, kv, lens, scale, fmt, dtype)
    assert (y[6] == 0).all() and (want[6] == 0).all()        # empty context
    ok, detail = within_value_bar(y, want, kv, lens, dtype, fp8=fmt)
    assert ok, detail
    if dtype == "f16":
        assert rel(y, want, dtype) <= REL_TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_kvfp8_one_token_context_gives_the_value_row_bit_exact(fmt):
    lens, Hq, Hkv, D = [1, 1, 1], 8, 2, 128
    kv, q = case_fp8(3, Hq, Hkv, D, lens, "f16", fmt, 71)
    c = Cache(kv, lens, Hkv, D, 72)
    y = run(q, c, lens, Hkv, 0.1, "f16", fp8=fmt)
    assert np.array_equal(y, fp8_ref(q, kv, lens, 0.1, fmt, "f16"))


def test_kvfp8_long_context_llama3_8b_heads():
    lens = [2000, 1777, 64, 3]
    kv, q = case_fp8(4, 32, 8, 128, lens, "f16", "e4m3", 81)
    c = Cache(kv, lens, 8, 128, 82)
    say("attention fp8 long")
    y = run(q, c, lens, 8, 0.0883883461356163, "f16", fp8="e4m3")
    want = fp8_ref(q, kv, lens, 0.0883883461356163, "e4m3", "f16")
    assert within_value_bar(y, want, kv, lens, "f16", fp8="e4m3")[0]
    assert rel(y, want, "f16") <= REL_TOL


def test_kvfp8_rejects_an_unknown_format():
    lens = [5]
    kv, q = case_fp8(1, 8, 2, 128, lens, "f16", "e4m3", 91)
    c = Cache(kv, lens, 2, 128, 92)
    q_t = dev(q.view(np.int16), torch.float16)
    with pytest.raises(ValueError):
        mp.attention_decode_kvfp8(q_t, c.gpu, dev(c.table), dev(np.asarray(lens, np.int32)), 2, 5,
                                  0.1, fp8_format="e3m4")
    st = mp.lib().mpgemm_attention_decode_kvfp8(
        q_t.data_ptr(), 0, 7, c.gpu.data_ptr(), c.gpu.numel() // mp.kv_block_bytes(2, 128),
        dev(c.table).data_ptr(), c.table.shape[1], dev(np.asarray(lens, np.int32)).data_ptr(), 1, 8,
        2, 128, 5, 0.1, q_t.data_ptr(), None, 0, None)
    assert st != 0


# ----------------------------------------------------- head sizes padded to 64 --------

@pytest.mark.parametrize("D", [48, 96, 160])
def test_kv_pack_of_padded_heads_matches_oracle_bytes(D):
    lens, Hkv = [150, 7], 2
    kv, _ = case(2, 4, Hkv, D, lens, "f16", D + 1)
    c = Cache(kv, lens, Hkv, D, 9)
    assert np.array_equal(c.gpu.cpu().numpy(), c.host)


@pytest.mark.parametrize("D", [16, 80, 96, 112, 176, 192, 208])
@pytest.mark.parametrize("kvfmt", [None, "e4m3"])
@pytest.mark.parametrize("bps", [None, "1"])
def test_attention_head_sizes_padded_to_64(D, kvfmt, bps, monkeypatch):
    if bps:
        monkeypatch.setenv("MPGEMM_ATTN_BPS", bps)
    lens, Hq, Hkv = [1, 64, 65, 700, 0, 130], 16, 4
    seed = 100 + D
    if kvfmt is None:
        kv, q = case(len(lens), Hq, Hkv, D, lens, "f16", seed)
    else:
        kv, q = case_fp8(len(lens), Hq, Hkv, D, lens, "f16", kvfmt, seed)
    c = Cache(kv, lens, Hkv, D, seed + 1)
    scale = float(np.float32(1 / np.sqrt(D)))
    say(f"attention D={D} kv={kvfmt or 'u8'} bps={bps}")
    y = run(q, c, lens, Hkv, scale, "f16", fp8=kvfmt)
    want = (oracle.attention_decode_kv8(q, *kv, lens, scale, "f16") if kvfmt is None
            else fp8_ref(q, kv, lens, scale, kvfmt, "f16"))
    assert (y[4] == 0).all()
    ok, detail = within_value_bar(y, want, kv, lens, "f16", fp8=kvfmt)
    assert ok, detail
    assert rel(y, want, "f16") <= REL_TOL


def test_one_token_context_is_bit_exact_for_a_padded_head():
    lens, Hq, Hkv, D = [1, 1], 8, 2, 80
    kv, q = case(2, Hq, Hkv, D, lens, "f16", 33)
    c = Cache(kv, lens, Hkv, D, 34)
    y = run(q, c, lens, Hkv, 0.1, "f16")
    assert np.array_equal(y, oracle.attention_decode_kv8(q, *kv, lens, 0.1, "f16"))
