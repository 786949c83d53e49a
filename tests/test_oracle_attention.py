"""Pins for the oracle's decode attention over an 8-bit KV cache and its packed KV layout,
each against something other than the oracle itself:
  * one token: the output is that token's dequantized value row, rounded once (exact
    rationals through Python's binary16 packer);
  * a zero query: uniform weights, so the output is the mean of the value rows (exact when
    the length is a power of two);
  * two tokens: the closed form (v0 + e^(s1-s0) v1) / (1 + e^(s1-s0));
  * grouped-query heads read KV head h // (Hq / Hkv); tokens past the length never matter;
    scaling q by 2 and the softmax scale by 1/2 changes nothing; token order does not
    matter; an empty context gives zeros;
  * the KV layout: K codes of a block are the 8-bit weight packing of K^T (d x token),
    V codes that of V (token x d) -- both layouts pinned elsewhere; pack/unpack round trip.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f16(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def f16_val(b) -> Fraction:
    return Fraction(float(np.uint16(b).view(np.float16)))


def rand_kv(B, T, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 256, (B, T, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (B, T, Hkv, D), dtype=np.uint8)
    ks = rng.uniform(0.005, 0.02, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    vs = rng.uniform(0.005, 0.02, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    kz = rng.integers(100, 156, (B, T, Hkv), dtype=np.uint8)
    vz = rng.integers(100, 156, (B, T, Hkv), dtype=np.uint8)
    return kc, ks, kz, vc, vs, vz


def rand_q(B, Hq, D, seed):
    return np.random.default_rng(seed).standard_normal((B, Hq, D)).astype(np.float16).view(np.uint16)


def att(q, kv, lens, scale, dtype="f16"):
    return oracle.attention_decode_kv8(q, *kv, lens, scale, dtype)


def test_single_token_gives_its_value_row():
    B, T, Hkv, Hq, D = 2, 3, 2, 4, 64
    kv = rand_kv(B, T, Hkv, D, 1)
    o = att(rand_q(B, Hq, D, 2), kv, [1, 1], 0.125)
    _, _, _, vc, vs, vz = kv
    for b in range(B):
        for h in range(Hq):
            j = h // 2
            want = [f16(float((int(vc[b, 0, j, d]) - int(vz[b, 0, j])) * f16_val(vs[b, 0, j])))
                    for d in range(D)]
            assert o[b, h].tolist() == want


@pytest.mark.parametrize("L", [1, 2, 8, 64])
def test_zero_query_averages_the_value_rows(L):
    B, Hkv, Hq, D = 1, 1, 2, 64
    kv = rand_kv(B, 70, Hkv, D, L)
    q = np.zeros((B, Hq, D), np.uint16)
    o = att(q, kv, [L], 0.1)
    _, _, _, vc, vs, vz = kv
    for d in range(D):
        vals = [f16_val(f16(float((int(vc[0, t, 0, d]) - int(vz[0, t, 0])) * f16_val(vs[0, t, 0]))))
                for t in range(L)]
        assert o[0, 0, d] == o[0, 1, d] == f16(float(sum(vals) / L)), d


def test_two_tokens_closed_form():
    D = 64
    kc = np.zeros((1, 2, 1, D), np.uint8)
    kz = np.zeros((1, 2, 1), np.uint8)
    kc[0, 0, 0, 0], kc[0, 1, 0, 0] = 10, 40                  # k_t[0] = code * 2^-4
    ks = np.full((1, 2, 1), 2.0 ** -4, np.float16).view(np.uint16)
    rng = np.random.default_rng(3)
    vc = rng.integers(0, 256, (1, 2, 1, D), dtype=np.uint8)
    vz = np.full((1, 2, 1), 128, np.uint8)
    vs = np.full((1, 2, 1), 2.0 ** -5, np.float16).view(np.uint16)
    q = np.zeros((1, 1, D), np.uint16)
    q[0, 0, 0] = f16(0.75)
    scale = 0.5
    o = att(q, (kc, ks, kz, vc, vs, vz), [2], scale)
    s0, s1 = 0.75 * 10 / 16 * scale, 0.75 * 40 / 16 * scale
    w1 = math.exp(s1 - s0)
    for d in range(D):
        v0 = (int(vc[0, 0, 0, d]) - 128) / 32
        v1 = (int(vc[0, 1, 0, d]) - 128) / 32
        want = (v0 + w1 * v1) / (1 + w1)
        got = float(np.uint16(o[0, 0, d]).view(np.float16))
        assert abs(got - want) <= 2.0 ** -10 * max(abs(want), 2.0 ** -14), d


def test_grouped_query_heads_read_their_kv_head():
    B, T, Hkv, Hq, D = 1, 16, 2, 8, 64
    kc, ks, kz, vc, vs, vz = rand_kv(B, T, Hkv, D, 4)
    vc[:, :, 0, :], vc[:, :, 1, :] = 20, 60                 # head j's values all equal
    vz[:] = 0
    vs[:] = np.float16(2.0 ** -4).view(np.uint16)
    o = att(rand_q(B, Hq, D, 5), (kc, ks, kz, vc, vs, vz), [T], 0.1)
    vals = np.asarray(o).view(np.float16).astype(np.float64)
    assert (vals[0, :4] == 20 / 16).all() and (vals[0, 4:] == 60 / 16).all()


def test_tokens_past_the_length_are_ignored():
    B, T, Hkv, Hq, D = 2, 40, 2, 4, 128
    kv = list(rand_kv(B, T, Hkv, D, 6))
    q = rand_q(B, Hq, D, 7)
    lens = [17, 33]
    o = att(q, kv, lens, 0.088)
    rng = np.random.default_rng(8)
    for b, L in enumerate(lens):
        for a in kv:
            a[b, L:] = rng.integers(0, 256, a[b, L:].shape).astype(a.dtype)
    assert np.array_equal(att(q, kv, lens, 0.088), o)


def test_scaling_q_up_and_the_softmax_scale_down_changes_nothing():
    B, T, Hkv, Hq, D = 1, 24, 1, 2, 64
    kv = rand_kv(B, T, Hkv, D, 9)
    q = rand_q(B, Hq, D, 10)
    q2 = (q.view(np.float16) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(att(q, kv, [T], 0.1), att(q2, kv, [T], 0.05))


def test_token_order_does_not_matter():
    B, T, Hkv, Hq, D = 1, 32, 1, 2, 64
    kv = rand_kv(B, T, Hkv, D, 11)
    q = rand_q(B, Hq, D, 12)
    perm = np.random.default_rng(13).permutation(T)
    kv2 = [a[:, perm] for a in kv]
    a = np.asarray(att(q, kv, [T], 0.125)).view(np.float16).astype(np.float64)
    b = np.asarray(att(q, kv2, [T], 0.125)).view(np.float16).astype(np.float64)
    assert np.abs(a - b).max() <= 2.0 ** -10 * np.abs(a).max()


def test_empty_context_gives_zeros():
    kv = rand_kv(1, 4, 1, 64, 14)
    o = att(rand_q(1, 2, 64, 15), kv, [0], 0.1)
    assert (o == 0).all()


def test_value_dequantization_is_exact_at_power_of_two_scales():
    D = 256
    vc = np.arange(256, dtype=np.uint8).reshape(1, 1, 1, D)
    kc = np.zeros((1, 1, 1, D), np.uint8)
    for z, e in ((0, -3), (128, -6), (255, -8)):
        vz = np.full((1, 1, 1), z, np.uint8)
        vs = np.full((1, 1, 1), 2.0 ** e, np.float16).view(np.uint16)
        ks = np.full((1, 1, 1), 1.0, np.float16).view(np.uint16)
        o = att(rand_q(1, 1, D, 16), (kc, ks, np.zeros_like(vz), vc, vs, vz), [1], 0.1)
        vals = np.asarray(o).view(np.float16).astype(np.float64)[0, 0]
        assert np.array_equal(vals, (np.arange(256) - z) * 2.0 ** e)


# ------------------------------------------------------------------- the KV layout ---

def unpadded(packed, K, N):
    """The 8-bit weight packing of a K x N matrix with K % 64 == 0 but not padded to 128
    rows: the packer pads each 16-column strip to a multiple of 128 rows, so the unpadded
    strip is the first K / 64 of its 1 KiB tiles."""
    per = -(-K // 128) * 2
    strips = [packed[(s * per) * 1024:(s * per + K // 64) * 1024] for s in range(N // 16)]
    return np.concatenate(strips)


@pytest.mark.parametrize("D", [64, 128])
def test_kv_block_is_the_weight_packing_of_k_transposed_and_v(D):
    Hkv = 2
    kc, ks, kz, vc, vs, vz = [a[0] for a in rand_kv(1, 64, Hkv, D, D)]
    HB = 128 * D + 384
    cache = np.zeros(oracle.kv_block_bytes(Hkv, D), np.uint8)
    oracle.kv_pack(cache, [0], 0, kc, ks, kz, vc, vs, vz)
    assert cache.size == Hkv * HB
    for h in range(Hkv):
        hb = cache[h * HB:(h + 1) * HB]
        kT, _ = oracle.pack_w8(np.ascontiguousarray(kc[:, h, :].T),
                               np.zeros((-(-D // 64), 64), np.uint16), None, 64)
        vp, _ = oracle.pack_w8(np.ascontiguousarray(vc[:, h, :]), np.zeros((1, D), np.uint16),
                               None, 64)
        assert np.array_equal(hb[:64 * D], unpadded(kT, D, 64))
        assert np.array_equal(hb[64 * D:128 * D], unpadded(vp, 64, D))
        meta = hb[128 * D:]
        assert np.array_equal(meta[:128].view(np.uint16), ks[:, h])
        assert np.array_equal(meta[128:256].view(np.uint16), vs[:, h])
        assert np.array_equal(meta[256:320], kz[:, h]) and np.array_equal(meta[320:], vz[:, h])


def test_kv_pack_in_pieces_through_a_block_table_round_trips():
    Hkv, D, T = 2, 128, 150
    kv = [a[0] for a in rand_kv(1, T, Hkv, D, 17)]
    table = np.array([5, 2, 7], np.int32)                    # 3 blocks, scattered
    cache = np.zeros(8 * oracle.kv_block_bytes(Hkv, D), np.uint8)
    for t0, t1 in ((0, 1), (1, 70), (70, 128), (128, 150)):   # prefill, then appends
        oracle.kv_pack(cache, table, t0, *[a[t0:t1] for a in kv])
    back = oracle.kv_unpack(cache, table, T, Hkv, D)
    for a, b in zip(kv, back):
        assert np.array_equal(a, b)
    untouched = [i for i in range(8) if i not in table]
    bb = oracle.kv_block_bytes(Hkv, D)
    assert all((cache[i * bb:(i + 1) * bb] == 0).all() for i in untouched)


@pytest.mark.parametrize("D", [16, 48, 80, 96, 112, 160, 192, 208])
def test_kv_head_of_any_multiple_of_16_is_stored_as_the_zero_padded_head(D):
    """A head of D values is laid out exactly as the head zero-padded to the next multiple
    of 64 (the k depth of one 8-bit tile), and unpacks back to the D values."""
    Hkv, T = 2, 70
    Dp = -(-D // 64) * 64
    kv = [a[0] for a in rand_kv(1, T, Hkv, D, D + 3)]
    assert oracle.kv_block_bytes(Hkv, D) == Hkv * (128 * Dp + 384)
    table = np.array([1, 0], np.int32)
    cache = np.full(2 * oracle.kv_block_bytes(Hkv, D), 0xAB, np.uint8)
    oracle.kv_pack(cache, table, 0, *kv)
    pad = [np.pad(a, ((0, 0), (0, 0), (0, Dp - D))) if a.ndim == 3 else a for a in kv]
    want = np.full(2 * oracle.kv_block_bytes(Hkv, Dp), 0xAB, np.uint8)
    oracle.kv_pack(want, table, 0, *pad)
    assert np.array_equal(cache, want)
    for x, y in zip(kv, oracle.kv_unpack(cache, table, T, Hkv, D)):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("D", [48, 96])
def test_attention_of_a_head_equals_that_of_the_zero_padded_head(D):
    """Zero query elements and any values past D change no score, and value columns past D
    feed only outputs past D: the outputs are the padded head's first D, bit for bit."""
    B, Hq, Hkv, T = 2, 8, 2, 90
    Dp = -(-D // 64) * 64
    kc, ks, kz, vc, vs, vz = rand_kv(B, T, Hkv, D, D + 5)
    q = rand_q(B, Hq, D, D + 6)
    lens = [90, 33]
    o = oracle.attention_decode_kv8(q, kc, ks, kz, vc, vs, vz, lens, 0.125)
    padc = lambda a: np.pad(a, ((0, 0), (0, 0), (0, 0), (0, Dp - D)))
    qp = np.pad(q, ((0, 0), (0, 0), (0, Dp - D)))
    op = oracle.attention_decode_kv8(qp, padc(kc), ks, kz, padc(vc), vs, vz, lens, 0.125)
    assert np.array_equal(o, op[..., :D])


# ------------------------------------------------------------- FP8 KV cache ---------

import torch  # noqa: E402

FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def fp8_value(code, fmt) -> Fraction:
    t = torch.tensor([int(code)], dtype=torch.uint8).view(FP8[fmt])
    return Fraction(float(t.to(torch.float64)[0]))


def finite_fp8(shape, fmt, seed):
    rng = np.random.default_rng(seed)
    v = np.clip(rng.standard_normal(shape).astype(np.float32) * 2, -400, 400)
    return torch.from_numpy(v).to(FP8[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_single_token_gives_its_value_row(fmt):
    B, T, Hkv, Hq, D = 1, 2, 2, 4, 64
    kc, vc = finite_fp8((B, T, Hkv, D), fmt, 1), finite_fp8((B, T, Hkv, D), fmt, 2)
    ks = np.full((B, T, Hkv), 0.5, np.float16).view(np.uint16)
    vs = np.random.default_rng(3).uniform(0.01, 0.1, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    q = rand_q(B, Hq, D, 4)
    o = oracle.attention_decode_kvfp8(q, kc, ks, vc, vs, [1], 0.1, fmt)
    for h in range(Hq):
        j = h // 2
        want = [f16(float(fp8_value(vc[0, 0, j, d], fmt) * f16_val(vs[0, 0, j]))) for d in range(D)]
        assert o[0, h].tolist() == want


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_zero_query_averages_the_value_rows(fmt):
    L, D = 8, 64
    kc, vc = finite_fp8((1, L, 1, D), fmt, 5), finite_fp8((1, L, 1, D), fmt, 6)
    ks = np.full((1, L, 1), 1.0, np.float16).view(np.uint16)
    vs = np.full((1, L, 1), 0.25, np.float16).view(np.uint16)
    o = oracle.attention_decode_kvfp8(np.zeros((1, 1, D), np.uint16), kc, ks, vc, vs, [L], 0.1, fmt)
    for d in range(D):
        vals = [f16_val(f16(float(fp8_value(vc[0, t, 0, d], fmt) / 4))) for t in range(L)]
        assert o[0, 0, d] == f16(float(sum(vals) / L))


def test_fp8_formats_differ_and_match_the_integer_cache_on_shared_values():
    """Codes whose E4M3 value is an integer v: the FP8 cache with scale s equals the 8-bit
    cache with codes v + 128, zero 128 and the same scale."""
    B, T, Hkv, Hq, D = 1, 20, 1, 2, 64
    rng = np.random.default_rng(7)
    ints = rng.integers(-16, 17, (B, T, Hkv, D))
    codes = torch.from_numpy(ints.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ks = rng.uniform(0.01, 0.05, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    vs = rng.uniform(0.01, 0.05, (B, T, Hkv)).astype(np.float16).view(np.uint16)
    q = rand_q(B, Hq, D, 8)
    a = oracle.attention_decode_kvfp8(q, codes, ks, codes, vs, [T], 0.1, "e4m3")
    u8 = (ints + 128).astype(np.uint8)
    z = np.full((B, T, Hkv), 128, np.uint8)
    b = oracle.attention_decode_kv8(q, u8, ks, z, u8, vs, z, [T], 0.1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, oracle.attention_decode_kvfp8(q, codes, ks, codes, vs, [T], 0.1, "e5m2"))
