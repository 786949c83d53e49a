// Device-side building blocks shared by the gfx950 kernels of libmpgemm.
//
// Source: "LMDeploy Accelerates Mixed-Precision LLM Inference with TurboMind"
// (arXiv 2508.15601), abbreviated [TurboMind].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mpgemm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum Act { kF16 = 0, kBF16 = 1 };

// Formats of the packed codes plane: 2-, 3-, 4- and 8-bit unsigned integers with a group
// zero point, or 8-bit OCP floating point (E4M3, E5M2) with a group scale only.
enum Code { kU4 = 0, kU8 = 1, kE4M3 = 2, kE5M2 = 3, kU2 = 4, kU3 = 5 };
template <int CODE>
constexpr int kCodeBits = CODE == kU4 ? 4 : (CODE == kU2 ? 2 : (CODE == kU3 ? 3 : 8));
template <int CODE>
constexpr bool kCodeFp8 = CODE == kE4M3 || CODE == kE5M2;

// Packed layout v1 (include/mpgemm.h): 16 columns x 128 k per 1 KiB tile, 16 bytes per lane.
constexpr int kTileK = 128;
constexpr int kTileN = 16;
constexpr int kTileWords = 256;  // 32-bit words per tile

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &v) {
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, v);
}

// ---------------------------------------------------------------- I2F dequantization --
//
// [TurboMind, Fig. 6 caption and the interleave diagram beside Fig. 24]: a packed word
// holds elements e0..e7 of one column at nibbles (LSB first) e0 e2 e4 e6 e1 e3 e5 e7, so
// "isolate" with the mask 0x000F000F leaves e0 in the low and e1 in the high half of a
// 32-bit register -- the (k, k+1) register order of the MFMA operand.  OR-ing the fp16
// pattern 0x6400 (1024.0, spacing 1) into each half turns a 4-bit q into 1024 + q exactly.
// The next nibble pair (e2, e3) sits 4 bits higher; OR-ing 0x5400 (64.0, spacing 1/16)
// reads it as 64 + q exactly, so it needs no shift.  One 8-bit shift exposes (e4, e5) and
// (e6, e7) the same way: four isolate-and-combine operations and one shift per 8 weights.

// (v & mask) | bits as one v_and_or_b32, with the mask in a scalar and the OR pattern in a
// vector register: VOP3 on gfx9 takes no literal and reads at most one scalar register, and
// given the constants themselves the compiler splits the operation into two
// literal-carrying VOP2s.  The empty statements only pin each constant to a register class;
// the operation stays the compiler's own, so its hazard checks see a vector ALU write (an
// MFMA must not read the result in the next two wait states, which the compiler cannot
// know of an instruction written as inline asm).
__device__ __forceinline__ uint32_t in_sgpr(uint32_t v) {
    asm("" : "+s"(v));
    return v;
}
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits) {
    return (v & in_sgpr(mask)) | in_vgpr(bits);
}

// fp16 path: w = fp16_rne((q - z) * s).  (B + q) + (-(B + z)) is exact (an integer of
// magnitude <= 15, B = 1024 or 64), then one packed multiply by s rounds once, to nearest
// even.  nz_hi2 / nz_lo2: half2 bits of -(1024 + z) / -(64 + z); s2: half2 bits of s.
__device__ __forceinline__ u32x4_t dequant_word_f16(uint32_t w, uint32_t nz_hi2,
                                                    uint32_t nz_lo2, uint32_t s2) {
    const uint32_t w8 = w >> 8;
    u32x4_t h;
    h[0] = and_or(w, 0x000F000Fu, 0x64006400u);    // e0, e1 -> 1024 + q
    h[1] = and_or(w, 0x00F000F0u, 0x54005400u);    // e2, e3 ->   64 + q
    h[2] = and_or(w8, 0x000F000Fu, 0x64006400u);   // e4, e5 -> 1024 + q
    h[3] = and_or(w8, 0x00F000F0u, 0x54005400u);   // e6, e7 ->   64 + q
    const half2_t s = bitcast<half2_t>(s2);
    u32x4_t r;
    r[0] = bitcast<uint32_t>((bitcast<half2_t>(h[0]) + bitcast<half2_t>(nz_hi2)) * s);
    r[1] = bitcast<uint32_t>((bitcast<half2_t>(h[1]) + bitcast<half2_t>(nz_lo2)) * s);
    r[2] = bitcast<uint32_t>((bitcast<half2_t>(h[2]) + bitcast<half2_t>(nz_hi2)) * s);
    r[3] = bitcast<uint32_t>((bitcast<half2_t>(h[3]) + bitcast<half2_t>(nz_lo2)) * s);
    return r;
}

// The same word's exact differences q - z as fp16 pairs, without the scale: the small-M
// kernel multiplies whole group sums by s in fp32 instead (one multiply per output and
// group rather than one per weight pair).  Every (q - z) is an integer of magnitude <= 15,
// exact in fp16, and its products with fp16 activations are exact in fp32.
__device__ __forceinline__ u32x4_t dequant_word_f16_int(uint32_t w, uint32_t nz_hi2,
                                                        uint32_t nz_lo2) {
    const uint32_t w8 = w >> 8;
    u32x4_t h;
    h[0] = and_or(w, 0x000F000Fu, 0x64006400u);
    h[1] = and_or(w, 0x00F000F0u, 0x54005400u);
    h[2] = and_or(w8, 0x000F000Fu, 0x64006400u);
    h[3] = and_or(w8, 0x00F000F0u, 0x54005400u);
    u32x4_t r;
    r[0] = bitcast<uint32_t>(bitcast<half2_t>(h[0]) + bitcast<half2_t>(nz_hi2));
    r[1] = bitcast<uint32_t>(bitcast<half2_t>(h[1]) + bitcast<half2_t>(nz_lo2));
    r[2] = bitcast<uint32_t>(bitcast<half2_t>(h[2]) + bitcast<half2_t>(nz_hi2));
    r[3] = bitcast<uint32_t>(bitcast<half2_t>(h[3]) + bitcast<half2_t>(nz_lo2));
    return r;
}

// bf16 codes for the small-M kernel's scaled group sums: every nibble moved to the low
// four bits of its 16-bit half and OR-ed into 0x4300 (bf16 128.0, whose last place is 1),
// which gives 128 + q exactly.  Pairs in element order (e0 e1) (e2 e3) (e4 e5) (e6 e7).  The
// caller subtracts (128 + z) times the group's activation sum from each group sum and
// scales it by s in fp32; no per-weight subtraction or multiply remains.
__device__ __forceinline__ u32x4_t dequant_word_bf16_biased(uint32_t w) {
    u32x4_t h;
    h[0] = and_or(w, 0x000F000Fu, 0x43004300u);
    h[1] = and_or(w >> 4, 0x000F000Fu, 0x43004300u);
    h[2] = and_or(w >> 8, 0x000F000Fu, 0x43004300u);
    h[3] = and_or(w >> 12, 0x000F000Fu, 0x43004300u);
    return h;
}

// bf16 path: w = bf16_rne((q - z) * s) with s in fp16.  The nibbles are spread to bytes
// and converted to fp32 (v_cvt_f32_ubyteN); q*s + (-z*s) is exact in fp32 (every term is
// an integer below 16 times an 11-bit significand), and the final conversion to bf16 is
// the single rounding.  Byte order after the spread: lo = e0 e4 e1 e5, hi = e2 e6 e3 e7.
//   s: the scale in fp32; nzs: -z * s in fp32 (exact).
__device__ __forceinline__ float ubyte(uint32_t v, int b) {
    return (float)((v >> (8 * b)) & 0xFFu);
}
// Two fp32 values rounded to bf16 (nearest even), lo in the low half.  Converted as one
// vector, so the compiler emits a single two-source v_cvt_pk_bf16_f32; two scalar casts
// became two conversions, a shift and an OR.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bitcast<uint32_t>(__builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ u32x4_t dequant_word_bf16(uint32_t w, float s, float nzs) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    const float e0 = __builtin_fmaf(ubyte(lo, 0), s, nzs);
    const float e4 = __builtin_fmaf(ubyte(lo, 1), s, nzs);
    const float e1 = __builtin_fmaf(ubyte(lo, 2), s, nzs);
    const float e5 = __builtin_fmaf(ubyte(lo, 3), s, nzs);
    const float e2 = __builtin_fmaf(ubyte(hi, 0), s, nzs);
    const float e6 = __builtin_fmaf(ubyte(hi, 1), s, nzs);
    const float e3 = __builtin_fmaf(ubyte(hi, 2), s, nzs);
    const float e7 = __builtin_fmaf(ubyte(hi, 3), s, nzs);
    u32x4_t r;
    r[0] = pack_bf16x2(e0, e1);
    r[1] = pack_bf16x2(e2, e3);
    r[2] = pack_bf16x2(e4, e5);
    r[3] = pack_bf16x2(e6, e7);
    return r;
}

// Per-(group, column) dequantization constants in the form each path wants.
struct DqF16 {
    uint32_t nz_hi2, nz_lo2, s2;
};
struct DqBF16 {
    float s, nzs;
    float nz_hi, nz_lo;          // -(1024 + z) s and -(64 + z) s, for the magic-number form
};

__device__ __forceinline__ DqF16 make_dq_f16(uint16_t s_bits, uint32_t z) {
    // -(1024 + z): sign, exponent of 1024 (0x6400), fraction z (spacing 1).
    // -(64 + z):   sign, exponent of 64 (0x5400), fraction 16 z (spacing 1/16).
    const uint32_t nh = 0xE400u | z;
    const uint32_t nl = 0xD400u | (z << 4);
    DqF16 d;
    d.nz_hi2 = nh | (nh << 16);
    d.nz_lo2 = nl | (nl << 16);
    d.s2 = (uint32_t)s_bits | ((uint32_t)s_bits << 16);
    return d;
}
__device__ __forceinline__ DqBF16 make_dq_bf16(uint16_t s_bits, uint32_t z) {
    DqBF16 d;
    d.s = (float)bitcast<_Float16>(s_bits);
    d.nzs = -(float)z * d.s;     // exact: 4-bit integer times 11-bit significand
    // exact too: integers of at most 11 bits (8-bit z: 1279) times an 11-bit significand
    d.nz_hi = -(1024.0f + (float)z) * d.s;
    d.nz_lo = -(64.0f + (float)z) * d.s;
    return d;
}

template <int ACT>
struct Dq;
template <>
struct Dq<kF16> {
    typedef DqF16 type;
    static __device__ __forceinline__ DqF16 make(uint16_t s, uint32_t z) { return make_dq_f16(s, z); }
    static __device__ __forceinline__ u32x4_t word(uint32_t w, const DqF16 &d) {
        return dequant_word_f16(w, d.nz_hi2, d.nz_lo2, d.s2);
    }
};
template <>
struct Dq<kBF16> {
    typedef DqBF16 type;
    static __device__ __forceinline__ DqBF16 make(uint16_t s, uint32_t z) { return make_dq_bf16(s, z); }
    static __device__ __forceinline__ u32x4_t word(uint32_t w, const DqBF16 &d) {
        return dequant_word_bf16(w, d.s, d.nzs);
    }
};

// ------------------------------------------------------- 8-bit codes (W8A16) --------
//
// A pair of 32-bit words holds the codes of k0 .. k0+7 of one column, k0 in the low byte.
// A byte permute against the fp16 pattern 0x64 builds each (k, k+1) register pair as
// (1024 + q) halves in one operation (v_perm_b32: selector bytes 0..3 pick the word,
// 4..7 the pattern); then, as for 4-bit codes, an exact packed add of -(1024 + z) (an
// integer of magnitude <= 255) and one rounding packed multiply by s.
__device__ __forceinline__ u32x4_t dequant_pair_w8_f16(uint32_t w0, uint32_t w1,
                                                       uint32_t nz2, uint32_t s2) {
    u32x4_t h;
    h[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);   // k0, k1
    h[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);   // k2, k3
    h[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);   // k4, k5
    h[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);   // k6, k7
    const half2_t s = bitcast<half2_t>(s2);
    const half2_t nz = bitcast<half2_t>(nz2);
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = bitcast<uint32_t>((bitcast<half2_t>(h[j]) + nz) * s);
    return r;
}
// The exact differences q - z (|q - z| <= 255, exact in fp16) of a pair of 8-bit code words,
// without the scale (see dequant_word_f16_int).
__device__ __forceinline__ u32x4_t dequant_pair_w8_f16_int(uint32_t w0, uint32_t w1,
                                                           uint32_t nz2) {
    u32x4_t h;
    h[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
    h[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
    h[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
    h[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
    const half2_t nz = bitcast<half2_t>(nz2);
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = bitcast<uint32_t>(bitcast<half2_t>(h[j]) + nz);
    return r;
}
// bf16: q * s + (-z * s) in fp32 (exact: 8-bit integer times 11-bit significand), one
// rounding to bf16.
__device__ __forceinline__ u32x4_t dequant_pair_w8_bf16(uint32_t w0, uint32_t w1, float s,
                                                        float nzs) {
    u32x4_t r;
    r[0] = pack_bf16x2(__builtin_fmaf(ubyte(w0, 0), s, nzs), __builtin_fmaf(ubyte(w0, 1), s, nzs));
    r[1] = pack_bf16x2(__builtin_fmaf(ubyte(w0, 2), s, nzs), __builtin_fmaf(ubyte(w0, 3), s, nzs));
    r[2] = pack_bf16x2(__builtin_fmaf(ubyte(w1, 0), s, nzs), __builtin_fmaf(ubyte(w1, 1), s, nzs));
    r[3] = pack_bf16x2(__builtin_fmaf(ubyte(w1, 2), s, nzs), __builtin_fmaf(ubyte(w1, 3), s, nzs));
    return r;
}

template <int ACT>
struct Dq8;
template <>
struct Dq8<kF16> {
    typedef DqF16 type;
    // -(1024 + z): sign, exponent of 1024 (0x6400), fraction z (spacing 1, z < 1024).
    static __device__ __forceinline__ DqF16 make(uint16_t s, uint32_t z) {
        const uint32_t nh = 0xE400u | z;
        DqF16 d;
        d.nz_hi2 = nh | (nh << 16);
        d.nz_lo2 = 0u;
        d.s2 = (uint32_t)s | ((uint32_t)s << 16);
        return d;
    }
    static __device__ __forceinline__ u32x4_t pair(uint32_t w0, uint32_t w1, const DqF16 &d) {
        return dequant_pair_w8_f16(w0, w1, d.nz_hi2, d.s2);
    }
};
template <>
struct Dq8<kBF16> {
    typedef DqBF16 type;
    static __device__ __forceinline__ DqBF16 make(uint16_t s, uint32_t z) { return make_dq_bf16(s, z); }
    static __device__ __forceinline__ u32x4_t pair(uint32_t w0, uint32_t w1, const DqBF16 &d) {
        return dequant_pair_w8_bf16(w0, w1, d.s, d.nzs);
    }
};

// ------------------------------------------------------- FP8 codes (W-FP8 A16) -------
//
// w = fp8(q) * s, rounded once.  A pair of words holds codes k0 .. k7 of one column, k0 in
// the low byte.  fp16: every E4M3 and E5M2 value is exactly an fp16 value, so each code
// pair converts exactly to an fp16 pair (E4M3 by the scaled convert at scale 1.0; E5M2 is
// the high byte of binary16, placed by a byte permute that zeroes the low bytes), and one
// packed multiply by s rounds.  bf16: s is an fp16 value, not a bf16 one, so each code pair
// converts exactly to fp32, multiplies by s exactly in fp32 (at most a 4-bit significand
// times an 11-bit one) and rounds once to bf16.
template <int CODE, bool HI>
__device__ __forceinline__ uint32_t fp8_pair_f16(uint32_t w) {
    if constexpr (CODE == kE4M3)
        return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
    else
        return __builtin_amdgcn_perm(w, w, HI ? 0x030C020Cu : 0x010C000Cu);
}
template <int CODE, bool HI>
__device__ __forceinline__ f32x2_t fp8_pair_f32(uint32_t w) {
    if constexpr (CODE == kE4M3)
        return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    else
        return __builtin_amdgcn_cvt_pk_f32_bf8(w, HI);
}

template <int ACT, int CODE>
struct DqF8;
template <int CODE>
struct DqF8<kF16, CODE> {
    typedef DqF16 type;
    static __device__ __forceinline__ DqF16 make(uint16_t s, uint32_t) {
        DqF16 d;
        d.nz_hi2 = d.nz_lo2 = 0u;
        d.s2 = (uint32_t)s | ((uint32_t)s << 16);
        return d;
    }
    static __device__ __forceinline__ u32x4_t pair(uint32_t w0, uint32_t w1, const DqF16 &d) {
        const half2_t s = bitcast<half2_t>(d.s2);
        u32x4_t r;
        r[0] = bitcast<uint32_t>(bitcast<half2_t>(fp8_pair_f16<CODE, false>(w0)) * s);
        r[1] = bitcast<uint32_t>(bitcast<half2_t>(fp8_pair_f16<CODE, true>(w0)) * s);
        r[2] = bitcast<uint32_t>(bitcast<half2_t>(fp8_pair_f16<CODE, false>(w1)) * s);
        r[3] = bitcast<uint32_t>(bitcast<half2_t>(fp8_pair_f16<CODE, true>(w1)) * s);
        return r;
    }
};
template <int CODE>
struct DqF8<kBF16, CODE> {
    typedef DqBF16 type;
    static __device__ __forceinline__ DqBF16 make(uint16_t s, uint32_t) {
        DqBF16 d;
        d.s = (float)bitcast<_Float16>(s);
        d.nzs = 0.f;
        return d;
    }
    static __device__ __forceinline__ u32x4_t pair(uint32_t w0, uint32_t w1, const DqBF16 &d) {
        const f32x2_t f0 = fp8_pair_f32<CODE, false>(w0), f1 = fp8_pair_f32<CODE, true>(w0);
        const f32x2_t f2 = fp8_pair_f32<CODE, false>(w1), f3 = fp8_pair_f32<CODE, true>(w1);
        u32x4_t r;
        r[0] = pack_bf16x2(f0.x * d.s, f0.y * d.s);
        r[1] = pack_bf16x2(f1.x * d.s, f1.y * d.s);
        r[2] = pack_bf16x2(f2.x * d.s, f2.y * d.s);
        r[3] = pack_bf16x2(f3.x * d.s, f3.y * d.s);
        return r;
    }
};

// ------------------------------------------------ 2-bit and 3-bit codes (sub-4-bit) ----
//
// A lane's 32 codes of a 128-deep tile (4 MFMA steps x 8) sit in b words (include/mpgemm.h):
// pair register r = 4t + j holds elements 2j, 2j+1 of step t in its low and high 16-bit
// halves.  Each code field of b bits sits inside the fp16 mantissa at bit p of its half, so
// one v_and_or_b32 with the fp16 pattern of B_p (the power of two whose mantissa step at
// bit p is 1) makes the pair B_p + q; an exact packed add of -(B_p + z) leaves q - z, and
// one packed multiply by s rounds (fp16).  bf16: (q - z) to fp32, exact products with s,
// one rounding.
//   2-bit: fields at p = 0, 2, 4, 6 (B = 1024, 256, 64, 16) of the word, or of the word
//          shifted right by 8; word r / 8.
//   3-bit: fields at p = 0, 3, 6 (B = 1024, 128, 16) of the word, or at 9, 12 read after a
//          shift by 9; word r / 5 for r < 15.  Pair 15 is gathered from bits 15 and 31 of
//          the three words (bit c of each code in word c), at p = 0.
template <int BITS>
struct LowBases;
template <>
struct LowBases<2> {
    static constexpr int kCount = 4;
    static constexpr uint32_t kPattern[4] = {0x64006400u, 0x5C005C00u, 0x54005400u, 0x4C004C00u};
    static constexpr float kValue[4] = {1024.f, 256.f, 64.f, 16.f};
};
template <>
struct LowBases<3> {
    static constexpr int kCount = 3;
    static constexpr uint32_t kPattern[3] = {0x64006400u, 0x58005800u, 0x4C004C00u};
    static constexpr float kValue[3] = {1024.f, 128.f, 16.f};
};

// Per-(group, column) constants: -(B_p + z) as fp16 pairs, and the scale.
template <int BITS>
struct DqLowConst {
    uint32_t nz[LowBases<BITS>::kCount];
    uint32_t s2;                 // fp16 pair of s
    float s;                     // s as fp32 (bf16 path)
};

// Biased pair register r (B_p + q in each half) from the lane's words, and its base index.
template <int BITS, int R>
__device__ __forceinline__ uint32_t low_pair(const u32x4_t &w, int &base) {
    if constexpr (BITS == 2) {
        constexpr int j = R % 4, sh = 8 * ((R % 8) / 4);
        base = j;
        const uint32_t src = sh ? (w[R / 8] >> sh) : w[R / 8];
        return and_or(src, 0x00030003u << (2 * j), LowBases<2>::kPattern[j]);
    } else if constexpr (R < 15) {
        constexpr int s5 = R % 5, j = s5 % 3;
        base = j;
        const uint32_t src = s5 >= 3 ? (w[R / 5] >> 9) : w[R / 5];
        return and_or(src, 0x00070007u << (3 * j), LowBases<3>::kPattern[j]);
    } else {
        base = 0;
        uint32_t h = and_or(w[0] >> 15, 0x00010001u, LowBases<3>::kPattern[0]);
        h = and_or(w[1] >> 14, 0x00020002u, h);
        return and_or(w[2] >> 13, 0x00040004u, h);
    }
}

template <int ACT, int BITS>
struct DqLow {
    typedef DqLowConst<BITS> type;
    // -(B_b + z) in fp16 is the sign bit, B_b's pattern and z in units of B_b's last place
    // (2^(-BITS b) for base b): z < 2^BITS shifted by BITS b stays below 2^10, inside the
    // mantissa, so the pattern is exact and built with integer operations.
    static __device__ __forceinline__ type make(uint16_t s, uint32_t z) {
        type d;
        const uint32_t zz = z * 0x00010001u;
#pragma unroll
        for (int b = 0; b < LowBases<BITS>::kCount; ++b)
            d.nz[b] = (zz << (BITS * b)) + (LowBases<BITS>::kPattern[b] | 0x80008000u);
        d.s2 = (uint32_t)s | ((uint32_t)s << 16);
        d.s = (float)bitcast<_Float16>(s);
        return d;
    }
    // The four MFMA steps' A operands of one lane-tile; d[t] holds step t's constants.
    static __device__ __forceinline__ void tile(const u32x4_t &w, const type *const (&d)[4],
                                                u32x4_t (&a)[4]) {
        [&]<int... R>(std::integer_sequence<int, R...>) {
            (([&] {
                 int b;
                 const uint32_t h = low_pair<BITS, R>(w, b);
                 const type &c = *d[R / 4];
                 const half2_t q = bitcast<half2_t>(h) + bitcast<half2_t>(c.nz[b]);   // exact
                 if constexpr (ACT == kF16) {
                     a[R / 4][R % 4] = bitcast<uint32_t>(q * bitcast<half2_t>(c.s2));
                 } else {
                     a[R / 4][R % 4] = pack_bf16x2((float)q.x * c.s, (float)q.y * c.s);
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, 16>{});
    }
    // fp16 only: the exact differences q - z as fp16 pairs, without the scale (the small-M
    // kernel scales whole group sums in fp32, as for 4-bit codes).
    static __device__ __forceinline__ void tile_int(const u32x4_t &w,
                                                    const type *const (&d)[4],
                                                    u32x4_t (&a)[4]) {
        [&]<int... R>(std::integer_sequence<int, R...>) {
            (([&] {
                 int b;
                 const uint32_t h = low_pair<BITS, R>(w, b);
                 a[R / 4][R % 4] = bitcast<uint32_t>(bitcast<half2_t>(h) +
                                                     bitcast<half2_t>(d[R / 4]->nz[b]));
             }()),
             ...);
        }(std::make_integer_sequence<int, 16>{});
    }
};

// The dequantization of code format CODE for activation format ACT: make(s, z) builds the
// per-(group, column) constants; pair(w0, w1, d) (8-bit formats) dequantizes codes k0..k7.
template <int ACT, int CODE>
struct DqSel {
    typedef DqF8<ACT, CODE> type;
};
template <int ACT>
struct DqSel<ACT, kU4> {
    typedef Dq<ACT> type;
};
template <int ACT>
struct DqSel<ACT, kU8> {
    typedef Dq8<ACT> type;
};
template <int ACT>
struct DqSel<ACT, kU2> {
    typedef DqLow<ACT, 2> type;
};
template <int ACT>
struct DqSel<ACT, kU3> {
    typedef DqLow<ACT, 3> type;
};
template <int ACT, int CODE>
using DqFor = typename DqSel<ACT, CODE>::type;

// ------------------------------------------------------------------------------ MFMA --
//
// v_mfma_f32_16x16x32_{f16,bf16}: D[i][j] += sum_k A[i][k] * B[k][j] over a 16x16x32
// block.  Operand lane l holds A row (l % 16) / B column (l % 16) at k = 8*(l/16) .. +7 as
// four 32-bit registers of (k, k+1) pairs; the fp32 result lane l holds D[4*(l/16) + r]
// [l % 16] in register r.  The kernels put dequantized weights in A (rows = n) and
// activations in B (columns = m), so lane l ends with four consecutive n of one row m.
template <int ACT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t &a, const u32x4_t &b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma16x16x32<kF16>(const u32x4_t &a, const u32x4_t &b,
                                                      f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(a), bitcast<half8_t>(b), c,
                                                  0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma16x16x32<kBF16>(const u32x4_t &a, const u32x4_t &b,
                                                       f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b),
                                                   c, 0, 0, 0);
}

// fp32 -> activation format, round to nearest even; one value.
template <int ACT>
__device__ __forceinline__ uint16_t round1(float v) {
    if constexpr (ACT == kF16)
        return bitcast<uint16_t>((_Float16)v);
    else
        return bitcast<uint16_t>((__bf16)v);
}

// fp32 -> activation format, round to nearest even; four values packed into 8 bytes.
template <int ACT>
__device__ __forceinline__ u32x2_t round4(const f32x4_t &v);
template <>
__device__ __forceinline__ u32x2_t round4<kF16>(const f32x4_t &v) {
    u32x2_t r;
    r[0] = (uint32_t)bitcast<uint16_t>((_Float16)v[0]) |
           ((uint32_t)bitcast<uint16_t>((_Float16)v[1]) << 16);
    r[1] = (uint32_t)bitcast<uint16_t>((_Float16)v[2]) |
           ((uint32_t)bitcast<uint16_t>((_Float16)v[3]) << 16);
    return r;
}
template <>
__device__ __forceinline__ u32x2_t round4<kBF16>(const f32x4_t &v) {
    u32x2_t r;
    r[0] = pack_bf16x2(v[0], v[1]);
    r[1] = pack_bf16x2(v[2], v[3]);
    return r;
}

// Stores four consecutive outputs of one row at p, of which only the first `avail` exist
// (a ragged last column block), rounded as round4: one 8-byte store when all four exist
// and p is 8-byte aligned (rows of a width that is a multiple of 4), 2-byte stores
// otherwise.
template <int ACT>
__device__ __forceinline__ void store4(uint16_t *p, int avail, const f32x4_t &v) {
    const u32x2_t r = round4<ACT>(v);
    if (avail >= 4 && ((uintptr_t)p & 7u) == 0) {
        *reinterpret_cast<u32x2_t *>(p) = r;
        return;
    }
    p[0] = (uint16_t)r[0];
    if (avail > 1) p[1] = (uint16_t)(r[0] >> 16);
    if (avail > 2) p[2] = (uint16_t)r[1];
    if (avail > 3) p[3] = (uint16_t)(r[1] >> 16);
}

// Meta plane readers (layout v1): strip-major scales, then 4-bit zeros at the same index.
__device__ __forceinline__ uint32_t read_zero(const uint8_t *zeros, size_t e) {
    const uint32_t b = zeros[e >> 1];
    return (e & 1) ? (b >> 4) : (b & 0xFu);
}

// ------------------------------------------------------------------- buffer loads --
//
// The GEMM kernels read through buffer resources: one 128-bit scalar descriptor per plane,
// a 32-bit per-lane byte offset that stays fixed across the K loop, and a wave-uniform
// scalar offset that advances it.  This keeps address arithmetic out of the vector ALU and
// out of vector registers.  A lane whose own offset lies past the descriptor's byte count
// reads zeros without touching memory (gfx9 raw-buffer range check), which the kernels use
// for rows past M.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // Third descriptor dword of gfx9-family raw buffers (32-bit data format, no swizzle).
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2_t buf_load_b64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ u32x4_t buf_load_b96(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    const u32x3_t v = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0));
    return u32x4_t{v.x, v.y, v.z, 0u};
}
__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Device-scope (sc1) buffer accesses: a store is acknowledged only once it is visible to
// every XCD, and a load does not take a possibly stale line from this XCD's L2.
constexpr int kCachePolicyDevice = 16;      // sc1 bit of the buffer cache-policy operand
__device__ __forceinline__ void buf_store_b128_device(rsrc_t r, uint32_t voff, u32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kCachePolicyDevice);
}
__device__ __forceinline__ u32x4_t buf_load_b128_device(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCachePolicyDevice));
}
// 32 wait states: longer than any MFMA of these kernels takes to write its result.  Kernels
// that issue MFMAs through inline asm (invisible to the compiler's hazard tracking) run it
// after their last MFMA, before any code that may read the accumulators.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Waits for every vector-memory access this wave has issued (loads and stores) to finish:
// vmcnt = 0, expcnt and lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace mpgemm
