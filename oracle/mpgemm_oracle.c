/*
 * CPU oracle for the W4A16 mixed-precision GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load this
 * library.  It shares no code with the HIP path (weight_only_quantized_mpgemm_amd/csrc):
 * no headers, no helpers, no tables.  It is plain, scalar and slow on purpose so that a
 * reader can check it against the definitions by eye.
 *
 * Source cited throughout: "LMDeploy Accelerates Mixed-Precision LLM Inference with
 * TurboMind" (arXiv 2508.15601), abbreviated [TurboMind].
 *
 *   - [TurboMind, Fig. 4 caption and Fig. 6 caption]: low-bit integers are turned into
 *     FP16 by "I2F" conversion and scaling before the tensor-core multiply.  The formula is
 *     not printed on the pages; the reading used here is the asymmetric group form
 *     w = (q - z) * s with one scale s and one integer zero z per (group of g consecutive
 *     k, column n), rounded once to the activation format (fp16; bf16 for bf16
 *     activations).  zero = 8 for symmetric codes.
 *   - The GEMM is Y[m][n] = sum_k X[m][k] * w[k][n].  The oracle forms the sum in fp64 in
 *     ascending k and rounds it once (round-to-nearest-even) to the activation format.
 *   - [TurboMind, Fig. 6 and Fig. 7 captions; the interleave diagram beside Fig. 24]:
 *     packing is an offline, lossless permutation.  The word-internal nibble order is the
 *     one that diagram shows (most to least significant: e7 e5 e3 e1 e6 e4 e2 e0).  The
 *     tile and lane placement is this library's own gfx950 layout, restated below from
 *     its specification (see include/mpgemm.h), not derived from the GPU code.
 *
 * Parity status: every function here is pinned by CPU tests (tests/test_oracle.py; the
 * 8-bit functions by tests/test_oracle_w8.py, the FP8 ones by tests/test_oracle_fp8.py,
 * packing of ragged shapes by tests/test_oracle_ragged.py, the 2-bit and 3-bit functions by
 * tests/test_oracle_lowbit.py, attention decode by tests/test_oracle_attention.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* ---------------------------------------------------------------- number formats --- */

/* IEEE 754 binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);     /* (1.f) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/*
 * Round a double to a binary format with `frac_bits` fraction bits, exponent bias `bias`
 * and all-ones exponent `emax_field`, ties to even.  The value is split into an integer
 * count of the format's spacing (ulp) at its exponent; rint() rounds that count in the
 * default ties-to-even mode.  Below the smallest normal the spacing stays fixed
 * (subnormals).  A count that carries into the next binade is encoded by the same sum.
 */
static uint16_t round_to_binary16_like(double x, int frac_bits, int bias, int emax_field) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    uint16_t inf_bits = (uint16_t)(emax_field << frac_bits);
    if (isnan(x)) return (uint16_t)(inf_bits | (1u << (frac_bits - 1)));  /* quiet NaN */
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | inf_bits);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);              /* a in [2^(e2-1), 2^e2) */
    int exp_unbiased = e2 - 1;
    int min_normal_exp = 1 - bias;
    if (exp_unbiased < min_normal_exp) exp_unbiased = min_normal_exp;
    if (exp_unbiased > emax_field - 1 - bias) {
        return (uint16_t)(sign | inf_bits);  /* at or above 2^(emax+1): beyond every finite */
    }
    double spacing = ldexp(1.0, exp_unbiased - frac_bits);
    double count = rint(a / spacing);       /* exact scaling, then ties-to-even */
    /* count lies in [2^frac_bits, 2^(frac_bits+1)] for normals, [0, 2^frac_bits] below. */
    /* Biased exponent field plus fraction; for the lowest binade the field is 1 and the
       sum reduces to the count itself, which is the subnormal encoding. */
    long bits = ((long)(exp_unbiased + bias) << frac_bits) + (long)count - (1L << frac_bits);
    if (bits >= (long)inf_bits) return (uint16_t)(sign | inf_bits);   /* overflow */
    return (uint16_t)(sign | (uint16_t)bits);
}

uint16_t oracle_f64_to_f16(double x) { return round_to_binary16_like(x, 10, 15, 31); }
uint16_t oracle_f64_to_bf16(double x) { return round_to_binary16_like(x, 7, 127, 255); }

static double act_to_f64(uint16_t v, int dtype) {
    return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(v) : oracle_f16_to_f64(v);
}
static uint16_t f64_to_act(double v, int dtype) {
    return dtype == ORACLE_BF16 ? oracle_f64_to_bf16(v) : oracle_f64_to_f16(v);
}

/* ---------------------------------------------------------------- dequantization --- */

/*
 * w[k][n] = round_act((q[k][n] - z[k/g][n]) * s[k/g][n])          [TurboMind, Fig. 6]
 *   codes  uint8 [K][N], low 4 bits used (the code is an unsigned 4-bit integer)
 *   scales fp16  [ceil(K/g)][N]
 *   zeros  uint8 [ceil(K/g)][N], low 4 bits used; NULL means symmetric codes with zero 8
 *   w      out, activation format bits, [K][N]
 */
void oracle_dequant(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                    int K, int N, int g, int dtype, uint16_t *w) {
    for (int k = 0; k < K; ++k) {
        int grp = k / g;
        for (int n = 0; n < N; ++n) {
            int q = codes[(size_t)k * N + n] & 0xf;
            int z = zeros ? (zeros[(size_t)grp * N + n] & 0xf) : 8;
            double s = oracle_f16_to_f64(scales[(size_t)grp * N + n]);
            double exact = (double)(q - z) * s;      /* exact: 5-bit integer x 11-bit scale */
            w[(size_t)k * N + n] = f64_to_act(exact, dtype);
        }
    }
}

/* ---------------------------------------------------------------------- the GEMM --- */

/*
 * Y[m][n] = round_act( sum_{k ascending} X[m][k] * w[k][n] ), sum in fp64.
 *   X [M][K], w [K][N], Y [M][N], all activation-format bits, row-major.
 *   threads: OpenMP threads over independent output rows (1 = serial).
 */
void oracle_gemm(const uint16_t *X, const uint16_t *w, int M, int N, int K, int dtype,
                 uint16_t *Y, int threads) {
#ifdef _OPENMP
    if (threads < 1) threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                acc += act_to_f64(X[(size_t)m * K + k], dtype) *
                       act_to_f64(w[(size_t)k * N + n], dtype);
            }
            Y[(size_t)m * N + n] = f64_to_act(acc, dtype);
        }
    }
}

/* ------------------------------------------------------------------ packed layout --- */

/*
 * Layout version 1 (restated from its specification in include/mpgemm.h):
 *
 * Codes plane, K*N/2 bytes.  The [K][N] code matrix is cut into tiles of 16 columns by
 * 128 rows of k.  Tile index T = (n/16)*(K/128) + k/128, tile base T*1024 bytes.  Within a
 * tile, with kk = k%128 and nn = n%16: lane L = nn + 16*((kk%32)/8), word t = kk/32, and
 * the 32-bit little-endian word sits at byte L*16 + t*4.  Element i = kk%8 of the word
 * occupies nibble p(i) = i/2 for even i and 4 + i/2 for odd i (bits 4p..4p+3), which
 * reads e7 e5 e3 e1 e6 e4 e2 e0 from the most significant nibble down
 * [TurboMind, interleave diagram beside Fig. 24].
 *
 * Meta plane.  Scales first: fp16 at element index (n/16)*(K/g)*16 + (k/g)*16 + n%16,
 * (K/g)*N*2 bytes.  Then, for asymmetric codes only, zeros: 4-bit values at the same
 * element index e, byte e/2, low nibble for even e, high nibble for odd e,
 * (K/g)*N/2 bytes.
 */
static int nibble_of_element(int i) { return (i % 2 == 0) ? i / 2 : 4 + i / 2; }

/*
 * Ragged shapes [TurboMind, Fig. 24: a data matrix padded up to the hardware tile]: the
 * planes describe the matrix padded to Kp x Np, Np = N rounded up to a multiple of 16,
 * Kp = K rounded up to a multiple of 128 (one tile of the layout).  The user arrays stay
 * [K][N] (codes) and [ceil(K/g)][N] (scales, zeros).  Padding: in columns n >= N, code 0,
 * scale 0 and zero 0; in rows k >= K of columns n < N, the code equals the element's zero
 * point (its group's zero, 0 in groups past ceil(K/g), 8 or 128 for symmetric codes), so
 * every padded weight dequantizes to zero.  Groups past ceil(K/g) have scale 0, zero 0.
 */
int oracle_padded_k(int K) { return (K + 127) / 128 * 128; }
int oracle_padded_n(int N) { return (N + 15) / 16 * 16; }
static int groups_of(int K, int g) { return (K + g - 1) / g; }

static size_t code_byte_offset(int k, int n, int K) {
    size_t T = (size_t)(n / 16) * (size_t)(K / 128) + (size_t)(k / 128);
    int kk = k % 128, nn = n % 16;
    int lane = nn + 16 * ((kk % 32) / 8);
    int word = kk / 32;
    return T * 1024 + (size_t)lane * 16 + (size_t)word * 4;
}

static size_t meta_index(int k, int n, int K, int g) {
    return (size_t)(n / 16) * (size_t)(K / g) * 16 + (size_t)(k / g) * 16 + (size_t)(n % 16);
}

size_t oracle_packed_code_bytes(int K, int N) {
    return (size_t)oracle_padded_k(K) * oracle_padded_n(N) / 2;
}
size_t oracle_packed_meta_bytes(int K, int N, int g, int symmetric) {
    size_t cells = (size_t)(oracle_padded_k(K) / g) * oracle_padded_n(N);
    return cells * 2 + (symmetric ? 0 : cells / 2);
}

/* Zero point of user element (k, n) as the padded matrix stores it. */
static int zero_point(const uint8_t *zeros, int r, int n, int N, int rows, int sym_zero) {
    if (!zeros) return sym_zero;
    return r < rows ? zeros[(size_t)r * N + n] : 0;
}

/* K, N: the user matrix (any K, N >= 1; see the ragged-shape rule above). */
void oracle_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                 int K, int N, int g, uint8_t *packed_codes, uint8_t *packed_meta) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    memset(packed_codes, 0, oracle_packed_code_bytes(K, N));
    memset(packed_meta, 0, oracle_packed_meta_bytes(K, N, g, zeros == NULL));
    for (int k = 0; k < Kp; ++k) {
        for (int n = 0; n < N; ++n) {              /* columns n >= N keep code 0 */
            uint32_t q = k < K ? (codes[(size_t)k * N + n] & 0xf)
                               : (uint32_t)(zero_point(zeros, k / g, n, N, rows, 8) & 0xf);
            size_t off = code_byte_offset(k, n, Kp);
            uint32_t word;
            memcpy(&word, packed_codes + off, 4);
            word |= q << (4 * nibble_of_element(k % 8));
            memcpy(packed_codes + off, &word, 4);
        }
    }
    uint16_t *meta_scales = (uint16_t *)packed_meta;
    uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            meta_scales[e] = scales[(size_t)r * N + n];
            if (zeros) {
                uint8_t z = zeros[(size_t)r * N + n] & 0xf;
                meta_zeros[e / 2] |= (uint8_t)((e % 2) ? (z << 4) : z);
            }
        }
    }
}

/* Inverse of oracle_pack (the user [K][N] part).  zeros is written only for asymmetric
 * packing. */
void oracle_unpack(const uint8_t *packed_codes, const uint8_t *packed_meta, int K, int N,
                   int g, int symmetric, uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    for (int k = 0; k < K; ++k) {
        for (int n = 0; n < N; ++n) {
            uint32_t word;
            memcpy(&word, packed_codes + code_byte_offset(k, n, Kp), 4);
            codes[(size_t)k * N + n] = (uint8_t)((word >> (4 * nibble_of_element(k % 8))) & 0xf);
        }
    }
    const uint16_t *meta_scales = (const uint16_t *)packed_meta;
    const uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            scales[(size_t)r * N + n] = meta_scales[e];
            if (!symmetric && zeros) {
                uint8_t b = meta_zeros[e / 2];
                zeros[(size_t)r * N + n] = (uint8_t)((e % 2) ? (b >> 4) : (b & 0xf));
            }
        }
    }
}

/* ------------------------------------------------------------ 8-bit weights (W8A16) --- */

/*
 * [TurboMind, abstract (pg1): the GEMM pipeline generalizes across precision formats].
 * The 8-bit reading of the same group form: w = round_act((q - z) * s) with q and z
 * unsigned 8-bit integers (0..255) and z = 128 for symmetric codes.  (q - z) is an
 * integer of at most 9 bits, so the product with an 11-bit fp16 scale is exact in fp64.
 *   codes  uint8 [K][N]; scales fp16 [ceil(K/g)][N]; zeros the same shape or NULL (z = 128)
 *   w      out, activation format bits, [K][N]
 */
void oracle_dequant_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       int K, int N, int g, int dtype, uint16_t *w) {
    for (int k = 0; k < K; ++k) {
        int r = k / g;                             /* group row of k */
        for (int n = 0; n < N; ++n) {
            int q8 = codes[(size_t)k * N + n];
            int z8 = zeros ? zeros[(size_t)r * N + n] : 128;
            double scale = oracle_f16_to_f64(scales[(size_t)r * N + n]);
            double d = (double)(q8 - z8);          /* exact integer in [-255, 255] */
            w[(size_t)k * N + n] = f64_to_act(d * scale, dtype);
        }
    }
}

/*
 * Packed layout for 8-bit codes (restated from its specification in include/mpgemm.h):
 *
 * Codes plane, K*N bytes, one byte per code.  Tiles of 16 columns by 64 rows of k, 1 KiB
 * each; tile index T = (n/16)*(K/64) + k/64, so the tiles of one 16-column strip follow
 * each other along k.  Within a tile, with kk = k%64 and nn = n%16: lane L = nn +
 * 16*((kk%32)/8), step t = kk/32, and the code sits at byte L*16 + t*8 + kk%8 (k ascending
 * inside each 8-byte run).
 *
 * Meta plane: scales exactly as for 4-bit codes (fp16 at element index
 * (n/16)*(K/g)*16 + (k/g)*16 + n%16); then, for asymmetric codes only, the zeros as one
 * byte per element at the same index, (K/g)*N bytes.
 */
static size_t code8_byte_offset(int k, int n, int K) {
    size_t T = (size_t)(n / 16) * (size_t)(K / 64) + (size_t)(k / 64);
    int kk = k % 64, col = n % 16;
    int lane8 = col + 16 * ((kk % 32) / 8);
    return T * 1024 + (size_t)lane8 * 16 + (size_t)(kk / 32) * 8 + (size_t)(kk % 8);
}

size_t oracle_packed_code_bytes_w8(int K, int N) {
    return (size_t)oracle_padded_k(K) * oracle_padded_n(N);
}
size_t oracle_packed_meta_bytes_w8(int K, int N, int g, int symmetric) {
    size_t cells = (size_t)(oracle_padded_k(K) / g) * oracle_padded_n(N);
    return cells * 2 + (symmetric ? 0 : cells);
}

/* K, N: the user matrix; padding as for 4-bit codes (symmetric zero point 128). */
void oracle_pack_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                    int K, int N, int g, uint8_t *packed_codes, uint8_t *packed_meta) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    memset(packed_codes, 0, oracle_packed_code_bytes_w8(K, N));
    memset(packed_meta, 0, oracle_packed_meta_bytes_w8(K, N, g, zeros == NULL));
    for (int k = 0; k < Kp; ++k)
        for (int n = 0; n < N; ++n)
            packed_codes[code8_byte_offset(k, n, Kp)] =
                k < K ? codes[(size_t)k * N + n]
                      : (uint8_t)zero_point(zeros, k / g, n, N, rows, 128);
    uint16_t *meta_scales = (uint16_t *)packed_meta;
    uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            meta_scales[e] = scales[(size_t)r * N + n];
            if (zeros) meta_zeros[e] = zeros[(size_t)r * N + n];
        }
    }
}

/* Inverse of oracle_pack_w8 (the user [K][N] part).  zeros is written only for asymmetric
 * packing. */
void oracle_unpack_w8(const uint8_t *packed_codes, const uint8_t *packed_meta, int K, int N,
                      int g, int symmetric, uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            codes[(size_t)k * N + n] = packed_codes[code8_byte_offset(k, n, Kp)];
    const uint16_t *meta_scales = (const uint16_t *)packed_meta;
    const uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            scales[(size_t)r * N + n] = meta_scales[e];
            if (!symmetric && zeros) zeros[(size_t)r * N + n] = meta_zeros[e];
        }
    }
}

/* ------------------------------------------------------ FP8 weights (W-FP8 A16) --- */

/*
 * [TurboMind, Fig. 19 caption: an FP8 Qwen3 8B model served by the same engine].  The FP8
 * reading of the group form: each code is an 8-bit floating-point number, scaled by the
 * fp16 group scale with no zero point, and the product is rounded once:
 *   w = round_act(fp8(q) * s).
 * The product (at most a 4-bit significand times an 11-bit one) is exact in fp64.  The
 * codes are stored in the 8-bit packed layout with no zero plane.  Two OCP FP8 encodings:
 *   E4M3 (format 0): 1 sign, 4 exponent bits with bias 7, 3 fraction bits; exponent 0 is
 *                    subnormal; 0x7F and 0xFF are NaN; no infinities (largest 448).
 *   E5M2 (format 1): 1 sign, 5 exponent bits with bias 15, 2 fraction bits; exponent 0 is
 *                    subnormal; exponent 31 is infinity (fraction 0) or NaN.
 */
double oracle_e4m3_to_f64(uint8_t b) {
    int sign = b >> 7;
    int e = (b >> 3) & 0xf;
    int f = b & 0x7;
    double v;
    if (e == 15 && f == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)f, -9);                  /* subnormal: f/8 * 2^-6 */
    } else {
        v = ldexp((double)(8 + f), e - 10);        /* (1.f) * 2^(e-7) */
    }
    return sign ? -v : v;                          /* E4M3 sign bit */
}

double oracle_e5m2_to_f64(uint8_t b) {
    int neg = (b & 0x80) != 0;
    int ex = (b >> 2) & 0x1f;
    int fr = b & 0x3;
    double v;
    if (ex == 31) {
        v = fr ? NAN : INFINITY;
    } else if (ex == 0) {
        v = ldexp((double)fr, -16);                /* subnormal: fr/4 * 2^-14 */
    } else {
        v = ldexp((double)(4 + fr), ex - 17);      /* (1.fr) * 2^(ex-15) */
    }
    return neg ? -v : v;
}

void oracle_dequant_fp8(const uint8_t *codes, const uint16_t *scales, int K, int N, int g,
                        int format, int dtype, uint16_t *w) {
    for (int k = 0; k < K; ++k) {
        int row = k / g;
        for (int n = 0; n < N; ++n) {
            uint8_t q = codes[(size_t)k * N + n];
            double v = format == 1 ? oracle_e5m2_to_f64(q) : oracle_e4m3_to_f64(q);
            double scale = oracle_f16_to_f64(scales[(size_t)row * N + n]);
            w[(size_t)k * N + n] = f64_to_act(v * scale, dtype);
        }
    }
}

/* ------------------------------------------ 2-bit and 3-bit weights (sub-4-bit) --- */

/*
 * "Progressive Mixed-Precision Decoding for Efficient LLM Inference" (arXiv 2410.13461),
 * abstract: 2/3-bit weights relieve the memory-boundedness of decoding; here with the
 * [TurboMind] pipeline.  The same group form with b-bit codes (b = 2 or 3):
 *   w = round_act((q - z) * s),  q, z in 0..2^b - 1,  z = 2^(b-1) for symmetric codes.
 *   codes uint8 [K][N] (low b bits used); scales fp16 [ceil(K/g)][N]; zeros uint8 of the
 *   same shape (low b bits used) or NULL.
 */
void oracle_dequant_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                           const uint8_t *zeros, int K, int N, int g, int dtype, uint16_t *w) {
    const int cmask = (1 << bits) - 1;
    for (int k = 0; k < K; ++k) {
        int gr = k / g;
        for (int n = 0; n < N; ++n) {
            int qb = codes[(size_t)k * N + n] & cmask;
            int zb = zeros ? (zeros[(size_t)gr * N + n] & cmask) : (1 << (bits - 1));
            double sb = oracle_f16_to_f64(scales[(size_t)gr * N + n]);
            w[(size_t)k * N + n] = f64_to_act((double)(qb - zb) * sb, dtype);
        }
    }
}

/*
 * Packed sub-4-bit layout (restated from its specification in include/mpgemm.h).  Tiles of
 * 16 columns x 128 rows of k over the padded matrix (Kp x Np as for 4-bit codes), 4*b
 * bytes per lane and 256*b bytes per tile; tile T = (n/16)*(Kp/128) + k/128.  With
 * kk = k%128 and nn = n%16: lane L = nn + 16*((kk%32)/8), step t = kk/32, element
 * i = kk%8; the lane's b little-endian 32-bit words start at byte T*256*b + L*4*b.  The
 * element belongs to pair register r = 4t + i/2, in its low 16-bit half for even i and its
 * high half for odd i (half offset h = 16*(i%2)).
 *   b = 2: word r/8; field of 2 bits at bit h + 2*((r%8)%4) + 8*((r%8)/4).
 *   b = 3: r < 15: word r/5, field of 3 bits at bit h + 3*(r%5).  r = 15: bit c (c = 0..2)
 *          of the code sits in word c at bit h + 15.
 * Meta plane exactly as for 4-bit codes (fp16 scales, then 4-bit zeros), padding as there
 * (padded rows of real columns carry the zero point, 2 or 4 when symmetric).
 */
size_t oracle_packed_code_bytes_lowbit(int bits, int K, int N) {
    return (size_t)oracle_padded_k(K) * oracle_padded_n(N) * bits / 8;
}

/* Sets code q of padded element (k, n) in the plane (which starts zeroed). */
static void put_lowbit(uint8_t *plane, int bits, int k, int n, int Kp, uint32_t q) {
    size_t T = (size_t)(n / 16) * (size_t)(Kp / 128) + (size_t)(k / 128);
    int kk = k % 128, L = n % 16 + 16 * ((kk % 32) / 8), t = kk / 32, i = kk % 8;
    int r = 4 * t + i / 2, h = 16 * (i % 2);
    uint8_t *lane_words = plane + T * 256 * bits + (size_t)L * 4 * bits;
    for (int c = 0; c < bits; ++c) {
        int word, bit;
        if (bits == 2) {
            word = r / 8;
            bit = h + 2 * ((r % 8) % 4) + 8 * ((r % 8) / 4) + c;
        } else if (r < 15) {
            word = r / 5;
            bit = h + 3 * (r % 5) + c;
        } else {
            word = c;
            bit = h + 15;
        }
        if ((q >> c) & 1u) lane_words[4 * word + bit / 8] |= (uint8_t)(1u << (bit % 8));
    }
}

static uint32_t get_lowbit(const uint8_t *plane, int bits, int k, int n, int Kp) {
    size_t T = (size_t)(n / 16) * (size_t)(Kp / 128) + (size_t)(k / 128);
    int kk = k % 128, L = n % 16 + 16 * ((kk % 32) / 8), t = kk / 32, i = kk % 8;
    int r = 4 * t + i / 2, h = 16 * (i % 2);
    const uint8_t *lane_words = plane + T * 256 * bits + (size_t)L * 4 * bits;
    uint32_t q = 0;
    for (int c = 0; c < bits; ++c) {
        int word, bit;
        if (bits == 2) {
            word = r / 8;
            bit = h + 2 * ((r % 8) % 4) + 8 * ((r % 8) / 4) + c;
        } else if (r < 15) {
            word = r / 5;
            bit = h + 3 * (r % 5) + c;
        } else {
            word = c;
            bit = h + 15;
        }
        q |= (uint32_t)((lane_words[4 * word + bit / 8] >> (bit % 8)) & 1u) << c;
    }
    return q;
}

void oracle_pack_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                        const uint8_t *zeros, int K, int N, int g, uint8_t *packed_codes,
                        uint8_t *packed_meta) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    const int cmask = (1 << bits) - 1;
    memset(packed_codes, 0, oracle_packed_code_bytes_lowbit(bits, K, N));
    memset(packed_meta, 0, oracle_packed_meta_bytes(K, N, g, zeros == NULL));
    for (int k = 0; k < Kp; ++k)
        for (int n = 0; n < N; ++n) {
            uint32_t q = k < K ? codes[(size_t)k * N + n]
                               : (uint32_t)zero_point(zeros, k / g, n, N, rows, 1 << (bits - 1));
            put_lowbit(packed_codes, bits, k, n, Kp, q & (uint32_t)cmask);
        }
    uint16_t *meta_scales = (uint16_t *)packed_meta;
    uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r)
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            meta_scales[e] = scales[(size_t)r * N + n];
            if (zeros) {
                uint8_t z = zeros[(size_t)r * N + n] & (uint8_t)cmask;
                meta_zeros[e / 2] |= (uint8_t)((e % 2) ? (z << 4) : z);
            }
        }
}

void oracle_unpack_lowbit(int bits, const uint8_t *packed_codes, const uint8_t *packed_meta,
                          int K, int N, int g, int symmetric, uint8_t *codes, uint16_t *scales,
                          uint8_t *zeros) {
    const int Kp = oracle_padded_k(K), Np = oracle_padded_n(N), rows = groups_of(K, g);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            codes[(size_t)k * N + n] = (uint8_t)get_lowbit(packed_codes, bits, k, n, Kp);
    const uint16_t *meta_scales = (const uint16_t *)packed_meta;
    const uint8_t *meta_zeros = packed_meta + (size_t)(Kp / g) * Np * 2;
    for (int r = 0; r < rows; ++r)
        for (int n = 0; n < N; ++n) {
            size_t e = meta_index(r * g, n, Kp, g);
            scales[(size_t)r * N + n] = meta_scales[e];
            if (!symmetric && zeros) {
                uint8_t b = meta_zeros[e / 2];
                zeros[(size_t)r * N + n] = (uint8_t)((e % 2) ? (b >> 4) : (b & 0xf));
            }
        }
}

/* ------------------------------------------- attention decode over an 8-bit KV cache --- */

/*
 * [TurboMind, Fig. 4 caption: the attention pipeline dequantizes the low-bit KV cache to
 * FP16 by I2F scaling; Fig. 10 caption: KV is processed in 64-token macro-tiles].  The
 * reading taken: 8-bit codes with one asymmetric scale (fp16) and zero (uint8) per
 * (token, KV head), dequantized and rounded once to the activation format,
 *   k[t][d] = round_act((kc[t][d] - kz[t]) * ks[t]),  v likewise,
 * then exact attention for one query token per sequence (decode), grouped-query heads
 * (query head h reads KV head h / (Hq / Hkv)):
 *   score[t] = (sum_d q[h][d] * k[t][d]) * scale,  p = softmax over t < len[b],
 *   o[h][d] = round_act(sum_t p[t] * v[t][d]),  all in fp64.  len[b] == 0 gives zeros.
 * Layouts (user form): q, o [B][Hq][D] activation bits; kc, vc [B][Tmax][Hkv][D] uint8;
 * ks, vs [B][Tmax][Hkv] fp16 bits; kz, vz [B][Tmax][Hkv] uint8; lens [B].
 */
void oracle_attention_decode_kv8(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                                 const uint8_t *kz, const uint8_t *vc, const uint16_t *vs,
                                 const uint8_t *vz, const int *lens, int B, int Hq, int Hkv,
                                 int D, int Tmax, float scale, int dtype, uint16_t *o) {
    const int group = Hq / Hkv;
    double *score = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        const int len = lens[b];
        for (int h = 0; h < Hq; ++h) {
            const int hk = h / group;
            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;
            double mx = -INFINITY;
            for (int t = 0; t < len; ++t) {
                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;
                const double s_k = oracle_f16_to_f64(ks[row]);
                double dot = 0.0;
                for (int d = 0; d < D; ++d) {
                    double kd = act_to_f64(
                        f64_to_act((double)((int)kc[row * D + d] - (int)kz[row]) * s_k, dtype), dtype);
                    dot += act_to_f64(qh[d], dtype) * kd;
                }
                score[t] = dot * (double)scale;
                if (score[t] > mx) mx = score[t];
            }
            double denom = 0.0;
            for (int t = 0; t < len; ++t) {
                score[t] = exp(score[t] - mx);
                denom += score[t];
            }
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int t = 0; t < len; ++t) {
                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;
                const double s_v = oracle_f16_to_f64(vs[row]);
                const double pt = score[t] / denom;
                for (int d = 0; d < D; ++d) {
                    double vd = act_to_f64(
                        f64_to_act((double)((int)vc[row * D + d] - (int)vz[row]) * s_v, dtype), dtype);
                    acc[d] += pt * vd;
                }
            }
            uint16_t *oh = o + ((size_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) oh[d] = f64_to_act(acc[d], dtype);
        }
    }
    free(score);
    free(acc);
}

/*
 * The same attention over an FP8 KV cache: k[t][d] = round_act(fp8(kc[t][d]) * ks[t]),
 * v alike, fp8 in the OCP format `format` (0 = E4M3, 1 = E5M2; see the FP8 weights above),
 * no zero points.  The other arguments and the arithmetic as oracle_attention_decode_kv8.
 */
void oracle_attention_decode_kvfp8(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                                   const uint8_t *vc, const uint16_t *vs, const int *lens,
                                   int B, int Hq, int Hkv, int D, int Tmax, float scale,
                                   int format, int dtype, uint16_t *o) {
    const int group = Hq / Hkv;
    double *score = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        const int len = lens[b];
        for (int h = 0; h < Hq; ++h) {
            const int hk = h / group;
            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;
            double mx = -INFINITY;
            for (int t = 0; t < len; ++t) {
                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;
                const double sk8 = oracle_f16_to_f64(ks[row]);
                double dot = 0.0;
                for (int d = 0; d < D; ++d) {
                    uint8_t c8 = kc[row * D + d];
                    double e8 = format == 1 ? oracle_e5m2_to_f64(c8) : oracle_e4m3_to_f64(c8);
                    dot += act_to_f64(qh[d], dtype) * act_to_f64(f64_to_act(e8 * sk8, dtype), dtype);
                }
                score[t] = dot * (double)scale;
                if (score[t] > mx) mx = score[t];
            }
            double denom = 0.0;
            for (int t = 0; t < len; ++t) {
                score[t] = exp(score[t] - mx);
                denom += score[t];
            }
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int t = 0; t < len; ++t) {
                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;
                const double sv8 = oracle_f16_to_f64(vs[row]);
                const double pt = score[t] / denom;
                for (int d = 0; d < D; ++d) {
                    uint8_t c8 = vc[row * D + d];
                    double e8 = format == 1 ? oracle_e5m2_to_f64(c8) : oracle_e4m3_to_f64(c8);
                    acc[d] += pt * act_to_f64(f64_to_act(e8 * sv8, dtype), dtype);
                }
            }
            uint16_t *oh = o + ((size_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) oh[d] = f64_to_act(acc[d], dtype);
        }
    }
    free(score);
    free(acc);
}

/*
 * Packed KV cache (restated from its specification in include/mpgemm.h).  Blocks of 64
 * tokens of one sequence, all KV heads; block j of sequence b is cache block
 * table[b][j].  A head of D values (D a multiple of 16) is stored padded to
 * Dp = D rounded up to a multiple of 64, the k depth of one 8-bit tile, with codes 0 at
 * d >= D.  Within a block, KV head h occupies HB = 128*Dp + 384 bytes at h*HB:
 *   bytes [0, 64*Dp):       K codes of the 64 tokens, in the 8-bit weight layout of the
 *                           Dp x 64 matrix K^T (k = d, n = token);
 *   bytes [64*Dp, 128*Dp):  V codes, in the 8-bit weight layout of the 64 x Dp matrix V
 *                           (k = token, n = d) -- V stored transposed for the matrix cores;
 *   then K scales [64] fp16, V scales [64] fp16, K zeros [64] uint8, V zeros [64] uint8.
 */
static size_t kv_padded_d(int D) { return (size_t)(D + 63) / 64 * 64; }

size_t oracle_kv_block_bytes(int Hkv, int D) { return (size_t)Hkv * (128 * kv_padded_d(D) + 384); }

/* Writes tokens t0 .. t0 + n - 1 of one sequence (user form kc, vc [n][Hkv][D]; ks, vs,
 * kz, vz [n][Hkv]) into the cache through that sequence's block-table row, codes 0 in the
 * padding d = D .. Dp-1. */
void oracle_kv_pack(const uint8_t *kc, const uint16_t *ks, const uint8_t *kz, const uint8_t *vc,
                    const uint16_t *vs, const uint8_t *vz, int n, int t0, int Hkv, int D,
                    const int *table_row, uint8_t *cache) {
    const size_t Dp = kv_padded_d(D), HB = 128 * Dp + 384;
    for (int i = 0; i < n; ++i) {
        const int t = t0 + i, slot = t % 64;
        uint8_t *blk = cache + (size_t)table_row[t / 64] * oracle_kv_block_bytes(Hkv, D);
        for (int h = 0; h < Hkv; ++h) {
            uint8_t *hb = blk + h * HB;
            const size_t row = (size_t)i * Hkv + h;
            for (int d = 0; d < (int)Dp; ++d) {
                hb[code8_byte_offset(d, slot, (int)Dp)] = d < D ? kc[row * D + d] : 0;
                hb[64 * Dp + code8_byte_offset(slot, d, 64)] = d < D ? vc[row * D + d] : 0;
            }
            uint16_t *sc = (uint16_t *)(hb + 128 * Dp);
            sc[slot] = ks[row];
            sc[64 + slot] = vs[row];
            hb[128 * Dp + 256 + slot] = kz[row];
            hb[128 * Dp + 320 + slot] = vz[row];
        }
    }
}

/* Reads tokens 0 .. T - 1 of one sequence back into the user form. */
void oracle_kv_unpack(const uint8_t *cache, const int *table_row, int T, int Hkv, int D,
                      uint8_t *kc, uint16_t *ks, uint8_t *kz, uint8_t *vc, uint16_t *vs,
                      uint8_t *vz) {
    const size_t Dp = kv_padded_d(D), HB = 128 * Dp + 384;
    for (int t = 0; t < T; ++t) {
        const int slot = t % 64;
        const uint8_t *blk = cache + (size_t)table_row[t / 64] * oracle_kv_block_bytes(Hkv, D);
        for (int h = 0; h < Hkv; ++h) {
            const uint8_t *hb = blk + h * HB;
            const size_t row = (size_t)t * Hkv + h;
            for (int d = 0; d < D; ++d) {
                kc[row * D + d] = hb[code8_byte_offset(d, slot, (int)Dp)];
                vc[row * D + d] = hb[64 * Dp + code8_byte_offset(slot, d, 64)];
            }
            const uint16_t *sc = (const uint16_t *)(hb + 128 * Dp);
            ks[row] = sc[slot];
            vs[row] = sc[64 + slot];
            kz[row] = hb[128 * Dp + 256 + slot];
            vz[row] = hb[128 * Dp + 320 + slot];
        }
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
