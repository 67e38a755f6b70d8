/*
 * bg_oracle.c -- plain CPU oracle for the W4A16 / W8A8 quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP kernels.
 *
 * Everything here is written as the plain definition of what the pages state,
 * step by step, with no blocking, fusion or reordering:
 *
 *   [LPI]  "Low-precision LLM inference: FP8/INT8/INT4/FP4 kernels and
 *          calibration (8/10)", blog.ruahverce.com
 *   [AIB]  "Quantization throughput by method: why W4A16 is overtaken by W8A8
 *          as batch grows", hrletsgo.me
 *
 * Floating-point discipline: build with -O2 -ffp-contract=off and without any
 * fast-math flag, on an SSE2 target (FLT_EVAL_METHOD == 0), so that every
 * float expression below is one IEEE-754 binary32 operation, correctly
 * rounded, and every double expression one binary64 operation.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *  - round() is round-half-to-even (rintf in the default rounding mode);
 *  - x/s is an IEEE correctly rounded binary32 division;
 *  - the INT4 codes are computed with the *stored* FP16-rounded group scale;
 *  - symmetric qmax is 7 (INT4) / 127 (INT8) / 448 (FP8 E4M3);
 *  - asymmetric INT4: range widened to include 0, s=(max-min)/15,
 *    z=clamp(round(-min/s),0,15);
 *  - an all-zero unit gets scale 1 (for the binary32 W8A8 scales: any scale
 *    that comes out 0, which also covers amax/qmax underflowing); an FP16
 *    scale that would round to 0 or overflow is clamped to [2^-24, 65504];
 *  - FP8 is OCP E4M3 "FN" (bias 7, max 448, no Inf, S.1111.111 = NaN), cast
 *    with round-to-nearest-even and saturation to +-448; NaN maps to NaN.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

/* granularity codes: same numbering as the public header, restated here */
enum { ORC_GRAN_TENSOR = 0, ORC_GRAN_ROW = 1, ORC_GRAN_ROW_G128 = 2, ORC_GRAN_BLOCK128 = 3 };

/* ------------------------------------------------------------------------ */
/* IEEE binary16 and bfloat16 codecs, from the format definitions.           */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = m ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);                  /* subnormal: m * 2^-24 */
    } else {
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    }
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest binary16, ties to even.
 * The value is exact in double; within its binade the binary16 quantum is
 * 2^(e-10) (e clamped to >= -14 for subnormals), so the rounded magnitude is
 * rint(|f| / quantum) * quantum.  Magnitudes that round to >= 2^16 overflow. */
uint16_t orc_f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return sign | 0x7E00;
    double a = fabs((double)f);
    if (isinf(f)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);          /* a = fr * 2^e, fr in [0.5,1): binade exponent e-1 */
    e -= 1;
    if (e < -14) e = -14;
    double quantum = ldexp(1.0, e - 10);
    double r = rint(a / quantum) * quantum;       /* RNE in double: exact */
    if (r >= 65536.0) return sign | 0x7C00;       /* overflow to infinity */
    if (r < ldexp(1.0, -14)) {                    /* subnormal or zero */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    }
    int er;
    frexp(r, &er);
    er -= 1;
    uint16_t frac = (uint16_t)((r / ldexp(1.0, er) - 1.0) * 1024.0);
    return sign | (uint16_t)((er + 15) << 10) | frac;
}

/* bfloat16 is the upper half of a binary32. */
float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.        */
/* Normal: 2^(e-7) * (1 + m/8), e = 1..15, except S.1111.111 which is NaN.   */
/* Subnormal: 2^-6 * m/8.  Largest finite 448.  No infinities.              */
/* [LPI] §7 "FP8 is a small floating point" (E4M3 = 1/4/3 bits; the variant */
/* must be pinned), Micikevicius et al. as cited there.                      */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Saturating round-to-nearest-even cast.  NaN -> 0x7F|sign; |v| >= 448
 * (including infinity) -> 448 with sign.  Otherwise the quantum of the
 * binade is 2^(e-3) with e clamped to >= -6 (the subnormal quantum is
 * 2^-9), and the magnitude is rint(|v| / quantum) * quantum.  Anything that
 * would round above 448 saturates to 448. */
uint8_t orc_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v)) return sign | 0x7F;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < -6) e = -6;
    double quantum = ldexp(1.0, e - 3);
    double r = rint(a / quantum) * quantum;
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    int er;
    frexp(r, &er);
    er -= 1;
    uint8_t mant = (uint8_t)((r / ldexp(1.0, er) - 1.0) * 8.0);
    return sign | (uint8_t)((er + 7) << 3) | mant;
}

/* ------------------------------------------------------------------------ */
/* INT4 weight quantization, group size G along K, FP16 scales.              */
/* [LPI] §2 eq. (1) q = clamp(round(x/s) + z, qmin, qmax), eq. (2)          */
/* x^ = s(q - z); §3 symmetric s = max|x| / qmax (eq. 3) and asymmetric      */
/* (observed min/max); §4 per-group scales; §5 one FP16 scale per 128.      */
/* ------------------------------------------------------------------------ */

/* The FP16 scale of one group: value v (binary32) rounded to binary16; an
 * all-zero group gets 1; results outside [2^-24, 65504] are clamped. */
static uint16_t group_scale_f16(float v, int all_zero) {
    if (all_zero) return 0x3C00;                  /* 1.0 */
    uint16_t h = orc_f32_to_f16(v);
    if (h == 0x0000) h = 0x0001;                  /* 2^-24 */
    if (h == 0x7C00) h = 0x7BFF;                  /* 65504 */
    return h;
}

/* Quantize W [N][K] (binary32) into unsigned 4-bit codes u [N][K] (0..15),
 * FP16 scale bits s16 [N][K/G] and zero-points z [N][K/G].
 * Symmetric: z = 8 is implied (u = q + 8); asymmetric: z explicit. */
void orc_w4_quantize(const float* w, int64_t N, int64_t K, int G, int asym,
                     uint8_t* u, uint16_t* s16, uint8_t* z) {
    int64_t ng = K / G;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ng; ++g) {
            const float* wg = w + n * K + g * G;
            uint8_t* ug = u + n * K + g * G;
            if (!asym) {
                float amax = 0.0f;
                for (int i = 0; i < G; ++i) {
                    float a = fabsf(wg[i]);
                    if (a > amax) amax = a;
                }
                uint16_t sh = group_scale_f16(amax / 7.0f, amax == 0.0f);
                float s = orc_f16_to_f32(sh);
                s16[n * ng + g] = sh;
                z[n * ng + g] = 8;
                for (int i = 0; i < G; ++i) {
                    float q = rintf(wg[i] / s);
                    if (q < -8.0f) q = -8.0f;
                    if (q > 7.0f) q = 7.0f;
                    ug[i] = (uint8_t)((int)q + 8);
                }
            } else {
                float mn = 0.0f, mx = 0.0f;               /* range includes 0 */
                for (int i = 0; i < G; ++i) {
                    if (wg[i] < mn) mn = wg[i];
                    if (wg[i] > mx) mx = wg[i];
                }
                float range = mx - mn;
                uint16_t sh = group_scale_f16(range / 15.0f, range == 0.0f);
                float s = orc_f16_to_f32(sh);
                float zf = rintf(-mn / s);
                if (zf < 0.0f) zf = 0.0f;
                if (zf > 15.0f) zf = 15.0f;
                s16[n * ng + g] = sh;
                z[n * ng + g] = (uint8_t)zf;
                for (int i = 0; i < G; ++i) {
                    float q = rintf(wg[i] / s) + zf;
                    if (q < 0.0f) q = 0.0f;
                    if (q > 15.0f) q = 15.0f;
                    ug[i] = (uint8_t)q;
                }
            }
        }
    }
}

/* Packed layout -- a layout the page leaves to the target kernel ([LPI] §24:
 * "is the weight packing order the one the kernel expects"; §11 pipeline:
 * quantize, pack and lay out for the target kernel).  Weights are cut into
 * tiles of 16 output channels x one group of G = 128 input channels; a tile is
 * 1 KB of codes stored contiguously as 64 slots of 16 bytes.  For weight
 * (n, k):  t = n / 16, r = n % 16, g = k / 128, c = k % 128,
 *          slot = 16 * (c / 32) + r,  word = (c % 32) / 8,  i = k % 8,
 *   qweight[((t * (K/128) + g) * 64 + slot) * 4 + word], nibble i/2 for even
 *   i and 4 + i/2 for odd i (even k in the low half-word, odd k in the high);
 *   scales[(t * (K/128) + g) * 16 + r]   (FP16 bits);
 *   zeros [(t * (K/256) + g/2) * 16 + r], low nibble for even g, high for odd.
 * Requires N % 16 == 0 and K % 256 == 0. */
static int nibble_of_k(int i) { return (i % 2 == 0) ? i / 2 : 4 + i / 2; }

static int64_t word_index(int64_t n, int64_t k, int64_t K) {
    int64_t t = n / 16, r = n % 16, g = k / 128, c = k % 128;
    int64_t slot = 16 * (c / 32) + r, word = (c % 32) / 8;
    return ((t * (K / 128) + g) * 64 + slot) * 4 + word;
}

void orc_w4_pack(const uint8_t* u, const uint16_t* s16_rowmajor, const uint8_t* z, int64_t N, int64_t K,
                 int asym, uint32_t* qweight, uint16_t* scales, uint8_t* zeros) {
    int64_t ng = K / 128;
    for (int64_t i = 0; i < N * K / 8; ++i) qweight[i] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k)
            qweight[word_index(n, k, K)] |= (uint32_t)(u[n * K + k] & 0xF) << (4 * nibble_of_k((int)(k % 8)));
        for (int64_t g = 0; g < ng; ++g) {
            int64_t t = n / 16, r = n % 16;
            scales[(t * ng + g) * 16 + r] = s16_rowmajor[n * ng + g];
            if (asym) {
                int64_t zi = (t * (ng / 2) + g / 2) * 16 + r;
                if (g % 2 == 0) zeros[zi] = (uint8_t)(z[n * ng + g] & 0xF);
                else zeros[zi] |= (uint8_t)((z[n * ng + g] & 0xF) << 4);
            }
        }
    }
}

/* Inverse of orc_w4_pack: codes u [N][K], scale bits [N][K/128] and
 * zero-points [N][K/128] (8 when zeros == NULL) in row-major order. */
void orc_w4_unpack(const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                   uint8_t* u, uint16_t* s16, uint8_t* z) {
    int64_t ng = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = n / 16, r = n % 16;
        for (int64_t k = 0; k < K; ++k)
            u[n * K + k] = (uint8_t)((qweight[word_index(n, k, K)] >> (4 * nibble_of_k((int)(k % 8)))) & 0xF);
        for (int64_t g = 0; g < ng; ++g) {
            s16[n * ng + g] = scales[(t * ng + g) * 16 + r];
            z[n * ng + g] = zeros ? (uint8_t)((zeros[(t * (ng / 2) + g / 2) * 16 + r] >> (4 * (g % 2))) & 0xF) : 8;
        }
    }
}

/* Dequantized weight from the packed form: w^[n,k] = s16 * (u - z), exact
 * in double.  z = 8 when zeros == NULL (symmetric). */
void orc_w4_dequant(const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                    int64_t N, int64_t K, int G, double* what) {
    (void)G;
    int64_t ng = K / 128;
    uint8_t* u = (uint8_t*)malloc((size_t)(N * K));
    uint16_t* s16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * ng));
    uint8_t* z = (uint8_t*)malloc((size_t)(N * ng));
    orc_w4_unpack(qweight, scales, zeros, N, K, u, s16, z);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            what[n * K + k] = (double)orc_f16_to_f32(s16[n * ng + k / 128]) * (double)((int)u[n * K + k] - (int)z[n * ng + k / 128]);
    free(u);
    free(s16);
    free(z);
}

/* W4A16 linear: Y[m,n] = sum_k x[m,k] * w^[n,k], in double, where x is the
 * exact value of the FP16 or BF16 activation.  [AIB] "W4A16" section (INT4
 * storage, dequantized just before a 16-bit GEMM); [LPI] §11 weight-only
 * INT4.  Y = X W^T with W stored [N][K]. */
void orc_gemm_w4a16(const uint16_t* x_bits, int x_is_bf16, int64_t M, int64_t K,
                    const uint32_t* qweight, const uint16_t* s16, const uint8_t* zeros,
                    int64_t N, int G, double* y) {
    double* what = (double*)malloc(sizeof(double) * (size_t)(N * K));
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
    orc_w4_dequant(qweight, s16, zeros, N, K, G, what);
    for (int64_t i = 0; i < M * K; ++i)
        xd[i] = x_is_bf16 ? (double)orc_bf16_to_f32(x_bits[i]) : (double)orc_f16_to_f32(x_bits[i]);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * what[n * K + k];
            y[m * N + n] = acc;
        }
    }
    free(what);
    free(xd);
}

/* ------------------------------------------------------------------------ */
/* Dynamic activation / weight quantizers for W8A8.                          */
/* Scale per unit: s = amax / qmax in binary32 (qmax 127 for INT8, 448 for  */
/* E4M3); a zero scale (all-zero unit, or amax/qmax underflow) becomes 1.  INT8: q = clamp(round(x/s),-128,127)*/
/* ([LPI] §2 eq. 1 with z = 0, §3 eq. 3).  FP8: q = e4m3_sat_rne(x/s)       */
/* ([LPI] §8 "Current scaling" and "Block scaling": scale = amax / max_fp8). */
/* Units ([LPI] §4): TENSOR = whole [R][C]; ROW = one row (per token, or per */
/* output channel of a weight); ROW_G128 = 1x128 along a row; BLOCK128 =    */
/* 128x128 tiles.  Scale layouts: TENSOR -> s[0] = scale, s[1] = amax;      */
/* ROW -> s[R]; ROW_G128 -> s[R][C/128]; BLOCK128 -> s[R/128][C/128].        */
/* ------------------------------------------------------------------------ */

static int64_t unit_of(int gran, int64_t r, int64_t c, int64_t C) {
    switch (gran) {
        case ORC_GRAN_TENSOR: return 0;
        case ORC_GRAN_ROW: return r;
        case ORC_GRAN_ROW_G128: return r * (C / 128) + c / 128;
        default: return (r / 128) * (C / 128) + c / 128;
    }
}

static int64_t n_units(int gran, int64_t R, int64_t C) {
    switch (gran) {
        case ORC_GRAN_TENSOR: return 1;
        case ORC_GRAN_ROW: return R;
        case ORC_GRAN_ROW_G128: return R * (C / 128);
        default: return (R / 128) * (C / 128);
    }
}

/* amax per unit, then scale per unit.  Returns a malloc'd array of the
 * binary32 scales (one per unit); writes them in the public layout. */
static float* unit_scales(const float* x, int64_t R, int64_t C, int gran, float qmax, float* s_out) {
    int64_t nu = n_units(gran, R, C);
    float* amax = (float*)calloc((size_t)nu, sizeof(float));
    float* s = (float*)malloc(sizeof(float) * (size_t)nu);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            float a = fabsf(x[r * C + c]);
            int64_t uidx = unit_of(gran, r, c, C);
            if (a > amax[uidx]) amax[uidx] = a;
        }
    for (int64_t i = 0; i < nu; ++i) {
        s[i] = amax[i] / qmax;
        if (s[i] == 0.0f) s[i] = 1.0f;     /* all-zero unit (or amax/qmax underflows) */
    }
    if (gran == ORC_GRAN_TENSOR) {
        s_out[0] = s[0];
        s_out[1] = amax[0];
    } else {
        for (int64_t i = 0; i < nu; ++i) s_out[i] = s[i];
    }
    free(amax);
    return s;
}

void orc_quant_int8(const float* x, int64_t R, int64_t C, int gran, int8_t* q, float* s_out) {
    float* s = unit_scales(x, R, C, gran, 127.0f, s_out);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            float v = rintf(x[r * C + c] / s[unit_of(gran, r, c, C)]);
            if (v < -128.0f) v = -128.0f;
            if (v > 127.0f) v = 127.0f;
            q[r * C + c] = (int8_t)v;
        }
    free(s);
}

void orc_quant_fp8(const float* x, int64_t R, int64_t C, int gran, uint8_t* q, float* s_out) {
    float* s = unit_scales(x, R, C, gran, 448.0f, s_out);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            q[r * C + c] = orc_e4m3_encode(x[r * C + c] / s[unit_of(gran, r, c, C)]);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* W8A8 GEMMs.  [AIB] "W8A8 / FP8" section (native INT8/FP8 GEMM, no upcast)*/
/* and [LPI] §22 (INT32 / FP32 accumulators).  A [M][K], W [N][K], Y=A W^T. */
/* ------------------------------------------------------------------------ */

/* Exact integer accumulators.  Returns 0 on success, 1 if some accumulator
 * does not fit in int32 (then acc holds the low 32 bits). */
int orc_gemm_i8_acc(const int8_t* a, const int8_t* w, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k) t += (int64_t)a[m * K + k] * (int64_t)w[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)t;
        }
    }
    return overflow;
}

/* The scale that applies to element (r, kidx) of an operand quantized with
 * granularity gran (the public scale layout). */
static double scale_at(const float* s, int gran, int64_t r, int64_t kidx, int64_t C) {
    switch (gran) {
        case ORC_GRAN_TENSOR: return (double)s[0];
        case ORC_GRAN_ROW: return (double)s[r];
        case ORC_GRAN_ROW_G128: return (double)s[r * (C / 128) + kidx / 128];
        default: return (double)s[(r / 128) * (C / 128) + kidx / 128];
    }
}

/* Y[m,n] = sum_k (dec(a[m,k]) * s_a) * (dec(w[n,k]) * s_w) in double, where
 * dec is the integer value (INT8) or the E4M3 value (FP8), and each scale is
 * the one the granularity assigns to that element.  This is the exact
 * dequantized GEMM; for per-row/per-tensor scales it equals
 * acc * s_a[m] * s_w[n], and for block scales it equals the sum over 128-wide
 * K blocks of the block partial sum times s_a[m,kb] * s_w[n/128,kb]. */
void orc_gemm_w8a8(const void* a, const float* a_s, int a_gran,
                   const void* w, const float* w_s, int w_gran,
                   int is_fp8, int64_t M, int64_t N, int64_t K, double* y) {
    double* ad = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double v = is_fp8 ? orc_e4m3_decode(((const uint8_t*)a)[m * K + k])
                              : (double)((const int8_t*)a)[m * K + k];
            ad[m * K + k] = v * scale_at(a_s, a_gran, m, k, K);
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double v = is_fp8 ? orc_e4m3_decode(((const uint8_t*)w)[n * K + k])
                              : (double)((const int8_t*)w)[n * K + k];
            wd[n * K + k] = v * scale_at(w_s, w_gran, n, k, K);
        }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += ad[m * K + k] * wd[n * K + k];
            y[m * N + n] = acc;
        }
    free(ad);
    free(wd);
}

/* W4A8 linear (the variant between W4A16 and W8A8: INT4 weights, dynamic
 * INT8 activations).  [LPI] §1 (the W4A8 row of the notation table and its
 * precision manifest: INT32/FP32 accumulation, BF16 or FP16 output), §14
 * (per-token activation scales), §20 and self-check Q2 (W4A8 lowers the
 * activations to 8 bits for a native low-precision GEMM; the INT4 weights
 * are dequantized on the way).  With a[m,k] the INT8 code of the
 * activation, s_a its scale (per row, or one per tensor) and w^ the dequantized
 * weight s16 * (u - z) of the packed form, the layer is the exact dequantized
 * product Y[m,n] = sum_k (a[m,k] * s_a) * w^[n,k], in double. */
void orc_gemm_w4a8(const int8_t* a, const float* a_s, int a_gran, int64_t M, int64_t K,
                   const uint32_t* qweight, const uint16_t* s16, const uint8_t* zeros,
                   int64_t N, int G, double* y) {
    double* what = (double*)malloc(sizeof(double) * (size_t)(N * K));
    double* ad = (double*)malloc(sizeof(double) * (size_t)(M * K));
    orc_w4_dequant(qweight, s16, zeros, N, K, G, what);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            ad[m * K + k] = (double)a[m * K + k] * scale_at(a_s, a_gran, m, k, K);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += ad[m * K + k] * what[n * K + k];
            y[m * N + n] = acc;
        }
    }
    free(what);
    free(ad);
}

/* ------------------------------------------------------------------------ */
/* SmoothQuant fold.  [LPI] §15: Y = X W^T = (X S^-1)(W S)^T for a diagonal  */
/* S over the input channels; S comes from calibration statistics and a      */
/* smoothing strength and is folded into the static weights, so the         */
/* activations reach the quantizer with their outlier channels shrunk.  The  */
/* page gives no formula for S; the reading here is the SmoothQuant rule     */
/* s_j = amax_x[j]^alpha / amax_w[j]^(1-alpha) (binary64, rounded once to    */
/* binary32), with s_j = 1 where either column maximum is 0.                 */
/* ------------------------------------------------------------------------ */

/* Column maxima |x[:, j]| of a binary32 matrix [R][C]. */
void orc_col_amax(const float* x, int64_t R, int64_t C, float* amax) {
    for (int64_t j = 0; j < C; ++j) amax[j] = 0.0f;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t j = 0; j < C; ++j) {
            float a = fabsf(x[r * C + j]);
            if (a > amax[j]) amax[j] = a;
        }
}

void orc_smooth_scales(const float* amax_x, const float* amax_w, int64_t C, double alpha, float* s) {
    for (int64_t j = 0; j < C; ++j) {
        if (amax_x[j] == 0.0f || amax_w[j] == 0.0f) {
            s[j] = 1.0f;
            continue;
        }
        s[j] = (float)(pow((double)amax_x[j], alpha) / pow((double)amax_w[j], 1.0 - alpha));
    }
}

/* out[r][j] = x[r][j] * m[j], one binary32 multiplication per element (X S^-1
 * with m = 1/s, or W S with m = s). */
void orc_col_mul(const float* x, int64_t R, int64_t C, const float* m, float* out) {
    for (int64_t r = 0; r < R; ++r)
        for (int64_t j = 0; j < C; ++j) out[r * C + j] = x[r * C + j] * m[j];
}

/* ------------------------------------------------------------------------ */
/* MXFP8: microscaled E4M3.  [LPI] §10: the OCP MX specification treats a   */
/* block of elements and its shared scale as one data format.  The block,    */
/* scale type and conversion are the OCP MX v1.0 ones (the pages name the    */
/* specification without restating it): 32 consecutive elements along K     */
/* share an E8M0 scale X = 2^(E - 127); E = floor(log2(max |v|)) - 8 + 127   */
/* (8 = the largest E4M3 exponent), clamped to 0..254, and every element is  */
/* the saturating RNE E4M3 cast of v / X.  An all-zero block gets X = 1;    */
/* a block holding an infinity gets E = 254 (log2 of it is infinite).       */
/* Scales are stored [rows][cols/32].                                        */
/* ------------------------------------------------------------------------ */

void orc_quant_mxfp8(const float* x, int64_t R, int64_t C, uint8_t* q, uint8_t* e8m0) {
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < C / 32; ++b) {
            const float* v = x + r * C + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            int e = 127;
            if (isinf(amax)) e = 254;          /* floor(log2 inf) = inf: the clamp's top */
            else if (amax > 0.0f) {
                e = ilogbf(amax) - 8 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            e8m0[r * (C / 32) + b] = (uint8_t)e;
            for (int i = 0; i < 32; ++i) q[r * C + b * 32 + i] = orc_e4m3_encode(ldexpf(v[i], 127 - e));
        }
}

/* Y[m,n] = sum_k (dec(a[m,k]) X_a[m,k/32]) (dec(w[n,k]) X_w[n,k/32]) in double
 * (exact: every term is a product of two E4M3 values and powers of two). */
void orc_gemm_mxfp8(const uint8_t* a, const uint8_t* ea, const uint8_t* w, const uint8_t* ew, int64_t M, int64_t N,
                    int64_t K, double* y) {
    double* ad = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            ad[m * K + k] = orc_e4m3_decode(a[m * K + k]) * ldexp(1.0, (int)ea[m * (K / 32) + k / 32] - 127);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            wd[n * K + k] = orc_e4m3_decode(w[n * K + k]) * ldexp(1.0, (int)ew[n * (K / 32) + k / 32] - 127);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += ad[m * K + k] * wd[n * K + k];
            y[m * N + n] = acc;
        }
    free(ad);
    free(wd);
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element-wise array helpers for the Python wrapper.                        */
/* ------------------------------------------------------------------------ */

void orc_f32_to_f16_n(const float* x, int64_t n, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_n(const uint16_t* h, int64_t n, float* x) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_f16_to_f32(h[i]);
}

void orc_bf16_to_f32_n(const uint16_t* b, int64_t n, float* x) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_bf16_to_f32(b[i]);
}

/* ------------------------------------------------------------------------ */
/* MXFP4: microscaled E2M1.  [LPI] §10: E2M1 is the usual FP4 element (1     */
/* sign, 2 exponent, 1 mantissa bit), and the OCP MX specification makes a   */
/* block of such elements with one shared scale a data format (MXFP4).  As   */
/* for MXFP8, the block (32 consecutive elements along K), the E8M0 scale     */
/* and the conversion are the OCP MX v1.0 ones: E = floor(log2(max |v|)) - 2 */
/* + 127 (2 = the largest E2M1 exponent), clamped to 0..254, elements are    */
/* the saturating RNE E2M1 cast of v / X, an all-zero block gets X = 1 and  */
/* a block holding an infinity E = 254.                                     */
/* Two elements per byte, the even element in the low nibble.               */
/* ------------------------------------------------------------------------ */

/* E2M1: bias 1.  Exponent field 0 is subnormal (m * 0.5); otherwise         */
/* 2^(e-1) * (1 + m/2).  Values 0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf or NaN.   */
double orc_e2m1_decode(uint8_t c) {
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* Saturating round-to-nearest-even cast.  The quantum of the binade is     */
/* 2^(e-1) with e = floor(log2 |v|) clamped to >= 0 (the subnormal quantum   */
/* is 0.5); the magnitude is rint(|v| / quantum) * quantum, capped at 6.     */
/* The sign is kept (a negative value that rounds to zero is -0).  NaN has   */
/* no E2M1 code: it becomes a signed zero.                                   */
uint8_t orc_e2m1_encode(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    if (isnan(v)) return sign;
    double a = fabs((double)v);
    if (a >= 6.0) return sign | 7;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < 0) e = 0;
    double quantum = ldexp(1.0, e - 1);
    double r = rint(a / quantum) * quantum;
    if (r > 6.0) r = 6.0;
    if (r == 0.0) return sign;
    if (r < 1.0) return sign | 1;                      /* the one subnormal, 0.5 */
    int er;
    frexp(r, &er);
    er -= 1;
    uint8_t mant = (uint8_t)((r / ldexp(1.0, er) - 1.0) * 2.0);
    return sign | (uint8_t)((er + 1) << 1) | mant;
}

/* q: [R][C/2] bytes (element 2i in the low nibble of byte i of its row),
 * e8m0: [R][C/32]. */
void orc_quant_mxfp4(const float* x, int64_t R, int64_t C, uint8_t* q, uint8_t* e8m0) {
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < C / 32; ++b) {
            const float* v = x + r * C + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            int e = 127;
            if (isinf(amax)) e = 254;          /* floor(log2 inf) = inf: the clamp's top */
            else if (amax > 0.0f) {
                e = ilogbf(amax) - 2 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            e8m0[r * (C / 32) + b] = (uint8_t)e;
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = orc_e2m1_encode(ldexpf(v[i], 127 - e));
                uint8_t hi = orc_e2m1_encode(ldexpf(v[i + 1], 127 - e));
                q[r * (C / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

/* Y[m,n] = sum_k (dec(a[m,k]) X_a[m,k/32]) (dec(w[n,k]) X_w[n,k/32]) in double
 * (exact: every term is a product of two E2M1 values and powers of two).
 * a: [M][K/2], w: [N][K/2] packed as orc_quant_mxfp4 writes them. */
void orc_gemm_mxfp4(const uint8_t* a, const uint8_t* ea, const uint8_t* w, const uint8_t* ew, int64_t M, int64_t N,
                    int64_t K, double* y) {
    double* ad = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = a[m * (K / 2) + k / 2];
            uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            ad[m * K + k] = orc_e2m1_decode(code) * ldexp(1.0, (int)ea[m * (K / 32) + k / 32] - 127);
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = w[n * (K / 2) + k / 2];
            uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            wd[n * K + k] = orc_e2m1_decode(code) * ldexp(1.0, (int)ew[n * (K / 32) + k / 32] - 127);
        }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += ad[m * K + k] * wd[n * K + k];
            y[m * N + n] = acc;
        }
    free(ad);
    free(wd);
}

void orc_e2m1_encode_n(const float* x, int64_t n, uint8_t* c) {
    for (int64_t i = 0; i < n; ++i) c[i] = orc_e2m1_encode(x[i]);
}

void orc_e2m1_decode_n(const uint8_t* c, int64_t n, double* x) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_e2m1_decode(c[i]);
}

/* ------------------------------------------------------------------------ */
/* LLM.int8() outlier side path.  [LPI] §16 (Mixed-precision Outlier Path): */
/* outlier feature channels take a higher-precision path, the remaining      */
/* channels the INT8 GEMM, and the two partial outputs are summed.  Readings */
/* of what the section leaves open: an outlier channel is an input column j  */
/* of X whose largest magnitude over the rows reaches a threshold tau; the   */
/* common part is per-token INT8 of X with the outlier columns set to zero   */
/* (the SmoothQuant column multiplier with factors 0 / 1) times the          */
/* per-channel INT8 weight; the side path multiplies the unquantized         */
/* activations of the outlier columns by the same stored weight columns,     */
/* dequantized with their channel scale.                                     */
/* ------------------------------------------------------------------------ */

/* The outlier channels of x [R][C]: every j with max_r |x[r][j]| >= tau, in
 * increasing order, into idx; returns how many. */
int64_t orc_outlier_channels(const float* x, int64_t R, int64_t C, float tau, int32_t* idx) {
    int64_t n = 0;
    for (int64_t j = 0; j < C; ++j) {
        float amax = 0.0f;
        for (int64_t r = 0; r < R; ++r)
            if (fabsf(x[r * C + j]) > amax) amax = fabsf(x[r * C + j]);
        if (amax >= tau) idx[n++] = (int32_t)j;
    }
    return n;
}

/* Y[m,n] = s_a[m] s_w[n] sum_k a[m,k] w[n,k]                  (INT8 part)
 *        + sum_{t < n_o} x[m, idx[t]] (s_w[n] w[n, idx[t]])    (side path)
 * in binary64: a / s_a are the per-token codes and scales of x with the
 * outlier columns zeroed (so those columns add nothing to the first sum),
 * w / s_w the per-channel INT8 weight. */
void orc_gemm_w8a8_outlier(const int8_t* a, const float* a_s, const int8_t* w, const float* w_s, const float* x,
                           const int32_t* idx, int64_t n_o, int64_t M, int64_t N, int64_t K, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)a[m * K + k] * (int64_t)w[n * K + k];
            double side = 0.0;
            for (int64_t t = 0; t < n_o; ++t) {
                int64_t k = idx[t];
                side += (double)x[m * K + k] * ((double)w_s[n] * (double)w[n * K + k]);
            }
            y[m * N + n] = (double)a_s[m] * (double)w_s[n] * (double)acc + side;
        }
}

void orc_e4m3_encode_n(const float* x, int64_t n, uint8_t* c) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) c[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* x) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_e4m3_decode(c[i]);
}
