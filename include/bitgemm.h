/*
 * bitgemm.h -- C ABI of the MI355X (gfx950) W4A16 / W8A8 quantized linear layer.
 *
 * Sources (cited by title and section):
 *   [LPI] "Low-precision LLM inference: FP8/INT8/INT4/FP4 kernels and
 *         calibration (8/10)", blog.ruahverce.com
 *   [AIB] "Quantization throughput by method: why W4A16 is overtaken by W8A8
 *         as batch grows", hrletsgo.me
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers to contiguous row-major buffers,
 *    aligned to 16 bytes.  The caller allocates and frees them.
 *  - Activations X are [M][K]; weights W are [N][K] (output channel major,
 *    K contiguous); the output is Y = X W^T, [M][N].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    validate arguments on the host and enqueue kernels: they never allocate,
 *    free, synchronize, or read device memory on the host, so every call may
 *    be captured into a HIP graph ([LPI] §28: device-side scales, no host
 *    amax).
 *  - Validation is fail-closed ([LPI] §24 kernel eligibility, §31
 *    fallback_policy fail-closed): an ineligible call returns a BG_ERR_* code
 *    before anything is launched and never falls back to another kernel.
 *    bg_last_error() then returns a message naming the failed condition.
 *  - A launch failure returns BG_ERR_HIP.
 *  - Calls that write overlapping outputs on concurrent streams race.
 */
#ifndef BITGEMM_H
#define BITGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BG_PACK_FORMAT_VERSION 1

typedef enum bg_status {
    BG_OK = 0,
    BG_ERR_NULL = 1,         /* a required pointer is NULL                       */
    BG_ERR_SHAPE = 2,        /* a size is out of range or not a tile multiple    */
    BG_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned                 */
    BG_ERR_DTYPE = 4,        /* dtype not accepted by this entry point           */
    BG_ERR_UNSUPPORTED = 5,  /* granularity / dtype combination not implemented  */
    BG_ERR_HIP = 6,          /* the HIP runtime rejected a launch                */
    BG_ERR_WORKSPACE = 7     /* workspace missing or smaller than required       */
} bg_status;

typedef enum bg_dtype {
    BG_F32 = 0, BG_F16 = 1, BG_BF16 = 2, BG_I8 = 3, BG_FP8_E4M3 = 4, BG_I32 = 5
} bg_dtype;

/* Scale granularity ([LPI] §4 "Scale granularity is the key"). */
typedef enum bg_gran {
    BG_GRAN_TENSOR = 0,    /* one scale for the whole tensor                       */
    BG_GRAN_ROW = 1,       /* one per row: per token (X) or per output channel (W) */
    BG_GRAN_ROW_G128 = 2,  /* one per 1x128 group along a row                      */
    BG_GRAN_BLOCK128 = 3   /* one per 128x128 block                                */
} bg_gran;

/* Kernel choice for the *_ex entry points (the plain ones use BG_ALGO_AUTO). */
typedef enum bg_algo {
    BG_ALGO_AUTO = 0,
    BG_ALGO_GEMV = 1,      /* W4A16 small-M: VALU dot products, wave reductions    */
    BG_ALGO_SKINNY = 2,    /* small-M on MFMA (M padded to the MFMA tile)          */
    BG_ALGO_TILED = 3,     /* large-M LDS-tiled MFMA GEMM                          */
    BG_ALGO_SPLITK = 4,    /* W4A16: K split over blocks, needs a workspace        */
    BG_ALGO_MID = 5        /* W4A16 mid-size M: wide N slab per block, activation
                              groups staged once per block; K split with a workspace */
} bg_algo;

/*
 * w4_pack -- quantize W [N][K] to 4-bit codes with one FP16 scale (and, if
 * asymmetric, one 4-bit zero-point) per group of `group` consecutive K.
 *
 * Defined by [LPI] §2 eq. (1) q = clamp(round(x/s) + z, qmin, qmax) and
 * eq. (2) x^ = s(q - z); §3 symmetric s = max|x|/qmax (eq. 3) and asymmetric
 * (observed min/max); §4 per-group scales; §5 FP16 scale per 128 weights.
 * Readings: round = round-half-to-even; x/s is an IEEE binary32 division by
 * the stored FP16 scale; symmetric s = fp16(amax/7), codes u = q + 8 in
 * 1..15; asymmetric: mn = min(0, min w), mx = max(0, max w),
 * s = fp16((mx - mn)/15), z = clamp(round(-mn/s), 0, 15), u in 0..15; an
 * all-zero group has s = 1; FP16 scales are clamped to [2^-24, 65504].
 *
 *   w        [N][K] of w_dtype (BG_F32, BG_F16 or BG_BF16), finite values
 *   group    must be 128
 * Output layout (tiled for the GEMM kernels, [LPI] §24 packing order of the
 * target kernel): 16 output channels x one 128-wide group form a 1 KB tile of
 * 64 slots x 4 uint32 words.  Weight (n, k) with t = n/16, r = n%16,
 * g = k/128, c = k%128 lives in slot 16*(c/32) + r, word (c%32)/8, nibble
 * i/2 (even i) or 4 + i/2 (odd i) for i = k%8 (even k in the low half-word):
 *   qweight  out [N/16][K/128][64][4] uint32
 *   scales   out [N/16][K/128][16] FP16 bit patterns, scale of (n, g) at [t][g][r]
 *   zeros    out [N/16][K/256][16] uint8, zero-points of groups 2h (low
 *            nibble) and 2h+1 (high nibble) at [t][h][r], when asymmetric != 0;
 *            must be NULL when symmetric
 * Requires N % 16 == 0, K % 256 == 0.
 */
bg_status w4_pack(const void* w, int w_dtype, int64_t N, int64_t K, int group, int asymmetric,
                  uint32_t* qweight, uint16_t* scales, uint8_t* zeros, void* stream);

/*
 * gemm_w4a16 -- Y = X W^T with W in the w4_pack format, dequantized on chip
 * (never materialized in HBM: [LPI] §23 fused fast path; [AIB] W4A16
 * section).  Y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] * (u[n,k] - z[n,g]),
 * z = 8 when zeros == NULL; FP32 accumulation ([LPI] §22), output rounded to
 * the activation dtype (round-to-nearest-even).
 *
 *   x        [M][K] of x_dtype (BG_F16 or BG_BF16)
 *   qweight, scales, zeros   as produced by w4_pack (zeros NULL = symmetric)
 *   y        out [M][N] of x_dtype
 * Requires 1 <= M <= 1048560, N % 16 == 0, K % 256 == 0, group == 128
 * (BG_ALGO_GEMV: M <= 256 and K <= 18432; BG_ALGO_SKINNY: K <= 65536, as
 * the small-M kernels hold a block's group scales and zero-points for all of
 * K in LDS; BG_ALGO_AUTO sends larger K to the tiled kernel).  Small M runs
 * the bandwidth-bound decode kernels, large M the LDS-tiled
 * MFMA kernel ([LPI] §24: small batch and large prefill use different kernels).
 */
bg_status gemm_w4a16(const void* x, int x_dtype, int64_t M, int64_t K,
                     const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                     int64_t N, int group, void* y, void* stream);

/* Same as gemm_w4a16 with an explicit kernel choice (BG_ALGO_*; not SPLITK). */
bg_status gemm_w4a16_ex(const void* x, int x_dtype, int64_t M, int64_t K,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        int64_t N, int group, void* y, int algo, void* stream);

/*
 * gemm_w4a16_ws -- gemm_w4a16 with a caller-provided device workspace, which
 * enables the split-K kernels (BG_ALGO_SPLITK):
 *   M <= 64  the small-M split-K kernel.  BG_ALGO_AUTO picks it for M from 8
 *            to 64 where it measured faster than BG_ALGO_SKINNY: M >= 8 with
 *            K >= 8192, M >= 17 with N > 4096, or M >= 24.
 *            Splitting K across workgroups lets each workgroup reuse its
 *            activations across 16 weight tiles.
 *   M > 64   the large-M kernel with K split into S slices of whole groups
 *            while its 256 x 128 output tiles do not fill one round of the
 *            device (S = min(256 / tiles, groups / 4); S = 1 is the plain
 *            kernel and needs no workspace).  BG_ALGO_AUTO picks it whenever
 *            S > 1 outside the mid-batch range below.
 * and the mid-batch kernel (BG_ALGO_MID) with K split so that its blocks
 * fill one round of the device; BG_ALGO_AUTO picks it where it measured
 * faster than both of the above: 17 <= M <= 128 on layers with N >= 16384,
 * 64 <= M <= 128 on the others.
 * The FP32 partials go to the workspace and a second kernel, enqueued on the
 * same stream, sums them in a fixed order, so results are deterministic.
 *   workspace        16-byte aligned device memory of at least
 *                    gemm_w4a16_workspace_bytes(M, N, K, algo) bytes.  It
 *                    needs no initialisation and its contents afterwards
 *                    are unspecified.  Calls that share a workspace must
 *                    not overlap in time (same stream, or otherwise
 *                    ordered).  May be NULL when the required size is 0.
 *   workspace_bytes  its size; BG_ERR_WORKSPACE if smaller than required.
 * Other arguments, layouts and errors as gemm_w4a16.
 */
bg_status gemm_w4a16_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        int64_t N, int group, void* y, void* workspace, int64_t workspace_bytes,
                        int algo, void* stream);

/* Workspace bytes gemm_w4a16_ws needs for this shape and kernel choice
 * (0 if none; BG_ALGO_AUTO = the kernel AUTO selects when given a workspace). */
int64_t gemm_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int algo);

/*
 * gemm_w4a16_noalloc -- gemm_w4a16_ws with BG_ALGO_AUTO for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split-K partials go to a
 * static device array of BG_NOALLOC_SCRATCH_BYTES inside the library instead
 * of a caller workspace; every GPU the library runs on holds its own copy
 * until the process ends.  Its address is looked up (hipGetSymbolAddress)
 * on the first call on each device; after that a call enqueues exactly the
 * kernels gemm_w4a16_ws enqueues for the same shape, so results are bit for
 * bit the same.  The call allocates and frees nothing.
 *
 *   arguments, layouts and results as gemm_w4a16; `stream` must belong to
 *   the current device (BG_ERR_UNSUPPORTED otherwise).
 * Errors as gemm_w4a16_ws, plus BG_ERR_WORKSPACE when the shape needs more
 * than BG_NOALLOC_SCRATCH_BYTES (gemm_w4a16_workspace_bytes(M, N, K,
 * BG_ALGO_AUTO) tells the size in advance), and BG_ERR_HIP if the address
 * lookup fails.
 * All calls on one GPU share its scratch array: calls that overlap in time on
 * the same GPU (different streams, or different host threads without
 * ordering) race and give wrong results.  The array needs no clearing: each
 * call writes every partial it later reads.
 */
#define BG_NOALLOC_SCRATCH_BYTES (16LL << 20)
bg_status gemm_w4a16_noalloc(const void* x, int x_dtype, int64_t M, int64_t K,
                             const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                             int64_t N, int group, void* y, void* stream);

/*
 * act_quant_int8 -- dynamic symmetric INT8 quantization of a [rows][cols]
 * tensor: per unit of granularity `gran`, s = amax/127 (binary32; s = 1 for an
 * all-zero unit) and q = clamp(round(x/s), -128, 127), round half to even.
 * [LPI] §2 eq. (1) with z = 0, §3 eq. (3), §4 per-token / per-channel
 * scales; §14 (W8A8 activations).  Weights for W8A8 are quantized with this
 * same call (BG_GRAN_ROW on W gives per-output-channel scales).
 *
 *   x       [rows][cols] of x_dtype (BG_F32, BG_F16 or BG_BF16), finite values
 *   gran    BG_GRAN_TENSOR: scales[0] = s, scales[1] = tensor amax (2 floats)
 *           BG_GRAN_ROW: scales[rows]
 *           BG_GRAN_ROW_G128: scales[rows][cols/128]
 *           BG_GRAN_BLOCK128: scales[rows/128][cols/128] (rows % 128 == 0)
 *   q       out [rows][cols] int8
 * Requires rows >= 1, cols % 128 == 0.
 */
bg_status act_quant_int8(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                         int8_t* q, float* scales, void* stream);

/*
 * act_quant_fp8 -- dynamic OCP FP8 E4M3 quantization: per unit, s = amax/448
 * and q = e4m3(x/s) with round-to-nearest-even and saturation to +-448.
 * [LPI] §7 (E4M3 = 1/4/3 bits; the variant pinned here is OCP E4M3FN: bias
 * 7, max 448, no infinities, S.1111.111 = NaN), §8 current scaling and block
 * scaling (scale_block = amax_block / max_representable_fp8).
 * Arguments and scale layouts as act_quant_int8; q holds E4M3 bytes.
 */
bg_status act_quant_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                        uint8_t* q, float* scales, void* stream);

/*
 * act_quant_int8_smooth / act_quant_fp8_smooth -- the same quantizers applied
 * to X diag(col_mul): element (r, j) is multiplied by col_mul[j] (one binary32
 * multiplication, fused into the load) before the unit's amax and the codes.
 * This is the online half of the SmoothQuant fold ([LPI] §15:
 * Y = X W^T = (X S^-1)(W S)^T for a diagonal S over the input channels):
 * activations pass col_mul = 1/s, and the weights are folded once with
 * col_mul = s before their own quantization.  S comes from calibration
 * statistics and a smoothing strength and is the caller's input.
 *   col_mul  cols floats, 16-byte aligned device memory; BG_ERR_NULL if NULL.
 * Other arguments, layouts and errors as act_quant_int8 / act_quant_fp8.
 */
bg_status act_quant_int8_smooth(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                                const float* col_mul, int8_t* q, float* scales, void* stream);
bg_status act_quant_fp8_smooth(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                               const float* col_mul, uint8_t* q, float* scales, void* stream);

/*
 * act_quant_mxfp8 -- MXFP8 quantization ([LPI] §10: the OCP MX block format,
 * a block of elements and its shared scale taken as one data format).  Each
 * run of 32 consecutive elements of a row shares an E8M0 scale 2^(e - 127):
 * e = floor(log2 amax) - 8 + 127 (8 = the largest E4M3 exponent), clamped to
 * 0..254, 127 for an all-zero block; each element is the saturating RNE E4M3
 * cast of v * 2^(127 - e) (OCP MX v1.0).
 *   x      [rows][cols] F32, F16 or BF16; cols % 32 == 0
 *   q      out E4M3 bytes [rows][cols]
 *   e8m0   out scale bytes, K-block-major: [cols/32][rows rounded up to 16]
 *          (scale of row r, block b at e8m0[b * rpad + r]; the padding bytes
 *          are not written)
 */
bg_status act_quant_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, void* stream);

/*
 * gemm_mxfp8 -- Y = (A X_a)(W X_w)^T for MXFP8 operands (act_quant_mxfp8 of
 * the activations [M][K] and of the weights [N][K]) on gfx950's block-scaled
 * FP8 matrix instruction: every MFMA takes the E8M0 scales of its 32-element
 * K runs, so the block scaling costs no vector instructions; FP32
 * accumulation, one RNE rounding to out_dtype.
 *   a, a_e8m0   E4M3 [M][K], E8M0 [K/32][M rounded up to 16]
 *   w, w_e8m0   E4M3 [N][K], E8M0 [K/32][N] (N % 16 == 0)
 *   y           out [M][N], BG_BF16, BG_F16 or BG_F32
 * Requires K % 128 == 0, N % 16 == 0, M * K and N * K below 2^31, 16-byte
 * aligned pointers.  No workspace.
 */
bg_status gemm_mxfp8(const uint8_t* a, const uint8_t* a_e8m0, const uint8_t* w, const uint8_t* w_e8m0,
                     int64_t M, int64_t N, int64_t K, void* y, int out_dtype, void* stream);

/*
 * act_quant_mxfp4 -- MXFP4 quantization ([LPI] §10: E2M1 = 1 sign, 2
 * exponent, 1 mantissa bit, and MXFP4 as the OCP MX block format of it).  As
 * act_quant_mxfp8, with e = floor(log2 amax) - 2 + 127 (2 = the largest E2M1
 * exponent) and each element the saturating RNE E2M1 cast of v * 2^(127 - e)
 * (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; a value that rounds
 * to zero keeps its sign; NaN, which E2M1 cannot hold, becomes a signed zero).
 *   x      [rows][cols] F32, F16 or BF16; cols % 32 == 0
 *   q      out packed codes [rows][cols/2] bytes: element 2i in the low
 *          nibble of byte i, element 2i + 1 in the high nibble
 *   e8m0   out scale bytes, K-block-major: [cols/32][rows rounded up to 16]
 *          (the padding bytes are not written)
 */
bg_status act_quant_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, void* stream);

/*
 * gemm_mxfp4 -- Y = (A X_a)(W X_w)^T for MXFP4 operands (act_quant_mxfp4 of
 * the activations [M][K] and of the weights [N][K]) on gfx950's block-scaled
 * matrix instruction with both operands in E2M1: each MFMA takes the E8M0
 * scales of its 32-element K blocks; FP32 accumulation, one RNE rounding to
 * out_dtype.
 *   a, a_e8m0   packed E2M1 [M][K/2], E8M0 [K/32][M rounded up to 16]
 *   w, w_e8m0   packed E2M1 [N][K/2], E8M0 [K/32][N] (N % 16 == 0)
 *   y           out [M][N], BG_BF16, BG_F16 or BG_F32
 * Requires K % 256 == 0, N % 16 == 0, M * K / 2 and N * K / 2 below 2^31,
 * 16-byte aligned pointers.  No workspace.
 */
bg_status gemm_mxfp4(const uint8_t* a, const uint8_t* a_e8m0, const uint8_t* w, const uint8_t* w_e8m0,
                     int64_t M, int64_t N, int64_t K, void* y, int out_dtype, void* stream);

/*
 * act_quant_int8_outlier -- the activation half of the LLM.int8() split ([LPI]
 * §16, Mixed-precision Outlier Path: outlier feature channels go to a
 * higher-precision side path, the rest to the INT8 GEMM).  An outlier channel
 * is a column j of x whose largest magnitude over the rows is >= tau (NaN
 * elements do not count).  The other columns are quantized per token as
 * act_quant_int8 with BG_GRAN_ROW does, with the outlier columns set to zero
 * first (they quantize to 0 and do not enter the row maxima).
 *   x       [rows][cols] F32, F16 or BF16; cols % 128 == 0
 *   tau     the threshold (not NaN; a negative tau makes every column an outlier)
 *   q       out INT8 codes [rows][cols]
 *   scales  out FP32 per-token scales [rows]
 *   idx     out int32 [cols] (device): the outlier columns in increasing order
 *           in idx[0 .. *count); the rest is not written
 *   count   out int32 (device): how many
 *   workspace, workspace_bytes  device scratch of at least
 *           act_quant_outlier_workspace_bytes(rows, cols) bytes, any contents;
 *           BG_ERR_WORKSPACE if smaller.
 * The count stays on the device: nothing here synchronizes with the host.
 */
int64_t act_quant_outlier_workspace_bytes(int64_t rows, int64_t cols);
bg_status act_quant_int8_outlier(const void* x, int x_dtype, int64_t rows, int64_t cols, float tau, int8_t* q,
                                 float* scales, int32_t* idx, int32_t* count, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/*
 * gemm_w8a8_outlier -- the GEMM half of the LLM.int8() split ([LPI] §16: the
 * two partial outputs are summed):
 *   Y[m][n] = s_w[n] (s_a[m] sum_k a[m][k] w[n][k] + sum_{t < count} x[m][j_t] w[n][j_t]),
 * j_t = idx[t]: the INT8 GEMM of the common channels (a from
 * act_quant_int8_outlier, zero on the outlier columns) plus the side path,
 * which multiplies the unquantized activations of the outlier columns by the
 * INT8 weight codes of the same columns (so with the channel scale s_w the
 * weight's own dequantized values), with FP32 accumulation.  The side path is
 * fused into the GEMM and runs on the BF16 matrix instruction: after the K
 * loop each block stages its rows' outlier activations (split into BF16 hi +
 * lo: exact for BF16 and FP16 inputs, within 2^-16 relative for FP32) and its
 * columns' weight codes (exact in BF16) in LDS, 64 channels at a time, and
 * accumulates them into the FP32 accumulators before the single rounding to
 * out_dtype.
 *   a, a_scales  INT8 [M][K], FP32 per-token scales [M]
 *   w, w_scales  INT8 [N][K], FP32 scales: [N] (w_gran BG_GRAN_ROW) or one
 *                (w_gran BG_GRAN_TENSOR)
 *   x            [M][K] F32, F16 or BF16: the activations a was quantized from
 *   idx, count   the outlier list (device); count is clamped to [0, K] and the
 *                entries to [0, K), so a bad list never reads outside x or w
 *   y            out [M][N], BG_BF16, BG_F16 or BG_F32
 * Requires K % 128 == 0 and K < 131072, N % 16 == 0, 16-byte aligned a, w,
 * y and scales, 4-byte aligned x, idx and count.  No workspace, no K split.
 */
bg_status gemm_w8a8_outlier(const int8_t* a, const float* a_scales, const int8_t* w, const float* w_scales,
                            int w_gran, const void* x, int x_dtype, const int32_t* idx, const int32_t* count,
                            int64_t M, int64_t N, int64_t K, void* y, int out_dtype, void* stream);

/*
 * gemm_w8a8 -- native INT8 or FP8 GEMM of quantized activations A [M][K] and
 * weights W [N][K] ([AIB] W8A8/FP8 section: no upcast, low-precision matrix
 * cores; [LPI] §9 FP8 GEMM contract, §22 INT32 / FP32 accumulators).
 *
 *   in_dtype BG_I8: INT32 accumulation, acc exact; Y = acc * s_a * s_w in FP32
 *            BG_FP8_E4M3: FP32 accumulation of exact E4M3 products
 *   a_gran / w_gran, scales laid out as produced by act_quant_*:
 *            TENSOR or ROW for either operand (scales applied in the
 *            epilogue), or, for FP8 only, a_gran = ROW_G128 with
 *            w_gran = BLOCK128: every 128-wide K block's partial sum is
 *            scaled by s_a[m][kb] * s_w[n/128][kb] ([LPI] §8 block scaling)
 *   out_dtype BG_BF16, BG_F16 or BG_F32 (round-to-nearest-even); BG_I32
 *            (in_dtype BG_I8 only) writes the raw INT32 accumulators
 *   y        out [M][N] of out_dtype
 * Requires 1 <= M <= 1048560, N % 16 == 0, K % 128 == 0, K < 131072 (at most
 * 130944) for BG_I8, so |acc| <= K * 128 * 128 < 2^31 even with every code at
 * -128; BLOCK128 needs N % 128 == 0.
 */
bg_status gemm_w8a8(const void* a, const float* a_scales, int a_gran,
                    const void* w, const float* w_scales, int w_gran,
                    int in_dtype, int64_t M, int64_t N, int64_t K,
                    void* y, int out_dtype, void* stream);

/* Same as gemm_w8a8 with an explicit kernel choice (BG_ALGO_SKINNY / TILED). */
bg_status gemm_w8a8_ex(const void* a, const float* a_scales, int a_gran,
                       const void* w, const float* w_scales, int w_gran,
                       int in_dtype, int64_t M, int64_t N, int64_t K,
                       void* y, int out_dtype, int algo, void* stream);

/*
 * gemm_w8a8_ws -- gemm_w8a8 with a caller-provided device workspace, which
 * lets the large-M kernel (BG_ALGO_TILED, or AUTO when it picks that kernel)
 * split K across workgroups when its output tiles would fill at most half a
 * round of the device (128 tiles): S = min(tiles per round / tiles,
 * (K / 128) / 8) slices of whole 128-wide K blocks, 128 x 128 tiles for
 * M <= 128.  AUTO with a workspace picks this path where it measured faster
 * than the small-M kernel: N >= 6144 at any M, K >= 8192 from M = 4, and
 * otherwise from M = 32.  Each slice writes
 * its raw partial sums (INT32 for INT8, so the result equals the unsplit
 * kernel's bit for bit; FP32 for FP8, already block-scaled for 128 x 128
 * blocks) to the workspace, and a second kernel, enqueued on the same stream,
 * adds the slices in a fixed order and applies the scales.
 *   workspace        16-byte aligned device memory of at least
 *                    gemm_w8a8_workspace_bytes(M, N, K, in_dtype, a_gran,
 *                    algo) bytes (S * M * N * 4 when K is split, else 0).  It
 *                    needs no initialisation and its contents afterwards
 *                    are unspecified.  Calls that share a workspace must not
 *                    overlap in time.  May be NULL when the size is 0.
 *   workspace_bytes  its size; BG_ERR_WORKSPACE if smaller than required.
 * Other arguments, layouts and errors as gemm_w8a8.
 */
bg_status gemm_w8a8_ws(const void* a, const float* a_scales, int a_gran,
                       const void* w, const float* w_scales, int w_gran,
                       int in_dtype, int64_t M, int64_t N, int64_t K,
                       void* y, int out_dtype, void* workspace, int64_t workspace_bytes,
                       int algo, void* stream);

/* Workspace bytes gemm_w8a8_ws needs for this shape, input type, activation
 * granularity and kernel choice (0 if none; BG_ALGO_AUTO = AUTO's choice). */
int64_t gemm_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int in_dtype, int a_gran, int algo);

/*
 * gemm_w4a8 -- W4A8 linear: INT8 activation codes times packed INT4 weights
 * on the INT8 matrix cores ([LPI] §1, the W4A8 row of the notation table and
 * its precision manifest: INT4 weights, INT8 activations, INT32/FP32
 * accumulation, BF16 or FP16 output; §14 per-token activation scales; §20
 * and self-check Q2: a native low-precision GEMM whose INT4 weights are
 * dequantized on the way).
 *
 *   y[m,n] = s_a[m] * sum_g s[n,g] * sum_{k in g} a[m,k] * (u[n,k] - z[n,g])
 *
 * The inner sums are exact INT32; each group's sum is scaled by its FP16
 * scale and accumulated in FP32, and s_a scales the row at the end.
 *   a, a_scales, a_gran  INT8 codes [M][K] and scales as act_quant_int8
 *                        produces them: BG_GRAN_ROW (per token, [M]) or
 *                        BG_GRAN_TENSOR (scales[0])
 *   qweight, scales, zeros, N, group   the packed weights of w4_pack
 *                        (zeros NULL = symmetric, z = 8), group == 128
 *   y, out_dtype         out [M][N], BG_BF16, BG_F16 or BG_F32
 *                        (round-to-nearest-even)
 * Requires 1 <= M, N % 16 == 0, K % 256 == 0, M * K < 2^31, 16-byte aligned
 * pointers.  M <= 32 runs the small-M kernel, which streams the packed
 * weight tiles once ([LPI] §26: decode is bound by the weight bytes) and
 * needs no workspace; larger M the 256 x 128-tile kernel.  Both compute the
 * same exact group sums and close them in the same order, up to FP32
 * rounding of the per-group accumulation.
 */
bg_status gemm_w4a8(const int8_t* a, const float* a_scales, int a_gran, int64_t M, int64_t K,
                    const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                    int64_t N, int group, void* y, int out_dtype, void* stream);

/*
 * gemm_w4a8_ws -- gemm_w4a8 with a caller-provided device workspace: for M > 32,
 * while the output tiles do not fill one round of the device (fewer than 256), K is
 * split into S = min(256 / tiles, groups / 4) slices of whole groups; each
 * slice writes its FP32 partial (row scale applied) to the workspace and a
 * second kernel, enqueued on the same stream, adds the slices in a fixed order
 * and writes out_dtype.
 *   workspace        16-byte aligned device memory of at least
 *                    gemm_w4a8_workspace_bytes(M, N, K) bytes (S * M * N * 4
 *                    when K is split, else 0); no initialisation needed,
 *                    contents afterwards unspecified; calls that share it
 *                    must not overlap in time.  May be NULL when the size is 0.
 *   workspace_bytes  its size; BG_ERR_WORKSPACE if smaller than required.
 * Other arguments, layouts and errors as gemm_w4a8.
 */
bg_status gemm_w4a8_ws(const int8_t* a, const float* a_scales, int a_gran, int64_t M, int64_t K,
                       const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                       int64_t N, int group, void* y, int out_dtype, void* workspace,
                       int64_t workspace_bytes, void* stream);

/* Workspace bytes gemm_w4a8_ws needs for this shape (0 if K is not split). */
int64_t gemm_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The kernel BG_ALGO_AUTO selects for a call of this shape (a BG_ALGO_* value). */
int gemm_w4a16_algo(int64_t M, int64_t N, int64_t K, int x_dtype);
int gemm_w8a8_algo(int64_t M, int64_t N, int64_t K, int in_dtype);

/* Static description of a status code. */
const char* bg_status_string(int status);
/* Message of the last failed call on this host thread ("" if none). */
const char* bg_last_error(void);
/* BG_PACK_FORMAT_VERSION of the library (layout of qweight/scales/zeros). */
int bg_pack_format_version(void);
/* Kernel template instance enqueued by the last successful call on this host
 * thread, e.g. "k_w4a16_gemv<true, 1, 32, 1>" -- a substring of the name a
 * profiler's kernel trace shows ([LPI] §24: record the kernel name). */
const char* bg_last_kernel(void);

#ifdef __cplusplus
}
#endif
#endif /* BITGEMM_H */
