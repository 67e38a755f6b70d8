// k_w4a16.hip -- W4A16 linear: Y = X W^T with W in the packed INT4 format.
//
// "Quantization throughput by method" (hrletsgo.me), W4A16 section: INT4
// storage, dequantized to 16 bits inside the GEMM; decode at small batch is
// bandwidth-bound.  "Low-precision LLM inference" §11 (weight-only INT4
// pipeline), §23 fused fast path (packed W4 + scales into the tile, dequant in
// registers, MMA, fused epilogue, single output write -- no dequantized
// weight ever reaches HBM), §22 FP32 accumulation.
//
// Exact dequantization without a floating-point subtraction per weight:
// a nibble u OR-ed into the mantissa of the constant MV (1024 for FP16, 128
// for BF16: the binade where one ulp is 1) gives the exact 16-bit value
// MV + u.  One v_and_or per two weights builds these pairs.  Per group g of
// 128 k:   sum_k x[k](u[k] - z) = sum_k x[k](MV + u[k]) - (MV + z) * Sx_g,
// with Sx_g = sum_{k in g} x[k] shared by all output columns.  The group
// scale then multiplies the FP32 partial sum once per group.
//
// Nibble pairing: from word w (k = 8j .. 8j+7, nibble i = k - 8j) the four
// 32-bit pairs are (w >> 4p) & 0x000F000F | magic = (MV+u_p, MV+u_{p+4}),
// p = 0..3; the activations are permuted to the same order
// (x_p, x_{p+4}) with v_perm, so every dot product pairs matching k.
#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

template <bool BF16>
struct W4Magic;
template <>
struct W4Magic<true> {
    static constexpr uint32_t bits = 0x43004300u;  // BF16 128.0 in both halves
    static constexpr float value = 128.0f;
};
template <>
struct W4Magic<false> {
    static constexpr uint32_t bits = 0x64006400u;  // FP16 1024.0 in both halves
    static constexpr float value = 1024.0f;
};

// dot2 of two packed 16-bit pairs into an FP32 accumulator.
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                               __builtin_bit_cast(bf162_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                      false);
}

// (x_p, x_{p+4}) pairs of 8 consecutive 16-bit activations held as 4 dwords.
__device__ __forceinline__ void pair_perm(const uint32_t X[4], uint32_t P[4]) {
    P[0] = __builtin_amdgcn_perm(X[2], X[0], 0x05040100u);
    P[1] = __builtin_amdgcn_perm(X[2], X[0], 0x07060302u);
    P[2] = __builtin_amdgcn_perm(X[3], X[1], 0x05040100u);
    P[3] = __builtin_amdgcn_perm(X[3], X[1], 0x07060302u);
}

// The four (MV+u_p, MV+u_{p+4}) pairs of one packed word.
template <bool BF16>
__device__ __forceinline__ void dequant_word(uint32_t w, uint32_t D[4]) {
    constexpr uint32_t m = W4Magic<BF16>::bits;
    D[0] = (w & 0x000F000Fu) | m;
    D[1] = ((w >> 4) & 0x000F000Fu) | m;
    D[2] = ((w >> 8) & 0x000F000Fu) | m;
    D[3] = ((w >> 12) & 0x000F000Fu) | m;
}

__device__ __forceinline__ uint32_t zero_point(const uint8_t* __restrict__ zr, int64_t n, int64_t ngroups,
                                               int64_t g) {
    if (zr == nullptr) return 8u;
    return (uint32_t)(zr[n * (ngroups >> 1) + (g >> 1)] >> (4 * (g & 1))) & 0xFu;
}

// ============================================================================
// Decode GEMV (VALU).  A row of W is split over LPR lanes; each lane handles
// 16-byte chunks (32 k, a quarter group) and RPW rows per wave slot, reusing
// its activations across those rows.  MB batch rows per block (grid.y tiles M).
// Partial sums are combined with an LPR-lane xor reduction.
// ============================================================================
template <bool BF16, int MB, int LPR, int RPW>
__global__ __launch_bounds__(256) void k_w4a16_gemv(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                    const uint32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ sc,
                                                    const uint8_t* __restrict__ zr, int64_t N,
                                                    uint16_t* __restrict__ y) {
    constexpr int ROWS_PER_SLOT = 64 / LPR;
    constexpr int ROWS_PER_WAVE = RPW * ROWS_PER_SLOT;
    constexpr int ROWS_PER_BLOCK = 4 * ROWS_PER_WAVE;
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONES = BF16 ? 0x3F803F80u : 0x3C003C00u;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kl = lane % LPR;
    const int rsub = lane / LPR;
    const int64_t m0 = (int64_t)blockIdx.y * MB;
    const int64_t nrow0 = (int64_t)blockIdx.x * ROWS_PER_BLOCK + wave * ROWS_PER_WAVE + rsub;
    const int64_t nchunks = K >> 5;
    const int64_t ngroups = K >> 7;

    float acc[RPW][MB];
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[s][b] = 0.0f;

    for (int64_t c = kl; c < nchunks; c += LPR) {
        const int64_t g = c >> 2;
        uint4 wv[RPW];
        float scale[RPW];
        float corr[RPW];
#pragma unroll
        for (int s = 0; s < RPW; ++s) {
            const int64_t n = nrow0 + s * ROWS_PER_SLOT;
            if (n < N) {
                wv[s] = reinterpret_cast<const uint4*>(qw + n * (K >> 3))[c];
                scale[s] = f16_to_f32(sc[n * ngroups + g]);
                corr[s] = MV + (float)zero_point(zr, n, ngroups, g);
            } else {
                wv[s] = make_uint4(0, 0, 0, 0);
                scale[s] = 0.0f;
                corr[s] = 0.0f;
            }
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (m0 + b >= M) break;
            const uint4* xp = reinterpret_cast<const uint4*>(x + (m0 + b) * K + c * 32);
            uint32_t P[4][4];
            float sx = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 r = xp[q];
                const uint32_t X[4] = {r.x, r.y, r.z, r.w};
                pair_perm(X, P[q]);
#pragma unroll
                for (int p = 0; p < 4; ++p) sx = dot2<BF16>(P[q][p], ONES, sx);
            }
#pragma unroll
            for (int s = 0; s < RPW; ++s) {
                const uint32_t W[4] = {wv[s].x, wv[s].y, wv[s].z, wv[s].w};
                float d = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t D[4];
                    dequant_word<BF16>(W[q], D);
#pragma unroll
                    for (int p = 0; p < 4; ++p) d = dot2<BF16>(D[p], P[q][p], d);
                }
                acc[s][b] += scale[s] * (d - corr[s] * sx);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < RPW; ++s) {
        const int64_t n = nrow0 + s * ROWS_PER_SLOT;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const float v = wave_sum<LPR>(acc[s][b]);
            if (kl == 0 && n < N && m0 + b < M)
                y[(m0 + b) * N + n] = BF16 ? f32_to_bf16(v) : f32_to_f16(v);
        }
    }
}

// ============================================================================
// MFMA kernel (v_mfma_f32_16x16x32_{bf16,f16}).  Block tile BM x BN, one
// 128-wide group per K step; 4 waves as WM x WN, each wave TM x TN 16x16
// tiles.  The activation tile is staged in LDS (XOR-swizzled 16-byte chunks
// so the 16 rows read by one MFMA operand hit distinct banks); each lane
// reads its packed weights straight from HBM (16 bytes = its quarter of a
// group row) and dequantizes them in registers.
//
// Operand k-assignment: in K step kk (0..3) of a group, lane quarter q
// (lane / 16) supplies word 4q + kk of the group row, i.e. k = 32q + 8kk +
// {0,4,1,5,2,6,3,7}; the activation operand uses the same k order, so the
// hardware's fixed pairing of operand slots multiplies matching k.  Output
// layout of a 16x16 f32 tile: lane l, register i holds row 4(l/16) + i,
// column l % 16.
//
// Sx_g for the zero-point/magic correction comes from one extra MFMA per
// m-tile per K step against an all-ones operand: its accumulator holds
// sum_k x[row][k] in exactly the rows the epilogue needs.
// ============================================================================
template <bool BF16, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_w4a16_mfma(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                    const uint32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ sc,
                                                    const uint8_t* __restrict__ zr, int64_t N,
                                                    uint16_t* __restrict__ y) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONES = BF16 ? 0x3F803F80u : 0x3C003C00u;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * 256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t m_blk = (int64_t)blockIdx.y * BM, n_blk = (int64_t)blockIdx.x * BN;
    const int64_t ngroups = K >> 7;
    const int64_t kwords = K >> 3;

    float4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = float4_t{0, 0, 0, 0};

    for (int64_t g = 0; g < ngroups; ++g) {
        // ---- stage the BM x 128 activation tile (16 chunks of 16 B per row) ----
        __syncthreads();
        for (int c = threadIdx.x; c < BM * 16; c += 256) {
            const int r = c >> 4, ch = c & 15;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m_blk + r < M) v = *reinterpret_cast<const uint4*>(x + (m_blk + r) * K + g * 128 + ch * 8);
            *reinterpret_cast<uint4*>(lds_a + r * 256 + ((ch ^ (r & 15)) << 4)) = v;
        }
        // ---- this lane's packed weights for the group: 16 B per n-tile ----
        uint4 wv[TN];
        float scale[TN], corr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n_blk + wn * WTN + j * 16 + l16;
            if (n < N) {
                wv[j] = *reinterpret_cast<const uint4*>(qw + n * kwords + g * 16 + q * 4);
                scale[j] = f16_to_f32(sc[n * ngroups + g]);
                corr[j] = MV + (float)zero_point(zr, n, ngroups, g);
            } else {
                wv[j] = make_uint4(0, 0, 0, 0);
                scale[j] = 0.0f;
                corr[j] = 0.0f;
            }
        }
        __syncthreads();

        float4_t part[TM][TN], sx[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            sx[i] = float4_t{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < TN; ++j) part[i][j] = float4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint32_t bfrag[TN][4];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t w = kk == 0 ? wv[j].x : kk == 1 ? wv[j].y : kk == 2 ? wv[j].z : wv[j].w;
                dequant_word<BF16>(w, bfrag[j]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 16 + l16;
                const int ch = q * 4 + kk;
                const uint4 v = *reinterpret_cast<const uint4*>(lds_a + r * 256 + ((ch ^ (r & 15)) << 4));
                const uint32_t X[4] = {v.x, v.y, v.z, v.w};
                uint32_t A[4];
                pair_perm(X, A);
                const uint32_t ones[4] = {ONES, ONES, ONES, ONES};
                if constexpr (BF16) {
                    const bf168_t a = __builtin_bit_cast(bf168_t, A);
                    sx[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(bf168_t, ones), sx[i], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a, __builtin_bit_cast(bf168_t, bfrag[j]), part[i][j], 0, 0, 0);
                } else {
                    const half8_t a = __builtin_bit_cast(half8_t, A);
                    sx[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8_t, ones), sx[i],
                                                                   0, 0, 0);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            a, __builtin_bit_cast(half8_t, bfrag[j]), part[i][j], 0, 0, 0);
                }
            }
        }
        // ---- per-group epilogue: acc += s * (part - (MV + z) * Sx) ----
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] += scale[j] * (part[i][j][e] - corr[j] * sx[i][e]);
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n_blk + wn * WTN + j * 16 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m_blk + wm * WTM + i * 16 + q * 4 + e;
                if (m < M && n < N) y[m * N + n] = BF16 ? f32_to_bf16(acc[i][j][e]) : f32_to_f16(acc[i][j][e]);
            }
        }
}

// ---------------------------------------------------------------- launch ----

template <bool BF16, int MB, int LPR, int RPW>
static const char* gemv_cfg(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                     const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    constexpr int rows_per_block = 4 * RPW * (64 / LPR);
    dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block), (unsigned)((M + MB - 1) / MB));
    hipLaunchKernelGGL((k_w4a16_gemv<BF16, MB, LPR, RPW>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y));
    return kname("k_w4a16_gemv", BF16, MB, LPR, RPW);
}

template <bool BF16, int MB>
static const char* gemv_mb(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                    const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    const int64_t chunks = K >> 5;
    if (chunks >= 256) return gemv_cfg<BF16, MB, 64, 1>(x, M, K, qw, sc, zr, N, y, s);
    if (chunks >= 64) return gemv_cfg<BF16, MB, 32, 1>(x, M, K, qw, sc, zr, N, y, s);
    return gemv_cfg<BF16, MB, 16, 1>(x, M, K, qw, sc, zr, N, y, s);
}

template <bool BF16>
static const char* gemv_dt(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                    const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (M <= 1) return gemv_mb<BF16, 1>(x, M, K, qw, sc, zr, N, y, s);
    if (M <= 2) return gemv_mb<BF16, 2>(x, M, K, qw, sc, zr, N, y, s);
    return gemv_mb<BF16, 4>(x, M, K, qw, sc, zr, N, y, s);
}

const char* launch_w4a16_gemv(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return gemv_dt<true>(x, M, K, qw, sc, zr, N, y, s);
    return gemv_dt<false>(x, M, K, qw, sc, zr, N, y, s);
}

template <bool BF16, int BM, int BN, int WM, int WN>
static const char* mfma_cfg(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                     const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL((k_w4a16_mfma<BF16, BM, BN, WM, WN>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y));
    return kname("k_w4a16_mfma", BF16, BM, BN, WM, WN);
}

const char* launch_w4a16_skinny(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                                const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return mfma_cfg<true, 16, 128, 1, 4>(x, M, K, qw, sc, zr, N, y, s);
    return mfma_cfg<false, 16, 128, 1, 4>(x, M, K, qw, sc, zr, N, y, s);
}

const char* launch_w4a16_tiled(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                               const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return mfma_cfg<true, 128, 128, 2, 2>(x, M, K, qw, sc, zr, N, y, s);
    return mfma_cfg<false, 128, 128, 2, 2>(x, M, K, qw, sc, zr, N, y, s);
}

}  // namespace bg
