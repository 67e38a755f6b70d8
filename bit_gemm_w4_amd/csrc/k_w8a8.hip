// k_w8a8.hip -- native INT8 / FP8-E4M3 GEMM (gemm_w8a8).
//
// "Quantization throughput by method" (hrletsgo.me), W8A8/FP8 section: weights
// and activations both in 8 bits, the GEMM runs on the low-precision matrix
// cores with no upcast.  "Low-precision LLM inference" §9 (FP8 GEMM contract:
// operand formats, scale mode and shape, accumulator/output dtype), §22
// (INT32 / FP32 accumulators), §8 block scaling.
//
// Y = A W^T, A [M][K], W [N][K], both K-contiguous.  INT8 uses
// v_mfma_i32_16x16x64_i8 (exact INT32 accumulators), FP8 uses
// v_mfma_f32_16x16x128_f8f6f4 with both operands E4M3 (one instruction covers
// a whole 128-wide scale block).  Block tile BM x BN x 128, four waves as
// WM x WN, A and W tiles staged in LDS with the 16-byte chunk index XOR-ed by
// (row & 7) so that the 8 lanes served per LDS cycle hit distinct banks.
//
// Operand k-assignment: lane quarter q = lane/16 supplies bytes
// [16*(4kk+q), +16) (INT8, K step kk = 0..1) or [32q, +32) (FP8); A and W use
// the same assignment, so matching k are multiplied.  Output: lane l,
// register e of a 16x16 tile is row 4(l/16)+e, column l%16.
#include <type_traits>

#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_I32 = 5 };
enum { GT = 0, GR = 1, GR128 = 2, GB128 = 3 };

template <bool FP8, bool BLOCK, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_w8a8_mfma(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                   int a_gran, const uint8_t* __restrict__ w,
                                                   const float* __restrict__ ws, int w_gran, int64_t M,
                                                   int64_t N, int64_t K, void* __restrict__ y, int out_dt) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[BN * 128];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t m_blk = (int64_t)blockIdx.y * BM, n_blk = (int64_t)blockIdx.x * BN;
    const int64_t nkb = K >> 7;

    using acc_t = typename std::conditional<FP8, float4_t, int4_t>::type;
    acc_t acc[TM][TN];
    float4_t facc[TM][TN];   // block-scaled FP8 only
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            acc[i][j] = acc_t{0, 0, 0, 0};
            facc[i][j] = float4_t{0, 0, 0, 0};
        }

    for (int64_t kb = 0; kb < nkb; ++kb) {
        __syncthreads();
        for (int c = threadIdx.x; c < BM * 8; c += 256) {
            const int r = c >> 3, ch = c & 7;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m_blk + r < M) v = *reinterpret_cast<const uint4*>(a + (m_blk + r) * K + kb * 128 + ch * 16);
            *reinterpret_cast<uint4*>(lds_a + r * 128 + ((ch ^ (r & 7)) << 4)) = v;
        }
        for (int c = threadIdx.x; c < BN * 8; c += 256) {
            const int r = c >> 3, ch = c & 7;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n_blk + r < N) v = *reinterpret_cast<const uint4*>(w + (n_blk + r) * K + kb * 128 + ch * 16);
            *reinterpret_cast<uint4*>(lds_w + r * 128 + ((ch ^ (r & 7)) << 4)) = v;
        }
        __syncthreads();

        if constexpr (FP8) {
            int8_t_v af[TM], wf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 16 + l16;
                const uint4 lo = *reinterpret_cast<const uint4*>(lds_a + r * 128 + (((2 * q) ^ (r & 7)) << 4));
                const uint4 hi = *reinterpret_cast<const uint4*>(lds_a + r * 128 + (((2 * q + 1) ^ (r & 7)) << 4));
                af[i] = int8_t_v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 16 + l16;
                const uint4 lo = *reinterpret_cast<const uint4*>(lds_w + r * 128 + (((2 * q) ^ (r & 7)) << 4));
                const uint4 hi = *reinterpret_cast<const uint4*>(lds_w + r * 128 + (((2 * q + 1) ^ (r & 7)) << 4));
                wf[j] = int8_t_v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            if constexpr (BLOCK) {
                // partial sum of this 128-wide K block, scaled by s_a[m][kb] * s_w[n/128][kb]
                float fa[TM][4];
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t m = m_blk + wm * WTM + i * 16 + q * 4 + e;
                        fa[i][e] = m < M ? as[m * nkb + kb] : 0.0f;
                    }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t n = n_blk + wn * WTN + j * 16 + l16;
                    const float fw = n < N ? ws[(n >> 7) * nkb + kb] : 0.0f;
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const float4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[i], wf[j], float4_t{0, 0, 0, 0}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) facc[i][j][e] += p[e] * (fa[i][e] * fw);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], wf[j], acc[i][j], 0, 0, 0,
                                                                                     0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                int4_t af[TM], wf[TN];
                const int ch = kk * 4 + q;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = wm * WTM + i * 16 + l16;
                    const uint4 v = *reinterpret_cast<const uint4*>(lds_a + r * 128 + ((ch ^ (r & 7)) << 4));
                    af[i] = int4_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int r = wn * WTN + j * 16 + l16;
                    const uint4 v = *reinterpret_cast<const uint4*>(lds_w + r * 128 + ((ch ^ (r & 7)) << 4));
                    wf[j] = int4_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], wf[j], acc[i][j], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: y = acc * s_a * s_w (or the block-scaled sum, or raw INT32) ----
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n_blk + wn * WTN + j * 16 + l16;
            float sw = 1.0f;
            if (!BLOCK && n < N && out_dt != O_I32) sw = w_gran == GT ? ws[0] : ws[n];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m_blk + wm * WTM + i * 16 + q * 4 + e;
                if (m >= M || n >= N) continue;
                const int64_t o = m * N + n;
                if (!FP8 && out_dt == O_I32) {
                    static_cast<int32_t*>(y)[o] = (int32_t)acc[i][j][e];
                    continue;
                }
                float v;
                if constexpr (BLOCK) {
                    v = facc[i][j][e];
                } else {
                    const float sa = a_gran == GT ? as[0] : as[m];
                    v = ((float)acc[i][j][e] * sa) * sw;
                }
                if (out_dt == O_BF16) static_cast<uint16_t*>(y)[o] = f32_to_bf16(v);
                else if (out_dt == O_F16) static_cast<uint16_t*>(y)[o] = f32_to_f16(v);
                else static_cast<float*>(y)[o] = v;
            }
        }
}

template <bool FP8, bool BLOCK, int BM, int BN, int WM, int WN>
static const char* cfg(const W8A8Args& g, hipStream_t s) {
    dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
    hipLaunchKernelGGL((k_w8a8_mfma<FP8, BLOCK, BM, BN, WM, WN>), grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(g.a), g.a_scales, g.a_gran, static_cast<const uint8_t*>(g.w),
                       g.w_scales, g.w_gran, g.M, g.N, g.K, g.y, g.out_dt);
    return kname("k_w8a8_mfma", FP8, BLOCK, BM, BN, WM, WN);
}

template <int BM, int BN, int WM, int WN>
static const char* dispatch(const W8A8Args& g, hipStream_t s) {
    const bool block = g.a_gran == GR128;
    if (!g.in_fp8) return cfg<false, false, BM, BN, WM, WN>(g, s);
    if (block) return cfg<true, true, BM, BN, WM, WN>(g, s);
    return cfg<true, false, BM, BN, WM, WN>(g, s);
}

const char* launch_w8a8_tiled(const W8A8Args& g, hipStream_t s) { return dispatch<128, 128, 2, 2>(g, s); }
const char* launch_w8a8_skinny(const W8A8Args& g, hipStream_t s) { return dispatch<16, 128, 1, 4>(g, s); }

}  // namespace bg
