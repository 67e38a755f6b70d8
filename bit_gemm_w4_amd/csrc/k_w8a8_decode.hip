// k_w8a8_decode.hip -- W8A8 GEMM for small M (decode): weight-bandwidth bound.
//
// "Quantization throughput by method" (hrletsgo.me), W8A8/FP8 section: at
// small batch the 8-bit weights halve the bytes a BF16 layer reads, and the
// GEMM runs on the low-precision matrix cores.  "Low-precision LLM inference"
// §8 (scale granularities, 128-wide blocks), §14 (W8A8), §22 (INT32 / FP32
// accumulators).
//
// A block owns 16 output columns and a band of 16*TM activation rows for the
// whole of K; its 4, 8 or 16 waves take the 128-wide K blocks round-robin, so the
// block streams its 16 weight rows front to back while every wave has its
// own loads in flight.  Each lane loads 32 bytes of K per weight row and per
// activation row and K block (16-byte buffer loads, software-pipelined
// STAGES deep, issued unconditionally so the in-order counter never drains).
// The partial tiles of the waves are added in LDS in wave order (fixed
// order: deterministic), then scaled and written.
//
// MFMA: INT8 v_mfma_i32_16x16x64_i8 twice per K block (lane l: 16 bytes at
// chunk l/16, then 4 + l/16), FP8 v_mfma_f32_16x16x128_f8f6f4 once per K block
// (32 bytes at chunks 2(l/16), 2(l/16)+1) -- the same K chunks for both
// operands.  The activation fragment is the first operand: lane l, register e
// holds row 4(l/16) + e and column l % 16.  Rows past M read row M-1 and are
// never written.  With 128x128 weight blocks and 1x128 activation groups
// (FP8), each K block's product is scaled by s_a[m][kb] * s_w[n/128][kb] and
// added in FP32.
#include <type_traits>

#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

namespace {
enum { DO_F32 = 0, DO_F16 = 1, DO_BF16 = 2, DO_I32 = 5 };
enum { DG_T = 0, DG_R = 1, DG_R128 = 2, DG_B128 = 3 };
// Stages in flight per wave for NW waves per block and a 16*TM-row band:
// deeper when fewer waves share a CU's registers (1024 threads leave 128
// VGPRs per lane, 512 threads 256).
template <int NW, int TM>
struct DecCfg {
    static constexpr int STAGES = NW == 4 ? (TM == 4 ? 4 : 8) : NW == 8 ? (TM == 4 ? 3 : 4) : (TM == 1 ? 4 : 2);
};
}  // namespace

template <int TM>
struct W8Stage {
    uint4 w[2];
    uint4 a[TM][2];
    float sc[TM][4];                    // block-scaled FP8: s_a * s_w per row, this K block
};

template <bool FP8, bool BLOCK, int TM, int DNW>
__global__ __launch_bounds__(DNW * 64) void k_w8a8_decode(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                          int a_gran, const uint8_t* __restrict__ w,
                                                          const float* __restrict__ ws, int w_gran, int64_t M,
                                                          int64_t N, int64_t K, void* __restrict__ y, int out_dt) {
    using acc_t = typename std::conditional<FP8, float4_t, int4_t>::type;
    constexpr int DSTAGES = DecCfg<DNW, TM>::STAGES;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * TM;
    const int nkb = (int)(K >> 7);
    const int c0 = FP8 ? 2 * q : q, c1 = FP8 ? 2 * q + 1 : 4 + q;   // 16-byte K chunks of a K block

    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + n0 * K), (short)0,
                                                      (int)((N - n0 < 16 ? N - n0 : 16) * K), 0x00020000);
    const int64_t rows_here = M - m0 < 16 * TM ? M - m0 : 16 * TM;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a + m0 * K), (short)0,
                                                      (int)(rows_here * K), 0x00020000);
    const uint32_t vw0 = (uint32_t)(l16 * K + c0 * 16), vw1 = (uint32_t)(l16 * K + c1 * 16);
    uint32_t va0[TM], va1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t r = 16 * i + l16 < rows_here ? 16 * i + l16 : rows_here - 1;   // rows past M: row M-1
        va0[i] = (uint32_t)(r * K + c0 * 16);
        va1[i] = (uint32_t)(r * K + c1 * 16);
    }
    // block-scaled FP8: the rows of this lane's output (first operand = activations)
    const int64_t nb = n0 >> 7;

    auto issue = [&](W8Stage<TM>& st, int j) {
        int kb = wave + j * DNW;
        kb = kb < nkb ? kb : nkb - 1;                            // past the end: reload the last block
        const int soff = kb * 128;
        st.w[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw0, soff, 0));
        st.w[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw1, soff, 0));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            st.a[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, va0[i], soff, 0));
            st.a[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, va1[i], soff, 0));
        }
        if constexpr (BLOCK) {
            const float sw = ws[nb * nkb + kb];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = m0 + 16 * i + 4 * q + e;
                    st.sc[i][e] = as[(m < M ? m : M - 1) * nkb + kb] * sw;
                }
        }
    };

    acc_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = acc_t{};
    auto consume = [&](const W8Stage<TM>& st) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (FP8) {
                const int8_t_v av = {(int)st.a[i][0].x, (int)st.a[i][0].y, (int)st.a[i][0].z, (int)st.a[i][0].w,
                                     (int)st.a[i][1].x, (int)st.a[i][1].y, (int)st.a[i][1].z, (int)st.a[i][1].w};
                const int8_t_v wv = {(int)st.w[0].x, (int)st.w[0].y, (int)st.w[0].z, (int)st.w[0].w,
                                     (int)st.w[1].x, (int)st.w[1].y, (int)st.w[1].z, (int)st.w[1].w};
                if constexpr (BLOCK) {
                    const float4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, wv, float4_t{0, 0, 0, 0},
                                                                                       0, 0, 0, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][e] += p[e] * st.sc[i][e];
                } else {
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, wv, acc[i], 0, 0, 0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int4_t av = {(int)st.a[i][h].x, (int)st.a[i][h].y, (int)st.a[i][h].z, (int)st.a[i][h].w};
                    const int4_t wv = {(int)st.w[h].x, (int)st.w[h].y, (int)st.w[h].z, (int)st.w[h].w};
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, wv, acc[i], 0, 0, 0);
                }
            }
        }
    };

    const int nmine = (nkb - wave + DNW - 1) / DNW;              // K blocks of this wave (may be 0)
    W8Stage<TM> stage[DSTAGES];
#pragma unroll
    for (int j = 0; j < DSTAGES; ++j) issue(stage[j], j);
    for (int j = 0; j < nmine; j += DSTAGES) {
#pragma unroll
        for (int u = 0; u < DSTAGES; ++u) {
            if (j + u < nmine) consume(stage[u]);
            issue(stage[u], j + u + DSTAGES);
        }
    }

    // ---- fixed-order sum of the waves' partial tiles ----
    acc_t* red = reinterpret_cast<acc_t*>(dyn_lds);              // [DNW][TM][64]
#pragma unroll
    for (int i = 0; i < TM; ++i) red[(wave * TM + i) * 64 + lane] = acc[i];
    __syncthreads();
    // wave v finishes band rows 16i of tiles i with i % DNW == v (TM <= DNW): one wave per band
    for (int i = wave; i < TM; i += DNW) {
        acc_t v = red[(0 * TM + i) * 64 + lane];
        for (int v2 = 1; v2 < DNW; ++v2) v += red[(v2 * TM + i) * 64 + lane];
        const int64_t n = n0 + l16;
        if (n >= N) continue;
        float sw = 1.0f;
        if (!BLOCK && out_dt != DO_I32) sw = w_gran == DG_T ? ws[0] : ws[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = m0 + 16 * i + 4 * q + e;
            if (m >= M) continue;
            const int64_t o = m * N + n;
            if (!FP8 && out_dt == DO_I32) {
                static_cast<int32_t*>(y)[o] = (int32_t)v[e];
                continue;
            }
            float f;
            if constexpr (BLOCK) {
                f = v[e];
            } else {
                const float sa = a_gran == DG_T ? as[0] : as[m];
                f = ((float)v[e] * sa) * sw;
            }
            if (out_dt == DO_BF16) static_cast<uint16_t*>(y)[o] = f32_to_bf16(f);
            else if (out_dt == DO_F16) static_cast<uint16_t*>(y)[o] = f32_to_f16(f);
            else static_cast<float*>(y)[o] = f;
        }
    }
}

template <bool FP8, bool BLOCK, int TM, int NW>
static const char* decode_cfg(const W8A8Args& g, hipStream_t s) {
    const dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)((g.M + 16 * TM - 1) / (16 * TM)));
    const size_t lds = (size_t)NW * TM * 64 * 16;
    auto kern = k_w8a8_decode<FP8, BLOCK, TM, NW>;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, static_cast<const uint8_t*>(g.a), g.a_scales, g.a_gran,
                       static_cast<const uint8_t*>(g.w), g.w_scales, g.w_gran, g.M, g.N, g.K, g.y, g.out_dt);
    return kname("k_w8a8_decode", FP8, BLOCK, TM, NW);
}

// Waves per block: as many as keep at least 4 K blocks per wave, and no more
// than needed for about 4096 waves in the grid.
template <bool FP8, bool BLOCK, int TM>
static const char* decode_nw(const W8A8Args& g, hipStream_t s) {
    const int64_t blocks = ((g.N + 15) / 16) * ((g.M + 16 * TM - 1) / (16 * TM));
    const int64_t nkb = g.K >> 7;
    if constexpr (TM < 4)                                         // (a 64-row band needs the registers of 8 waves)
        if (nkb >= 64 && blocks * 8 < 4096) return decode_cfg<FP8, BLOCK, TM, 16>(g, s);
    if (nkb >= 32 && blocks * 4 < 4096) return decode_cfg<FP8, BLOCK, TM, 8>(g, s);
    return decode_cfg<FP8, BLOCK, TM, 4>(g, s);
}

template <int TM>
static const char* decode_tm(const W8A8Args& g, hipStream_t s) {
    if (!g.in_fp8) return decode_nw<false, false, TM>(g, s);
    if (g.a_gran == DG_R128) return decode_nw<true, true, TM>(g, s);
    return decode_nw<true, false, TM>(g, s);
}

const char* launch_w8a8_skinny(const W8A8Args& g, hipStream_t s) {
    if (g.M <= 16) return decode_tm<1>(g, s);
    if (g.M <= 32) return decode_tm<2>(g, s);
    return decode_tm<4>(g, s);
}

}  // namespace bg
