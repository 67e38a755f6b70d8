// k_w8a8_decode.hip -- W8A8 GEMM for small M (decode): weight-bandwidth bound.
//
// "Quantization throughput by method" (hrletsgo.me), W8A8/FP8 section: at
// small batch the 8-bit weights halve the bytes a BF16 layer reads, and the
// GEMM runs on the low-precision matrix cores.  "Low-precision LLM inference"
// §8 (scale granularities, 128-wide blocks), §14 (W8A8), §22 (INT32 / FP32
// accumulators).
//
// A block owns 16*TN output columns (TN weight tiles of 16 rows) and a band
// of 16*TM activation rows for the whole of K; its 4, 8 or 16 waves take the
// 128-wide K blocks round-robin, so the block streams its weight rows front
// to back while every wave has its own loads in flight.  Each lane loads 32
// bytes of K per weight row and K block (16-byte buffer loads, software-
// pipelined STAGES deep, issued unconditionally so the in-order counter never
// drains; past the wave's last K block they address beyond the buffer and
// return zeros without a memory access).  Loads of 16 rows x 64 bytes stream
// as fast as contiguous ones on this device (measured: the same bytes in 16 x
// 64-byte row pieces or in 1 KB runs of one row, within 2 %).
//
// XL (M <= 16, when the rows fit): the block first copies its activation rows
// (all of K) into LDS, and the activation operand is read from there, so a
// stage holds weights only (deeper pipeline, no per-lane activation loads
// that repeat a row 16 times at small M).  Otherwise the activation fragments
// are loaded with the weights.
//
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
// added in FP32 (16*TN divides 128, so a block's tiles share one weight block).
#include <type_traits>

#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

namespace {
enum { DO_F32 = 0, DO_F16 = 1, DO_BF16 = 2, DO_I32 = 5 };
enum { DG_T = 0, DG_R = 1, DG_R128 = 2, DG_B128 = 3 };
// Stages in flight per wave for NW waves per block, a 16*TM-row band and TN
// tiles: deeper when fewer waves share a CU's registers (1024 threads leave
// 128 VGPRs per lane, 512 threads 256) and when the activations are in LDS --
// except for four-tile blocks, whose 8 KB stages keep more requests in
// flight than the memory side serves well (gate_up at B = 16: 27.7 us with
// two stages, 29.4 with three, 29.5 with four; the one- and two-tile
// configurations measured best or within 1 % at four).  Without staged rows
// a stage also carries the activation fragments; 16-wave blocks of one band
// keep two (down at B = 16: 18.2 us against 19.4 with four, 20.8 with three),
// and so do 8-wave blocks of two bands (o at B = 24 / 32: 8.8 / 9.4 us
// against 9.7 / 10.4 with four).
template <int NW, int TM, int TN, bool XL>
struct DecCfg {
    static constexpr int STAGES = XL        ? (TN == 4 ? 2 : 4)
                                  : NW == 4 ? (TM == 4 ? 4 : 8)
                                  : NW == 8 ? (TM == 4 ? 3 : TM == 2 ? 2 : 4)
                                            : 2;
};
}  // namespace

template <int TM, int TN, bool XL>
struct W8Stage {
    uint4 w[TN][2];
    uint4 a[XL ? 1 : TM][2];
    float sc[TM][4];                    // block-scaled FP8: s_a * s_w per row, this K block
};

template <bool FP8, bool BLOCK, int TM, int TN, int DNW, bool XL>
__global__ __launch_bounds__(DNW * 64) void k_w8a8_decode(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                          int a_gran, const uint8_t* __restrict__ w,
                                                          const float* __restrict__ ws, int w_gran, int64_t M,
                                                          int64_t N, int64_t K, void* __restrict__ y, int out_dt) {
    static_assert(!XL || TM == 1, "LDS-staged activations: one 16-row band");
    static_assert(128 % (16 * TN) == 0, "a block's tiles lie in one 128-wide weight block");
    using acc_t = typename std::conditional<FP8, float4_t, int4_t>::type;
    constexpr int DSTAGES = DecCfg<DNW, TM, TN, XL>::STAGES;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * TN;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * TM;
    const int nkb = (int)(K >> 7);
    const int c0 = FP8 ? 2 * q : q, c1 = FP8 ? 2 * q + 1 : 4 + q;   // 16-byte K chunks of a K block

    // weight rows past N (last block) read zeros
    const int64_t wrows = N - n0 < 16 * TN ? N - n0 : 16 * TN;
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + n0 * K), (short)0, (int)(wrows * K),
                                                      0x00020000);
    const int64_t rows_here = M - m0 < 16 * TM ? M - m0 : 16 * TM;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a + m0 * K), (short)0,
                                                      (int)(rows_here * K), 0x00020000);
    uint32_t vw0[TN], vw1[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        vw0[j] = (uint32_t)((16 * j + l16) * K + c0 * 16);
        vw1[j] = (uint32_t)((16 * j + l16) * K + c1 * 16);
    }
    uint32_t va0[TM], va1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t r = 16 * i + l16 < rows_here ? 16 * i + l16 : rows_here - 1;   // rows past M: row M-1
        va0[i] = (uint32_t)(r * K + c0 * 16);
        va1[i] = (uint32_t)(r * K + c1 * 16);
    }
    // block-scaled FP8: the weight block of this block's columns
    const int64_t nb = n0 >> 7;
    const int64_t pitch = K + 16;                                 // LDS row pitch: rows 4 banks apart

    auto issue = [&](W8Stage<TM, TN, XL>& st, int jj) {
        int kb = wave + jj * DNW;
        const bool real = kb < nkb;
        kb = real ? kb : nkb - 1;
        const int soff = real ? kb * 128 : kBufOOB;              // past the end: zeros, no memory access
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            st.w[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw0[j], soff, 0));
            st.w[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, vw1[j], soff, 0));
        }
        if constexpr (!XL) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                st.a[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, va0[i], soff, 0));
                st.a[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, va1[i], soff, 0));
            }
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

    // XL: the first batch of activation chunks is requested before the weight
    // stages, so that the in-order counter returns it first
    constexpr int XB = 4;
    const int cpr = (int)(K >> 4);                                // 16-byte chunks per row
    const int xtotal = XL ? (int)rows_here * cpr : 0;
    uint4 xv[XB];
    auto x_load = [&](uint4 (&v)[XB], int cb) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = cb + u * DNW * 64;
            if (c < xtotal) v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, c * 16, 0, 0));
        }
    };
    auto x_store = [&](const uint4 (&v)[XB], int cb) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = cb + u * DNW * 64;
            if (c < xtotal) {
                const int r = c / cpr, kc = c - r * cpr;
                *reinterpret_cast<uint4*>(dyn_lds + r * pitch + kc * 16) = v[u];
            }
        }
    };
    if constexpr (XL) x_load(xv, threadIdx.x);

    W8Stage<TM, TN, XL> stage[DSTAGES];
#pragma unroll
    for (int j = 0; j < DSTAGES; ++j) issue(stage[j], j);

    if constexpr (XL) {
        x_store(xv, threadIdx.x);
        for (int cb = threadIdx.x + XB * DNW * 64; cb < xtotal; cb += XB * DNW * 64) {
            uint4 v[XB];
            x_load(v, cb);
            x_store(v, cb);
        }
        __syncthreads();
    }
    const int arow = l16 < rows_here ? l16 : (int)rows_here - 1;

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
    auto consume = [&](const W8Stage<TM, TN, XL>& st, int kb) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            uint4 a0, a1;
            if constexpr (XL) {
                const uint8_t* ap = dyn_lds + arow * pitch + kb * 128;
                a0 = *reinterpret_cast<const uint4*>(ap + c0 * 16);
                a1 = *reinterpret_cast<const uint4*>(ap + c1 * 16);
            } else {
                a0 = st.a[i][0];
                a1 = st.a[i][1];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (FP8) {
                    const int8_t_v av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                         (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    const int8_t_v wv = {(int)st.w[j][0].x, (int)st.w[j][0].y, (int)st.w[j][0].z, (int)st.w[j][0].w,
                                         (int)st.w[j][1].x, (int)st.w[j][1].y, (int)st.w[j][1].z, (int)st.w[j][1].w};
                    if constexpr (BLOCK) {
                        const float4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, wv, float4_t{0, 0, 0, 0}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][e] += p[e] * st.sc[i][e];
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, wv, acc[i][j], 0, 0, 0, 0,
                                                                                      0, 0);
                    }
                } else {
                    const int4_t av0 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w};
                    const int4_t wv0 = {(int)st.w[j][0].x, (int)st.w[j][0].y, (int)st.w[j][0].z, (int)st.w[j][0].w};
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av0, wv0, acc[i][j], 0, 0, 0);
                    const int4_t av1 = {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    const int4_t wv1 = {(int)st.w[j][1].x, (int)st.w[j][1].y, (int)st.w[j][1].z, (int)st.w[j][1].w};
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av1, wv1, acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    const int nmine = (nkb - wave + DNW - 1) / DNW;              // K blocks of this wave (may be 0)
    for (int j = 0; j < nmine; j += DSTAGES) {
#pragma unroll
        for (int u = 0; u < DSTAGES; ++u) {
            if (j + u < nmine) consume(stage[u], wave + (j + u) * DNW);
            issue(stage[u], j + u + DSTAGES);
        }
    }

    // ---- fixed-order sum of the waves' partial tiles ----
    if constexpr (XL) __syncthreads();                            // the staged rows are dead
    acc_t* red = reinterpret_cast<acc_t*>(dyn_lds);              // [DNW][TM * TN][64]
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) red[((wave * TM + i) * TN + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    // wave v finishes the (band, tile) pairs u = v, v + DNW, ...
    for (int u = wave; u < TM * TN; u += DNW) {
        const int i = u / TN, j = u - i * TN;
        acc_t v = red[u * 64 + lane];
        for (int v2 = 1; v2 < DNW; ++v2) v += red[(v2 * TM * TN + u) * 64 + lane];
        const int64_t n = n0 + 16 * j + l16;
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

template <bool FP8, bool BLOCK, int TM, int TN, int NW, bool XL>
static const char* decode_cfg(const W8A8Args& g, hipStream_t s) {
    const dim3 grid((unsigned)(((g.N + 15) / 16 + TN - 1) / TN), (unsigned)((g.M + 16 * TM - 1) / (16 * TM)));
    size_t lds = (size_t)NW * TM * TN * 64 * 16;
    if (XL) {
        const size_t xb = (size_t)(g.M < 16 ? g.M : 16) * (g.K + 16);
        lds = xb > lds ? xb : lds;
    }
    auto kern = k_w8a8_decode<FP8, BLOCK, TM, TN, NW, XL>;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, static_cast<const uint8_t*>(g.a), g.a_scales, g.a_gran,
                       static_cast<const uint8_t*>(g.w), g.w_scales, g.w_gran, g.M, g.N, g.K, g.y, g.out_dt);
    return kname("k_w8a8_decode", FP8, BLOCK, TM, TN, NW, XL);
}

// Activation rows staged in LDS (M <= 16) while they take at most 144 KB
// (K <= 9200 at M = 16, K <= 14336 through M = 10): measured on the
// projection shapes (graph-replayed, weights rotated past the MALL), one tile
// per block with 8 waves unless the grid would not fill the device evenly --
// two tiles for 256 < N/16 < 1024 (qkv: 192 blocks beat 384), with 8 waves
// from M = 5 (qkv at B = 16: 9.6 against 10.3 us with 4); on wide layers
// four tiles with 4 waves from M = 5 on (the staged rows are then shared by
// four tiles), below that one tile with 4 waves (gate_up at B = 4: 25.6
// against 26.3 us with 8).
bool w8_decode_xl(int64_t M, int64_t K) { return M <= 16 && (M < 16 ? M : 16) * (K + 16) <= 144 * 1024; }

template <bool FP8, bool BLOCK>
static const char* decode_xl(const W8A8Args& g, hipStream_t s) {
    const int64_t tiles = (g.N + 15) / 16;
    if (tiles >= 1024) {
        if (g.M > 4) return decode_cfg<FP8, BLOCK, 1, 4, 4, true>(g, s);
        return decode_cfg<FP8, BLOCK, 1, 1, 4, true>(g, s);
    }
    if (tiles > 256) {
        if (g.M > 4) return decode_cfg<FP8, BLOCK, 1, 2, 8, true>(g, s);
        return decode_cfg<FP8, BLOCK, 1, 2, 4, true>(g, s);
    }
    return decode_cfg<FP8, BLOCK, 1, 1, 8, true>(g, s);
}

// Waves per block: as many as keep at least 4 K blocks per wave, and no more
// than needed for about 4096 waves in the grid.
template <bool FP8, bool BLOCK, int TM>
static const char* decode_nw(const W8A8Args& g, hipStream_t s) {
    if constexpr (TM == 1)
        if (w8_decode_xl(g.M, g.K)) return decode_xl<FP8, BLOCK>(g, s);
    const int64_t blocks = ((g.N + 15) / 16) * ((g.M + 16 * TM - 1) / (16 * TM));
    const int64_t nkb = g.K >> 7;
    if constexpr (TM < 4)                                         // (a 64-row band needs the registers of 8 waves)
        if (nkb >= 64 && blocks * 8 < 4096) return decode_cfg<FP8, BLOCK, TM, 1, 16, false>(g, s);
    if (nkb >= 32 && blocks * 4 < 4096) return decode_cfg<FP8, BLOCK, TM, 1, 8, false>(g, s);
    return decode_cfg<FP8, BLOCK, TM, 1, 4, false>(g, s);
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
