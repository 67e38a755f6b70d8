// k_w4a16_mid.hip -- W4A16 linear for mid-size batches (17 <= M <= 128):
// Y = X W^T with W in the packed INT4 format.
//
// "Quantization throughput by method" (hrletsgo.me), W4A16 section: around
// the critical batch (about 74 rows on the page's hardware) the W4A16 linear
// turns from weight-bandwidth bound to compute bound, so the kernel has to
// read every weight byte once AND keep the matrix cores busy.  "Low-precision
// LLM inference" §11 (INT4 weights, 16-bit activations), §23 (packed weights
// and scales into the tile, dequantization in registers, one output write),
// §22 (FP32 accumulation).
//
// Block: WM x WN waves over a band of 16*TMW*WM activation rows and
// 16*TNW*WN output columns (TNW weight tiles of 16 columns per wave), for its
// range of K.  All waves work on the same 128-wide group at a time: the
// group's activation rows are staged in LDS once per block (a double-buffered
// ring, one barrier per group), while each wave streams its own weight tiles
// straight from memory into registers, STAGES groups ahead (the WM waves of a
// column range read the same tiles: the second read is a cache hit).  Every
// activation fragment a wave reads from LDS feeds TNW = 4 tiles of MFMAs, so
// the LDS traffic stays below what the matrix cores consume (one tile per
// fragment would make the kernel LDS-bound at half the MFMA rate), and every
// weight tile is dequantized by WM <= 2 waves -- the 256-row prefill tile
// dequantizes each one four times and pads a 74-row batch to 256.
//
// Dequantization and exactness as in the decode kernels: the MFMA consumes
// the exact 16-bit values MV + u (v_bitop3 on the packed nibbles), and per
// group the zero-point and MV are removed with (MV + z) * Sx before the FP16
// scale multiplies the FP32 group sum.  Sx (sum of a row's 128 activations of
// the group) is computed while the group is staged: the 16 lanes that copy a
// row's 16-byte chunks add their 8 values and combine them in a fixed xor
// tree, so the result does not depend on timing.  BF16: the removal is one
// more MFMA per row tile and weight tile and group, on the matrix cores
// instead of the vector ALU (which bounds this kernel): Sx is split exactly
// into three BF16 parts (8 + 8 + 8 significant bits), staged as K slots 0..2
// of the first lane quarter, against -(MV + z) (exact in BF16) in the weight
// operand.  FP16 keeps the FP32 correction (an FP16 part could overflow).
//
// K split: with a workspace the K range is cut into S slices of whole groups
// when the blocks of one slice do not fill the device; slice sl writes FP32
// partials to ws[sl][M][N] and k_w4a16_gemm_reduce (k_w4a16_gemm.hip) adds
// them in slice order on the same stream.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_w4.h"

namespace bg {

namespace {
constexpr int MID_STAGES = 2;
constexpr int XPITCH = 128 + 8;         // LDS row pitch of a staged group, in 16-bit elements
}  // namespace

template <int TNW>
struct MidStage {
    uint4 w[TNW];
    uint32_t s[TNW];
    uint32_t z[TNW];
};

template <bool BF16, int TMW, int TNW, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void k_w4a16_mid(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                                       const uint8_t* __restrict__ zr, int64_t N,
                                                       uint16_t* __restrict__ y, float* __restrict__ ws, int gs) {
    constexpr int NW = WM * WN;
    constexpr int BM = 16 * TMW * WM;
    constexpr int NT = NW * 64;
    constexpr int CHUNKS = BM * 16;                                   // 16-byte chunks of a staged group
    constexpr int CPT = (CHUNKS + NT - 1) / NT;                       // chunks per thread
    constexpr int XBUF = BM * XPITCH * 2;                             // bytes of one staged group
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    static_assert(NT % 64 == 0 && (CHUNKS % 16) == 0, "a row's 16 chunks sit in 16 consecutive lanes");
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    uint16_t* xbuf = reinterpret_cast<uint16_t*>(dyn_lds);                       // [2][BM][XPITCH]
    float* sxbuf = reinterpret_cast<float*>(dyn_lds + 2 * XBUF);                 // FP16: [2][BM]
    uint2* sxpart = reinterpret_cast<uint2*>(dyn_lds + 2 * XBUF);                // BF16: [2][BM] 3 parts

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int ntiles = (int)(N >> 4);
    const int ngroups = (int)(K >> 7);
    const int sl = blockIdx.z;
    const int g0 = sl * gs;
    const int ng = (ngroups - g0) < gs ? (ngroups - g0) : gs;          // >= 1 by construction
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int rows = (M - m0) < BM ? (int)(M - m0) : BM;
    const int wm = wave / WN, wn = wave - wm * WN;
    const int rw0 = 16 * TMW * wm;                                     // this wave's first row in the band
    const int t0 = (blockIdx.x * WN + wn) * TNW;                       // this wave's first tile
    const int my_tiles = t0 >= ntiles ? 0 : (ntiles - t0 < TNW ? ntiles - t0 : TNW);

    // weights, scales, zero bytes of this wave's tiles, K range of the slice;
    // reads past the wave's tiles (ragged N) return 0
    const bool has_z = zr != nullptr;
    const int tt = my_tiles > 0 ? t0 : 0;
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + (int64_t)tt * ngroups * 256), (short)0,
                                                      my_tiles * ngroups * 1024, 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + (int64_t)tt * ngroups * 16), (short)0,
                                                      my_tiles * ngroups * 32, 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(has_z ? zr + (int64_t)tt * (ngroups >> 1) * 16 : zr), (short)0,
        has_z ? my_tiles * (ngroups >> 1) * 16 : 0, 0x00020000);
    // activation rows of the band (rows past M read row M - 1: they only feed
    // output rows that are never written)
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + m0 * K), (short)0,
                                                      (int)((int64_t)rows * K * 2), 0x00020000);

    auto issue = [&](MidStage<TNW>& st, int i) {
        const int g = g0 + (i < ng - 1 ? i : ng - 1);
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            st.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16,
                                                                                       (j * ngroups + g) * 1024, 0));
            st.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, l16 * 2, (j * ngroups + g) * 32, 0);
            st.z[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, l16, (j * (ngroups >> 1) + (g >> 1)) * 16, 0);
        }
    };

    // staging of group i of the slice: chunk c = tid + u * NT is row c / 16,
    // 16-byte part c % 16 (8 consecutive k).  Every thread issues all CPT
    // loads (past the last chunk it reloads that chunk, and past the slice's
    // last group that group): unconditional loads keep the compiler's count
    // of loads in flight exact, so each wait covers exactly the loads it needs.
    uint4 xr[CPT];
    int xoff[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        int c = tid + u * NT;
        c = c < CHUNKS ? c : CHUNKS - 1;
        int r = c >> 4;
        r = r < rows ? r : rows - 1;
        xoff[u] = r * (int)K * 2 + (c & 15) * 16;
    }
    auto x_load = [&](int i) {
        const int g = g0 + (i < ng - 1 ? i : ng - 1);
#pragma unroll
        for (int u = 0; u < CPT; ++u)
            xr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[u], g * 256, 0));
    };
    auto x_store = [&](int buf) {
        uint16_t* xb = xbuf + buf * (BM * XPITCH);
        float* sxb = sxbuf + buf * BM;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * NT;
            // sum of this lane's 8 values, then the 16 lanes of the row in a
            // fixed xor tree (every lane of a row is in the same wave)
            float s = dot2<BF16>(xr[u].x, ONE2, 0.0f);
            s = dot2<BF16>(xr[u].y, ONE2, s);
            s = dot2<BF16>(xr[u].z, ONE2, s);
            s = dot2<BF16>(xr[u].w, ONE2, s);
            s += __shfl_xor(s, 8, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 1, 64);
            if (c < CHUNKS) {
                *reinterpret_cast<uint4*>(xb + (c >> 4) * XPITCH + (c & 15) * 8) = xr[u];
                if ((c & 15) == 0) {
                    if constexpr (BF16) {
                        // s = hi + mid + lo exactly: each residual is exact in FP32
                        // and the last one has at most 8 significant bits
                        const uint32_t hi = f32_to_bf16(s);
                        const float r1 = s - bf16_to_f32(hi);
                        const uint32_t mid = f32_to_bf16(r1);
                        const uint32_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
                        sxpart[buf * BM + (c >> 4)] = uint2{hi | (mid << 16), lo};
                    } else {
                        sxb[c >> 4] = s;
                    }
                }
            }
        }
    };

    MidStage<TNW> stage[MID_STAGES];
    x_load(0);
    x_store(0);
    x_load(1);
#pragma unroll
    for (int s = 0; s < MID_STAGES; ++s) issue(stage[s], s);
    __syncthreads();

    float4_t acc[TMW][TNW];
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = float4_t{0, 0, 0, 0};

    auto consume = [&](const MidStage<TNW>& st, int i) {
        const int g = g0 + i;
        const uint16_t* xb = xbuf + (i & 1) * (BM * XPITCH);
        const float* sxb = sxbuf + (i & 1) * BM;
        float scale[TNW], corr[TNW];
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            scale[j] = f16_to_f32(st.s[j] & 0xFFFFu);
            corr[j] = MV + (float)(has_z ? (st.z[j] >> (4 * (g & 1))) & 0xF : 8u);
        }
        float4_t part[TMW][TNW];
#pragma unroll
        for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
            for (int j = 0; j < TNW; ++j) part[ii][j] = float4_t{0, 0, 0, 0};
        uint32_t D[TNW][2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if ((kk & 1) == 0) {
#pragma unroll
                for (int j = 0; j < TNW; ++j)
                    dequant_pair<BF16>(kk == 0 ? st.w[j].x : st.w[j].z, kk == 0 ? st.w[j].y : st.w[j].w, D[j][0],
                                       D[j][1]);
            }
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii) {
                // lane (l16, q): row rw0 + 16 ii + l16, k = 32 q + 8 kk .. + 7 of the group
                const uint4 av =
                    *reinterpret_cast<const uint4*>(xb + (rw0 + 16 * ii + l16) * XPITCH + q * 32 + kk * 8);
                const uint32_t a[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
                for (int j = 0; j < TNW; ++j) part[ii][j] = mfma16<BF16>(a, D[j][kk & 1], part[ii][j]);
            }
        }
        if constexpr (BF16) {
            // - (MV + z) * Sx on the matrix cores: K slots 0..2 of lane quarter 0
            uint32_t cb[TNW][4];
#pragma unroll
            for (int j = 0; j < TNW; ++j) {
                const uint32_t zz = has_z ? (st.z[j] >> (4 * (g & 1))) & 0xFu : 8u;
                const uint32_t cc = q == 0 ? ((zz | (zz << 16)) | 0xC300C300u) : 0u;   // -(128 + z), twice
                cb[j][0] = cc;
                cb[j][1] = cc;
                cb[j][2] = 0u;
                cb[j][3] = 0u;
            }
            const uint2* sp = sxpart + (i & 1) * BM;
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii) {
                const uint2 v = sp[rw0 + 16 * ii + l16];
                const uint32_t a[4] = {q == 0 ? v.x : 0u, q == 0 ? v.y : 0u, 0u, 0u};
#pragma unroll
                for (int j = 0; j < TNW; ++j) part[ii][j] = mfma16<BF16>(a, cb[j], part[ii][j]);
            }
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
                for (int j = 0; j < TNW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[ii][j][e] += scale[j] * part[ii][j][e];
        } else {
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii) {
                // output rows rw0 + 16 ii + 4 q + e of this lane
                const float4 sx = *reinterpret_cast<const float4*>(sxb + rw0 + 16 * ii + 4 * q);
                const float sxv[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
                for (int j = 0; j < TNW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[ii][j][e] += scale[j] * (part[ii][j][e] - corr[j] * sxv[e]);
            }
        }
    };

    // group i: consume it from buffer i & 1, stage group i + 1 into the other
    // buffer (its last readers finished before the previous barrier), request
    // group i + 2, refill the weight stage, barrier.  Staging, requests and
    // barriers run for every step of the unrolled loop (past the slice's end
    // they move clamped copies nobody reads), so the loads in flight are the
    // same at every wait.
    for (int i = 0; i < ng; i += MID_STAGES) {
#pragma unroll
        for (int s = 0; s < MID_STAGES; ++s) {
            if (i + s < ng) consume(stage[s], i + s);
            x_store((i + s + 1) & 1);
            x_load(i + s + 2);
            issue(stage[s], i + s + MID_STAGES);
            __syncthreads();
        }
    }

    // ---- output: BF16/FP16 rows < M, or FP32 partials of the slice ----
    if (my_tiles == 0) return;
#pragma unroll
    for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            if (j >= my_tiles) continue;
            const int64_t n = (int64_t)(t0 + j) * 16 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rw0 + 16 * ii + 4 * q + e;
                if (r >= rows) continue;
                const int64_t m = m0 + r;
                if (ws) ws[((int64_t)sl * M + m) * N + n] = acc[ii][j][e];
                else y[m * N + n] = to_out<BF16>(acc[ii][j][e]);
            }
        }
}

// ---- configuration (shared by the workspace query and the launch) ----
namespace {
struct MidCfg {
    int TMW, WM, S, gs;
    int64_t ws_bytes, lds_bytes;
    unsigned nblocks, bands;
};
constexpr int MID_TNW = 4;

// Row bands of up to 96 rows; a band of R row tiles (16 rows) is split over
// WM = 2 waves from R = 4 (WM = 1 below), each with TMW = ceil(R / WM) <= 3
// row tiles (the accumulators of 3 x 4 tiles, twice, fill the 256 registers
// a lane has at two waves per SIMD); 8 waves in all, 4 tiles each (256
// columns per block with WM = 2, 512 with WM = 1).  K is split while one slice's blocks fill less than one
// round of 256 CUs, at least 3 groups per slice.
MidCfg mid_cfg(int64_t M, int64_t N, int64_t K, bool with_ws) {
    MidCfg c{};
    const int64_t bands = (M + 95) / 96;
    const int64_t band_rows = (M + bands - 1) / bands;
    const int64_t R = (band_rows + 15) / 16;
    c.WM = R >= 4 ? 2 : 1;
    c.TMW = (int)((R + c.WM - 1) / c.WM);
    const int WN = 8 / c.WM;
    const int64_t ntiles = N >> 4, ngroups = K >> 7;
    const int64_t nb = (ntiles + WN * MID_TNW - 1) / (WN * MID_TNW);
    int64_t S = 1;
    if (with_ws) {
        S = 256 / (nb * bands);
        if (S > ngroups / 3) S = ngroups / 3;
        if (S < 1) S = 1;
    }
    int64_t gs = (ngroups + S - 1) / S;
    S = (ngroups + gs - 1) / gs;
    c.S = (int)S;
    c.gs = (int)gs;
    c.nblocks = (unsigned)nb;
    c.bands = (unsigned)bands;
    c.ws_bytes = S > 1 ? S * M * N * 4 : 0;
    const int64_t BM = 16 * c.TMW * c.WM;
    c.lds_bytes = 2 * BM * XPITCH * 2 + 2 * BM * 8;
    return c;
}

template <bool BF16, int TMW, int WM>
const char* mid_launch(const MidCfg& c, const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                       const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    constexpr int WN = 8 / WM;
    auto kern = k_w4a16_mid<BF16, TMW, MID_TNW, WM, WN>;
    if (c.lds_bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)c.lds_bytes);
    float* wsf = c.S > 1 ? static_cast<float*>(ws) : nullptr;
    hipLaunchKernelGGL(kern, dim3(c.nblocks, c.bands, (unsigned)c.S), dim3(WM * WN * 64), (size_t)c.lds_bytes, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y), wsf, c.gs);
    if (c.S > 1) launch_w4a16_gemm_reduce(BF16, wsf, c.S, M, N, y, s);
    return kname("k_w4a16_mid", BF16, TMW, MID_TNW, WM, WN);
}

template <bool BF16>
const char* mid_dt(const MidCfg& c, const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                   const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    if (c.WM == 1) {
        if (c.TMW == 1) return mid_launch<BF16, 1, 1>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        if (c.TMW == 2) return mid_launch<BF16, 2, 1>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        return mid_launch<BF16, 3, 1>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    }
    if (c.TMW == 2) return mid_launch<BF16, 2, 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    return mid_launch<BF16, 3, 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
}
}  // namespace

int64_t w4a16_mid_workspace(int64_t M, int64_t N, int64_t K) { return mid_cfg(M, N, K, true).ws_bytes; }

const char* launch_w4a16_mid(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                             const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    const MidCfg c = mid_cfg(M, N, K, ws != nullptr);
    if (x_bf16) return mid_dt<true>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    return mid_dt<false>(c, x, M, K, qw, sc, zr, N, y, ws, s);
}

}  // namespace bg
