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
// Block: WM x WN waves over a band of 16*TMW*WM activation rows and 64*WN
// output columns (4 weight tiles of 16 columns per wave), for its range of K.
// All waves step through the 128-wide groups together, one barrier per
// group.  A group's activation rows go from memory straight into LDS
// (buffer_load ... lds, no registers) in a ring of three buffers, 16-byte
// chunks XOR-swizzled by row so the fragment reads are free of bank
// conflicts; each wave reads all its fragments of the group at once, then
// copies the group after next into the ring.  Each wave streams its own
// weight tiles straight from memory into registers, two groups ahead (the
// WM waves of a column range read the same tiles: the second read is a
// cache hit).  Every activation fragment feeds 4 tiles of MFMAs (LDS traffic
// well below what the matrix cores consume) and every weight tile is
// dequantized by WM <= 2 waves for up to 48 rows each.
//
// Exactness as in the decode kernels: the MFMA consumes the exact 16-bit
// values MV + u (v_bitop3 on the packed nibbles) and the group's FP32 sum
// P = sum_k x (MV + u) is scaled by the group's FP16 scale s and added to the
// FP32 accumulator.  The zero point and MV come off as
// -s (MV + z) Sx, Sx = sum_k x of the row over the group: Sx is an MFMA of a
// row of ones against the activation fragment (the fragment as the second
// operand leaves Sx of row r in the lanes of output column r), and four
// groups' products are added by one FP32 MFMA (16x16x4, k = the four
// groups: lane q of a row holds Sx of group 4t + q, lane q of a column
// -s (MV + z) of the same group).  No vector-ALU work per row beyond the one
// scale multiply-add per group, for BF16 and FP16 alike.
//
// K split: with a workspace the K range is cut into S slices of whole groups
// when the blocks of one slice do not fill the device; slice sl writes FP32
// partials to ws[sl][M][N] and k_w4a16_gemm_reduce (k_w4a16_gemm.hip) adds
// them in slice order on the same stream.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_pipe.h"
#include "bg_w4.h"

namespace bg {

namespace {
constexpr int MID_XS = 3;               // LDS ring of staged activation groups
constexpr int MID_WST = 2;              // weight stages in registers
constexpr int MID_TNW = 4;              // weight tiles per wave
}  // namespace

template <int TNW>
struct MidStage {
    uint4 w[TNW];
    uint32_t s[TNW];
    uint32_t z[TNW];
};

template <bool BF16, int TMW, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void k_w4a16_mid(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                                       const uint8_t* __restrict__ zr, int64_t N,
                                                       uint16_t* __restrict__ y, float* __restrict__ ws, int gs) {
    constexpr int TNW = MID_TNW, NW = WM * WN;
    constexpr int BM = 16 * TMW * WM;
    constexpr int NCOPY = BM / 4;                                     // 1 KB copies (4 rows) per staged group
    constexpr int LX = (NCOPY + NW - 1) / NW;                         // copies per wave per group
    constexpr int LW = 3 * TNW;                                       // weight loads per lane per group
    constexpr int TP = 2;                                             // weight tiles per MFMA pass
    constexpr int XB = BM * 256;                                      // bytes of one staged group
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    static_assert(LX + 2 * LW < 64, "vmcnt is a 6-bit field");
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

    // weights, scales, zero bytes of this wave's tiles; reads past the
    // wave's tiles (ragged N) return 0
    const bool has_z = zr != nullptr;
    const int tt = my_tiles > 0 ? t0 : 0;
    // The group waits below count this wave's weight, scale and zero loads.
    // Loads through restrict arguments that no inline assembly names may be
    // moved across those waits (a "memory" clobber does not cover them), so
    // the three pointers pass through an empty asm first: loads through them
    // then stay where the source puts them.
    asm volatile("" : "+s"(qw), "+s"(sc), "+s"(zr));
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + (int64_t)tt * ngroups * 256), (short)0,
                                                      my_tiles * ngroups * 1024, 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + (int64_t)tt * ngroups * 16), (short)0,
                                                      my_tiles * ngroups * 32, 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(has_z ? zr + (int64_t)tt * (ngroups >> 1) * 16 : zr), (short)0,
        has_z ? my_tiles * (ngroups >> 1) * 16 : 0, 0x00020000);
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + m0 * K), (short)0,
                                                      (int)((int64_t)rows * K * 2), 0x00020000);

    // group i of the slice: past its last group every load repeats that
    // group (in bounds, never consumed), so each wave issues the same loads
    // at every step and the waits below count them exactly
    auto w_issue = [&](MidStage<TNW>& st, int i) {
        const int g = g0 + (i < ng - 1 ? i : ng - 1);
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            st.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16,
                                                                                       (j * ngroups + g) * 1024, 0));
            st.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, l16 * 2, (j * ngroups + g) * 32, 0);
            st.z[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, l16, (j * (ngroups >> 1) + (g >> 1)) * 16, 0);
        }
    };
    // copy c of a group fills LDS rows 4c .. 4c + 3 of its buffer (1 KB):
    // lane l writes row 4c + l / 16, 16-byte slot l % 16, which holds chunk
    // (l % 16) ^ (row % 16) of the row.  Rows past M copy row M - 1 (they
    // only feed output rows that are never written); a wave with fewer than
    // LX copies of its own repeats the last one (same bytes, same place).
    int xoff[LX];
    uint32_t xdst[LX];
#pragma unroll
    for (int u = 0; u < LX; ++u) {
        const int c = (u * NW + wave) < NCOPY ? u * NW + wave : NCOPY - 1;
        const int r = 4 * c + (lane >> 4);
        const int rr = r < rows ? r : rows - 1;
        xoff[u] = rr * (int)K * 2 + (((lane & 15) ^ (r & 15)) << 4);
        xdst[u] = (uint32_t)c * 1024;
    }
    auto x_issue = [&](int i) {
        const int g = g0 + (i < ng - 1 ? i : ng - 1);
        uint8_t* buf = dyn_lds + (i % MID_XS) * XB;
#pragma unroll
        for (int u = 0; u < LX; ++u) copy16_to_lds(rx, buf + xdst[u], xoff[u], g * 256);
    };

    // fragment (ii, kk) of lane (l16, q): row rw0 + 16 ii + l16, chunk 4q + kk
    // (k = 32q + 8kk .. + 7 of the group), at slot (4q + kk) ^ l16
    const uint8_t* xrow = dyn_lds + (rw0 + l16) * 256;
    const int sw0 = ((4 * q) ^ l16) << 4;

    float4_t acc[TMW][TNW];
#pragma unroll
    for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[ii][j] = float4_t{0, 0, 0, 0};
    float sel[TMW], bsel[TNW];                                        // correction operands of the current four groups
#pragma unroll
    for (int ii = 0; ii < TMW; ++ii) sel[ii] = 0.0f;
#pragma unroll
    for (int j = 0; j < TNW; ++j) bsel[j] = 0.0f;
    const uint32_t ones[4] = {ONE2, ONE2, ONE2, ONE2};

    auto consume = [&](const MidStage<TNW>& st, int i) {
        const int g = g0 + i;
        uint32_t xf[TMW][4][4];
        const uint8_t* xb = xrow + (i % MID_XS) * XB;
#pragma unroll
        for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4 v = *reinterpret_cast<const uint4*>(xb + ii * 4096 + (sw0 ^ (kk << 4)));
                xf[ii][kk][0] = v.x;
                xf[ii][kk][1] = v.y;
                xf[ii][kk][2] = v.z;
                xf[ii][kk][3] = v.w;
            }
        // every read of this buffer is issued: the group after next may now be copied
        asm volatile("" ::: "memory");
        x_issue(i + 2);
        asm volatile("" ::: "memory");

        // The MFMAs run as independent accumulation chains interleaved k step
        // by k step: TP weight tiles at a time, every row tile, and the row
        // sums Sx (ones x fragment^T) beside the first pair.  A chain's next
        // MFMA waits for the previous one's result, which a lone chain
        // exposes in full (measured on this chip: 45 cycles per 16x16x32
        // MFMA for one chain against 19 for independent ones).
        const bool mine = (i & 3) == q, first = (i & 3) == 0;
        float4_t sxa[TMW];
#pragma unroll
        for (int ii = 0; ii < TMW; ++ii) sxa[ii] = float4_t{0, 0, 0, 0};
#pragma unroll
        for (int j0 = 0; j0 < TNW; j0 += TP) {
            uint32_t D[TP][4][4];
#pragma unroll
            for (int jj = 0; jj < TP; ++jj) dequant_tile<BF16>(st.w[j0 + jj], D[jj]);
            float4_t part[TMW][TP];
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
                for (int jj = 0; jj < TP; ++jj) part[ii][jj] = float4_t{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ii = 0; ii < TMW; ++ii) {
                    if (j0 == 0) sxa[ii] = mfma16<BF16>(ones, xf[ii][kk], sxa[ii]);
#pragma unroll
                    for (int jj = 0; jj < TP; ++jj) part[ii][jj] = mfma16<BF16>(xf[ii][kk], D[jj][kk], part[ii][jj]);
                }
            if (j0 == 0) {
                // lane q of the four-group window takes group 4t + q; the
                // window's first group clears the other lanes (a last window
                // of fewer than four groups leaves them at zero)
#pragma unroll
                for (int ii = 0; ii < TMW; ++ii) sel[ii] = mine ? sxa[ii][0] : (first ? 0.0f : sel[ii]);
            }
#pragma unroll
            for (int jj = 0; jj < TP; ++jj) {
                const int j = j0 + jj;
                const float s = f16_to_f32(st.s[j] & 0xFFFFu);
#pragma unroll
                for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[ii][j][e] += s * part[ii][jj][e];
                const float zv = (float)(has_z ? (st.z[j] >> (4 * (g & 1))) & 0xFu : 8u);
                bsel[j] = mine ? -s * (MV + zv) : (first ? 0.0f : bsel[j]);
            }
        }
        if ((i & 3) == 3 || i == ng - 1) {
#pragma unroll
            for (int ii = 0; ii < TMW; ++ii)
#pragma unroll
                for (int j = 0; j < TNW; ++j)
                    acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sel[ii], bsel[j], acc[ii][j], 0, 0, 0);
        }
    };

    // group i: its copies have landed (own: the wait; everyone's: the
    // barrier) once at most its weight loads, the next group's copies and
    // the next group's weight loads are in flight; then the fragments are
    // read, the group after next is copied (ring slot of group i - 1, whose
    // reads all finished before this barrier), the group is consumed and its
    // weight stage refilled with the group after next
    MidStage<TNW> stage[MID_WST];
    x_issue(0);
    asm volatile("" ::: "memory");
    w_issue(stage[0], 0);
    asm volatile("" ::: "memory");
    x_issue(1);
    asm volatile("" ::: "memory");
    w_issue(stage[1], 1);
    auto step = [&](MidStage<TNW>& st, int i) {
        wait_vmcnt<LX + 2 * LW>();
        block_barrier();
        consume(st, i);
        asm volatile("" ::: "memory");
        w_issue(st, i + MID_WST);
    };
    static_assert(MID_WST == 2, "two stages: the loop body takes two groups");
    int i = 0;
    for (; i + 1 < ng; i += 2) {                                       // no branch inside: exact load counts
        step(stage[0], i);
        step(stage[1], i + 1);
    }
    if (i < ng) step(stage[0], i);
    wait_vmcnt<0>();                                                   // no copy into LDS outlives the block

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
    int TMW, WM, WN, S, gs;
    int64_t ws_bytes, lds_bytes;
    unsigned nblocks, bands;
};
constexpr int MID_WAVES = 8;            // waves per block

// Row bands of up to 96 rows; a band of R row tiles (16 rows) is split over
// WM = 2 waves from R = 4 (WM = 1 below), each with TMW = ceil(R / WM) <= 3
// row tiles; MID_WAVES waves in all, 4 tiles each.  K is split while one
// slice's blocks fill less than one round of 256 CUs, at least 3 groups per
// slice.
MidCfg mid_cfg(int64_t M, int64_t N, int64_t K, bool with_ws) {
    MidCfg c{};
    const int64_t bands = (M + 95) / 96;
    const int64_t band_rows = (M + bands - 1) / bands;
    const int64_t R = (band_rows + 15) / 16;
    c.WM = R >= 4 ? 2 : 1;
    c.TMW = (int)((R + c.WM - 1) / c.WM);
    c.WN = MID_WAVES / c.WM;
    const int64_t ntiles = N >> 4, ngroups = K >> 7;
    const int64_t nb = (ntiles + c.WN * MID_TNW - 1) / (c.WN * MID_TNW);
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
    c.lds_bytes = MID_XS * 16 * c.TMW * c.WM * 256;
    return c;
}

template <bool BF16, int TMW, int WM, int WN>
const char* mid_launch(const MidCfg& c, const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                       const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    auto kern = k_w4a16_mid<BF16, TMW, WM, WN>;
    if (c.lds_bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)c.lds_bytes);
    float* wsf = c.S > 1 ? static_cast<float*>(ws) : nullptr;
    hipLaunchKernelGGL(kern, dim3(c.nblocks, c.bands, (unsigned)c.S), dim3(WM * WN * 64), (size_t)c.lds_bytes, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y), wsf, c.gs);
    if (c.S > 1) launch_w4a16_gemm_reduce(BF16, wsf, c.S, M, N, y, s);
    return kname("k_w4a16_mid", BF16, TMW, MID_TNW, WM, WN);
}

template <bool BF16, int NWV>
const char* mid_shape(const MidCfg& c, const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                      const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    if (c.WM == 1) {
        if (c.TMW == 1) return mid_launch<BF16, 1, 1, NWV>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        if (c.TMW == 2) return mid_launch<BF16, 2, 1, NWV>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        return mid_launch<BF16, 3, 1, NWV>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    }
    if (c.TMW == 2) return mid_launch<BF16, 2, 2, NWV / 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    return mid_launch<BF16, 3, 2, NWV / 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
}
}  // namespace

int64_t w4a16_mid_workspace(int64_t M, int64_t N, int64_t K) { return mid_cfg(M, N, K, true).ws_bytes; }

const char* launch_w4a16_mid(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                             const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    const MidCfg c = mid_cfg(M, N, K, ws != nullptr);
    if (x_bf16) return mid_shape<true, MID_WAVES>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    return mid_shape<false, MID_WAVES>(c, x, M, K, qw, sc, zr, N, y, ws, s);
}

}  // namespace bg
