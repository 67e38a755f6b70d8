// k_w4a16_gemm.hip -- W4A16 linear for large M (prefill): Y = X W^T with W
// in the packed INT4 format, on the BF16/FP16 matrix cores.
//
// "Quantization throughput by method" (hrletsgo.me), W4A16 section: past the
// critical batch the W4A16 GEMM is compute-bound and the dequantization sits
// on its critical path.  "Low-precision LLM inference" §11 (INT4 weights,
// 16-bit activations), §23 (packed weights and scales go into the tile,
// dequantization in registers, one output write), §22 (FP32 accumulation).
//
// Exactness: a nibble OR-ed into the mantissa of MV (BF16 128.0 / FP16
// 1024.0) is the exact 16-bit value MV + u, so each 128-wide group is
// accumulated as T = sum_k x (MV + u) in FP32 by the MFMA, and the group's
// contribution s * (T - (MV + z) * Sx) is added once per group, with
// Sx = sum_k x over the group -- no rounding of the dequantized weight.
//
// Block tile 256 (rows of X) x 128 (output columns = 8 weight tiles), four
// waves as 2 x 2, each 128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16.  K
// advances in stages of 64 (half a group); each stage buffer holds
//   A: 256 rows x 128 bytes, 16-byte chunks XOR-swizzled by (row & 7),
//   W: the matching halves (512 bytes) of the 8 weight tiles,
//   the group's FP16 scales (8 x 32 bytes) and zero-point bytes (8 x 16),
// all copied by buffer_load ... lds; four buffers, two stages in flight while
// one is read (the pipeline of k_w8a8_gemm).
//
// K assignment: in K step s (16 k) of a stage, lane l (h = l / 32) supplies
// the 8 consecutive k starting at 32 (s / 2) + 16 h + 8 (s % 2) of its row of
// X and the same k of its output column of W: in the tile layout that is word
// 2h + s % 2 of slot 16 (s / 2) + n % 16 of the stage's half tile, which is
// read as one 8-byte LDS load per two K steps.  W is the MFMA's first operand,
// so lane l, register e holds output row l % 32 and column 8(e/4) + 4h + e%4.
// A lane's X values of a group are half of its row's k; Sx adds the partner
// lane l ^ 32's half.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_pipe.h"
#include "bg_w4.h"

namespace bg {

namespace {
constexpr int PBM = 256, PBN = 128;                 // block tile
constexpr int PKS = 64;                             // K per stage (half a group)
constexpr int P_A = PBM * PKS * 2;                  // 32 KB of activations
constexpr int P_W = (PBN / 16) * 512;               // 4 KB: half of each of 8 weight tiles
constexpr int P_S = (PBN / 16) * 32;                // 256 B: FP16 scales of the group
constexpr int P_Z = (PBN / 16) * 16;                // 128 B: zero-point bytes of the group pair
constexpr int P_STAGE = P_A + P_W + P_S + P_Z;
constexpr int P_NB = 4;
constexpr int P_LOADS = P_A / 4096 + 1 + 1;         // per wave per stage: 8 A, 1 W, 1 scales-or-zeros
static_assert((P_NB - 2) * P_LOADS < 64, "vmcnt range");
}  // namespace

template <bool BF16>
__global__ __launch_bounds__(256, 1) void k_w4a16_gemm(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const uint32_t* __restrict__ qw,
                                                       const uint16_t* __restrict__ sc,
                                                       const uint8_t* __restrict__ zr, int64_t N,
                                                       uint16_t* __restrict__ y) {
    constexpr int WTM = PBM / 2, WTN = PBN / 2, TM = WTM / 32, TN = WTN / 32;
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    constexpr int EPI_PITCH = WTN * 2 + 16;
    constexpr int EPI_BYTES = 4 * WTM * EPI_PITCH;
    constexpr int LDS_BYTES = P_NB * P_STAGE > EPI_BYTES ? P_NB * P_STAGE : EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const bool has_z = zr != nullptr;

    int tm, tn;
    grouped_tile(blockIdx.x, (int)((M + PBM - 1) / PBM), (int)((N + PBN - 1) / PBN), tm, tn);
    const int64_t m0 = (int64_t)tm * PBM, n0 = (int64_t)tn * PBN;
    const int64_t ngroups = K >> 7, ntiles = N >> 4, t0 = n0 >> 4;
    const int64_t tiles_here = ntiles - t0 < PBN / 16 ? ntiles - t0 : PBN / 16;

    // ---- buffer resources (rows / tiles past the end read as zero) ----
    const int64_t rows_a = M - m0 < PBM ? M - m0 : PBM;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + m0 * K), (short)0,
                                                      (int)(rows_a * K * 2), 0x00020000);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + t0 * ngroups * 256), (short)0,
                                                      (int)(tiles_here * ngroups * 1024), 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + t0 * ngroups * 16), (short)0,
                                                      (int)(tiles_here * ngroups * 32), 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(has_z ? zr + t0 * (ngroups >> 1) * 16 : zr), (short)0,
        has_z ? (int)(tiles_here * (ngroups >> 1) * 16) : 0, 0x00020000);

    // per-lane global offsets (the stage index goes into the scalar offset)
    uint32_t voff_a[P_A / 4096];
#pragma unroll
    for (int t = 0; t < P_A / 4096; ++t) {
        const int j = wave * (P_A / 4096) + t;                   // 1 KB run = 8 rows
        const int r = 8 * j + (lane >> 3);
        voff_a[t] = (uint32_t)(r * K * 2) + (uint32_t)((((lane & 7) ^ (r & 7)) << 4));
    }
    // W: wave w copies the stage halves of weight tiles 2w, 2w + 1
    const uint32_t voff_w = (uint32_t)((2 * wave + (lane >> 5)) * ngroups * 1024) + (uint32_t)((lane & 31) * 16);
    // scales (waves 0, 1: tiles 4w .. 4w+3, 32 bytes each) or zero bytes (waves 2, 3: 8 tiles x 16 bytes)
    const bool meta_lane = lane < 8;
    const uint32_t voff_m = wave < 2 ? (uint32_t)((4 * wave + (lane >> 1)) * ngroups * 32 + (lane & 1) * 16)
                                     : (uint32_t)(lane * (ngroups >> 1) * 16);
    auto issue = [&](int ks) {                                   // stage ks = half group
        uint8_t* buf = lds + (ks % P_NB) * P_STAGE;
#pragma unroll
        for (int t = 0; t < P_A / 4096; ++t)
            copy16_to_lds(ra, buf + (wave * (P_A / 4096) + t) * 1024, voff_a[t], ks * PKS * 2);
        copy16_to_lds(rw, buf + P_A + wave * 1024, voff_w, ks * 512);
        const int g = ks >> 1;
        if (meta_lane) {
            if (wave < 2) copy16_to_lds(rs, buf + P_A + P_W + wave * 128, voff_m, g * 32);
            else copy16_to_lds(rz, buf + P_A + P_W + P_S, voff_m, (g >> 1) * 16);
        }
    };

    // ---- fragment addresses ----
    const uint32_t lds0 = lds_addr(lds);
    // X row wm*128 + 32i + l32 (swizzle depends on l32 only); chunk c = 4(s/2) + 2h + s%2
    uint32_t offa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = 4 * (s >> 1) + 2 * h + (s & 1);
        offa[s] = (uint32_t)((wm * WTM + l32) * 128 + ((c ^ (l32 & 7)) << 4));
    }
    // W: weight tile wn*4 + 2j + l32/16, slot (16 (s/2) + l32 % 16), words 2h, 2h+1
    const uint32_t offw = (uint32_t)(P_A + (wn * 4 + (l32 >> 4)) * 512 + (l32 & 15) * 16 + 8 * h);

    struct StageFr {
        int4_t a[TM][4];                                         // X fragments per K step
        uint2 w[TN][2];                                          // packed words: K steps (0,1), (2,3)
    };
    auto read_frags = [&](StageFr& f, int ks) {
        const uint32_t base = lds0 + (uint32_t)((ks % P_NB) * P_STAGE);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < TM; ++i) f.a[i][s] = ds_read16(base + offa[s] + (uint32_t)(i * 32 * 128));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            f.w[j][0] = ds_read8(base + offw + (uint32_t)(j * 2 * 512));
            f.w[j][1] = ds_read8(base + offw + (uint32_t)(j * 2 * 512 + 16 * 16));
        }
    };
    auto settle_frags = [&](StageFr& f) {
        wait_lgkm0();
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s) settle(f.a[i][s]);
#pragma unroll
        for (int j = 0; j < TN; ++j) settle(f.w[j][0]), settle(f.w[j][1]);
    };

    float16_t acc[TM][TN], tmp[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = float16_t{}, tmp[i][j] = float16_t{};
    float sx[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) sx[i] = 0.0f;

    auto mfma = [&](const int4_t& bv, const int4_t& av, float16_t c) -> float16_t {
        if constexpr (BF16)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf168_t, bv),
                                                           __builtin_bit_cast(bf168_t, av), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, bv),
                                                          __builtin_bit_cast(half8_t, av), c, 0, 0, 0);
    };
    // group end: acc += s * (T - (MV + z) * Sx), scales and zeros from the stage buffer
    auto close_group = [&](int ks) {
        const uint8_t* buf = lds + (ks % P_NB) * P_STAGE;
        const int g = ks >> 1;
        float sxf[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) sxf[i] = sx[i] + __shfl_xor(sx[i], 32), sx[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                // columns 8 q4 + 4h .. +3 of the j-th 32: tile wn*4 + 2j + q4/2, column 8 (q4 % 2) + 4h
                const int tt = wn * 4 + 2 * j + (q4 >> 1), col = 8 * (q4 & 1) + 4 * h;
                uint2 s4 = ds_read8(lds_addr(buf + P_A + P_W + tt * 32 + col * 2));
                uint32_t z4 = ds_read4(lds_addr(buf + P_A + P_W + P_S + tt * 16 + col));
                wait_lgkm0();
                settle(s4), settle(z4);
                const float sv[4] = {f16_to_f32(s4.x & 0xFFFF), f16_to_f32(s4.x >> 16), f16_to_f32(s4.y & 0xFFFF),
                                     f16_to_f32(s4.y >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float c = MV + (has_z ? (float)((z4 >> (8 * r + 4 * (g & 1))) & 0xF) : 8.0f);
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const float t = tmp[i][j][4 * q4 + r] - c * sxf[i];
                        acc[i][j][4 * q4 + r] += sv[r] * t;
                    }
                }
            }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) tmp[i][j] = float16_t{};
    };

    // One step: stage ks's fragments were requested into `cur`; the barrier
    // publishes stage ks + 1 and frees the buffer of stage ks - 1 (every wave
    // holds its stage-ks fragments), which receives stage ks + P_NB - 1.
    const int nks = (int)(K / PKS);
    auto step = [&](StageFr& cur, StageFr& nxt, int ks) {
        settle_frags(cur);
        wait_vmcnt<(P_NB - 3) * P_LOADS>();
        block_barrier();
        issue(ks + P_NB - 1);
        // Sx partials of this stage (VALU, overlaps the MFMAs)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                sx[i] = dot2<BF16>((uint32_t)cur.a[i][s].x, ONE2, sx[i]);
                sx[i] = dot2<BF16>((uint32_t)cur.a[i][s].y, ONE2, sx[i]);
                sx[i] = dot2<BF16>((uint32_t)cur.a[i][s].z, ONE2, sx[i]);
                sx[i] = dot2<BF16>((uint32_t)cur.a[i][s].w, ONE2, sx[i]);
            }
        // 32 MFMAs; the 20 reads of the next stage spread between them
        constexpr int NMF = 4 * TM * TN, NRD = 4 * TM + 2 * TN;
        const uint32_t nb = lds0 + (uint32_t)(((ks + 1) % P_NB) * P_STAGE);
        int4_t pbv = int4_t{}, pav = int4_t{};                   // operands of the previous MFMA
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            const int s = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
            const uint2 wp = cur.w[j][s >> 1];
            uint32_t d[4];
            dequant_word<BF16>((s & 1) ? wp.y : wp.x, d);
            const int4_t bv = int4_t{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
            tmp[i][j] = mfma(bv, cur.a[i][s], tmp[i][j]);
            if (t == 0) pbv = bv, pav = cur.a[i][s];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = t * NRD / NMF; r < (t + 1) * NRD / NMF; ++r) {
                if (r < 4 * TM) {
                    const int rs_ = r / TM, ri = r % TM;
                    nxt.a[ri][rs_] =
                        ds_read16_after(nb + offa[rs_] + (uint32_t)(ri * 32 * 128), bv, cur.a[i][s], pbv, pav);
                } else {
                    const int rj = (r - 4 * TM) >> 1, rh = (r - 4 * TM) & 1;
                    nxt.w[rj][rh] = ds_read8_after(nb + offw + (uint32_t)(rj * 2 * 512 + rh * 16 * 16), bv,
                                                   cur.a[i][s], pbv, pav);
                }
            }
            pbv = bv, pav = cur.a[i][s];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (ks & 1) close_group(ks);
    };

    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<(P_NB - 2) * P_LOADS>();
    block_barrier();
    StageFr f0, f1;
    read_frags(f0, 0);
    for (int ks = 0; ks < nks; ks += 2) {                        // K is a multiple of 256: nks is even
        step(f0, f1, ks);
        step(f1, f0, ks + 1);
    }
    wait_vmcnt<0>();
    wait_lgkm0();

    // ---- epilogue: stage this wave's 128 x 64 tile in LDS, write 16-byte row segments ----
    block_barrier();
    const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
    uint8_t* stage = lds + wave * WTM * EPI_PITCH;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 packed;
                packed.x = (uint32_t)to_out<BF16>(acc[i][j][4 * q4]) | ((uint32_t)to_out<BF16>(acc[i][j][4 * q4 + 1]) << 16);
                packed.y = (uint32_t)to_out<BF16>(acc[i][j][4 * q4 + 2]) |
                           ((uint32_t)to_out<BF16>(acc[i][j][4 * q4 + 3]) << 16);
                *reinterpret_cast<uint2*>(stage + (i * 32 + l32) * EPI_PITCH + (j * 32 + 8 * q4 + 4 * h) * 2) = packed;
            }
    constexpr int LPR = WTN / 8, RPI = 64 / LPR;
    const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll 4
    for (int r0 = 0; r0 < WTM; r0 += RPI) {
        const int r = r0 + rr;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * EPI_PITCH + cc * 16);
        const int64_t m = mw + r, n = nw + cc * 8;
        if (m < M && n < N) *reinterpret_cast<uint4*>(y + m * N + n) = v;
    }
}

template <bool BF16>
static const char* gemm_launch(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                               const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    const int64_t tiles = ((M + PBM - 1) / PBM) * ((N + PBN - 1) / PBN);
    hipLaunchKernelGGL(k_w4a16_gemm<BF16>, dim3((unsigned)tiles), dim3(256), 0, s, static_cast<const uint16_t*>(x), M,
                       K, qw, sc, zr, N, static_cast<uint16_t*>(y));
    return kname("k_w4a16_gemm", BF16);
}

const char* launch_w4a16_gemm(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return gemm_launch<true>(x, M, K, qw, sc, zr, N, y, s);
    return gemm_launch<false>(x, M, K, qw, sc, zr, N, y, s);
}

}  // namespace bg
