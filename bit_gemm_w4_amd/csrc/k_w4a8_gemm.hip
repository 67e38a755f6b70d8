// k_w4a8_gemm.hip -- W4A8 linear: Y = (A s_a) W^T with A the INT8 activation
// codes (dynamic per-token or per-tensor scale s_a) and W in the packed INT4
// format, on the INT8 matrix cores.
//
// "Low-precision LLM inference" §1 (W4A8: INT4 weights, INT8 activations,
// INT32/FP32 accumulation, BF16 or FP16 output), §14 (per-token activation
// scales), §20 (a W4A8 kernel pays for the dequantization of its INT4
// weights) and self-check Q2 (W4A8 lowers the activations too, to reach a
// native low-precision GEMM).
//
// Exactness: a nibble u and its group's zero point z (both 0..15) give the
// signed byte u - z exactly, four at a time: (u + 0x80 - z) per byte never
// carries, and flipping bit 7 turns it into the two's complement of u - z.
// v_mfma_i32_32x32x32_i8 then accumulates the group's T = sum_k a (u - z)
// exactly in INT32 (|T| <= 128 * 128 * 15 < 2^24, so T is also exact in
// FP32), and acc += s * T closes each group in FP32; s_a scales each output
// row in the epilogue.
//
// Block tile 256 rows of A x 128 output columns (8 weight tiles), 8 waves
// (4 x 2, two per SIMD) of 64 x 64 = 2 x 2 MFMA tiles.  K advances in stages
// of 64 (half a group); each stage buffer holds
//   A: 256 rows x 64 bytes, 16-byte chunks swizzled by bits 0..3 of the row,
//   W: the matching halves (512 bytes) of the 8 weight tiles,
// copied by buffer_load ... lds; six buffers: while stage ks + 1 is read,
// stages ks + 2 .. ks + 6 are in flight (the buffer of stage ks is refilled as
// soon as every wave holds its fragments).  The group's FP16 scales and
// zero-point bytes go to slot g % 4 of a separate ring.  With six buffers the
// stage issued while group g closes belongs to group g + 3, whose slot is the
// one group g - 1 released, never g's or g + 1's.
//
// K assignment: in K step s (32 k) of a stage, lane l (h = l / 32) supplies
// the 16 consecutive k starting at 32 s + 16 h of its row of A and the same k
// of its output column of W: in the tile layout that is words 2h, 2h + 1 of
// slot 16 s + n % 16 of the stage's half tile (one 8-byte LDS load).  A packed
// word holds its even k in the low nibbles and its odd k in the high ones;
// two byte permutes put them back in k order.  W is the MFMA's first operand,
// so lane l, register e holds output row l % 32 and column 8(e/4) + 4h + e%4.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_pipe.h"
#include "bg_w4.h"

namespace bg {

namespace {
constexpr int QBM = 256, QBN = 128;                 // block tile
constexpr int QKS = 64;                             // K per stage (half a group)
constexpr int Q_A = QBM * QKS;                      // 16 KB of activation codes
constexpr int Q_W = (QBN / 16) * 512;               // 4 KB: half of each of 8 weight tiles
constexpr int Q_S = (QBN / 16) * 32;                // 256 B: FP16 scales of the group
constexpr int Q_Z = (QBN / 16) * 16;                // 128 B: zero-point bytes of the group pair
constexpr int Q_STAGE = Q_A + Q_W;
constexpr int Q_META = Q_S + 2 * Q_Z;               // scales + zero bytes of one group (zero bytes twice)
constexpr int Q_MSLOTS = 4;                         // group g's metadata lives in slot g % 4
constexpr int Q_NB = 6;
constexpr int Q_WM = 4, Q_NW = 2 * Q_WM;            // waves: 4 x 2

enum { QO_F32 = 0, QO_F16 = 1, QO_BF16 = 2 };

// 16-byte chunk swizzle of a 64-byte LDS row: the fragment reads (32
// consecutive rows, chunk 2s + h) hit the LDS without bank conflicts --
// measured with the bank-conflict counter on that pattern, where
// ((r >> 1) ^ (r >> 3)) & 3 spent half of the LDS cycles in conflicts.
__device__ __forceinline__ int qswz(int r) { return (r ^ (r >> 2)) & 3; }

}  // namespace

__global__ __launch_bounds__(64 * Q_NW, 1) void k_w4a8_gemm(const int8_t* __restrict__ a,
                                                          const float* __restrict__ as, int a_row,
                                                          int64_t M, int64_t K, const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ sc,
                                                          const uint8_t* __restrict__ zr, int64_t N,
                                                          void* __restrict__ y, int out_dt, float* __restrict__ ws,
                                                          int S, int gs) {
    constexpr int NW = Q_NW;
    constexpr int WTM = QBM / Q_WM, WTN = QBN / 2, TM = WTM / 32, TN = WTN / 32;
    // copies per wave per stage: A_LD of A (1 KB = 16 rows each), then one of W
    // (waves 0..3) or of metadata (waves 4..7)
    constexpr int A_LD = Q_A / 1024 / NW;
    constexpr int LOADS = A_LD + 1;
    static_assert((Q_NB - 1) * LOADS < 64, "vmcnt range");
    constexpr int EPI_PITCH = WTN * 2 + 16;
    constexpr int EPI_BYTES = NW * WTM * EPI_PITCH;
    constexpr int RING_BYTES = Q_NB * Q_STAGE + Q_MSLOTS * Q_META;
    constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const bool has_z = zr != nullptr;

    // block b: output tile b % T, K slice b / T (groups [sl gs, sl gs + gs))
    int tm, tn;
    const int tiles_m = (int)((M + QBM - 1) / QBM), tiles_n = (int)((N + QBN - 1) / QBN);
    const int sl = blockIdx.x / (tiles_m * tiles_n);
    grouped_tile(blockIdx.x - sl * tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * QBM, n0 = (int64_t)tn * QBN;
    const int64_t ngroups = K >> 7, ntiles = N >> 4, t0 = n0 >> 4;
    const int g_beg = sl * gs, g_end = g_beg + gs < ngroups ? g_beg + gs : (int)ngroups;
    const int64_t tiles_here = ntiles - t0 < QBN / 16 ? ntiles - t0 : QBN / 16;

    // ---- buffer resources (rows / tiles past the end read as zero) ----
    const int64_t rows_a = M - m0 < QBM ? M - m0 : QBM;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a + m0 * K), (short)0, (int)(rows_a * K),
                                                      0x00020000);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + t0 * ngroups * 256), (short)0,
                                                      (int)(tiles_here * ngroups * 1024), 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + t0 * ngroups * 16), (short)0,
                                                      (int)(tiles_here * ngroups * 32), 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(has_z ? zr + t0 * (ngroups >> 1) * 16 : zr), (short)0,
        has_z ? (int)(tiles_here * (ngroups >> 1) * 16) : 0, 0x00020000);

    // per-lane global offsets (the stage goes into the scalar offset)
    uint32_t voff_a[A_LD];
#pragma unroll
    for (int t = 0; t < A_LD; ++t) {
        const int r = 16 * (wave * A_LD + t) + (lane >> 2);
        voff_a[t] = (uint32_t)(r * K) + (uint32_t)((((lane & 3) ^ qswz(r)) << 4));
    }
    // W: wave w < 4 copies the stage halves of weight tiles 2w, 2w + 1
    const int ww = wave & 3;
    const uint32_t voff_w = (uint32_t)((2 * ww + (lane >> 5)) * ngroups * 1024) + (uint32_t)((lane & 31) * 16);
    // metadata (waves 4..7), 4 bytes per lane and every lane active (LDS
    // copies narrower than 16 bytes put each lane's data in a 4-byte slot):
    // even waves copy the group's 256 scale bytes (tile lane / 8, bytes
    // 4 (lane % 8)), odd waves its 128 zero-point bytes (tile (lane % 32) / 4,
    // bytes 4 (lane % 4)), lanes 32..63 the same bytes again into a spare
    // 128; the two pairs copy the same bytes to the same place
    const bool m_scales = (wave & 1) == 0;
    const uint32_t voff_m = m_scales ? (uint32_t)((lane >> 3) * ngroups * 32 + (lane & 7) * 4)
                                     : (uint32_t)(((lane & 31) >> 2) * (ngroups >> 1) * 16 + (lane & 3) * 4);
    // Every step issues the same number of copies (the stage waits count
    // them); the stages past the end of the slice repeat its last stage's
    // bytes into a free buffer that is never consumed, so no copy leaves its
    // tensor.
    const int ks0 = 2 * g_beg, ks1 = 2 * g_end, ks_last = ks1 - 1;
    auto issue_one = [&](int ks, int t) {
        uint8_t* buf = lds + (ks % Q_NB) * Q_STAGE;
        const int kc = ks < ks_last ? ks : ks_last;
        if (t < A_LD) {
            copy16_to_lds(ra, buf + (wave * A_LD + t) * 1024, voff_a[t], kc * QKS);
        } else if (wave < 4) {
            copy16_to_lds(rw, buf + Q_A + ww * 1024, voff_w, kc * 512);
        } else {
            // both stages of group g copy its metadata to slot g % 4 (the same
            // bytes); past the end the slots of groups that never come
            const int g = kc >> 1;
            uint8_t* meta = lds + Q_NB * Q_STAGE + ((ks >> 1) % Q_MSLOTS) * Q_META;
            if (m_scales)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)meta, 4, voff_m + (uint32_t)(g * 32), 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_ptr_t)(meta + Q_S), 4,
                                                         voff_m + (uint32_t)((g >> 1) * 16), 0, 0, 0);
        }
    };
    auto issue = [&](int ks) {
#pragma unroll
        for (int t = 0; t < LOADS; ++t) issue_one(ks, t);
    };

    // ---- fragment addresses ----
    const uint32_t lds0 = lds_addr(lds);
    // A row wm*WTM + 32i + l32 (swizzle depends on l32 only), chunk 2s + h
    uint32_t offa[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        offa[s] = (uint32_t)((wm * WTM + l32) * QKS + (((2 * s + h) ^ qswz(l32)) << 4));
    // W: weight tile wn*4 + 2j + l32/16, slot 16 s + l32 % 16, words 2h, 2h + 1
    const uint32_t offw = (uint32_t)(Q_A + (wn * 4 + (l32 >> 4)) * 512 + (l32 & 15) * 16 + 8 * h);

    struct StageFr {
        int4_t a[TM][2];                                         // A fragments per K step
        uint2 w[TN][2];                                          // packed words per K step
    };
    auto read_frags = [&](StageFr& f, int ks) {
        const uint32_t base = lds0 + (uint32_t)((ks % Q_NB) * Q_STAGE);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < TM; ++i) f.a[i][s] = ds_read16(base + offa[s] + (uint32_t)(i * 32 * QKS));
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s) f.w[j][s] = ds_read8(base + offw + (uint32_t)(j * 2 * 512 + s * 16 * 16));
    };
    auto settle_frags = [&](StageFr& f) {
        wait_lgkm0();
#pragma unroll
        for (int i = 0; i < TM; ++i) settle(f.a[i][0]), settle(f.a[i][1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) settle(f.w[j][0]), settle(f.w[j][1]);
    };

    float16_t acc[TM][TN];
    int16_t_v tmp[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = float16_t{}, tmp[i][j] = int16_t_v{};

    // Zero point of this lane's weight column for group g, folded into the
    // per-byte constant 0x80 - z (z = 8 without zero points).
    const int zcol = l32 & 15;
    const uint32_t meta0 = lds0 + (uint32_t)(Q_NB * Q_STAGE);
    auto zaddr = [&](int g, int j) {
        return meta0 + (uint32_t)((g % Q_MSLOTS) * Q_META + Q_S + (wn * 4 + 2 * j + (l32 >> 4)) * 16 + (zcol & ~3));
    };
    auto zconst = [&](uint32_t zd, int g) -> uint32_t {
        const uint32_t z = has_z ? (zd >> (8 * (zcol & 3) + 4 * (g & 1))) & 0xFu : 8u;
        return 0x80808080u - z * 0x01010101u;
    };
    uint32_t zc[TN], zd_next[TN];
    // scales of this lane's output columns 8 q4 + 4h .. +3 of the j-th 32
    // (weight tile wn*4 + 2j + q4/2, column 8 (q4 % 2) + 4h) for group g
    auto saddr = [&](int g, int j, int q4) {
        return meta0 + (uint32_t)((g % Q_MSLOTS) * Q_META + (wn * 4 + 2 * j + (q4 >> 1)) * 32 + (8 * (q4 & 1) + 4 * h) * 2);
    };

    // Group end: acc += s * T with the group's FP16 scales (read after MFMAs
    // whose operands b1, a1, b0, a0 they must not overwrite).
    auto close_group = [&](int g, int4_t b1, int4_t a1, int4_t b0, int4_t a0) {
        uint2 s4[TN][4];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) s4[j][q4] = ds_read8_after(saddr(g, j, q4), b1, a1, b0, a0);
        wait_lgkm0();
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                settle(s4[j][q4]);
                const uint2 sv2 = s4[j][q4];
                const float sv[4] = {f16_to_f32(sv2.x & 0xFFFF), f16_to_f32(sv2.x >> 16), f16_to_f32(sv2.y & 0xFFFF),
                                     f16_to_f32(sv2.y >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < TM; ++i) acc[i][j][4 * q4 + r] += sv[r] * (float)tmp[i][j][4 * q4 + r];
            }
    };

    // One step: stage ks's fragments were requested into `cur`; the barrier
    // publishes stage ks + 1 and frees the buffer of stage ks, which receives
    // stage ks + Q_NB.  first: ks opens a group (its first MFMA per tile starts
    // from zero); otherwise ks closes it and reads the next group's zero points.
    // The reads of stage ks + 1 are spread between the MFMAs, one each.
    auto step = [&](StageFr& cur, StageFr& nxt, int ks, bool first) {
        settle_frags(cur);
        wait_vmcnt<(Q_NB - 2) * LOADS>();
        block_barrier();
        issue(ks + Q_NB);
        constexpr int NMF = 2 * TM * TN, NRD = 2 * TM + 2 * TN;
        static_assert(NRD == NMF, "one read per MFMA");
        const uint32_t nb = lds0 + (uint32_t)(((ks + 1) % Q_NB) * Q_STAGE);
        int4_t pbv = int4_t{}, pav = int4_t{};                   // operands of the previous MFMA
        int4_t ppbv = int4_t{}, ppav = int4_t{};                 // ... and of the one before
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            const int s = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
            const int4_t bv = w4_to_i8(cur.w[j][s], zc[j]);
            tmp[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, cur.a[i][s],
                                                              (first && s == 0) ? int16_t_v{} : tmp[i][j], 0, 0, 0);
            if (t == 0) pbv = bv, pav = cur.a[i][s];
            __builtin_amdgcn_sched_barrier(0);
            if (t < 2 * TM) {
                const int rs_ = t / TM, ri = t % TM;
                nxt.a[ri][rs_] = ds_read16_after(nb + offa[rs_] + (uint32_t)(ri * 32 * QKS), bv, cur.a[i][s], pbv, pav);
            } else {
                const int rj = (t - 2 * TM) >> 1, rh = (t - 2 * TM) & 1;
                nxt.w[rj][rh] =
                    ds_read8_after(nb + offw + (uint32_t)(rj * 2 * 512 + rh * 16 * 16), bv, cur.a[i][s], pbv, pav);
            }
            if (!first && t < TN) zd_next[t] = ds_read4_after(zaddr((ks + 1) >> 1, t), bv, cur.a[i][s], pbv, pav);
            ppbv = pbv, ppav = pav;
            pbv = bv, pav = cur.a[i][s];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!first) {
            close_group(ks >> 1, pbv, pav, ppbv, ppav);
            wait_lgkm0();                                        // the zero-point reads
#pragma unroll
            for (int j = 0; j < TN; ++j) settle(zd_next[j]), zc[j] = zconst(zd_next[j], (ks + 1) >> 1);
        }
    };

#pragma unroll
    for (int t = 0; t < Q_NB; ++t) issue(ks0 + t);
    wait_vmcnt<(Q_NB - 1) * LOADS>();
    block_barrier();
    StageFr f0, f1;
    read_frags(f0, ks0);
#pragma unroll
    for (int j = 0; j < TN; ++j) zd_next[j] = ds_read4(zaddr(g_beg, j));
    wait_lgkm0();
#pragma unroll
    for (int j = 0; j < TN; ++j) settle(zd_next[j]), zc[j] = zconst(zd_next[j], g_beg);
    for (int ks = ks0; ks < ks1; ks += 2) {
        step(f0, f1, ks, true);
        step(f1, f0, ks + 1, false);
    }
    wait_vmcnt<0>();                                             // no copy may land after the block exits
    // the last step read the (unused) stage after the slice into f0: those
    // registers stay allocated until the reads have landed, or a value the
    // compiler put there (the group close, the epilogue) would be overwritten
    settle_frags(f0);

    // ---- epilogue: row scale s_a, then the output type ----
    const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
    float sa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = mw + 32 * i + l32;
        sa[i] = a_row ? (m < M ? as[m] : 0.0f) : as[0];
    }
    // F32 output, or (S > 1) this slice's partial tile -> ws[sl][M][N], which
    // k_w4a8_reduce adds up in slice order
    if (out_dt == QO_F32 || S > 1) {
        float* yf = S > 1 ? ws + (int64_t)sl * M * N : static_cast<float*>(y);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + 32 * i + l32;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int64_t n = nw + 32 * j + 8 * q4 + 4 * h;      // N % 16 == 0: all four or none
                    if (m < M && n < N)
                        *reinterpret_cast<float4*>(yf + m * N + n) =
                            make_float4(acc[i][j][4 * q4] * sa[i], acc[i][j][4 * q4 + 1] * sa[i],
                                        acc[i][j][4 * q4 + 2] * sa[i], acc[i][j][4 * q4 + 3] * sa[i]);
                }
        }
        return;
    }
    // 16-bit outputs: stage this wave's tile in LDS, write 16-byte row segments
    block_barrier();
    uint8_t* stage = lds + wave * WTM * EPI_PITCH;
    const bool bf = out_dt == QO_BF16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint32_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = acc[i][j][4 * q4 + r] * sa[i];
                    o[r] = bf ? f32_to_bf16(v) : f32_to_f16(v);
                }
                *reinterpret_cast<uint2*>(stage + (i * 32 + l32) * EPI_PITCH + (j * 32 + 8 * q4 + 4 * h) * 2) =
                    make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            }
    constexpr int LPR = WTN / 8, RPI = 64 / LPR;
    const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll 4
    for (int r0 = 0; r0 < WTM; r0 += RPI) {
        const int r = r0 + rr;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * EPI_PITCH + cc * 16);
        const int64_t m = mw + r, n = nw + cc * 8;
        if (m < M && n < N) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + m * N + n) = v;
    }
}

// y[m][n] = sum over the S slices of ws[s][m][n], in slice order (results do
// not depend on timing), written as out_dt.  One thread per 8 consecutive
// outputs of a row (N % 16 == 0).
__global__ __launch_bounds__(256) void k_w4a8_reduce(const float* __restrict__ ws, int S, int64_t M, int64_t N,
                                                     void* __restrict__ y, int out_dt) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e >= M * N) return;
    const int64_t slice = M * N;
    constexpr int RB = 8;                                      // slices in flight per batch
    float v[8];
    for (int b0 = 0; b0 < S; b0 += RB) {
        float4 lo[RB], hi[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (b0 + r < S) {
                lo[r] = *reinterpret_cast<const float4*>(ws + (b0 + r) * slice + e);
                hi[r] = *reinterpret_cast<const float4*>(ws + (b0 + r) * slice + e + 4);
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (b0 + r >= S) break;
            const float p[8] = {lo[r].x, lo[r].y, lo[r].z, lo[r].w, hi[r].x, hi[r].y, hi[r].z, hi[r].w};
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = b0 + r == 0 ? p[c] : v[c] + p[c];
        }
    }
    if (out_dt == QO_F32) {
        float* yf = static_cast<float*>(y) + e;
        *reinterpret_cast<float4*>(yf) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(yf + 4) = make_float4(v[4], v[5], v[6], v[7]);
        return;
    }
    const bool bf = out_dt == QO_BF16;
    uint32_t o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = bf ? f32_to_bf16(v[c]) : f32_to_f16(v[c]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + e) =
        make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16));
}

// K slices: while the output tiles do not fill one round (one block per CU),
// split K into whole groups, at least 4 per slice.
W4GemmSplit w4a8_gemm_split(int64_t M, int64_t N, int64_t K) {
    W4GemmSplit c{1, (int)(K >> 7), 0};
    const int64_t tiles = ((M + QBM - 1) / QBM) * ((N + QBN - 1) / QBN), ngroups = K >> 7;
    int64_t S = 256 / tiles;
    if (S > ngroups / 4) S = ngroups / 4;
    if (S < 2) return c;
    const int64_t gs = (ngroups + S - 1) / S;
    S = (ngroups + gs - 1) / gs;
    if (S < 2) return c;
    c.S = (int)S;
    c.gs = (int)gs;
    c.ws_bytes = S * M * N * 4;
    return c;
}

const char* launch_w4a8_gemm(const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K, const uint32_t* qw,
                             const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, int out_dt, void* ws,
                             hipStream_t s) {
    const W4GemmSplit c = ws ? w4a8_gemm_split(M, N, K) : W4GemmSplit{1, (int)(K >> 7), 0};
    const int64_t tiles = ((M + QBM - 1) / QBM) * ((N + QBN - 1) / QBN);
    hipLaunchKernelGGL(k_w4a8_gemm, dim3((unsigned)(tiles * c.S)), dim3(64 * Q_NW), 0, s, a, as, a_row ? 1 : 0, M, K,
                       qw, sc, zr, N, y, out_dt, static_cast<float*>(ws), c.S, c.gs);
    if (c.S > 1) {
        const int64_t threads = M * N / 8;
        hipLaunchKernelGGL(k_w4a8_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(ws), c.S, M, N, y, out_dt);
        return "k_w4a8_gemm + k_w4a8_reduce";
    }
    return "k_w4a8_gemm";
}

}  // namespace bg
