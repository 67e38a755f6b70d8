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
// 1024.0) is the exact 16-bit value MV + u.  FP16: one packed subtraction of
// (MV + z) gives the exact integer u - z, and the MFMA accumulates the group's
// T = sum_k x (u - z).  BF16 (no packed BF16 arithmetic): the MFMA
// accumulates sum_k x (MV + u) and one extra K step per group adds
// -(MV + z) * Sx, Sx = sum_k x over the group, split exactly into three BF16
// parts.  Either way the group's contribution s * T is added once per group in
// FP32 -- no rounding of the dequantized weight.
//
// Block tile 256 (rows of X) x 128 (output columns = 8 weight tiles), WM x 2
// waves, each (256 / WM) x 64 of v_mfma_f32_32x32x16 tiles.  K advances in
// stages of 64 (half a group); each stage buffer holds
//   A: 256 rows x 128 bytes, 16-byte chunks XOR-swizzled by xswz(row),
//   W: the matching halves (512 bytes) of the 8 weight tiles,
// all copied by buffer_load ... lds; four buffers: while stage ks + 1 is read,
// stages ks + 2 .. ks + 4 are in flight (the buffer of stage ks is refilled as
// soon as every wave holds its fragments).  The group's FP16 scales (8 x 32
// bytes) and zero-point bytes (8 x 16) go to slot g % 4 of a separate ring,
// so they stay put until the group is closed.
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

// 16-byte chunk swizzle of a 128-byte activation row in LDS.  It depends on
// bits 0..4 of the row only (fragments 32 rows apart share it), and with it
// the fragment reads (32 consecutive rows, chunk c ^ xswz) hit the LDS
// without bank conflicts -- measured with the bank-conflict counter on that
// read pattern, where row & 7 spent half of the LDS cycles in conflicts.
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 2)) & 7; }

namespace {
constexpr int PBM = 256, PBN = 128;                 // block tile
constexpr int PKS = 64;                             // K per stage (half a group)
constexpr int P_A = PBM * PKS * 2;                  // 32 KB of activations
constexpr int P_W = (PBN / 16) * 512;               // 4 KB: half of each of 8 weight tiles
constexpr int P_S = (PBN / 16) * 32;                // 256 B: FP16 scales of the group
constexpr int P_Z = (PBN / 16) * 16;                // 128 B: zero-point bytes of the group pair
constexpr int P_STAGE = P_A + P_W;
constexpr int P_META = P_S + 2 * P_Z;               // scales + zero bytes of one group (zero bytes twice)
constexpr int P_MSLOTS = 4;                         // group g's metadata lives in slot g % 4
constexpr int P_NB = 4;
}  // namespace

template <bool BF16, int WM>
__global__ __launch_bounds__(128 * WM, 1) void k_w4a16_gemm(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const uint32_t* __restrict__ qw,
                                                       const uint16_t* __restrict__ sc,
                                                       const uint8_t* __restrict__ zr, int64_t N,
                                                       uint16_t* __restrict__ y, float* __restrict__ ws, int S,
                                                       int gs) {
    constexpr int NW = 2 * WM;                                   // waves: WM x 2
    constexpr int WTM = PBM / WM, WTN = PBN / 2, TM = WTM / 32, TN = WTN / 32;
    // copies per wave per stage: A_LD of X (1 KB each), then one of W and one of
    // metadata (4 waves) or one of W-or-metadata (8 waves)
    constexpr int A_LD = P_A / 1024 / NW;
    constexpr int P_LOADS = A_LD + (NW == 4 ? 2 : 1);
    static_assert((P_NB - 1) * P_LOADS < 64, "vmcnt range");
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    constexpr int EPI_PITCH = WTN * 2 + 16;
    constexpr int EPI_BYTES = NW * WTM * EPI_PITCH;
    constexpr int RING_BYTES = P_NB * P_STAGE + P_MSLOTS * P_META;
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
    const int tiles_m = (int)((M + PBM - 1) / PBM), tiles_n = (int)((N + PBN - 1) / PBN);
    const int sl = blockIdx.x / (tiles_m * tiles_n);
    // one 256-row band of X per XCD at a time: its 2 MB over K is 8x a block's
    // packed weights (M = 2048: gate_up 582 us against 589 with bands of 8
    // row tiles, down 283 against 289)
    grouped_tile<1>(blockIdx.x - sl * tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * PBM, n0 = (int64_t)tn * PBN;
    const int64_t ngroups = K >> 7, ntiles = N >> 4, t0 = n0 >> 4;
    const int g_beg = sl * gs, g_end = g_beg + gs < ngroups ? g_beg + gs : (int)ngroups;
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
    uint32_t voff_a[A_LD];
#pragma unroll
    for (int t = 0; t < A_LD; ++t) {
        const int j = wave * A_LD + t;                           // 1 KB run = 8 rows
        const int r = 8 * j + (lane >> 3);
        voff_a[t] = (uint32_t)(r * K * 2) + (uint32_t)((((lane & 7) ^ xswz(r)) << 4));
    }
    // W: wave w < 4 copies the stage halves of weight tiles 2w, 2w + 1
    const int ww = wave & 3;
    const uint32_t voff_w = (uint32_t)((2 * ww + (lane >> 5)) * ngroups * 1024) + (uint32_t)((lane & 31) * 16);
    // metadata, 4 bytes per lane and every lane active (LDS copies narrower
    // than 16 bytes put each lane's data in a 4-byte slot): even waves copy
    // the group's 256 scale bytes (tile lane / 8, bytes 4 (lane % 8)), odd
    // waves its 128 zero-point bytes (tile (lane % 32) / 4, bytes 4 (lane % 4)),
    // lanes 32..63 the same bytes again into a spare 128; waves 0..3 with four
    // waves, 4..7 with eight (pairs copy the same bytes to the same place)
    const bool m_scales = (wave & 1) == 0;
    const uint32_t voff_m = m_scales ? (uint32_t)((lane >> 3) * ngroups * 32 + (lane & 7) * 4)
                                     : (uint32_t)(((lane & 31) >> 2) * (ngroups >> 1) * 16 + (lane & 3) * 4);
    // Stages past the end of K repeat the last stage's bytes (metadata: the
    // last group's) into free buffers and slots that are never consumed, so
    // no copy leaves its tensor.
    const int ks_last = (int)(2 * ngroups) - 1;
    auto copy_meta = [&](int ks) {
        // both stages of group g copy its metadata to slot g % 4 (the same bytes)
        const int g = (ks < ks_last ? ks : ks_last) >> 1;
        uint8_t* meta = lds + P_NB * P_STAGE + ((ks >> 1) % P_MSLOTS) * P_META;
        if (m_scales)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)meta, 4, voff_m + (uint32_t)(g * 32), 0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_ptr_t)(meta + P_S), 4,
                                                     voff_m + (uint32_t)((g >> 1) * 16), 0, 0, 0);
    };
    // copy number t (0 .. P_LOADS-1) of stage ks = half group
    auto issue_one = [&](int ks, int t) {
        uint8_t* buf = lds + (ks % P_NB) * P_STAGE;
        const int kc = ks < ks_last ? ks : ks_last;
        if (t < A_LD) {
            copy16_to_lds(ra, buf + (wave * A_LD + t) * 1024, voff_a[t], kc * PKS * 2);
        } else if (t == A_LD && (NW == 4 || wave < 4)) {
            copy16_to_lds(rw, buf + P_A + ww * 1024, voff_w, kc * 512);
        } else {
            copy_meta(ks);
        }
    };
    auto issue = [&](int ks) {
#pragma unroll
        for (int t = 0; t < P_LOADS; ++t) issue_one(ks, t);
    };

    // ---- fragment addresses ----
    const uint32_t lds0 = lds_addr(lds);
    // X row wm*WTM + 32i + l32 (swizzle depends on l32 only); chunk c = 4(s/2) + 2h + s%2
    uint32_t offa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = 4 * (s >> 1) + 2 * h + (s & 1);
        offa[s] = (uint32_t)((wm * WTM + l32) * 128 + ((c ^ xswz(l32)) << 4));
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
    float sx[TM];                                                // BF16: Sx partials of this lane's k
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

    // Zero point of this lane's weight column (row l32 of W fragment j) for a
    // group, from the zero bytes of a stage buffer: FP16 keeps the pair
    // (MV + z, MV + z) to subtract, BF16 the bits of -(MV + z).
    const int zcol = l32 & 15;
    const uint32_t meta0 = lds_addr(lds) + (uint32_t)(P_NB * P_STAGE);
    auto zaddr = [&](int g, int j) {
        return meta0 + (uint32_t)((g % P_MSLOTS) * P_META + P_S + (wn * 4 + 2 * j + (l32 >> 4)) * 16 + (zcol & ~3));
    };
    auto zword = [&](uint32_t zd, int g) -> uint32_t {
        const uint32_t z = has_z ? (zd >> (8 * (zcol & 3) + 4 * (g & 1))) & 0xFu : 8u;
        if constexpr (BF16) return 0xC300u | z;                  // -(128 + z)
        else return (0x6400u | z) * 0x00010001u;                 // (1024 + z) in both halves
    };
    uint32_t zw[TN], zd_next[TN];
    // scales of this lane's columns 8 q4 + 4h .. +3 of the j-th 32 (weight tile
    // wn*4 + 2j + q4/2, column 8 (q4 % 2) + 4h) in the metadata slot of group g
    auto saddr = [&](int g, int j, int q4) {
        return meta0 + (uint32_t)((g % P_MSLOTS) * P_META + (wn * 4 + 2 * j + (q4 >> 1)) * 32 + (8 * (q4 & 1) + 4 * h) * 2);
    };

    // Group end.  BF16: one more MFMA K step per tile adds -(MV + z) * Sx,
    // with Sx split exactly into three BF16 parts (hi + mid + lo, truncation
    // leaves at most 16 then 8 significant bits) -- products of BF16 pairs
    // are exact in the FP32 accumulator.  FP16 dequantized u - z directly.
    // Then acc += s * T with the group's FP16 scales (16 reads issued
    // together, one wait; they follow MFMAs whose operands b1, a1, b0, a0
    // they must not overwrite).
    auto close_group = [&](int g, int4_t b1, int4_t a1, int4_t b0, int4_t a0) {
        if constexpr (BF16) {
            int4_t xf[TM], wf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const float sxf = sx[i] + __shfl_xor(sx[i], 32);
                sx[i] = 0.0f;
                const uint32_t hi = __float_as_uint(sxf) >> 16;
                const float r1 = sxf - __uint_as_float(hi << 16);
                const uint32_t mid = __float_as_uint(r1) >> 16;
                const float r2 = r1 - __uint_as_float(mid << 16);
                const uint32_t lo = __float_as_uint(r2) >> 16;
                xf[i] = h ? int4_t{0, 0, 0, 0} : int4_t{(int)(hi | (mid << 16)), (int)lo, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
                wf[j] = h ? int4_t{0, 0, 0, 0} : int4_t{(int)(zw[j] | (zw[j] << 16)), (int)zw[j], 0, 0};
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    tmp[i][j] = mfma(wf[j], xf[i], tmp[i][j]);
                    b0 = b1, a0 = a1, b1 = wf[j], a1 = xf[i];
                }
            __builtin_amdgcn_sched_barrier(0);
        }
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
                    for (int i = 0; i < TM; ++i) acc[i][j][4 * q4 + r] += sv[r] * tmp[i][j][4 * q4 + r];
            }
    };

    // One step: stage ks's fragments were requested into `cur`; the barrier
    // publishes stage ks + 1 and frees the buffer of stage ks (every wave
    // holds its stage-ks fragments), which receives stage ks + P_NB.
    // first: ks opens a group (its first MFMA per tile starts from zero);
    // otherwise ks closes the group and reads the zero points of the next one.
    // Copies and reads of stage ks + 1 are spread between the MFMAs.
    auto step = [&](StageFr& cur, StageFr& nxt, int ks, bool first) {
        settle_frags(cur);
        wait_vmcnt<(P_NB - 2) * P_LOADS>();
        block_barrier();
        issue(ks + P_NB);
        if constexpr (BF16) {
            // Sx partials of this stage (VALU, overlaps the MFMAs)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    sx[i] = dot2<BF16>((uint32_t)cur.a[i][s2].x, ONE2, sx[i]);
                    sx[i] = dot2<BF16>((uint32_t)cur.a[i][s2].y, ONE2, sx[i]);
                    sx[i] = dot2<BF16>((uint32_t)cur.a[i][s2].z, ONE2, sx[i]);
                    sx[i] = dot2<BF16>((uint32_t)cur.a[i][s2].w, ONE2, sx[i]);
                }
        }
        // 32 MFMAs; the 20 reads of the next stage spread between them
        constexpr int NMF = 4 * TM * TN, NRD = 4 * TM + 2 * TN;
        const uint32_t nb = lds0 + (uint32_t)(((ks + 1) % P_NB) * P_STAGE);
        int4_t pbv = int4_t{}, pav = int4_t{};                   // operands of the previous MFMA
        int4_t ppbv = int4_t{}, ppav = int4_t{};                 // ... and of the one before
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            const int s = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
            const uint2 wp = cur.w[j][s >> 1];
            uint32_t d[4];
            dequant_word<BF16>((s & 1) ? wp.y : wp.x, d);
            if constexpr (!BF16) {
#pragma unroll
                for (int p = 0; p < 4; ++p) d[p] = sub_h2(d[p], zw[j]);
            }
            const int4_t bv = int4_t{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
            tmp[i][j] = mfma(bv, cur.a[i][s], (first && s == 0) ? float16_t{} : tmp[i][j]);
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
            if (!first && t < TN) zd_next[t] = ds_read4_after(zaddr((ks + 1) >> 1, t), bv, cur.a[i][s], pbv, pav);

            ppbv = pbv, ppav = pav;
            pbv = bv, pav = cur.a[i][s];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!first) {
            close_group(ks >> 1, pbv, pav, ppbv, ppav);
            wait_lgkm0();                                        // the zero-point reads (stage ks + 1 stays put)
#pragma unroll
            for (int j = 0; j < TN; ++j) settle(zd_next[j]), zw[j] = zword(zd_next[j], (ks + 1) >> 1);
        }
    };

    // stages 2 g_beg .. 2 g_end - 1 (stages past the slice copy bytes never consumed)
    const int ks0 = 2 * g_beg, ks1 = 2 * g_end;
#pragma unroll
    for (int t = 0; t < P_NB; ++t) issue(ks0 + t);
    wait_vmcnt<(P_NB - 1) * P_LOADS>();
    block_barrier();
    StageFr f0, f1;
    read_frags(f0, ks0);
#pragma unroll
    for (int j = 0; j < TN; ++j) zd_next[j] = ds_read4(zaddr(g_beg, j));
    wait_lgkm0();
#pragma unroll
    for (int j = 0; j < TN; ++j) settle(zd_next[j]), zw[j] = zword(zd_next[j], g_beg);
    for (int ks = ks0; ks < ks1; ks += 2) {
        step(f0, f1, ks, true);
        step(f1, f0, ks + 1, false);
    }
    wait_vmcnt<0>();
    // the last step read the (unused) stage after the slice into f0: those
    // registers stay allocated until the reads have landed, or a value the
    // compiler put there (the group close, the epilogue) would be overwritten
    settle_frags(f0);
    const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
    if (S > 1) {
        // FP32 partial tile of slice sl -> ws[sl][M][N] (k_w4a16_gemm_reduce adds
        // the slices): lane l, register e of tile (i, j) holds row 32 i + l % 32,
        // columns 32 j + 8 (e / 4) + 4 h + e % 4 -- four consecutive floats
        float* part = ws + (int64_t)sl * M * N;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + 32 * i + l32;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int64_t n = nw + 32 * j + 8 * q4 + 4 * h;
                    if (m < M && n < N)
                        *reinterpret_cast<float4*>(part + m * N + n) =
                            make_float4(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                                        acc[i][j][4 * q4 + 3]);
                }
        }
        return;
    }

    // ---- epilogue: stage this wave's tile in LDS, write 16-byte row segments ----
    block_barrier();
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

// y[m][n] = sum over the S slices of ws[s][m][n], in slice order (results do
// not depend on timing).  One thread per 8 consecutive outputs of a row.
template <bool BF16>
__global__ __launch_bounds__(256) void k_w4a16_gemm_reduce(const float* __restrict__ ws, int S, int64_t M, int64_t N,
                                                           uint16_t* __restrict__ y) {
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
    uint4 o;
    o.x = (uint32_t)to_out<BF16>(v[0]) | ((uint32_t)to_out<BF16>(v[1]) << 16);
    o.y = (uint32_t)to_out<BF16>(v[2]) | ((uint32_t)to_out<BF16>(v[3]) << 16);
    o.z = (uint32_t)to_out<BF16>(v[4]) | ((uint32_t)to_out<BF16>(v[5]) << 16);
    o.w = (uint32_t)to_out<BF16>(v[6]) | ((uint32_t)to_out<BF16>(v[7]) << 16);
    *reinterpret_cast<uint4*>(y + e) = o;
}

void launch_w4a16_gemm_reduce(bool bf16, const float* ws, int S, int64_t M, int64_t N, void* y, hipStream_t s) {
    const int64_t threads = M * N / 8;
    if (bf16)
        hipLaunchKernelGGL((k_w4a16_gemm_reduce<true>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, ws,
                           S, M, N, static_cast<uint16_t*>(y));
    else
        hipLaunchKernelGGL((k_w4a16_gemm_reduce<false>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, ws,
                           S, M, N, static_cast<uint16_t*>(y));
}

// K slices for the large-M kernel: while its tiles do not fill one round (one
// block per CU), split K into whole groups, at least 4 per slice.
W4GemmSplit w4a16_gemm_split(int64_t M, int64_t N, int64_t K) {
    W4GemmSplit c{1, (int)(K >> 7), 0};
    const int64_t tiles = ((M + PBM - 1) / PBM) * ((N + PBN - 1) / PBN), ngroups = K >> 7;
    int64_t S = 256 / tiles;
    if (S > ngroups / 4) S = ngroups / 4;
    if (S < 2) return c;
    const int64_t gs = (ngroups + S - 1) / S;
    c.S = (int)((ngroups + gs - 1) / gs);
    c.gs = (int)gs;
    c.ws_bytes = c.S > 1 ? (int64_t)c.S * M * N * 4 : 0;
    if (c.S < 2) c = W4GemmSplit{1, (int)ngroups, 0};
    return c;
}

template <bool BF16, int WM>
static const char* gemm_launch(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                               const uint8_t* zr, int64_t N, void* y, float* ws, const W4GemmSplit& c,
                               hipStream_t s) {
    const int64_t tiles = ((M + PBM - 1) / PBM) * ((N + PBN - 1) / PBN);
    hipLaunchKernelGGL((k_w4a16_gemm<BF16, WM>), dim3((unsigned)(tiles * c.S)), dim3(128 * WM), 0, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y), ws, c.S,
                       c.gs);
    if (c.S > 1) {
        const int64_t threads = M * N / 8;
        hipLaunchKernelGGL((k_w4a16_gemm_reduce<BF16>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(ws), c.S, M, N, static_cast<uint16_t*>(y));
    }
    return kname("k_w4a16_gemm", BF16, WM);
}

const char* launch_w4a16_gemm(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s) {
    // eight waves (two per SIMD): one wave's dequantization and group
    // arithmetic overlap the other's MFMAs (measured 15% faster than four)
    constexpr int WM = 4;
    const W4GemmSplit c = ws ? w4a16_gemm_split(M, N, K) : W4GemmSplit{1, (int)(K >> 7), 0};
    float* wsf = static_cast<float*>(ws);
    if (x_bf16) return gemm_launch<true, WM>(x, M, K, qw, sc, zr, N, y, wsf, c, s);
    return gemm_launch<false, WM>(x, M, K, qw, sc, zr, N, y, wsf, c, s);
}

}  // namespace bg
