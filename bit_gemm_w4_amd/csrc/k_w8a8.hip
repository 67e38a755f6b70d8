// k_w8a8.hip -- native INT8 / FP8-E4M3 GEMM (gemm_w8a8) and its variants:
// MXFP8 / MXFP4 (gemm_mxfp8, gemm_mxfp4) and the LLM.int8() side path
// (gemm_w8a8_outlier).
//
// "Quantization throughput by method" (hrletsgo.me), W8A8/FP8 section: weights
// and activations both in 8 bits, the GEMM runs on the low-precision matrix
// cores with no upcast.  "Low-precision LLM inference" §8 (scale recipe and
// 128-wide block scaling), §10 (MX block formats), §14 (W8A8), §16 (outlier
// side path), §22 (INT32 / FP32 accumulators).
//
// Y = A W^T, A [M][K], W [N][K], both K-contiguous.  This file holds the
// large-M kernel (32x32 MFMA tiles, multi-stage LDS pipeline, below); the
// small-M kernel is in k_w8a8_decode.hip.  The K assignment of operand bytes
// to lanes is the same for A and W, so matching k are multiplied whatever the
// hardware's own k order is.
#include <type_traits>

#include "bg_device.h"
#include "bg_internal.h"
#include "bg_pipe.h"

namespace bg {

enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_I32 = 5 };
enum { GT = 0, GR = 1, GR128 = 2, GB128 = 3, GMX32 = 4, GMX4 = 5 };

// ============================================================================
// Large-M GEMM.  Block tile BM x BN; K advances in stages of 64 bytes (one LDS
// row per operand row), NB stage buffers (as many as fit in 160 KB, at most 6;
// 5 for 128 x 128 tiles, which run two blocks per CU):
// while stage kb + 1 is read, stages kb + 2 .. kb + NB are in flight (the
// buffer of stage kb is refilled as soon as every wave holds its fragments).  Global -> LDS copies are
// buffer_load_dwordx4 ... lds (no trip through VGPRs): lane i of a wave writes
// bytes [16i, 16i+16) of a 1 KB LDS run = 16 rows x 64 bytes, so the 16-byte
// chunk swizzle is applied on the global side (lane i fetches chunk
// (i & 3) ^ swz(row)).  swz(r) = (r ^ (r >> 2)) & 3: the fragment reads
// (lane l: row base + l % 32, chunk (l / 32) ^ swz or (2 + l / 32) ^ swz)
// then hit the LDS without bank conflicts -- measured with the bank-conflict
// counter on that exact pattern, where ((r >> 1) ^ (r >> 3)) & 3 spent half
// of the LDS cycles in conflicts.
// 2 x WN waves (WN = 2: one wave per SIMD; WN = 4: two, so one wave's LDS
// and memory waits overlap the other's MFMAs); each owns a (BM/2) x (BN/WN)
// tile of 32x32 MFMA tiles:
// v_mfma_i32_32x32x32_i8 (lane l supplies 16 bytes of row l%32: chunk l/32
// in the first half of the stage, 2 + l/32 in the second),
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (32 bytes: both chunks) or,
// for MXFP4, with E2M1 operands (16 bytes, one chunk per K step of 64
// elements, two steps per stage).  The W fragment is the
// first operand, so output lane l, register e holds row l%32 of the A tile
// and column 8(e/4) + 4(l/32) + e%4 of the W tile.
// Block order: grouped_tile (XCD-aware, bands of 8 row tiles; 4 for the
// 256 x 128 tiles, whose activation rows are twice their weight rows).
// ============================================================================
constexpr int GK = 64;                                           // K bytes per stage

__device__ __forceinline__ int gswz(int r) { return (r ^ (r >> 2)) & 3; }

template <int TM, int TN, int MXR>
struct Frags {
    int4_t a[TM][2], b[TN][2];                  // two 16-byte K chunks per 32-row fragment
    uint32_t sa[TM][MXR], sb[TN][MXR];          // MX: the lane's E8M0 byte(s) of each fragment row
};

// MX: 0 = none, MX_F8 = MXFP8 operands, MX_F4 = MXFP4 operands
enum { MX_F8 = 1, MX_F4 = 2 };

// One element of x [.][K] (F32 / F16 / BF16) as a float.
__device__ __forceinline__ float load1_f32(const void* x, int dt, int64_t i) {
    if (dt == DT_F32) return static_cast<const float*>(x)[i];
    const uint32_t h = static_cast<const uint16_t*>(x)[i];
    return dt == DT_BF16 ? bf16_to_f32(h) : f16_to_f32(h);
}

// OL (INT8 only): the LLM.int8() side path.  The common columns of the
// activations arrive as INT8 codes (outlier columns zero); after the K loop
// the block adds, for each listed outlier column k, x[m][k] * w[n][k] from the
// unquantized activations and the INT8 weight codes (the weight scale applies
// to both parts in the epilogue).
template <bool FP8, bool BLOCK, int BM, int BN, int WN, int MX = 0, bool OL = false>
__global__ __launch_bounds__(128 * WN, 1) void k_w8a8_gemm(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                      int a_gran, const uint8_t* __restrict__ w,
                                                      const float* __restrict__ ws, int w_gran, int64_t M,
                                                      int64_t N, int64_t K, void* __restrict__ y, int out_dt,
                                                      void* __restrict__ part, int S, int spl,
                                                      const void* __restrict__ ox, int ox_dt,
                                                      const int32_t* __restrict__ oidx,
                                                      const int32_t* __restrict__ ocnt) {
    constexpr int NW = 2 * WN;                                   // waves
    constexpr int WTM = BM / 2, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWS = BM + BN;                                // LDS rows per stage
    // MXFP4: a stage's 64 bytes of a row are 128 elements, two MFMA K steps
    // of 64 (32 bytes each); MXFP8: 64 elements, one step
    constexpr bool F4 = MX == MX_F4;
    // MX: a stage also holds the E8M0 bytes of its RUNS 32-wide K blocks: A
    // blocks RUNS kb .. RUNS kb + RUNS - 1 (BM bytes each), then the same for
    // W (BN each)
    constexpr int RUNS = F4 ? 4 : 2;
    constexpr int MXR = F4 ? 2 : 1;                              // scale bytes per fragment row and stage
    constexpr int MXS = MX ? RUNS * ROWS : 0;
    constexpr int STAGE_BYTES = ROWS * GK + MXS;
    constexpr int LOADS = ROWS / (16 * NW);                      // 1 KB wave-loads per wave per stage
    // MX: the scale area is copied 256 bytes per wave-copy, MXC copies per
    // wave and stage
    static_assert(!MX || (FP8 && !BLOCK), "MX scaling is an FP8-family variant");
    static_assert(!BLOCK || FP8, "128 x 128 block scales are an FP8 variant (one MFMA per tile and stage)");
    constexpr int MX_AREA = RUNS * ROWS;
    constexpr int MXC = MX ? (MX_AREA + 256 * NW - 1) / (256 * NW) : 0;
    constexpr int LOADS_T = LOADS + MXC;
    // stage buffers: 128 x 128 keeps 5 (80 KB), so two blocks share a CU
    constexpr int NB_FIT = (160 * 1024) / STAGE_BYTES;
    constexpr int NB_MAX = BM * BN <= 128 * 128 || BLOCK ? 5 : 6;
    constexpr int NB = NB_FIT > NB_MAX ? NB_MAX : NB_FIT;
    static_assert(ROWS % (16 * NW) == 0 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
    static_assert(!BLOCK || WTN <= 128, "one 128-column weight scale block per wave");
    static_assert(NB >= 3 && (NB - 1) * LOADS_T + (BLOCK ? 4 * TM : 0) < 64, "stage count / vmcnt range");
    static_assert(!BLOCK || NB == 5, "the block-scale load count in the stage waits assumes five buffers");
    static_assert(STAGE_BYTES % 16 == 0, "stage alignment");
    constexpr int EPI_PITCH = WTN * 2 + 16;                      // bytes per staged output row (padded, 16-aligned)
    constexpr int EPI_BYTES = NW * WTM * EPI_PITCH;
    constexpr int LDS_BYTES = NB * STAGE_BYTES > EPI_BYTES ? NB * STAGE_BYTES : EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;

    // ---- tile and K slice of this block: tile b % T, slice b / T (stages
    // [sl spl, sl spl + spl) of 64 bytes) ----
    int tm, tn;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int sl = blockIdx.x / (tiles_m * tiles_n);
    // (down at M = 2048, 256 x 128 tiles: 134.4 / 124.8 us INT8 / FP8 with
    // bands of 4 against 136.1 / 127.9 with 8; the square tiles keep 8)
    grouped_tile<(BM == 256 && BN == 128) ? 4 : 8>(blockIdx.x - sl * tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    // ---- global -> LDS copies (rows past M or N read as zero) ----
    const int64_t KB = F4 ? K >> 1 : K;                          // bytes per row
    const int64_t rows_a = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a + m0 * KB), (short)0,
                                                      (int)(rows_a * KB), 0x00020000);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + n0 * KB), (short)0,
                                                      (int)(rows_w * KB), 0x00020000);
    uint32_t voff[LOADS];
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
        const int j = wave * LOADS + t;                          // wave-load index in the stage
        const int r = (j < BM / 16 ? 16 * j : 16 * (j - BM / 16)) + (lane >> 2);
        voff[t] = (uint32_t)(r * KB) + (uint32_t)((((lane & 3) ^ gswz(r)) << 4));
    }
    const int nkb = (int)(KB / GK);
    const int kb0 = sl * spl, kb1 = kb0 + spl < nkb ? kb0 + spl : nkb;
    // MX scales are K-block-major, [K/32][rows padded to 16] bytes, so a K
    // block's bytes for the tile's rows are one contiguous run.  The stage's
    // scale area holds the runs A(RUNS kb + r), r < RUNS, then W's; wave-copy
    // c of wave w moves the area's bytes [256 p, 256 p + 256), p = w + NW c,
    // with one 4-byte-per-lane copy, every lane active (each lane picks its
    // run and row), and copies past the area repeat its last 256 bytes.
    // (as / ws point to the E8M0 bytes.)
    static_assert(!MX || (MX_AREA % 256 == 0 && (RUNS * BM) % 256 == 0), "MX scale area in whole waves");
    const int64_t mpad = (M + 15) & ~(int64_t)15, npad = (N + 15) & ~(int64_t)15;
    constexpr int MXC1 = MXC > 0 ? MXC : 1;
    int mx_piece[MXC1];
    uint32_t mx_voff[MXC1];
    int64_t mx_stride[MXC1];
    __amdgpu_buffer_rsrc_t rsx[MXC1];
#pragma unroll
    for (int c = 0; c < MXC1; ++c) {
        const int p = wave + NW * c;
        mx_piece[c] = 256 * p < MX_AREA ? p : MX_AREA / 256 - 1;
        const int pos = mx_piece[c] * 256 + lane * 4;            // byte of the scale area
        const bool on_a = mx_piece[c] * 256 < RUNS * BM;          // wave-uniform
        const int run = on_a ? pos / BM : (pos - RUNS * BM) / BN;
        const int row = on_a ? pos % BM : (pos - RUNS * BM) % BN;
        mx_stride[c] = on_a ? mpad : npad;
        rsx[c] = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<uint8_t*>(const_cast<float*>(on_a ? as : ws)) + (MX ? (on_a ? m0 : n0) : 0), (short)0,
            MX ? (int)((K >> 5) * mx_stride[c] - (on_a ? m0 : n0)) : 0, 0x00020000);
        mx_voff[c] = (uint32_t)(run * mx_stride[c] + row);
    }
    auto mx_copy = [&](int kb, int c) {
        if constexpr (MX) {
            const int kc = kb < nkb - 1 ? kb : nkb - 1;          // past the end: repeat the last stage's runs
            // the whole offset per lane, so the range check covers it
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsx[c], (lds_ptr_t)(lds + (kb % NB) * STAGE_BYTES + ROWS * GK + mx_piece[c] * 256), 4,
                mx_voff[c] + (uint32_t)(RUNS * kc * mx_stride[c]), 0, 0, 0);
        }
    };
    // Stage kb goes to buffer kb % NB.  Stages past the end of K repeat the
    // last stage's bytes into a free buffer that is never consumed (so no copy
    // leaves its tensor).  With MX, copies LOADS .. LOADS_T - 1 are the scale runs.
    auto issue_one = [&](int kb, int t) {
        if (MX && t >= LOADS) {
            mx_copy(kb, t - LOADS);
            return;
        }
        const int j = wave * LOADS + t;
        const int kc = kb < nkb - 1 ? kb : nkb - 1;
        copy16_to_lds(j < BM / 16 ? ra : rw, lds + (kb % NB) * STAGE_BYTES + j * 16 * GK, voff[t], kc * GK);
    };
    auto issue = [&](int kb) {
#pragma unroll
        for (int t = 0; t < LOADS_T; ++t) issue_one(kb, t);
    };

    // ---- fragment addresses: lane l reads chunks h and 2 + h of row l % 32 ----
    // (the same K chunks for A and W, so matching k meet in the MFMA).  The
    // swizzle of row r depends on bits 0..3 of r only, so fragments 32 rows
    // apart differ by a constant 2 KB.
    const uint32_t lds0 = lds_addr(lds);
    const int ra0 = wm * WTM + l32, rb0 = BM + wn * WTN + l32;
    const uint32_t offa0 = (uint32_t)(ra0 * GK + ((h ^ gswz(ra0)) << 4));
    const uint32_t offa1 = (uint32_t)(ra0 * GK + (((2 + h) ^ gswz(ra0)) << 4));
    const uint32_t offb0 = (uint32_t)(rb0 * GK + ((h ^ gswz(rb0)) << 4));
    const uint32_t offb1 = (uint32_t)(rb0 * GK + (((2 + h) ^ gswz(rb0)) << 4));
    // MX: the lane's scale byte of a fragment row for MFMA step c of the
    // stage: block 2c + h (MXFP8 has the one step c = 0), i.e. run 2c + h,
    // and the row's byte in the run.  (The scaled MFMA takes the scale of K
    // block b of a row from lane half b; an MXFP4 lane half holds exactly its
    // block's 32 elements, an MXFP8 lane half the 16-byte chunks h and 2 + h,
    // which the hardware reads as K block h.)
    const uint32_t mxa0 = (uint32_t)(ROWS * GK + h * BM + ra0);
    const uint32_t mxb0 = (uint32_t)(ROWS * GK + RUNS * BM + h * BN + (rb0 - BM));
    auto mx_base = [&](int kb) { return lds0 + (uint32_t)((kb % NB) * STAGE_BYTES); };
    constexpr int NFRAG = 2 * (TM + TN);
    using FragsT = Frags<TM, TN, MXR>;
    // read number r of a stage (0 .. NREAD-1): A fragments first, then W, then
    // (MX) the scale bytes of the A and W fragment rows, step by step
    auto mx_addr = [&](uint32_t mxb, int i) {
        const int c = i / (TM + TN), f = i % (TM + TN);
        return f < TM ? mxb + mxa0 + (uint32_t)(c * 2 * BM + f * 32)
                      : mxb + mxb0 + (uint32_t)(c * 2 * BN + (f - TM) * 32);
    };
    auto mx_slot = [&](FragsT& f, int i) -> uint32_t& {
        const int c = i / (TM + TN), g = i % (TM + TN);
        return g < TM ? f.sa[g][c] : f.sb[g - TM][c];
    };
    auto read_one = [&](FragsT& f, uint32_t base, uint32_t mxb, int r) {
        if (r >= NFRAG) {
            const int i = r - NFRAG;
            mx_slot(f, i) = ds_read1(mx_addr(mxb, i));
            return;
        }
        const int frag = r >> 1, c = r & 1;
        if (frag < TM)
            f.a[frag][c] = ds_read16(base + (c ? offa1 : offa0) + (uint32_t)(frag * 32 * GK));
        else
            f.b[frag - TM][c] = ds_read16(base + (c ? offb1 : offb0) + (uint32_t)((frag - TM) * 32 * GK));
    };
    // the same, issued right after MFMAs whose operands must stay untouched
    // (an MXFP4 operand is the fragment's 16 bytes: the MFMA reads 4 registers)
    using op_t = typename std::conditional<FP8 && !F4, int8_t_v, int4_t>::type;
    auto read_one_after = [&](FragsT& f, uint32_t base, uint32_t mxb, int r, const op_t& a1, const op_t& b1,
                              const op_t& a0, const op_t& b0) {
        if (r >= NFRAG) {
            const int i = r - NFRAG;
            mx_slot(f, i) = ds_read1_after(mx_addr(mxb, i), a1, b1, a0, b0);
            return;
        }
        const int frag = r >> 1, c = r & 1;
        if (frag < TM)
            f.a[frag][c] = ds_read16_after(base + (c ? offa1 : offa0) + (uint32_t)(frag * 32 * GK), a1, b1, a0, b0);
        else
            f.b[frag - TM][c] =
                ds_read16_after(base + (c ? offb1 : offb0) + (uint32_t)((frag - TM) * 32 * GK), a1, b1, a0, b0);
    };
    auto stage_base = [&](int kb) { return lds0 + (uint32_t)((kb % NB) * STAGE_BYTES); };
    auto settle_frags = [&](FragsT& f) {
        wait_lgkm0();
#pragma unroll
        for (int i = 0; i < TM; ++i) settle(f.a[i][0]), settle(f.a[i][1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) settle(f.b[j][0]), settle(f.b[j][1]);
        if constexpr (MX) {
#pragma unroll
            for (int c = 0; c < MXR; ++c) {
#pragma unroll
                for (int i = 0; i < TM; ++i) settle(f.sa[i][c]);
#pragma unroll
                for (int j = 0; j < TN; ++j) settle(f.sb[j][c]);
            }
        }
    };

    using acc_t = typename std::conditional<FP8, float16_t, int16_t_v>::type;
    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
    float16_t facc[BLOCK ? TM : 1][BLOCK ? TN : 1];
    if constexpr (BLOCK) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) facc[i][j] = float16_t{};
    }
    // every second stage closes a 128-wide K block: facc += partial * s_a[m][kb] * s_w[n/128][kb].
    // The scales of K block c are loaded at the close of block c - SCP (a ring
    // of SCP blocks in registers, rotated at every close), so most of their
    // latency is hidden.  The loads are unconditional (rows past M read row
    // M - 1, blocks past the end of K the last one).  The stage waits below
    // do not count them: they read through restrict pointers that no inline
    // assembly names, so the compiler may move them across the waits (it
    // sank the first ring's loads below the prologue wait, which then let the
    // first stage's fragment reads race its copies).
    constexpr int SCP = 4;
    const int64_t nkb128 = K >> 7;
    const int64_t nbw = (n0 + wn * WTN) >> 7;                    // this wave's 128-column weight block
    float sa_ring[BLOCK ? SCP : 1][BLOCK ? TM : 1];
    float sw_ring[BLOCK ? SCP : 1];
    auto load_scales = [&](float (&sa)[BLOCK ? TM : 1], float& sw, int64_t c) {
        if constexpr (BLOCK) {
            const int64_t cc = c < nkb128 ? c : nkb128 - 1;
            sw = ws[(nbw < (N >> 7) ? nbw : (N >> 7) - 1) * nkb128 + cc];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int64_t m = m0 + wm * WTM + i * 32 + l32;
                sa[i] = as[(m < M ? m : M - 1) * nkb128 + cc];
            }
        }
    };
    auto close_block = [&](int kb) {
        if constexpr (BLOCK) {
            const int64_t kb128 = kb >> 1;
            const bool n_ok = n0 + wn * WTN < N;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int64_t m = m0 + wm * WTM + i * 32 + l32;
                const float sc = (m < M && n_ok) ? sa_ring[0][i] * sw_ring[0] : 0.0f;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) facc[i][j][e] += acc[i][j][e] * sc;
                }
            }
#pragma unroll
            for (int r = 0; r + 1 < SCP; ++r) {
                sw_ring[r] = sw_ring[r + 1];
#pragma unroll
                for (int i = 0; i < TM; ++i) sa_ring[r][i] = sa_ring[r + 1][i];
            }
            load_scales(sa_ring[SCP - 1], sw_ring[SCP - 1], kb128 + SCP);
        }
    };

    // One step: stage kb's fragments were requested into `cur`; after they
    // land, the barrier (a) shows every wave holds its stage-kb fragments, so
    // the buffer of stage kb is free and receives stage kb+NB, and (b)
    // publishes stage kb+1, whose fragment reads are then spread between the
    // MFMAs of stage kb.
    constexpr int NREAD = NFRAG + (MX ? MXR * (TM + TN) : 0);
    constexpr int NMFMA = FP8 && !F4 ? TM * TN : 2 * TM * TN;
    constexpr int NSLOT = NMFMA - NMFMA / 4;
    // first: kb opens a 128-wide K block (even kb); with block scales its
    // MFMAs start from zero instead of the closed block's partial sums
    auto step = [&](FragsT& cur, FragsT& nxt, int kb, bool first) {
        settle_frags(cur);
        // this wave's copies of stage kb+1 landed: younger than them are at
        // least the copies of the NB-2 later stages (block-scale loads, which
        // the compiler may place anywhere, are not counted: a wait can only
        // end later for them)
        wait_vmcnt<(NB - 2) * LOADS_T>();
        block_barrier();
        const uint32_t nb_base = stage_base(kb + 1), nb_mx = mx_base(kb + 1);
        // MX: this stage's E8M0 bytes of the fragment rows for MFMA step c,
        // byte i of pka[c] / j of pkb[c] (the MFMA takes byte 0 of a constant
        // shift of them)
        uint32_t pka[MXR], pkb[MXR];
#pragma unroll
        for (int c = 0; c < MXR; ++c) {
            pka[c] = 0, pkb[c] = 0;
            if constexpr (MX) {
#pragma unroll
                for (int i = 0; i < TM; ++i) pka[c] |= cur.sa[i][c] << (8 * i);
#pragma unroll
                for (int j = 0; j < TN; ++j) pkb[c] |= cur.sb[j][c] << (8 * j);
            }
        }
        // reads of stage kb+1 follow the first NSLOT MFMAs (NREAD/NSLOT per MFMA,
        // every read exactly once), so the last quarter of the MFMAs covers
        // their latency; the copies of stage kb+NB are spread over all MFMAs
        // (a burst of them would hold up the first MFMA); scheduling barriers
        // keep the compiler from regrouping
        op_t pa = op_t{}, pb = op_t{};                           // operands of the previous MFMA
#pragma unroll
        for (int t = 0; t < NMFMA; ++t) {
            op_t av, bv;
            int i, j;
            if constexpr (F4) {
                const int half = t / (TM * TN);
                i = (t % (TM * TN)) / TN, j = t % TN;
                av = cur.a[i][half];
                bv = cur.b[j][half];
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    __builtin_shufflevector(bv, bv, 0, 1, 2, 3, -1, -1, -1, -1),
                    __builtin_shufflevector(av, av, 0, 1, 2, 3, -1, -1, -1, -1), acc[i][j], 4, 4, 0,
                    (int)(pkb[half] >> (8 * j)), 0, (int)(pka[half] >> (8 * i)));
            } else if constexpr (FP8) {
                i = t / TN, j = t % TN;
                av = __builtin_shufflevector(cur.a[i][0], cur.a[i][1], 0, 1, 2, 3, 4, 5, 6, 7);
                bv = __builtin_shufflevector(cur.b[j][0], cur.b[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
                if constexpr (MX)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bv, av, acc[i][j], 0, 0, 0, (int)(pkb[0] >> (8 * j)), 0, (int)(pka[0] >> (8 * i)));
                else
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bv, av, (BLOCK && first) ? acc_t{} : acc[i][j], 0, 0, 0, 0, 0, 0);
            } else {
                const int half = t / (TM * TN);
                i = (t % (TM * TN)) / TN, j = t % TN;
                av = cur.a[i][half];
                bv = cur.b[j][half];
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, av, acc[i][j], 0, 0, 0);
            }
            if (t == 0) pa = av, pb = bv;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = t < NSLOT ? t * NREAD / NSLOT : NREAD; r < (t < NSLOT ? (t + 1) * NREAD / NSLOT : NREAD); ++r)
                read_one_after(nxt, nb_base, nb_mx, r, av, bv, pa, pb);
#pragma unroll
            for (int l = (t * LOADS_T + NMFMA - 1) / NMFMA; l < ((t + 1) * LOADS_T + NMFMA - 1) / NMFMA; ++l)
                issue_one(kb + NB, l);
            pa = av, pb = bv;
            __builtin_amdgcn_sched_barrier(0);
        }
        if (BLOCK && (kb & 1)) close_block(kb);
    };

    // OL: the outlier count, and this thread's values of the first 8
    // outlier channels (the first copy batch of the side path), are requested
    // before the K loop, so their latency hides behind it.  A thread's copy
    // elements in a batch lie in one channel per wave (BM and BN are
    // multiples of 64), so the channel indices are wave-uniform scalar loads.
    constexpr int OL_NT = 128 * WN, OL_XPT = OL ? 8 * BM / OL_NT : 1, OL_WPT = OL ? 8 * BN / OL_NT : 1;
    [[maybe_unused]] int ol_cnt = 0;
    [[maybe_unused]] float ol_x0[OL_XPT], ol_w0[OL_WPT];
    auto ol_col = [&](int i) -> int64_t {
        const int64_t c = oidx[i];
        return c < 0 ? 0 : c >= K ? K - 1 : c;
    };
    auto ol_load = [&](int c0, int b, int ch, float (&xv)[OL_XPT], float (&wv)[OL_WPT]) {
#pragma unroll
        for (int u = 0; u < OL_XPT; ++u) {
            const int f = threadIdx.x + OL_NT * u, r = f % BM;
            const int t = __builtin_amdgcn_readfirstlane(b + f / BM);
            xv[u] = t < ch && m0 + r < M ? load1_f32(ox, ox_dt, (m0 + r) * K + ol_col(c0 + t)) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < OL_WPT; ++u) {
            const int f = threadIdx.x + OL_NT * u, c = f % BN;
            const int t = __builtin_amdgcn_readfirstlane(b + f / BN);
            wv[u] = t < ch && n0 + c < N ? (float)(int8_t)w[(n0 + c) * K + ol_col(c0 + t)] : 0.0f;
        }
    };
    if constexpr (OL) {
        const int64_t c_raw = *ocnt;
        ol_cnt = (int)(c_raw < 0 ? 0 : c_raw > K ? K : c_raw);
        ol_load(0, 0, ol_cnt < 64 ? ol_cnt : 64, ol_x0, ol_w0);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) issue(kb0 + t);
    if constexpr (BLOCK) {
        // ring for the first SCP blocks (not counted by the wait below)
#pragma unroll
        for (int r = 0; r < SCP; ++r) load_scales(sa_ring[r], sw_ring[r], kb0 / 2 + r);
    }
    wait_vmcnt<(NB - 1) * LOADS_T>();
    block_barrier();
    FragsT f0, f1;
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_one(f0, stage_base(kb0), mx_base(kb0), r);
    for (int kb = kb0; kb < kb1; kb += 2) {                      // slices hold whole 128-byte K blocks
        step(f0, f1, kb, true);
        step(f1, f0, kb + 1, false);
    }
    wait_vmcnt<0>();                                             // no copy may land after the block exits
    // the last step read the (unused) stage after the slice into f0: those
    // registers stay allocated until the reads have landed, or a value the
    // compiler put there (a close, the epilogue) would be overwritten
    settle_frags(f0);

    // ---- side path (OL) ----
    // acc becomes the float (acc * s_a[m]) in place, then gains
    // sum_k x[m][k] w[n][k] over the outlier columns on the BF16 matrix
    // cores: an INT8 weight code is exact in BF16, and each activation is
    // split into BF16 hi = RNE(x) and lo = RNE(x - hi), two MFMAs per K step
    // (exact for BF16 inputs, where lo = 0, and for FP16 inputs, whose 11
    // significant bits fit in hi and lo; an FP32 input keeps 16 of its 24,
    // the rest below 2^-16 of its magnitude).  The channels go in chunks of
    // CH: the block copies the chunk's values of its BM rows of x and BN rows
    // of w into the free stage buffers as BF16 rows (PX / PW bytes apart;
    // channels past the count up to a multiple of 16 are zero), 8 channels
    // per batch with all of a thread's loads in flight together; then each
    // tile (i, j) of the wave runs the chunk's K steps of v_mfma_f32_32x32x16
    // with the W rows as the first operand and its own (float) acc as the
    // accumulator.  The count and the indices are clamped to [0, K] and
    // [0, K) so a bad list never reads outside x or w.
    if constexpr (OL) {
        static_assert(!FP8 && !BLOCK && !MX, "the side path is an INT8 variant");
        constexpr int CH = 64, PX = 2 * CH * 2 + 16, PW = CH * 2 + 16;
        static_assert(BM * PX + BN * PW <= LDS_BYTES, "side-path chunk fits the stage buffers");
        uint8_t* xo = lds;                                        // [BM][PX]: hi plane, then lo plane
        uint8_t* wo = lds + BM * PX;                              // [BN][PW]
        const int cnt = ol_cnt;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = m0 + wm * WTM + i * 32 + l32;
            const float s_a = a_gran == GT ? as[0] : (m < M ? as[m] : 0.0f);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = __float_as_int((float)acc[i][j][e] * s_a);
        }
        constexpr int NT = OL_NT, XPT = OL_XPT, WPT = OL_WPT;
        static_assert(8 * BM % NT == 0 && 8 * BN % NT == 0 && BM % 64 == 0 && BN % 64 == 0, "whole batches per thread");
        for (int c0 = 0; c0 < cnt; c0 += CH) {
            const int ch = cnt - c0 < CH ? cnt - c0 : CH, ch16 = (ch + 15) & ~15;
            block_barrier();                                     // stage buffers / previous chunk free
            for (int b = 0; b < ch16; b += 8) {
                float xv[XPT], wv[WPT];
                if (c0 == 0 && b == 0) {
#pragma unroll
                    for (int u = 0; u < XPT; ++u) xv[u] = ol_x0[u];
#pragma unroll
                    for (int u = 0; u < WPT; ++u) wv[u] = ol_w0[u];
                } else {
                    ol_load(c0, b, ch, xv, wv);
                }
#pragma unroll
                for (int u = 0; u < XPT; ++u) {
                    const int f = threadIdx.x + NT * u, t = b + f / BM, r = f % BM;
                    const uint16_t hi = f32_to_bf16(xv[u]);
                    *reinterpret_cast<uint16_t*>(xo + r * PX + t * 2) = hi;
                    *reinterpret_cast<uint16_t*>(xo + r * PX + CH * 2 + t * 2) = f32_to_bf16(xv[u] - bf16_to_f32(hi));
                }
#pragma unroll
                for (int u = 0; u < WPT; ++u) {
                    const int f = threadIdx.x + NT * u, t = b + f / BN, c = f % BN;
                    *reinterpret_cast<uint16_t*>(wo + c * PW + t * 2) = f32_to_bf16(wv[u]);
                }
            }
            block_barrier();
            // (plain LDS loads: the compiler sees these register writes and
            // keeps them clear of the MFMAs still reading earlier operands)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float16_t c = __builtin_bit_cast(float16_t, acc[i][j]);
                    const uint8_t* xrow = xo + (wm * WTM + i * 32 + l32) * PX + h * 16;
                    const uint8_t* wrow = wo + (wn * WTN + j * 32 + l32) * PW + h * 16;
                    for (int ks = 0; ks < ch16; ks += 16) {
                        const bf168_t wb = __builtin_bit_cast(bf168_t, *reinterpret_cast<const int4_t*>(wrow + ks * 2));
                        const bf168_t xa = __builtin_bit_cast(bf168_t, *reinterpret_cast<const int4_t*>(xrow + ks * 2));
                        const bf168_t xl =
                            __builtin_bit_cast(bf168_t, *reinterpret_cast<const int4_t*>(xrow + CH * 2 + ks * 2));
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb, xa, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb, xl, c, 0, 0, 0);
                    }
                    acc[i][j] = __builtin_bit_cast(acc_t, c);
                }
        }
    }

    // ---- epilogue ----
    // The W fragment is the MFMA's first operand, so lane l, register e of
    // tile (i, j) holds output row m = 32i + l%32 and column
    // n = 32j + 8(e/4) + 4(l/32) + e%4: four consecutive columns per group.
    // Scales: one per row (TENSOR or ROW), four consecutive per column group.
    // 16-bit outputs are staged per wave in LDS (rows padded by 16 bytes) and
    // written back as 16-byte row segments; FP32 / INT32 go out directly as
    // 16-byte groups.
    // A K slice of a split GEMM (S > 1) writes its raw partial through the same
    // code to part[sl][M][N]: INT32 accumulators for INT8, FP32 for FP8 (block
    // scales already applied); k_w8a8_reduce adds the slices and scales them.
    block_barrier();                                             // all waves done with the stage buffers
    const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
    const bool split = S > 1;
    if (split) y = static_cast<uint8_t*>(part) + (int64_t)sl * M * N * 4;
    const int odt = split ? (FP8 ? O_F32 : O_I32) : out_dt;
    if (!FP8 && odt == O_I32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + i * 32 + l32;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int64_t n = nw + j * 32 + 8 * q4 + 4 * h;      // N % 16 == 0: all four or none
                    int4_t o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = (int)acc[i][j][4 * q4 + r];
                    if (m < M && n < N) *reinterpret_cast<int4_t*>(static_cast<int32_t*>(y) + m * N + n) = o;
                }
        }
        return;
    }
    // scales: sa per row; for each 32-column strip j, its 16 sw (four
    // consecutive per column group) are loaded together -- one wait per strip
    float sa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = mw + i * 32 + l32;
        sa[i] = BLOCK || MX || OL || split ? 1.0f : a_gran == GT ? as[0] : (m < M ? as[m] : 0.0f);
    }
    uint8_t* stage = lds + wave * WTM * EPI_PITCH;
    const bool bf = odt == O_BF16;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        float sw[4][4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int64_t n = nw + j * 32 + 8 * q4 + 4 * h;
            float4 w4 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            if (!BLOCK && !MX && !split) {
                if (w_gran == GT) w4 = make_float4(ws[0], ws[0], ws[0], ws[0]);
                else w4 = n < N ? *reinterpret_cast<const float4*>(ws + n) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            sw[q4][0] = w4.x, sw[q4][1] = w4.y, sw[q4][2] = w4.z, sw[q4][3] = w4.w;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = mw + i * 32 + l32;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int64_t n = nw + j * 32 + 8 * q4 + 4 * h;          // N % 16 == 0: all four or none
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (BLOCK) v[r] = facc[i][j][4 * q4 + r];
                    else if constexpr (OL) v[r] = __int_as_float(acc[i][j][4 * q4 + r]) * sw[q4][r];
                    else v[r] = ((float)acc[i][j][4 * q4 + r] * sa[i]) * sw[q4][r];
                }
                if (odt == O_F32) {
                    if (m < M && n < N)
                        *reinterpret_cast<float4*>(static_cast<float*>(y) + m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    uint2 packed;
                    packed.x = bf ? (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16)
                                  : (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
                    packed.y = bf ? (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)
                                  : (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
                    *reinterpret_cast<uint2*>(stage + (i * 32 + l32) * EPI_PITCH + (j * 32 + 8 * q4 + 4 * h) * 2) =
                        packed;
                }
            }
        }
    }
    if (odt == O_F32) return;
    // 16-bit outputs: this wave's tile was staged in LDS (rows padded by 16
    // bytes) and goes out as 16-byte row segments,
    // row by row: WTN * 2 bytes = WTN / 8 lanes per row
    constexpr int LPR = WTN / 8, RPI = 64 / LPR;                 // lanes per row, rows per instruction
    const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll 4
    for (int r0 = 0; r0 < WTM; r0 += RPI) {
        const int r = r0 + rr;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * EPI_PITCH + cc * 16);
        const int64_t m = mw + r, n = nw + cc * 8;
        if (m < M && n < N) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + m * N + n) = v;
    }
}

// Sum of the S partial slices of the split-K GEMM, in slice order, then the
// epilogue of the unsplit kernel: y = ((float)acc * s_a[m]) * s_w[n] (INT32
// sums are exact, so INT8 results equal the unsplit kernel's), or the sum
// itself for block-scaled FP8 (scales already applied) and raw INT32 output.
// One thread per four consecutive outputs of a row.
template <bool INT_PART>
__global__ __launch_bounds__(256) void k_w8a8_reduce(const void* __restrict__ part, int S, int64_t M, int64_t N,
                                                     const float* __restrict__ as, int a_gran,
                                                     const float* __restrict__ ws, int w_gran, bool scaled,
                                                     void* __restrict__ y, int out_dt) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= M * N) return;
    const int64_t m = e / N, n = e - m * N;
    constexpr int RB = 8;                                        // slices in flight per batch
    int4_t vi = int4_t{0, 0, 0, 0};
    float4 vf = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b0 = 0; b0 < S; b0 += RB) {
        int4_t pi[RB];
        float4 pf[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (b0 + r >= S) break;
            if constexpr (INT_PART) pi[r] = *reinterpret_cast<const int4_t*>(static_cast<const int32_t*>(part) + (b0 + r) * M * N + e);
            else pf[r] = *reinterpret_cast<const float4*>(static_cast<const float*>(part) + (b0 + r) * M * N + e);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (b0 + r >= S) break;
            if constexpr (INT_PART) vi += pi[r];
            else if (b0 + r == 0) vf = pf[r];
            else vf = make_float4(vf.x + pf[r].x, vf.y + pf[r].y, vf.z + pf[r].z, vf.w + pf[r].w);
        }
    }
    if (INT_PART && out_dt == O_I32) {
        *reinterpret_cast<int4_t*>(static_cast<int32_t*>(y) + e) = vi;
        return;
    }
    float v[4];
    if constexpr (INT_PART) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (float)vi[r];
    } else {
        v[0] = vf.x, v[1] = vf.y, v[2] = vf.z, v[3] = vf.w;
    }
    if (scaled) {
        const float sa = a_gran == GT ? as[0] : as[m];
        const float4 sw4 = w_gran == GT ? make_float4(ws[0], ws[0], ws[0], ws[0])
                                        : *reinterpret_cast<const float4*>(ws + n);
        v[0] = (v[0] * sa) * sw4.x, v[1] = (v[1] * sa) * sw4.y, v[2] = (v[2] * sa) * sw4.z, v[3] = (v[3] * sa) * sw4.w;
    }
    if (out_dt == O_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + e) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        const bool bf = out_dt == O_BF16;
        uint2 o;
        o.x = bf ? (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16)
                 : (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
        o.y = bf ? (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)
                 : (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + e) = o;
    }
}

template <bool FP8, bool BLOCK, int BM, int BN, int WN, int MX = 0, bool OL = false>
static const char* gemm_cfg(const W8A8Args& g, const W8Split& c, void* ws, hipStream_t s) {
    const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_w8a8_gemm<FP8, BLOCK, BM, BN, WN, MX, OL>), dim3((unsigned)(tiles * c.S)), dim3(128 * WN), 0,
                       s, static_cast<const uint8_t*>(g.a), g.a_scales, g.a_gran, static_cast<const uint8_t*>(g.w),
                       g.w_scales, g.w_gran, g.M, g.N, g.K, g.y, g.out_dt, ws, c.S, c.spl, g.ox, g.ox_dt, g.oidx,
                       g.ocnt);
    if (c.S > 1) {
        const int64_t threads = g.M * g.N / 4;
        const bool scaled = !BLOCK && g.out_dt != O_I32;
        hipLaunchKernelGGL((k_w8a8_reduce<!FP8>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           static_cast<const void*>(ws), c.S, g.M, g.N, g.a_scales, g.a_gran, g.w_scales, g.w_gran,
                           scaled, g.y, g.out_dt);
    }
    return OL ? kname("k_w8a8_gemm", FP8, BLOCK, BM, BN, WN, MX, OL) : kname("k_w8a8_gemm", FP8, BLOCK, BM, BN, WN, MX);
}

// Tile choice for the large-M GEMM: estimated time = rounds of resident
// blocks x time of one round.  Relative round times (K fixed) measured on the
// 4096..28672-wide projection shapes: 256 x 256 (one block per CU) 75,
// 256 x 128 (one per CU) 46.4 (256 x 256 now runs 8 waves, two per SIMD,
// about 8 % faster than those rounds: no decision on these shapes changes); block-scaled FP8, which keeps two accumulator
// sets, uses 128 x 128 (two per CU).  With a workspace, grids of at most
// half a round split K (S = min(blocks per round / tiles, 128-byte K blocks /
// 8) slices of whole 128-byte blocks); M <= 128 then uses 128 x 128 tiles
// (two blocks per CU) rather than half-empty 256-row ones.
W8Split w8a8_tiled_split(const W8A8Args& g, bool with_ws) {
    W8Split c{};
    c.S = 1;
    const bool block = g.in_fp8 && g.a_gran == GR128;
    const bool mx = g.a_gran == GMX32 || g.a_gran == GMX4;
    c.spl = (int)((g.a_gran == GMX4 ? g.K / 2 : g.K) / GK);
    auto tiles = [&](int64_t bm, int64_t bn) { return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn); };
    auto cost = [&](int64_t bm, int64_t bn, double round) { return (double)((tiles(bm, bn) + 255) / 256) * round; };
    if (block) c.bm = 128, c.bn = 128;
    else if (cost(256, 256, 75.0) <= cost(256, 128, 46.4)) c.bm = 256, c.bn = 256;
    else c.bm = 256, c.bn = 128;
    // MX: the same tiles, 128 x 128 for M <= 128; no K split
    if (mx && g.M <= 128) c.bm = 128, c.bn = 128;
    if (mx || !with_ws || tiles(c.bm, c.bn) > 128) return c;    // over half a round: no split
    const int64_t nk128 = g.K >> 7;
    const bool small_m = g.M <= 128;
    const int64_t bm = small_m ? 128 : c.bm, bn = small_m ? 128 : c.bn;
    const int64_t per_round = bm == 128 ? 512 : 256;             // resident blocks per round
    const int64_t t = tiles(bm, bn);
    int64_t S = per_round / t;
    if (S > nk128 / 8) S = nk128 / 8;
    if (S < 2) return c;
    const int64_t per = (nk128 + S - 1) / S;                     // 128-byte K blocks per slice
    S = (nk128 + per - 1) / per;
    if (S < 2) return c;
    c.bm = (int)bm, c.bn = (int)bn;
    c.S = (int)S;
    c.spl = (int)(2 * per);
    c.ws_bytes = S * g.M * g.N * 4;
    return c;
}

template <bool FP8, bool BLOCK, int MX = 0, bool OL = false>
static const char* gemm_shape(const W8A8Args& g, const W8Split& c, void* ws, hipStream_t s) {
    if (c.bm == 128) return gemm_cfg<FP8, BLOCK, 128, 128, 2, MX, OL>(g, c, ws, s);
    if constexpr (!BLOCK) {
        if (c.bn == 256) return gemm_cfg<FP8, false, 256, 256, 4, MX, OL>(g, c, ws, s);
        return gemm_cfg<FP8, false, 256, 128, 2, MX, OL>(g, c, ws, s);
    }
    return nullptr;
}

const char* launch_w8a8_tiled(const W8A8Args& g, void* ws, hipStream_t s) {
    if (g.oidx) return gemm_shape<false, false, 0, true>(g, w8a8_tiled_split(g, false), nullptr, s);
    const W8Split c = w8a8_tiled_split(g, ws != nullptr);
    if (g.a_gran == GMX32) return gemm_shape<true, false, MX_F8>(g, c, nullptr, s);
    if (g.a_gran == GMX4) return gemm_shape<true, false, MX_F4>(g, c, nullptr, s);
    if (g.in_fp8 && g.a_gran == GR128) return gemm_shape<true, true>(g, c, ws, s);
    if (g.in_fp8) return gemm_shape<true, false>(g, c, ws, s);
    return gemm_shape<false, false>(g, c, ws, s);
}


}  // namespace bg
