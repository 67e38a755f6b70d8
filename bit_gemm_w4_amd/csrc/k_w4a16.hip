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
// Packed word j holds k = 8j..8j+7 with even k in the low half-word and odd k
// in the high half-word, so (w >> 4p) & 0x000F000F | magic is the pair
// (MV + u[8j+2p], MV + u[8j+2p+1]) -- consecutive k, matching activations in
// their natural order: no permutation is needed on either operand.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_w4.h"

namespace bg {

// ============================================================================
// Small-M kernel (decode).  A block owns 16*TN output columns (TN weight tiles)
// and a band of activation rows for the WHOLE of K; its NW waves split the
// 128-wide groups of K between them and their partial results are summed
// through LDS at the end.  This gives thousands of waves even for N = 4096
// (enough loads in flight to cover HBM latency) without any cross-block
// reduction or scratch memory.  Groups are dealt to the waves round-robin, so
// the block sweeps its tiles front to back as one contiguous stream.
//
// Lane l (l16 = l % 16, q = l / 16) consumes, per group, slot l of each 1 KB
// weight tile -- words 4q..4q+3 of the group row of column l16, i.e.
// k = 32q .. 32q+31 -- so a wave reads a tile with one contiguous load.
//
// Two inner products share everything else:
//  * MFMA (VROWS == 0), rows m0 .. m0+16*TM: v_mfma_f32_16x16x32_{bf16,f16};
//    in K step kk the lane supplies word 4q+kk and activations k = 32q+8kk..+7
//    of row l16 (same k assignment for both operands).  One extra MFMA per
//    m-tile against an all-ones operand yields Sx_g directly in the output
//    layout (lane l, register e -> row 4(l/16)+e, column l%16).
//  * VALU (VROWS = 1, 2 or 4 rows): v_dot2_f32_{bf16,f16} of the lane's 32 k
//    against each row; Sx_g comes from a per-block table built in LDS.
//
// Software pipeline: the loads of one group form a stage; STAGES stages are
// in flight in registers and the loads of group g + STAGES are issued right
// after group g is consumed.  The vector-memory counter retires loads in issue
// order, so consuming group g waits only for g's own loads.
//
// Group scales and zero-points: each wave copies those of its own groups
// (32 bytes of scales and the 16 zero-point bytes per tile and group) into a
// wave-private LDS area with a few 16-byte loads before its first weight
// stage, so the stream of global loads is the 1 KB weight tiles alone (a
// tiny scattered scale and zero-point request per tile and group measured
// about 7 % of the call on the widest layer).  No block barrier waits for
// these copies: a wave reads only what its own lanes wrote, and the in-order
// memory counter has released them before the wave's first weight stage.
//
// XLDS: the block first copies its activation rows (all of K) into LDS and the
// activation operand is read from there (ds_read, a separate counter), so a
// stage holds only the 16 bytes of weights per tile and lane and the
// pipeline runs deep.  Without XLDS the activation fragments travel in the
// stage registers and the pipeline is shallower.  Rows >= M only ever feed
// output rows >= M (MFMA row i reads only operand row i), so lanes for such
// rows read row M-1 instead of zero-filling.
template <int TM, int TN, bool XLDS>
struct DecStage {
    uint4 w[TN];
    uint4 a[XLDS ? 1 : TM][XLDS ? 1 : 4];
};

template <bool BF16, int TM, int TN, int NW, bool XLDS, int VROWS>
__global__ __launch_bounds__(NW * 64) void k_w4a16_decode(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ sc,
                                                          const uint8_t* __restrict__ zr, int64_t N,
                                                          uint16_t* __restrict__ y, uint64_t rcp) {
    constexpr bool VALU = VROWS > 0;
    static_assert(!VALU || (XLDS && TM == 1), "the VALU product reads activations from LDS");
    // groups in flight per wave, chosen so that a CU keeps roughly 24-64 KB of
    // weights in flight: more requests than that compete at the memory side
    // (gate_up with two groups per wave of its four- and seven-tile blocks is
    // 0.3-0.6 us slower per call than with one, qkv at B = 16 0.3 us slower
    // with four groups of its two-tile blocks than with two); fewer leave
    // HBM idle (qkv and down at B = 1, with 4-8 one-tile waves per CU: 0.4-
    // 1 us slower with two groups than with three).  One-tile blocks of 16
    // waves: two.  (The VALU product keeps 3 / 4 groups for one / two tiles.)
    constexpr int STAGES = VALU   ? (TN == 1 ? 3 : 4)
                           : XLDS ? (TN == 1 ? (NW == 16 ? 2 : 3) : TN == 2 ? 2 : 1)
                                  : 3;
    // X staging batch: 16 chunks per thread for blocks of seven or more
    // tiles (the 16-row, one-round configuration: all of a block's rows in
    // one batch, issued before the weight stages; gate_up at B = 16 19.4 ->
    // 18.9 us), else 8 (16 costs the small layers registers)
    constexpr int XB = TN >= 7 ? 16 : 8;
    constexpr int BAND = VALU ? VROWS : 16 * TM;                       // activation rows per block
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    constexpr int TILE_FLOATS = VALU ? TN * VROWS * 64 : TM * TN * 4 * 64;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    float* red = reinterpret_cast<float*>(dyn_lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t ntiles = N >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * TN;
    const int64_t m0 = (int64_t)blockIdx.y * BAND;
    const int ngroups = (int)(K >> 7);
    // wave w takes groups w, w + NW, w + 2 NW, ...: at any moment the waves of
    // a block read neighbouring 1 KB tiles, i.e. one contiguous stretch of HBM
    const int n_mine = ngroups > wave ? (ngroups - wave + NW - 1) / NW : 0;
    const int64_t rows = (M - m0) < BAND ? (M - m0) : BAND;           // real rows of this block
    const int64_t xstride = K + 8;                                    // LDS row pitch in halves
    const int64_t x_bytes = XLDS ? rows * xstride * 2 : 0;
    // LDS: [per wave: its groups' scales and zero bytes][X rows][VALU: Sx table]
    // A (group i of the wave, tile j) record is 48 bytes: 16 FP16 scales, then
    // the 16 zero-point bytes of the group pair.
    const bool has_z = zr != nullptr;
    const int nmax = (ngroups + NW - 1) / NW;                         // most groups of any wave
    uint8_t* wsz = dyn_lds + wave * nmax * TN * 48;                   // this wave's records
    uint8_t* x_l = dyn_lds + NW * nmax * TN * 48;
    float* sxt = reinterpret_cast<float*>(x_l + x_bytes);             // VALU: Sx[row][group]

    // Buffer descriptors over this block's tiles: per-lane offsets live in
    // VGPRs, the group offset is wave-uniform (scalar unit), and reads past the
    // last tile of N (or of a missing zero-point tensor) return 0.
    const int64_t my_tiles = (ntiles - t0) < TN ? (ntiles - t0) : TN;
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + t0 * ngroups * 256), (short)0,
                                                      (int)(my_tiles * ngroups * 1024), 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + t0 * ngroups * 16), (short)0,
                                                      (int)(my_tiles * ngroups * 32), 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(has_z ? zr + t0 * (ngroups >> 1) * 16 : zr),
                                                      (short)0, has_z ? (int)(my_tiles * (ngroups >> 1) * 16) : 0,
                                                      0x00020000);
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + m0 * K), (short)0,
                                                      (int)(rows * K * 2), 0x00020000);
    int arow[VALU ? 1 : TM];                  // MFMA: activation row each lane feeds (clamped)
    if constexpr (!VALU) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = 16 * i + l16;
            arow[i] = r < rows ? r : (int)rows - 1;
        }
    }
    const uint32_t ones[4] = {ONE2, ONE2, ONE2, ONE2};

    // Every stage issues the same loads, so the compiler can wait for exactly
    // one stage.  Past the wave's last group the loads address beyond the
    // buffer's range (kBufOOB): they return zeros without a memory access.
    auto issue = [&](DecStage<TM, TN, XLDS>& st, int i) {
        const bool real = i < n_mine;
        const int g = i * NW + wave;
#pragma unroll
        for (int j = 0; j < TN; ++j)
            st.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rw, lane * 16, real ? (j * ngroups + g) * 1024 : kBufOOB, 0));
        if constexpr (!XLDS) {
#pragma unroll
            for (int ii = 0; ii < TM; ++ii)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    st.a[ii][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rx, (int)(arow[ii] * K * 2) + q * 64 + kk * 16,
                                                                 real ? g * 256 : kBufOOB, 0));
        }
    };

    // This wave's scale and zero records: 16 records per pass of 64 lanes,
    // lane = 4 * record + part (parts 0 and 1: the two 16-byte halves of the
    // scales; part 2: the zero bytes; part 3 idle).
    const int nrec = n_mine * TN;
    auto sz_issue = [&](int r0, uint4& v) {
        const int rec = r0 + (lane >> 2), part = lane & 3;
        const int i = rec / TN, j = rec - i * TN;
        const int g = i * NW + wave;
        if (rec < nrec && part < 2)
            v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (j * ngroups + g) * 32 + part * 16,
                                                                                 0, 0));
        else if (rec < nrec && part == 2 && has_z)
            v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rz, (j * (ngroups >> 1) + (g >> 1)) * 16, 0, 0));
    };
    auto sz_store = [&](int r0, const uint4& v) {
        const int rec = r0 + (lane >> 2), part = lane & 3;
        if (rec < nrec && part < 3) *reinterpret_cast<uint4*>(wsz + rec * 48 + part * 16) = v;
    };
    // blocks of four or more tiles request their first two passes of records
    // (32) before anything else, so that no later wait for them also waits
    // for the weight stages (gate_up at B = 16: 18.8 -> 17.4 us); narrower
    // blocks, with at most 16 records per wave on these shapes, keep one pass
    // (all four passes of the seven-tile blocks early: no further gain)
    constexpr int SZ_EARLY = TN >= 4 ? 32 : 16;
    uint4 szv[SZ_EARLY / 16];
#pragma unroll
    for (int p = 0; p < SZ_EARLY / 16; ++p) {
        szv[p] = uint4{0, 0, 0, 0};
        sz_issue(16 * p, szv[p]);
    }

    // XLDS: rows [m0, m0 + rows) of X are copied into LDS in 16-byte chunks,
    // XB per thread in flight together (one memory round trip per batch).  The
    // first batch is requested before the weight stages, so that the
    // in-order memory counter releases it first.  Chunk c is row c / cpr,
    // found by a multiply with rcp = ceil(2^40 / cpr) (computed on the host):
    // exact for c < 2^21 and cpr <= 2^17, which K <= 2^20 and at most 16
    // rows guarantee.
    const int cpr = (int)(K >> 3);                                     // chunks per row
    const int total = XLDS ? (int)rows * cpr : 0;
    auto x_load = [&](uint4 (&v)[XB], int c0) {
#pragma unroll
        for (int u = 0; u < XB; ++u)
            if (c0 + u * NW * 64 < total)
                v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (c0 + u * NW * 64) * 16,
                                                                                       0, 0));
    };
    auto x_store = [&](const uint4 (&v)[XB], int c0) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = c0 + u * NW * 64;
            if (c < total) {
                const int r = (int)(((uint64_t)c * rcp) >> 40), kc = c - r * cpr;
                *reinterpret_cast<uint4*>(x_l + ((int64_t)r * xstride + kc * 8) * 2) = v[u];
            }
        }
    };
    uint4 xv0[XB];
    if constexpr (XLDS) x_load(xv0, threadIdx.x);

    DecStage<TM, TN, XLDS> stage[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue(stage[s], s);

    // X first (it is shared by the block, and usually cache-resident), then
    // this wave's own records: only the block barrier waits for the X copy,
    // and each wave waits for its scale load alone, which the memory counter
    // returns before the wave's first weight stage
    if constexpr (XLDS) {
        x_store(xv0, threadIdx.x);
        for (int c0 = threadIdx.x + XB * NW * 64; c0 < total; c0 += XB * NW * 64) {
            uint4 v[XB];
            x_load(v, c0);
            x_store(v, c0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < SZ_EARLY / 16; ++p) sz_store(16 * p, szv[p]);
    for (int r0 = SZ_EARLY; r0 < nrec; r0 += 16) {
        uint4 v = uint4{0, 0, 0, 0};
        sz_issue(r0, v);
        sz_store(r0, v);
    }
    if constexpr (VALU) {
        // Sx[row][g]: sum of the 128 activations of each group
        for (int64_t e = threadIdx.x; e < rows * ngroups; e += NW * 64) {
            const int64_t r = e / ngroups, g = e - r * ngroups;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(x_l + (r * xstride + g * 128) * 2);
            float sum = 0.0f;
            for (int k2 = 0; k2 < 64; ++k2) sum = dot2<BF16>(p[k2], ONE2, sum);
            sxt[e] = sum;
        }
        __syncthreads();
    }

    float4_t acc[VALU ? 1 : TM][TN];
    float vacc[TN][VALU ? VROWS : 1];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int i = 0; i < (VALU ? 1 : TM); ++i) acc[i][j] = float4_t{0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < (VALU ? VROWS : 1); ++b) vacc[j][b] = 0.0f;
    }

    auto consume = [&](const DecStage<TM, TN, XLDS>& st, int i) {
        const int g = i * NW + wave;
        float scale[TN], corr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint8_t* rec = wsz + (i * TN + j) * 48;
            scale[j] = f16_to_f32(*reinterpret_cast<const uint16_t*>(rec + l16 * 2));
            corr[j] = MV + (float)(has_z ? (rec[32 + l16] >> (4 * (g & 1))) & 0xF : 8u);
        }
        if constexpr (VALU) {
            uint32_t D[TN][4][4];
#pragma unroll
            for (int j = 0; j < TN; ++j) dequant_tile<BF16>(st.w[j], D[j]);
#pragma unroll
            for (int b = 0; b < VROWS; ++b) {
                if (b >= rows) break;
                const uint8_t* xr = x_l + (b * xstride + (int64_t)g * 128 + q * 32) * 2;
                uint4 xv[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) xv[kk] = *reinterpret_cast<const uint4*>(xr + kk * 16);
                // only quarter 0 subtracts the whole group's correction
                const float sx = q == 0 ? sxt[b * ngroups + g] : 0.0f;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float d = 0.0f;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        d = dot2<BF16>(D[j][kk][0], xv[kk].x, d);
                        d = dot2<BF16>(D[j][kk][1], xv[kk].y, d);
                        d = dot2<BF16>(D[j][kk][2], xv[kk].z, d);
                        d = dot2<BF16>(D[j][kk][3], xv[kk].w, d);
                    }
                    vacc[j][b] += scale[j] * (d - corr[j] * sx);
                }
            }
        } else {
            float4_t part[TM][TN], sx[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                sx[i] = float4_t{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < TN; ++j) part[i][j] = float4_t{0, 0, 0, 0};
            }
            // one word pair (two K steps) of every tile at a time: 8 registers
            // of dequantized operands per tile in flight
            uint32_t D[TN][2][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if ((kk & 1) == 0) {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        dequant_pair<BF16>(kk == 0 ? st.w[j].x : st.w[j].z, kk == 0 ? st.w[j].y : st.w[j].w, D[j][0],
                                           D[j][1]);
                }
                uint32_t bfrag[TN][4];
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bfrag[j][r] = D[j][kk & 1][r];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    uint4 av;
                    if constexpr (XLDS)
                        av = *reinterpret_cast<const uint4*>(x_l +
                                                             (arow[i] * xstride + (int64_t)g * 128 + q * 32 + kk * 8) * 2);
                    else
                        av = st.a[i][kk];
                    const uint32_t a[4] = {av.x, av.y, av.z, av.w};
                    sx[i] = mfma16<BF16>(a, ones, sx[i]);
#pragma unroll
                    for (int j = 0; j < TN; ++j) part[i][j] = mfma16<BF16>(a, bfrag[j], part[i][j]);
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] += scale[j] * (part[i][j][e] - corr[j] * sx[i][e]);
        }
    };

    for (int i = 0; i < n_mine; i += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
            if (i + s < n_mine) consume(stage[s], i + s);
            issue(stage[s], i + s + STAGES);
        }
    }

    // ---- sum the NW partial tiles through LDS (reusing the staging space) ----
    __syncthreads();
    if constexpr (VALU) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int b = 0; b < VROWS; ++b) red[wave * TILE_FLOATS + (j * VROWS + b) * 64 + lane] = vacc[j][b];
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    red[wave * TILE_FLOATS + ((i * TN + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if constexpr (VALU) {
        // output (j, b, column l16): sum over waves and the 4 lane quarters
        for (int t = threadIdx.x; t < TN * VROWS * 16; t += NW * 64) {
            const int c16 = t & 15, jb = t >> 4;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) v += red[w * TILE_FLOATS + jb * 64 + qq * 16 + c16];
            const int j = jb / VROWS, b = jb % VROWS;
            const int64_t m = m0 + b;
            const int64_t n = (t0 + j) * 16 + c16;
            if (m < M && n < N) y[m * N + n] = to_out<BF16>(v);
        }
    } else {
        for (int t = threadIdx.x; t < TILE_FLOATS; t += NW * 64) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[w * TILE_FLOATS + t];
            const int ln = t & 63, e = (t >> 6) & 3, ij = t >> 8;
            const int i = ij / TN, j = ij % TN;
            const int64_t m = m0 + 16 * i + 4 * (ln >> 4) + e;
            const int64_t n = (t0 + j) * 16 + (ln & 15);
            if (m < M && n < N) y[m * N + n] = to_out<BF16>(v);
        }
    }
}

// ============================================================================
// Split-K small-M kernel (M <= 64), for callers that provide a workspace.
//
// Grid (column groups of SPK_NW weight tiles) x (S slices of K).  A block
// stages only its K-slice of the activation rows in LDS -- once, shared by
// its 16 waves -- and every wave streams the slice of ONE weight tile, so the
// activation bytes each CU reads are amortised over 16 tiles (at M = 16 the
// activations of a group are 4x the bytes of one weight tile).  With S = 1 the
// block writes the output; otherwise it writes its FP32 partial tile (rows
// < M only) to the workspace and k_w4a16_splitk_reduce, launched next on the
// same stream, adds the S partials in slice order -- a fixed order, so
// results do not depend on timing.  Stream order makes the partials visible
// to the second kernel; an in-kernel handoff would need a device-scope
// release/acquire per block, which on a multi-L2 device writes back and
// invalidates whole caches and measured slower than the second launch.
//
// Inner product as in the MFMA variant of k_w4a16_decode; Sx_g comes from a
// table the block builds next to the staged activations.
// ============================================================================
constexpr int SPK_NW = 16;
// two groups in flight per wave (16 waves, about one block per CU): down at
// B = 16 12.37 us against 12.71 with four and 12.78 with three
constexpr int SPK_STAGES = 2;

struct SpkStage {
    uint4 w;
    uint32_t s;
    uint32_t z;
};

template <bool BF16, int TM>
__global__ __launch_bounds__(SPK_NW * 64) void k_w4a16_splitk(const uint16_t* __restrict__ x, int64_t M,
                                                              int64_t K, const uint32_t* __restrict__ qw,
                                                              const uint16_t* __restrict__ sc,
                                                              const uint8_t* __restrict__ zr, int64_t N,
                                                              uint16_t* __restrict__ y, float* __restrict__ ws,
                                                              int S, int gs) {
    constexpr int NW = SPK_NW, STAGES = SPK_STAGES, BAND = 16 * TM;
    constexpr float MV = W4Magic<BF16>::value;
    constexpr uint32_t ONE2 = W4Magic<BF16>::ones;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int ntiles = (int)(N >> 4);
    const int ngroups = (int)(K >> 7);
    const int cg = blockIdx.x, sl = blockIdx.y;
    const int g0 = sl * gs;
    const int ng = (ngroups - g0) < gs ? (ngroups - g0) : gs;        // >= 1 by construction of S
    const int tile = cg * NW + wave;
    const bool tok = tile < ntiles;
    const int tt = tok ? tile : 0;
    const int rows = M < BAND ? (int)M : BAND;
    const int xpitch = ng * 128 + 8;                                   // halves per staged row
    uint16_t* xl = reinterpret_cast<uint16_t*>(dyn_lds);
    float* sxt = reinterpret_cast<float*>(dyn_lds + rows * xpitch * 2);   // Sx[group][row]

    const int zb0 = g0 >> 1;
    const int zb1 = (g0 + ng - 1) >> 1;
    const bool has_z = zr != nullptr;
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + ((int64_t)tt * ngroups + g0) * 256),
                                                      (short)0, tok ? ng * 1024 : 0, 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + ((int64_t)tt * ngroups + g0) * 16),
                                                      (short)0, tok ? ng * 32 : 0, 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(has_z ? zr + ((int64_t)tt * (ngroups >> 1) + zb0) * 16 : zr), (short)0,
        (tok && has_z) ? (zb1 - zb0 + 1) * 16 : 0, 0x00020000);
    // X from the slice's first column; the last valid byte is the end of row rows-1
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (int64_t)g0 * 128), (short)0,
                                                      (int)(((int64_t)(rows - 1) * K + ng * 128) * 2), 0x00020000);

    auto issue = [&](SpkStage& st, int i) {
        const bool real = i < ng;                     // else: out of range, zeros, no memory access
        st.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16, real ? i * 1024 : kBufOOB, 0));
        st.s = __builtin_amdgcn_raw_buffer_load_b16(rs, l16 * 2, real ? i * 32 : kBufOOB, 0);
        st.z = __builtin_amdgcn_raw_buffer_load_b8(rz, l16, real ? (((g0 + i) >> 1) - zb0) * 16 : kBufOOB, 0);
    };
    SpkStage stage[STAGES];
#pragma unroll
    for (int st = 0; st < STAGES; ++st) issue(stage[st], st);

    // stage X[0:rows, slice] (16-byte chunks, XB per thread in flight
    // together), then the per-group row sums
    constexpr int XB = 4;
    const int cpr = ng * 16;                                            // chunks per row
    const int total = rows * cpr;
    for (int c0 = threadIdx.x; c0 < total; c0 += XB * NW * 64) {
        uint4 v[XB];
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = c0 + u * NW * 64;
            const int r = c / cpr, kc = c - r * cpr;
            if (c < total)
                v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rx, (int)(r * (int)K * 2) + kc * 16, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = c0 + u * NW * 64;
            if (c < total) {
                const int r = c / cpr, kc = c - r * cpr;
                *reinterpret_cast<uint4*>(xl + r * xpitch + kc * 8) = v[u];
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ng * BAND; e += NW * 64) {
        const int gl = e / BAND, r0 = e - gl * BAND;
        const int r = r0 < rows ? r0 : rows - 1;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(xl + r * xpitch + gl * 128);
        float sum = 0.0f;
        for (int k2 = 0; k2 < 64; ++k2) sum = dot2<BF16>(p[k2], ONE2, sum);
        sxt[e] = sum;
    }
    __syncthreads();

    int arow[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = 16 * i + l16;
        arow[i] = r < rows ? r : rows - 1;
    }
    float4_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = float4_t{0, 0, 0, 0};

    auto consume = [&](const SpkStage& st, int gl) {
        const float scale = f16_to_f32(st.s & 0xFFFFu);
        const float corr = MV + (float)(has_z ? (st.z >> (4 * ((g0 + gl) & 1))) & 0xF : 8u);
        float4_t part[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) part[i] = float4_t{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint32_t b[4];
            dequant_word<BF16>(kk == 0 ? st.w.x : kk == 1 ? st.w.y : kk == 2 ? st.w.z : st.w.w, b);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint4 av = *reinterpret_cast<const uint4*>(xl + arow[i] * xpitch + gl * 128 + q * 32 + kk * 8);
                const uint32_t a[4] = {av.x, av.y, av.z, av.w};
                part[i] = mfma16<BF16>(a, b, part[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const float4 sx = *reinterpret_cast<const float4*>(sxt + gl * BAND + 16 * i + 4 * q);
            acc[i][0] += scale * (part[i][0] - corr * sx.x);
            acc[i][1] += scale * (part[i][1] - corr * sx.y);
            acc[i][2] += scale * (part[i][2] - corr * sx.z);
            acc[i][3] += scale * (part[i][3] - corr * sx.w);
        }
    };
    for (int i = 0; i < ng; i += STAGES) {
#pragma unroll
        for (int st = 0; st < STAGES; ++st) {
            if (i + st < ng) consume(stage[st], i + st);
            issue(stage[st], i + st + STAGES);
        }
    }

    auto store_y = [&](int i, const float4_t& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = 16 * i + 4 * q + e;
            const int64_t n = (int64_t)tile * 16 + l16;
            if (tok && m < M) y[m * N + n] = to_out<BF16>(v[e]);
        }
    };
    if (S == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i) store_y(i, acc[i]);
        return;
    }
    // ---- partial tile -> workspace (summed by k_w4a16_splitk_reduce) ----
    const int64_t tiles_pad = (int64_t)gridDim.x * NW;
#pragma unroll
    for (int i = 0; i < TM; ++i)
        if (16 * i + 4 * q < M)
            *reinterpret_cast<float4_t*>(ws + (((int64_t)sl * tiles_pad + tile) * TM + i) * 256 + lane * 4) = acc[i];
}

// Sum of the S partial tiles of the split-K kernel, in slice order.  One
// thread per output value -- (tile, 16-row band, lane, row e of the lane's
// four), i.e. one float of a slice's partial tile -- so the grid has as many
// threads as a slice has floats and spreads its loads over the device.
template <bool BF16, int TM>
__global__ __launch_bounds__(256) void k_w4a16_splitk_reduce(const float* __restrict__ ws, int S, int64_t tiles_pad,
                                                             int64_t M, int64_t N, uint16_t* __restrict__ y) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;     // float index within a slice
    const int lane = (int)((t >> 2) & 63), e = (int)(t & 3);
    const int64_t ti = t >> 8;
    const int i = (int)(ti % TM);
    const int64_t tile = ti / TM;
    const int q = lane >> 4, l16 = lane & 15;
    const int64_t m = 16 * i + 4 * q + e;
    if (tile * 16 >= N || m >= M) return;
    const int64_t slice = tiles_pad * TM * 256;
    const float* p = ws + t;
    // all loads of a batch of up to 16 slices are in flight together; the sum
    // still runs in slice order
    constexpr int RB = 16;
    float v = 0.0f;
    for (int b0 = 0; b0 < S; b0 += RB) {
        float part[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) part[r] = b0 + r < S ? p[(b0 + r) * slice] : 0.0f;
#pragma unroll
        for (int r = 0; r < RB; ++r)
            if (b0 + r < S) v = b0 + r == 0 ? part[r] : v + part[r];
    }
    y[m * N + tile * 16 + l16] = to_out<BF16>(v);
}

constexpr int64_t kLdsMax = 160 * 1024;

template <typename Kern>
static void allow_lds(Kern kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)bytes);
}

// LDS bytes of the decode kernel: the block's scales and zero bytes, then the
// staged activation rows (+ Sx table for the VALU product), or the
// cross-wave reduction buffer, whichever is larger.
static int64_t decode_scale_lds(int TN, int NW, int64_t K) {
    return (int64_t)NW * (((K >> 7) + NW - 1) / NW) * TN * 48;
}
static int64_t decode_lds(int tile_floats, int NW, int TN, bool xlds, bool valu, int64_t rows, int64_t K) {
    const int64_t red = (int64_t)NW * tile_floats * 4;
    const int64_t xb = decode_scale_lds(TN, NW, K) +
                       (xlds ? rows * (K + 8) * 2 + (valu ? rows * (K >> 7) * 4 : 0) : 0);
    return red > xb ? red : xb;
}

template <bool BF16, int TM, int TN, int NW, bool XLDS, int VROWS>
static const char* decode_cfg(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                              const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    constexpr int BAND = VROWS > 0 ? VROWS : 16 * TM;
    constexpr int TILE_FLOATS = VROWS > 0 ? TN * VROWS * 64 : TM * TN * 4 * 64;
    dim3 grid((unsigned)(((N >> 4) + TN - 1) / TN), (unsigned)((M + BAND - 1) / BAND));
    const int64_t rows = M < BAND ? M : BAND;
    const size_t lds = (size_t)decode_lds(TILE_FLOATS, NW, TN, XLDS, VROWS > 0, rows, K);
    auto kern = k_w4a16_decode<BF16, TM, TN, NW, XLDS, VROWS>;
    allow_lds(kern, lds);
    const uint64_t cpr = (uint64_t)(K >> 3);
    const uint64_t rcp = ((uint64_t(1) << 40) + cpr - 1) / cpr;
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N,
                       static_cast<uint16_t*>(y), rcp);
    return kname("k_w4a16_decode", BF16, TM, TN, NW, XLDS, VROWS);
}

// Waves per block: enough blocks x waves to keep ~16 waves per CU resident
// (at least 4), never more waves than K has groups -- ~8 for a single
// staged row (measured at B = 1: down 7.7 us with 8 waves per block against
// 8.3 with 16, qkv 6.0 with 4 against 6.15 with 8, o equal; at B = 4 the
// extra waves pay off again on down) and for blocks of four or more tiles
// (gate_up at B = 4: 15.0 us with 4 waves, 16.6 with 8).
template <bool BF16, int TM, int TN, bool XLDS, int VROWS>
static const char* decode_nw(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                             const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    constexpr int BAND = VROWS > 0 ? VROWS : 16 * TM;
    const int64_t blocks = (((N >> 4) + TN - 1) / TN) * ((M + BAND - 1) / BAND);
    const int64_t ngroups = K >> 7;
    const int64_t waves_per_device = XLDS && TM == 1 && VROWS == 0 && (M == 1 || TN >= 4) ? 2048 : 4096;
    int64_t want = (waves_per_device + blocks - 1) / blocks;
    if (want > ngroups) want = ngroups;
    // 16 waves per block caps a thread at 128 VGPRs: only the light variants
    constexpr bool fits16 = VROWS > 0 ? (VROWS == 1 && TN == 1) : (TM * TN == 1 || (XLDS && TM * TN == 2));
    if constexpr (fits16) {
        if (want >= 16) return decode_cfg<BF16, TM, TN, 16, XLDS, VROWS>(x, M, K, qw, sc, zr, N, y, s);
    }
    if constexpr (TM < 4) {
        if (want >= 8) return decode_cfg<BF16, TM, TN, 8, XLDS, VROWS>(x, M, K, qw, sc, zr, N, y, s);
    }
    // at least 4 waves: a single wave per block cannot keep enough loads in flight
    if (ngroups >= 4) return decode_cfg<BF16, TM, TN, 4, XLDS, VROWS>(x, M, K, qw, sc, zr, N, y, s);
    return decode_cfg<BF16, TM, TN, 1, XLDS, VROWS>(x, M, K, qw, sc, zr, N, y, s);
}

// (tn_max tiles and 16 waves: at least the scale area of any configuration
// the caller may pick)
static bool xlds_fits(int64_t rows, int64_t K, bool valu, int tn_max) {
    return decode_scale_lds(tn_max, 16, K) + rows * (K + 8) * 2 + (valu ? rows * (K >> 7) * 4 : 0) <= kLdsMax;
}

// Two weight tiles per block on wide layers, and from M = 9 on N > 4096 (the
// activation rows a block stages are then shared by twice the weight bytes);
// one otherwise (more blocks for short layers).  When the staged rows take
// more than half the LDS, a CU holds one block: the tiles are then dealt so
// that the grid is one round of at most 256 blocks (7 tiles per block on a
// 28672-wide layer instead of 1.75 rounds of 4).
template <bool BF16>
static const char* decode_dt(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                             const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    const bool wide = N >= 16384 || (M > 8 && N > 4096);
    if (M <= 16) {
        if (xlds_fits(M, K, false, 8)) {
            if (M * (K + 8) * 2 > 80 * 1024) {
                const int64_t per = ((N >> 4) + 255) / 256;               // tiles per block for one round
                if (per > 7) return decode_nw<BF16, 1, 8, true, 0>(x, M, K, qw, sc, zr, N, y, s);
                if (per > 4) return decode_nw<BF16, 1, 7, true, 0>(x, M, K, qw, sc, zr, N, y, s);
                if (per > 2) return decode_nw<BF16, 1, 4, true, 0>(x, M, K, qw, sc, zr, N, y, s);
                if (per > 1) return decode_nw<BF16, 1, 2, true, 0>(x, M, K, qw, sc, zr, N, y, s);
                return decode_nw<BF16, 1, 1, true, 0>(x, M, K, qw, sc, zr, N, y, s);
            }
            // (four tiles per block on the widest layers through M = 8: gate_up
            // 14.8 / 15.2 / 16.3 / 16.3 us at B = 1 / 4 / 6 / 8 against
            // 15.0 / 16.2 / 17.5 / 19.0 with two and 15.2 / 17.3 / 20.5 / 23.9
            // with one)
            if (N >= 16384 && M <= 8) return decode_nw<BF16, 1, 4, true, 0>(x, M, K, qw, sc, zr, N, y, s);
            if (wide) return decode_nw<BF16, 1, 2, true, 0>(x, M, K, qw, sc, zr, N, y, s);
            return decode_nw<BF16, 1, 1, true, 0>(x, M, K, qw, sc, zr, N, y, s);
        }
        if (wide) return decode_nw<BF16, 1, 2, false, 0>(x, M, K, qw, sc, zr, N, y, s);
        return decode_nw<BF16, 1, 1, false, 0>(x, M, K, qw, sc, zr, N, y, s);
    }
    if (M <= 32) return decode_nw<BF16, 2, 1, false, 0>(x, M, K, qw, sc, zr, N, y, s);
    return decode_nw<BF16, 4, 1, false, 0>(x, M, K, qw, sc, zr, N, y, s);
}

const char* launch_w4a16_skinny(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                                const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return decode_dt<true>(x, M, K, qw, sc, zr, N, y, s);
    return decode_dt<false>(x, M, K, qw, sc, zr, N, y, s);
}

// VALU GEMV: row bands of 1, 2 or 4 activation rows (grid.y covers larger M).
template <bool BF16>
static const char* gemv_dt(const void* x, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* sc,
                           const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    const bool wide = N >= 16384;
    if (M <= 1) {
        if (wide) return decode_nw<BF16, 1, 2, true, 1>(x, M, K, qw, sc, zr, N, y, s);
        return decode_nw<BF16, 1, 1, true, 1>(x, M, K, qw, sc, zr, N, y, s);
    }
    if (M <= 2) {
        if (wide) return decode_nw<BF16, 1, 2, true, 2>(x, M, K, qw, sc, zr, N, y, s);
        return decode_nw<BF16, 1, 1, true, 2>(x, M, K, qw, sc, zr, N, y, s);
    }
    if (wide) return decode_nw<BF16, 1, 2, true, 4>(x, M, K, qw, sc, zr, N, y, s);
    return decode_nw<BF16, 1, 1, true, 4>(x, M, K, qw, sc, zr, N, y, s);
}

bool w4a16_gemv_supported(int64_t M, int64_t K) { return xlds_fits(M < 4 ? M : 4, K, true, 2); }

const char* launch_w4a16_gemv(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    if (x_bf16) return gemv_dt<true>(x, M, K, qw, sc, zr, N, y, s);
    return gemv_dt<false>(x, M, K, qw, sc, zr, N, y, s);
}

// ---- split-K configuration (shared by the workspace query and the launch) ----
struct SplitCfg {
    int TM, S, gs, colgroups;
    int64_t ws_bytes, lds_bytes;
};

static SplitCfg splitk_cfg(int64_t M, int64_t N, int64_t K) {
    SplitCfg c{};
    c.TM = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    const int64_t rows = M < 16 * c.TM ? M : 16 * c.TM;
    const int64_t ntiles = N >> 4, ngroups = K >> 7;
    c.colgroups = (int)((ntiles + SPK_NW - 1) / SPK_NW);
    // slices: about one block per CU, at least one group per slice, LDS-bounded
    int64_t S = (256 + c.colgroups / 2) / c.colgroups;
    if (S < 1) S = 1;
    if (S > ngroups) S = ngroups;
    int64_t gs = (ngroups + S - 1) / S;
    const int64_t per_group = rows * 256 + 16 * c.TM * 4;                   // staged halves + Sx table
    int64_t gs_max = (96 * 1024 - rows * 16) / per_group;
    if (gs_max < 1) gs_max = 1;
    if (gs > gs_max) gs = gs_max;
    S = (ngroups + gs - 1) / gs;
    c.S = (int)S;
    c.gs = (int)gs;
    c.lds_bytes = rows * (gs * 128 + 8) * 2 + gs * 16 * c.TM * 4;
    c.ws_bytes = S > 1 ? S * c.colgroups * SPK_NW * c.TM * 1024 : 0;
    return c;
}

int64_t w4a16_splitk_workspace(int64_t M, int64_t N, int64_t K) { return splitk_cfg(M, N, K).ws_bytes; }

template <bool BF16, int TM>
static const char* splitk_launch(const SplitCfg& c, const void* x, int64_t M, int64_t K, const uint32_t* qw,
                                 const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws,
                                 hipStream_t s) {
    auto kern = k_w4a16_splitk<BF16, TM>;
    allow_lds(kern, (size_t)c.lds_bytes);
    hipLaunchKernelGGL(kern, dim3((unsigned)c.colgroups, (unsigned)c.S), dim3(SPK_NW * 64), (size_t)c.lds_bytes, s,
                       static_cast<const uint16_t*>(x), M, K, qw, sc, zr, N, static_cast<uint16_t*>(y),
                       static_cast<float*>(ws), c.S, c.gs);
    if (c.S > 1) {
        const int64_t tiles_pad = (int64_t)c.colgroups * SPK_NW;
        const int64_t threads = tiles_pad * TM * 256;
        hipLaunchKernelGGL((k_w4a16_splitk_reduce<BF16, TM>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(ws), c.S, tiles_pad, M, N, static_cast<uint16_t*>(y));
    }
    return kname("k_w4a16_splitk", BF16, TM);
}

const char* launch_w4a16_splitk(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                                const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws,
                                hipStream_t s) {
    const SplitCfg c = splitk_cfg(M, N, K);
    if (x_bf16) {
        if (c.TM == 1) return splitk_launch<true, 1>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        if (c.TM == 2) return splitk_launch<true, 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
        return splitk_launch<true, 4>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    }
    if (c.TM == 1) return splitk_launch<false, 1>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    if (c.TM == 2) return splitk_launch<false, 2>(c, x, M, K, qw, sc, zr, N, y, ws, s);
    return splitk_launch<false, 4>(c, x, M, K, qw, sc, zr, N, y, ws, s);
}

const char* launch_w4a16_tiled(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                               const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s) {
    return launch_w4a16_gemm(x, x_bf16, M, K, qw, sc, zr, N, y, nullptr, s);
}

}  // namespace bg
