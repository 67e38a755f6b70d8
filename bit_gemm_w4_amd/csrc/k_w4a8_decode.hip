// k_w4a8_decode.hip -- W4A8 at small M (decode): Y = (A s_a) W^T with A the
// INT8 activation codes of at most 32 rows (one or two 16-row bands, TM) and
// W in the packed INT4 format.
//
// "Low-precision LLM inference" §1 (W4A8: INT4 weights, INT8 activations,
// INT32/FP32 accumulation), §14 (per-token activation scales), §26 (decode
// is bound by the weight bytes).  At small M the packed weights are the
// bytes that matter, so this kernel streams them like the W4A16 decode
// kernel and computes on the INT8 matrix cores.
//
// A block owns 16*TN output columns (TN weight tiles) and all of K; its NW
// waves take the 128-wide groups round-robin, so the block sweeps its tiles
// front to back as one stream of 1 KB tile loads (one per wave, tile and
// group), software-pipelined STAGES deep and issued unconditionally (past a
// wave's last group the loads address beyond the buffer: zeros, no memory
// access).  XL: the activation rows (all of K, INT8) are copied into LDS
// once per block; when they do not fit (16 rows of K = 14336), each stage
// also carries the lane's two 16-byte activation fragments of the group,
// read from the (cache-resident) rows directly.  Each wave copies its own
// groups' FP16 scales and zero-point bytes into a wave-private LDS area (48
// bytes per tile and group), so the weight tiles are the only other global
// stream.
//
// Lane l (l16 = l % 16, q = l / 16) holds, per group, slot l of each 1 KB
// tile: words 4q .. 4q+3 of column l16, i.e. k = 32q .. 32q+31.  In MFMA
// step s (of two per group) it supplies the 16 consecutive k starting at
// 32q + 16s: those of column l16 as the signed bytes u - z (exact, see
// w4_to_i8) and those of activation row l16 from LDS, so matching k meet in
// v_mfma_i32_16x16x64_i8.  The group's INT32 sum T is exact (|T| <= 128 * 128
// * 15 < 2^24, so exact in FP32 too) and acc += s_w * T closes the group in
// FP32; the waves' partial tiles are added in LDS in wave order and s_a
// scales each row in the epilogue -- the arithmetic of the large-M kernel.
#include "bg_device.h"
#include "bg_internal.h"
#include "bg_w4.h"

namespace bg {

namespace {
enum { WO_F32 = 0, WO_F16 = 1, WO_BF16 = 2 };

template <int TM, int TN, bool XL>
struct Q8Stage {
    uint4 w[TN];
    uint4 a[XL ? 1 : TM][2];
};
}  // namespace

template <int TM, int TN, int NW, bool XL>
__global__ __launch_bounds__(NW * 64) void k_w4a8_decode(const int8_t* __restrict__ a, const float* __restrict__ as,
                                                         int a_row, int64_t M, int64_t K,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ sc,
                                                         const uint8_t* __restrict__ zr, int64_t N,
                                                         void* __restrict__ y, int out_dt, uint64_t rcp) {
    // two groups in flight per wave: deeper pipelines keep more requests in
    // flight than the memory side serves well (the twelve Llama-3-8B decode
    // calls at B = 1, 4, 16: 111.1 us in all against 115.8 with the earlier
    // 4 / 3 / 2 groups for one / two / more tiles; gate_up at B = 16 18.3
    // against 19.6; three groups only helped down at B = 1 and 4, by 0.15 us)
    constexpr int STAGES = 2;
    static_assert(XL || TN <= 2, "activation fragments in the stages: at most two tiles");
    static_assert(TM == 1 || TN <= 4, "two bands: at most four tiles");
    constexpr int XB = 4;                                              // activation chunks per batch
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t ntiles = N >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * TN;
    const int ngroups = (int)(K >> 7);
    const int n_mine = ngroups > wave ? (ngroups - wave + NW - 1) / NW : 0;
    const int rows = M < 16 * TM ? (int)M : 16 * TM;
    const int64_t pitch = K + 16;                                      // LDS row pitch: rows 4 banks apart
    const bool has_z = zr != nullptr;
    // LDS: [per wave: its groups' scale and zero records][activation rows]
    const int nmax = (ngroups + NW - 1) / NW;
    uint8_t* wsz = dyn_lds + wave * nmax * TN * 48;
    uint8_t* x_l = dyn_lds + NW * nmax * TN * 48;

    const int64_t my_tiles = (ntiles - t0) < TN ? (ntiles - t0) : TN;
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw + t0 * ngroups * 256), (short)0,
                                                      (int)(my_tiles * ngroups * 1024), 0x00020000);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sc + t0 * ngroups * 16), (short)0,
                                                      (int)(my_tiles * ngroups * 32), 0x00020000);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(has_z ? zr + t0 * (ngroups >> 1) * 16 : zr),
                                                      (short)0, has_z ? (int)(my_tiles * (ngroups >> 1) * 16) : 0,
                                                      0x00020000);
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a), (short)0, (int)(rows * K), 0x00020000);

    int arow[TM];                                                     // rows past M: row M - 1, never written
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = 16 * i + l16 < rows ? 16 * i + l16 : rows - 1;
    auto issue = [&](Q8Stage<TM, TN, XL>& st, int i) {
        const bool real = i < n_mine;
        const int g = i * NW + wave;
#pragma unroll
        for (int j = 0; j < TN; ++j)
            st.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rw, lane * 16, real ? (j * ngroups + g) * 1024 : kBufOOB, 0));
        if constexpr (!XL) {
#pragma unroll
            for (int b = 0; b < TM; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    st.a[b][s2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                ra, (int)(arow[b] * K) + q * 32 + s2 * 16,
                                                                real ? g * 128 : kBufOOB, 0));
        }
    };

    // this wave's scale and zero records: 16 per pass of 64 lanes, lane =
    // 4 * record + part (parts 0, 1: the two halves of the 16 FP16 scales;
    // part 2: the 16 zero bytes of the group pair; part 3 idle)
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
    uint4 szv = uint4{0, 0, 0, 0};
    sz_issue(0, szv);

    // activation rows -> LDS, 16-byte chunks, XB per thread in flight; chunk
    // c is row c / cpr, found by a multiply with rcp = ceil(2^40 / cpr)
    // (host-computed; exact for c < 2^21)
    const int cpr = (int)(K >> 4);
    const int total = XL ? rows * cpr : 0;
    auto x_load = [&](uint4 (&v)[XB], int c0) {
#pragma unroll
        for (int u = 0; u < XB; ++u)
            if (c0 + u * NW * 64 < total)
                v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, (c0 + u * NW * 64) * 16,
                                                                                       0, 0));
    };
    auto x_store = [&](const uint4 (&v)[XB], int c0) {
#pragma unroll
        for (int u = 0; u < XB; ++u) {
            const int c = c0 + u * NW * 64;
            if (c < total) {
                const int r = (int)(((uint64_t)c * rcp) >> 40), kc = c - r * cpr;
                *reinterpret_cast<uint4*>(x_l + (int64_t)r * pitch + kc * 16) = v[u];
            }
        }
    };
    uint4 xv0[XB];
    x_load(xv0, threadIdx.x);

    Q8Stage<TM, TN, XL> stage[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue(stage[s], s);

    x_store(xv0, threadIdx.x);
    for (int c0 = threadIdx.x + XB * NW * 64; c0 < total; c0 += XB * NW * 64) {
        uint4 v[XB];
        x_load(v, c0);
        x_store(v, c0);
    }
    __syncthreads();
    sz_store(0, szv);
    for (int r0 = 16; r0 < nrec; r0 += 16) {
        uint4 v = uint4{0, 0, 0, 0};
        sz_issue(r0, v);
        sz_store(r0, v);
    }

    float4_t acc[TM][TN];
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[b][j] = float4_t{0, 0, 0, 0};

    auto consume = [&](const Q8Stage<TM, TN, XL>& st, int i) {
        const int g = i * NW + wave;
        int4_t a0[TM], a1[TM];
#pragma unroll
        for (int b = 0; b < TM; ++b) {
            uint4 x0, x1;
            if constexpr (XL) {
                const uint8_t* xr = x_l + (int64_t)arow[b] * pitch + (int64_t)g * 128 + q * 32;
                x0 = *reinterpret_cast<const uint4*>(xr);
                x1 = *reinterpret_cast<const uint4*>(xr + 16);
            } else {
                x0 = st.a[b][0];
                x1 = st.a[b][1];
            }
            a0[b] = int4_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
            a1[b] = int4_t{(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint8_t* rec = wsz + (i * TN + j) * 48;
            const float s_w = f16_to_f32(*reinterpret_cast<const uint16_t*>(rec + l16 * 2));
            const uint32_t z = has_z ? (rec[32 + l16] >> (4 * (g & 1))) & 0xFu : 8u;
            const uint32_t zc = 0x80808080u - z * 0x01010101u;
            const int4_t w0 = w4_to_i8(make_uint2(st.w[j].x, st.w[j].y), zc);
            const int4_t w1 = w4_to_i8(make_uint2(st.w[j].z, st.w[j].w), zc);
#pragma unroll
            for (int b = 0; b < TM; ++b) {
                int4_t t = int4_t{0, 0, 0, 0};
                t = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[b], w0, t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[b], w1, t, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[b][j][e] += s_w * (float)t[e];
            }
        }
    };

    for (int i = 0; i < n_mine; i += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
            if (i + s < n_mine) consume(stage[s], i + s);
            issue(stage[s], i + s + STAGES);
        }
    }

    // ---- sum the NW partial tiles in wave order through LDS ----
    __syncthreads();
    float* red = reinterpret_cast<float*>(dyn_lds);                   // [NW][TM][TN][4][64]
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(((wave * TM + b) * TN + j) * 4 + e) * 64 + lane] = acc[b][j][e];
    __syncthreads();
    for (int t = threadIdx.x; t < TM * TN * 256; t += NW * 64) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w * TM * TN * 256 + t];
        const int ln = t & 63, e = (t >> 6) & 3, bj = t >> 8;
        const int b = bj / TN, j = bj - b * TN;
        const int64_t m = 16 * b + 4 * (ln >> 4) + e;
        const int64_t n = (t0 + j) * 16 + (ln & 15);
        if (m >= M || n >= N) continue;
        const float f = v * (a_row ? as[m] : as[0]);
        const int64_t o = m * N + n;
        if (out_dt == WO_BF16) static_cast<uint16_t*>(y)[o] = f32_to_bf16(f);
        else if (out_dt == WO_F16) static_cast<uint16_t*>(y)[o] = f32_to_f16(f);
        else static_cast<float*>(y)[o] = f;
    }
}

constexpr int64_t kW4A8DecodeLds = 144 * 1024;

// LDS bytes: the waves' records and (XL) the activation rows, or the
// reduction buffer, whichever is larger.
static int64_t w4a8_decode_lds(int TM, int TN, int NW, bool xl, int64_t M, int64_t K) {
    const int64_t rows = M < 16 * TM ? M : 16 * TM;
    const int64_t xb = (int64_t)NW * (((K >> 7) + NW - 1) / NW) * TN * 48 + (xl ? rows * (K + 16) : 0);
    const int64_t red = (int64_t)NW * TM * TN * 256 * 4;
    return xb > red ? xb : red;
}

// Bands: one up to 16 rows, two up to 32.  Tiles per block: two on wide
// layers (N >= 16384); when the staged rows take more than 80 KB (a CU then
// holds one block) the tiles are dealt so the grid is about one round of 256
// blocks (at most four with two bands).  Without room for the rows (XL
// false) at most two.  Waves per block: about 16 per CU resident, never more
// than K has groups, at most 8 with four or more tiles (registers).
struct Q8Cfg {
    int TM, TN, NW;
    bool xl;
};
static Q8Cfg w4a8_decode_cfg(int64_t M, int64_t N, int64_t K) {
    const int TM = M <= 16 ? 1 : 2;
    const int64_t rows = M < 16 * TM ? M : 16 * TM, ntiles = N >> 4, ngroups = K >> 7;
    int TN = N >= 16384 ? 2 : 1;
    bool xl = true;
    if (rows * (K + 16) > 80 * 1024) {
        const int64_t per = (ntiles + 255) / 256;
        TN = per > 4 ? 8 : per > 2 ? 4 : per > 1 ? 2 : 1;
        if (TM == 2 && TN > 4) TN = 4;
    }
    for (;;) {
        const int64_t blocks = (ntiles + TN - 1) / TN;
        int64_t want = (4096 + blocks - 1) / blocks;
        if (want > ngroups) want = ngroups;
        int NW = want >= 16 ? 16 : want >= 8 ? 8 : 4;
        if ((TN >= 4 || TM * TN >= 4) && NW > 8) NW = 8;
        if (!xl || w4a8_decode_lds(TM, TN, NW, true, M, K) <= kW4A8DecodeLds) return Q8Cfg{TM, TN, NW, xl};
        xl = false;                                  // the rows do not fit: fragments in the stages
        TN = N >= 16384 ? 2 : 1;
    }
}

bool w4a8_decode_fits(int64_t M, int64_t N, int64_t K) {
    if (M > 32) return false;
    const Q8Cfg c = w4a8_decode_cfg(M, N, K);
    return w4a8_decode_lds(c.TM, c.TN, c.NW, c.xl, M, K) <= kW4A8DecodeLds;
}

template <int TM, int TN, int NW, bool XL>
static const char* decode_cfg(const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, int out_dt, hipStream_t s) {
    const dim3 grid((unsigned)(((N >> 4) + TN - 1) / TN));
    const size_t lds = (size_t)w4a8_decode_lds(TM, TN, NW, XL, M, K);
    auto kern = k_w4a8_decode<TM, TN, NW, XL>;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    const uint64_t cpr = (uint64_t)(K >> 4);
    const uint64_t rcp = ((uint64_t(1) << 40) + cpr - 1) / cpr;
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, a, as, (int)a_row, M, K, qw, sc, zr, N, y, out_dt, rcp);
    return kname("k_w4a8_decode", TM, TN, NW, XL);
}

template <int TM, int TN, bool XL>
static const char* decode_nw(int NW, const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K,
                             const uint32_t* qw, const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, int out_dt,
                             hipStream_t s) {
    if constexpr (TN < 4 && TM * TN < 4) {
        if (NW == 16) return decode_cfg<TM, TN, 16, XL>(a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    }
    if (NW >= 8) return decode_cfg<TM, TN, 8, XL>(a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    return decode_cfg<TM, TN, 4, XL>(a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
}

template <int TM>
static const char* decode_tn(const Q8Cfg& c, const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K,
                             const uint32_t* qw, const uint16_t* sc, const uint8_t* zr, int64_t N, void* y,
                             int out_dt, hipStream_t s) {
    if (!c.xl) {
        if (c.TN == 2) return decode_nw<TM, 2, false>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
        return decode_nw<TM, 1, false>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    }
    if constexpr (TM == 1) {
        if (c.TN == 8) return decode_nw<TM, 8, true>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    }
    if (c.TN >= 4) return decode_nw<TM, 4, true>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    if (c.TN == 2) return decode_nw<TM, 2, true>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    return decode_nw<TM, 1, true>(c.NW, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
}

// Requires w4a8_decode_fits(M, N, K).
const char* launch_w4a8_decode(const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K,
                               const uint32_t* qw, const uint16_t* sc, const uint8_t* zr, int64_t N, void* y,
                               int out_dt, hipStream_t s) {
    const Q8Cfg c = w4a8_decode_cfg(M, N, K);
    if (c.TM == 2) return decode_tn<2>(c, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
    return decode_tn<1>(c, a, as, a_row, M, K, qw, sc, zr, N, y, out_dt, s);
}

}  // namespace bg
