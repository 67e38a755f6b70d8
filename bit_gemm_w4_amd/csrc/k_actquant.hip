// k_actquant.hip -- dynamic INT8 / FP8-E4M3 quantizers (act_quant_int8/fp8).
//
// "Low-precision LLM inference": §2 eq. (1) with z = 0 and §3 eq. (3)
// (s = amax / qmax); §4 granularities (per tensor, per token/row, per group,
// per block); §8 current scaling (amax of the tensor being quantized) and
// block scaling (scale_block = amax_block / max_fp8).  qmax is 127 (INT8) or
// 448 (E4M3); a scale that comes out 0 (all-zero unit) is replaced by 1.
//
// Every kernel keeps its unit in registers between the amax reduction and
// the quantization, so HBM is read once and written once (2 B in, 1 B out per
// element for BF16): these kernels are bandwidth-bound, and the per-token
// amax is the reduction the page warns can sit on the critical path (§4).
// Per-tensor scaling needs a grid-wide amax: a one-thread fill kernel clears
// the amax slot (no hipMemset, so the sequence is graph-capturable), the amax
// kernel combines block maxima with an integer atomic max on the float bits
// (valid because amax >= 0), and the quantize kernel reads the slot.
//
// CM (the SmoothQuant fold, §15: Y = (X S^-1)(W S)^T): every element is first
// multiplied by its column's factor cm[j] (1/s_j for activations, s_j for the
// weights folded offline) -- one binary32 multiplication, fused into the load,
// so the smoothed tensor never goes back to HBM.
#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

#pragma clang fp contract(off)

enum { G_TENSOR = 0, G_ROW = 1, G_ROW_G128 = 2, G_BLOCK128 = 3 };

// The scale of a unit and what its quotients v / s need: the codes are the
// roundings of the correctly rounded binary32 quotient.  Rather than one
// IEEE division per element (a long instruction sequence on this device), a
// unit computes r = RN(1/s) once and each element takes Markstein's
// correction of q0 = RN(v r): with the exact remainder e = v - q0 s (one
// fma), RN(q0 + e r) is the correctly rounded quotient, since r is within
// half an ulp of 1/s and q0 within one ulp of v/s (P. Markstein, IBM J. Res.
// Dev. 34(1), 1990; the theorem holds without overflow or underflow).  Units
// whose scale lies outside [2^-100, 2^100] (r could overflow, or the
// remainder underflow) divide instead.
struct QScale {
    float s, r;
    bool mk;
};

template <bool FP8>
__device__ __forceinline__ QScale unit_scale(float amax) {
    float s = amax / (FP8 ? 448.0f : 127.0f);
    s = s == 0.0f ? 1.0f : s;
    return QScale{s, 1.0f / s, s >= 0x1p-100f && s <= 0x1p100f};
}

__device__ __forceinline__ void quotients8(const float v[8], const QScale& u, float d[8]) {
    if (u.mk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q0 = v[i] * u.r;
            // (the sign is v's, as in v / s: -0 and quotients that round to
            // zero stay negative)
            d[i] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, u.s, v[i]), u.r, q0), v[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = v[i] / u.s;
    }
}

// Quantize 8 values with the unit's scale and store 8 bytes at q[idx].
template <bool FP8>
__device__ __forceinline__ void quant_store8(const float v[8], const QScale& u, void* q, int64_t idx) {
    float d[8];
    quotients8(v, u, d);
    uint32_t lo = 0, hi = 0;
    if constexpr (FP8) {
        lo = e4m3x2(d[0], d[1]) | (e4m3x2(d[2], d[3]) << 16);
        hi = e4m3x2(d[4], d[5]) | (e4m3x2(d[6], d[7]) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = __builtin_rintf(d[i]);
            r = __builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
            const uint32_t b = (uint32_t)((int)r & 0xFF);
            if (i < 4) lo |= b << (8 * i);
            else hi |= b << (8 * (i - 4));
        }
    }
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(q) + idx) = make_uint2(lo, hi);
}

// 8 consecutive elements (columns col .. col + 7) as floats, times their
// column factors when CM.
template <int DT, bool CM>
__device__ __forceinline__ void load8(const void* x, int64_t idx, const float* __restrict__ cm, int64_t col,
                                      float v[8]) {
    load8_f32<DT>(x, idx, v);
    if constexpr (CM) {
        const float4 a = *reinterpret_cast<const float4*>(cm + col);
        const float4 b = *reinterpret_cast<const float4*>(cm + col + 4);
        v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
        v[4] *= b.x; v[5] *= b.y; v[6] *= b.z; v[7] *= b.w;
    }
}

__device__ __forceinline__ float amax8(const float v[8]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    return a;
}

// Max over a 256-thread block; every thread gets the result.
__device__ __forceinline__ float block_max256(float a, float* red) {
    a = wave_max<64>(a);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = a;
    __syncthreads();
    a = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    return a;
}

// ---- per row (token / output channel), rows up to 256 * 8 * IT long ----
// IT (chunks of 8 per thread) is sized to the row, so short rows keep few
// registers and many rows resident per CU.
constexpr int ROW_MAXIT = 8;

// The chunk at byte offset off of the row behind buffer resource rs as 8
// floats (16 bytes of F16 / BF16 or 32 of F32), times the 8 column factors at
// byte offset coff of rc when CM.  Offset kBufOOB reads zeros, so a thread
// can issue all its chunks unconditionally and keep them in flight together.
template <int DT, bool CM>
__device__ __forceinline__ void load8_buf(__amdgpu_buffer_rsrc_t rs, int off, __amdgpu_buffer_rsrc_t rc, int coff,
                                          float v[8]) {
    if constexpr (DT == DT_F32) {
        const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        const float4 b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 16, 0));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DT_BF16) {
                v[2 * i] = __uint_as_float(u[i] << 16);
                v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            } else {
                v[2 * i] = f16_to_f32(u[i] & 0xFFFFu);
                v[2 * i + 1] = f16_to_f32(u[i] >> 16);
            }
        }
    }
    if constexpr (CM) {
        const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff, 0, 0));
        const float4 b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff, 16, 0));
        v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
        v[4] *= b.x; v[5] *= b.y; v[6] *= b.z; v[7] *= b.w;
    }
}

template <int DT, bool FP8, bool CM, int IT>
__global__ __launch_bounds__(256) void k_quant_row(const void* __restrict__ x, int64_t C,
                                                   void* __restrict__ q, float* __restrict__ scales,
                                                   const float* __restrict__ cm) {
    __shared__ float red[4];
    constexpr int EB = DT == DT_F32 ? 4 : 2;
    const int64_t r = blockIdx.x;
    const int nchunk = (int)(C >> 3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(x) + r * C * EB), (short)0, (int)(C * EB), 0x00020000);
    const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(cm), (short)0, CM ? (int)(C * 4) : 0,
                                                      0x00020000);
    float v[IT][8];
    float a = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int c = it * 256 + (int)threadIdx.x;
        load8_buf<DT, CM>(rs, c < nchunk ? c * 8 * EB : kBufOOB, rc, c < nchunk ? c * 32 : kBufOOB, v[it]);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) a = __builtin_fmaxf(a, amax8(v[it]));     // out-of-range chunks are 0
    const QScale u = unit_scale<FP8>(block_max256(a, red));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t c = (int64_t)it * 256 + threadIdx.x;
        if (c < nchunk) quant_store8<FP8>(v[it], u, q, r * C + c * 8);
    }
    if (threadIdx.x == 0) scales[r] = u.s;
}

// Rows longer than 256 * 8 * ROW_MAXIT: amax pass, then a second read.
template <int DT, bool FP8, bool CM>
__global__ __launch_bounds__(256) void k_quant_row_2pass(const void* __restrict__ x, int64_t C,
                                                         void* __restrict__ q,
                                                         float* __restrict__ scales,
                                                         const float* __restrict__ cm) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const int64_t nchunk = C >> 3;
    float v[8];
    float a = 0.0f;
    for (int64_t c = threadIdx.x; c < nchunk; c += 256) {
        load8<DT, CM>(x, r * C + c * 8, cm, c * 8, v);
        a = __builtin_fmaxf(a, amax8(v));
    }
    const QScale u = unit_scale<FP8>(block_max256(a, red));
    for (int64_t c = threadIdx.x; c < nchunk; c += 256) {
        load8<DT, CM>(x, r * C + c * 8, cm, c * 8, v);
        quant_store8<FP8>(v, u, q, r * C + c * 8);
    }
    if (threadIdx.x == 0) scales[r] = u.s;
}

// ---- 1 x 128 groups: 16 consecutive lanes per group ----
template <int DT, bool FP8, bool CM>
__global__ __launch_bounds__(256) void k_quant_g128(const void* __restrict__ x, int64_t total_chunks,
                                                    void* __restrict__ q, float* __restrict__ scales,
                                                    const float* __restrict__ cm, int64_t C) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total_chunks) return;          // total_chunks is a multiple of 16
    float v[8];
    load8<DT, CM>(x, t * 8, cm, CM ? (t % (C >> 3)) * 8 : 0, v);
    const QScale u = unit_scale<FP8>(wave_max<16>(amax8(v)));
    quant_store8<FP8>(v, u, q, t * 8);
    if ((t & 15) == 0) scales[t >> 4] = u.s;
}

// ---- MXFP8 / MXFP4: 32-element blocks along a row, 4 consecutive lanes per block ----
// OCP MX: E8M0 scale 2^(e - 127), e = floor(log2 amax) - emax + 127 (emax =
// the largest element exponent: 8 for E4M3, 2 for E2M1) clamped to 0..254,
// 127 for an all-zero block, 254 for a block holding an infinity; the
// elements are the saturating RNE casts of
// v * 2^(127 - e) (exact power-of-two scaling).  FP4 elements are packed two
// per byte, the even element in the low nibble.  Scales are K-block-major,
// [cols/32][rows rounded up to 16], so one K block's scales of consecutive
// rows are contiguous.

// E2M1 code of r: the magnitude code counts the rounding boundaries r passes
// (the midpoints of 0, 0.5, 1, 1.5, 2, 3, 4, 6; a midpoint itself goes to
// the neighbour with the even mantissa bit, so ">" where the lower neighbour
// is even and ">=" where the upper one is), which also saturates at 6; the
// sign bit is r's own, so values that round to zero keep it.
__device__ __forceinline__ uint32_t e2m1_code(float r) {
    const float a = __builtin_fabsf(r);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(r) >> 28) & 8u);
}

template <int DT, bool FP4>
__global__ __launch_bounds__(256) void k_quant_mx32(const void* __restrict__ x, int64_t total_chunks,
                                                    int64_t C, int64_t rpad, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ e8m0) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total_chunks) return;          // total_chunks is a multiple of 4: whole blocks retire together
    float v[8];
    load8_f32<DT>(x, t * 8, v);
    const float amax = wave_max<4>(amax8(v));
    int e = 127;
    if (__builtin_isinf(amax)) e = 254;     // floor(log2 inf) = inf: the clamp's top
    else if (amax > 0.0f) {
        e = ilogbf(amax) - (FP4 ? 2 : 8) + 127;
        e = e < 0 ? 0 : e > 254 ? 254 : e;
    }
    if constexpr (FP4) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(ldexpf(v[i], 127 - e)) << (4 * i);
        *reinterpret_cast<uint32_t*>(q + t * 4) = word;
    } else {
        uint32_t lo = 0, hi = 0;
        lo = e4m3x2(ldexpf(v[0], 127 - e), ldexpf(v[1], 127 - e)) | (e4m3x2(ldexpf(v[2], 127 - e), ldexpf(v[3], 127 - e)) << 16);
        hi = e4m3x2(ldexpf(v[4], 127 - e), ldexpf(v[5], 127 - e)) | (e4m3x2(ldexpf(v[6], 127 - e), ldexpf(v[7], 127 - e)) << 16);
        *reinterpret_cast<uint2*>(q + t * 8) = make_uint2(lo, hi);
    }
    if ((t & 3) == 0) {
        const int64_t row = t / (C >> 3), blk = (t - row * (C >> 3)) >> 2;
        e8m0[blk * rpad + row] = (uint8_t)e;
    }
}

template <bool FP4>
static void quant_mx32(const void* x, int dt, int64_t chunks, int64_t C, int64_t rpad, uint8_t* q, uint8_t* e8m0,
                       hipStream_t s) {
    const dim3 grid((unsigned)((chunks + 255) / 256));
    if (dt == DT_F32)
        hipLaunchKernelGGL((k_quant_mx32<DT_F32, FP4>), grid, dim3(256), 0, s, x, chunks, C, rpad, q, e8m0);
    else if (dt == DT_F16)
        hipLaunchKernelGGL((k_quant_mx32<DT_F16, FP4>), grid, dim3(256), 0, s, x, chunks, C, rpad, q, e8m0);
    else
        hipLaunchKernelGGL((k_quant_mx32<DT_BF16, FP4>), grid, dim3(256), 0, s, x, chunks, C, rpad, q, e8m0);
}

const char* launch_quant_mx32(const void* x, int dt, int64_t R, int64_t C, bool fp4, uint8_t* q, uint8_t* e8m0,
                              hipStream_t s) {
    const int64_t chunks = R * (C >> 3), rpad = (R + 15) & ~(int64_t)15;
    if (fp4) quant_mx32<true>(x, dt, chunks, C, rpad, q, e8m0, s);
    else quant_mx32<false>(x, dt, chunks, C, rpad, q, e8m0, s);
    return kname("k_quant_mx32", dt, fp4);
}

// ---- 128 x 128 blocks: one workgroup per block ----
template <int DT, bool FP8, bool CM>
__global__ __launch_bounds__(256) void k_quant_block128(const void* __restrict__ x, int64_t C,
                                                        void* __restrict__ q,
                                                        float* __restrict__ scales,
                                                        const float* __restrict__ cm) {
    __shared__ float red[4];
    const int64_t nb_c = C >> 7;
    const int64_t rb = blockIdx.x / nb_c, cb = blockIdx.x - rb * nb_c;
    const int lane_c = threadIdx.x & 15, lane_r = threadIdx.x >> 4;   // 16 x 16 threads
    float v[8][8];
    float a = 0.0f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int64_t row = rb * 128 + it * 16 + lane_r;
        load8<DT, CM>(x, row * C + cb * 128 + lane_c * 8, cm, cb * 128 + lane_c * 8, v[it]);
        a = __builtin_fmaxf(a, amax8(v[it]));
    }
    const QScale u = unit_scale<FP8>(block_max256(a, red));
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int64_t row = rb * 128 + it * 16 + lane_r;
        quant_store8<FP8>(v[it], u, q, row * C + cb * 128 + lane_c * 8);
    }
    if (threadIdx.x == 0) scales[blockIdx.x] = u.s;
}

// ---- whole tensor ----
__global__ void k_clear_amax(float* __restrict__ scales) { scales[1] = 0.0f; }

// Both passes walk the tensor in tiles of TU * 256 chunks (8 elements each),
// tile t = blockIdx.x, + gridDim.x, ...; a thread issues its TU chunks of a
// tile unconditionally (buffer loads; chunks past the end read zeros), so
// they are in flight together.  The amax pass runs at most one block per CU
// with 8 chunks per thread: every block ends in an atomic on the one amax
// slot, and those serialize (measured: 1024 blocks' atomics cost 12 us on a
// 2048 x 4096 tensor, 256 blocks' about 3 us).
constexpr int TU = 4, TU_AMAX = 8;
constexpr unsigned AMAX_GRID = 256;

template <int DT, bool CM, int TUN>
__device__ __forceinline__ void load_tile(const void* x, const float* cm, int64_t nchunk, int64_t C, int64_t t,
                                          float (&v)[TUN][8]) {
    constexpr int EB = DT == DT_F32 ? 4 : 2;
    constexpr int64_t TILE_CHUNKS = TUN * 256;
    const int64_t c0 = t * TILE_CHUNKS;
    const int64_t n = nchunk - c0 < TILE_CHUNKS ? nchunk - c0 : TILE_CHUNKS;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(x) + c0 * 8 * EB), (short)0, (int)(n * 8 * EB), 0x00020000);
    const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(cm), (short)0, CM ? (int)(C * 4) : 0,
                                                      0x00020000);
#pragma unroll
    for (int u = 0; u < TUN; ++u) {
        const int i = u * 256 + (int)threadIdx.x;
        // column of the chunk's first element (rows are whole chunks: C % 8 == 0)
        const int col = CM ? (int)(((c0 + i) % (C >> 3)) * 8) : 0;
        load8_buf<DT, CM>(rs, i < n ? i * 8 * EB : kBufOOB, rc, i < n ? col * 4 : kBufOOB, v[u]);
    }
}

template <int DT, bool CM>
__global__ __launch_bounds__(256) void k_amax_tensor(const void* __restrict__ x, int64_t nchunk,
                                                     float* __restrict__ scales, const float* __restrict__ cm,
                                                     int64_t C) {
    __shared__ float red[4];
    float a = 0.0f;
    const int64_t tiles = (nchunk + TU_AMAX * 256 - 1) / (TU_AMAX * 256);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        float v[TU_AMAX][8];
        load_tile<DT, CM, TU_AMAX>(x, cm, nchunk, C, t, v);
#pragma unroll
        for (int u = 0; u < TU_AMAX; ++u) a = __builtin_fmaxf(a, amax8(v[u]));
    }
    a = block_max256(a, red);
    // Only blocks that would raise the running maximum take the atomic (all
    // blocks hitting one address serialize); the check reads the slot at
    // agent scope (not a stale cache line), and the value only grows, so a
    // skipped block never held a larger maximum.
    if (threadIdx.x == 0) {
        const unsigned cur = __hip_atomic_load(reinterpret_cast<unsigned int*>(scales + 1), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (__float_as_uint(a) > cur) atomicMax(reinterpret_cast<unsigned int*>(scales + 1), __float_as_uint(a));
    }
}

template <int DT, bool FP8, bool CM>
__global__ __launch_bounds__(256) void k_quant_tensor(const void* __restrict__ x, int64_t nchunk,
                                                      void* __restrict__ q,
                                                      float* __restrict__ scales,
                                                      const float* __restrict__ cm, int64_t C) {
    const QScale us = unit_scale<FP8>(scales[1]);
    const int64_t tiles = (nchunk + TU * 256 - 1) / (TU * 256);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        float v[TU][8];
        load_tile<DT, CM, TU>(x, cm, nchunk, C, t, v);
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const int64_t c = t * TU * 256 + u * 256 + threadIdx.x;
            if (c < nchunk) quant_store8<FP8>(v[u], us, q, c * 8);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = us.s;
}

static unsigned grid_for(int64_t nchunk, int tu, unsigned cap) {
    int64_t b = (nchunk + tu * 256 - 1) / (tu * 256);
    if (b > cap) b = cap;                  // tile-stride beyond the cap
    return (unsigned)(b < 1 ? 1 : b);
}

template <int DT, bool FP8, bool CM>
static const char* launch_typed(const void* x, int64_t R, int64_t C, int gran, void* q, float* sc, const float* cm,
                                hipStream_t s) {
    switch (gran) {
        case G_ROW:
            if (C <= 256 * 8 * ROW_MAXIT) {
                const int64_t per = (C / 8 + 255) / 256;         // chunks per thread
                if (per <= 1)
                    hipLaunchKernelGGL((k_quant_row<DT, FP8, CM, 1>), dim3((unsigned)R), dim3(256), 0, s, x, C, q, sc,
                                       cm);
                else if (per <= 2)
                    hipLaunchKernelGGL((k_quant_row<DT, FP8, CM, 2>), dim3((unsigned)R), dim3(256), 0, s, x, C, q, sc,
                                       cm);
                else if (per <= 4)
                    hipLaunchKernelGGL((k_quant_row<DT, FP8, CM, 4>), dim3((unsigned)R), dim3(256), 0, s, x, C, q, sc,
                                       cm);
                else
                    hipLaunchKernelGGL((k_quant_row<DT, FP8, CM, ROW_MAXIT>), dim3((unsigned)R), dim3(256), 0, s, x,
                                       C, q, sc, cm);
                return kname("k_quant_row", DT, FP8, CM);
            }
            hipLaunchKernelGGL((k_quant_row_2pass<DT, FP8, CM>), dim3((unsigned)R), dim3(256), 0, s, x, C, q, sc, cm);
            return kname("k_quant_row_2pass", DT, FP8, CM);
        case G_ROW_G128: {
            const int64_t chunks = R * (C >> 3);
            hipLaunchKernelGGL((k_quant_g128<DT, FP8, CM>), dim3((unsigned)((chunks + 255) / 256)), dim3(256),
                               0, s, x, chunks, q, sc, cm, C);
            return kname("k_quant_g128", DT, FP8, CM);
        }
        case G_BLOCK128:
            hipLaunchKernelGGL((k_quant_block128<DT, FP8, CM>), dim3((unsigned)((R >> 7) * (C >> 7))), dim3(256),
                               0, s, x, C, q, sc, cm);
            return kname("k_quant_block128", DT, FP8, CM);
        default: {
            const int64_t chunks = R * (C >> 3);
            hipLaunchKernelGGL(k_clear_amax, dim3(1), dim3(1), 0, s, sc);
            hipLaunchKernelGGL((k_amax_tensor<DT, CM>), dim3(grid_for(chunks, TU_AMAX, AMAX_GRID)), dim3(256), 0, s, x,
                               chunks, sc, cm, C);
            hipLaunchKernelGGL((k_quant_tensor<DT, FP8, CM>), dim3(grid_for(chunks, TU, 256 * 8)), dim3(256), 0, s,
                               x, chunks, q, sc, cm, C);
            return kname("k_quant_tensor", DT, FP8, CM);
        }
    }
}

template <bool FP8, bool CM>
static const char* launch_fp(const void* x, int dt, int64_t R, int64_t C, int gran, void* q, float* scales,
                             const float* cm, hipStream_t s) {
    if (dt == DT_F32) return launch_typed<DT_F32, FP8, CM>(x, R, C, gran, q, scales, cm, s);
    if (dt == DT_F16) return launch_typed<DT_F16, FP8, CM>(x, R, C, gran, q, scales, cm, s);
    return launch_typed<DT_BF16, FP8, CM>(x, R, C, gran, q, scales, cm, s);
}

const char* launch_act_quant(const void* x, int dt, int64_t R, int64_t C, int gran, bool out_fp8, void* q,
                             float* scales, const float* col_mul, hipStream_t s) {
    if (col_mul) {
        if (out_fp8) return launch_fp<true, true>(x, dt, R, C, gran, q, scales, col_mul, s);
        return launch_fp<false, true>(x, dt, R, C, gran, q, scales, col_mul, s);
    }
    if (out_fp8) return launch_fp<true, false>(x, dt, R, C, gran, q, scales, nullptr, s);
    return launch_fp<false, false>(x, dt, R, C, gran, q, scales, nullptr, s);
}

}  // namespace bg
