// bg_device.h -- device-side helpers shared by the gfx950 kernels.
//
// Number formats (see "Low-precision LLM inference", §5 FP16 scales and §7
// FP8 E4M3): FP16 / BF16 conversions are round-to-nearest-even; the E4M3
// encoder is OCP E4M3FN (bias 7, max 448) with saturation, RNE and NaN -> NaN.
// Kernels that must be bit-exact turn FP contraction off locally, so every
// float expression is one correctly rounded IEEE operation; the compiler's
// default float division on gfx950 is correctly rounded, and fp32 / fp16
// denormals are preserved (IEEE mode).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef int int16_t_v __attribute__((ext_vector_type(16)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// A buffer-load offset beyond the range of every buffer resource the kernels
// build (each well below 1 GiB, offsets included): such a load returns zeros
// without a memory access.  Software pipelines issue it for the stages past
// a wave's last unit of work.
constexpr int kBufOOB = 0x40000000;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Load 8 consecutive elements of a 16-bit or 32-bit tensor as floats (exact).
template <int DT>
__device__ __forceinline__ void load8_f32(const void* base, int64_t idx, float v[8]) {
    if constexpr (DT == DT_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DT_BF16) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            } else {
                v[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
                v[2 * i + 1] = f16_to_f32(w[i] >> 16);
            }
        }
    }
}

// Saturating RNE cast of two floats to OCP E4M3 bytes (byte 0 = a, byte 1 = b).
// The hardware converter on gfx950 produces OCP E4M3 with round-to-nearest-even;
// clamping to +-448 first makes it saturating, and NaN is selected explicitly.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    float ca = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
    float cb = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
    uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (a != a) p = (p & 0xFF00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
    if (b != b) p = (p & 0x00FFu) | (((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu) << 8;
    return p;
}

// Wave-level reductions over groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
template <int W>
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = __builtin_fminf(v, __shfl_xor(v, o, 64));
    return v;
}
template <int W>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace bg
