// bg_w4.h -- INT4 weight helpers shared by the W4A16 and W4A8 kernels (device only).
//
// A nibble u OR-ed into the mantissa of the constant MV (BF16 128.0, FP16
// 1024.0: the binade where one ulp is 1) is the exact 16-bit value MV + u.
// Packed word j of a weight row holds k = 8j .. 8j+7, even k in the low
// half-word and odd k in the high one, so (w >> 4p) & 0x000F000F | MV is the
// pair (MV + u[8j+2p], MV + u[8j+2p+1]).
#pragma once
#include "bg_device.h"

namespace bg {

template <bool BF16>
struct W4Magic;
template <>
struct W4Magic<true> {
    static constexpr uint32_t bits = 0x43004300u;  // BF16 128.0 in both halves
    static constexpr float value = 128.0f;
    static constexpr uint32_t ones = 0x3F803F80u;  // BF16 1.0 pair
};
template <>
struct W4Magic<false> {
    static constexpr uint32_t bits = 0x64006400u;  // FP16 1024.0 in both halves
    static constexpr float value = 1024.0f;
    static constexpr uint32_t ones = 0x3C003C00u;  // FP16 1.0 pair
};

// dot2 of two packed 16-bit pairs into an FP32 accumulator.
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                               __builtin_bit_cast(bf162_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                      false);
}

// (a & b) | c in one instruction: v_bitop3_b32 with the truth table of
// (A & B) | C over the operand constants A = 0xF0, B = 0xCC, C = 0xAA.  A
// builtin rather than inline assembly, so the compiler sees the VGPR write
// and keeps the wait states an MFMA reading it needs.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, (0xF0 & 0xCC) | 0xAA);
}

// The four (MV+u[2p], MV+u[2p+1]) pairs of one packed word: 3 shifts + 4 and_or.
template <bool BF16>
__device__ __forceinline__ void dequant_word(uint32_t w, uint32_t D[4]) {
    constexpr uint32_t m = W4Magic<BF16>::bits;
    D[0] = and_or(w, 0x000F000Fu, m);
    D[1] = and_or(w >> 4, 0x000F000Fu, m);
    D[2] = and_or(w >> 8, 0x000F000Fu, m);
    D[3] = and_or(w >> 12, 0x000F000Fu, m);
}

// Words lo, hi (consecutive in a slot) -> their four pairs each.  Plain
// shifts the compiler sees: it keeps the wait states around the matrix
// cores (an MFMA reads its accumulator input and writes its result several
// cycles after issue), which it cannot do for a VALU instruction hidden in
// inline assembly.
template <bool BF16>
__device__ __forceinline__ void dequant_pair(uint32_t lo, uint32_t hi, uint32_t Dlo[4], uint32_t Dhi[4]) {
    dequant_word<BF16>(lo, Dlo);
    dequant_word<BF16>(hi, Dhi);
}

// The 16 pairs of a lane's 16-byte slot: D[kk][p] = pair p of word kk.
template <bool BF16>
__device__ __forceinline__ void dequant_tile(const uint4& w, uint32_t D[4][4]) {
    dequant_pair<BF16>(w.x, w.y, D[0], D[1]);
    dequant_pair<BF16>(w.z, w.w, D[2], D[3]);
}

// Difference of two FP16 pairs (one v_pk_add_f16 with negation).
__device__ __forceinline__ uint32_t sub_h2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b));
}

template <bool BF16>
__device__ __forceinline__ float4_t mfma16(const uint32_t a[4], const uint32_t b[4], float4_t c) {
    const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
    const uint4 bv = make_uint4(b[0], b[1], b[2], b[3]);
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, av), __builtin_bit_cast(bf168_t, bv),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), __builtin_bit_cast(half8_t, bv),
                                                      c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_out(float v) {
    return BF16 ? f32_to_bf16(v) : f32_to_f16(v);
}

// The 16 signed bytes u - z of two packed words (k in order), z folded into
// zc = 0x80808080 - z * 0x01010101: (u + 0x80 - z) per byte never carries,
// and flipping bit 7 makes it the two's complement of u - z.  A word holds
// its even k in the low nibbles and its odd k in the high ones; two byte
// permutes put them back in k order.
__device__ __forceinline__ int4_t w4_to_i8(uint2 wp, uint32_t zc) {
    uint32_t d[4];
    const uint32_t w2[2] = {wp.x, wp.y};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const uint32_t lo = w2[p] & 0x0F0F0F0Fu;            // bytes: k0 k4 k1 k5
        const uint32_t hi = (w2[p] >> 4) & 0x0F0F0F0Fu;     // bytes: k2 k6 k3 k7
        d[2 * p] = (__builtin_amdgcn_perm(hi, lo, 0x06040200u) + zc) ^ 0x80808080u;      // k0 k1 k2 k3
        d[2 * p + 1] = (__builtin_amdgcn_perm(hi, lo, 0x07050301u) + zc) ^ 0x80808080u;  // k4 k5 k6 k7
    }
    return int4_t{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
}

}  // namespace bg
