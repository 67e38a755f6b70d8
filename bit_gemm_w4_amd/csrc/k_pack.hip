// k_pack.hip -- INT4 group quantizer + nibble packer (w4_pack).
//
// "Low-precision LLM inference", §2 eq. (1) q = clamp(round(x/s)+z, qmin, qmax),
// eq. (2) x^ = s(q-z); §3 symmetric s = max|x|/qmax (eq. 3), asymmetric from the
// observed min/max; §4 one scale per group of 128 along K; §5 FP16 scales.
//
// Packed layout (tiled for the GEMM kernels): 16 output channels x one group
// of 128 k form a 1 KB tile of 64 slots x 4 words, slot = 16 * (c / 32) + n % 16
// and word = (c % 32) / 8 for c = k % 128 -- exactly the 16 bytes one MFMA
// lane consumes per group, so a wave reads each tile with one contiguous
// 1 KB load.  Inside a word, even k sit in the low half-word (nibble i <->
// k = 8j + 2i) and odd k in the high half-word (nibble 4+i <-> k = 8j + 2i + 1),
// so one mask per nibble pair yields two consecutive-k 16-bit lanes.  Scales
// are [N/16][K/128][16] and zero-point bytes [N/16][K/256][16].
//
// One thread produces one packed word (8 consecutive k of one row); the 16
// threads of a 128-wide group are 16 consecutive lanes, so the group
// reduction is a 4-step xor shuffle and no LDS is needed.  A 256-thread
// block covers 16 groups.  The kernel is HBM-bound (reads 4 or 2 bytes and
// writes 0.5 byte per weight) and runs once per weight tensor, offline.
#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

#pragma clang fp contract(off)

// FP16 bit pattern of the group scale: RNE of v, 1.0 for an all-zero group,
// clamped into [2^-24, 65504] so that the codes are always finite.
__device__ __forceinline__ uint16_t group_scale_bits(float v, bool all_zero) {
    if (all_zero) return 0x3C00u;
    uint16_t h = f32_to_f16(v);
    if (h == 0) h = 1;
    if (h == 0x7C00u) h = 0x7BFFu;
    return h;
}

// bit offset of k = 8j + i inside word j
__device__ __forceinline__ constexpr int nibble_shift(int i) { return (i & 1) ? 16 + 4 * (i >> 1) : 4 * (i >> 1); }

template <int DT, bool ASYM>
__global__ __launch_bounds__(256) void k_w4_pack(const void* __restrict__ w, int64_t N, int64_t K,
                                                 uint32_t* __restrict__ qweight,
                                                 uint16_t* __restrict__ scales,
                                                 uint8_t* __restrict__ zeros) {
    const int64_t words_per_row = K >> 3;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= N * words_per_row) return;   // whole 32-lane halves exit together
    const int64_t n = tid / words_per_row;
    const int64_t j = tid - n * words_per_row;
    const int64_t g = j >> 4;               // group of 128 = 16 words
    const int64_t ngroups = K >> 7;
    const int64_t t = n >> 4, r = n & 15;
    const int c = (int)(j & 15) * 8;        // k offset inside the group
    const int64_t out_word = ((t * ngroups + g) * 64 + 16 * (c >> 5) + r) * 4 + ((c & 31) >> 3);
    float v[8];
    load8_f32<DT>(w, n * K + j * 8, v);

    uint32_t word = 0;
    if constexpr (!ASYM) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        amax = wave_max<16>(amax);
        const uint16_t sh = group_scale_bits(amax / 7.0f, amax == 0.0f);
        const float s = f16_to_f32(sh);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float q = __builtin_rintf(v[i] / s);
            q = __builtin_fminf(__builtin_fmaxf(q, -8.0f), 7.0f);
            word |= (uint32_t)((int)q + 8) << nibble_shift(i);
        }
        if ((j & 15) == 0) scales[(t * ngroups + g) * 16 + r] = sh;
    } else {
        float mn = 0.0f, mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mn = __builtin_fminf(mn, v[i]);
            mx = __builtin_fmaxf(mx, v[i]);
        }
        mn = wave_min<16>(mn);
        mx = wave_max<16>(mx);
        const float range = mx - mn;
        const uint16_t sh = group_scale_bits(range / 15.0f, range == 0.0f);
        const float s = f16_to_f32(sh);
        float zf = __builtin_rintf(-mn / s);
        zf = __builtin_fminf(__builtin_fmaxf(zf, 0.0f), 15.0f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float q = __builtin_rintf(v[i] / s) + zf;
            q = __builtin_fminf(__builtin_fmaxf(q, 0.0f), 15.0f);
            word |= (uint32_t)(int)q << nibble_shift(i);
        }
        // groups 2h and 2h+1 sit in lanes [32h', 32h'+16) and [32h'+16, 32h'+32)
        const uint32_t zi = (uint32_t)(int)zf;
        const uint32_t z_odd = (uint32_t)__shfl_down((int)zi, 16, 32);
        if ((j & 31) == 0) zeros[(t * (ngroups >> 1) + (g >> 1)) * 16 + r] = (uint8_t)(zi | (z_odd << 4));
        if ((j & 15) == 0) scales[(t * ngroups + g) * 16 + r] = sh;
    }
    qweight[out_word] = word;
}

template <int DT>
static const char* launch_dt(const void* w, int64_t N, int64_t K, bool asym, uint32_t* qw,
                             uint16_t* sc, uint8_t* zr, hipStream_t s) {
    const int64_t threads = N * (K >> 3);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (asym)
        hipLaunchKernelGGL((k_w4_pack<DT, true>), dim3(blocks), dim3(256), 0, s, w, N, K, qw, sc, zr);
    else
        hipLaunchKernelGGL((k_w4_pack<DT, false>), dim3(blocks), dim3(256), 0, s, w, N, K, qw, sc, zr);
    return kname("k_w4_pack", DT, asym);
}

const char* launch_w4_pack(const void* w, int dt, int64_t N, int64_t K, bool asym, uint32_t* qweight,
                           uint16_t* scales, uint8_t* zeros, hipStream_t s) {
    if (dt == DT_F32) return launch_dt<DT_F32>(w, N, K, asym, qweight, scales, zeros, s);
    if (dt == DT_F16) return launch_dt<DT_F16>(w, N, K, asym, qweight, scales, zeros, s);
    return launch_dt<DT_BF16>(w, N, K, asym, qweight, scales, zeros, s);
}

}  // namespace bg
