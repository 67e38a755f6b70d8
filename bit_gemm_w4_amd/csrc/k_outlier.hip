// k_outlier.hip -- outlier channels of the LLM.int8() side path.
//
// "Low-precision LLM inference", §16 (Mixed-precision Outlier Path): outlier
// feature channels take a higher-precision path and the remaining channels
// the INT8 GEMM.  An outlier channel is an input column j whose largest
// magnitude over the rows reaches the threshold tau.  Three kernels find
// them without atomics or hipMemset (so the sequence can be captured):
//   k_colmax_part    column maxima of row slices, [S][C] partials;
//   k_colmax_mask    the maximum over the slices, compared with tau, as a
//                    column multiplier: 0 on outlier columns, 1 elsewhere;
//   k_outlier_list   one block: the outlier columns in increasing order and
//                    their count.
// The per-token INT8 quantizer then runs with that multiplier (the outlier
// columns quantize to 0 and drop out of the row maxima), and the GEMM adds
// the side path over the listed columns.
#include "bg_device.h"
#include "bg_internal.h"

namespace bg {

#pragma clang fp contract(off)

constexpr int CM_THREADS = 128;                 // threads per column-maximum block, 8 columns each

// Column maxima of rows [y * rps, min(R, (y + 1) * rps)): thread t of block
// (x, y) owns columns 8 (128 x + t) .. + 7 (C % 8 == 0).
template <int DT>
__global__ __launch_bounds__(CM_THREADS) void k_colmax_part(const void* __restrict__ x, int64_t R, int64_t C,
                                                             int64_t rps, float* __restrict__ part) {
    const int64_t c8 = (int64_t)blockIdx.x * CM_THREADS + threadIdx.x;
    if (c8 * 8 >= C) return;
    const int64_t r0 = (int64_t)blockIdx.y * rps, r1 = r0 + rps < R ? r0 + rps : R;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t r = r0;
    // eight rows' loads in flight per step
    for (; r + 8 <= r1; r += 8) {
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) load8_f32<DT>(x, (r + u) * C + c8 * 8, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[u][i]));
    }
    for (; r < r1; ++r) {
        float v[8];
        load8_f32<DT>(x, r * C + c8 * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[i]));
    }
    float4* out = reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * C + c8 * 8);
    out[0] = make_float4(m[0], m[1], m[2], m[3]);
    out[1] = make_float4(m[4], m[5], m[6], m[7]);
}

// mask[j] = 0 where max_s part[s][j] >= tau, else 1.  A block takes 64
// columns; its four waves take every fourth slice, eight loads in flight,
// and combine through LDS.
__global__ __launch_bounds__(256) void k_colmax_mask(const float* __restrict__ part, int S, int64_t C, float tau,
                                                     float* __restrict__ mask) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + lane;
    float m = 0.0f;
    if (j < C) {
        int s = wave;
        for (; s + 28 < S; s += 32) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(s + 4 * u) * C + j];
#pragma unroll
            for (int u = 0; u < 8; ++u) m = __builtin_fmaxf(m, v[u]);
        }
        for (; s < S; s += 4) m = __builtin_fmaxf(m, part[(int64_t)s * C + j]);
    }
    red[wave][lane] = m;
    __syncthreads();
    if (wave == 0 && j < C) {
        m = __builtin_fmaxf(__builtin_fmaxf(red[0][lane], red[1][lane]), __builtin_fmaxf(red[2][lane], red[3][lane]));
        mask[j] = m >= tau ? 0.0f : 1.0f;
    }
}

// One block of 1024 threads: thread t owns columns [t * per, (t + 1) * per);
// a block-wide exclusive scan of the per-thread counts gives each thread its
// first slot in idx.
__global__ __launch_bounds__(1024) void k_outlier_list(const float* __restrict__ mask, int64_t C,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ int wave_tot[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t per = (C + 1023) / 1024;
    const int64_t c0 = (int64_t)t * per, c1 = c0 + per < C ? c0 + per : C;
    int n = 0;
    for (int64_t j = c0; j < c1; ++j) n += mask[j] == 0.0f;
    // inclusive scan within the wave, then over the 16 wave totals
    int inc = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += w < wave ? wave_tot[w] : 0;
        total += wave_tot[w];
    }
    int pos = before + inc - n;
    for (int64_t j = c0; j < c1; ++j)
        if (mask[j] == 0.0f) idx[pos++] = (int32_t)j;
    if (t == 0) *count = total;
}

// Row slices: up to 128, so that a 4096-column input runs 512 blocks of
// eight 16-byte loads in flight per thread.
int outlier_slices(int64_t R) { return (int)(R < 128 ? R : 128); }

int64_t outlier_ws_bytes(int64_t R, int64_t C) { return ((int64_t)outlier_slices(R) * C + C) * 4; }

const char* launch_outlier_detect(const void* x, int dt, int64_t R, int64_t C, float tau, float* ws, int32_t* idx,
                                  int32_t* count, const float** mask_out, hipStream_t s) {
    const int S = outlier_slices(R);
    const int64_t rps = (R + S - 1) / S;
    float* part = ws;
    float* mask = ws + (int64_t)S * C;
    const dim3 grid((unsigned)((C / 8 + CM_THREADS - 1) / CM_THREADS), (unsigned)S);
    if (dt == DT_F32)
        hipLaunchKernelGGL((k_colmax_part<DT_F32>), grid, dim3(CM_THREADS), 0, s, x, R, C, rps, part);
    else if (dt == DT_F16)
        hipLaunchKernelGGL((k_colmax_part<DT_F16>), grid, dim3(CM_THREADS), 0, s, x, R, C, rps, part);
    else
        hipLaunchKernelGGL((k_colmax_part<DT_BF16>), grid, dim3(CM_THREADS), 0, s, x, R, C, rps, part);
    hipLaunchKernelGGL(k_colmax_mask, dim3((unsigned)((C + 63) / 64)), dim3(256), 0, s,
                       static_cast<const float*>(part), S, C, tau, mask);
    hipLaunchKernelGGL(k_outlier_list, dim3(1), dim3(1024), 0, s, static_cast<const float*>(mask), C, idx, count);
    *mask_out = mask;
    return kname("k_colmax_part", dt);
}

}  // namespace bg
