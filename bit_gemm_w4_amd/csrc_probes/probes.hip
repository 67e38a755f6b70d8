// probes.hip -- microbenchmarks of the device's own rates, used to read the
// kernels' measurements: matrix-core throughput per MFMA shape, LDS read
// bandwidth, and streaming throughput from L2 and from the last-level cache
// into registers or straight into LDS.  Not part of the library; built into
// its own shared object by bit_gemm_w4_amd/probes.py.
//
// Every kernel touches only its output array (one value per thread) and, for
// the streaming probe, an input buffer addressed through a buffer resource
// whose range is the buffer's size.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_v __attribute__((ext_vector_type(8)));
typedef int int16_t_v __attribute__((ext_vector_type(16)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

enum { P_BF16_16 = 0, P_BF16_32 = 1, P_I8_16 = 2, P_I8_32 = 3, P_F8_16 = 4, P_F8_32 = 5, P_F32_16 = 6 };

// NACC independent accumulator chains per wave, `iters` rounds of one MFMA each.
template <int KIND, int NACC>
__global__ __launch_bounds__(256) void k_mfma(float* out, int iters, int seed) {
    float4_t f4[NACC];
    float16_t f16[NACC];
    int4_t i4[NACC];
    int16_t_v i16[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) f4[i] = float4_t{}, f16[i] = float16_t{}, i4[i] = int4_t{}, i16[i] = int16_t_v{};
    int8_t_v av, bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) av[e] = seed + e + (int)threadIdx.x, bv[e] = 3 * seed + e;
    const int4_t a4 = int4_t{av[0], av[1], av[2], av[3]}, b4 = int4_t{bv[0], bv[1], bv[2], bv[3]};
    const bf168_t ab = __builtin_bit_cast(bf168_t, a4), bb = __builtin_bit_cast(bf168_t, b4);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            if constexpr (KIND == P_BF16_16) f4[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, f4[i], 0, 0, 0);
            else if constexpr (KIND == P_BF16_32) f16[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, f16[i], 0, 0, 0);
            else if constexpr (KIND == P_I8_16) i4[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a4, b4, i4[i], 0, 0, 0);
            else if constexpr (KIND == P_I8_32) i16[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, i16[i], 0, 0, 0);
            else if constexpr (KIND == P_F8_16)
                f4[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f4[i], 0, 0, 0, 0, 0, 0);
            else if constexpr (KIND == P_F8_32)
                f16[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, f16[i], 0, 0, 0, 0, 0, 0);
            else f4[i] = __builtin_amdgcn_mfma_f32_16x16x4f32((float)seed, (float)it, f4[i], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) s += f4[i][0] + f16[i][0] + (float)i4[i][0] + (float)i16[i][0];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

// LDS read bandwidth: 16 bytes per lane per ds_read_b128, conflict-free
// addresses, eight reads per round.
__global__ __launch_bounds__(256) void k_lds(float* out, int iters) {
    __shared__ __attribute__((aligned(16))) uint4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
    __syncthreads();
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 v = buf[(threadIdx.x + u * 256 + (it & 7) * 64) & 4095];
            acc.x ^= v.x, acc.y += v.y, acc.z ^= v.z, acc.w += v.w;
        }
    }
    out[blockIdx.x * 256 + threadIdx.x] = (float)(acc.x + acc.y + acc.z + acc.w);
}

// Streaming: each wave reads 1 KB pieces (16 bytes per lane) of `src`, DEPTH
// pieces in flight, either into registers or by buffer_load ... lds into a
// wave-private LDS ring.  Pieces advance by a stride coprime to the piece
// count, so every read stays inside the buffer.
template <bool TO_LDS, int DEPTH>
__global__ __launch_bounds__(256) void k_stream(const uint8_t* src, int64_t nbytes, float* out, int iters) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * DEPTH * 1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, (int)nbytes, 0x00020000);
    const int64_t pieces = nbytes >> 10;
    int64_t p = ((int64_t)blockIdx.x * 4 + wave) * 977 % pieces;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
        uint4 r[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int off = (int)(p << 10) + lane * 16;
            if constexpr (TO_LDS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + (wave * DEPTH + d) * 1024), 16, off, 0, 0, 0);
            else
                r[d] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            p += 13;
            if (p >= pieces) p -= pieces;
        }
        if constexpr (TO_LDS) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) acc.x ^= r[d].x, acc.y += r[d].y;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (TO_LDS) acc.x ^= *reinterpret_cast<const uint32_t*>(lds + wave * DEPTH * 1024 + lane * 16);
    out[blockIdx.x * 256 + threadIdx.x] = (float)(acc.x + acc.y);
}

// An empty kernel: what a launch costs by itself (replayed in a graph).
__global__ void k_empty() {}

// Reads nbytes once and nothing else: thread t of T takes the 16-byte chunks
// t, t + T, t + 2T, ..., RD of them in flight; chunks past the end read
// zeros through the buffer resource (no memory access).  TAG only gives the
// layers their own kernel names in a trace.
template <int TAG, int RD>
__global__ __launch_bounds__(256) void k_read_once(const uint8_t* src, int64_t nbytes, float* out) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, (int)nbytes, 0x00020000);
    const int64_t nchunk = nbytes >> 4, T = (int64_t)gridDim.x * 256;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int64_t c = t; c < nchunk; c += RD * T) {
        uint4 r[RD];
#pragma unroll
        for (int u = 0; u < RD; ++u) {
            const int64_t cc = c + u * T;
            r[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, cc < nchunk ? (int)(cc << 4) : (int)0x80000000u, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < RD; ++u) acc.x ^= r[u].x, acc.y += r[u].y, acc.z ^= r[u].z, acc.w += r[u].w;
    }
    out[t] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

extern "C" {
// out: blocks * 256 floats; nacc: 1, 2, 4 or 8 independent accumulator chains
// per wave (other values: 4).  Returns 0, or 1 for an unknown kind.
int probe_mfma(int kind, int nacc, float* out, int blocks, int iters, hipStream_t s) {
#define PM(K)                                                                                           \
    if (kind == K) {                                                                                    \
        if (nacc == 8) hipLaunchKernelGGL((k_mfma<K, 8>), dim3(blocks), dim3(256), 0, s, out, iters, 1); \
        else if (nacc == 2) hipLaunchKernelGGL((k_mfma<K, 2>), dim3(blocks), dim3(256), 0, s, out, iters, 1); \
        else if (nacc == 1) hipLaunchKernelGGL((k_mfma<K, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 1); \
        else hipLaunchKernelGGL((k_mfma<K, 4>), dim3(blocks), dim3(256), 0, s, out, iters, 1);         \
        return 0;                                                                                       \
    }
    PM(P_BF16_16) PM(P_BF16_32) PM(P_I8_16) PM(P_I8_32) PM(P_F8_16) PM(P_F8_32) PM(P_F32_16)
#undef PM
    return 1;
}
int probe_lds(float* out, int blocks, int iters, hipStream_t s) {
    hipLaunchKernelGGL(k_lds, dim3(blocks), dim3(256), 0, s, out, iters);
    return 0;
}
int probe_empty(hipStream_t s) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    return 0;
}
// nbytes: a multiple of 16, below 2^31; out: blocks * 256 floats; tag 0..3;
// depth (loads in flight per thread) 4, 8, 16 or 32.
int probe_read_once(int tag, int depth, const void* src, int64_t nbytes, float* out, int blocks, hipStream_t s) {
    if (nbytes < 16 || nbytes >= ((int64_t)1 << 31) || (nbytes & 15) || tag < 0 || tag > 3) return 1;
    if (depth != 4 && depth != 8 && depth != 16 && depth != 32) return 1;
    const uint8_t* p = static_cast<const uint8_t*>(src);
#define PR(T, D)                                                                                        \
    if (tag == T && depth == D) hipLaunchKernelGGL((k_read_once<T, D>), dim3(blocks), dim3(256), 0, s, p, nbytes, out);
#define PRT(T) PR(T, 4) PR(T, 8) PR(T, 16) PR(T, 32)
    PRT(0) PRT(1) PRT(2) PRT(3)
#undef PRT
#undef PR
    return 0;
}
// nbytes: a multiple of 1024, below 2^31.
int probe_stream(int to_lds, const void* src, int64_t nbytes, float* out, int blocks, int iters, hipStream_t s) {
    if (nbytes < 1024 || nbytes >= ((int64_t)1 << 31) || (nbytes & 1023)) return 1;
    const uint8_t* p = static_cast<const uint8_t*>(src);
    if (to_lds) hipLaunchKernelGGL((k_stream<true, 16>), dim3(blocks), dim3(256), 0, s, p, nbytes, out, iters);
    else hipLaunchKernelGGL((k_stream<false, 16>), dim3(blocks), dim3(256), 0, s, p, nbytes, out, iters);
    return 0;
}
}
