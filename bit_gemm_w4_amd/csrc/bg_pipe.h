// bg_pipe.h -- building blocks of the LDS-pipelined GEMM kernels (device only).
//
// Global -> LDS copies use buffer_load_dwordx4 ... lds: lane i of a wave
// writes 16 bytes at dst + 16 i (dst is wave-uniform), so a swizzled LDS
// layout is produced by choosing which global chunk each lane fetches.  Rows
// past the end of a buffer resource read as zero.
//
// The compiler cannot tell which of those copies an LDS read depends on and
// would wait for all copies in flight before any LDS read, so operand reads
// are inline assembly and the kernels order everything themselves:
// s_waitcnt vmcnt(n) (own copies landed) + block barrier (everyone's), then
// reads; s_waitcnt lgkmcnt(0) + settle() before the values are used (settle
// passes a value through an empty asm so no consumer moves above the wait).
#pragma once
#include "bg_device.h"

namespace bg {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from a buffer resource into LDS: lane i writes dst + 16 i.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint8_t* dst, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int4_t ds_read16(uint32_t addr) {
    int4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint2 ds_read8(uint32_t addr) {
    uint2 v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
// An LDS read issued right after MFMAs: an MFMA keeps reading its source
// registers for several cycles after issue, and the compiler does not see an
// inline-asm load as a register write it must keep clear of them, so the
// operands of the last two MFMAs are passed in as inputs and the result is
// early-clobber -- it can never be allocated over them.  (Callers place a
// scheduling barrier between an MFMA and the reads that follow it, so no
// read moves above its MFMA.)
__device__ __forceinline__ int4_t ds_read16_after(uint32_t addr, const int4_t& a1, const int4_t& b1,
                                                  const int4_t& a0, const int4_t& b0) {
    int4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ int4_t ds_read16_after(uint32_t addr, const int8_t_v& a1, const int8_t_v& b1,
                                                  const int8_t_v& a0, const int8_t_v& b0) {
    int4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint2 ds_read8_after(uint32_t addr, const int4_t& a1, const int4_t& b1, const int4_t& a0,
                                                const int4_t& b0) {
    uint2 v;
    asm volatile("ds_read_b64 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read4_after(uint32_t addr, const int4_t& a1, const int4_t& b1,
                                                   const int4_t& a0, const int4_t& b0) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read4_after(uint32_t addr, const int8_t_v& a1, const int8_t_v& b1,
                                                   const int8_t_v& a0, const int8_t_v& b0) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read1_after(uint32_t addr, const int8_t_v& a1, const int8_t_v& b1,
                                                   const int8_t_v& a0, const int8_t_v& b0) {
    uint32_t v;
    asm volatile("ds_read_u8 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read1_after(uint32_t addr, const int4_t& a1, const int4_t& b1,
                                                   const int4_t& a0, const int4_t& b0) {
    uint32_t v;
    asm volatile("ds_read_u8 %0, %1" : "=&v"(v) : "v"(addr), "v"(a1), "v"(b1), "v"(a0), "v"(b0) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read1(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t ds_read4(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void settle(T& v) {
    asm volatile("" : "+v"(v));
}

// Tile of block b for a grid of tiles_m x tiles_n tiles.  Blocks are dealt
// round-robin to the 8 XCDs, so b is first remapped to (b % 8) * (nt / 8) +
// b / 8 (when nt % 8 == 0), giving each XCD a contiguous run of tiles; runs
// are ordered in bands of GROUP_M row tiles, so the blocks resident on one
// XCD share row tiles and column tiles in its L2.  GROUP_M = 1 (row-major
// runs: an XCD's resident blocks share one row tile) suits kernels whose
// activation tile is many times their weight tile.
template <int GROUP_M = 8>
__device__ __forceinline__ void grouped_tile(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nt = tiles_m * tiles_n;
    if (nt % 8 == 0) b = (b % 8) * (nt / 8) + b / 8;
    const int band = b / (GROUP_M * tiles_n);
    const int local = b - band * GROUP_M * tiles_n;
    const int first_m = band * GROUP_M;
    const int gsz = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    tm = first_m + local % gsz;
    tn = local / gsz;
}

}  // namespace bg
