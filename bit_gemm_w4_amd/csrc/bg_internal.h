// bg_internal.h -- host-side launchers behind the C ABI (not exported).
// Every launcher returns the name of the kernel it enqueued (the template
// instance, as profilers print it) and assumes its arguments were validated by the C-ABI layer
// (shapes, alignment, dtypes) and only enqueues kernels on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <type_traits>

namespace bg {

// "base<a, b, ...>" for a kernel template instance (bools print as true/false,
// as demangled names do).  Returns a thread-local buffer overwritten by the
// next call on the same thread.
template <typename... A>
const char* kname(const char* base, A... a) {
    thread_local char buf[160];
    int n = std::snprintf(buf, sizeof buf, "%s<", base);
    bool first = true;
    auto put = [&](auto v) {
        const char* sep = first ? "" : ", ";
        first = false;
        if constexpr (std::is_same_v<decltype(v), bool>)
            n += std::snprintf(buf + n, sizeof buf - n, "%s%s", sep, v ? "true" : "false");
        else
            n += std::snprintf(buf + n, sizeof buf - n, "%s%d", sep, (int)v);
    };
    (put(a), ...);
    std::snprintf(buf + n, sizeof buf - n, ">");
    return buf;
}

// w4_pack: N x K weights of dtype dt (0 f32, 1 f16, 2 bf16).
const char* launch_w4_pack(const void* w, int dt, int64_t N, int64_t K, bool asym,
                    uint32_t* qweight, uint16_t* scales, uint8_t* zeros, hipStream_t s);

// act_quant: out_fp8 selects E4M3 (else INT8); gran = bg_gran value; col_mul
// (C floats, or NULL) multiplies column j by col_mul[j] before quantizing.
const char* launch_act_quant(const void* x, int dt, int64_t R, int64_t C, int gran, bool out_fp8,
                             void* q, float* scales, const float* col_mul, hipStream_t s);

// W4A16 kernels (x_bf16: activations/output are BF16, else FP16).
// The VALU GEMV stages up to 4 activation rows of length K in LDS.
bool w4a16_gemv_supported(int64_t M, int64_t K);
// The small-M kernels stage the block's group scales and zero-points in LDS
// for all of K: they take K up to this bound (larger K goes to the tiled kernel).
constexpr int64_t kW4DecodeMaxK = 65536;
const char* launch_w4a16_gemv(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                       const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s);
const char* launch_w4a16_skinny(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                         const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s);
// Split-K small-M kernel (M <= 64): needs a workspace of
// w4a16_splitk_workspace(M, N, K) bytes (0: none), any contents; enqueues
// the partial-product kernel and, when K is split, the reduction kernel.
int64_t w4a16_splitk_workspace(int64_t M, int64_t N, int64_t K);
const char* launch_w4a16_splitk(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                                const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws,
                                hipStream_t s);
const char* launch_w4a16_tiled(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                        const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, hipStream_t s);
// Large-M LDS-pipelined kernel (k_w4a16_gemm.hip).  With a workspace (ws
// non-NULL, at least w4a16_gemm_split(M, N, K).ws_bytes, any contents) K is
// split into S slices when the output tiles do not fill the device; the FP32
// partials are then summed by a second kernel on the same stream.
struct W4GemmSplit {
    int S, gs;              // slices, groups per slice
    int64_t ws_bytes;       // S * M * N * 4 when S > 1, else 0
};
W4GemmSplit w4a16_gemm_split(int64_t M, int64_t N, int64_t K);
// Sum of S FP32 partial outputs ws[S][M][N] in slice order -> y (BF16 or FP16).
void launch_w4a16_gemm_reduce(bool bf16, const float* ws, int S, int64_t M, int64_t N, void* y, hipStream_t s);
// Mid-batch kernel (k_w4a16_mid.hip, 17 <= M <= 128 intended; any M works):
// one wide N slab per block, the activation group staged once per block.
// With a workspace (ws non-NULL, at least w4a16_mid_workspace(M, N, K)
// bytes, any contents) K is split when one slice does not fill the device.
int64_t w4a16_mid_workspace(int64_t M, int64_t N, int64_t K);
const char* launch_w4a16_mid(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                             const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s);
const char* launch_w4a16_gemm(const void* x, bool x_bf16, int64_t M, int64_t K, const uint32_t* qw,
                              const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, void* ws, hipStream_t s);

// MXFP8 quantizer: E4M3 codes [R][C] and E8M0 scales [C/32][R rounded up to
// 16] (C % 32 == 0).
// LLM.int8() outlier channels of x [R][C] (C % 8 == 0): idx / count, and the
// 0 / 1 column multiplier (in ws) for the per-token quantizer.
int64_t outlier_ws_bytes(int64_t R, int64_t C);
const char* launch_outlier_detect(const void* x, int dt, int64_t R, int64_t C, float tau, float* ws, int32_t* idx,
                                  int32_t* count, const float** mask_out, hipStream_t s);

const char* launch_quant_mx32(const void* x, int dt, int64_t R, int64_t C, bool fp4, uint8_t* q, uint8_t* e8m0,
                              hipStream_t s);

// W8A8: in_fp8 selects E4M3 x E4M3 (else INT8 x INT8); out_dt: 0 f32, 1 f16, 2 bf16, 5 i32.
// a_gran = w_gran = 4 (MX32, FP8 only): a_scales / w_scales point to E8M0
// bytes [K/32][rows rounded up to 16], applied by the MFMA; no K split.
// block_scaled: a_gran = ROW_G128 and w_gran = BLOCK128 (FP8 only).
struct W8A8Args {
    const void* a;
    const float* a_scales;
    int a_gran;
    const void* w;
    const float* w_scales;
    int w_gran;
    bool in_fp8;
    int64_t M, N, K;
    void* y;
    int out_dt;
    // LLM.int8() side path (INT8 only, no K split): x [M][K] in ox_dt, the
    // outlier columns oidx[0 .. *ocnt) (device memory)
    const void* ox = nullptr;
    int ox_dt = 0;
    const int32_t* oidx = nullptr;
    const int32_t* ocnt = nullptr;
};
// Large-M W8A8 tile shape and K split.  With a workspace (at least ws_bytes,
// any contents) grids of less than one round split K into S slices of spl
// 64-byte stages; the partials are then summed (and scaled) by a second
// kernel on the same stream.
struct W8Split {
    int bm, bn, S, spl;
    int64_t ws_bytes;
};
W8Split w8a8_tiled_split(const W8A8Args& args, bool with_ws);
const char* launch_w8a8_tiled(const W8A8Args& args, void* ws, hipStream_t s);
const char* launch_w8a8_skinny(const W8A8Args& args, hipStream_t s);

// W4A8: INT8 activation codes a [M][K] with per-row (a_row) or per-tensor
// scales, packed INT4 weights; out_dt: 0 f32, 1 f16, 2 bf16.  With a
// workspace (non-NULL, at least w4a8_gemm_split(M, N, K).ws_bytes, any
// contents) K is split into S slices when the output tiles do not fill the
// device; a second kernel on the same stream sums the FP32 partials.
W4GemmSplit w4a8_gemm_split(int64_t M, int64_t N, int64_t K);
// W4A8 at M <= 16 (k_w4a8_decode): whether the activation rows and the
// waves' scale records fit its LDS budget, and the launch (no workspace).
bool w4a8_decode_fits(int64_t M, int64_t N, int64_t K);
const char* launch_w4a8_decode(const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K, const uint32_t* qw,
                               const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, int out_dt, hipStream_t s);
const char* launch_w4a8_gemm(const int8_t* a, const float* as, bool a_row, int64_t M, int64_t K, const uint32_t* qw,
                             const uint16_t* sc, const uint8_t* zr, int64_t N, void* y, int out_dt, void* ws,
                             hipStream_t s);

}  // namespace bg
