// capi.hip -- the exported C ABI (include/bitgemm.h): argument validation
// (fail-closed, "Low-precision LLM inference" §24 eligibility checklist and
// §31 fallback_policy) and kernel dispatch by M ("small batch and large
// prefill get different kernels", §24).  Validation touches no HIP API, so
// a rejected call never reaches the device.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/bitgemm.h"
#include "bg_internal.h"

#define BG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";
thread_local char g_last_kernel[160] = "";

void note_kernel(const char* name) {
    std::snprintf(g_last_kernel, sizeof(g_last_kernel), "%s", name ? name : "");
}

bg_status fail(bg_status st, const char* fmt, long long a = 0, long long b = 0) {
    std::snprintf(g_last_error, sizeof(g_last_error), fmt, a, b);
    return st;
}

// The same, with the entry point's name in front.
bg_status fail_in(const char* fn, bg_status st, const char* fmt, long long a = 0, long long b = 0) {
    const int n = std::snprintf(g_last_error, sizeof(g_last_error), "%s: ", fn);
    std::snprintf(g_last_error + n, sizeof(g_last_error) - n, fmt, a, b);
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bg_status launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(g_last_error, sizeof(g_last_error), "%s: launch failed: %s", what, hipGetErrorString(e));
        return BG_ERR_HIP;
    }
    g_last_error[0] = '\0';
    return BG_OK;
}

constexpr int64_t kMaxRows = int64_t(1) << 24;   // N, act_quant rows
constexpr int64_t kMaxDim = int64_t(1) << 20;    // K, cols
constexpr int64_t kMaxM = int64_t(65535) * 16;   // GEMM M: grid.y stays below 65536
constexpr int64_t kMaxGemvM = 256;               // explicit GEMV requests
constexpr int64_t kI8MaxKExcl = int64_t(1) << 17; // INT8 K bound: K * 2^14 < 2^31

// W4A16: small-M MFMA kernel up to kW4SkinnyMax rows, tiled MFMA kernel beyond;
// the VALU GEMV is selected explicitly only (BG_ALGO_GEMV).
constexpr int64_t kW4GemvMax = 0;
constexpr int64_t kW4SkinnyMax = 64;
constexpr int64_t kW8SkinnyMax = 32;

int w4_auto_algo(int64_t M, int64_t K) {
    if (K > bg::kW4DecodeMaxK) return BG_ALGO_TILED;
    if (M <= kW4GemvMax) return BG_ALGO_GEMV;
    if (M <= kW4SkinnyMax) return BG_ALGO_SKINNY;
    return BG_ALGO_TILED;
}

// W8A8: the small-M kernel streams the weights once per band of up to 64
// rows; the tiled kernel is flat in M until its 256 x 128 tiles fill the
// device. Measured on the 8B projection shapes: through M = 16 the small-M
// kernel (activations staged in LDS) wins on every shape, by 1.3-1.5x on the
// 28672-wide layer; above that the tiled grid wins once it has >= 128 tiles
// or M > 128, or M > 64 with a short K.
int w8_auto_algo(int64_t M, int64_t N, int64_t K) {
    if (M <= 16) return BG_ALGO_SKINNY;
    const int64_t tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (tiles >= 128 || M > 128) return BG_ALGO_TILED;
    if (M <= kW8SkinnyMax) return BG_ALGO_SKINNY;
    if (tiles < 48 && (M <= 64 || K >= 8192)) return BG_ALGO_SKINNY;
    return BG_ALGO_TILED;
}

// W8A8 with a workspace: the small-M kernel through M = 16, and through
// M = 32 on layers up to 4096 x 8192; beyond that the large-M kernel with K
// split wherever it measured faster than the small-M kernel on the
// projection shapes (N >= 6144, or K >= 8192, or M >= 32), else the choice
// above.
int w8_auto_algo_ws(int64_t M, int64_t N, int64_t K, int in_dtype, int a_gran) {
    if (M <= 16 || (M <= 32 && N <= 4096 && K <= 8192)) return BG_ALGO_SKINNY;
    bg::W8A8Args g{nullptr, nullptr, a_gran, nullptr, nullptr, 0, in_dtype == BG_FP8_E4M3, M, N, K, nullptr, BG_BF16};
    const bool fits = N >= 6144 || K >= 8192 || M >= 32;
    if (fits && bg::w8a8_tiled_split(g, true).S > 1) return BG_ALGO_TILED;
    return w8_auto_algo(M, N, K);
}

// Workspace bytes of a W4A16 kernel choice (0: none).
int64_t w4_ws_need(int algo, int64_t M, int64_t N, int64_t K) {
    if (algo == BG_ALGO_MID) return bg::w4a16_mid_workspace(M, N, K);
    if (algo != BG_ALGO_SPLITK) return 0;
    return M > kW4SkinnyMax ? bg::w4a16_gemm_split(M, N, K).ws_bytes : bg::w4a16_splitk_workspace(M, N, K);
}

// With a workspace, small M runs split-K where the small-M kernel's per-block
// re-staging of the activation rows costs more than split-K's cross-block
// reduction: from the measured crossovers (graph-replayed, cold weights) on
// the 4096/14336-wide projection shapes (N = 6144 and 4096 at K = 4096 stay
// on the small-M kernel through M = 16).
// Past the small-M range, split-K (of the large-M kernel) while its output
// tiles do not fill the device.
int w4_auto_algo_ws(int64_t M, int64_t N, int64_t K) {
    // mid-batch kernel: measured faster than the split small-M and the tiled
    // kernels on the projection shapes past M = 16 on the 28672-wide layer
    // (24.7 against 27.3 us at M = 24) and from M = 64 on the others, through
    // M = 128 (the tiled kernel wins again at M = 256)
    if (M <= 128 && (M >= 64 || (M > 16 && N >= 16384))) return BG_ALGO_MID;
    if (M > kW4SkinnyMax) return bg::w4a16_gemm_split(M, N, K).S > 1 ? BG_ALGO_SPLITK : BG_ALGO_TILED;
    // (measured: down, K = 14336, is faster split at every M >= 8; gate_up,
    // N = 28672, is faster unsplit through M = 16 -- 19.2-19.8 us against
    // 20.6-21.7 -- since the small-M kernel deals its tiles in one round)
    const bool split = (M >= 8 && K >= 8192) || (M > 16 && N > 4096) || M >= 24;
    if (split) return BG_ALGO_SPLITK;
    return K > bg::kW4DecodeMaxK ? BG_ALGO_TILED : BG_ALGO_SKINNY;
}

}  // namespace

BG_EXPORT bg_status w4_pack(const void* w, int w_dtype, int64_t N, int64_t K, int group, int asymmetric,
                            uint32_t* qweight, uint16_t* scales, uint8_t* zeros, void* stream) {
    if (!w || !qweight || !scales) return fail(BG_ERR_NULL, "w4_pack: w, qweight and scales must be non-NULL");
    if (asymmetric && !zeros) return fail(BG_ERR_NULL, "w4_pack: asymmetric packing needs a zeros buffer");
    if (!asymmetric && zeros) return fail(BG_ERR_UNSUPPORTED, "w4_pack: zeros must be NULL when symmetric");
    if (w_dtype != BG_F32 && w_dtype != BG_F16 && w_dtype != BG_BF16)
        return fail(BG_ERR_DTYPE, "w4_pack: w_dtype %lld is not F32/F16/BF16", w_dtype);
    if (group != 128) return fail(BG_ERR_UNSUPPORTED, "w4_pack: group %lld (only 128 is supported)", group);
    if (N < 16 || N > kMaxRows || N % 16) return fail(BG_ERR_SHAPE, "w4_pack: N=%lld must be a multiple of 16", N);
    if (K < 256 || K > kMaxDim || K % 256) return fail(BG_ERR_SHAPE, "w4_pack: K=%lld must be a multiple of 256", K);
    if (N * (K / 8) / 256 >= (int64_t(1) << 31)) return fail(BG_ERR_SHAPE, "w4_pack: N*K=%lld too large", N * K);
    if (!aligned16(w) || !aligned16(qweight) || !aligned16(scales) || (zeros && !aligned16(zeros)))
        return fail(BG_ERR_ALIGN, "w4_pack: pointers must be 16-byte aligned");
    note_kernel(bg::launch_w4_pack(w, w_dtype, N, K, asymmetric != 0, qweight, scales, zeros,
                       static_cast<hipStream_t>(stream)));
    return launched("w4_pack");
}

BG_EXPORT int gemm_w4a16_algo(int64_t M, int64_t N, int64_t K, int x_dtype) {
    (void)N; (void)x_dtype;
    return w4_auto_algo(M, K);
}

static bg_status w4a16_impl(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int64_t N, int group, void* y,
                            void* ws, int64_t ws_bytes, bool with_ws, int algo, void* stream) {
    if (!x || !qweight || !scales || !y) return fail(BG_ERR_NULL, "gemm_w4a16: x, qweight, scales and y must be non-NULL");
    if (x_dtype != BG_F16 && x_dtype != BG_BF16)
        return fail(BG_ERR_DTYPE, "gemm_w4a16: x_dtype %lld is not F16/BF16", x_dtype);
    if (group != 128) return fail(BG_ERR_UNSUPPORTED, "gemm_w4a16: group %lld (only 128 is supported)", group);
    if (M < 1 || M > kMaxM) return fail(BG_ERR_SHAPE, "gemm_w4a16: M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail(BG_ERR_SHAPE, "gemm_w4a16: N=%lld must be a multiple of 16", N);
    if (K < 256 || K > kMaxDim || K % 256) return fail(BG_ERR_SHAPE, "gemm_w4a16: K=%lld must be a multiple of 256", K);
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y) || (zeros && !aligned16(zeros)) ||
        (ws && !aligned16(ws)))
        return fail(BG_ERR_ALIGN, "gemm_w4a16: pointers must be 16-byte aligned");
    if (algo == BG_ALGO_AUTO) algo = with_ws ? w4_auto_algo_ws(M, N, K) : w4_auto_algo(M, K);
    if (algo == BG_ALGO_GEMV && (M > kMaxGemvM || !bg::w4a16_gemv_supported(M, K)))
        return fail(BG_ERR_SHAPE, "gemm_w4a16: the GEMV kernel takes M <= 256 and K <= 18432 (M=%lld, K=%lld)", M, K);
    if (algo == BG_ALGO_SKINNY && K > bg::kW4DecodeMaxK)
        return fail(BG_ERR_SHAPE, "gemm_w4a16: the small-M kernel takes K <= 65536 (K=%lld)", K);
    if (algo == BG_ALGO_SPLITK && !with_ws)
        return fail(BG_ERR_WORKSPACE, "gemm_w4a16: the split-K kernels need gemm_w4a16_ws");
    if (with_ws && (algo == BG_ALGO_SPLITK || algo == BG_ALGO_MID)) {
        const int64_t need = w4_ws_need(algo, M, N, K);
        if (need > 0 && (!ws || ws_bytes < need))
            return fail(BG_ERR_WORKSPACE, "gemm_w4a16: workspace of %lld bytes needed (got %lld)", need, ws ? ws_bytes : 0);
    }
    const bool bf16 = x_dtype == BG_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (algo) {
        case BG_ALGO_GEMV: note_kernel(bg::launch_w4a16_gemv(x, bf16, M, K, qweight, scales, zeros, N, y, s)); break;
        case BG_ALGO_SKINNY: note_kernel(bg::launch_w4a16_skinny(x, bf16, M, K, qweight, scales, zeros, N, y, s)); break;
        case BG_ALGO_TILED: note_kernel(bg::launch_w4a16_tiled(x, bf16, M, K, qweight, scales, zeros, N, y, s)); break;
        case BG_ALGO_MID:
            note_kernel(bg::launch_w4a16_mid(x, bf16, M, K, qweight, scales, zeros, N, y, with_ws ? ws : nullptr, s));
            break;
        case BG_ALGO_SPLITK:
            if (M > kW4SkinnyMax)
                note_kernel(bg::launch_w4a16_gemm(x, bf16, M, K, qweight, scales, zeros, N, y, ws, s));
            else
                note_kernel(bg::launch_w4a16_splitk(x, bf16, M, K, qweight, scales, zeros, N, y, ws, s));
            break;
        default: return fail(BG_ERR_UNSUPPORTED, "gemm_w4a16: unknown algo %lld", algo);
    }
    return launched("gemm_w4a16");
}

BG_EXPORT bg_status gemm_w4a16_ex(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* qweight,
                                  const uint16_t* scales, const uint8_t* zeros, int64_t N, int group, void* y,
                                  int algo, void* stream) {
    return w4a16_impl(x, x_dtype, M, K, qweight, scales, zeros, N, group, y, nullptr, 0, false, algo, stream);
}

BG_EXPORT bg_status gemm_w4a16_ws(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* qweight,
                                  const uint16_t* scales, const uint8_t* zeros, int64_t N, int group, void* y,
                                  void* workspace, int64_t workspace_bytes, int algo, void* stream) {
    return w4a16_impl(x, x_dtype, M, K, qweight, scales, zeros, N, group, y, workspace, workspace_bytes, true, algo,
                      stream);
}

BG_EXPORT int64_t gemm_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int algo) {
    if (M < 1 || M > kMaxM || N < 16 || N % 16 || K < 256 || K % 256) return 0;
    if (algo == BG_ALGO_AUTO) algo = w4_auto_algo_ws(M, N, K);
    return w4_ws_need(algo, M, N, K);
}

BG_EXPORT bg_status gemm_w4a16(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* qweight,
                               const uint16_t* scales, const uint8_t* zeros, int64_t N, int group, void* y,
                               void* stream) {
    return gemm_w4a16_ex(x, x_dtype, M, K, qweight, scales, zeros, N, group, y, BG_ALGO_AUTO, stream);
}

// ---- gemm_w4a16_noalloc: split-K partials in a static device array ----
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc).  `scratch` lives in the code
// object: every GPU that runs the library holds its own copy, at its own
// address, until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol); it uses the
// device address hipGetSymbolAddress returns, looked up once per device with
// that device current.
static __device__ __align__(256) uint8_t scratch[BG_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

bg_status hip_fail(const char* what, hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "gemm_w4a16_noalloc: %s: %s", what, hipGetErrorString(e));
    return BG_ERR_HIP;
}

// Device address of `scratch` on the device `stream` runs on, which must be
// the current device.
bg_status scratch_address(void* stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) return fail(BG_ERR_UNSUPPORTED, "gemm_w4a16_noalloc: device %lld out of range", dev);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return hip_fail("hipStreamGetDevice", e);
        if (sdev != dev)
            return fail(BG_ERR_UNSUPPORTED, "gemm_w4a16_noalloc: the stream is on device %lld, the current device is %lld",
                        sdev, dev);
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return hip_fail("hipGetSymbolAddress(scratch)", e);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BG_OK;
}

}  // namespace

BG_EXPORT bg_status gemm_w4a16_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* qweight,
                                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int group, void* y,
                                       void* stream) {
    // the shape checks of gemm_w4a16 come first, so the size asked of the
    // scratch is only computed for an eligible call
    if (!x || !qweight || !scales || !y) return fail(BG_ERR_NULL, "gemm_w4a16: x, qweight, scales and y must be non-NULL");
    if (M < 1 || M > kMaxM) return fail(BG_ERR_SHAPE, "gemm_w4a16: M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail(BG_ERR_SHAPE, "gemm_w4a16: N=%lld must be a multiple of 16", N);
    if (K < 256 || K > kMaxDim || K % 256) return fail(BG_ERR_SHAPE, "gemm_w4a16: K=%lld must be a multiple of 256", K);
    const int algo = w4_auto_algo_ws(M, N, K);
    const int64_t need = w4_ws_need(algo, M, N, K);
    if (need > BG_NOALLOC_SCRATCH_BYTES)
        return fail(BG_ERR_WORKSPACE,
                    "gemm_w4a16_noalloc: this shape needs %lld bytes of scratch; the static scratch holds %lld "
                    "(use gemm_w4a16_ws with a larger workspace)",
                    need, (long long)BG_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
        const bg_status st = scratch_address(stream, &ws);
        if (st != BG_OK) return st;
    }
    return w4a16_impl(x, x_dtype, M, K, qweight, scales, zeros, N, group, y, ws, need, true, algo, stream);
}

static bg_status act_quant(const char* name, bool fp8, const void* x, int x_dtype, int64_t rows, int64_t cols,
                           int gran, const float* col_mul, bool smooth, void* q, float* scales, void* stream) {
    if (!x || !q || !scales) return fail(BG_ERR_NULL, "act_quant: x, q and scales must be non-NULL");
    if (smooth && !col_mul) return fail(BG_ERR_NULL, "act_quant: col_mul must be non-NULL");
    if (x_dtype != BG_F32 && x_dtype != BG_F16 && x_dtype != BG_BF16)
        return fail(BG_ERR_DTYPE, "act_quant: x_dtype %lld is not F32/F16/BF16", x_dtype);
    if (gran < BG_GRAN_TENSOR || gran > BG_GRAN_BLOCK128)
        return fail(BG_ERR_UNSUPPORTED, "act_quant: unknown granularity %lld", gran);
    if (rows < 1 || rows > kMaxRows) return fail(BG_ERR_SHAPE, "act_quant: rows=%lld out of range", rows);
    if (cols < 128 || cols > kMaxDim || cols % 128)
        return fail(BG_ERR_SHAPE, "act_quant: cols=%lld must be a multiple of 128", cols);
    if (gran == BG_GRAN_BLOCK128 && rows % 128)
        return fail(BG_ERR_SHAPE, "act_quant: BLOCK128 needs rows %% 128 == 0 (rows=%lld)", rows);
    if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || (col_mul && !aligned16(col_mul)))
        return fail(BG_ERR_ALIGN, "act_quant: pointers must be 16-byte aligned");
    note_kernel(bg::launch_act_quant(x, x_dtype, rows, cols, gran, fp8, q, scales, smooth ? col_mul : nullptr,
                                     static_cast<hipStream_t>(stream)));
    return launched(name);
}

BG_EXPORT bg_status act_quant_int8(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran, int8_t* q,
                                   float* scales, void* stream) {
    return act_quant("act_quant_int8", false, x, x_dtype, rows, cols, gran, nullptr, false, q, scales, stream);
}

BG_EXPORT bg_status act_quant_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran, uint8_t* q,
                                  float* scales, void* stream) {
    return act_quant("act_quant_fp8", true, x, x_dtype, rows, cols, gran, nullptr, false, q, scales, stream);
}

BG_EXPORT bg_status act_quant_int8_smooth(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                                          const float* col_mul, int8_t* q, float* scales, void* stream) {
    return act_quant("act_quant_int8_smooth", false, x, x_dtype, rows, cols, gran, col_mul, true, q, scales, stream);
}

BG_EXPORT bg_status act_quant_fp8_smooth(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                                         const float* col_mul, uint8_t* q, float* scales, void* stream) {
    return act_quant("act_quant_fp8_smooth", true, x, x_dtype, rows, cols, gran, col_mul, true, q, scales, stream);
}

static bg_status act_quant_mx(const char* fn, bool fp4, const void* x, int x_dtype, int64_t rows, int64_t cols,
                              uint8_t* q, uint8_t* e8m0, void* stream) {
    if (!x || !q || !e8m0) return fail_in(fn, BG_ERR_NULL, "x, q and e8m0 must be non-NULL");
    if (x_dtype != BG_F32 && x_dtype != BG_F16 && x_dtype != BG_BF16)
        return fail_in(fn, BG_ERR_DTYPE, "x_dtype %lld is not F32/F16/BF16", x_dtype);
    if (rows < 1 || rows > kMaxRows) return fail_in(fn, BG_ERR_SHAPE, "rows=%lld out of range", rows);
    if (cols < 32 || cols > kMaxDim || cols % 32)
        return fail_in(fn, BG_ERR_SHAPE, "cols=%lld must be a multiple of 32", cols);
    if (!aligned16(x) || !aligned16(q)) return fail_in(fn, BG_ERR_ALIGN, "x and q must be 16-byte aligned");
    note_kernel(bg::launch_quant_mx32(x, x_dtype, rows, cols, fp4, q, e8m0, static_cast<hipStream_t>(stream)));
    return launched(fn);
}

BG_EXPORT bg_status act_quant_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                                    uint8_t* e8m0, void* stream) {
    return act_quant_mx("act_quant_mxfp8", false, x, x_dtype, rows, cols, q, e8m0, stream);
}

BG_EXPORT bg_status act_quant_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                                    uint8_t* e8m0, void* stream) {
    return act_quant_mx("act_quant_mxfp4", true, x, x_dtype, rows, cols, q, e8m0, stream);
}

// K granularity: one pair of 64-byte stages, i.e. 128 MXFP8 or 256 MXFP4 elements.
static bg_status gemm_mx(const char* fn, bool fp4, const uint8_t* a, const uint8_t* a_e8m0, const uint8_t* w,
                         const uint8_t* w_e8m0, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                         void* stream) {
    if (!a || !a_e8m0 || !w || !w_e8m0 || !y)
        return fail_in(fn, BG_ERR_NULL, "a, a_e8m0, w, w_e8m0 and y must be non-NULL");
    if (out_dtype != BG_BF16 && out_dtype != BG_F16 && out_dtype != BG_F32)
        return fail_in(fn, BG_ERR_DTYPE, "out_dtype %lld is not BF16/F16/F32", out_dtype);
    const int64_t kq = fp4 ? 256 : 128;
    const int64_t row_bytes = fp4 ? K / 2 : K;
    if (M < 1 || M > kMaxM) return fail_in(fn, BG_ERR_SHAPE, "M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail_in(fn, BG_ERR_SHAPE, "N=%lld must be a multiple of 16", N);
    if (K < kq || K > kMaxDim || K % kq)
        return fail_in(fn, BG_ERR_SHAPE, "K=%lld must be a multiple of %lld", K, kq);
    if (M * row_bytes >= (int64_t(1) << 31) || N * row_bytes >= (int64_t(1) << 31))
        return fail_in(fn, BG_ERR_SHAPE, "the A and W operands must each be below 2^31 bytes");
    if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned16(a_e8m0) || !aligned16(w_e8m0))
        return fail_in(fn, BG_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int gran = fp4 ? 5 : 4;
    bg::W8A8Args g{a, reinterpret_cast<const float*>(a_e8m0), gran, w, reinterpret_cast<const float*>(w_e8m0), gran,
                   true, M, N, K, y, out_dtype};
    note_kernel(bg::launch_w8a8_tiled(g, nullptr, static_cast<hipStream_t>(stream)));
    return launched(fn);
}

BG_EXPORT bg_status gemm_mxfp8(const uint8_t* a, const uint8_t* a_e8m0, const uint8_t* w, const uint8_t* w_e8m0,
                               int64_t M, int64_t N, int64_t K, void* y, int out_dtype, void* stream) {
    return gemm_mx("gemm_mxfp8", false, a, a_e8m0, w, w_e8m0, M, N, K, y, out_dtype, stream);
}

BG_EXPORT bg_status gemm_mxfp4(const uint8_t* a, const uint8_t* a_e8m0, const uint8_t* w, const uint8_t* w_e8m0,
                               int64_t M, int64_t N, int64_t K, void* y, int out_dtype, void* stream) {
    return gemm_mx("gemm_mxfp4", true, a, a_e8m0, w, w_e8m0, M, N, K, y, out_dtype, stream);
}

BG_EXPORT int gemm_w8a8_algo(int64_t M, int64_t N, int64_t K, int in_dtype) {
    (void)in_dtype;
    return w8_auto_algo(M, N, K);
}

static bg_status w8a8_impl(const void* a, const float* a_scales, int a_gran, const void* w, const float* w_scales,
                           int w_gran, int in_dtype, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                           void* ws, int64_t ws_bytes, bool with_ws, int algo, void* stream) {
    if (!a || !w || !y) return fail(BG_ERR_NULL, "gemm_w8a8: a, w and y must be non-NULL");
    if (in_dtype != BG_I8 && in_dtype != BG_FP8_E4M3)
        return fail(BG_ERR_DTYPE, "gemm_w8a8: in_dtype %lld is not I8/FP8_E4M3", in_dtype);
    const bool raw = out_dtype == BG_I32;
    if (raw && in_dtype != BG_I8) return fail(BG_ERR_DTYPE, "gemm_w8a8: I32 output needs I8 inputs");
    if (!raw && out_dtype != BG_BF16 && out_dtype != BG_F16 && out_dtype != BG_F32)
        return fail(BG_ERR_DTYPE, "gemm_w8a8: out_dtype %lld is not BF16/F16/F32/I32", out_dtype);
    if (!raw && (!a_scales || !w_scales)) return fail(BG_ERR_NULL, "gemm_w8a8: scales must be non-NULL");
    const bool per = (a_gran == BG_GRAN_TENSOR || a_gran == BG_GRAN_ROW) &&
                     (w_gran == BG_GRAN_TENSOR || w_gran == BG_GRAN_ROW);
    const bool block = a_gran == BG_GRAN_ROW_G128 && w_gran == BG_GRAN_BLOCK128;
    if (!raw && !per && !(block && in_dtype == BG_FP8_E4M3))
        return fail(BG_ERR_UNSUPPORTED, "gemm_w8a8: granularity pair (%lld, %lld) not supported", a_gran, w_gran);
    if (M < 1 || M > kMaxM) return fail(BG_ERR_SHAPE, "gemm_w8a8: M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail(BG_ERR_SHAPE, "gemm_w8a8: N=%lld must be a multiple of 16", N);
    if (K < 128 || K > kMaxDim || K % 128) return fail(BG_ERR_SHAPE, "gemm_w8a8: K=%lld must be a multiple of 128", K);
    // |acc| <= K * 128 * 128 must stay below 2^31: K <= 130944 (K = 131072
    // with every code at -128 would reach exactly 2^31 and wrap)
    if (in_dtype == BG_I8 && K >= kI8MaxKExcl)
        return fail(BG_ERR_SHAPE, "gemm_w8a8: K=%lld too long for exact INT32 accumulation (K < 131072)", K);
    if (block && N % 128) return fail(BG_ERR_SHAPE, "gemm_w8a8: BLOCK128 weights need N %% 128 == 0 (N=%lld)", N);
    if (!aligned16(a) || !aligned16(w) || !aligned16(y) || (a_scales && !aligned16(a_scales)) ||
        (w_scales && !aligned16(w_scales)) || (ws && !aligned16(ws)))
        return fail(BG_ERR_ALIGN, "gemm_w8a8: pointers must be 16-byte aligned");
    if (algo == BG_ALGO_AUTO) algo = with_ws ? w8_auto_algo_ws(M, N, K, in_dtype, a_gran) : w8_auto_algo(M, N, K);
    bg::W8A8Args g{a, a_scales, raw ? BG_GRAN_ROW : a_gran, w, w_scales, raw ? BG_GRAN_ROW : w_gran,
                   in_dtype == BG_FP8_E4M3, M, N, K, y, out_dtype};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (algo == BG_ALGO_TILED && with_ws) {
        const int64_t need = bg::w8a8_tiled_split(g, true).ws_bytes;
        if (need > 0 && (!ws || ws_bytes < need))
            return fail(BG_ERR_WORKSPACE, "gemm_w8a8: workspace of %lld bytes needed (got %lld)", need, ws ? ws_bytes : 0);
    }
    switch (algo) {
        case BG_ALGO_SKINNY: note_kernel(bg::launch_w8a8_skinny(g, s)); break;
        case BG_ALGO_TILED: note_kernel(bg::launch_w8a8_tiled(g, with_ws ? ws : nullptr, s)); break;
        default: return fail(BG_ERR_UNSUPPORTED, "gemm_w8a8: unknown algo %lld", algo);
    }
    return launched("gemm_w8a8");
}

BG_EXPORT bg_status gemm_w8a8_ex(const void* a, const float* a_scales, int a_gran, const void* w,
                                 const float* w_scales, int w_gran, int in_dtype, int64_t M, int64_t N, int64_t K,
                                 void* y, int out_dtype, int algo, void* stream) {
    return w8a8_impl(a, a_scales, a_gran, w, w_scales, w_gran, in_dtype, M, N, K, y, out_dtype, nullptr, 0, false,
                     algo, stream);
}

BG_EXPORT bg_status gemm_w8a8_ws(const void* a, const float* a_scales, int a_gran, const void* w,
                                 const float* w_scales, int w_gran, int in_dtype, int64_t M, int64_t N, int64_t K,
                                 void* y, int out_dtype, void* workspace, int64_t workspace_bytes, int algo,
                                 void* stream) {
    return w8a8_impl(a, a_scales, a_gran, w, w_scales, w_gran, in_dtype, M, N, K, y, out_dtype, workspace,
                     workspace_bytes, true, algo, stream);
}

BG_EXPORT int64_t gemm_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int in_dtype, int a_gran, int algo) {
    if (M < 1 || M > kMaxM || N < 16 || N > kMaxRows || N % 16 || K < 128 || K > kMaxDim || K % 128) return 0;
    if (algo == BG_ALGO_AUTO) algo = w8_auto_algo_ws(M, N, K, in_dtype, a_gran);
    if (algo != BG_ALGO_TILED) return 0;
    bg::W8A8Args g{nullptr, nullptr, a_gran, nullptr, nullptr, 0, in_dtype == BG_FP8_E4M3, M, N, K, nullptr, BG_BF16};
    return bg::w8a8_tiled_split(g, true).ws_bytes;
}

BG_EXPORT bg_status gemm_w8a8(const void* a, const float* a_scales, int a_gran, const void* w,
                              const float* w_scales, int w_gran, int in_dtype, int64_t M, int64_t N, int64_t K,
                              void* y, int out_dtype, void* stream) {
    return gemm_w8a8_ex(a, a_scales, a_gran, w, w_scales, w_gran, in_dtype, M, N, K, y, out_dtype, BG_ALGO_AUTO,
                        stream);
}

// ---- LLM.int8() outlier side path ----

BG_EXPORT int64_t act_quant_outlier_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows < 1 || rows > kMaxRows || cols < 128 || cols > kMaxDim || cols % 128) return 0;
    return bg::outlier_ws_bytes(rows, cols);
}

BG_EXPORT bg_status act_quant_int8_outlier(const void* x, int x_dtype, int64_t rows, int64_t cols, float tau,
                                           int8_t* q, float* scales, int32_t* idx, int32_t* count, void* workspace,
                                           int64_t workspace_bytes, void* stream) {
    const char* fn = "act_quant_int8_outlier";
    if (!x || !q || !scales || !idx || !count || !workspace)
        return fail_in(fn, BG_ERR_NULL, "x, q, scales, idx, count and workspace must be non-NULL");
    if (x_dtype != BG_F32 && x_dtype != BG_F16 && x_dtype != BG_BF16)
        return fail_in(fn, BG_ERR_DTYPE, "x_dtype %lld is not F32/F16/BF16", x_dtype);
    if (tau != tau) return fail_in(fn, BG_ERR_UNSUPPORTED, "tau is NaN");
    if (rows < 1 || rows > kMaxRows) return fail_in(fn, BG_ERR_SHAPE, "rows=%lld out of range", rows);
    if (cols < 128 || cols > kMaxDim || cols % 128)
        return fail_in(fn, BG_ERR_SHAPE, "cols=%lld must be a multiple of 128", cols);
    const int64_t need = bg::outlier_ws_bytes(rows, cols);
    if (workspace_bytes < need)
        return fail_in(fn, BG_ERR_WORKSPACE, "workspace of %lld bytes needed (got %lld)", need, workspace_bytes);
    if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(idx) & 3u) || (reinterpret_cast<uintptr_t>(count) & 3u))
        return fail_in(fn, BG_ERR_ALIGN, "x, q, scales and workspace must be 16-byte aligned, idx and count 4-byte");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float* mask = nullptr;
    bg::launch_outlier_detect(x, x_dtype, rows, cols, tau, static_cast<float*>(workspace), idx, count, &mask, s);
    note_kernel(bg::launch_act_quant(x, x_dtype, rows, cols, BG_GRAN_ROW, false, q, scales, mask, s));
    return launched(fn);
}

BG_EXPORT bg_status gemm_w8a8_outlier(const int8_t* a, const float* a_scales, const int8_t* w, const float* w_scales,
                                      int w_gran, const void* x, int x_dtype, const int32_t* idx,
                                      const int32_t* count, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                                      void* stream) {
    const char* fn = "gemm_w8a8_outlier";
    if (!a || !a_scales || !w || !w_scales || !x || !idx || !count || !y)
        return fail_in(fn, BG_ERR_NULL, "a, a_scales, w, w_scales, x, idx, count and y must be non-NULL");
    if (w_gran != BG_GRAN_TENSOR && w_gran != BG_GRAN_ROW)
        return fail_in(fn, BG_ERR_UNSUPPORTED, "w_gran %lld is not TENSOR/ROW", w_gran);
    if (x_dtype != BG_F32 && x_dtype != BG_F16 && x_dtype != BG_BF16)
        return fail_in(fn, BG_ERR_DTYPE, "x_dtype %lld is not F32/F16/BF16", x_dtype);
    if (out_dtype != BG_BF16 && out_dtype != BG_F16 && out_dtype != BG_F32)
        return fail_in(fn, BG_ERR_DTYPE, "out_dtype %lld is not BF16/F16/F32", out_dtype);
    if (M < 1 || M > kMaxM) return fail_in(fn, BG_ERR_SHAPE, "M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail_in(fn, BG_ERR_SHAPE, "N=%lld must be a multiple of 16", N);
    if (K < 128 || K >= kI8MaxKExcl || K % 128)
        return fail_in(fn, BG_ERR_SHAPE, "K=%lld must be a multiple of 128 and below 131072", K);
    if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned16(a_scales) || !aligned16(w_scales) ||
        (reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(idx) & 3u) ||
        (reinterpret_cast<uintptr_t>(count) & 3u))
        return fail_in(fn, BG_ERR_ALIGN, "a, w, y and the scales must be 16-byte aligned, x, idx and count 4-byte");
    bg::W8A8Args g{a, a_scales, BG_GRAN_ROW, w, w_scales, w_gran, false, M, N, K, y, out_dtype};
    g.ox = x;
    g.ox_dt = x_dtype;
    g.oidx = idx;
    g.ocnt = count;
    note_kernel(bg::launch_w8a8_tiled(g, nullptr, static_cast<hipStream_t>(stream)));
    return launched(fn);
}

static bg_status w4a8_impl(const int8_t* a, const float* a_scales, int a_gran, int64_t M, int64_t K,
                           const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t N, int group,
                           void* y, int out_dtype, void* ws, int64_t ws_bytes, bool with_ws, void* stream) {
    if (!a || !a_scales || !qweight || !scales || !y)
        return fail(BG_ERR_NULL, "gemm_w4a8: a, a_scales, qweight, scales and y must be non-NULL");
    if (a_gran != BG_GRAN_TENSOR && a_gran != BG_GRAN_ROW)
        return fail(BG_ERR_UNSUPPORTED, "gemm_w4a8: a_gran %lld is not TENSOR/ROW", a_gran);
    if (out_dtype != BG_BF16 && out_dtype != BG_F16 && out_dtype != BG_F32)
        return fail(BG_ERR_DTYPE, "gemm_w4a8: out_dtype %lld is not BF16/F16/F32", out_dtype);
    if (group != 128) return fail(BG_ERR_UNSUPPORTED, "gemm_w4a8: group %lld (only 128 is supported)", group);
    if (M < 1 || M > kMaxM) return fail(BG_ERR_SHAPE, "gemm_w4a8: M=%lld out of range", M);
    if (N < 16 || N > kMaxRows || N % 16) return fail(BG_ERR_SHAPE, "gemm_w4a8: N=%lld must be a multiple of 16", N);
    if (K < 256 || K > kMaxDim || K % 256) return fail(BG_ERR_SHAPE, "gemm_w4a8: K=%lld must be a multiple of 256", K);
    if (M * K >= (int64_t(1) << 31)) return fail(BG_ERR_SHAPE, "gemm_w4a8: M*K=%lld too large", M * K);
    if (!aligned16(a) || !aligned16(a_scales) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y) ||
        (zeros && !aligned16(zeros)) || (ws && !aligned16(ws)))
        return fail(BG_ERR_ALIGN, "gemm_w4a8: pointers must be 16-byte aligned");
    if (bg::w4a8_decode_fits(M, N, K)) {
        note_kernel(bg::launch_w4a8_decode(a, a_scales, a_gran == BG_GRAN_ROW, M, K, qweight, scales, zeros, N, y,
                                           out_dtype, static_cast<hipStream_t>(stream)));
        return launched("gemm_w4a8");
    }
    void* use_ws = nullptr;
    if (with_ws) {
        const int64_t need = bg::w4a8_gemm_split(M, N, K).ws_bytes;
        if (need > 0) {
            if (!ws || ws_bytes < need)
                return fail(BG_ERR_WORKSPACE, "gemm_w4a8: workspace of %lld bytes needed (got %lld)", need,
                            ws ? ws_bytes : 0);
            use_ws = ws;
        }
    }
    note_kernel(bg::launch_w4a8_gemm(a, a_scales, a_gran == BG_GRAN_ROW, M, K, qweight, scales, zeros, N, y,
                                     out_dtype, use_ws, static_cast<hipStream_t>(stream)));
    return launched("gemm_w4a8");
}

BG_EXPORT bg_status gemm_w4a8(const int8_t* a, const float* a_scales, int a_gran, int64_t M, int64_t K,
                              const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t N,
                              int group, void* y, int out_dtype, void* stream) {
    return w4a8_impl(a, a_scales, a_gran, M, K, qweight, scales, zeros, N, group, y, out_dtype, nullptr, 0, false,
                     stream);
}

BG_EXPORT bg_status gemm_w4a8_ws(const int8_t* a, const float* a_scales, int a_gran, int64_t M, int64_t K,
                                 const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                 int group, void* y, int out_dtype, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
    return w4a8_impl(a, a_scales, a_gran, M, K, qweight, scales, zeros, N, group, y, out_dtype, workspace,
                     workspace_bytes, true, stream);
}

BG_EXPORT int64_t gemm_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kMaxM || N < 16 || N > kMaxRows || N % 16 || K < 256 || K > kMaxDim || K % 256) return 0;
    if (bg::w4a8_decode_fits(M, N, K)) return 0;
    return bg::w4a8_gemm_split(M, N, K).ws_bytes;
}

BG_EXPORT const char* bg_status_string(int status) {
    switch (status) {
        case BG_OK: return "ok";
        case BG_ERR_NULL: return "null pointer";
        case BG_ERR_SHAPE: return "unsupported shape";
        case BG_ERR_ALIGN: return "misaligned pointer";
        case BG_ERR_DTYPE: return "unsupported dtype";
        case BG_ERR_UNSUPPORTED: return "unsupported combination";
        case BG_ERR_HIP: return "HIP runtime error";
        case BG_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

BG_EXPORT const char* bg_last_error(void) { return g_last_error; }

BG_EXPORT int bg_pack_format_version(void) { return BG_PACK_FORMAT_VERSION; }

BG_EXPORT const char* bg_last_kernel(void) { return g_last_kernel; }
