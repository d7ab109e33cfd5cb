// C ABI of the q4rac library: argument validation, workspace sizing and launch
// sequencing.  Declarations and the meaning of every argument are in
// include/q4rac.h.  Every check runs on the host before the first launch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/q4rac.h"
#include "q4_internal.h"

using namespace q4;

namespace {

thread_local char g_err[512] = "";

q4_status_t fail(q4_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

q4_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return Q4_OK;
  return fail(Q4_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

#define Q4_REQUIRE_PTR(p)                                                         \
  do {                                                                            \
    if (!(p)) return fail(Q4_EINVAL, "%s: '%s' is null", __func__, #p);            \
    if (!aligned16(p)) return fail(Q4_EALIGN, "%s: '%s' is not 16-byte aligned", __func__, #p); \
  } while (0)
// scalar-accessed buffers (tensor scales, index lists, scores) need only their
// element alignment
#define Q4_REQUIRE_SCALAR(p, a)                                                   \
  do {                                                                            \
    if (!(p)) return fail(Q4_EINVAL, "%s: '%s' is null", __func__, #p);            \
    if (!aligned(p, a)) return fail(Q4_EALIGN, "%s: '%s' is not %d-byte aligned", __func__, #p, (int)(a)); \
  } while (0)
#define Q4_OPT_PTR(p)                                                             \
  do {                                                                            \
    if ((p) && !aligned16(p))                                                     \
      return fail(Q4_EALIGN, "%s: '%s' is not 16-byte aligned", __func__, #p);     \
  } while (0)

hipStream_t S(void* s) { return (hipStream_t)s; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// channels of a quantized tensor / the GEMM reduction length: the kernels
// address a tile's rows with 32-bit offsets (a 40-row window of x, a 256-row
// tile of codes)
constexpr int64_t kMaxCols = (int64_t)1 << 24;

int32_t round_up32(int32_t k) { return (k + 31) & ~31; }

}  // namespace

extern "C" {

const char* q4_last_error(void) { return g_err; }
int32_t q4_version(void) { return 105; }

// ======================================================================== quantize
size_t q4_quantize_workspace_size(int64_t rows, int64_t cols, int32_t fmt) {
  (void)fmt;
  if (rows < 0 || cols <= 0) return 0;
  return quantize_workspace_bytes(rows, cols);
}

static q4_status_t quantize_common(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                                   const float* ts_in, uint8_t* codes, uint8_t* scales,
                                   float* ts_out, double* chan_score, int32_t topk,
                                   int32_t* chan_idx, void* ws, size_t ws_bytes, void* stream,
                                   const char* fn) {
  const int blk = mx ? 32 : 16;
  if (rows < 0 || cols <= 0 || cols % blk != 0 || rows >= kMaxDim || cols > kMaxCols)
    return fail(Q4_ESHAPE,
                "%s: need rows >= 0 and 0 < cols <= 2^24 with cols %% %d == 0 (got %lld x %lld)", fn,
                blk, (long long)rows, (long long)cols);
  if (topk < 0 || topk > cols || topk > Q4_MAX_TOPK)
    return fail(Q4_EINVAL, "%s: topk %d outside [0, min(cols, %d)]", fn, topk, Q4_MAX_TOPK);
  if (rows > 0) {
    if (!x) return fail(Q4_EINVAL, "%s: 'x' is null", fn);
    if (!aligned16(x)) return fail(Q4_EALIGN, "%s: 'x' is not 16-byte aligned", fn);
    if (!codes || !scales) return fail(Q4_EINVAL, "%s: 'codes'/'scales' is null", fn);
    if (!aligned16(codes) || !aligned16(scales))
      return fail(Q4_EALIGN, "%s: 'codes'/'scales' not 16-byte aligned", fn);
  }
  if (!mx && !ts_out) return fail(Q4_EINVAL, "%s: 'tensor_scale_out' is null", fn);
  if (ts_in && !aligned(ts_in, 4)) return fail(Q4_EALIGN, "%s: 'tensor_scale_in' not aligned", fn);
  if (ts_out && !aligned(ts_out, 4)) return fail(Q4_EALIGN, "%s: 'tensor_scale_out' not aligned", fn);
  if (chan_score && !aligned(chan_score, 8)) return fail(Q4_EALIGN, "%s: 'chan_score' not aligned", fn);
  if (topk > 0 && !chan_idx) return fail(Q4_EINVAL, "%s: 'chan_idx' is null with topk > 0", fn);
  if (topk == 0 && chan_idx) return fail(Q4_EINVAL, "%s: 'chan_idx' given with topk == 0", fn);
  if (chan_idx && !aligned(chan_idx, 4)) return fail(Q4_EALIGN, "%s: 'chan_idx' not aligned", fn);
  const size_t need = quantize_workspace_bytes(rows, cols);
  if (!ws || ws_bytes < need)
    return fail(Q4_EWORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
  if (!aligned16(ws)) return fail(Q4_EALIGN, "%s: 'workspace' not aligned", fn);
  return hip_status(launch_quantize(mx, x, rows, cols, ts_in, codes, scales, ts_out, chan_score,
                                    topk, chan_idx, ws, S(stream)),
                    fn);
}

q4_status_t nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols,
                           const float* tensor_scale_in, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale_out, double* chan_score, int32_t topk,
                           int32_t* chan_idx, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return quantize_common(false, x, rows, cols, tensor_scale_in, codes, scales, tensor_scale_out,
                         chan_score, topk, chan_idx, workspace, workspace_bytes, stream,
                         "nvfp4_quantize");
}

}  // extern "C"

// ------------------------------------------------------------ no-allocation quantize
// nvfp4_quantize_noalloc takes its scratch (amax slots, fp64 partial channel
// sums, the score buffer) from this file-scope device array instead of a
// caller workspace.  In host code the name `scratch` is only a host-side
// stand-in: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address reaches a kernel.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)24 << 20;
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kNoAllocMaxDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static q4_status_t scratch_for_current_device(void** out, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(Q4_EUNSUPPORTED, "%s: device %d beyond the %d devices supported", fn, dev,
                kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(Q4_EHIP, "%s: no device address for the scratch array", fn);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return Q4_OK;
}

extern "C" {

size_t nvfp4_quantize_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

q4_status_t nvfp4_quantize_noalloc(const uint16_t* x, int64_t rows, int64_t cols,
                                   const float* tensor_scale_in, uint8_t* codes, uint8_t* scales,
                                   float* tensor_scale_out, double* chan_score, int32_t topk,
                                   int32_t* chan_idx, void* stream) {
  const char* fn = "nvfp4_quantize_noalloc";
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows >= kMaxDim || cols > kMaxCols)
    return fail(Q4_ESHAPE,
                "%s: need rows >= 0 and 0 < cols <= 2^24 with cols %% 16 == 0 (got %lld x %lld)", fn,
                (long long)rows, (long long)cols);
  const size_t need = quantize_workspace_bytes(rows, cols);
  if (need > kNoAllocScratchBytes)
    return fail(Q4_EWORKSPACE,
                "%s: a %lld x %lld tensor needs %zu bytes of scratch, above the static %zu "
                "(use nvfp4_quantize with a workspace)",
                fn, (long long)rows, (long long)cols, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const q4_status_t st = scratch_for_current_device(&ws, fn);
  if (st != Q4_OK) return st;
  return quantize_common(false, x, rows, cols, tensor_scale_in, codes, scales, tensor_scale_out,
                         chan_score, topk, chan_idx, ws, kNoAllocScratchBytes, stream, fn);
}

q4_status_t mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, double* chan_score, int32_t topk, int32_t* chan_idx,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_common(true, x, rows, cols, nullptr, codes, scales, nullptr, chan_score, topk,
                         chan_idx, workspace, workspace_bytes, stream, "mxfp4_quantize");
}

// Trainer-side weight fake quantization (QDQ): quantize as nvfp4_quantize,
// then the dequantized values.  Workspace: the quantizer's, then codes,
// scales and s_t.
size_t nvfp4_qdq_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return quantize_workspace_bytes(rows, cols) + align256((size_t)rows * (size_t)cols / 2) +
         align256((size_t)rows * (size_t)cols / 16) + 256;
}

q4_status_t nvfp4_qdq(const uint16_t* x, int64_t rows, int64_t cols, const float* tensor_scale_in,
                      void* y, int32_t y_dtype, float* tensor_scale_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_qdq";
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows >= kMaxDim || cols > kMaxCols)
    return fail(Q4_ESHAPE, "%s: need rows >= 0 and 0 < cols <= 2^24 with cols %% 16 == 0", fn);
  if (y_dtype != Q4_OUT_F32 && y_dtype != Q4_OUT_BF16) return fail(Q4_EINVAL, "%s: bad y_dtype", fn);
  if (rows > 0) {
    Q4_REQUIRE_PTR(y);
  }
  if (tensor_scale_out) Q4_REQUIRE_SCALAR(tensor_scale_out, 4);
  const size_t need = nvfp4_qdq_workspace_size(rows, cols);
  if (!workspace || workspace_bytes < need)
    return fail(Q4_EWORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need,
                workspace_bytes);
  Q4_REQUIRE_PTR(workspace);
  uint8_t* base = (uint8_t*)workspace;
  const size_t qb = quantize_workspace_bytes(rows, cols);
  uint8_t* codes = base + qb;
  uint8_t* scales = codes + align256((size_t)rows * (size_t)cols / 2);
  float* ts = tensor_scale_out ? tensor_scale_out
                               : (float*)(scales + align256((size_t)rows * (size_t)cols / 16));
  q4_status_t st = quantize_common(false, x, rows, cols, tensor_scale_in, codes, scales, ts,
                                   nullptr, 0, nullptr, base, qb, stream, fn);
  if (st != Q4_OK) return st;
  return hip_status(launch_dequant_nvfp4(codes, scales, ts, rows, cols, y_dtype == Q4_OUT_BF16, y,
                                         S(stream)),
                    fn);
}

size_t q4_select_workspace_size(int64_t cols) {
  (void)cols;
  return 0;
}

q4_status_t q4_select_channels(const double* chan_score, int64_t cols, int32_t topk,
                               int32_t* chan_idx, void* workspace, size_t workspace_bytes,
                               void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (cols <= 0 || cols >= kMaxDim) return fail(Q4_ESHAPE, "q4_select_channels: cols %lld", (long long)cols);
  if (topk < 0 || topk > cols || topk > Q4_MAX_TOPK)
    return fail(Q4_EINVAL, "q4_select_channels: topk %d outside [0, min(cols, %d)]", topk, Q4_MAX_TOPK);
  Q4_REQUIRE_SCALAR(chan_score, 8);
  if (topk > 0) Q4_REQUIRE_SCALAR(chan_idx, 4);
  return hip_status(launch_select(chan_score, cols, topk, chan_idx, S(stream)),
                    "q4_select_channels");
}

q4_status_t q4_residual_gather(int32_t fmt, const uint16_t* x, int64_t rows, int64_t cols,
                               const uint8_t* codes, const uint8_t* scales,
                               const float* tensor_scale, const int32_t* chan_idx, int32_t k,
                               uint16_t* R, int64_t ld_r, int32_t* status, void* stream) {
  if (fmt != Q4_NVFP4 && fmt != Q4_MXFP4) return fail(Q4_EINVAL, "q4_residual_gather: bad format %d", fmt);
  const bool mx = fmt == Q4_MXFP4;
  const int blk = mx ? 32 : 16;
  if (rows < 0 || cols <= 0 || cols % blk || rows >= kMaxDim || cols >= kMaxDim)
    return fail(Q4_ESHAPE, "q4_residual_gather: bad shape %lld x %lld", (long long)rows, (long long)cols);
  if (k < 0 || k > cols || k > Q4_MAX_TOPK || ld_r < k || ld_r <= 0)
    return fail(Q4_EINVAL, "q4_residual_gather: need 0 <= k <= min(cols, %d) and ld_r >= max(k, 1)", Q4_MAX_TOPK);
  if (mx && tensor_scale) return fail(Q4_EINVAL, "q4_residual_gather: MXFP4 takes no tensor scale");
  if (!mx) Q4_REQUIRE_SCALAR(tensor_scale, 4);
  if (rows > 0) {
    Q4_REQUIRE_PTR(x);
    Q4_REQUIRE_PTR(codes);
    Q4_REQUIRE_PTR(scales);
    Q4_REQUIRE_PTR(R);
  }
  if (k > 0) Q4_REQUIRE_SCALAR(chan_idx, 4);
  if (status) Q4_REQUIRE_SCALAR(status, 4);
  return hip_status(launch_residual_gather(mx, x, rows, cols, codes, scales, tensor_scale,
                                           chan_idx, k, R, ld_r, S(stream), status),
                    "q4_residual_gather");
}

// ======================================================================== GEMM
// An empty product (M or N zero) still reports on its channel set: a gather
// of zero rows validates the set and writes the status word.
static q4_status_t empty_status(const char* fn, int32_t fmt, int64_t K, const float* a_ts,
                                const int32_t* chan_set, int32_t k, int32_t* status, void* stream) {
  if (!status) return Q4_OK;
  hipError_t e;
  if (k == 0)
    e = launch_fill_u32((uint32_t*)status, 1, 0u, S(stream));
  else
    e = launch_residual_gather(fmt == Q4_MXFP4, nullptr, 0, K, nullptr, nullptr, a_ts, chan_set,
                               k, nullptr, k, S(stream), status);
  return hip_status(e, fn);
}

static q4_status_t check_gemm(const char* fn, int32_t fmt, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts,
                              void* Y, int32_t y_dtype) {
  if (fmt != Q4_NVFP4 && fmt != Q4_MXFP4) return fail(Q4_EINVAL, "%s: bad format %d", fn, fmt);
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || M >= kMaxDim || N >= kMaxDim || K > kMaxCols)
    return fail(Q4_ESHAPE,
                "%s: need M, N >= 0 and 0 < K <= 2^24 with K %% 32 == 0 (got %lld, %lld, %lld)", fn,
                (long long)M, (long long)N, (long long)K);
  if (y_dtype != Q4_OUT_F32 && y_dtype != Q4_OUT_BF16) return fail(Q4_EINVAL, "%s: bad y_dtype", fn);
  if (M > 0 && N > 0) {
    Q4_REQUIRE_PTR(a_codes);
    Q4_REQUIRE_PTR(a_scales);
    Q4_REQUIRE_PTR(w_codes);
    Q4_REQUIRE_PTR(w_scales);
    Q4_REQUIRE_PTR(Y);
  }
  if (fmt == Q4_NVFP4) {
    Q4_REQUIRE_SCALAR(a_ts, 4);
    Q4_REQUIRE_SCALAR(w_ts, 4);
  } else if (a_ts || w_ts) {
    return fail(Q4_EINVAL, "%s: MXFP4 operands take no tensor scale", fn);
  }
  return Q4_OK;
}

q4_status_t w4a4_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                      const uint8_t* a_scales, const float* a_tensor_scale,
                      const uint8_t* w_codes, const uint8_t* w_scales,
                      const float* w_tensor_scale, void* Y, int32_t y_dtype, void* stream) {
  q4_status_t st = check_gemm("w4a4_gemm", fmt, M, N, K, a_codes, a_scales, a_tensor_scale,
                              w_codes, w_scales, w_tensor_scale, Y, y_dtype);
  if (st != Q4_OK) return st;
  if (M == 0 || N == 0) return Q4_OK;
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = (int32_t)K;
  g.mx = fmt == Q4_MXFP4;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_ts = a_tensor_scale;
  g.w_codes = w_codes;
  g.w_scales = w_scales;
  g.w_ts = w_tensor_scale;
  g.Y = Y;
  g.ldy = N;
  g.y_bf16 = y_dtype == Q4_OUT_BF16;
  g.epilogue = kEpiStore;
  return hip_status(launch_w4a4_gemm(g, 0, S(stream)), "w4a4_gemm");
}

// tiled fp16 scale records of A and W for the dense 256 x 256 kernel
static size_t scale_tiles_bytes(int64_t M, int64_t N, int64_t K) {
  if (K <= 0 || K % 128 != 0) return 0;
  return align256((size_t)tile_rows_pad(M) * (size_t)(K / 128) * 16) +
         align256((size_t)tile_rows_pad(N) * (size_t)(K / 128) * 16);
}

size_t rac_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t k) {
  if (M < 0 || N < 0 || k < 0) return 0;
  const int64_t kp = round_up32(k);
  return align256((size_t)M * kp * 2) + align256((size_t)N * kp * 2) + scale_tiles_bytes(M, N, K);
}

q4_status_t rac_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint16_t* x,
                     const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                     const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale,
                     const uint16_t* w_hi_t, const int32_t* chan_set, int32_t k, void* Y,
                     int32_t y_dtype, void* workspace, size_t workspace_bytes, int32_t* status,
                     void* stream) {
  q4_status_t st = check_gemm("rac_gemm", fmt, M, N, K, a_codes, a_scales, a_tensor_scale,
                              w_codes, w_scales, w_tensor_scale, Y, y_dtype);
  if (st != Q4_OK) return st;
  if (k < 0 || k > K || k > Q4_MAX_TOPK)
    return fail(Q4_EINVAL, "rac_gemm: k %d outside [0, min(K, %d)]", k, Q4_MAX_TOPK);
  if (k > 0) {
    if (M > 0) Q4_REQUIRE_PTR(x);
    if (N > 0) Q4_REQUIRE_PTR(w_hi_t);
    Q4_REQUIRE_SCALAR(chan_set, 4);
    const size_t need = rac_gemm_workspace_size(M, N, K, k);
    if (!workspace || workspace_bytes < need)
      return fail(Q4_EWORKSPACE, "rac_gemm: workspace of %zu bytes needed (got %zu)", need,
                  workspace_bytes);
    Q4_REQUIRE_PTR(workspace);
  }
  if (status) Q4_REQUIRE_SCALAR(status, 4);
  if (M == 0 || N == 0) return empty_status("rac_gemm", fmt, K, a_tensor_scale, chan_set, k, status, stream);
  const bool mx = fmt == Q4_MXFP4;
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = (int32_t)K;
  g.mx = mx;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_ts = a_tensor_scale;
  g.w_codes = w_codes;
  g.w_scales = w_scales;
  g.w_ts = w_tensor_scale;
  g.Y = Y;
  g.ldy = N;
  g.y_bf16 = y_dtype == Q4_OUT_BF16;
  g.epilogue = kEpiStore;
  const int32_t kp = round_up32(k);
  const size_t rac_bytes = align256((size_t)M * kp * 2) + align256((size_t)N * kp * 2);
  // the dense 256 x 256 kernel reads block scales as tiled fp16 records when
  // the workspace has room for them
  uint8_t* ta = nullptr;
  uint8_t* tw = nullptr;
  if (!mx && K % 128 == 0 && M >= 512 && N >= 512 && records_fit(M, K) && records_fit(N, K) &&
      workspace && ((uintptr_t)workspace & 15u) == 0 &&
      workspace_bytes >= rac_bytes + scale_tiles_bytes(M, N, K)) {
    ta = (uint8_t*)workspace + rac_bytes;
    tw = ta + align256((size_t)tile_rows_pad(M) * (size_t)(K / 128) * 16);
    g.a_scales_t = ta;
    g.w_scales_t = tw;
    g.a_rows_pad = tile_rows_pad(M);
    g.w_rows_pad = tile_rows_pad(N);
  }
  uint16_t* R = nullptr;
  uint16_t* W_S = nullptr;
  if (k > 0) {
    R = (uint16_t*)workspace;
    W_S = (uint16_t*)((uint8_t*)workspace + align256((size_t)M * kp * 2));
    g.r_res = R;
    g.ld_r = kp;
    g.w_sel = W_S;
    g.kp = kp;
  }
  hipError_t e = launch_rac_prep(mx, x, M, N, (int32_t)K, a_codes, a_scales, a_tensor_scale,
                                 w_scales, w_tensor_scale, w_hi_t, chan_set, k, kp, R, W_S, ta, tw,
                                 tile_rows_pad(M), tile_rows_pad(N), S(stream), status);
  if (e != hipSuccess) return hip_status(e, "rac_gemm (operand preparation)");
  return hip_status(launch_w4a4_gemm(g, 0, S(stream)), "rac_gemm");
}

// ======================================================================== MoE
// Page-literal compensation (Eq. 21): workspace = R' [M][kp] bf16, W' [N][kp]
// bf16, the residual-amax slots, s_R, then the scale records as in rac_gemm.
constexpr int32_t kEq21MaxSlots = 1024;
static int32_t eq21_slots(int64_t M, int64_t K) {
  const int64_t blocks = M * (K / 16);
  const int64_t g = (blocks + 255) / 256;
  return (int32_t)(g < 1 ? 1 : (g > kEq21MaxSlots ? kEq21MaxSlots : g));
}

size_t rac_gemm_eq21_workspace_size(int64_t M, int64_t N, int64_t K, int32_t k) {
  if (M < 0 || N < 0 || k < 0) return 0;
  const int64_t kp = round_up32(k);
  return align256((size_t)M * kp * 2) + align256((size_t)N * kp * 2) +
         align256((size_t)kEq21MaxSlots * 4) + 256 + scale_tiles_bytes(M, N, K);
}

q4_status_t rac_gemm_eq21(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                          const uint8_t* a_codes, const uint8_t* a_scales,
                          const float* a_tensor_scale, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* w_tensor_scale,
                          const int32_t* chan_set, int32_t k, void* Y, int32_t y_dtype,
                          float* resid_tensor_scale_out, void* workspace, size_t workspace_bytes,
                          int32_t* status, void* stream) {
  q4_status_t st = check_gemm("rac_gemm_eq21", Q4_NVFP4, M, N, K, a_codes, a_scales,
                              a_tensor_scale, w_codes, w_scales, w_tensor_scale, Y, y_dtype);
  if (st != Q4_OK) return st;
  if (k < 0 || k > K || k > Q4_MAX_TOPK)
    return fail(Q4_EINVAL, "rac_gemm_eq21: k %d outside [0, min(K, %d)]", k, Q4_MAX_TOPK);
  if (resid_tensor_scale_out) Q4_REQUIRE_SCALAR(resid_tensor_scale_out, 4);
  if (k > 0) {
    if (M > 0) Q4_REQUIRE_PTR(x);
    Q4_REQUIRE_SCALAR(chan_set, 4);
    const size_t need = rac_gemm_eq21_workspace_size(M, N, K, k);
    if (!workspace || workspace_bytes < need)
      return fail(Q4_EWORKSPACE, "rac_gemm_eq21: workspace of %zu bytes needed (got %zu)", need,
                  workspace_bytes);
    Q4_REQUIRE_PTR(workspace);
  }
  if (status) Q4_REQUIRE_SCALAR(status, 4);
  if (M == 0 || N == 0)
    return empty_status("rac_gemm_eq21", Q4_NVFP4, K, a_tensor_scale, chan_set, k, status, stream);
  if (k == 0) {
    if (status) {
      const hipError_t e = launch_fill_u32((uint32_t*)status, 1, 0u, S(stream));
      if (e != hipSuccess) return hip_status(e, "rac_gemm_eq21 (status)");
    }
    return w4a4_gemm(Q4_NVFP4, M, N, K, a_codes, a_scales, a_tensor_scale, w_codes, w_scales,
                     w_tensor_scale, Y, y_dtype, stream);
  }
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = (int32_t)K;
  g.mx = 0;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_ts = a_tensor_scale;
  g.w_codes = w_codes;
  g.w_scales = w_scales;
  g.w_ts = w_tensor_scale;
  g.Y = Y;
  g.ldy = N;
  g.y_bf16 = y_dtype == Q4_OUT_BF16;
  g.epilogue = kEpiStore;
  const int32_t kp = round_up32(k);
  uint8_t* base = (uint8_t*)workspace;
  uint16_t* R = (uint16_t*)base;
  uint16_t* W_S = (uint16_t*)(base + align256((size_t)M * kp * 2));
  uint32_t* slots = (uint32_t*)((uint8_t*)W_S + align256((size_t)N * kp * 2));
  float* r_ts = (float*)((uint8_t*)slots + align256((size_t)kEq21MaxSlots * 4));
  uint8_t* ta = nullptr;
  uint8_t* tw = nullptr;
  if (K % 128 == 0 && M >= 512 && N >= 512 && records_fit(M, K) && records_fit(N, K)) {
    ta = (uint8_t*)r_ts + 256;
    tw = ta + align256((size_t)tile_rows_pad(M) * (size_t)(K / 128) * 16);
    g.a_scales_t = ta;
    g.w_scales_t = tw;
    g.a_rows_pad = tile_rows_pad(M);
    g.w_rows_pad = tile_rows_pad(N);
  }
  g.r_res = R;
  g.ld_r = kp;
  g.w_sel = W_S;
  g.kp = kp;
  g.r_ts = r_ts;
  hipError_t e = launch_eq21_prep(x, M, N, (int32_t)K, a_codes, a_scales, a_tensor_scale,
                                  w_codes, w_scales, chan_set, k, kp, R, W_S, slots,
                                  eq21_slots(M, K), r_ts, resid_tensor_scale_out, ta, tw,
                                  tile_rows_pad(M), tile_rows_pad(N), S(stream), status);
  if (e != hipSuccess) return hip_status(e, "rac_gemm_eq21 (operand preparation)");
  return hip_status(launch_w4a4_gemm(g, 0, S(stream)), "rac_gemm_eq21");
}

q4_status_t q4_moe_route(const float* logits, int64_t T, int32_t E, int32_t topk,
                         int32_t* topk_idx, float* topk_w, void* stream) {
  if (T < 0 || T >= kMaxDim) return fail(Q4_ESHAPE, "q4_moe_route: bad T");
  if (E < 1 || E > 1024) return fail(Q4_ESHAPE, "q4_moe_route: need 1 <= E <= 1024");
  if (topk < 1 || topk > E || topk > 16) return fail(Q4_EINVAL, "q4_moe_route: need 1 <= topk <= min(E, 16)");
  if (T > 0) {
    Q4_REQUIRE_SCALAR(logits, 4);
    Q4_REQUIRE_SCALAR(topk_idx, 4);
    Q4_REQUIRE_SCALAR(topk_w, 4);
  }
  return hip_status(launch_moe_route(logits, T, E, topk, topk_idx, topk_w, S(stream)),
                    "q4_moe_route");
}

static int64_t moe_max_tiles(int64_t T, int32_t E, int32_t topk) {
  return (T * topk + kGemmBM - 1) / kGemmBM + E;
}
static int64_t moe_max_tiles_skinny(int64_t T, int32_t E, int32_t topk) {
  return (T * topk + kSkinnyBM - 1) / kSkinnyBM + E;
}
static int64_t moe_max_tiles_wide(int64_t T, int32_t E, int32_t topk) {
  return (T * topk + kWideBM - 1) / kWideBM + E;
}
// few rows per expert (decode-shaped): the grouped GEMMs stream the weights
// with 32-row tiles instead of 256-row tiles
static bool moe_skinny(int64_t T, int32_t E, int32_t topk) { return T * topk <= 64 * (int64_t)E; }

size_t q4_moe_sort_workspace_size(int64_t T, int32_t E, int32_t topk) {
  if (T < 0 || E < 1 || topk < 1) return 0;
  return moe_sort_workspace_bytes(T, E, topk) + align256((size_t)T * topk * 4) +
         align256((size_t)moe_max_tiles(T, E, topk) * 16) + 256;
}

q4_status_t q4_moe_sort(const int32_t* topk_idx, int64_t T, int32_t E, int32_t topk,
                        int32_t* perm, int32_t* offsets, void* workspace, size_t workspace_bytes,
                        int32_t* status, void* stream) {
  if (T < 0 || T * 16 >= kMaxDim) return fail(Q4_ESHAPE, "q4_moe_sort: bad T");
  if (E < 1 || E > 1024) return fail(Q4_ESHAPE, "q4_moe_sort: need 1 <= E <= 1024");
  if (topk < 1 || topk > E || topk > 16) return fail(Q4_EINVAL, "q4_moe_sort: need 1 <= topk <= min(E, 16)");
  Q4_REQUIRE_SCALAR(offsets, 4);
  if (T > 0) {
    Q4_REQUIRE_SCALAR(topk_idx, 4);
    Q4_REQUIRE_SCALAR(perm, 4);
  }
  const size_t need = q4_moe_sort_workspace_size(T, E, topk);
  if (!workspace || workspace_bytes < need)
    return fail(Q4_EWORKSPACE, "q4_moe_sort: workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  Q4_REQUIRE_PTR(workspace);
  if (status) Q4_REQUIRE_SCALAR(status, 4);
  uint8_t* w = (uint8_t*)workspace;
  int32_t* counts = (int32_t*)w;
  w += moe_sort_workspace_bytes(T, E, topk);
  int32_t* inv = (int32_t*)w;
  w += align256((size_t)T * topk * 4);
  int32_t* tiles = (int32_t*)w;
  w += align256((size_t)moe_max_tiles(T, E, topk) * 16);
  int32_t* ntiles = (int32_t*)w;
  return hip_status(launch_moe_sort(topk_idx, T, E, topk, perm, offsets, inv, tiles, ntiles,
                                    counts, S(stream), nullptr, 0, nullptr, nullptr, status),
                    "q4_moe_sort");
}

q4_status_t q4_transpose_bf16(const uint16_t* in, int64_t batch, int64_t rows, int64_t cols,
                              uint16_t* out, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || batch >= 65536 || rows >= kMaxDim || cols >= kMaxDim)
    return fail(Q4_ESHAPE, "q4_transpose_bf16: bad shape");
  if (batch * rows * cols > 0) {
    Q4_REQUIRE_PTR(in);
    Q4_REQUIRE_PTR(out);
  }
  return hip_status(launch_transpose_bf16(in, batch, rows, cols, out, S(stream), true),
                    "q4_transpose_bf16");
}

q4_status_t q4_moe_pack_w13(const uint16_t* w13, int32_t E, int32_t F, int32_t H, uint16_t* out,
                            void* stream) {
  if (E < 0 || E >= 65536 || F <= 0 || F % 32 || H <= 0 || 2 * F >= 65536)
    return fail(Q4_ESHAPE, "q4_moe_pack_w13: need F %% 32 == 0, F > 0, H > 0, 2F < 65536, E < 65536");
  if (E > 0) {
    Q4_REQUIRE_PTR(w13);
    Q4_REQUIRE_PTR(out);
  }
  return hip_status(launch_moe_pack_w13(w13, E, F, H, out, S(stream)), "q4_moe_pack_w13");
}

size_t q4_scale_records_size(int32_t fmt, int64_t batch, int64_t rows, int64_t K) {
  if ((fmt != Q4_NVFP4 && fmt != Q4_MXFP4) || batch < 0 || rows < 0 || K <= 0 || K % 128 ||
      rows >= kMaxDim || K >= kMaxDim)
    return 0;
  // NVFP4: the fp16 records (16 B) followed by the raw E4M3 records (8 B)
  return (size_t)batch * (size_t)(K / 128) * (size_t)tile_rows_pad(rows) * (fmt == Q4_MXFP4 ? 4 : 24);
}

// bytes of the fp16 part of an NVFP4 record buffer (the E4M3 part follows)
static size_t fp16_records_bytes(int64_t batch, int64_t rows, int64_t K) {
  return (size_t)batch * (size_t)(K / 128) * (size_t)tile_rows_pad(rows) * 16;
}

q4_status_t q4_scale_records(int32_t fmt, const uint8_t* scales, int64_t batch, int64_t rows,
                             int64_t K, uint8_t* out, size_t out_bytes, void* stream) {
  const char* fn = "q4_scale_records";
  if (fmt != Q4_NVFP4 && fmt != Q4_MXFP4) return fail(Q4_EINVAL, "%s: bad format %d", fn, fmt);
  if (batch < 0 || batch >= 65536 || rows < 0 || rows >= kMaxDim || K <= 0 || K >= kMaxDim)
    return fail(Q4_ESHAPE, "%s: bad shape", fn);
  if (K % 128) return fail(Q4_ESHAPE, "%s: need K %% 128 == 0 (got %lld)", fn, (long long)K);
  const size_t need = q4_scale_records_size(fmt, batch, rows, K);
  if (need == 0) return Q4_OK;
  Q4_REQUIRE_PTR(out);
  if (out_bytes < need) return fail(Q4_EWORKSPACE, "%s: %zu bytes needed (got %zu)", fn, need, out_bytes);
  if (rows > 0) Q4_REQUIRE_PTR(scales);
  if (fmt == Q4_MXFP4)
    return hip_status(launch_mx_scale_records(scales, batch, rows, (int32_t)K, tile_rows_pad(rows),
                                              out, S(stream)), fn);
  hipError_t e = launch_scale_tile_batched(scales, batch, rows, (int32_t)K, tile_rows_pad(rows), out,
                                           S(stream));
  if (e == hipSuccess)
    e = launch_e4m3_scale_records(scales, batch, rows, (int32_t)K, tile_rows_pad(rows),
                                  out + fp16_records_bytes(batch, rows, K), S(stream));
  return hip_status(e, fn);
}

// workspace fields of the grouped expert layer
namespace {
struct MoeLayout {
  size_t off[Q4_MOE_WS_FIELDS];
  size_t inv_perm, tiles, ntiles, tiles_s, ntiles_s, counts, a_rows, w13_sel, w2_sel, qws;
  size_t x_rec, h_rec;   // sorted-row scale records of the two sites (0: none)
  size_t h_part;         // fp64 [2 * M tiles][F]: h's residual sums (quantizing W13 epilogue)
  bool tiled13, tiled2;  // shapes on which the records can be used
  int64_t rows_pad;
  size_t total;
};

MoeLayout moe_layout(int32_t fmt, int64_t T, int32_t E, int32_t H, int32_t F, int32_t topk,
                     int32_t rac_k) {
  MoeLayout L{};
  const bool mx = fmt == Q4_MXFP4;
  const int64_t R = T * topk;
  const int64_t kp = round_up32(rac_k);
  const int sdiv = mx ? 32 : 16;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.off[0] = take((size_t)R * 4);              // perm
  L.off[1] = take((size_t)(E + 1) * 4);        // offsets
  L.off[2] = take((size_t)T * H / 2);          // x codes
  L.off[3] = take((size_t)T * H / sdiv);       // x scales
  L.off[4] = take(4);                          // x tensor scale
  L.off[5] = take((size_t)(rac_k > 0 ? rac_k : 1) * 4);
  L.off[6] = take((size_t)T * (kp ? kp : 1) * 2);
  L.off[7] = take((size_t)R * F * 2);          // h
  L.off[8] = take((size_t)R * F / 2);          // h codes
  L.off[9] = take((size_t)R * F / sdiv);       // h scales
  L.off[10] = take(4);
  L.off[11] = take((size_t)(rac_k > 0 ? rac_k : 1) * 4);
  L.off[12] = take((size_t)R * (kp ? kp : 1) * 2);
  L.off[13] = take((size_t)R * H * 4);         // out, Y's type (room for fp32)
  L.off[14] = take((size_t)H * 8);             // x scores
  L.off[15] = take((size_t)F * 8);             // h scores
  L.inv_perm = take((size_t)R * 4);
  L.tiles = take((size_t)moe_max_tiles(T, E, topk) * 16);
  L.ntiles = take(4);
  L.tiles_s = take((size_t)moe_max_tiles_skinny(T, E, topk) * 16);
  L.ntiles_s = take(4);
  L.counts = take(moe_sort_workspace_bytes(T, E, topk));
  L.a_rows = take((size_t)R * 4);
  L.w13_sel = take((size_t)E * 2 * F * (kp ? kp : 1) * 2);
  L.w2_sel = take((size_t)E * H * (kp ? kp : 1) * 2);
  const size_t qa = quantize_workspace_bytes(T, H), qb = quantize_workspace_bytes(R, F);
  L.qws = take(qa > qb ? qa : qb);
  // NVFP4 prefill shapes whose grouped GEMMs can read tiled scale records
  // (256 x 256 tiles: K % 128 == 0, K >= 512, N % 256 == 0)
  const bool grouped_big = !mx && !moe_skinny(T, E, topk);
  L.tiled13 = grouped_big && H % 128 == 0 && H >= 512 && (2 * (int64_t)F) % 256 == 0 &&
              records_fit(R, H) && records_fit(2 * (int64_t)F, H);
  L.tiled2 = grouped_big && F % 128 == 0 && F >= 512 && H % 256 == 0 && records_fit(R, F) &&
             records_fit(H, F);
  L.rows_pad = tile_rows_pad(R);
  L.x_rec = L.tiled13 ? take((size_t)(H / 128) * L.rows_pad * 16) : 0;
  L.h_rec = L.tiled2 ? take((size_t)(F / 128) * L.rows_pad * 16) : 0;
  L.h_part = grouped_big ? take((size_t)2 * moe_max_tiles(T, E, topk) * F * 8) : 0;
  L.total = o;
  return L;
}
}  // namespace

size_t moe_workspace_size(int32_t fmt, int64_t T, int32_t E, int32_t H, int32_t F, int32_t topk,
                          int32_t rac_k) {
  if (T < 0 || E < 1 || H <= 0 || F <= 0 || topk < 1 || rac_k < 0) return 0;
  return moe_layout(fmt, T, E, H, F, topk, rac_k).total;
}

q4_status_t moe_workspace_layout(int32_t fmt, int64_t T, int32_t E, int32_t H, int32_t F,
                                 int32_t topk, int32_t rac_k, size_t* offsets) {
  if (!offsets) return fail(Q4_EINVAL, "moe_workspace_layout: 'offsets' is null");
  if (T < 0 || E < 1 || H <= 0 || F <= 0 || topk < 1 || rac_k < 0)
    return fail(Q4_ESHAPE, "moe_workspace_layout: bad shape");
  MoeLayout L = moe_layout(fmt, T, E, H, F, topk, rac_k);
  memcpy(offsets, L.off, sizeof(L.off));
  return Q4_OK;
}

q4_status_t moe_w4a4_grouped_gemm_ex(int32_t fmt, const uint16_t* tokens, int64_t T, int32_t H,
                                     const int32_t* topk_idx, const float* topk_w, int32_t topk,
                                     int32_t E, int32_t F, const uint8_t* w13_codes,
                                     const uint8_t* w13_scales, const float* w13_tensor_scales,
                                     const uint8_t* w2_codes, const uint8_t* w2_scales,
                                     const float* w2_tensor_scales, const uint16_t* w13_hi_t,
                                     const uint16_t* w2_hi_t, const uint8_t* w13_scale_records,
                                     const uint8_t* w2_scale_records, const float* h_tensor_scale,
                                     int32_t rac_k, void* Y,
                                     int32_t y_dtype, void* workspace, size_t workspace_bytes,
                                     int32_t* status, uint32_t flags, void* stream) {
  const char* fn = "moe_w4a4_grouped_gemm";
  if (flags & ~(uint32_t)Q4_MOE_FUSE_H_QUANT) return fail(Q4_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  const bool fuse_req = (flags & Q4_MOE_FUSE_H_QUANT) != 0;
  if (fuse_req && !h_tensor_scale)
    return fail(Q4_EINVAL, "%s: Q4_MOE_FUSE_H_QUANT needs h_tensor_scale", fn);
  if (fmt != Q4_NVFP4 && fmt != Q4_MXFP4) return fail(Q4_EINVAL, "%s: bad format %d", fn, fmt);
  const bool mx = fmt == Q4_MXFP4;
  if (T < 0 || T * 16 >= kMaxDim) return fail(Q4_ESHAPE, "%s: bad T", fn);
  if (E < 1 || E > 1024) return fail(Q4_ESHAPE, "%s: need 1 <= E <= 1024", fn);
  if (topk < 1 || topk > E || topk > 16) return fail(Q4_EINVAL, "%s: need 1 <= topk <= min(E, 16)", fn);
  if (H <= 0 || H % 32 || F <= 0 || F % 32 || H > kMaxCols || F > kMaxCols)
    return fail(Q4_ESHAPE, "%s: need 0 < H, F <= 2^24, multiples of 32 (got H %d, F %d)", fn, H, F);
  if ((int64_t)E * 2 * F >= kMaxDim || (int64_t)E * H >= kMaxDim) return fail(Q4_ESHAPE, "%s: too many weight rows", fn);
  if (rac_k < 0 || rac_k > F || rac_k > H || rac_k > Q4_MAX_TOPK)
    return fail(Q4_EINVAL, "%s: rac_k %d outside [0, min(H, F, %d)]", fn, rac_k, Q4_MAX_TOPK);
  if (y_dtype != Q4_OUT_F32 && y_dtype != Q4_OUT_BF16) return fail(Q4_EINVAL, "%s: bad y_dtype", fn);
  Q4_REQUIRE_PTR(w13_codes);
  Q4_REQUIRE_PTR(w13_scales);
  Q4_REQUIRE_PTR(w2_codes);
  Q4_REQUIRE_PTR(w2_scales);
  if (!mx) {
    Q4_REQUIRE_SCALAR(w13_tensor_scales, 4);
    Q4_REQUIRE_SCALAR(w2_tensor_scales, 4);
  } else if (w13_tensor_scales || w2_tensor_scales) {
    return fail(Q4_EINVAL, "%s: MXFP4 weights take no tensor scales", fn);
  }
  if (w13_scale_records) Q4_REQUIRE_PTR(w13_scale_records);
  if (w2_scale_records) Q4_REQUIRE_PTR(w2_scale_records);
  if (h_tensor_scale) {
    if (mx) return fail(Q4_EINVAL, "%s: MXFP4 has no tensor scale to supply", fn);
    Q4_REQUIRE_SCALAR(h_tensor_scale, 4);
  }
  if (rac_k > 0) {
    Q4_REQUIRE_PTR(w13_hi_t);
    Q4_REQUIRE_PTR(w2_hi_t);
  }
  if (T > 0) {
    Q4_REQUIRE_PTR(tokens);
    Q4_REQUIRE_SCALAR(topk_idx, 4);
    Q4_REQUIRE_SCALAR(topk_w, 4);
    Q4_REQUIRE_PTR(Y);
  }
  const MoeLayout L = moe_layout(fmt, T, E, H, F, topk, rac_k);
  if (!workspace || workspace_bytes < L.total)
    return fail(Q4_EWORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, L.total, workspace_bytes);
  Q4_REQUIRE_PTR(workspace);
  if (status) Q4_REQUIRE_SCALAR(status, 4);
  if (T == 0) return status ? hip_status(launch_fill_u32((uint32_t*)status, 1, 0u, S(stream)), fn) : Q4_OK;

  uint8_t* w = (uint8_t*)workspace;
  auto P = [&](size_t off) { return (void*)(w + off); };
  const int64_t R = T * topk;
  const int32_t kp = rac_k > 0 ? round_up32(rac_k) : 0;
  hipStream_t s = S(stream);
  int32_t* perm = (int32_t*)P(L.off[0]);
  int32_t* offsets = (int32_t*)P(L.off[1]);
  int32_t* inv = (int32_t*)P(L.inv_perm);
  int32_t* tiles = (int32_t*)P(L.tiles);
  int32_t* ntiles = (int32_t*)P(L.ntiles);
  int32_t* a_rows = (int32_t*)P(L.a_rows);
  hipError_t e;
#define Q4_TRY(call, what)                 \
  do {                                     \
    e = (call);                            \
    if (e != hipSuccess) return hip_status(e, what); \
  } while (0)
  // NVFP4 prefill shapes read the weights' tiled scale records when given.
  // With them, GEMMs whose N is a multiple of 512 run on 128 x 512 tiles
  // (half the empty rows of 256-row tiles at a few hundred rows per expert);
  // a W13 GEMM asked to quantize h in its epilogue keeps the 256-row tiles.
  const bool rec13 = L.tiled13 && w13_scale_records, rec2 = L.tiled2 && w2_scale_records;
  const bool wide13 = rec13 && !fuse_req && grouped_wide_ok(H, 2 * (int64_t)F);
  const bool wide2 = rec2 && grouped_wide_ok(F, H);
  // the sort also writes each sorted row's token and a second tile table:
  // 32-row tiles of the skinny kernel (decode-shaped layers) or 128-row
  // tiles of the 128 x 512 kernel
  const bool skinny = moe_skinny(T, E, topk);
  const bool table2 = skinny || wide13 || wide2;
  Q4_TRY(launch_moe_sort(topk_idx, T, E, topk, perm, offsets, inv, tiles, ntiles,
                         (int32_t*)P(L.counts), s, a_rows,
                         skinny ? kSkinnyBM : (table2 ? kWideBM : 0),
                         table2 ? (int32_t*)P(L.tiles_s) : nullptr,
                         table2 ? (int32_t*)P(L.ntiles_s) : nullptr, status), "moe sort");
  auto grouped_gemm = [&](GemmArgs& gg) {
    if (skinny) {
      gg.tiles = (const int32_t*)P(L.tiles_s);
      gg.ntiles_dev = (const int32_t*)P(L.ntiles_s);
      return launch_skinny_gemm(gg, moe_max_tiles_skinny(T, E, topk), s);
    }
    if (gg.wide) {
      gg.tiles = (const int32_t*)P(L.tiles_s);
      gg.ntiles_dev = (const int32_t*)P(L.ntiles_s);
      return launch_w4a4_gemm(gg, moe_max_tiles_wide(T, E, topk), s);
    }
    return launch_w4a4_gemm(gg, moe_max_tiles(T, E, topk), s);
  };
  // ---- activation site 1: tokens
  uint8_t* xc = (uint8_t*)P(L.off[2]);
  uint8_t* xs = (uint8_t*)P(L.off[3]);
  float* xts = mx ? nullptr : (float*)P(L.off[4]);
  int32_t* xS = (int32_t*)P(L.off[5]);
  uint16_t* xR = (uint16_t*)P(L.off[6]);
  Q4_TRY(launch_quantize(mx, tokens, T, H, nullptr, xc, xs, xts, (double*)P(L.off[14]), rac_k,
                         rac_k ? xS : nullptr, P(L.qws), s), "moe quantize tokens");
  if (rec13)
    Q4_TRY(launch_scale_tile_sorted(xs, a_rows, R, H, offsets, E, L.rows_pad, (uint8_t*)P(L.x_rec),
                                    s), "moe token scale records");
  // Decode-shaped layers read the selected weight columns straight from
  // W_hi^T inside the streaming GEMM (bf16, with the plain bf16 residual);
  // otherwise they are gathered first.  NVFP4 gathered operands are fp16 in
  // the W4A4 sum's units (R 2^-e_x, W_S / (s_W f_x) per expert).
  const bool direct13 = skinny && kp && skinny_direct_ok(mx, H, 2 * (int64_t)F);
  const bool direct2 = skinny && kp && skinny_direct_ok(mx, F, H);
  if (kp) {
    Q4_TRY(launch_residual_gather(mx, tokens, T, H, xc, xs, xts, xS, rac_k, xR, kp, s, nullptr,
                                  !mx && !direct13), "moe residual tokens");
    if (!direct13)
      Q4_TRY(launch_wsel_gather(w13_hi_t, E, H, 2 * (int64_t)F, xS, rac_k, kp,
                                (uint16_t*)P(L.w13_sel), s, mx ? nullptr : w13_tensor_scales, xts),
             "moe w13 gather");
  }
  uint16_t* hbuf = (uint16_t*)P(L.off[7]);
  GemmArgs g{};
  g.M = R;
  g.N = 2 * (int64_t)F;
  g.K = H;
  g.mx = mx;
  g.a_codes = xc;
  g.a_scales = xs;
  g.a_ts = xts;
  g.w_codes = w13_codes;
  g.w_scales = w13_scales;
  g.w_ts = w13_tensor_scales;
  g.r_res = kp ? xR : nullptr;
  g.ld_r = kp;
  g.w_sel = kp && !direct13 ? (const uint16_t*)P(L.w13_sel) : nullptr;
  g.kp = kp;
  if (direct13) {
    g.w_hi_t = w13_hi_t;
    g.w_hi_batch = E;
    g.sel = xS;
    g.sel_k = rac_k;
  }
  g.Y = hbuf;
  g.ldy = F;
  g.y_bf16 = 1;
  g.epilogue = kEpiSwiGLU;
  g.tiles = tiles;
  g.ntiles_dev = ntiles;
  g.a_rows = a_rows;
  g.a_src_rows = T;
  if (rec13) {
    g.a_scales_t = (const uint8_t*)P(L.x_rec);
    g.w_scales_t = w13_scale_records;
    g.a_rows_pad = L.rows_pad;
    g.w_rows_pad = tile_rows_pad(2 * (int64_t)F);
    g.wide = wide13;
  } else if (skinny && w13_scale_records && H % 128 == 0) {
    // decode-shaped: the streaming kernel reads the weights' scale records,
    // NVFP4 the raw E4M3 part (half the bytes of the fp16 records)
    g.w_rows_pad = tile_rows_pad(2 * (int64_t)F);
    if (mx)
      g.w_scales_t = w13_scale_records;
    else
      g.w_rec8 = w13_scale_records + fp16_records_bytes(E, 2 * (int64_t)F, H);
  }
  // ---- activation site 2: h (sorted rows)
  uint8_t* hc = (uint8_t*)P(L.off[8]);
  uint8_t* hs = (uint8_t*)P(L.off[9]);
  float* hts = mx ? nullptr : (float*)P(L.off[10]);
  int32_t* hS = (int32_t*)P(L.off[11]);
  uint16_t* hR = (uint16_t*)P(L.off[12]);
  double* hscore = (double*)P(L.off[15]);
  // Asked for (Q4_MOE_FUSE_H_QUANT, with a supplied s_h) and on the 256 x 256
  // kernel, the W13 epilogue quantizes h as it stores it (codes, scales,
  // residual sums per half tile): no separate pass over h.  Otherwise the
  // quantizer runs on h (with the supplied s_h, when there is one, in place of
  // h's amax).
  const bool fuse_h = fuse_req && L.h_part && grouped_big_path(g);
  if (fuse_h) {
    g.epilogue = kEpiSwiGLUQuant;
    g.q_codes = hc;
    g.q_scales = hs;
    g.q_ts = h_tensor_scale;
    g.q_partial = (double*)P(L.h_part);
  }
  Q4_TRY(grouped_gemm(g), "moe w13 gemm");
  if (fuse_h) {
    Q4_TRY(launch_copy_scale(h_tensor_scale, hts, s), "moe h tensor scale");
    Q4_TRY(launch_score_reduce_dev((const double*)P(L.h_part), ntiles, 2, F, hscore, s),
           "moe h scores");
    if (rac_k) Q4_TRY(launch_select(hscore, F, rac_k, hS, s), "moe h selection");
  } else {
    Q4_TRY(launch_quantize(mx, hbuf, R, F, h_tensor_scale, hc, hs, hts, hscore, rac_k,
                           rac_k ? hS : nullptr, P(L.qws), s), "moe quantize h");
  }
  if (rec2)
    Q4_TRY(launch_scale_tile_sorted(hs, nullptr, R, F, offsets, E, L.rows_pad, (uint8_t*)P(L.h_rec),
                                    s), "moe h scale records");
  if (kp) {
    Q4_TRY(launch_residual_gather(mx, hbuf, R, F, hc, hs, hts, hS, rac_k, hR, kp, s, nullptr,
                                  !mx && !direct2), "moe residual h");
    if (!direct2)
      Q4_TRY(launch_wsel_gather(w2_hi_t, E, F, H, hS, rac_k, kp, (uint16_t*)P(L.w2_sel), s,
                                mx ? nullptr : w2_tensor_scales, hts), "moe w2 gather");
  }
  GemmArgs g2{};
  g2.M = R;
  g2.N = H;
  g2.K = F;
  g2.mx = mx;
  g2.a_codes = hc;
  g2.a_scales = hs;
  g2.a_ts = hts;
  g2.w_codes = w2_codes;
  g2.w_scales = w2_scales;
  g2.w_ts = w2_tensor_scales;
  g2.r_res = kp ? hR : nullptr;
  g2.ld_r = kp;
  g2.w_sel = kp && !direct2 ? (const uint16_t*)P(L.w2_sel) : nullptr;
  g2.kp = kp;
  if (direct2) {
    g2.w_hi_t = w2_hi_t;
    g2.w_hi_batch = E;
    g2.sel = hS;
    g2.sel_k = rac_k;
  }
  g2.Y = P(L.off[13]);
  g2.ldy = H;
  g2.y_bf16 = y_dtype == Q4_OUT_BF16;   // expert outputs in the layer's output type
  g2.epilogue = kEpiStore;
  g2.tiles = tiles;
  g2.ntiles_dev = ntiles;
  g2.a_rows = nullptr;
  if (rec2) {
    g2.a_scales_t = (const uint8_t*)P(L.h_rec);
    g2.w_scales_t = w2_scale_records;
    g2.a_rows_pad = L.rows_pad;
    g2.w_rows_pad = tile_rows_pad(H);
    g2.wide = wide2;
  } else if (skinny && w2_scale_records && F % 128 == 0) {
    g2.w_rows_pad = tile_rows_pad(H);
    if (mx)
      g2.w_scales_t = w2_scale_records;
    else
      g2.w_rec8 = w2_scale_records + fp16_records_bytes(E, H, F);
  }
  Q4_TRY(grouped_gemm(g2), "moe w2 gemm");
  Q4_TRY(launch_moe_combine(P(L.off[13]), g2.y_bf16, inv, topk_w, topk_idx, E, T, topk, H, Y,
                            y_dtype == Q4_OUT_BF16, s), "moe combine");
#undef Q4_TRY
  return Q4_OK;
}

q4_status_t moe_w4a4_grouped_gemm(int32_t fmt, const uint16_t* tokens, int64_t T, int32_t H,
                                  const int32_t* topk_idx, const float* topk_w, int32_t topk,
                                  int32_t E, int32_t F, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const float* w13_tensor_scales,
                                  const uint8_t* w2_codes, const uint8_t* w2_scales,
                                  const float* w2_tensor_scales, const uint16_t* w13_hi_t,
                                  const uint16_t* w2_hi_t, const uint8_t* w13_scale_records,
                                  const uint8_t* w2_scale_records, const float* h_tensor_scale,
                                  int32_t rac_k, void* Y,
                                  int32_t y_dtype, void* workspace, size_t workspace_bytes,
                                  int32_t* status, void* stream) {
  return moe_w4a4_grouped_gemm_ex(fmt, tokens, T, H, topk_idx, topk_w, topk, E, F, w13_codes,
                                  w13_scales, w13_tensor_scales, w2_codes, w2_scales,
                                  w2_tensor_scales, w13_hi_t, w2_hi_t, w13_scale_records,
                                  w2_scale_records, h_tensor_scale, rac_k, Y, y_dtype, workspace,
                                  workspace_bytes, status, 0u, stream);
}

}  // extern "C"
