// One-launch operand preparation for a dense W4A4 + RAC GEMM (gfx950).
//
// QUADS (arXiv 2607.15810) section 3.3, Eq. 21: before the product, the
// residual of the selected channels (R, bf16) and the matching weight columns
// (W_S, bf16) are gathered; the dense 256 x 256 kernel also reads the NVFP4
// block scales of both operands as tiled fp16 records.  The four jobs are
// small and independent, so one grid runs them side by side: its workgroups
// are split into consecutive ranges, one per job, instead of four launches
// that each drain before the next starts.
#include "q4_internal.h"
#include "q4_prep.h"

namespace q4 {
namespace {

struct PrepArgs {
  // residual gather
  const uint16_t* x;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_ts;
  uint16_t* R;
  // weight-column gather
  const uint16_t* w_hi_t;
  uint16_t* W_S;
  const int32_t* idx;
  // scale records
  const uint8_t* w_scales;
  uint4* a_tiles;
  uint4* w_tiles;
  int64_t M, N, a_pad, w_pad;
  int32_t K, k, kp;
  // workgroup ranges, in launch order: W_S tiles, R, A records, W records
  int64_t n_ws, n_r, n_ta, n_tw;
  int64_t ws_gx;  // W_S tiles along N
};

template <bool MX>
__global__ __launch_bounds__(256) void rac_prep_kernel(PrepArgs p) {
  __shared__ uint16_t tile[64][66];
  int64_t b = blockIdx.x;
  if (b < p.n_ws) {
    const int64_t by = b / p.ws_gx;
    wsel_gather_part(p.w_hi_t, p.K, p.N, p.idx, p.k, p.kp, p.W_S, 0, b - by * p.ws_gx, (int)by,
                     tile);
    return;
  }
  b -= p.n_ws;
  if (b < p.n_r) {
    residual_gather_part<MX>(p.x, p.M, p.K, p.a_codes, p.a_scales, p.a_ts, p.idx, p.k, p.R, p.kp,
                             b, p.n_r);
    return;
  }
  b -= p.n_r;
  if (b < p.n_ta) {
    scale_tile_part(p.a_scales, p.M, p.K, p.a_pad, p.a_tiles, b, p.n_ta);
    return;
  }
  b -= p.n_ta;
  scale_tile_part(p.w_scales, p.N, p.K, p.w_pad, p.w_tiles, b, p.n_tw);
}

int64_t grid_stride_blocks(int64_t items) {
  const int64_t g = (items + 255) / 256;
  return g > 8192 ? 8192 : g;
}

}  // namespace

hipError_t launch_rac_prep(bool mx, const uint16_t* x, int64_t M, int64_t N, int32_t K,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                           const uint8_t* w_scales, const uint16_t* w_hi_t, const int32_t* idx,
                           int32_t k, int32_t kp, uint16_t* R, uint16_t* W_S, uint8_t* a_tiles,
                           uint8_t* w_tiles, int64_t a_pad, int64_t w_pad, hipStream_t stream) {
  PrepArgs p{};
  p.x = x;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_ts = a_ts;
  p.R = R;
  p.w_hi_t = w_hi_t;
  p.W_S = W_S;
  p.idx = idx;
  p.w_scales = w_scales;
  p.a_tiles = (uint4*)a_tiles;
  p.w_tiles = (uint4*)w_tiles;
  p.M = M;
  p.N = N;
  p.a_pad = a_pad;
  p.w_pad = w_pad;
  p.K = K;
  p.k = k;
  p.kp = kp;
  const bool rac = k > 0 && kp > 0 && R && W_S;
  const bool tiles = !mx && a_tiles && w_tiles;
  p.ws_gx = (N + 63) / 64;
  p.n_ws = rac ? p.ws_gx * ((kp + 63) / 64) : 0;
  p.n_r = rac ? grid_stride_blocks(M * ((kp + 7) / 8)) : 0;
  p.n_ta = tiles ? grid_stride_blocks((int64_t)(K / 128) * a_pad) : 0;
  p.n_tw = tiles ? grid_stride_blocks((int64_t)(K / 128) * w_pad) : 0;
  const int64_t grid = p.n_ws + p.n_r + p.n_ta + p.n_tw;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (mx)
    hipLaunchKernelGGL(rac_prep_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rac_prep_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace q4
