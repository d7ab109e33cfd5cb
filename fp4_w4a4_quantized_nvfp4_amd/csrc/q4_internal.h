// Internal declarations of the q4rac library (host launchers and shared types).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4_device.h"

namespace q4 {

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

__global__ void tensor_scale_kernel(const float* ts_in, float* ts_out);

// ---------------------------------------------------------------- quantizer
size_t quantize_workspace_bytes(int64_t rows, int64_t cols);
// values c sb s_t of an NVFP4 tensor [rows][cols] as fp32 or bf16 (one rounding)
hipError_t launch_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* ts,
                                int64_t rows, int64_t cols, int32_t y_bf16, void* y,
                                hipStream_t stream);
hipError_t launch_quantize(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                           const float* ts_in, uint8_t* codes, uint8_t* scales, float* ts_out,
                           double* chan_score, int32_t topk, int32_t* chan_idx, void* ws,
                           hipStream_t stream);
hipError_t launch_select(const double* scores, int64_t cols, int32_t topk, int32_t* idx,
                         hipStream_t stream);
// scores[j] = sum over r < mult * ngroups_dev[0], ascending, of partial[r][j]
hipError_t launch_score_reduce_dev(const double* partial, const int32_t* ngroups_dev, int32_t mult,
                                   int64_t cols, double* scores, hipStream_t stream);
// ts_out[0] = ts_in[0] (1 when ts_in is null)
hipError_t launch_copy_scale(const float* ts_in, float* ts_out, hipStream_t stream);
// p[0..n) = v (a kernel, not a memset, so the write may sit in a captured graph)
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);
hipError_t launch_residual_gather(bool mx, const uint16_t* x, int64_t rows, int64_t cols,
                                  const uint8_t* codes, const uint8_t* scales, const float* ts,
                                  const int32_t* idx, int32_t k, uint16_t* R, int64_t ld_r,
                                  hipStream_t stream, int32_t* status = nullptr,
                                  bool units = false);
// units (NVFP4): R as the fp16 GEMM operand bf16(r) 2^-e, s_t = f 2^e
hipError_t launch_wsel_gather(const uint16_t* w_hi_t, int64_t batch, int64_t K, int64_t N,
                              const int32_t* idx, int32_t k, int32_t kp, uint16_t* ws,
                              hipStream_t stream, const float* w_ts = nullptr,
                              const float* a_ts = nullptr);
// w_hi_t channel-major [K][batch][N]; w_ts [batch], a_ts [1] (NVFP4): W_S as
// the fp16 GEMM operand w / (s_W f)
// out[b][c][r] = in[b][r][c]; interleave: out[c][b][r] = in[b][r][c]
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t batch, int64_t rows, int64_t cols,
                                 uint16_t* out, hipStream_t stream, bool interleave = false);
hipError_t launch_moe_pack_w13(const uint16_t* w13, int32_t E, int32_t F, int32_t H,
                               uint16_t* out, hipStream_t stream);

// ---------------------------------------------------------------- GEMM
// kEpiSwiGLUQuant: the SwiGLU epilogue that also quantizes h to NVFP4 under a
// supplied tensor scale (grouped 256 x 256 kernel only)
enum GemmEpilogue : int32_t { kEpiStore = 0, kEpiSwiGLU = 1, kEpiSwiGLUQuant = 2 };

// One W4A4 (+ residual) GEMM, dense or grouped by expert.
struct GemmArgs {
  int64_t M;                 // dense: rows of A / Y.  grouped: total sorted rows
  int64_t N;                 // output columns per expert (packed W13: 2F)
  int32_t K;
  int32_t mx;                // 0 NVFP4, 1 MXFP4
  const uint8_t* a_codes;    // [A rows][K/2]
  const uint8_t* a_scales;   // [A rows][K/16 | K/32]
  const float* a_ts;         // [1] or null
  const uint8_t* w_codes;    // [E][N][K/2]
  const uint8_t* w_scales;   // [E][N][K/16 | K/32]
  const float* w_ts;         // [E] or null
  const uint16_t* r_res;     // bf16 [A rows][ld_r] residual (null: no compensation)
  int32_t ld_r;
  const uint16_t* w_sel;     // bf16 [E][N][kp] selected weight columns
  int32_t kp;                // compensated channels, a multiple of 32 (0: none)
  // null: the compensation term R W_S^T is added as it is.  Set: it is
  // multiplied by -(r_ts[0] * w_ts[e]) (the residual's own tensor scale and
  // the weight's, subtracted: the FP4-quantized residual form of Eq. 21)
  // (NVFP4: R and W_S are fp16.  With r_ts null they are in the units of the
  // W4A4 sum, R = bf16(r) 2^-e_A and W_S = w / (s_W f_A) for s_A = f_A 2^e_A,
  // and add to the unscaled sum before the single s_A s_W multiply; with r_ts
  // they are the exact Eq. 21 values c sb.  MXFP4: bf16 R and W_S, added as
  // they are.)
  const float* r_ts;
  void* Y;                   // store: [rows][ldy] fp32|bf16.  SwiGLU: bf16 [rows][N/2]
  int64_t ldy;
  int32_t y_bf16;
  int32_t epilogue;
  // grouped
  const int32_t* tiles;      // int4 {expert, row_begin, row_end, 0} per M tile (null: dense)
  const int32_t* ntiles_dev; // number of valid M tiles (device)
  const int32_t* a_rows;     // A row of each output row (null: identity)
  int64_t a_src_rows;        // rows of the A operand that a_rows indexes (0: M)
  // optional tiled fp16 scale records (NVFP4, K % 128 == 0): see launch_scale_tile
  // (dense), launch_scale_tile_sorted and launch_scale_tile_batched (grouped:
  // A by sorted row, W one block of nk * w_rows_pad records per expert)
  const uint8_t* a_scales_t;
  const uint8_t* w_scales_t;
  int64_t a_rows_pad;        // rows of the tiled records (a multiple of 256)
  int64_t w_rows_pad;
  // kEpiSwiGLUQuant: h's NVFP4 codes [rows][N/4] and E4M3 scales [rows][N/32]
  // under the tensor scale q_ts[0], and the fp64 sums of its squared
  // residuals per h column over each 128-row half of each M tile,
  // q_partial [2 * M tiles][N/2] (half tile 2 t + i of M tile t)
  uint8_t* q_codes;
  uint8_t* q_scales;
  const float* q_ts;
  double* q_partial;
  // direct compensation (streaming kernel, skinny_direct_ok): the selected
  // weight columns are read in the GEMM from W_hi^T, channel-major
  // interleaved [K][w_hi_batch][N] bf16, at the channels sel[0 .. kp) (sel_k
  // of them valid), instead of a gathered w_sel; r_res is then the plain
  // bf16 residual and both go to bf16 MFMAs after the s_A s_W scaling
  const uint16_t* w_hi_t;
  int64_t w_hi_batch;
  const int32_t* sel;
  int32_t sel_k;
  // optional raw E4M3 scale records of the weights for the streaming kernel
  // (NVFP4, K % 128 == 0): [E][K/128][w_rows_pad][8 B], record (c, r) the
  // scale bytes of row r's blocks 8 c .. 8 c + 7 (launch_e4m3_scale_records)
  const uint8_t* w_rec8;
  // grouped, with tiled records: 128 x 512 tiles, `tiles` then listing M
  // tiles of kWideBM rows (grouped_wide_ok)
  int32_t wide;
};

// whether a grouped GEMM runs on the 256 x 256 kernel (the one with the
// quantizing SwiGLU epilogue)
bool grouped_big_path(const GemmArgs& g);
// whether a grouped NVFP4 GEMM with tiled scale records (K % 128 == 0,
// K >= 512) and N columns can run on 128 x 512 tiles
bool grouped_wide_ok(int64_t K, int64_t N);

hipError_t launch_w4a4_gemm(const GemmArgs& g, int64_t max_mtiles, hipStream_t stream);
// scale records [K/128][rows_pad][16 B] of an NVFP4 operand for the dense kernel
hipError_t launch_scale_tile(const uint8_t* scales, int64_t rows, int32_t K, int64_t rows_pad,
                             uint8_t* out, hipStream_t stream);
inline int64_t tile_rows_pad(int64_t rows) { return (rows + 255) / 256 * 256; }
// The 256 x 256 kernel addresses its operands through buffer resources with
// 32-bit offsets: tiled scale records of an operand of `rows` rows fit when
// all K / 128 chunks of them (16 bytes per padded row) span at most 4 GiB
inline bool records_fit(int64_t rows, int64_t K) {
  return tile_rows_pad(rows) * (K / 128) * 16 <= (int64_t)0xffffffffLL;
}
// records of `batch` operands [rows][K / 16]: [batch][K / 128][rows_pad][16 B]
hipError_t launch_scale_tile_batched(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                     int64_t rows_pad, uint8_t* out, hipStream_t stream);
// MXFP4 scale records of `batch` operands [rows][K / 32]: [batch][K / 128][rows_pad][4 B],
// record (c, r) = the E8M0 bytes of blocks 4c .. 4c + 3 of row r (rows past `rows` zero)
hipError_t launch_mx_scale_records(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                   int64_t rows_pad, uint8_t* out, hipStream_t stream);
// records of the R token-sorted rows of a grouped A operand (source row
// a_rows[r], or r without a_rows; expert ranges `offsets` [E + 1]):
// [K / 128][rows_pad][16 B], each swizzled for its row's offset in its expert
hipError_t launch_scale_tile_sorted(const uint8_t* scales, const int32_t* a_rows, int64_t R,
                                    int32_t K, const int32_t* offsets, int32_t E, int64_t rows_pad,
                                    uint8_t* out, hipStream_t stream);
// R and W_S of a dense RAC GEMM (when k > 0 and R, W_S are given) and the
// scale records of both operands (NVFP4, when a_tiles and w_tiles are given)
// in one launch
// Page-literal (Eq. 21) compensation operands of a dense NVFP4 GEMM: the
// residual's tensor amax (per-workgroup maxima in `slots`, nslots of them),
// then in one launch s_R (to r_ts and, if given, r_ts_out), R' [M][kp], W'
// [N][kp] and, when a_tiles and w_tiles are given, both operands' scale records
hipError_t launch_eq21_prep(const uint16_t* x, int64_t M, int64_t N, int32_t K,
                            const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                            const uint8_t* w_codes, const uint8_t* w_scales, const int32_t* idx,
                            int32_t k, int32_t kp, uint16_t* R, uint16_t* W_S, uint32_t* slots,
                            int32_t nslots, float* r_ts, float* r_ts_out, uint8_t* a_tiles,
                            uint8_t* w_tiles, int64_t a_pad, int64_t w_pad, hipStream_t stream,
                            int32_t* status = nullptr);
hipError_t launch_rac_prep(bool mx, const uint16_t* x, int64_t M, int64_t N, int32_t K,
                           const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                           const uint8_t* w_scales, const float* w_ts, const uint16_t* w_hi_t,
                           const int32_t* idx,
                           int32_t k, int32_t kp, uint16_t* R, uint16_t* W_S, uint8_t* a_tiles,
                           uint8_t* w_tiles, int64_t a_pad, int64_t w_pad, hipStream_t stream,
                           int32_t* status = nullptr);

constexpr int kGemmBM = 256;
constexpr int kGemmBN = 128;

// ---------------------------------------------------------------- MoE
hipError_t launch_moe_route(const float* logits, int64_t T, int32_t E, int32_t topk,
                            int32_t* idx, float* w, hipStream_t stream);
size_t moe_sort_workspace_bytes(int64_t T, int32_t E, int32_t topk);
// optional: a_rows[r] = token of sorted row r; a second tile table with bm2
// rows per tile (tiles2, ntiles2)
hipError_t launch_moe_sort(const int32_t* idx, int64_t T, int32_t E, int32_t topk, int32_t* perm,
                           int32_t* offsets, int32_t* inv_perm, int32_t* tiles,
                           int32_t* ntiles, int32_t* counts, hipStream_t stream,
                           int32_t* a_rows = nullptr, int32_t bm2 = 0, int32_t* tiles2 = nullptr,
                           int32_t* ntiles2 = nullptr, int32_t* status = nullptr);
// out: the W2 rows, fp32 or (out_bf16) bf16; H % 8 == 0 for bf16 rows
hipError_t launch_moe_combine(const void* out, int32_t out_bf16, const int32_t* inv_perm,
                              const float* topk_w, const int32_t* topk_idx, int32_t E, int64_t T,
                              int32_t topk, int32_t H, void* Y, int32_t y_bf16,
                              hipStream_t stream);
// grouped GEMM over tiles of at most kSkinnyBM rows (few rows per expert)
constexpr int kSkinnyBM = 32;
// M tile rows of the grouped 128 x 512 tiles (GemmArgs::wide)
constexpr int kWideBM = 128;
hipError_t launch_skinny_gemm(const GemmArgs& g, int64_t max_tiles, hipStream_t stream);
// raw E4M3 scale records of `batch` NVFP4 operands [rows][K / 16]:
// [batch][K / 128][rows_pad][8 B] (rows past `rows` zero)
hipError_t launch_e4m3_scale_records(const uint8_t* scales, int64_t batch, int64_t rows, int32_t K,
                                     int64_t rows_pad, uint8_t* out, hipStream_t stream);
// whether launch_skinny_gemm runs a kernel that can read the compensation
// columns directly (GemmArgs::w_hi_t)
bool skinny_direct_ok(bool mx, int64_t K, int64_t N);

}  // namespace q4
