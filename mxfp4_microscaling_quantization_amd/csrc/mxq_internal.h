// Host-side launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

enum Fmt : int { kMX = 0, kNV = 1 };

struct FastDivHost {
  uint32_t d, m, s;
};

// d >= 1; valid for numerators below 2^30.
inline FastDivHost make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint32_t s = 30 + l;
  const uint64_t m = ((1ull << s) + d - 1) / d;
  return FastDivHost{d, (uint32_t)m, s};
}

// Everything one row-wise launch needs. Element counts refer to one slab of
// rows; the slab's first element has index sr_base in the whole tensor.
struct RowLaunch {
  const void* x;
  int64_t ldx;        // input row stride, elements
  int64_t rows, cols;
  int dtype;          // 0 bf16, 1 fp32
  int fmt;            // kMX / kNV
  int sr;            // 0 nearest even, 1 stochastic (word stream), 2 stochastic (halves)
  bool rht;
  uint32_t sign_mask;
  uint64_t sr_seed, sr_base;
  uint8_t* codes;
  uint8_t* scales;
  const float* amax;   // NVFP4: the tensor amax, or the tensor scale when st_given
  bool st_given;
  float* tensor_scale;
};

hipError_t launch_quantize_rows(const RowLaunch& a, hipStream_t st);

struct TileLaunch {
  const void* x;
  int64_t ldx;
  int64_t rows, cols;
  int dtype;
  int fmt;
  int sr;            // 0 nearest even, 1 stochastic (word stream), 2 stochastic (halves)
  bool rht;
  bool want_row, want_col;
  uint32_t sign_mask;
  uint64_t sr_seed, sr_offset;
  int64_t total_rows, total_cols;  // of the whole tensor (SR indices)
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col;
  int64_t ld_col_codes, ld_col_scales;  // row strides of the column-wise outputs
  const float* amax;   // NVFP4: the tensor amax, or the tensor scale when st_given
  bool st_given;
  float* tensor_scale;
};

hipError_t launch_quantize_tiles(const TileLaunch& a, hipStream_t st);
// NVFP4 with 16x16 block scales (uses x, ldx, rows, cols, dtype, want_row/col, the
// outputs, ld_col_*, amax and tensor_scale of the TileLaunch)
hipError_t launch_quantize_2d(const TileLaunch& a, hipStream_t st);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int fmt, int64_t rows,
                             int64_t cols, const float* tensor_scale, void* y, int out_dtype,
                             hipStream_t st);

hipError_t launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       float* amax_out, hipStream_t st);
// Replaces the amax held in *slot by the NVFP4 tensor scale RN_fp32(amax / 2688)
// (NaN for a non-finite amax), in place: one thread.
hipError_t launch_tensor_scale_in_place(float* slot, hipStream_t st);

hipError_t launch_rht_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, bool colwise,
                           uint32_t sign_mask, float* amax_out, hipStream_t st);
hipError_t launch_rht_apply(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint32_t sign_mask, float* y, hipStream_t st);

hipError_t launch_fp8_to_mxfp4(const uint8_t* q8, const float* s128, int64_t rows, int64_t cols,
                               uint8_t* codes, uint8_t* e8m0, hipStream_t st);

// MXFP4 rows -> FP8 columns per 128-token expert group. Group slots of the grid:
// an upper bound of sum_e ceil(n_e / 128) for any split of the rows into experts.
inline int64_t rc_group_slots(int64_t rows, int64_t n_experts) { return (rows + 127 * n_experts) / 128; }
hipError_t launch_fp4_row_to_fp8_col(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                                     const int64_t* offsets, int n_experts, uint8_t* q8, int64_t ld_q8,
                                     float* s, int64_t ld_s, hipStream_t st);

hipError_t launch_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* e8m0, int64_t rows,
                               int64_t cols, uint8_t* q8, float* s128, hipStream_t st);

}  // namespace mxq
