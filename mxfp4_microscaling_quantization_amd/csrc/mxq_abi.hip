// C ABI of libmxq: argument validation and dispatch to the kernel launchers.
// Declarations and the contract of every entry point are in include/mxq.h.
#include <stdint.h>

#include "../../include/mxq.h"
#include "mxq_internal.h"

using namespace mxq;

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Size limits of every entry point: at most 2^40 elements and 2^30 columns (launch
// grids and per-launch element indices then stay within 32 bits).
bool too_large(int64_t rows, int64_t cols) {
  return cols > ((int64_t)1 << 30) || rows > ((int64_t)1 << 40) / cols;
}

mxq_status from_hip(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_EHIP; }

// Philox4x32-10 on the host (same published definition as the device copy).
uint32_t philox_word0(uint64_t counter, uint64_t seed) {
  uint32_t c0 = (uint32_t)counter, c1 = (uint32_t)(counter >> 32), c2 = 0, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// Shared checks of the quantise entry points.
mxq_status check_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                          mxq_format fmt, mxq_axis axis, mxq_round rnd, uint64_t sr_offset, const uint8_t* codes_row,
                          const uint8_t* scales_row, const uint8_t* codes_col,
                          const uint8_t* scales_col, const float* amax, const float* tensor_scale) {
  if (dt != MXQ_BF16 && dt != MXQ_F32) return MXQ_EINVAL;
  if (fmt != MXQ_MXFP4 && fmt != MXQ_NVFP4 && fmt != MXQ_NVFP4_2D) return MXQ_EINVAL;
  if (axis != MXQ_ROWWISE && axis != MXQ_COLWISE && axis != MXQ_BOTH) return MXQ_EINVAL;
  if (rnd != MXQ_RNE && rnd != MXQ_SR && rnd != MXQ_SR16) return MXQ_EINVAL;
  if (fmt == MXQ_NVFP4_2D && rnd != MXQ_RNE) return MXQ_EUNSUPPORTED;
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!x) return MXQ_EINVAL;
  const bool row = axis & MXQ_ROWWISE, col = axis & MXQ_COLWISE;
  if (row && (!codes_row || !scales_row)) return MXQ_EINVAL;
  if (col && (!codes_col || !scales_col)) return MXQ_EINVAL;
  // NVFP4 without an amax computes it first, in the tensor-scale slot
  if (fmt != MXQ_MXFP4 && !amax && !tensor_scale) return MXQ_EINVAL;
  const int64_t bs = fmt == MXQ_MXFP4 ? 32 : 16;
  if (cols == 0 || ldx < cols) return MXQ_ESHAPE;
  if (row && cols % bs) return MXQ_ESHAPE;
  if (col && (rows % bs || cols % 8)) return MXQ_ESHAPE;
  if (fmt == MXQ_NVFP4_2D && (rows % 16 || cols % 16)) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  const int64_t esz = dt == MXQ_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * esz) % 16) return MXQ_EALIGN;
  if (row && (!aligned(codes_row, 16) || !aligned(scales_row, 4))) return MXQ_EALIGN;
  if (col && (!aligned(codes_col, 16) || !aligned(scales_col, 4))) return MXQ_EALIGN;
  if (fmt != MXQ_MXFP4 && ((amax && !aligned(amax, 4)) || (tensor_scale && !aligned(tensor_scale, 4))))
    return MXQ_EALIGN;
  // the halves stream serves eight elements per generator call from element offsets
  // that are multiples of 8
  if (rnd == MXQ_SR16 && sr_offset % 8) return MXQ_EALIGN;
  return MXQ_OK;
}

mxq_status quantize_impl(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                         mxq_format fmt, mxq_axis axis, bool rht, uint32_t sign_mask, mxq_round rnd,
                         uint64_t sr_seed, uint64_t sr_offset, uint8_t* codes_row,
                         uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                         const float* amax, float* tensor_scale, void* stream) {
  mxq_status s = check_quantize(x, dt, rows, cols, ldx, fmt, axis, rnd, sr_offset, codes_row, scales_row,
                                codes_col, scales_col, amax, tensor_scale);
  if (s != MXQ_OK || rows == 0) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool col = axis & MXQ_COLWISE;
  // NVFP4 with no amax given: the tensor amax (of the transform along the block axis
  // when the Hadamard transform is fused) is computed into the tensor-scale slot and
  // turned into s_t there; the quantiser then reads s_t from that slot.
  bool st_given = false;
  if (fmt != MXQ_MXFP4 && !amax) {
    hipError_t e = rht ? launch_rht_amax(x, dt, rows, cols, ldx, axis == MXQ_COLWISE, sign_mask & 0xFFFFu,
                                         tensor_scale, st)
                       : launch_amax(x, dt, rows, cols, ldx, tensor_scale, st);
    if (e == hipSuccess) e = launch_tensor_scale_in_place(tensor_scale, st);
    if (e != hipSuccess) return MXQ_EHIP;
    amax = tensor_scale;
    tensor_scale = nullptr;
    st_given = true;
  }
  if (fmt == MXQ_NVFP4_2D) {
    TileLaunch a{};
    a.x = x;
    a.ldx = ldx;
    a.rows = rows;
    a.cols = cols;
    a.dtype = dt;
    a.fmt = kNV;
    a.want_row = axis & MXQ_ROWWISE;
    a.want_col = col;
    a.codes_row = codes_row;
    a.scales_row = scales_row;
    a.codes_col = codes_col;
    a.scales_col = scales_col;
    a.ld_col_codes = rows / 2;
    a.ld_col_scales = rows / 16;
    a.amax = amax;
    a.st_given = st_given;
    a.tensor_scale = tensor_scale;
    return from_hip(launch_quantize_2d(a, st));
  }
  if (!col) {
    RowLaunch a{};
    a.x = x;
    a.ldx = ldx;
    a.rows = rows;
    a.cols = cols;
    a.dtype = dt;
    a.fmt = fmt == MXQ_MXFP4 ? kMX : kNV;
    a.sr = (int)rnd;  // 0 nearest even, 1 word stream, 2 halves stream
    a.rht = rht;
    a.sign_mask = sign_mask & 0xFFFFu;
    a.sr_seed = sr_seed;
    a.sr_base = sr_offset;
    a.codes = codes_row;
    a.scales = scales_row;
    a.amax = amax;
    a.st_given = st_given;
    a.tensor_scale = tensor_scale;
    return from_hip(launch_quantize_rows(a, st));
  }
  TileLaunch a{};
  a.x = x;
  a.ldx = ldx;
  a.rows = rows;
  a.cols = cols;
  a.dtype = dt;
  a.fmt = fmt == MXQ_MXFP4 ? kMX : kNV;
  a.sr = (int)rnd;  // 0 nearest even, 1 word stream, 2 halves stream
  a.rht = rht;
  a.want_row = axis & MXQ_ROWWISE;
  a.want_col = true;
  a.sign_mask = sign_mask & 0xFFFFu;
  a.sr_seed = sr_seed;
  a.sr_offset = sr_offset;
  a.total_rows = rows;
  a.total_cols = cols;
  a.codes_row = a.want_row ? codes_row : nullptr;
  a.scales_row = a.want_row ? scales_row : nullptr;
  a.codes_col = codes_col;
  a.scales_col = scales_col;
  const int64_t bs = fmt == MXQ_MXFP4 ? 32 : 16;
  a.ld_col_codes = rows / 2;
  a.ld_col_scales = rows / bs;
  a.amax = amax;
  a.st_given = st_given;
  a.tensor_scale = tensor_scale;
  return from_hip(launch_quantize_tiles(a, st));
}

}  // namespace

extern "C" {

mxq_status mxq_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        mxq_format fmt, mxq_axis axis, mxq_round rnd, uint64_t sr_seed,
                        uint64_t sr_offset, uint8_t* codes_row, uint8_t* scales_row,
                        uint8_t* codes_col, uint8_t* scales_col, const float* amax,
                        float* tensor_scale, void* stream) {
  return quantize_impl(x, dt, rows, cols, ldx, fmt, axis, false, 0u, rnd, sr_seed, sr_offset,
                       codes_row, scales_row, codes_col, scales_col, amax, tensor_scale, stream);
}

mxq_status mxq_rht_quantize_mask(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                                 mxq_format fmt, mxq_axis axis, uint16_t sign_mask, mxq_round rnd,
                                 uint64_t sr_seed, uint64_t sr_offset, uint8_t* codes_row,
                                 uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                                 const float* amax, float* tensor_scale, void* stream) {
  if (fmt == MXQ_NVFP4_2D) return MXQ_EUNSUPPORTED;
  if (fmt != MXQ_MXFP4 && fmt != MXQ_NVFP4) return MXQ_EINVAL;
  // NVFP4 takes one tensor scale per call, from the amax of the transform along the
  // block axis; the row- and column-wise transforms differ, so one axis per call
  if (fmt == MXQ_NVFP4 && axis == MXQ_BOTH) return MXQ_EUNSUPPORTED;
  return quantize_impl(x, dt, rows, cols, ldx, fmt, axis, true, sign_mask, rnd, sr_seed, sr_offset,
                       codes_row, scales_row, codes_col, scales_col, amax, tensor_scale, stream);
}

mxq_status mxq_rht_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                            mxq_format fmt, mxq_axis axis, uint64_t rht_seed, mxq_round rnd,
                            uint64_t sr_seed, uint64_t sr_offset, uint8_t* codes_row,
                            uint8_t* scales_row, uint8_t* codes_col, uint8_t* scales_col,
                            const float* amax, float* tensor_scale, void* stream) {
  return mxq_rht_quantize_mask(x, dt, rows, cols, ldx, fmt, axis, mxq_rht_signs(rht_seed), rnd, sr_seed,
                               sr_offset, codes_row, scales_row, codes_col, scales_col, amax, tensor_scale,
                               stream);
}

mxq_status mxq_dequantize(const uint8_t* codes, const uint8_t* scales, mxq_format fmt,
                          int64_t rows, int64_t cols, const float* tensor_scale, void* y,
                          mxq_dtype out_dt, void* stream) {
  if (fmt == MXQ_NVFP4_2D) fmt = MXQ_NVFP4;  // same layout
  if (fmt != MXQ_MXFP4 && fmt != MXQ_NVFP4) return MXQ_EINVAL;
  if (out_dt != MXQ_BF16 && out_dt != MXQ_F32) return MXQ_EINVAL;
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!codes || !scales || !y) return MXQ_EINVAL;
  if (fmt == MXQ_NVFP4 && !tensor_scale) return MXQ_EINVAL;
  const int64_t bs = fmt == MXQ_MXFP4 ? 32 : 16;
  if (cols == 0 || cols % bs) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  if (!aligned(codes, 16) || !aligned(y, 16)) return MXQ_EALIGN;
  return from_hip(launch_dequantize(codes, scales, fmt == MXQ_MXFP4 ? kMX : kNV, rows, cols,
                                    tensor_scale, y, out_dt, reinterpret_cast<hipStream_t>(stream)));
}

mxq_status mxq_fp8_to_mxfp4(const uint8_t* q8, const float* s128, int64_t rows, int64_t cols,
                            uint8_t* codes, uint8_t* e8m0, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!q8 || !s128 || !codes || !e8m0) return MXQ_EINVAL;
  if (cols == 0 || cols % 128) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  if (!aligned(q8, 16) || !aligned(s128, 4) || !aligned(codes, 16)) return MXQ_EALIGN;
  return from_hip(launch_fp8_to_mxfp4(q8, s128, rows, cols, codes, e8m0,
                                      reinterpret_cast<hipStream_t>(stream)));
}

mxq_status mxq_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                            uint8_t* q8, float* s128, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!codes || !e8m0 || !q8 || !s128) return MXQ_EINVAL;
  if (cols == 0 || cols % 128) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  if (!aligned(codes, 16) || !aligned(e8m0, 4) || !aligned(q8, 16) || !aligned(s128, 4))
    return MXQ_EALIGN;
  return from_hip(launch_mxfp4_to_fp8(codes, e8m0, rows, cols, q8, s128,
                                      reinterpret_cast<hipStream_t>(stream)));
}

mxq_status mxq_fp4_row_to_fp8_col(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                                  const int64_t* offsets, int64_t n_experts, uint8_t* q8_col,
                                  int64_t ld_q8, float* s_col, int64_t ld_s, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (n_experts < 1 || n_experts > 4096) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!codes || !e8m0 || !offsets || !q8_col || !s_col) return MXQ_EINVAL;
  if (cols == 0 || cols % 32) return MXQ_ESHAPE;
  if (rows >= ((int64_t)1 << 31) || too_large(rows, cols)) return MXQ_ESHAPE;
  if (ld_q8 < rows || ld_s < rc_group_slots(rows, n_experts)) return MXQ_ESHAPE;
  // the grid enumerates group slots x 256-column tiles
  if (rc_group_slots(rows, n_experts) * ((cols + 255) / 256) >= ((int64_t)1 << 31)) return MXQ_ESHAPE;
  if (ld_q8 % 16 || !aligned(codes, 16) || !aligned(q8_col, 16) || !aligned(s_col, 4) || !aligned(offsets, 8))
    return MXQ_EALIGN;
  return from_hip(launch_fp4_row_to_fp8_col(codes, e8m0, rows, cols, offsets, (int)n_experts, q8_col, ld_q8,
                                            s_col, ld_s, reinterpret_cast<hipStream_t>(stream)));
}

mxq_status mxq_rht_apply(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                         uint16_t sign_mask, float* y, void* stream) {
  if (dt != MXQ_BF16 && dt != MXQ_F32) return MXQ_EINVAL;
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  if (!x || !y) return MXQ_EINVAL;
  if (cols == 0 || cols % 16 || ldx < cols) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  const int64_t esz = dt == MXQ_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(y, 16)) return MXQ_EALIGN;
  return from_hip(launch_rht_apply(x, dt, rows, cols, ldx, sign_mask & 0xFFFFu, y,
                                   reinterpret_cast<hipStream_t>(stream)));
}

mxq_status mxq_amax(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                    float* amax_out, void* stream) {
  if (dt != MXQ_BF16 && dt != MXQ_F32) return MXQ_EINVAL;
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (!amax_out) return MXQ_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rows == 0) return from_hip(launch_amax(x, dt, 0, cols, ldx, amax_out, st));
  if (!x) return MXQ_EINVAL;
  if (cols == 0 || cols % 8 || ldx < cols) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  const int64_t esz = dt == MXQ_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(amax_out, 4)) return MXQ_EALIGN;
  return from_hip(launch_amax(x, dt, rows, cols, ldx, amax_out, st));
}

mxq_status mxq_rht_amax(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        mxq_axis axis, uint16_t sign_mask, float* amax_out, void* stream) {
  if (dt != MXQ_BF16 && dt != MXQ_F32) return MXQ_EINVAL;
  if (axis != MXQ_ROWWISE && axis != MXQ_COLWISE) return MXQ_EINVAL;
  if (rows < 0 || cols < 0) return MXQ_EINVAL;
  if (!amax_out) return MXQ_EINVAL;
  const bool colwise = axis == MXQ_COLWISE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rows == 0) return from_hip(launch_rht_amax(x, dt, 0, cols, ldx, colwise, 0, amax_out, st));
  if (!x) return MXQ_EINVAL;
  if (cols == 0 || ldx < cols) return MXQ_ESHAPE;
  if (colwise ? (rows % 16 || cols % 8) : (cols % 16 != 0)) return MXQ_ESHAPE;
  if (too_large(rows, cols)) return MXQ_ESHAPE;
  const int64_t esz = dt == MXQ_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(amax_out, 4)) return MXQ_EALIGN;
  return from_hip(launch_rht_amax(x, dt, rows, cols, ldx, colwise, sign_mask & 0xFFFFu, amax_out, st));
}

uint16_t mxq_rht_signs(uint64_t rht_seed) { return (uint16_t)(philox_word0(0, rht_seed) & 0xFFFFu); }

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_EINVAL: return "MXQ_EINVAL: null pointer, enum out of range or negative size";
    case MXQ_ESHAPE: return "MXQ_ESHAPE: dimension not a multiple of the block size, or ldx < cols";
    case MXQ_EALIGN: return "MXQ_EALIGN: pointer or row stride not aligned as required";
    case MXQ_EUNSUPPORTED: return "MXQ_EUNSUPPORTED: combination not provided";
    case MXQ_EHIP: return "MXQ_EHIP: kernel launch failed";
  }
  return "unknown mxq_status";
}

}  // extern "C"
