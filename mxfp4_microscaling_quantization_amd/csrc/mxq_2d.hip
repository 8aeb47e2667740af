// NVFP4 with 16x16 block scales (weights): one E4M3 scale per 16x16 tile, stored
// in the 1x16 layout of row-wise NVFP4 (each tile's scale repeated on its 16 rows),
// so that the transposed output is exactly the transpose of the row-wise one.
//
// A 256-thread workgroup owns a 128 x 128 tile (64 x 128 for fp32 input): 64 (32)
// blocks of 16 x 16. The tile is staged in LDS; each block's amax is reduced by the
// threads that share it (partial maxima through LDS); thread b then derives block
// b's scale code. Rows and columns are then encoded from LDS with the shared codes:
// a row task is one 8-element chunk (as in the row kernel), a column task one
// column over 32 rows (as in the column kernel).
#include <algorithm>

#include "mxq_blocks.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int k2dThreads = 256;
constexpr int k2dTileC = 128;

template <typename T>
struct Shape2d {
  static constexpr int R = sizeof(T) == 2 ? 128 : 64;
  static constexpr int BR = R / 16, BC = k2dTileC / 16;  // blocks down and across
  static constexpr int B = BR * BC;                      // blocks per tile
  static constexpr int TPB = k2dThreads / B;             // threads per block (4 or 8)
  static constexpr int G = R / 32;                       // 32-row groups of a column
};

struct Params2d {
  const void* x;
  int64_t ldx;
  int64_t rows, cols;  // slab extent
  uint32_t tiles_c;
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col;
  int64_t ld_col_codes, ld_col_scales;
  const float* amax;
  int st_given;      // *amax holds the tensor scale, not the amax
  float* tensor_scale;
};

// LDS column of element column c in tile row r: 32-row groups are XOR-shifted so
// that the column reads of phase 3 spread over all banks (as in the column kernel).
template <int G>
__device__ __forceinline__ int swz2(int r, int c) {
  return c ^ (((r >> 5) & (G - 1)) * (64 / G));
}

// Codes of 8 values with a block's scale code k (bits 0-7) and NaN flag (bit 8).
__device__ __forceinline__ uint32_t nv2d_codes8(const float* v, uint32_t kb, const NvTensor& t) {
  if (t.mode != 0) return t.mode == 2 ? 0u : fp4x8_from_f32(v, 0.0f) & 0x88888888u;
  const uint32_t k = kb & 0xFFu;
  if (kb >> 8) return 0u;
  uint32_t c = nv_codes8_rne(v, t, max(k, 1u));
  if (k == 0u) c &= 0x88888888u;
  return c;
}

__device__ __forceinline__ uint32_t nv2d_byte(uint32_t kb, const NvTensor& t) {
  if (t.mode != 0) return t.mode == 2 ? 0x7Fu : 0u;
  return (kb >> 8) ? 0x7Fu : (kb & 0xFFu);
}

template <typename T, bool ROW, bool COL>
__global__ __launch_bounds__(k2dThreads) void quantize_2d_kernel(Params2d p) {
  using S = Shape2d<T>;
  __shared__ T tile[S::R][k2dTileC] __attribute__((aligned(16)));  // read and written as 16-byte chunks
  __shared__ uint32_t part[k2dThreads];  // per-thread partial maxima (|x| bits)
  __shared__ uint32_t kblk[S::B];        // block scale codes (bit 8: NaN block)
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  const uint32_t t = threadIdx.x;
  const NvTensor nt = nv_tensor_load(p.amax, p.st_given);
  if (p.tensor_scale && blockIdx.x == 0 && t == 0) *p.tensor_scale = nt.st;

  const uint32_t tr = blockIdx.x / p.tiles_c, tc = blockIdx.x - tr * p.tiles_c;
  const int64_t r0 = (int64_t)tr * S::R, c0 = (int64_t)tc * k2dTileC;
  // rows and columns are multiples of 16: every block is wholly inside or outside
  const int nr = (int)std::min<int64_t>(S::R, p.rows - r0);
  const int nc = (int)std::min<int64_t>(k2dTileC, p.cols - c0);
  constexpr int kChunksPerRow = k2dTileC / 8;
  constexpr int kChunks = S::R * k2dTileC / 8 / k2dThreads;

  // ---- phase 1: stage the tile
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const uint32_t q = t + j * k2dThreads;
    const int row = (int)(q / kChunksPerRow), cc = (int)(q % kChunksPerRow);
    Raw<T> r;
    if (row < nr && cc * 8 < nc) load_raw(x, (size_t)(r0 + row) * p.ldx + c0 + cc * 8, r);
    else zero_raw(r);
    *reinterpret_cast<Raw<T>*>(&tile[row][swz2<S::G>(row, cc * 8)]) = r;
  }
  __syncthreads();

  // ---- phase 2: block amax (|x| as fp32 bits: NaN > Inf > finite), block codes
  {
    const int b = (int)t / S::TPB, sub = (int)t % S::TPB;
    const int br = b / S::BC, bc = b % S::BC;
    constexpr int kRowsPer = 16 / S::TPB;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kRowsPer; ++i) {
      const int row = br * 16 + sub * kRowsPer + i;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Raw<T> r = *reinterpret_cast<const Raw<T>*>(&tile[row][swz2<S::G>(row, bc * 16 + h * 8)]);
        float v[8];
        to_f32(r, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, as_u(v[e]) & 0x7FFFFFFFu);
      }
    }
    part[t] = m;
  }
  __syncthreads();
  if (t < (uint32_t)S::B) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < S::TPB; ++i) m = max(m, part[t * S::TPB + i]);
    const bool nanb = m >= 0x7F800000u;
    uint32_t k = 0;
    if (nt.mode == 0) k = nv_block_scale_fast(ldexpf(as_f(nanb ? 0u : m), -nt.et), nt.st_n);
    kblk[t] = k | (nanb ? 0x100u : 0u);
  }
  __syncthreads();

  // ---- phase 3: one 8x8 block of elements per thread, encoded once. A 16x16 tile
  // shares one scale, so an element's code is the same in both outputs: the row
  // codes are stored as they are, and the block's nibbles are transposed in
  // registers and parked in LDS for the column-wise stores.
  constexpr int kB8 = k2dTileC / 8;  // 8-column blocks across
  // column c: rows 8b..8b+7 in dword b; it takes the staged tile's place once every
  // thread has read its elements
  uint32_t(*ct)[S::R / 8] = reinterpret_cast<uint32_t(*)[S::R / 8]>(&tile[0][0]);
  static_assert(k2dTileC * (S::R / 8) * 4 <= sizeof(tile), "the transposed codes fit the tile");
  {
    const int rb = (int)t / kB8, cb = (int)t % kB8;
    const bool valid = rb * 8 < nr && cb * 8 < nc;
    const uint32_t kb = valid ? kblk[(rb >> 1) * S::BC + (cb >> 1)] : 0u;
    uint32_t code[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (valid) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = rb * 8 + i;
        const Raw<T> r = *reinterpret_cast<const Raw<T>*>(&tile[row][swz2<S::G>(row, cb * 8)]);
        float v[8];
        to_f32(r, v);
        code[i] = nv2d_codes8(v, kb, nt);
      }
      if constexpr (ROW) {
        const int64_t col = c0 + cb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t lr = r0 + rb * 8 + i;
          *reinterpret_cast<uint32_t*>(p.codes_row + (lr * p.cols + col) / 2) = code[i];
          if ((cb & 1) == 0) p.scales_row[lr * (p.cols / 16) + col / 16] = (uint8_t)nv2d_byte(kb, nt);
        }
      }
    }
    if constexpr (COL) {
      __syncthreads();  // the tile has been read: its space holds the transposed codes
      if (valid) {
        // 8x8 nibble transpose: swap 4x4, then 2x2, then 1x1 sub-blocks
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x = ((code[i] >> 16) ^ code[i + 4]) & 0x0000FFFFu;
          code[i] ^= x << 16;
          code[i + 4] ^= x;
        }
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t x = ((code[i + k] >> 8) ^ code[i + k + 2]) & 0x00FF00FFu;
            code[i + k] ^= x << 8;
            code[i + k + 2] ^= x;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const uint32_t x = ((code[i] >> 4) ^ code[i + 1]) & 0x0F0F0F0Fu;
          code[i] ^= x << 4;
          code[i + 1] ^= x;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ct[cb * 8 + j][rb] = code[j];
      }
    }
  }

  // ---- phase 4: column-wise stores (one column over 32 rows per task)
  if constexpr (COL) {
    __syncthreads();
#pragma unroll 1
    for (int k = t; k < k2dTileC * S::G; k += k2dThreads) {
      const int c = k / S::G, h = k % S::G;
      const int vrows = nr - h * 32;
      if (vrows <= 0 || c >= nc) continue;
      const uint32_t kb0 = kblk[(2 * h) * S::BC + c / 16];
      const int64_t col = c0 + c, grow0 = r0 + h * 32;
      uint8_t* cdst = p.codes_col + col * p.ld_col_codes + grow0 / 2;
      uint8_t* sdst = p.scales_col + col * p.ld_col_scales;
      sdst[grow0 / 16] = (uint8_t)nv2d_byte(kb0, nt);
      if (vrows >= 32) {
        const uint32_t kb1 = kblk[(2 * h + 1) * S::BC + c / 16];
        *reinterpret_cast<uint4*>(cdst) = make_uint4(ct[c][4 * h], ct[c][4 * h + 1], ct[c][4 * h + 2], ct[c][4 * h + 3]);
        sdst[grow0 / 16 + 1] = (uint8_t)nv2d_byte(kb1, nt);
      } else {
        *reinterpret_cast<uint2*>(cdst) = make_uint2(ct[c][4 * h], ct[c][4 * h + 1]);
      }
    }
  }
}

template <typename T, bool ROW, bool COL>
hipError_t launch_2d_t(const TileLaunch& a, hipStream_t st) {
  using S = Shape2d<T>;
  // slabs of at most 2^22 tiles
  const int64_t tiles_per_row = (a.cols + k2dTileC - 1) / k2dTileC;
  const int64_t max_rows = (int64_t)S::R * std::max<int64_t>(1, ((int64_t)1 << 22) / tiles_per_row);
  for (int64_t s0 = 0; s0 < a.rows; s0 += max_rows) {
    const int64_t nr = std::min(max_rows, a.rows - s0);
    Params2d p;
    p.x = reinterpret_cast<const uint8_t*>(a.x) + (size_t)s0 * a.ldx * sizeof(T);
    p.ldx = a.ldx;
    p.rows = nr;
    p.cols = a.cols;
    p.tiles_c = (uint32_t)tiles_per_row;
    p.codes_row = ROW ? a.codes_row + s0 * (a.cols / 2) : nullptr;
    p.scales_row = ROW ? a.scales_row + s0 * (a.cols / 16) : nullptr;
    // the column outputs are addressed from the slab's first row
    p.codes_col = COL ? a.codes_col + s0 / 2 : nullptr;
    p.scales_col = COL ? a.scales_col + s0 / 16 : nullptr;
    p.ld_col_codes = a.ld_col_codes;
    p.ld_col_scales = a.ld_col_scales;
    p.amax = a.amax;
    p.st_given = a.st_given ? 1 : 0;
    p.tensor_scale = s0 == 0 ? a.tensor_scale : nullptr;
    const uint32_t grid = (uint32_t)(((nr + S::R - 1) / S::R) * tiles_per_row);
    hipLaunchKernelGGL((quantize_2d_kernel<T, ROW, COL>), dim3(grid), dim3(k2dThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_2d_axes(const TileLaunch& a, hipStream_t st) {
  if (a.want_row && a.want_col) return launch_2d_t<T, true, true>(a, st);
  if (a.want_row) return launch_2d_t<T, true, false>(a, st);
  return launch_2d_t<T, false, true>(a, st);
}

}  // namespace

hipError_t launch_quantize_2d(const TileLaunch& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  return a.dtype == 0 ? launch_2d_axes<uint16_t>(a, st) : launch_2d_axes<float>(a, st);
}

}  // namespace mxq
