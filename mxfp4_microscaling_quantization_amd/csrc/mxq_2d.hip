// NVFP4 with 16x16 block scales (weights): one E4M3 scale per 16x16 tile, stored
// in the 1x16 layout of row-wise NVFP4 (each tile's scale repeated on its 16 rows),
// so that the transposed output is exactly the transpose of the row-wise one.
//
// A 256-thread workgroup owns a 128 x 128 tile of 64 blocks. The four lanes of a
// DPP quad own one block, each an 8 x 8 quarter of it held in registers (8 rows of
// one 16-byte bf16 chunk, or two for fp32): the block's amax is reduced over the
// quad with two DPP exchanges, every lane derives the block's scale code, encodes
// its 8 x 8 codes once and stores their rows directly (the row-wise output). The
// codes are then transposed as 8 x 8 nibble blocks in registers and only they pass
// through LDS (8 KB), from which the column-wise output leaves as 64-byte runs per
// column. One barrier per tile, and the raw tile never touches LDS.
#include <algorithm>

#include "mxq_blocks.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int k2dThreads = 256;
constexpr int k2dTile = 128;               // rows and columns of a tile
constexpr int k2dBlocks = k2dTile / 16;    // 16 x 16 blocks down and across

struct Params2d {
  const void* x;
  int64_t ldx;
  int64_t rows, cols;  // slab extent
  uint32_t tiles_r, tiles_c;
  uint32_t sb_c, sbs;  // 4 x 4 superblocks of tiles: across, in all
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col;
  int64_t ld_col_codes, ld_col_scales;
  const float* amax;
  int st_given;      // *amax holds the tensor scale, not the amax
  float* tensor_scale;
};

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

// |x| bits of the largest magnitude of a chunk (NaN > Inf > finite as integers).
__device__ __forceinline__ uint32_t absmax_bits(const Raw<uint16_t>& r) {
  const uint32_t w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m << 16;
}
__device__ __forceinline__ uint32_t absmax_bits(const Raw<float>& r) {
  float v[8];
  to_f32(r, v);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, as_u(v[i]) & 0x7FFFFFFFu);
  return m;
}

template <typename T, bool ROW, bool COL>
__global__ __launch_bounds__(k2dThreads) void quantize_2d_kernel(Params2d p) {
  // transposed codes: column c of the tile, rows 8 g .. 8 g + 7 in dword g
  __shared__ uint32_t ct[COL ? k2dTile : 1][k2dTile / 8];
  __shared__ uint32_t kblk[k2dBlocks * k2dBlocks];  // block scale codes (bit 8: NaN block)
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  const uint32_t t = threadIdx.x;
  const NvTensor nt = nv_tensor_load(p.amax, p.st_given);
  if (p.tensor_scale && blockIdx.x == 0 && t == 0) *p.tensor_scale = nt.st;

  // Workgroups are dealt to the eight XCDs in turn; the 16 tiles of a 4 x 4 superblock
  // go to one XCD in consecutive turns, so the eight-byte scale pieces that four
  // horizontally (row scales) or vertically (column scales) adjacent tiles share in
  // a 64-byte sector meet in one L2
  const uint32_t xcd = blockIdx.x & 7u, slot = blockIdx.x >> 3;
  const uint32_t sb = (slot >> 4) * 8u + xcd, w = slot & 15u;
  if (sb >= p.sbs) return;
  const uint32_t sbr = sb / p.sb_c, sbc = sb - sbr * p.sb_c;
  const uint32_t tr = 4u * sbr + (w >> 2), tc = 4u * sbc + (w & 3u);
  if (tr >= p.tiles_r || tc >= p.tiles_c) return;
  const int64_t r0 = (int64_t)tr * k2dTile, c0 = (int64_t)tc * k2dTile;
  // rows and columns are multiples of 16: every block is wholly inside or outside
  const int nr = (int)std::min<int64_t>(k2dTile, p.rows - r0);
  const int nc = (int)std::min<int64_t>(k2dTile, p.cols - c0);
  // lane (b, q): block b = (br, bc) of the tile, quarter q = (qr, qc) of the block
  const int b = (int)(t >> 2), q = (int)(t & 3u);
  const int br = b / k2dBlocks, bc = b % k2dBlocks;
  const int row0 = br * 16 + (q >> 1) * 8, col0 = bc * 16 + (q & 1) * 8;  // in the tile
  const bool valid = br * 16 < nr && bc * 16 < nc;

  Raw<T> r[8];
  uint32_t m = 0;
  if (valid) {
    const T* xq = x + (uint64_t)(r0 + row0) * (uint64_t)p.ldx + (uint64_t)(c0 + col0);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_raw(xq, (uint64_t)i * (uint64_t)p.ldx, r[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, absmax_bits(r[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) zero_raw(r[i]);
  }
  // the block's amax over its four quarters (one DPP quad)
  m = max(m, dpp<kQuadSwap1>(m));
  m = max(m, dpp<kQuadSwap2>(m));
  const bool nanb = m >= 0x7F800000u;
  uint32_t kb = 0;
  if (nt.mode == 0) kb = nv_block_scale_fast(ldexpf(as_f(nanb ? 0u : m), -nt.et), nt.st_n);
  kb |= nanb ? 0x100u : 0u;
  const uint32_t byte = nv2d_byte(kb, nt);

  // encode the quarter once: row i of it in code[i], column j in nibble j
  uint32_t code[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    to_f32(r[i], v);
    code[i] = nv2d_codes8(v, kb, nt);
  }
  if constexpr (ROW) {
    if (valid) {
      const uint64_t cols = (uint64_t)p.cols;
      uint8_t* crow = p.codes_row + (uint64_t)(r0 + row0) * (cols / 2) + (uint64_t)(c0 + col0) / 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(crow + (uint64_t)i * (cols / 2)) = code[i];
    }
  }
  if (q == 0) kblk[b] = byte;
  if constexpr (COL) {
    // 8x8 nibble transpose: swap 4x4, then 2x2, then 1x1 sub-blocks; code[j] then
    // holds column j of the quarter, row i in nibble i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = ((code[i] >> 16) ^ code[i + 4]) & 0x0000FFFFu;
      code[i] ^= d << 16;
      code[i + 4] ^= d;
    }
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t d = ((code[i + k] >> 8) ^ code[i + k + 2]) & 0x00FF00FFu;
        code[i + k] ^= d << 8;
        code[i + k + 2] ^= d;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t d = ((code[i] >> 4) ^ code[i + 1]) & 0x0F0F0F0Fu;
      code[i] ^= d << 4;
      code[i + 1] ^= d;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ct[col0 + j][row0 >> 3] = code[j];
  }
  __syncthreads();
  if constexpr (ROW) {
    // row scales: a tile row's eight block bytes, one 8-byte piece per row of the tile
    if ((int)t < nr) {
      const uint64_t cols = (uint64_t)p.cols;
      uint8_t* sdst = p.scales_row + (uint64_t)(r0 + t) * (cols / 16) + (uint64_t)c0 / 16;
      const int nb = nc / 16;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < k2dBlocks; ++i) {
        const uint32_t v = kblk[((int)t / 16) * k2dBlocks + i] & 0xFFu;
        if (i < 4) lo |= v << (8 * i);
        else hi |= v << (8 * (i - 4));
      }
      if (nb == k2dBlocks && ((uintptr_t)sdst & 7u) == 0) {
        *reinterpret_cast<uint2*>(sdst) = make_uint2(lo, hi);
      } else {
        for (int i = 0; i < nb; ++i) sdst[i] = (uint8_t)((i < 4 ? lo >> (8 * i) : hi >> (8 * (i - 4))) & 0xFFu);
      }
    }
  }
  if constexpr (COL) {
    // column c leaves as nr / 2 bytes: four lanes x 16 bytes per column
    constexpr int kPieces = k2dTile * (k2dTile / 32);  // 16-byte pieces of the tile
#pragma unroll
    for (int k = 0; k < kPieces / k2dThreads; ++k) {
      const int pc = (int)t + k * k2dThreads;
      const int c = pc >> 2, h = pc & 3;  // column, 32-row group
      if (c < nc && h * 32 < nr) {
        uint8_t* cdst = p.codes_col + (uint64_t)(c0 + c) * (uint64_t)p.ld_col_codes + (uint64_t)(r0 + h * 32) / 2;
        if (h * 32 + 16 < nr) {
          store_nt(reinterpret_cast<uint4*>(cdst), make_uint4(ct[c][4 * h], ct[c][4 * h + 1], ct[c][4 * h + 2], ct[c][4 * h + 3]));
        } else {  // the tile's last 16 rows: 8 bytes (rows % 16 == 0 keeps the run 8-byte aligned)
          *reinterpret_cast<uint2*>(cdst) = make_uint2(ct[c][4 * h], ct[c][4 * h + 1]);
        }
      }
    }
    // column scales: one byte per 16 rows
    if ((int)t < nc) {
      uint8_t* sdst = p.scales_col + (uint64_t)(c0 + t) * (uint64_t)p.ld_col_scales + (uint64_t)r0 / 16;
      const int nb = nr / 16;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < k2dBlocks; ++i) {
        const uint32_t v = kblk[i * k2dBlocks + (int)t / 16] & 0xFFu;
        if (i < 4) lo |= v << (8 * i);
        else hi |= v << (8 * (i - 4));
      }
      if (nb == k2dBlocks && ((uintptr_t)sdst & 7u) == 0) {
        *reinterpret_cast<uint2*>(sdst) = make_uint2(lo, hi);
      } else {
        for (int i = 0; i < nb; ++i) sdst[i] = (uint8_t)((i < 4 ? lo >> (8 * i) : hi >> (8 * (i - 4))) & 0xFFu);
      }
    }
  }
}

template <typename T, bool ROW, bool COL>
hipError_t launch_2d_t(const TileLaunch& a, hipStream_t st) {
  // slabs of at most 2^22 tiles
  const int64_t tiles_per_row = (a.cols + k2dTile - 1) / k2dTile;
  const int64_t max_rows = (int64_t)k2dTile * std::max<int64_t>(1, ((int64_t)1 << 22) / tiles_per_row);
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
    p.tiles_r = (uint32_t)((nr + k2dTile - 1) / k2dTile);
    p.tiles_c = (uint32_t)tiles_per_row;
    p.sb_c = (p.tiles_c + 3u) / 4u;
    p.sbs = ((p.tiles_r + 3u) / 4u) * p.sb_c;
    const uint32_t grid = (p.sbs + 7u) / 8u * 128u;
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
