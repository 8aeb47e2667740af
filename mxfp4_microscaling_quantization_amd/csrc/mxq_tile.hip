// Column-wise (and fused row + column) quantisation from one read of the input.
//
// A 256-thread workgroup owns one tile (shape per variant, see TileShape; 32 KB of
// LDS, 64 KB for the fused MXFP4 tile). Phase 1: every thread loads 16-byte chunks
// (a wave reads whole 256- or 512-byte row segments per instruction), quantises
// them row-wise if asked (blocks along the row span a DPP quad, exactly as in the
// row kernel) and parks the raw values in LDS. Phase 2: a task is one column over
// 32 rows; the 32-row groups of a column sit on neighbouring lanes, so each store
// instruction writes a contiguous run of 16 bytes per group for each of its
// columns. The LDS tile is XOR-swizzled so that phase 2 reads hit all 32 banks,
// and the optional Hadamard transform runs along the rows in registers.
//
// Workgroups are dealt to the eight XCDs in turn; vertically adjacent tiles go to
// one XCD in consecutive turns, so the pieces of a 128-byte line of column codes
// are written through the same L2.
#include <algorithm>

#include "mxq_blocks.h"
#include "mxq_internal.h"

namespace mxq {

constexpr int kTileThreads = 256;
// Tile shape per variant, as measured on inputs read from HBM: 128 x 128 for the
// column-only and the NVFP4 kernels; the fused row + column MXFP4 kernels use 256
// columns, so each row's codes leave as a whole 128-byte line (128 rows, or 64 with
// the Hadamard transform, whose heavier register use favours the smaller tile).
// fp32 tiles have half the rows. V vertically adjacent tiles (256 rows of bf16) are
// dealt to the same XCD in consecutive turns.
template <typename T, int FMT, bool RHT, bool ROW>
struct TileShape {
  static constexpr bool kWide = ROW && FMT == kMX;
  static constexpr int C = kWide ? 256 : 128;                // a multiple of 64
  static constexpr int R16 = kWide && RHT ? 64 : 128;        // rows for bf16 input
  static constexpr int R = sizeof(T) == 2 ? R16 : R16 / 2;  // at least 32
  static constexpr int G = R / 32;                           // 32-row groups of a column
  static constexpr int V = 256 / R16;
};

struct TileParams {
  const void* x;
  int64_t ldx;
  int64_t rows, cols;          // slab extent
  int64_t total_rows;          // whole tensor (column-wise SR index and strides)
  int64_t row0;                // slab's first row in the whole tensor
  uint32_t tiles_r, tiles_c;   // tiles down and across the slab
  uint32_t groups;             // groups of kVGroup vertically adjacent tiles
  uint32_t sign_mask;
  uint64_t sr_seed, sr_offset;
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col;
  int64_t ld_col_codes, ld_col_scales;
  const float* amax;
  int st_given;      // *amax holds the tensor scale, not the amax
  float* tensor_scale;
};

__device__ __forceinline__ float absmax32(const float* v) {
  float m = __builtin_elementwise_maximum(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
#pragma unroll
  for (int i = 2; i < 32; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[i]));
  return m;
}

// MXFP4 encode of 32 values held by one thread (real values times 2^kShift);
// codes into 4 dwords, returns the block byte.
template <bool SR, int kShift, bool kBf16 = false>
__device__ __forceinline__ uint32_t mx_encode32(const float* v, const uint32_t* u, uint32_t out[4]) {
  const uint32_t byte = mx_byte<kShift>(as_u(absmax32(v)));
  const uint32_t b = min(byte, 252u);
  if constexpr (SR) {
    const float inv = as_f((254u - b - kShift) << 23);  // exact: a window of K = 1 suffices
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (kBf16 && kShift == 0) {
        uint32_t packed;
        if (mx_sr_hw8(v + 8 * d, u + 8 * d, b, packed)) {
          out[d] = byte == 255u ? 0u : packed;
          continue;
        }
      }
      float q[8];
      uint32_t low = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float q0, q1;
        e2m1_sr_carry2<1>(fabsf(v[d * 8 + i]) * inv, fabsf(v[d * 8 + i + 1]) * inv, u[d * 8 + i], u[d * 8 + i + 1],
                          low, q0, q1);
        q[i] = with_sign_of(q0, v[d * 8 + i]);
        q[i + 1] = with_sign_of(q1, v[d * 8 + i + 1]);
      }
      if (low < 2u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = with_sign_of(e2m1_sr_value(fabsf(v[d * 8 + i]) * inv, u[d * 8 + i]), v[d * 8 + i]);
      }
      out[d] = byte == 255u ? 0u : fp4x8_from_f32(q, 1.0f);
    }
  } else {
    const float scale = e8m0_operand(b + kShift);
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = byte == 255u ? 0u : fp4x8_from_f32(v + 8 * d, scale);
  }
  return byte;
}

// NVFP4 encode of one 16-block held by one thread; codes into 2 dwords.
template <bool SR>
__device__ __forceinline__ uint32_t nv_encode16(const float* v, const uint32_t* u, const NvTensor& t,
                                                uint32_t out[2]) {
  if (t.mode != 0) {
    out[0] = t.mode == 2 ? 0u : fp4x8_from_f32(v, 0.0f) & 0x88888888u;
    out[1] = t.mode == 2 ? 0u : fp4x8_from_f32(v + 8, 0.0f) & 0x88888888u;
    return t.mode == 2 ? 0x7Fu : 0u;
  }
  const float am = __builtin_elementwise_maximum(absmax8(v), absmax8(v + 8));
  const uint32_t amb = as_u(am) & 0x7FFFFFFFu;
  const bool nanb = amb >= 0x7F800000u;
  const uint32_t k = nv_block_scale_fast(ldexpf(as_f(nanb ? 0u : amb), -t.et), t.st_n);
  if constexpr (SR) {
    out[0] = nv_codes8_sr(v, u, t, max(k, 1u));
    out[1] = nv_codes8_sr(v + 8, u + 8, t, max(k, 1u));
  } else {
    out[0] = nv_codes8_rne(v, t, max(k, 1u));
    out[1] = nv_codes8_rne(v + 8, t, max(k, 1u));
  }
  if (k == 0u) {
    out[0] &= 0x88888888u;
    out[1] &= 0x88888888u;
  }
  if (nanb) out[0] = out[1] = 0u;
  return nanb ? 0x7Fu : k;
}

// LDS column index of element column c in tile row r. Phase 2 reads, at one
// instant, columns 16a .. 16a+15 in rows 32h + i for h = 0..3 (rows 32 apart start
// on the same bank); XOR-ing the column with 16h spreads those 64 lanes over all
// 32 banks (bf16; fp32 rows span two bank sweeps and see at most two-way sharing).
// Chunks of eight columns stay contiguous.
template <int G>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ (((r >> 5) & (G - 1)) * (64 / G));
}

template <typename T, int FMT, int SR, bool RHT, bool ROW, bool COL>
__global__ __launch_bounds__(kTileThreads) void quantize_tile_kernel(TileParams p) {
  // LDS tile of raw input values, row-major [128][128], XOR-swizzled columns
  using Shape = TileShape<T, FMT, RHT, ROW>;
  constexpr int kTileR = Shape::R, kTileC = Shape::C, kRowGroups = Shape::G, kVGroup = Shape::V;
  __shared__ T tile[kTileR][kTileC] __attribute__((aligned(16)));  // written as 16-byte chunks
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  const uint32_t t = threadIdx.x;
  NvTensor nt;
  if constexpr (FMT == kNV) {
    nt = nv_tensor_load(p.amax, p.st_given);
    if (p.tensor_scale && blockIdx.x == 0 && t == 0) *p.tensor_scale = nt.st;
    if constexpr (RHT) nv_tensor_times4(nt);
  }
  SignFlips flips;
  if constexpr (RHT && ROW) flips = make_flips<T>(p.sign_mask, t & 1u);
  constexpr int kChunks = kTileR * kTileC / 8 / kTileThreads;  // chunks per thread
  constexpr int kChunksPerRow = kTileC / 8;

  // tile origin and extent within the slab
  // Workgroups are dealt to the eight XCDs in turn (blockIdx mod 8). The kVGroup
  // tiles of one vertical group go to the same XCD in consecutive turns, so the
  // column codes they share in a 128-byte line meet in one L2.
  const uint32_t xcd = blockIdx.x & 7u, slot = blockIdx.x >> 3;
  const uint32_t g = (slot / kVGroup) * 8u + xcd;
  if (g >= p.groups) return;
  const uint32_t gr = g / p.tiles_c, tc = g - gr * p.tiles_c;
  const uint32_t tr = gr * kVGroup + slot % kVGroup;
  if (tr >= p.tiles_r) return;
  const int64_t r0 = (int64_t)tr * kTileR, c0 = (int64_t)tc * kTileC;
  const int nr = (int)std::min<int64_t>(kTileR, p.rows - r0);
  const int nc = (int)std::min<int64_t>(kTileC, p.cols - c0);
  // A thread keeps its chunk column cc for every chunk j; its row advances by kRowStep.
  constexpr int kRowStep = kTileThreads / kChunksPerRow;
  const int cc = (int)(t % kChunksPerRow), row_t = (int)(t / kChunksPerRow);
  const bool col_ok = cc * 8 < nc;
  const T* xt = x + (uint64_t)(r0 + row_t) * (uint64_t)p.ldx + (uint64_t)(c0 + cc * 8);
  Raw<T> cur[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    if (row_t + j * kRowStep < nr && col_ok) load_raw(xt, (uint64_t)(j * kRowStep) * (uint64_t)p.ldx, cur[j]);
    else zero_raw(cur[j]);
  }

  // ---- phase 1: row-wise quantise (optional), park raw values in LDS
  constexpr int bs = FMT == kMX ? 32 : 16;
  static_assert(kRowStep % 8 == 0, "rows of one thread differ by multiples of 8");
  const uint32_t csign0 = (p.sign_mask >> (row_t & 15)) & 1u;
  const uint32_t csign1 = (p.sign_mask >> ((row_t + 8) & 15)) & 1u;
  const uint64_t col = (uint64_t)(c0 + cc * 8);
  const uint64_t cols = (uint64_t)p.cols;
  uint8_t* crow = nullptr;
  uint8_t* srow = nullptr;
  if constexpr (ROW) {
    const uint64_t lr = (uint64_t)(r0 + row_t);  // row within the slab
    crow = p.codes_row + lr * (cols >> 1) + (col >> 1);
    srow = p.scales_row + lr * (cols / bs) + col / bs;
  }
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int row = row_t + j * kRowStep;
    if constexpr (RHT && COL) {
      // the column transform's sign of this row (its position mod 16 along the
      // column) is applied here, once per stored chunk; kRowStep is a multiple of
      // 8, so a thread's rows take two positions mod 16
      Raw<T> sr = cur[j];
      flip_all(sr, ((j * kRowStep) & 8) ? csign1 : csign0);
      *reinterpret_cast<Raw<T>*>(&tile[row][swz<kRowGroups>(row, cc * 8)]) = sr;
    } else {
      *reinterpret_cast<Raw<T>*>(&tile[row][swz<kRowGroups>(row, cc * 8)]) = cur[j];
    }
    if constexpr (ROW) {
      Raw<T> rr = cur[j];
      if constexpr (RHT) flip(rr, flips);
      float v[8];
      to_f32(rr, v);
      if constexpr (RHT) h16_pair(v, t & 1u);
      uint32_t u[8];
      if constexpr (SR != kRne) {
        const uint64_t grow = (uint64_t)(p.row0 + r0 + row);
        sr_values<SR, 8>(p.sr_offset + grow * cols + col, p.sr_seed, u);
      }
      uint32_t byte, packed;
      if constexpr (FMT == kMX) packed = mx_encode8<SR != kRne, RHT ? 2 : 0, sizeof(T) == 2 && !RHT>(v, u, byte);
      else packed = nv_encode8<SR != kRne>(v, u, nt, byte);
      if (row < nr && col_ok) {
        *reinterpret_cast<uint32_t*>(crow + (uint64_t)(j * kRowStep) * (cols >> 1)) = packed;
        if (col % bs == 0) srow[(uint64_t)(j * kRowStep) * (cols / bs)] = (uint8_t)byte;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: one column over 32 rows per task, (kTileC x kRowGroups) tasks.
  // Neighbouring lanes hold the 32-row groups of one column, so a store
  // instruction writes kRowGroups x 16 contiguous bytes per column.
  if constexpr (COL) {
#pragma unroll 1
    for (int k = t; k < kTileC * kRowGroups; k += kTileThreads) {
      const int c = k / kRowGroups;
      const int h = k % kRowGroups;
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        // the Hadamard signs were applied when the tile was stored
        const int r = h * 32 + i;
        if constexpr (sizeof(T) == 2) v[i] = as_f((uint32_t)tile[r][swz<kRowGroups>(r, c)] << 16);
        else v[i] = tile[r][swz<kRowGroups>(r, c)];
      }
      if constexpr (RHT) {
        h16_local(v);
        h16_local(v + 16);
      }
      const int vrows = nr - h * 32;  // valid rows of this 32-row group
      const int64_t col = c0 + c;
      if (vrows > 0 && c < nc) {
        const int64_t grow0 = p.row0 + r0 + h * 32;  // first row of the group in the whole tensor
        uint32_t u[32];
        sr_values<SR, 32>(p.sr_offset + (uint64_t)(col * p.total_rows + grow0), p.sr_seed, u);
        uint8_t* cdst = p.codes_col + col * p.ld_col_codes + grow0 / 2;
        uint8_t* sdst = p.scales_col + col * p.ld_col_scales;
        if constexpr (FMT == kMX) {
          uint32_t out[4];
          const uint32_t byte = mx_encode32<SR != kRne, RHT ? 2 : 0, sizeof(T) == 2 && !RHT>(v, u, out);
          *reinterpret_cast<uint4*>(cdst) = make_uint4(out[0], out[1], out[2], out[3]);
          sdst[grow0 / 32] = (uint8_t)byte;
        } else {
          uint32_t out[4];
          const uint32_t b0 = nv_encode16<SR != kRne>(v, u, nt, out);
          const uint32_t b1 = nv_encode16<SR != kRne>(v + 16, u + 16, nt, out + 2);
          // 8-byte stores: rows % 16 == 0 only guarantees 8-byte aligned column runs
          *reinterpret_cast<uint2*>(cdst) = make_uint2(out[0], out[1]);
          sdst[grow0 / 16] = (uint8_t)b0;
          if (vrows >= 32) {
            *reinterpret_cast<uint2*>(cdst + 8) = make_uint2(out[2], out[3]);
            sdst[grow0 / 16 + 1] = (uint8_t)b1;
          }
        }
      }
    }
  }
}

template <typename T, int FMT, int SR, bool RHT, bool ROW>
static hipError_t launch_tiles_shape(const TileLaunch& a, hipStream_t st) {
  using Shape = TileShape<T, FMT, RHT, ROW>;
  constexpr int kTileR = Shape::R, kTileC = Shape::C, kVGroup = Shape::V;
  // slabs of at most 2^22 tiles (cols <= 2^30 gives at most 2^23 tiles per tile row)
  const int64_t tiles_per_row = (a.cols + kTileC - 1) / kTileC;
  const int64_t max_rows = (int64_t)kTileR * std::max<int64_t>(1, ((int64_t)1 << 22) / tiles_per_row);
  for (int64_t s0 = 0; s0 < a.rows; s0 += max_rows) {
    const int64_t nr = std::min(max_rows, a.rows - s0);
    TileParams p;
    const size_t esz = sizeof(T);
    p.x = reinterpret_cast<const uint8_t*>(a.x) + (size_t)s0 * a.ldx * esz;
    p.ldx = a.ldx;
    p.rows = nr;
    p.cols = a.cols;
    p.total_rows = a.total_rows;
    p.row0 = a.row0 + s0;
    const int64_t tiles_r = (nr + kTileR - 1) / kTileR;
    const int64_t tiles_c = (a.cols + kTileC - 1) / kTileC;
    p.tiles_r = (uint32_t)tiles_r;
    p.tiles_c = (uint32_t)tiles_c;
    p.groups = (uint32_t)(((tiles_r + kVGroup - 1) / kVGroup) * tiles_c);
    p.sign_mask = a.sign_mask;
    p.sr_seed = a.sr_seed;
    p.sr_offset = a.sr_offset;
    const int bs = FMT == kMX ? 32 : 16;
    p.codes_row = a.codes_row ? a.codes_row + s0 * (a.cols / 2) : nullptr;
    p.scales_row = a.scales_row ? a.scales_row + s0 * (a.cols / bs) : nullptr;
    p.codes_col = a.codes_col;
    p.scales_col = a.scales_col;
    p.ld_col_codes = a.ld_col_codes;
    p.ld_col_scales = a.ld_col_scales;
    p.amax = a.amax;
    p.st_given = a.st_given ? 1 : 0;
    p.tensor_scale = s0 == 0 ? a.tensor_scale : nullptr;
    const uint32_t grid = 8u * kVGroup * ((p.groups + 7u) / 8u);
    hipLaunchKernelGGL((quantize_tile_kernel<T, FMT, SR, RHT, ROW, true>), dim3(grid), dim3(kTileThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int FMT, int SR, bool RHT>
static hipError_t launch_tiles_t(const TileLaunch& a, hipStream_t st) {
  return a.want_row ? launch_tiles_shape<T, FMT, SR, RHT, true>(a, st)
                    : launch_tiles_shape<T, FMT, SR, RHT, false>(a, st);
}

template <typename T, int FMT>
static hipError_t launch_tiles_f(const TileLaunch& a, hipStream_t st) {
  if (a.sr == kSrWords)
    return a.rht ? launch_tiles_t<T, FMT, kSrWords, true>(a, st) : launch_tiles_t<T, FMT, kSrWords, false>(a, st);
  if (a.sr == kSrHalves)
    return a.rht ? launch_tiles_t<T, FMT, kSrHalves, true>(a, st) : launch_tiles_t<T, FMT, kSrHalves, false>(a, st);
  return a.rht ? launch_tiles_t<T, FMT, kRne, true>(a, st) : launch_tiles_t<T, FMT, kRne, false>(a, st);
}

hipError_t launch_quantize_tiles(const TileLaunch& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  if (a.dtype == 0)
    return a.fmt == kMX ? launch_tiles_f<uint16_t, kMX>(a, st) : launch_tiles_f<uint16_t, kNV>(a, st);
  return a.fmt == kMX ? launch_tiles_f<float, kMX>(a, st) : launch_tiles_f<float, kNV>(a, st);
}

}  // namespace mxq
