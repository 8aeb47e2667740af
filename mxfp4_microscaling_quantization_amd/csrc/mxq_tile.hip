// Column-wise (and fused row + column) quantisation from one read of the input.
//
// Two kernels. bf16 input with nearest-even rounding (MXFP4 both ways, NVFP4
// column-wise) walks 256-column strips (quantize_strip_kernel below): the column
// codes of 256 rows leave as whole 128-byte lines. Everything else (fp32 input,
// stochastic rounding, NVFP4 with both outputs) uses the tile kernel:
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
#include <type_traits>

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

// ---- Strip walker (bf16 input).
//
// A workgroup owns a strip of 256 columns and walks down it in 64-row steps, one
// flush unit of 256 rows after another. Each step: the raw tile goes to LDS (with
// the column transform's signs), the row-wise blocks are quantised from registers as
// in the tile kernel, and the column tasks (one column over 32 rows, two per thread)
// encode from LDS into registers. After four steps a column holds 256 rows of codes,
// one 128-byte line: the lines are assembled in LDS and leave as whole-line stores,
// and the column scales leave as one run per column. Row scales are staged in LDS
// and leave as one run per row. The next step's input is loaded while the current
// step's column tasks run.
constexpr int kStripC = 256;  // columns of a strip
constexpr int kStepR = 64;    // rows of a step
constexpr int kFlushR = 256;  // rows of a flush unit

struct StripParams {
  const uint16_t* x;
  int64_t ldx;
  int64_t rows, cols;     // slab extent
  int64_t row0;           // slab's first row in the whole tensor (a multiple of kFlushR)
  uint32_t strips;        // strips across the slab
  uint32_t flushes;       // flush units down the slab
  uint32_t per_wg;        // flush units per workgroup
  uint32_t units;         // workgroups down one strip
  uint32_t sign_mask;
  uint8_t *codes_row, *scales_row, *codes_col, *scales_col;
  int64_t ld_col_codes, ld_col_scales;
  const float* amax;
  int st_given;
  float* tensor_scale;
};

// Stores bytes [0, n) of an LDS run (16-byte aligned, n <= 16) at p: dword stores
// when p and n allow them, else byte stores.
__device__ __forceinline__ void store_run(uint8_t* p, const uint8_t* src, int n) {
  if ((((uintptr_t)p | (uintptr_t)n) & 3u) == 0) {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d = reinterpret_cast<uint32_t*>(p);
    if ((((uintptr_t)p) & 7u) == 0 && n >= 8) {
      *reinterpret_cast<uint2*>(d) = make_uint2(s[0], s[1]);
      if (n == 12) d[2] = s[2];
      if (n == 16) *reinterpret_cast<uint2*>(d + 2) = make_uint2(s[2], s[3]);
    } else {
      for (int i = 0; i < (n >> 2); ++i) d[i] = s[i];
    }
  } else {
    for (int i = 0; i < n; ++i) p[i] = src[i];
  }
}

// The lane index as a value the compiler cannot see through: per-lane addresses
// derived from it are recomputed where they are used instead of being held in
// registers across the whole walk.
__device__ __forceinline__ uint32_t opaque_lane() {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Four workgroups per CU (what the 37 KB of LDS allows): the register bound this asks
// for (128) fits every variant without spills.
template <int FMT, int SR, bool RHT, bool ROW>
__global__ __launch_bounds__(kTileThreads, 4) void quantize_strip_kernel(StripParams p) {
  static_assert(SR == kRne, "the strip walk serves nearest-even rounding");
  constexpr int bs = FMT == kMX ? 32 : 16;
  constexpr int kChunksPerRow = kStripC / 8;                // 32 lanes per row
  constexpr int kRowStep = kTileThreads / kChunksPerRow;    // 8 rows between a thread's chunks
  constexpr int kChunks = kStepR / kRowStep;                // 8 chunks per thread and step
  static_assert(kRowStep == 8 && kChunks == 8, "chunk layout");
  // bf16 tile of a step (XOR-swizzled as in the tile kernel), then the column-code
  // lines of a flush unit (column c at c * 128, 16-byte slot s at (s ^ (c & 7)) * 16)
  __shared__ __attribute__((aligned(16))) uint8_t buf[kStepR * kStripC * 2];
  __shared__ __attribute__((aligned(16))) uint8_t rsc[kStepR * 16];   // row scales of a step
  __shared__ __attribute__((aligned(16))) uint8_t csc[kStripC * 16];  // column scales of a flush unit
  NvTensor nt;
  if constexpr (FMT == kNV) {
    nt = nv_tensor_load(p.amax, p.st_given);
    if (p.tensor_scale && blockIdx.x == 0 && threadIdx.x == 0) *p.tensor_scale = nt.st;
    if constexpr (RHT) nv_tensor_times4(nt);
  }

  const uint32_t unit = blockIdx.x / p.strips, strip = blockIdx.x - unit * p.strips;
  if (unit >= p.units) return;
  const uint32_t f0 = unit * p.per_wg, f1 = min(f0 + p.per_wg, p.flushes);
  const int64_t c0 = (int64_t)strip * kStripC;
  const int nc = (int)std::min<int64_t>(kStripC, p.cols - c0);
  const uint64_t ldx = (uint64_t)p.ldx;
  const uint64_t cols = (uint64_t)p.cols;

  // A thread's chunks: column cc * 8 of the strip, rows row_t + 8 j of the step.
  Raw<uint16_t> cur[kChunks];
  auto load_chunk = [&](int64_t r0, int j, uint32_t t) {
    const int cc = (int)(t % kChunksPerRow), row_t = (int)(t / kChunksPerRow);
    const int nr = (int)std::min<int64_t>(kStepR, p.rows - r0);
    const uint16_t* xs = p.x + (uint64_t)(r0 + row_t) * ldx + (uint64_t)c0 + (uint64_t)(cc * 8);
    if (row_t + j * kRowStep < nr && cc * 8 < nc) load_raw(xs, (uint64_t)(j * kRowStep) * ldx, cur[j]);
    else zero_raw(cur[j]);
  };
  auto load_step = [&](int64_t r0) {
    const uint32_t t = opaque_lane();
#pragma unroll
    for (int j = 0; j < kChunks; ++j) load_chunk(r0, j, t);
  };
  load_step((int64_t)f0 * kFlushR);

#pragma unroll 1
  for (uint32_t f = f0; f < f1; ++f) {
    const int64_t fr = (int64_t)f * kFlushR;
    const int vrows = (int)std::min<int64_t>(kFlushR, p.rows - fr);  // valid rows of the unit
    uint32_t acc[4][2][4] = {};  // steps past the last row stay zero
    uint32_t scol[2][2] = {{0u, 0u}, {0u, 0u}};  // column scale bytes of the unit's steps
    // the four steps of the unit, written out (a compile-time step index keeps the
    // code registers statically addressed)
    auto step = [&](auto sq_c) {
      constexpr int sq = decltype(sq_c)::value;
      const int64_t r0 = fr + sq * kStepR;
      if (r0 < p.rows) {
        const int nr = (int)std::min<int64_t>(kStepR, p.rows - r0);
        __syncthreads();  // the previous step's (or flush's) LDS reads are done
        // ---- phase 1: park the raw tile, quantise rows from registers
        {
          const uint32_t t = opaque_lane();
          const int cc = (int)(t % kChunksPerRow), row_t = (int)(t / kChunksPerRow);
          const bool col_ok = cc * 8 < nc;
          const uint64_t col = (uint64_t)c0 + (uint64_t)(cc * 8);
          // rows row_t + 8 j lie in the first 32-row group for j < 4 and in the
          // second for j >= 4 (swizzled column cc * 8 ^ 32)
          uint8_t* const wr0 = buf + (row_t * kStripC + cc * 8) * 2;
          uint8_t* const wr1 = buf + (row_t * kStripC + ((cc * 8) ^ 32)) * 2;
          uint8_t* const crow = ROW ? p.codes_row + (uint64_t)(r0 + row_t) * (cols >> 1) + (col >> 1) : nullptr;
#pragma unroll
          for (int j = 0; j < kChunks; ++j) {
            const int row = row_t + j * kRowStep;
            uint8_t* const w = (j < 4 ? wr0 : wr1) + j * kRowStep * kStripC * 2;
            if constexpr (RHT) {
              // the column transform's sign of this row (its position mod 16)
              Raw<uint16_t> sr = cur[j];
              flip_all(sr, (p.sign_mask >> ((row_t + 8 * (j & 1)) & 15)) & 1u);
              *reinterpret_cast<Raw<uint16_t>*>(w) = sr;
            } else {
              *reinterpret_cast<Raw<uint16_t>*>(w) = cur[j];
            }
            if constexpr (ROW) {
              Raw<uint16_t> rr = cur[j];
              if constexpr (RHT) flip(rr, make_flips<uint16_t>(p.sign_mask, t & 1u));
              float v[8];
              to_f32(rr, v);
              if constexpr (RHT) h16_pair(v, t & 1u);
              uint32_t byte, packed;
              if constexpr (FMT == kMX) packed = mx_encode8<false, RHT ? 2 : 0, !RHT>(v, nullptr, byte);
              else packed = nv_encode8<false>(v, nullptr, nt, byte);
              if (row < nr && col_ok) {
                *reinterpret_cast<uint32_t*>(crow + (uint64_t)(j * kRowStep) * (cols >> 1)) = packed;
                if ((cc * 8) % bs == 0) rsc[row * 16 + (cc * 8) / bs] = (uint8_t)byte;
              }
            }
          }
        }
        // next step's input, in flight while the column tasks run
        asm volatile("" ::: "memory");
        if (r0 + kStepR < p.rows && (sq < 3 || f + 1 < f1)) load_step(r0 + kStepR);
        __syncthreads();
        const uint32_t t = opaque_lane();
        if constexpr (ROW) {
          if ((int)t < nr)
            store_run(p.scales_row + (uint64_t)(r0 + t) * (cols / bs) + (uint64_t)c0 / bs, rsc + t * 16, nc / bs);
        }
        // ---- phase 2: column tasks (column k / 2, 32-row group k % 2 for k = t + 256 m),
        // codes to registers. Group h reads rows 32 h .. 32 h + 31, whose swizzled
        // column is c ^ 32 h; column c + 128 sits 256 bytes further.
        const int h = (int)(t & 1u);
        const uint8_t* const rd = buf + (h * 32 * kStripC + (((int)(t >> 1)) ^ (32 * h))) * 2;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float v[32];
#pragma unroll
          for (int i = 0; i < 32; ++i)
            v[i] = as_f((uint32_t)(*reinterpret_cast<const uint16_t*>(rd + 256 * m + i * kStripC * 2)) << 16);
          if constexpr (RHT) {
            h16_local(v);
            h16_local(v + 16);
          }
          if constexpr (FMT == kMX) {
            const uint32_t byte = mx_encode32<false, RHT ? 2 : 0, !RHT>(v, nullptr, acc[sq][m]);
            scol[m][0] |= byte << (8 * sq);
          } else {
            const uint32_t b0 = nv_encode16<false>(v, nullptr, nt, acc[sq][m]);
            const uint32_t b1 = nv_encode16<false>(v + 16, nullptr, nt, acc[sq][m] + 2);
            scol[m][sq >> 1] |= (b0 | (b1 << 8)) << (16 * (sq & 1));
          }
          // keep one task's values from being held across the next task's reads
          asm volatile("" ::"v"(acc[sq][m][0]), "v"(acc[sq][m][1]), "v"(acc[sq][m][2]), "v"(acc[sq][m][3]) : "memory");
        }
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    // ---- flush: whole 128-byte lines of column codes, one scale run per column.
    // Task (c, h) has c = t / 2 + 128 m, so c & 7 does not depend on m: the line
    // slot of step q is (2 q + h) ^ (c & 7).
    __syncthreads();
    {
      const uint32_t t = opaque_lane();
      const int ch = (int)(t >> 1), h = (int)(t & 1u), sw = ch & 7;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int c = ch + 128 * m;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<uint4*>(buf + c * 128 + (((2 * q + h) ^ sw) * 16)) =
              make_uint4(acc[q][m][0], acc[q][m][1], acc[q][m][2], acc[q][m][3]);
          if constexpr (FMT == kMX) csc[c * 16 + 2 * q + h] = (uint8_t)(scol[m][0] >> (8 * q));
          else *reinterpret_cast<uint16_t*>(csc + c * 16 + 4 * q + 2 * h) = (uint16_t)(scol[m][q >> 1] >> (16 * (q & 1)));
        }
      }
    }
    __syncthreads();
    {
      // piece j = t % 8 of column t / 8 + 32 it: one LDS base and one global base
      const uint32_t t = opaque_lane();
      const int c8 = (int)(t >> 3), j = (int)(t & 7u);
      const int left = vrows - 32 * j;  // valid rows of the piece's 32-row group
      const uint8_t* lsrc = buf + c8 * 128 + ((j ^ (c8 & 7)) * 16);
      uint8_t* dst = p.codes_col + (uint64_t)(c0 + c8) * (uint64_t)p.ld_col_codes + (uint64_t)(p.row0 + fr) / 2 + 16 * j;
      const uint64_t dstep = 32 * (uint64_t)p.ld_col_codes;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        if (c8 + 32 * it < nc && left > 0) {
          const uint4 w = *reinterpret_cast<const uint4*>(lsrc + it * 32 * 128);
          uint8_t* d = dst + it * dstep;
          if (FMT == kMX || (left >= 32 && ((uintptr_t)d & 15u) == 0)) {
            *reinterpret_cast<uint4*>(d) = w;
          } else {
            // NVFP4 column runs are only 8-byte aligned; a group may hold 16 valid rows
            *reinterpret_cast<uint2*>(d) = make_uint2(w.x, w.y);
            if (left >= 32) *reinterpret_cast<uint2*>(d + 8) = make_uint2(w.z, w.w);
          }
        }
      }
      if ((int)t < nc)
        store_run(p.scales_col + (uint64_t)(c0 + t) * (uint64_t)p.ld_col_scales + (uint64_t)(p.row0 + fr) / bs,
                  csc + t * 16, vrows / bs);
    }
  }
}

template <int FMT, int SR, bool RHT, bool ROW>
static hipError_t launch_strips(const TileLaunch& a, hipStream_t st) {
  const int64_t strips = (a.cols + kStripC - 1) / kStripC;
  // slabs of at most 2^22 workgroups, on flush-unit boundaries
  const int64_t max_rows = (int64_t)kFlushR * std::max<int64_t>(1, ((int64_t)1 << 22) / strips);
  for (int64_t s0 = 0; s0 < a.rows; s0 += max_rows) {
    const int64_t nr = std::min(max_rows, a.rows - s0);
    StripParams p;
    p.x = reinterpret_cast<const uint16_t*>(a.x) + (size_t)s0 * a.ldx;
    p.ldx = a.ldx;
    p.rows = nr;
    p.cols = a.cols;
    p.row0 = s0;
    p.strips = (uint32_t)strips;
    const int64_t flushes = (nr + kFlushR - 1) / kFlushR;
    p.flushes = (uint32_t)flushes;
    // about four resident workgroups per CU on 256 CUs; longer walks once that is met
    p.per_wg = (uint32_t)std::min<int64_t>(4, std::max<int64_t>(1, flushes * strips / 1024));
    p.units = (uint32_t)((flushes + p.per_wg - 1) / p.per_wg);
    p.sign_mask = a.sign_mask;
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
    const uint32_t grid = p.units * p.strips;
    hipLaunchKernelGGL((quantize_strip_kernel<FMT, SR, RHT, ROW>), dim3(grid), dim3(kTileThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int FMT, int SR, bool RHT, bool ROW>
static hipError_t launch_tiles_shape(const TileLaunch& a, hipStream_t st) {
  // bf16 with nearest-even rounding walks strips (NVFP4 column-wise only); stochastic
  // rounding's random words and the NVFP4 row side need more registers than the
  // walk leaves for four resident workgroups per CU, and stay on tiles.
  if constexpr (sizeof(T) == 2 && SR == kRne && !(FMT == kNV && ROW)) {
    return launch_strips<FMT, SR, RHT, ROW>(a, st);
  } else {
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
      p.row0 = s0;
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
