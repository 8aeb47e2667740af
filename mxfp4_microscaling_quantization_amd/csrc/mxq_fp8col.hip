// MXFP4 rows -> FP8 columns: the fused dequantise / transpose / requantise step that
// feeds the weight gradient of MoE experts ("Practical FP4 Training for Large-Scale
// MoE Models on Hopper GPUs", section 2C: one kernel fuses the three steps, ragged
// per-expert token counts are handled through precomputed offsets with no padding).
//
// Input: row-wise MXFP4 of X [R, C] whose rows are tokens grouped by expert. Output:
// X^T [C, R] in E4M3 with one power-of-two fp32 scale per 128 consecutive tokens of
// one expert in one column (the expert's last group keeps the remainder), the
// smallest that keeps the group within 448; a group that meets a NaN block gets a
// NaN scale and codes 0x7F.
//
// A workgroup owns one 128-token group and 256 columns:
//  1. it finds its expert and group from the offsets (each workgroup scans the
//     per-expert group counts; the offsets are clamped to [0, R], so malformed
//     offsets cannot address outside the tensors);
//  2. thread (ig, cj) loads 16 tokens x 8 columns: 16 dwords of codes (a wave reads
//     whole 128-byte lines of two 16-token strips) and the 16 scale bytes;
//  3. the column maxima are reduced through LDS (|x| as fp32 bits compare as
//     integers); thread c then turns column c's maximum into the scale exponent;
//  4. each thread converts its 16 x 8 elements; two tokens of one column go through
//     one E4M3 conversion, so a dword holds four consecutive tokens of a column and
//     the tile lands in LDS already transposed (column-major, 16-byte writes);
//  5. each column's run of n bytes is written in 16-byte aligned pieces (the run
//     starts wherever the expert starts; the pieces at both ends are partial).
//
// Elements are dequantised exactly with the scaled FP4 conversion and requantised
// with the scaled FP8 conversion (a power-of-two scale, one rounding to nearest
// even). That needs normal fp32 values and in-range scale exponents: whenever a
// nonzero block of the group has a scale byte outside [10, 252] (values beyond any
// bf16/fp32 input's quantisation), the workgroup takes an exact integer path
// instead.
#include <algorithm>

#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int kRcThreads = 256;
constexpr int kRcCols = 256;       // columns per workgroup
constexpr int kRcGroup = 128;      // tokens per FP8 group
constexpr int kRcStride = 144;     // LDS bytes per column: 16 guard bytes + 128 tokens
constexpr int kRcTileBytes = kRcCols * kRcStride + 32;  // + slack for the realigning reads

struct RcParams {
  const uint8_t* codes;     // [rows, cols/2]
  const uint8_t* e8m0;      // [rows, cols/32]
  const int64_t* offsets;   // [n_experts + 1]
  uint8_t* q8;              // [cols, ld_q8]
  uint32_t* s;              // [cols, ld_s]
  int64_t rows, cols, ld_q8, ld_s;
  int n_experts;
  uint32_t groups;          // group slots
  uint32_t tiles_c;         // 256-column tiles
  uint32_t per_xcd;         // workgroups per XCD
};

__device__ __forceinline__ int64_t clamp_token(int64_t v, int64_t rows) {
  return v < 0 ? 0 : (v > rows ? rows : v);
}

// fp32 bits of 2^k for -149 <= k <= 127.
__device__ __forceinline__ uint32_t pow2_bits(int k) {
  return k >= -126 ? (uint32_t)(k + 127) << 23 : 1u << (k + 149);
}

// Exact E4M3 magnitude code of v(m) 2^(8-d): a nonzero E2M1 magnitude m (1..7)
// whose binade lies d >= 0 below the group's top binade, under the scale 2^(F-8).
__device__ __forceinline__ uint32_t e4m3_of_shifted_e2m1(uint32_t m, int d) {
  const uint32_t f = m >= 2u ? (m & 1u) : 0u;  // the E2M1 mantissa bit
  if (d <= 14) return ((uint32_t)(15 - d) << 3) | (f << 2);
  const uint32_t num = 2u + f;  // (2 + f) 2^(16-d) quanta of 2^-9
  if (d <= 16) return num << (16 - d);
  const int sh = min(d - 16, 8);
  const uint32_t q = num >> sh, rem = num & ((1u << sh) - 1u), half = 1u << (sh - 1);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

// Integer key of an element for the exact path: E + floor(log2 v(m)) + 128 for a
// nonzero magnitude (>= 128), 0 for zero. Keys order like the magnitudes' binades.
__device__ __forceinline__ uint32_t binade_key(uint32_t m, uint32_t e) {
  return m ? e + (m >> 1) + 128u : 0u;
}

// Finds the expert and group of group slot gi: first token and token count (0 when
// the slot is past the last group). All threads take part; the result is uniform.
__device__ void find_group(const RcParams& p, uint32_t gi, int64_t& t0, int& n) {
  __shared__ uint32_t wave_tot[kRcThreads / 64];
  __shared__ int64_t sel_t0;
  __shared__ int sel_n;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (p.n_experts + kRcThreads - 1) / kRcThreads;
  const int e0 = min(t * per, p.n_experts), e1 = min(e0 + per, p.n_experts);
  uint32_t sum = 0;
  for (int e = e0; e < e1; ++e) {
    const int64_t lo = clamp_token(p.offsets[e], p.rows), hi = clamp_token(p.offsets[e + 1], p.rows);
    sum += hi > lo ? (uint32_t)((hi - lo + kRcGroup - 1) / kRcGroup) : 0u;
  }
  // inclusive scan over the wave, then over the waves
  uint32_t inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t v = __shfl_up(inc, d, 64);
    if (lane >= d) inc += v;
  }
  if (t == 0) sel_n = 0;
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const uint32_t excl = before + inc - sum;
  if (gi >= excl && gi < excl + sum) {
    uint32_t g = gi - excl;
    for (int e = e0; e < e1; ++e) {
      const int64_t lo = clamp_token(p.offsets[e], p.rows), hi = clamp_token(p.offsets[e + 1], p.rows);
      const uint32_t cnt = hi > lo ? (uint32_t)((hi - lo + kRcGroup - 1) / kRcGroup) : 0u;
      if (g < cnt) {
        sel_t0 = lo + (int64_t)g * kRcGroup;
        sel_n = (int)std::min<int64_t>(kRcGroup, hi - sel_t0);
        break;
      }
      g -= cnt;
    }
  }
  __syncthreads();
  t0 = sel_t0;
  n = sel_n;
}

__global__ __launch_bounds__(kRcThreads) void fp4_row_to_fp8_col_kernel(RcParams p) {
  __shared__ uint4 tile_q[kRcTileBytes / 16];         // transposed E4M3, column-major
  __shared__ uint32_t red[8][kRcCols];                // per-strip column maxima
  __shared__ uint8_t nanred[8][kRcCols / 8];          // per-strip NaN flags (per 8 columns)
  __shared__ int col_k[kRcCols];                      // scale exponent of each column
  __shared__ uint8_t col_nan[kRcCols];
  uint8_t* tile = reinterpret_cast<uint8_t*>(tile_q);

  // XCD-aware order: the workgroups of one XCD take consecutive group slots of one
  // column tile, so the pieces two neighbouring groups share meet in one L2
  const uint32_t L = (blockIdx.x & 7u) * p.per_xcd + (blockIdx.x >> 3);
  if (L >= p.groups * p.tiles_c) return;
  const uint32_t tc = L / p.groups, gi = L - tc * p.groups;

  int64_t t0;
  int n;
  find_group(p, gi, t0, n);
  if (n == 0) return;

  const int t = threadIdx.x, ig = t >> 5, cj = t & 31;
  const int64_t c0 = (int64_t)tc * kRcCols;
  const int nc = (int)std::min<int64_t>(kRcCols, p.cols - c0);
  const bool colv = 8 * cj < nc;

  // ---- load 16 tokens x 8 columns
  uint32_t w[16], e[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = 16 * ig + k;
    w[k] = 0u;
    e[k] = 127u;
    if (colv && r < n) {
      const int64_t row = t0 + r;
      w[k] = *reinterpret_cast<const uint32_t*>(p.codes + row * (p.cols / 2) + (c0 + 8 * cj) / 2);
      e[k] = p.e8m0[row * (p.cols / 32) + (c0 + 8 * cj) / 32];
    }
  }
  bool nan_l = false, slow_l = false;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    nan_l |= e[k] == 255u;
    slow_l |= (w[k] & 0x77777777u) != 0u && e[k] != 255u && (e[k] < 10u || e[k] > 252u);
  }
  const bool slow = __syncthreads_or(slow_l);

  // ---- column maxima: |x| as fp32 bits (fast) or binade keys (exact path)
  uint32_t cm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cm[j] = 0u;
  if (!slow) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float sc = e8m0_operand(e[k] == 255u ? 127u : e[k]);
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 0);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 1);
      const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 2);
      const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 3);
      const float v[8] = {a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j] = max(cm[j], as_u(v[j]) & 0x7FFFFFFFu);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (e[k] == 255u) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j] = max(cm[j], binade_key((w[k] >> (4 * j)) & 7u, e[k]));
    }
  }
  *reinterpret_cast<uint4*>(&red[ig][8 * cj]) = make_uint4(cm[0], cm[1], cm[2], cm[3]);
  *reinterpret_cast<uint4*>(&red[ig][8 * cj + 4]) = make_uint4(cm[4], cm[5], cm[6], cm[7]);
  nanred[ig][cj] = nan_l ? 1 : 0;
  __syncthreads();
  {
    uint32_t m = 0;
    bool nanc = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m = max(m, red[i][t]);
      nanc |= nanred[i][t >> 3] != 0;
    }
    // top binade F of the column's largest magnitude; scale 2^(F-8) (k = 0 if all zero)
    int k = 0;
    if (m) k = (slow ? (int)m - 256 : (int)(m >> 23) - 127) - 8;
    col_k[t] = k;
    col_nan[t] = nanc ? 1 : 0;
    if (t < nc) p.s[(c0 + t) * p.ld_s + gi] = nanc ? 0x7FC00000u : pow2_bits(k);
  }
  __syncthreads();

  // ---- convert: dword q of column j holds tokens 4q..4q+3 of the thread's strip
  uint32_t out[8][4];
  if (!slow) {
    float sc_col[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sc_col[j] = e8m0_operand((uint32_t)(col_k[8 * cj + j] + 127));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * q + i;
        const float sc = e8m0_operand(e[k] == 255u ? 127u : e[k]);
        const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 0);
        const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 1);
        const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 2);
        const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 3);
        v[i][0] = a.x; v[i][1] = a.y; v[i][2] = b.x; v[i][3] = b.y;
        v[i][4] = c.x; v[i][5] = c.y; v[i][6] = d.x; v[i][7] = d.y;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s16x2_t h = {0, 0};
        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, v[0][j], v[1][j], sc_col[j], false);
        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, v[2][j], v[3][j], sc_col[j], true);
        out[j][q] = __builtin_bit_cast(uint32_t, h);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int F = col_k[8 * cj + j] + 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t dw = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 4 * q + i;
          const uint32_t nib = (w[k] >> (4 * j)) & 0xFu, m = nib & 7u;
          uint32_t b = 0;
          if (m && e[k] != 255u) b = e4m3_of_shifted_e2m1(m, F + 256 - (int)binade_key(m, e[k]));
          dw |= (b | ((nib & 8u) << 4)) << (8 * i);
        }
        out[j][q] = dw;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cj + j;
    uint4 o = make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
    if (col_nan[c]) o = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
    *reinterpret_cast<uint4*>(tile + c * kRcStride + 16 + 16 * ig) = o;
  }
  __syncthreads();

  // ---- store: column c's n bytes start at token t0, mis bytes into a 16-byte piece
  const int mis = (int)(t0 & 15);
  const int pieces = (mis + n + 15) >> 4;  // 1..9
  const int sh = (16 - mis) & 3;           // byte offset of the run inside its LDS dword
  const uint32_t* tw = reinterpret_cast<const uint32_t*>(tile);
  auto store_piece = [&](int c, int j) {
    const int s0 = 16 * j - mis;  // tile token of the piece's first byte (may be < 0)
    const int lo = max(0, -s0), hi = min(16, n - s0);
    const int a = c * kRcStride + 16 + s0;  // >= 1
    const int dw = a >> 2;
    uint32_t d[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = tw[dw + i];
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], (uint32_t)sh);
    uint8_t* g = p.q8 + (c0 + c) * p.ld_q8 + (t0 - mis) + 16 * j;
    if (lo == 0 && hi == 16) {
      *reinterpret_cast<uint4*>(g) = make_uint4(o[0], o[1], o[2], o[3]);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b0 = max(lo, 4 * i), b1 = min(hi, 4 * i + 4);
      if (b0 == 4 * i && b1 == 4 * i + 4) {
        *reinterpret_cast<uint32_t*>(g + 4 * i) = o[i];
      } else {
        for (int b = b0; b < b1; ++b) g[b] = (uint8_t)(o[i] >> (8 * (b - 4 * i)));
      }
    }
  };
#pragma unroll 1
  for (int pass = 0; pass < kRcCols / 32; ++pass) {
    const int c = pass * 32 + (t >> 3), j = t & 7;
    if (c < nc && j < pieces) store_piece(c, j);
  }
  if (pieces == 9 && t < nc) store_piece(t, 8);
}

}  // namespace

hipError_t launch_fp4_row_to_fp8_col(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t cols,
                                     const int64_t* offsets, int n_experts, uint8_t* q8, int64_t ld_q8,
                                     float* s, int64_t ld_s, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  RcParams p;
  p.codes = codes;
  p.e8m0 = e8m0;
  p.offsets = offsets;
  p.q8 = q8;
  p.s = reinterpret_cast<uint32_t*>(s);
  p.rows = rows;
  p.cols = cols;
  p.ld_q8 = ld_q8;
  p.ld_s = ld_s;
  p.n_experts = n_experts;
  p.groups = (uint32_t)rc_group_slots(rows, n_experts);
  p.tiles_c = (uint32_t)((cols + kRcCols - 1) / kRcCols);
  const uint64_t total = (uint64_t)p.groups * p.tiles_c;
  p.per_xcd = (uint32_t)((total + 7) / 8);
  hipLaunchKernelGGL(fp4_row_to_fp8_col_kernel, dim3(8 * p.per_xcd), dim3(kRcThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxq
