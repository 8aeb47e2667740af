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
constexpr int kRcGroupsPerWG = 4;  // consecutive groups per workgroup (the next one is loaded ahead)
constexpr int kRcNanCol = 1 << 20;  // column exponent marking a NaN group

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
  uint32_t ranges;          // runs of kRcGroupsPerWG group slots
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

// Finds the first token and token count of group slots gi0 .. gi0 + kRcGroupsPerWG - 1
// (count 0 past the last group; the nonempty slots form a prefix). All threads take
// part; the results land in LDS.
__device__ void find_groups(const RcParams& p, uint32_t gi0, int64_t* sel_t0, int* sel_n) {
  __shared__ uint32_t wave_tot[kRcThreads / 64];
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
  if (t < kRcGroupsPerWG) sel_n[t] = 0;
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const uint32_t excl = before + inc - sum;
  if (sum && gi0 < excl + sum && gi0 + kRcGroupsPerWG > excl) {
    uint32_t g0 = excl;  // slot of expert e's first group
    for (int e = e0; e < e1; ++e) {
      const int64_t lo = clamp_token(p.offsets[e], p.rows), hi = clamp_token(p.offsets[e + 1], p.rows);
      const uint32_t cnt = hi > lo ? (uint32_t)((hi - lo + kRcGroup - 1) / kRcGroup) : 0u;
      // the expert's slots g0 .. g0 + cnt - 1 that fall in the workgroup's range
      // (capped at the slot count: with overlapping offsets the experts' groups can
      // add up to more slots than the scale rows hold)
      const uint32_t s0 = max(g0, gi0), s1 = min(min(g0 + cnt, gi0 + kRcGroupsPerWG), p.groups);
      for (uint32_t slot = s0; slot < s1; ++slot) {
        const int64_t first = lo + (int64_t)(slot - g0) * kRcGroup;
        sel_t0[slot - gi0] = first;
        sel_n[slot - gi0] = (int)std::min<int64_t>(kRcGroup, hi - first);
      }
      g0 += cnt;
    }
  }
  __syncthreads();
}

// LDS row of tile column c = 8 cj + j: the eight columns a thread converts go to rows
// j * 32 + cj, so the lanes of a wave write consecutive rows.
__device__ __forceinline__ int lds_row(int cj, int j) { return 32 * j + cj; }

// The exact path, for workgroups whose group holds blocks with extreme scale bytes
// (rare: such bytes never come from quantising bf16 or fp32 data). It re-reads the
// thread's elements from memory, one token at a time.
__device__ __forceinline__ void exact_column_keys(const RcParams& p, int64_t t0, int n, int64_t c0, int ig,
                                                  int cj, uint32_t* cm) {
#pragma unroll 1
  for (int k = 0; k < 16; ++k) {
    const int r = 16 * ig + k;
    if (r >= n) break;
    const int64_t row = t0 + r;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p.codes + row * (p.cols / 2) + (c0 + 8 * cj) / 2);
    const uint32_t e = p.e8m0[row * (p.cols / 32) + (c0 + 8 * cj) / 32];
    if (e == 255u) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) cm[j] = max(cm[j], binade_key((w >> (4 * j)) & 7u, e));
  }
}

__device__ __forceinline__ void exact_convert(const RcParams& p, int64_t t0, int n, int64_t c0, int ig, int cj,
                                              const int* col_k, uint8_t* tile) {
#pragma unroll 1
  for (int k = 0; k < 16; ++k) {
    const int r = 16 * ig + k;
    if (r >= n) break;
    const int64_t row = t0 + r;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p.codes + row * (p.cols / 2) + (c0 + 8 * cj) / 2);
    const uint32_t e = p.e8m0[row * (p.cols / 32) + (c0 + 8 * cj) / 32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t nib = (w >> (4 * j)) & 0xFu, m = nib & 7u;
      uint32_t b = 0;
      if (m && e != 255u) b = e4m3_of_shifted_e2m1(m, col_k[8 * cj + j] + 8 + 256 - (int)binade_key(m, e));
      tile[lds_row(cj, j) * kRcStride + 16 + r] = (uint8_t)(b | ((nib & 8u) << 4));
    }
  }
}

// Writes bytes [lo, hi) of a 16-byte output piece (0 <= lo < hi <= 16, not the whole
// piece, which the callers store as one 16-byte store) as at most
// seven naturally aligned stores, each under its own predicate (no loop: the lanes
// of a wave that store partial pieces start and end at different bytes, and a
// per-lane loop would issue the union of all their paths). From b = lo upwards: a
// byte to reach 2-byte alignment, a short to reach 4, a dword to reach 8, an 8-byte
// store when 8 aligned bytes remain, then a dword, a short and a byte for the rest.
__device__ __forceinline__ void store_partial(uint8_t* g, const uint32_t* o, int lo, int hi) {
  // the dword holding byte b (b < 16), by selects rather than a dynamic index
  auto dword = [&](int b) { const int i = b >> 2; return i == 0 ? o[0] : i == 1 ? o[1] : i == 2 ? o[2] : o[3]; };
  int b = lo;
  if ((b & 1) && b < hi) {
    g[b] = (uint8_t)(dword(b) >> (8 * (b & 3)));
    b += 1;
  }
  if ((b & 2) && b + 2 <= hi) {
    *reinterpret_cast<uint16_t*>(g + b) = (uint16_t)(dword(b) >> (8 * (b & 3)));
    b += 2;
  }
  if ((b & 4) && b + 4 <= hi) {
    *reinterpret_cast<uint32_t*>(g + b) = dword(b);
    b += 4;
  }
  if ((b & 7) == 0 && b + 8 <= hi) {
    *reinterpret_cast<uint2*>(g + b) = b == 0 ? make_uint2(o[0], o[1]) : make_uint2(o[2], o[3]);
    b += 8;
  }
  if (b + 4 <= hi) {
    *reinterpret_cast<uint32_t*>(g + b) = dword(b);
    b += 4;
  }
  if (b + 2 <= hi) {
    *reinterpret_cast<uint16_t*>(g + b) = (uint16_t)(dword(b) >> (8 * (b & 3)));
    b += 2;
  }
  if (b < hi) g[b] = (uint8_t)(dword(b) >> (8 * (b & 3)));
}

__global__ __launch_bounds__(kRcThreads, 3) void fp4_row_to_fp8_col_kernel(RcParams p) {
  // transposed E4M3, one row per column; before that, the per-strip column maxima
  __shared__ uint4 tile_q[kRcTileBytes / 16];
  static_assert(8 * kRcCols * 4 <= kRcTileBytes, "the maxima share the tile's space");
  uint32_t(*red)[kRcCols] = reinterpret_cast<uint32_t(*)[kRcCols]>(tile_q);
  __shared__ int col_k[kRcCols];  // scale exponent of each column
  __shared__ uint8_t e_lds[2][kRcCols / 32][kRcGroup] __attribute__((aligned(16)));  // scale bytes, per block
  // each column's unfinished 16-byte piece, by group parity (written while the
  // previous group's carry is still being read)
  __shared__ uint4 carry[2][kRcCols];
  __shared__ int64_t sel_t0[kRcGroupsPerWG];
  __shared__ int sel_n[kRcGroupsPerWG];
  uint8_t* tile = reinterpret_cast<uint8_t*>(tile_q);

  // XCD-aware order: the workgroups of one XCD take consecutive group ranges of one
  // column tile, so the pieces two neighbouring ranges share meet in one L2
  const uint32_t L = (blockIdx.x & 7u) * p.per_xcd + (blockIdx.x >> 3);
  if (L >= p.ranges * p.tiles_c) return;
  const uint32_t tc = L / p.ranges, rg = L - tc * p.ranges;
  const uint32_t gi0 = rg * kRcGroupsPerWG;
  find_groups(p, gi0, sel_t0, sel_n);
  int ng = 0;
  while (ng < kRcGroupsPerWG && sel_n[ng] > 0) ++ng;
  if (ng == 0) return;

  const int t = threadIdx.x, ig = t >> 5, cj = t & 31;
  const int64_t c0 = (int64_t)tc * kRcCols;
  const int nc = (int)std::min<int64_t>(kRcCols, p.cols - c0);
  const bool colv = 8 * cj < nc;
  const uint32_t cstride = (uint32_t)(p.cols / 2), estride = (uint32_t)(p.cols / 32);
  const uint32_t colo = 4u * (uint32_t)min(cj, nc / 8 - 1);  // past the tile: repeat its last columns
  const int nbt = nc / 32;                                    // scale blocks in the tile

  // codes of the thread's 16 tokens x 8 columns of group i; lanes past the group's
  // last token read that token again (an L2 hit; their values are masked), so the
  // next expert's tokens are not fetched for a short group
  auto load_codes = [&](int i, uint32_t* ww) {
    const int64_t g0 = sel_t0[i];
    const int lim = sel_n[i] - 1;
    const uint8_t* cb = p.codes + g0 * (int64_t)cstride + c0 / 2 + colo;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      ww[k] = *reinterpret_cast<const uint32_t*>(cb + (uint64_t)min(16 * ig + k, lim) * cstride);
  };
  // scale bytes travel through LDS (thread t stages four blocks of token t / 2), so
  // that each thread then reads its 16 tokens' bytes with one 16-byte LDS read
  auto load_scales = [&](int i, uint32_t* eq) {
    const int64_t g0 = sel_t0[i];
    const int lim = sel_n[i] - 1;
    const uint8_t* e8 = p.e8m0 + g0 * (int64_t)estride + c0 / 32 + (uint64_t)min(t >> 1, lim) * estride;
#pragma unroll
    for (int q = 0; q < 4; ++q) eq[q] = e8[min(4 * (t & 1) + q, nbt - 1)];
  };
  auto stage_scales = [&](int buf, const uint32_t* eq) {
#pragma unroll
    for (int q = 0; q < 4; ++q) e_lds[buf][4 * (t & 1) + q][t >> 1] = (uint8_t)eq[q];
  };

  uint32_t w[16], eq[4];
  load_codes(0, w);
  load_scales(0, eq);
  stage_scales(0, eq);
  __syncthreads();

  // the piece left unfinished by the previous group (same for every column)
  bool carry_valid = false;
  int64_t carry_pos = 0;  // absolute token of its first byte (a multiple of 16)
  int carry_lo = 0, carry_hi = 0;
  const uint32_t* tw = reinterpret_cast<const uint32_t*>(tile);
  uint8_t* const qcol = p.q8 + c0 * p.ld_q8;  // row c of the output tile: qcol + c * ld_q8

#pragma unroll 1
  for (int i = 0; i < ng; ++i) {
    const int64_t t0 = sel_t0[i];
    const int n = sel_n[i];
    const uint32_t gi = gi0 + i;
    const int buf = i & 1;
    uint32_t wn[16];
    if (i + 1 < ng) {  // in flight while this group is converted
      load_codes(i + 1, wn);
      load_scales(i + 1, eq);
    }
    const uint4 ep = *reinterpret_cast<const uint4*>(&e_lds[buf][cj >> 2][16 * ig]);
    const uint32_t epw[4] = {ep.x, ep.y, ep.z, ep.w};
    auto ebyte = [&](int k) { return (epw[k >> 2] >> (8 * (k & 3))) & 0xFFu; };

    // mask tokens past the group and columns past the tile; screen for the exact path
    uint32_t emin = 255u, emax = 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool valid = colv && 16 * ig + k < n;
      if (!valid) w[k] = 0u;
      const uint32_t e = ebyte(k);
      emin = min(emin, (w[k] & 0x77777777u) ? e : 127u);
      emax = max(emax, valid ? e : 0u);  // 255 marks a NaN block
    }
    const bool slow = __syncthreads_or(emin < 10u || emax > 252u);

    // ---- column maxima: |x| (finite, nonnegative: the fp32 bits order like the
    // values) or binade keys (exact path)
    uint32_t cm[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t nanl = 0;
    if (!slow) {
      float fm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float sc = e8m0_operand(ebyte(k));
        const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 0);
        const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 1);
        const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 2);
        const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 3);
        fm[0] = fmaxf(fm[0], fabsf(a.x));
        fm[1] = fmaxf(fm[1], fabsf(a.y));
        fm[2] = fmaxf(fm[2], fabsf(b.x));
        fm[3] = fmaxf(fm[3], fabsf(b.y));
        fm[4] = fmaxf(fm[4], fabsf(c.x));
        fm[5] = fmaxf(fm[5], fabsf(c.y));
        fm[6] = fmaxf(fm[6], fabsf(d.x));
        fm[7] = fmaxf(fm[7], fabsf(d.y));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j] = as_u(fm[j]);
    } else if (colv) {
      exact_column_keys(p, t0, n, c0, ig, cj, cm);
      // a NaN block (byte 0xFF) in the strip marks the thread's eight columns
#pragma unroll
      for (int k = 0; k < 16; ++k) nanl |= 16 * ig + k < n && ebyte(k) == 255u ? 1u : 0u;
    }
    // bit 31 of a maximum is free (magnitudes and keys stay below it): the NaN flag
#pragma unroll
    for (int j = 0; j < 8; ++j) cm[j] |= nanl << 31;
    *reinterpret_cast<uint4*>(&red[ig][8 * cj]) = make_uint4(cm[0], cm[1], cm[2], cm[3]);
    *reinterpret_cast<uint4*>(&red[ig][8 * cj + 4]) = make_uint4(cm[4], cm[5], cm[6], cm[7]);
    __syncthreads();
    {
      uint32_t m = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) m = max(m, red[r][t]);
      const bool nanc = m >> 31;
      m &= 0x7FFFFFFFu;
      // top binade F of the column's largest magnitude; scale 2^(F-8) (k = 0 if all zero)
      int k = 0;
      if (m) k = (slow ? (int)m - 256 : (int)(m >> 23) - 127) - 8;
      col_k[t] = nanc ? kRcNanCol : k;
      if (t < nc) p.s[(c0 + t) * p.ld_s + gi] = nanc ? 0x7FC00000u : pow2_bits(k);
    }
    __syncthreads();

    // ---- convert: dword q of column j holds tokens 4q..4q+3 of the thread's strip
    if (!slow) {
      // convert the codes a second time rather than keep 128 values live across
      // the barriers (the empty asm hides the earlier conversions from CSE)
#pragma unroll
      for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(w[k]));
      float scol[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) scol[j] = e8m0_operand((uint32_t)(col_k[8 * cj + j] + 127));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = 4 * q + r;
          const float sc = e8m0_operand(ebyte(k));
          const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 0);
          const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 1);
          const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 2);
          const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 3);
          v[r][0] = a.x; v[r][1] = a.y; v[r][2] = b.x; v[r][3] = b.y;
          v[r][4] = c.x; v[r][5] = c.y; v[r][6] = d.x; v[r][7] = d.y;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s16x2_t h = {0, 0};
          h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, v[0][j], v[1][j], scol[j], false);
          h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, v[2][j], v[3][j], scol[j], true);
          *reinterpret_cast<uint32_t*>(tile + lds_row(cj, j) * kRcStride + 16 + 16 * ig + 4 * q) =
              __builtin_bit_cast(uint32_t, h);
        }
      }
    } else if (colv) {
      exact_convert(p, t0, n, c0, ig, cj, col_k, tile);
    }
    __syncthreads();
    if (i + 1 < ng) {  // the prefetched group becomes current before the stores are issued
#pragma unroll
      for (int k = 0; k < 16; ++k) w[k] = wn[k];
      stage_scales(buf ^ 1, eq);
    }

    // ---- store. The group's bytes cover tokens [t0, t0 + n); piece q covers
    // [base + 16 q, base + 16 q + 16) with base = t0 - mis. Piece 0 takes in the
    // carried bytes [carry_lo, mis) when the previous group ended inside it; a last
    // piece that ends inside the 16 bytes is carried to the next group, and written
    // partially only after the workgroup's last group.
    const int mis = (int)(t0 & 15);
    const int64_t base = t0 - mis;
    const int pieces = (mis + n + 15) >> 4;  // 1..9
    const int tail = (mis + n) & 15;         // bytes of the last piece when it is partial
    const bool last = i + 1 == ng;
    // a carried piece elsewhere (offsets not contiguous) is written out first
    const bool joins = carry_valid && carry_pos == base && carry_hi == mis;
    if (carry_valid && !joins) {
      for (int c = t; c < nc; c += kRcThreads) {
        const uint4 cv = carry[buf ^ 1][c];
        const uint32_t o[4] = {cv.x, cv.y, cv.z, cv.w};
        store_partial(qcol + (int64_t)c * p.ld_q8 + carry_pos, o, carry_lo, carry_hi);
      }
    }
    const int lo0 = joins ? carry_lo : mis;
    const int sh = (16 - mis) & 3;  // byte offset of the run inside its LDS dword
    auto store_piece = [&](int cjj, int j, int q) {
      const int c = 8 * cjj + j;
      const int s0 = 16 * q - mis;  // token of the piece's first byte within the group
      const int lo = q == 0 ? lo0 : 0;
      const int hi = q == pieces - 1 && tail ? tail : 16;
      const int dw = (lds_row(cjj, j) * kRcStride + 16 + s0) >> 2;
      uint32_t d[5];
#pragma unroll
      for (int r = 0; r < 5; ++r) d[r] = tw[dw + r];
      uint32_t o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = __builtin_amdgcn_alignbyte(d[r + 1], d[r], (uint32_t)sh);
      if (slow && col_k[c] == kRcNanCol) {
        // a NaN group: its own bytes are 0x7F (carried bytes keep theirs)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = 0x7F7F7F7Fu;
      }
      if (q == 0 && joins) {  // merge the carried bytes [0, mis)
        const uint4 cv = carry[buf ^ 1][c];
        const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b0 = 4 * r;
          const uint32_t m = mis >= b0 + 4 ? 0xFFFFFFFFu : (mis <= b0 ? 0u : (1u << (8 * (mis - b0))) - 1u);
          o[r] = (cw[r] & m) | (o[r] & ~m);
        }
      }
      uint8_t* g = qcol + (int64_t)c * p.ld_q8 + base + 16 * q;
      if (hi < 16 && !last) {
        carry[buf][c] = make_uint4(o[0], o[1], o[2], o[3]);  // finished by the next group
      } else if (lo == 0 && hi == 16) {
        *reinterpret_cast<uint4*>(g) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        store_partial(g, o, lo, hi);
      }
    };
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
      const int cjj = t >> 3, q = t & 7;
      if (8 * cjj + j < nc && q < pieces) store_piece(cjj, j, q);
    }
    if (pieces == 9) {
      const int cjj = t & 31, j = t >> 5;
      if (8 * cjj + j < nc) store_piece(cjj, j, 8);
    }
    carry_valid = tail != 0 && !last;
    carry_pos = base + 16 * (pieces - 1);
    carry_lo = pieces == 1 ? lo0 : 0;
    carry_hi = tail;
    if (!last) __syncthreads();  // the next group's maxima overwrite the tile buffer
  }
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
  p.ranges = (p.groups + kRcGroupsPerWG - 1) / kRcGroupsPerWG;
  const uint64_t total = (uint64_t)p.ranges * p.tiles_c;
  p.per_xcd = (uint32_t)((total + 7) / 8);
  hipLaunchKernelGGL(fp4_row_to_fp8_col_kernel, dim3(8 * p.per_xcd), dim3(kRcThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxq
