// FP8 (E4M3, one fp32 power-of-two scale per 1x128 group) <-> MXFP4.
//
// Both directions work on 16-element chunks: a lane moves 16 bytes of E4M3 or 8
// bytes of codes, an MXFP4 block spans a lane pair and an FP8 group 8 lanes. Each
// lane reads its group's scale word itself (8 lanes share one cached load), so no
// cross-lane traffic is needed beyond one DPP swap for the block maximum.
//
// MXFP4 -> FP8 never leaves the integer domain: per block the shift
// d = S - E_j (S the group's largest exponent) selects an 8-entry byte table
// (E4M3 of each E2M1 magnitude scaled by 2^-d, held in LDS for d = 0..14), and
// v_perm_b32 maps four nibbles to four bytes at a time.
#include <algorithm>

#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

constexpr int kF8Threads = 256;
constexpr int kF8Unroll = 4;
constexpr uint32_t kF8ChunksPerWG = kF8Threads * kF8Unroll;
// MXFP4 -> FP8 writes twice what it reads; with 2 chunks per lane and nontemporal
// loads it streams measurably faster (≈ 8 %) than with 4 and plain loads.
constexpr int kF8BackUnroll = 2;
constexpr uint32_t kF8BackChunksPerWG = kF8Threads * kF8BackUnroll;

struct F8Params {
  const uint8_t* q8;
  const uint32_t* s128;
  uint8_t* codes;
  uint8_t* e8m0;
  uint32_t chunks;  // 16-element chunks
};

// floor(log2 v) for a nonzero E4M3 magnitude code k (1..126).
__device__ __forceinline__ int e4m3_floor_log2(uint32_t k) {
  const int e = (int)(k >> 3);
  return e ? e - 7 : (31 - __clz((int)k)) - 9;
}

__global__ __launch_bounds__(kF8Threads) void fp8_to_mxfp4_kernel(F8Params p) {
  const uint32_t base = blockIdx.x * kF8ChunksPerWG + threadIdx.x;
  uint4 q[kF8Unroll];
  uint32_t s[kF8Unroll];
#pragma unroll
  for (int j = 0; j < kF8Unroll; ++j) {
    const uint32_t c = base + j * kF8Threads;
    q[j] = make_uint4(0, 0, 0, 0);
    s[j] = 0x3F800000u;
    if (c < p.chunks) {
      q[j] = load_nt(reinterpret_cast<const uint4*>(p.q8) + c);
      s[j] = p.s128[c >> 3];
    }
  }
#pragma unroll
  for (int j = 0; j < kF8Unroll; ++j) {
    const uint32_t c = base + j * kF8Threads;
    const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, (w[i >> 2] >> (8 * (i & 3))) & 0x7Fu);
    am = max(am, dpp<kQuadSwap1>(am));
    const int sexp = (int)((s[j] >> 23) & 0xFFu);
    uint32_t byte;
    int D;
    if (am == 0x7Fu || sexp == 255) {
      byte = 255u;
      D = 0;
    } else if (am == 0u) {
      byte = 0u;
      D = 0;
    } else {
      int E = e4m3_floor_log2(am) + sexp - 127 - 2;
      E = std::min(127, std::max(-127, E));
      byte = (uint32_t)(E + 127);
      D = std::min(126, std::max(-126, sexp - 127 - E));
    }
    uint32_t out[2] = {0u, 0u};
    // the conversion divides by 2^(sb - 127): sb = E - (sexp - 127) + 127 = 127 - D
    const int sb = 127 - D;
    if (sb >= 0 && sb <= 254) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
      }
      const float scale = e8m0_operand((uint32_t)sb);
      out[0] = fp4x8_from_f32(v, scale);
      out[1] = fp4x8_from_f32(v + 8, scale);
    } else {  // exponents beyond the conversion's scale range: ALU rounding
      const float f = as_f((uint32_t)(127 + D) << 23);  // 2^D
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t b = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const float y = e4m3_value(b & 0x7Fu) * f;
        const uint32_t code = e2m1_rne(y) | ((b >> 7) << 3);
        out[i >> 3] |= code << (4 * (i & 7));
      }
    }
    if (byte == 255u) out[0] = out[1] = 0u;
    if (c < p.chunks) {
      store_nt(reinterpret_cast<uint2*>(p.codes) + c, make_uint2(out[0], out[1]));
      if ((c & 1u) == 0u) p.e8m0[c >> 1] = (uint8_t)byte;
    }
  }
}

struct F8BackParams {
  const uint2* codes;
  const uint32_t* e8m0;  // 4 block exponents of a group per word
  uint4* q8;
  uint32_t* s128;
  uint32_t chunks;
};

__global__ __launch_bounds__(kF8Threads) void mxfp4_to_fp8_kernel(F8BackParams p) {
  // table[d] = E4M3 bytes of the magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 times 2^-d
  __shared__ uint2 table[15];
  if (threadIdx.x < 15) {
    const uint32_t d = threadIdx.x;
    uint32_t lo = 0, hi = 0;
    for (uint32_t m = 0; m < 8; ++m) {
      const float v = e2m1_value(m) * as_f((127u - d) << 23);
      const uint32_t b = e4m3_rne(v);
      if (m < 4) lo |= b << (8 * m);
      else hi |= b << (8 * (m - 4));
    }
    table[d] = make_uint2(lo, hi);
  }
  __syncthreads();
  const uint32_t base = blockIdx.x * kF8BackChunksPerWG + threadIdx.x;
  uint2 cw[kF8BackUnroll];
  uint32_t gw[kF8BackUnroll];
#pragma unroll
  for (int j = 0; j < kF8BackUnroll; ++j) {
    const uint32_t c = base + j * kF8Threads;
    cw[j] = make_uint2(0, 0);
    gw[j] = 0;
    if (c < p.chunks) {
      cw[j] = load_nt(p.codes + c);
      gw[j] = p.e8m0[c >> 3];
    }
  }
#pragma unroll
  for (int j = 0; j < kF8BackUnroll; ++j) {
    const uint32_t c = base + j * kF8Threads;
    if (c >= p.chunks) continue;
    const uint32_t g = gw[j];
    const uint32_t e0 = g & 0xFFu, e1 = (g >> 8) & 0xFFu, e2 = (g >> 16) & 0xFFu, e3 = g >> 24;
    const uint32_t S = max(max(e0, e1), max(e2, e3));
    const bool nan = (e0 == 255u) | (e1 == 255u) | (e2 == 255u) | (e3 == 255u);
    const uint32_t ej = (g >> (8 * ((c >> 1) & 3u))) & 0xFFu;
    const uint2 tab = table[min(S - ej, 14u)];
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = h ? cw[j].y : cw[j].x;
      const uint32_t sel_ev = w & 0x07070707u;         // magnitudes of elements 0, 2, 4, 6
      const uint32_t sel_od = (w >> 4) & 0x07070707u;  // magnitudes of elements 1, 3, 5, 7
      uint32_t ev = __builtin_amdgcn_perm(tab.y, tab.x, sel_ev);
      uint32_t od = __builtin_amdgcn_perm(tab.y, tab.x, sel_od);
      ev |= (w << 4) & 0x80808080u;  // sign bits 3, 11, 19, 27 -> 7, 15, 23, 31
      od |= w & 0x80808080u;
      o[2 * h] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
      o[2 * h + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
    }
    if (nan) o[0] = o[1] = o[2] = o[3] = 0x7F7F7F7Fu;
    store_nt(p.q8 + c, make_uint4(o[0], o[1], o[2], o[3]));
    if ((c & 7u) == 0u) p.s128[c >> 3] = nan ? 0x7FC00000u : (S ? (S << 23) : 0x00400000u);
  }
}

hipError_t launch_fp8_to_mxfp4(const uint8_t* q8, const float* s128, int64_t rows, int64_t cols,
                               uint8_t* codes, uint8_t* e8m0, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cpr = cols / 16;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    F8Params p;
    p.q8 = q8 + r0 * cols;
    p.s128 = reinterpret_cast<const uint32_t*>(s128) + r0 * (cols / 128);
    p.codes = codes + r0 * (cols / 2);
    p.e8m0 = e8m0 + r0 * (cols / 32);
    p.chunks = (uint32_t)(nr * cpr);
    const uint32_t grid = (p.chunks + kF8ChunksPerWG - 1) / kF8ChunksPerWG;
    hipLaunchKernelGGL(fp8_to_mxfp4_kernel, dim3(grid), dim3(kF8Threads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* e8m0, int64_t rows,
                               int64_t cols, uint8_t* q8, float* s128, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cpr = cols / 16;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    F8BackParams p;
    p.codes = reinterpret_cast<const uint2*>(codes + r0 * (cols / 2));
    p.e8m0 = reinterpret_cast<const uint32_t*>(e8m0 + r0 * (cols / 32));
    p.q8 = reinterpret_cast<uint4*>(q8 + r0 * cols);
    p.s128 = reinterpret_cast<uint32_t*>(s128) + r0 * (cols / 128);
    p.chunks = (uint32_t)(nr * cpr);
    const uint32_t grid = (p.chunks + kF8BackChunksPerWG - 1) / kF8BackChunksPerWG;
    hipLaunchKernelGGL(mxfp4_to_fp8_kernel, dim3(grid), dim3(kF8Threads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mxq
