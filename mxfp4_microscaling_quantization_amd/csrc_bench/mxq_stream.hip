// Streaming reference kernels for the benchmark (libmxq_stream.so, not part of the
// quantisation library): plain copies with the read/write byte mix of each codec
// kernel, and a byte mover with the tile kernels' exact access pattern. They move
// the same bytes in the same order as the kernels they stand beside and compute
// nothing, so their throughput on the same sizes is what that memory traffic can
// reach on this chip.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int B>
struct Vec;
template <>
struct Vec<4> {
  typedef uint32_t T;
  static __device__ __forceinline__ uint32_t fold(T v) { return v; }
  static __device__ __forceinline__ T make(uint32_t x) { return x; }
};
template <>
struct Vec<8> {
  typedef u32x2 T;
  static __device__ __forceinline__ uint32_t fold(T v) { return v.x ^ v.y; }
  static __device__ __forceinline__ T make(uint32_t x) { return T{x, x + 1u}; }
};
template <>
struct Vec<16> {
  typedef u32x4 T;
  static __device__ __forceinline__ uint32_t fold(T v) { return v.x ^ v.y ^ v.z ^ v.w; }
  static __device__ __forceinline__ T make(uint32_t x) { return T{x, x + 1u, x + 2u, x + 3u}; }
};

// Unit u reads RB bytes at src + u * RB and writes WB bytes at dst + u * WB (WB = 0:
// read only). Lane t of workgroup b takes units b * 1024 + j * 256 + t, so every
// load and store instruction of a wave covers one contiguous run, as in the codec
// kernels. NTL / NTS: nontemporal loads / stores.
template <int RB, int WB, bool NTL, bool NTS, int U>
__global__ __launch_bounds__(kThreads) void stream_mix_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, uint32_t units) {
  typedef typename Vec<RB>::T RT;
  const uint32_t base = blockIdx.x * (kThreads * U) + threadIdx.x;
  RT v[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t u = base + j * kThreads;
    const RT* p = reinterpret_cast<const RT*>(src) + u;
    if (u < units) v[j] = NTL ? __builtin_nontemporal_load(p) : *p;
    else v[j] = Vec<RB>::make(0u);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const uint32_t u = base + j * kThreads;
    const uint32_t f = Vec<RB>::fold(v[j]);
    if constexpr (WB > 0) {
      typedef typename Vec<WB>::T WT;
      WT* q = reinterpret_cast<WT*>(dst) + u;
      if (u < units) {
        if constexpr (NTS) __builtin_nontemporal_store(Vec<WB>::make(f), q);
        else *q = Vec<WB>::make(f);
      }
    } else {
      acc ^= f;
    }
  }
  if constexpr (WB == 0) {
    // keeps the loads alive; the data never holds this pattern
    if (acc == 0x9E3779B9u && threadIdx.x == 0) reinterpret_cast<uint32_t*>(dst)[blockIdx.x] = acc;
  }
}

template <int RB, int WB, int U>
hipError_t launch_mix_u(const void* src, void* dst, int64_t units, int flags, hipStream_t st) {
  const uint32_t grid = (uint32_t)((units + kThreads * U - 1) / (kThreads * U));
  const bool ntl = flags & 1, nts = flags & 2;
  const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
  uint8_t* d = reinterpret_cast<uint8_t*>(dst);
  if (ntl && nts) hipLaunchKernelGGL((stream_mix_kernel<RB, WB, true, true, U>), dim3(grid), dim3(kThreads), 0, st, s, d, (uint32_t)units);
  else if (ntl) hipLaunchKernelGGL((stream_mix_kernel<RB, WB, true, false, U>), dim3(grid), dim3(kThreads), 0, st, s, d, (uint32_t)units);
  else if (nts) hipLaunchKernelGGL((stream_mix_kernel<RB, WB, false, true, U>), dim3(grid), dim3(kThreads), 0, st, s, d, (uint32_t)units);
  else hipLaunchKernelGGL((stream_mix_kernel<RB, WB, false, false, U>), dim3(grid), dim3(kThreads), 0, st, s, d, (uint32_t)units);
  return hipGetLastError();
}

// flags bits 2-3: lane units per thread, 0 -> kUnroll, 1 -> 1, 2 -> 2
template <int RB, int WB>
hipError_t launch_mix(const void* src, void* dst, int64_t units, int flags, hipStream_t st) {
  const int u = (flags >> 2) & 3;
  if (u == 1) return launch_mix_u<RB, WB, 1>(src, dst, units, flags, st);
  if (u == 2) return launch_mix_u<RB, WB, 2>(src, dst, units, flags, st);
  return launch_mix_u<RB, WB, kUnroll>(src, dst, units, flags, st);
}

// ---------------------------------------------------------------------------
// The fused row + column tile pattern: a bf16 [R, C] tensor read in TR x TC tiles
// (TC = 256), each 16-byte chunk folded to 4 bytes at the row-code position and one
// byte per 32-element row block at the row-scale position; the tile parked in LDS;
// then, per column and 32-row group, 16 bytes at the column-code position [C, R/2]
// and one byte at the column-scale position [C, R/32]. Workgroups are dealt to the
// XCDs as the tile kernel deals them (V vertically adjacent tiles per XCD turn).
template <int TR>
__global__ __launch_bounds__(kThreads) void tile_pattern_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, uint8_t* codes_row, uint8_t* scales_row,
                                                                uint8_t* codes_col, uint8_t* scales_col,
                                                                uint32_t tiles_r, uint32_t tiles_c, uint32_t groups) {
  constexpr int TC = 256, G = TR / 32, V = 256 / TR;
  constexpr int kChunksPerRow = TC / 8, kRowStep = kThreads / kChunksPerRow, kChunks = TR * TC / 8 / kThreads;
  __shared__ uint16_t tile[TR][TC] __attribute__((aligned(16)));
  const uint32_t t = threadIdx.x;
  const uint32_t xcd = blockIdx.x & 7u, slot = blockIdx.x >> 3;
  const uint32_t g = (slot / V) * 8u + xcd;
  if (g >= groups) return;
  const uint32_t gr = g / tiles_c, tc = g - gr * tiles_c;
  const uint32_t tr = gr * V + slot % V;
  if (tr >= tiles_r) return;
  const int64_t r0 = (int64_t)tr * TR, c0 = (int64_t)tc * TC;
  const int cc = (int)(t % kChunksPerRow), row_t = (int)(t / kChunksPerRow);
  const uint16_t* xt = x + (r0 + row_t) * cols + c0 + cc * 8;
  u32x4 cur[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j)
    cur[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xt + (int64_t)(j * kRowStep) * cols));
  uint8_t* crow = codes_row + (r0 + row_t) * (cols / 2) + (c0 + cc * 8) / 2;
  uint8_t* srow = scales_row + (r0 + row_t) * (cols / 32) + (c0 + cc * 8) / 32;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int row = row_t + j * kRowStep;
    const int sc = (cc * 8) ^ (((row >> 5) & (G - 1)) * (64 / G));
    *reinterpret_cast<u32x4*>(&tile[row][sc]) = cur[j];
    const uint32_t f = cur[j].x ^ cur[j].y ^ cur[j].z ^ cur[j].w;
    *reinterpret_cast<uint32_t*>(crow + (int64_t)(j * kRowStep) * (cols / 2)) = f;
    if ((cc & 3) == 0) srow[(int64_t)(j * kRowStep) * (cols / 32)] = (uint8_t)f;
  }
  __syncthreads();
#pragma unroll 1
  for (int k = t; k < TC * G; k += kThreads) {
    const int c = k / G, h = k % G;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int r = h * 32 + i;
      w[i >> 3] ^= (uint32_t)tile[r][c ^ (((r >> 5) & (G - 1)) * (64 / G))] << (4 * (i & 7));
    }
    const int64_t col = c0 + c, grow0 = r0 + h * 32;
    *reinterpret_cast<u32x4*>(codes_col + col * (rows / 2) + grow0 / 2) = u32x4{w[0], w[1], w[2], w[3]};
    scales_col[col * (rows / 32) + grow0 / 32] = (uint8_t)(w[0] ^ w[3]);
  }
}

// ---------------------------------------------------------------------------
// VALU issue probe: every lane runs `iters` iterations of eight independent
// dependency chains of one instruction kind (written out, so each iteration issues
// exactly eight VALU instructions): 0 v_add_u32, 1 v_bitop3_b32, 2 v_mad_u64_u32.
// Timed over enough waves to fill every SIMD, it gives the rate at which the chip
// retires that instruction (wave instructions per second), and its SQ_INSTS_VALU
// count shows how the counter counts it.
template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_probe_kernel(uint32_t* out, uint32_t iters, uint32_t seed) {
  const uint32_t b = threadIdx.x * 0x9E3779B9u + seed;
  uint32_t a[8];
  uint64_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = b + (uint32_t)i * 0x85EBCA6Bu;
    c[i] = ((uint64_t)a[i] << 32) | b;
  }
#pragma unroll 1
  for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0) asm volatile("v_add_u32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
      else if constexpr (KIND == 1) asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96" : "+v"(a[i]) : "v"(b), "v"(a[(i + 1) & 7]));
      else asm volatile("v_mad_u64_u32 %0, vcc, %1, %2, %0" : "+v"(c[i]) : "v"(a[i]), "v"(b) : "vcc");
    }
  }
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s ^= a[i] ^ (uint32_t)c[i] ^ (uint32_t)(c[i] >> 32);
  if (s == 0x9E3779B9u) out[blockIdx.x] = s;  // keeps the chains alive
}

}  // namespace

extern "C" {

// VALU issue probe (see valu_probe_kernel): `blocks` workgroups of 256 lanes, kind
// 0 / 1 / 2; out holds one dword per workgroup. Returns 0, 1 for a bad kind, 2 for a
// launch failure.
int mxq_valu_probe(void* out, int blocks, int iters, int kind, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  if (blocks <= 0 || iters <= 0) return 1;
  if (kind == 0) hipLaunchKernelGGL((valu_probe_kernel<0>), dim3(blocks), dim3(kThreads), 0, st, o, (uint32_t)iters, 7u);
  else if (kind == 1) hipLaunchKernelGGL((valu_probe_kernel<1>), dim3(blocks), dim3(kThreads), 0, st, o, (uint32_t)iters, 7u);
  else if (kind == 2) hipLaunchKernelGGL((valu_probe_kernel<2>), dim3(blocks), dim3(kThreads), 0, st, o, (uint32_t)iters, 7u);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Streaming mix: `units` units of rd_bytes read and wr_bytes written (rd in {4, 8,
// 16}, wr in {0, 4, 8, 16}); flags bit 0 nontemporal loads, bit 1 nontemporal
// stores, bits 2-3 lane units per thread (0: 4, 1: 1, 2: 2; 3 is rejected). src holds units * rd bytes, dst units * wr bytes (read only: one dword per
// 1024 units). 0 < units < 2^31. Returns 0, 1 for an unsupported mix or size, 2 for a
// launch failure.
int mxq_stream_mix(const void* src, void* dst, int64_t units, int rd_bytes, int wr_bytes, int flags,
                   void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (units <= 0 || units >= ((int64_t)1 << 31) || ((flags >> 2) & 3) == 3) return 1;
  hipError_t e;
  if (rd_bytes == 16 && wr_bytes == 4) e = launch_mix<16, 4>(src, dst, units, flags, st);
  else if (rd_bytes == 4 && wr_bytes == 16) e = launch_mix<4, 16>(src, dst, units, flags, st);
  else if (rd_bytes == 16 && wr_bytes == 8) e = launch_mix<16, 8>(src, dst, units, flags, st);
  else if (rd_bytes == 8 && wr_bytes == 16) e = launch_mix<8, 16>(src, dst, units, flags, st);
  else if (rd_bytes == 16 && wr_bytes == 16) e = launch_mix<16, 16>(src, dst, units, flags, st);
  else if (rd_bytes == 16 && wr_bytes == 0) e = launch_mix<16, 0>(src, dst, units, flags, st);
  else return 1;
  return e == hipSuccess ? 0 : 2;
}

// The fused row + column tile access pattern over a bf16 [rows, cols] tensor
// (rows % tile_rows == 0, cols % 256 == 0, tile_rows 64 or 128); outputs sized as
// the MXFP4 row- and column-wise outputs. Returns 0, 1 for bad sizes, 2 for a
// launch failure.
int mxq_stream_tile_pattern(const void* x, int64_t rows, int64_t cols, int tile_rows, void* codes_row,
                            void* scales_row, void* codes_col, void* scales_col, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rows <= 0 || cols <= 0 || cols % 256 || (tile_rows != 64 && tile_rows != 128) || rows % tile_rows) return 1;
  const uint32_t tiles_r = (uint32_t)(rows / tile_rows), tiles_c = (uint32_t)(cols / 256);
  const uint32_t V = 256 / tile_rows;
  const uint32_t groups = ((tiles_r + V - 1) / V) * tiles_c;
  const uint32_t grid = 8u * V * ((groups + 7u) / 8u);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
  uint8_t *a = (uint8_t*)codes_row, *b = (uint8_t*)scales_row, *c = (uint8_t*)codes_col, *d = (uint8_t*)scales_col;
  if (tile_rows == 64)
    hipLaunchKernelGGL((tile_pattern_kernel<64>), dim3(grid), dim3(kThreads), 0, st, xs, rows, cols, a, b, c, d,
                       tiles_r, tiles_c, groups);
  else
    hipLaunchKernelGGL((tile_pattern_kernel<128>), dim3(grid), dim3(kThreads), 0, st, xs, rows, cols, a, b, c, d,
                       tiles_r, tiles_c, groups);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
