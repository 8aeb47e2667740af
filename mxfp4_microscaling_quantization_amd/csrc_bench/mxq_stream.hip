// Streaming reference kernels for the benchmark (libmxq_stream.so, not part of the
// quantisation library): plain copies with the read/write byte mix of each codec
// kernel, and byte movers with the access patterns of the fused row + column kernel
// and of the 16x16 NVFP4 kernel. They move the same bytes in the same order as the
// kernels they stand beside and compute nothing, so their throughput on the same
// sizes is what that memory traffic can reach on this chip.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <algorithm>
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
// The fused row + column strip pattern (the bf16 MXFP4 row + column kernel's memory
// traffic, moving bytes only): a workgroup walks a 256-column strip in 64-row steps
// over `per_wg` units of 256 rows. Each step parks the tile in LDS, folds each
// 16-byte chunk to 4 bytes at the row-code position, stages one byte per 32-element
// row block and stores it as one 8-byte run per row; the column tasks (one column
// over 32 rows) fold 32 values to 16 bytes kept in registers. After four steps the
// column codes leave as whole 128-byte lines assembled in LDS and the column scales
// as one 8-byte run per column.
__device__ __forceinline__ uint32_t opaque_lane() {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__global__ __launch_bounds__(kThreads) void strip_pattern_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t cols, uint8_t* codes_row, uint8_t* scales_row,
                                                                 uint8_t* codes_col, uint8_t* scales_col,
                                                                 uint32_t strips, uint32_t flushes, uint32_t per_wg) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[64 * 256 * 2];
  __shared__ __attribute__((aligned(16))) uint8_t rsc[64 * 8];
  __shared__ __attribute__((aligned(16))) uint8_t csc[256 * 8];
  const uint32_t unit = blockIdx.x / strips, strip = blockIdx.x - unit * strips;
  const uint32_t f0 = unit * per_wg, f1 = min(f0 + per_wg, flushes);
  if (f0 >= flushes) return;
  const int64_t c0 = (int64_t)strip * 256;
  u32x4 cur[8];
  auto load_step = [&](int64_t r0) {
    const uint32_t t = opaque_lane();
    const uint16_t* xs = x + (r0 + (t >> 5)) * cols + c0 + (t & 31u) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) cur[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xs + (int64_t)(8 * j) * cols));
  };
  load_step((int64_t)f0 * 256);
#pragma unroll 1
  for (uint32_t f = f0; f < f1; ++f) {
    const int64_t fr = (int64_t)f * 256;
    uint32_t acc[4][2][4];
    uint32_t scol[2] = {0u, 0u};
    auto step = [&](auto sq_c) {
      constexpr int sq = decltype(sq_c)::value;
      const int64_t r0 = fr + sq * 64;
      __syncthreads();
      {
        const uint32_t t = opaque_lane();
        const int cc = (int)(t & 31u), row_t = (int)(t >> 5);
        uint8_t* const wr0 = buf + (row_t * 256 + cc * 8) * 2;
        uint8_t* const wr1 = buf + (row_t * 256 + ((cc * 8) ^ 32)) * 2;
        uint8_t* const crow = codes_row + (r0 + row_t) * (cols / 2) + (c0 + cc * 8) / 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          *reinterpret_cast<u32x4*>((j < 4 ? wr0 : wr1) + j * 8 * 256 * 2) = cur[j];
          const uint32_t v = cur[j].x ^ cur[j].y ^ cur[j].z ^ cur[j].w;
          *reinterpret_cast<uint32_t*>(crow + (int64_t)(8 * j) * (cols / 2)) = v;
          if ((cc & 3) == 0) rsc[(row_t + 8 * j) * 8 + cc / 4] = (uint8_t)v;
        }
      }
      asm volatile("" ::: "memory");
      if (sq < 3 || f + 1 < f1) load_step(r0 + 64);
      __syncthreads();
      const uint32_t t = opaque_lane();
      if (t < 64) *reinterpret_cast<uint2*>(scales_row + (r0 + t) * (cols / 32) + c0 / 32) = *reinterpret_cast<const uint2*>(rsc + t * 8);
      const int h = (int)(t & 1u);
      const uint8_t* const rd = buf + (h * 32 * 256 + (((int)(t >> 1)) ^ (32 * h))) * 2;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 32; ++i)
          w[i >> 3] ^= (uint32_t)(*reinterpret_cast<const uint16_t*>(rd + 256 * m + i * 512)) << (4 * (i & 7));
        asm volatile("" ::"v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]) : "memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[sq][m][q] = w[q];
        scol[m] |= ((w[0] ^ w[3]) & 0xFFu) << (8 * sq);
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    __syncthreads();
    {
      const uint32_t t = opaque_lane();
      const int ch = (int)(t >> 1), h = (int)(t & 1u), sw = ch & 7;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int c = ch + 128 * m;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<u32x4*>(buf + c * 128 + (((2 * q + h) ^ sw) * 16)) = u32x4{acc[q][m][0], acc[q][m][1], acc[q][m][2], acc[q][m][3]};
          csc[c * 8 + 2 * q + h] = (uint8_t)(scol[m] >> (8 * q));
        }
      }
    }
    __syncthreads();
    {
      const uint32_t t = opaque_lane();
      const int c8 = (int)(t >> 3), j = (int)(t & 7u);
      const uint8_t* lsrc = buf + c8 * 128 + ((j ^ (c8 & 7)) * 16);
      uint8_t* dst = codes_col + (c0 + c8) * (rows / 2) + fr / 2 + 16 * j;
#pragma unroll
      for (int it = 0; it < 8; ++it)
        *reinterpret_cast<u32x4*>(dst + (int64_t)it * 32 * (rows / 2)) = *reinterpret_cast<const u32x4*>(lsrc + it * 4096);
      *reinterpret_cast<uint2*>(scales_col + (c0 + t) * (rows / 32) + fr / 32) = *reinterpret_cast<const uint2*>(csc + t * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// The 16x16 NVFP4 pattern (the bf16 W and W^T kernel's memory traffic, moving bytes
// only): a workgroup owns a 128 x 128 tile; the four lanes of a quad own a 16 x 16
// block, each an 8 x 8 quarter (8 rows of one 16-byte chunk), folded to 4 bytes per
// row at the row-code position; the quarter's eight column dwords go through LDS and
// leave as 16-byte pieces, four lanes (64 bytes) per column; one 8-byte run per row
// and per column of the tile for the scales. The 16 tiles of a 4 x 4 superblock go to
// one XCD in consecutive turns, as in the kernel.
__global__ __launch_bounds__(kThreads) void pattern_2d_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                              uint8_t* codes_row, uint8_t* scales_row,
                                                              uint8_t* codes_col, uint8_t* scales_col, uint32_t tiles_c,
                                                              uint32_t sb_c, uint32_t sbs) {
  __shared__ uint32_t ct[128][16];
  __shared__ uint32_t kblk[64];
  const uint32_t t = threadIdx.x;
  const uint32_t xcd = blockIdx.x & 7u, slot = blockIdx.x >> 3;
  const uint32_t sb = (slot >> 4) * 8u + xcd, w = slot & 15u;
  if (sb >= sbs) return;
  const uint32_t sbr = sb / sb_c, sbc = sb - sbr * sb_c;
  const uint32_t tr = 4u * sbr + (w >> 2), tc = 4u * sbc + (w & 3u);
  if ((int64_t)tr * 128 >= rows || tc >= tiles_c) return;
  const int64_t r0 = (int64_t)tr * 128, c0 = (int64_t)tc * 128;
  const int b = (int)(t >> 2), q = (int)(t & 3u);
  const int row0 = (b >> 3) * 16 + (q >> 1) * 8, col0 = (b & 7) * 16 + (q & 1) * 8;
  const uint16_t* xq = x + (r0 + row0) * cols + c0 + col0;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xq + (int64_t)i * cols));
  uint32_t code[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) code[i] = v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  uint8_t* crow = codes_row + (r0 + row0) * (cols / 2) + (c0 + col0) / 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(crow + (int64_t)i * (cols / 2)) = code[i];
  if (q == 0) kblk[b] = code[0] & 0xFFu;
#pragma unroll
  for (int j = 0; j < 8; ++j) ct[col0 + j][row0 >> 3] = code[j] ^ (uint32_t)j;
  __syncthreads();
  if (t < 128) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= kblk[(t >> 4) * 8 + i] << (8 * i);
      hi |= kblk[(t >> 4) * 8 + 4 + i] << (8 * i);
    }
    *reinterpret_cast<u32x2*>(scales_row + (r0 + t) * (cols / 16) + c0 / 16) = u32x2{lo, hi};
    uint32_t clo = 0, chi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      clo |= kblk[i * 8 + (t >> 4)] << (8 * i);
      chi |= kblk[(4 + i) * 8 + (t >> 4)] << (8 * i);
    }
    *reinterpret_cast<u32x2*>(scales_col + (c0 + t) * (rows / 16) + r0 / 16) = u32x2{clo, chi};
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int pc = (int)t + k * 256, c = pc >> 2, h = pc & 3;
    __builtin_nontemporal_store(u32x4{ct[c][4 * h], ct[c][4 * h + 1], ct[c][4 * h + 2], ct[c][4 * h + 3]},
                                reinterpret_cast<u32x4*>(codes_col + (c0 + c) * (rows / 2) + (r0 + h * 32) / 2));
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

// The fused row + column strip access pattern over a bf16 [rows, cols] tensor
// (rows % 256 == 0, cols % 256 == 0), with as many 256-row units per workgroup as
// the bf16 MXFP4 row + column kernel takes; outputs sized as the MXFP4 row- and
// column-wise outputs. Returns 0, 1 for bad sizes, 2 for a launch failure.
int mxq_stream_strip_pattern(const void* x, int64_t rows, int64_t cols, void* codes_row, void* scales_row,
                             void* codes_col, void* scales_col, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rows <= 0 || cols <= 0 || cols % 256 || rows % 256 || rows >= ((int64_t)1 << 30)) return 1;
  const int64_t strips = cols / 256, flushes = rows / 256;
  const int64_t per_wg = std::min<int64_t>(4, std::max<int64_t>(1, flushes * strips / 1024));
  const int64_t units = (flushes + per_wg - 1) / per_wg;
  if (units * strips >= ((int64_t)1 << 31)) return 1;
  hipLaunchKernelGGL(strip_pattern_kernel, dim3((uint32_t)(units * strips)), dim3(kThreads), 0, st,
                     reinterpret_cast<const uint16_t*>(x), rows, cols, (uint8_t*)codes_row, (uint8_t*)scales_row,
                     (uint8_t*)codes_col, (uint8_t*)scales_col, (uint32_t)strips, (uint32_t)flushes, (uint32_t)per_wg);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The 16x16 NVFP4 access pattern over a bf16 [rows, cols] tensor (both multiples of
// 128); outputs sized as the NVFP4 row- and column-wise outputs. Returns 0, 1 for bad
// sizes, 2 for a launch failure.
int mxq_stream_2d_pattern(const void* x, int64_t rows, int64_t cols, void* codes_row, void* scales_row,
                          void* codes_col, void* scales_col, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (rows <= 0 || cols <= 0 || rows % 128 || cols % 128 || rows / 128 * (cols / 128) >= ((int64_t)1 << 24)) return 1;
  const uint32_t tiles_r = (uint32_t)(rows / 128), tiles_c = (uint32_t)(cols / 128);
  const uint32_t sb_c = (tiles_c + 3u) / 4u, sbs = ((tiles_r + 3u) / 4u) * sb_c;
  const uint32_t grid = (sbs + 7u) / 8u * 128u;
  hipLaunchKernelGGL(pattern_2d_kernel, dim3(grid), dim3(kThreads), 0, st, reinterpret_cast<const uint16_t*>(x), rows,
                     cols, (uint8_t*)codes_row, (uint8_t*)scales_row, (uint8_t*)codes_col, (uint8_t*)scales_col,
                     tiles_c, sb_c, sbs);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
