// Row-wise kernels: MXFP4 / NVFP4 quantisation (nearest-even or stochastic, with
// an optional fused 16-point Hadamard transform along the row), dequantisation,
// tensor amax, and the stand-alone transform.
//
// Work split. A row-major tensor with cols % 8 == 0 is a sequence of 8-element
// chunks (16 bytes of bf16). Lane t of a 256-thread workgroup takes chunks
// base + j*256 + t for j < 4, so every load instruction of a wave reads 1 KiB of
// contiguous bf16 and every code store writes 256 contiguous bytes. A 32-element
// MXFP4 block spans 4 neighbouring lanes (a DPP quad), a 16-element NVFP4 block or
// Hadamard chunk spans 2. Output offsets follow from the chunk index alone,
// because outputs are dense; only the input address needs the row, found by a
// division by an invariant when rows are strided.
#include <algorithm>

#include "mxq_blocks.h"
#include "mxq_internal.h"

namespace mxq {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr uint32_t kChunksPerWG = kThreads * kUnroll;
// Dequantisation writes 4x what it reads; with 2 chunks per lane its stores stream
// measurably faster than with 4 (more workgroups in flight, each shorter).
constexpr int kDeqUnroll = 2;
constexpr uint32_t kDeqChunksPerWG = kThreads * kDeqUnroll;

struct RowParams {
  const void* x;
  int64_t ldx;
  uint32_t chunks;   // 8-element chunks in this slab
  FastDiv cpr;       // chunks per row
  uint8_t* codes;
  uint8_t* scales;
  uint64_t sr_seed, sr_base;
  uint32_t sign_mask;
  const float* amax;
  int st_given;      // *amax holds the tensor scale, not the amax
  float* tensor_scale;
};

template <bool CONTIG>
__device__ __forceinline__ size_t in_offset(uint32_t c, const RowParams& p) {
  if (CONTIG) return (size_t)c * 8;
  const uint32_t row = fdiv(c, p.cpr);
  const uint32_t c8 = c - row * p.cpr.d;
  return (size_t)row * (size_t)p.ldx + (size_t)c8 * 8;
}

template <typename T, int FMT, int SR, bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(RowParams p) {
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  const uint32_t base = blockIdx.x * kChunksPerWG + threadIdx.x;
  NvTensor nt;
  if constexpr (FMT == kNV) {
    nt = nv_tensor_load(p.amax, p.st_given);
    if (p.tensor_scale && blockIdx.x == 0 && threadIdx.x == 0) *p.tensor_scale = nt.st;
    if constexpr (RHT) nv_tensor_times4(nt);
  }
  // a chunk's parity (its half of a 16-element Hadamard chunk) is the lane's parity
  SignFlips flips;
  if constexpr (RHT) flips = make_flips<T>(p.sign_mask, threadIdx.x & 1u);
  Raw<T> raw[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const uint32_t c = base + j * kThreads;
    if (c < p.chunks) load_raw(x, in_offset<CONTIG>(c, p), raw[j]);
    else zero_raw(raw[j]);
  }
  // the random values of every chunk first: the generator chains of the chunks are
  // independent, so they issue interleaved (the encoders below branch per chunk)
  u32x4 rw[kUnroll][SR == kSrWords ? 2 : 1];
  if constexpr (SR == kSrWords) {
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint64_t n = p.sr_base + (uint64_t)(base + j * kThreads) * 8;
      if ((p.sr_base & 3u) == 0u) {  // uniform: whole Philox calls
        rw[j][0] = philox_words4(n, p.sr_seed);
        rw[j][1] = philox_words4(n + 4, p.sr_seed);
      } else {
        uint32_t u[8];
        philox_words<8>(n, p.sr_seed, u);
        rw[j][0] = u32x4{u[0], u[1], u[2], u[3]};
        rw[j][1] = u32x4{u[4], u[5], u[6], u[7]};
      }
    }
  } else if constexpr (SR == kSrHalves) {
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      rw[j][0] = philox_halves_words(p.sr_base + (uint64_t)(base + j * kThreads) * 8, p.sr_seed);
    // keeps the four chains together: left alone, the compiler sinks each into its
    // chunk's encoder, where it runs as one long dependent chain (measured slower)
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      asm volatile("" : "+v"(rw[j][0].x), "+v"(rw[j][0].y), "+v"(rw[j][0].z), "+v"(rw[j][0].w));
  }
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const uint32_t c = base + j * kThreads;
    uint32_t byte;
    uint32_t packed;
    if constexpr (FMT == kMX && !SR && !RHT && sizeof(T) == 2) {
      packed = mx_encode8_bf16(raw[j].w, byte);
    } else {
      if constexpr (RHT) flip(raw[j], flips);
      float v[8];
      to_f32(raw[j], v);
      if constexpr (RHT) h16_pair(v, threadIdx.x & 1u);
      uint32_t u[8];
      if constexpr (SR == kSrWords) {
        u[0] = rw[j][0].x; u[1] = rw[j][0].y; u[2] = rw[j][0].z; u[3] = rw[j][0].w;
        u[4] = rw[j][1].x; u[5] = rw[j][1].y; u[6] = rw[j][1].z; u[7] = rw[j][1].w;
      } else if constexpr (SR == kSrHalves) {
        expand_halves(rw[j][0], u);
      }
      if constexpr (FMT == kMX) packed = mx_encode8<SR != kRne, RHT ? 2 : 0, sizeof(T) == 2 && !RHT>(v, u, byte);
      else packed = nv_encode8<SR != kRne>(v, u, nt, byte);
    }
    if (c < p.chunks) {
      reinterpret_cast<uint32_t*>(p.codes)[c] = packed;
      if constexpr (FMT == kMX) {
        if ((c & 3u) == 0u) p.scales[c >> 2] = (uint8_t)byte;
      } else {
        if ((c & 1u) == 0u) p.scales[c >> 1] = (uint8_t)byte;
      }
    }
  }
}

template <typename T, int FMT, int SR, bool RHT>
static hipError_t launch_rows_t(const RowLaunch& a, hipStream_t st) {
  // slabs of whole rows with fewer than 2^30 chunks keep every index in 32 bits
  const int64_t cpr = a.cols / 8;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < a.rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, a.rows - r0);
    RowParams p;
    p.x = reinterpret_cast<const T*>(a.x) + r0 * a.ldx;
    p.ldx = a.ldx;
    p.chunks = (uint32_t)(nr * cpr);
    FastDivHost fd = make_fastdiv((uint32_t)cpr);
    p.cpr = FastDiv{fd.d, fd.m, fd.s};
    p.codes = a.codes + r0 * (a.cols / 2);
    const int bs = FMT == kMX ? 32 : 16;
    p.scales = a.scales + r0 * (a.cols / bs);
    p.sr_seed = a.sr_seed;
    p.sr_base = a.sr_base + (uint64_t)(r0 * a.cols);
    p.sign_mask = a.sign_mask;
    p.amax = a.amax;
    p.st_given = a.st_given ? 1 : 0;
    p.tensor_scale = r0 == 0 ? a.tensor_scale : nullptr;
    const uint32_t grid = (p.chunks + kChunksPerWG - 1) / kChunksPerWG;
    const bool contig = a.ldx == a.cols;
    if (contig)
      hipLaunchKernelGGL((quantize_rows_kernel<T, FMT, SR, RHT, true>), dim3(grid), dim3(kThreads), 0,
                         st, p);
    else
      hipLaunchKernelGGL((quantize_rows_kernel<T, FMT, SR, RHT, false>), dim3(grid), dim3(kThreads), 0,
                         st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int FMT>
static hipError_t launch_rows_f(const RowLaunch& a, hipStream_t st) {
  if (a.sr == kSrWords)
    return a.rht ? launch_rows_t<T, FMT, kSrWords, true>(a, st) : launch_rows_t<T, FMT, kSrWords, false>(a, st);
  if (a.sr == kSrHalves)
    return a.rht ? launch_rows_t<T, FMT, kSrHalves, true>(a, st) : launch_rows_t<T, FMT, kSrHalves, false>(a, st);
  return a.rht ? launch_rows_t<T, FMT, kRne, true>(a, st) : launch_rows_t<T, FMT, kRne, false>(a, st);
}

hipError_t launch_quantize_rows(const RowLaunch& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  if (a.dtype == 0)
    return a.fmt == kMX ? launch_rows_f<uint16_t, kMX>(a, st) : launch_rows_f<uint16_t, kNV>(a, st);
  return a.fmt == kMX ? launch_rows_f<float, kMX>(a, st) : launch_rows_f<float, kNV>(a, st);
}

// ---------------------------------------------------------------------------
// Dequantisation. Each lane turns one dword of codes (8 elements) into 8 outputs.

struct DeqParams {
  const uint32_t* codes;
  const uint8_t* scales;
  uint32_t chunks;
  const float* tensor_scale;
  void* y;
};

// RN to bf16 of the exact product a * s_t (a = v * s_b exact, at most 6 bits):
// the fp32 product is made round-to-odd with the exact fma residual, which makes
// the second rounding to bf16 a correct single rounding. Products are formed at
// s_t * 2^k (k = 64 for tiny s_t) so the residual never underflows.
__device__ __forceinline__ uint32_t bf16_of_product(float a, float st_scaled, int k) {
  const float p = a * st_scaled;
  const float r = fmaf(a, st_scaled, -p);
  uint32_t b = as_u(p);
  if (r != 0.0f && (b & 1u) == 0u && (b & 0x7FFFFFFFu) != 0u && (b & 0x7FFFFFFFu) < 0x7F800000u) {
    const bool away = (r > 0.0f) == (p > 0.0f);
    b = away ? b + 1u : b - 1u;
  }
  const uint32_t sign = b & 0x80000000u;
  uint32_t mag = b & 0x7FFFFFFFu;
  if (mag >= 0x7F800000u) return (sign >> 16) | 0x7F80u | ((mag > 0x7F800000u) ? 0x40u : 0u);
  if (k) {
    const float pm = as_f(mag);
    if (pm >= 0x1p-62f) {
      mag -= (uint32_t)k << 23;  // now the unscaled value, a normal fp32
    } else {
      // bf16 subnormal: multiples of 2^-133 = 2^-69 in the scaled domain
      const uint32_t q = (uint32_t)__builtin_rintf(pm * 0x1p69f);
      return (sign >> 16) | q;
    }
  }
  const uint32_t rnd = mag + 0x7FFFu + ((mag >> 16) & 1u);
  return (sign >> 16) | (rnd >> 16);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DeqParams p) {
  const uint32_t base = blockIdx.x * kDeqChunksPerWG + threadIdx.x;
  float st = 0.0f, st_s = 0.0f;
  int k = 0;
  if constexpr (FMT == kNV) {
    st = *p.tensor_scale;
    k = (fabsf(st) < 0x1p-60f) ? 64 : 0;
    st_s = ldexpf(st, k);
  }
  uint32_t w[kDeqUnroll];
  uint32_t sb[kDeqUnroll];
#pragma unroll
  for (int j = 0; j < kDeqUnroll; ++j) {
    const uint32_t c = base + j * kThreads;
    w[j] = 0;
    sb[j] = 0;
    if (c < p.chunks) {
      w[j] = load_nt(p.codes + c);
      sb[j] = p.scales[FMT == kMX ? (c >> 2) : (c >> 1)];
    }
  }
#pragma unroll
  for (int j = 0; j < kDeqUnroll; ++j) {
    const uint32_t c = base + j * kThreads;
    if (c >= p.chunks) continue;
    uint4 ov;
    if constexpr (FMT == kMX) {
      const uint32_t byte = sb[j];
      const float scale = e8m0_operand(min(byte, 254u));
      const bool nan = byte == 255u;
      uint32_t o[4];
      o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 0));
      o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 1));
      o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 2));
      o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 3));
      ov = nan ? make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u) : make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      const uint32_t byte = sb[j];
      const bool nan = (byte & 0x7Fu) == 0x7Fu || !(fabsf(st) <= 3.40282347e38f);
      const float sbv = as_f(as_u(e4m3_value(byte & 0x7Fu)) | ((byte & 0x80u) << 24));
      // signed E2M1 values, exact
      float a[8];
      const f32x2_t d[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 3)};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        a[2 * h] = d[h].x * sbv;  // exact: at most 6 significant bits
        a[2 * h + 1] = d[h].y * sbv;
      }
      // RN_bf16(RN_f32(a s_t)) equals RN_bf16(a s_t) unless the fp32 product lands
      // exactly on a bf16 midpoint (low half 0x8000): only such lanes take the
      // exact residual path.
      float pr[8];
      bool mid = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = a[i] * st;
        mid |= (uint16_t)as_u(pr[i]) == 0x8000u;
      }
      uint32_t o[4];
      if (!mid) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const bf16x2_t r = {(__bf16)pr[2 * h], (__bf16)pr[2 * h + 1]};
          o[h] = __builtin_bit_cast(uint32_t, r);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          o[h] = bf16_of_product(a[2 * h], st_s, k) | (bf16_of_product(a[2 * h + 1], st_s, k) << 16);
      }
      ov = nan ? make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u) : make_uint4(o[0], o[1], o[2], o[3]);
    }
    store_nt(reinterpret_cast<uint4*>(p.y) + c, ov);
  }
}

// fp32 output. A unit is 4 elements: 2 code bytes in, 16 bytes out. Consecutive
// lanes take consecutive units, so every store instruction writes 1 KiB of whole
// lines (a lane owning 8 elements would write its 32 bytes as two half-lines).
template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_f32_kernel(DeqParams p) {
  constexpr int kU = 2 * kDeqUnroll;
  const uint32_t units = p.chunks * 2u;
  const uint32_t base = blockIdx.x * (kThreads * kU) + threadIdx.x;
  const uint16_t* codes = reinterpret_cast<const uint16_t*>(p.codes);
  float st = 0.0f;
  if constexpr (FMT == kNV) st = *p.tensor_scale;
  uint32_t w[kU];
  uint32_t sb[kU];
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    const uint32_t u = base + j * kThreads;
    w[j] = 0;
    sb[j] = 0;
    if (u < units) {
      w[j] = codes[u];
      sb[j] = p.scales[FMT == kMX ? (u >> 3) : (u >> 2)];
    }
  }
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    const uint32_t u = base + j * kThreads;
    if (u >= units) continue;
    float v[4];
    bool nan;
    if constexpr (FMT == kMX) {
      const uint32_t byte = sb[j];
      const float scale = e8m0_operand(min(byte, 254u));
      nan = byte == 255u;
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], scale, 0);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], scale, 1);
      v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    } else {
      const uint32_t byte = sb[j];
      nan = (byte & 0x7Fu) == 0x7Fu || !(fabsf(st) <= 3.40282347e38f);
      const float sbv = as_f(as_u(e4m3_value(byte & 0x7Fu)) | ((byte & 0x80u) << 24));
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 0);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 1);
      // v * s_b is exact (at most 6 significant bits); one rounding with s_t
      v[0] = (a.x * sbv) * st; v[1] = (a.y * sbv) * st; v[2] = (b.x * sbv) * st; v[3] = (b.y * sbv) * st;
    }
    const float qn = as_f(0x7FC00000u);
    store_nt(reinterpret_cast<float4*>(p.y) + u,
             nan ? make_float4(qn, qn, qn, qn) : make_float4(v[0], v[1], v[2], v[3]));
  }
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int fmt, int64_t rows,
                             int64_t cols, const float* tensor_scale, void* y, int out_dtype,
                             hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cpr = cols / 8;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  const int bs = fmt == kMX ? 32 : 16;
  const size_t osz = out_dtype == 0 ? 2 : 4;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    DeqParams p;
    p.codes = reinterpret_cast<const uint32_t*>(codes + r0 * (cols / 2));
    p.scales = scales + r0 * (cols / bs);
    p.chunks = (uint32_t)(nr * cpr);
    p.tensor_scale = tensor_scale;
    p.y = reinterpret_cast<uint8_t*>(y) + (size_t)r0 * cols * osz;
    const uint32_t grid = (p.chunks + kDeqChunksPerWG - 1) / kDeqChunksPerWG;
    // both kernels cover kDeqChunksPerWG chunks (8 elements each) per workgroup
    if (fmt == kMX) {
      if (out_dtype == 0) hipLaunchKernelGGL((dequant_kernel<kMX>), dim3(grid), dim3(kThreads), 0, st, p);
      else hipLaunchKernelGGL((dequant_f32_kernel<kMX>), dim3(grid), dim3(kThreads), 0, st, p);
    } else {
      if (out_dtype == 0) hipLaunchKernelGGL((dequant_kernel<kNV>), dim3(grid), dim3(kThreads), 0, st, p);
      else hipLaunchKernelGGL((dequant_f32_kernel<kNV>), dim3(grid), dim3(kThreads), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Tensor amax: a grid-stride pass over 8-element chunks; |x| compared as fp32 bit
// patterns (NaN > Inf > finite), wave and workgroup reductions, one atomic max
// per workgroup on a slot the preceding one-thread kernel zeroed.

__global__ void amax_init_kernel(float* out) { *reinterpret_cast<uint32_t*>(out) = 0u; }

__global__ void tensor_scale_in_place_kernel(float* slot) { *slot = nv_tensor(*slot).st; }

hipError_t launch_tensor_scale_in_place(float* slot, hipStream_t st) {
  hipLaunchKernelGGL(tensor_scale_in_place_kernel, dim3(1), dim3(1), 0, st, slot);
  return hipGetLastError();
}

template <typename T, bool CONTIG>
__global__ __launch_bounds__(kThreads) void amax_kernel(RowParams p, uint32_t* out) {
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  // m: the largest |x| bit pattern (NaN > Inf > finite), as fp32 bits
  uint32_t m = 0;
  constexpr int U = 8;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t c0 = blockIdx.x * kThreads + threadIdx.x; c0 < p.chunks; c0 += stride * U) {
    Raw<T> r[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t c = c0 + j * stride;
      if (c < p.chunks) load_raw(x, in_offset<CONTIG>(c, p), r[j]);
      else zero_raw(r[j]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {r[j].w.x, r[j].w.y, r[j].w.z, r[j].w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu) << 16);
      } else {
        float v[8];
        to_f32(r[j], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, as_u(v[i]) & 0x7FFFFFFFu);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = red[0];
    for (int i = 1; i < kThreads / 64; ++i) t = max(t, red[i]);
    atomicMax(out, t);
  }
}

hipError_t launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       float* amax_out, hipStream_t st) {
  hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1), 0, st, amax_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) return e;
  const int64_t cpr = cols / 8;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  const size_t esz = dtype == 0 ? 2 : 4;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    RowParams p{};
    p.x = reinterpret_cast<const uint8_t*>(x) + (size_t)r0 * ldx * esz;
    p.ldx = ldx;
    p.chunks = (uint32_t)(nr * cpr);
    FastDivHost fd = make_fastdiv((uint32_t)cpr);
    p.cpr = FastDiv{fd.d, fd.m, fd.s};
    // few workgroups: each ends with one atomic on the same word, and contention on
    // that word costs more than the shorter grid-stride loops save
    const uint32_t want = (p.chunks + kThreads * 8 - 1) / (kThreads * 8);
    const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(want, 512));
    uint32_t* out = reinterpret_cast<uint32_t*>(amax_out);
    const bool contig = ldx == cols;
    if (dtype == 0) {
      if (contig) hipLaunchKernelGGL((amax_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, st, p, out);
      else hipLaunchKernelGGL((amax_kernel<uint16_t, false>), dim3(grid), dim3(kThreads), 0, st, p, out);
    } else {
      if (contig) hipLaunchKernelGGL((amax_kernel<float, true>), dim3(grid), dim3(kThreads), 0, st, p, out);
      else hipLaunchKernelGGL((amax_kernel<float, false>), dim3(grid), dim3(kThreads), 0, st, p, out);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Amax of the Hadamard transform: max |(1/4) H16 (s * x)| over every 16-chunk along
// the rows (the tensor amax for NVFP4 quantisation of the transformed tensor). The
// factor 1/4 is exact and applied to each thread's maximum.
template <typename T, bool CONTIG>
__global__ __launch_bounds__(kThreads) void rht_amax_rows_kernel(RowParams p, uint32_t* out) {
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  // a chunk's parity (its half of a 16-element chunk) is the lane's parity: the
  // grid stride is even, and so is the chunk count (cols % 16 == 0), so the two lanes
  // of a pair always leave the loop together
  const SignFlips flips = make_flips<T>(p.sign_mask, threadIdx.x & 1u);
  float m = 0.0f;
  constexpr int U = 4;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t c0 = blockIdx.x * kThreads + threadIdx.x; c0 < p.chunks; c0 += stride * U) {
    Raw<T> r[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t c = c0 + j * stride;
      if (c < p.chunks) load_raw(x, in_offset<CONTIG>(c, p), r[j]);
      else zero_raw(r[j]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      flip(r[j], flips);
      float v[8];
      to_f32(r[j], v);
      h16_pair(v, threadIdx.x & 1u);
      m = __builtin_elementwise_maximum(m, absmax8(v));
    }
  }
  uint32_t mb = as_u(m * 0.25f) & 0x7FFFFFFFu;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o));
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mb;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = red[0];
    for (int i = 1; i < kThreads / 64; ++i) v = max(v, red[i]);
    atomicMax(out, v);
  }
}

// The same along the columns: a unit is 16 rows x 8 columns; the transform runs down
// each column in registers (row i of the unit takes sign bit i).
struct RhtColParams {
  const void* x;
  int64_t ldx;
  uint32_t cpr;    // 8-column chunks per row
  uint32_t units;  // (rows / 16) * cpr
  uint32_t sign_mask;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rht_amax_cols_kernel(RhtColParams p, uint32_t* out) {
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  float m = 0.0f;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < p.units; u += gridDim.x * kThreads) {
    const uint32_t g = u / p.cpr, c = u - g * p.cpr;
    Raw<T> r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) load_raw(x, (size_t)(16 * g + i) * p.ldx + (size_t)c * 8, r[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = raw_elem(r[i], j);
        v[i] = ((p.sign_mask >> i) & 1u) ? -e : e;
      }
      h16_local(v);
      m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(absmax8(v), absmax8(v + 8)));
    }
  }
  uint32_t mb = as_u(m * 0.25f) & 0x7FFFFFFFu;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, o));
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mb;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = red[0];
    for (int i = 1; i < kThreads / 64; ++i) v = max(v, red[i]);
    atomicMax(out, v);
  }
}

hipError_t launch_rht_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, bool colwise,
                           uint32_t sign_mask, float* amax_out, hipStream_t st) {
  hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1), 0, st, amax_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) return e;
  const size_t esz = dtype == 0 ? 2 : 4;
  uint32_t* out = reinterpret_cast<uint32_t*>(amax_out);
  const int64_t cpr = cols / 8;
  if (!colwise) {
    const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
    for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
      const int64_t nr = std::min(max_rows, rows - r0);
      RowParams p{};
      p.x = reinterpret_cast<const uint8_t*>(x) + (size_t)r0 * ldx * esz;
      p.ldx = ldx;
      p.chunks = (uint32_t)(nr * cpr);
      FastDivHost fd = make_fastdiv((uint32_t)cpr);
      p.cpr = FastDiv{fd.d, fd.m, fd.s};
      p.sign_mask = sign_mask;
      const uint32_t want = (p.chunks + kThreads * 4 - 1) / (kThreads * 4);
      const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(want, 512));
      const bool contig = ldx == cols;
      if (dtype == 0) {
        if (contig) hipLaunchKernelGGL((rht_amax_rows_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, st, p, out);
        else hipLaunchKernelGGL((rht_amax_rows_kernel<uint16_t, false>), dim3(grid), dim3(kThreads), 0, st, p, out);
      } else {
        if (contig) hipLaunchKernelGGL((rht_amax_rows_kernel<float, true>), dim3(grid), dim3(kThreads), 0, st, p, out);
        else hipLaunchKernelGGL((rht_amax_rows_kernel<float, false>), dim3(grid), dim3(kThreads), 0, st, p, out);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // column direction: slabs of whole 16-row groups with fewer than 2^30 units
  const int64_t max_rows = 16 * std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    RhtColParams p;
    p.x = reinterpret_cast<const uint8_t*>(x) + (size_t)r0 * ldx * esz;
    p.ldx = ldx;
    p.cpr = (uint32_t)cpr;
    p.units = (uint32_t)((nr / 16) * cpr);
    p.sign_mask = sign_mask;
    const uint32_t want = (p.units + kThreads - 1) / kThreads;
    const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>(want, 1024));
    if (dtype == 0) hipLaunchKernelGGL((rht_amax_cols_kernel<uint16_t>), dim3(grid), dim3(kThreads), 0, st, p, out);
    else hipLaunchKernelGGL((rht_amax_cols_kernel<float>), dim3(grid), dim3(kThreads), 0, st, p, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


// ---------------------------------------------------------------------------
// The transform alone, fp32 out.

template <typename T, bool CONTIG>
__global__ __launch_bounds__(kThreads) void rht_apply_kernel(RowParams p, float* y) {
  const T* __restrict__ x = reinterpret_cast<const T*>(p.x);
  const uint32_t base = blockIdx.x * kChunksPerWG + threadIdx.x;
  const SignFlips flips = make_flips<T>(p.sign_mask, threadIdx.x & 1u);
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const uint32_t c = base + j * kThreads;
    Raw<T> r;
    if (c < p.chunks) load_raw(x, in_offset<CONTIG>(c, p), r);
    else zero_raw(r);
    flip(r, flips);
    float v[8];
    to_f32(r, v);
    h16_pair(v, threadIdx.x & 1u);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= 0.25f;
    if (c < p.chunks) {
      float4* o = reinterpret_cast<float4*>(y) + (size_t)c * 2;
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

hipError_t launch_rht_apply(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint32_t sign_mask, float* y, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cpr = cols / 8;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  const size_t esz = dtype == 0 ? 2 : 4;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, rows - r0);
    RowParams p{};
    p.x = reinterpret_cast<const uint8_t*>(x) + (size_t)r0 * ldx * esz;
    p.ldx = ldx;
    p.chunks = (uint32_t)(nr * cpr);
    FastDivHost fd = make_fastdiv((uint32_t)cpr);
    p.cpr = FastDiv{fd.d, fd.m, fd.s};
    p.sign_mask = sign_mask;
    float* yo = y + (size_t)r0 * cols;
    const uint32_t grid = (p.chunks + kChunksPerWG - 1) / kChunksPerWG;
    const bool contig = ldx == cols;
    if (dtype == 0) {
      if (contig) hipLaunchKernelGGL((rht_apply_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, st, p, yo);
      else hipLaunchKernelGGL((rht_apply_kernel<uint16_t, false>), dim3(grid), dim3(kThreads), 0, st, p, yo);
    } else {
      if (contig) hipLaunchKernelGGL((rht_apply_kernel<float, true>), dim3(grid), dim3(kThreads), 0, st, p, yo);
      else hipLaunchKernelGGL((rht_apply_kernel<float, false>), dim3(grid), dim3(kThreads), 0, st, p, yo);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mxq
