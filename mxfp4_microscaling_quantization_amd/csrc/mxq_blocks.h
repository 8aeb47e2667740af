// Block-level encoders shared by the row-wise and tiled kernels: raw 16-byte
// loads, the 16-point Hadamard butterfly over a lane pair, and the MXFP4 / NVFP4
// encoders of 8 values per lane (blocks spanning 4 or 2 lanes of a DPP quad).
#pragma once

#include "mxq_device.h"

namespace mxq {

template <typename T>
struct Raw;
template <>
struct Raw<uint16_t> {
  uint4 w;
};
template <>
struct Raw<float> {
  float4 a, b;
};

__device__ __forceinline__ void load_raw(const uint16_t* x, size_t off, Raw<uint16_t>& r) {
  r.w = load_nt(reinterpret_cast<const uint4*>(x + off));
}
__device__ __forceinline__ void load_raw(const float* x, size_t off, Raw<float>& r) {
  r.a = load_nt(reinterpret_cast<const float4*>(x + off));
  r.b = load_nt(reinterpret_cast<const float4*>(x + off + 4));
}
__device__ __forceinline__ void zero_raw(Raw<uint16_t>& r) { r.w = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_raw(Raw<float>& r) {
  r.a = make_float4(0, 0, 0, 0);
  r.b = r.a;
}

__device__ __forceinline__ void to_f32(const Raw<uint16_t>& r, float v[8]) {
  const uint32_t w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = as_f(w[i] << 16);
    v[2 * i + 1] = as_f(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void to_f32(const Raw<float>& r, float v[8]) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}

// y = (1/4) H16 (s * x) over the 16 elements held by a lane pair (this lane holds
// positions half*8 .. half*8+7). Stages h = 1, 2, 4 inside the lane, h = 8 across
// the pair; fp32 throughout, then the exact scaling by 1/4.
__device__ __forceinline__ void rht16_pair(float v[8], uint32_t half, uint32_t sign_mask) {
  const uint32_t bits = sign_mask >> (half * 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = as_f(as_u(v[i]) ^ (((bits >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dppf<kQuadSwap1>(v[i]);
    v[i] = half ? (o - v[i]) : (v[i] + o);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= 0.25f;
}

__device__ __forceinline__ void sr_words8(uint64_t n, uint64_t seed, uint32_t u[8]) {
  philox_words<8>(n, seed, u);
}

// MXFP4: 8 values of one lane (a quarter of a 32-block) -> 8 codes, block byte.
template <bool SR>
__device__ __forceinline__ uint32_t mx_encode8(const float v[8], const uint32_t u[8],
                                               uint32_t& byte) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = max(am, as_u(v[i]) & 0x7FFFFFFFu);
  am = max(am, dpp<kQuadSwap1>(am));
  am = max(am, dpp<kQuadSwap2>(am));
  const uint32_t ea = am >> 23;  // 255: NaN or Inf in the block
  byte = ea >= 255u ? 255u : (ea > 2u ? ea - 2u : 0u);
  uint32_t packed = 0;
  if constexpr (SR) {
    const float inv = as_f((254u - min(byte, 252u)) << 23);  // 2^-E
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = fabsf(v[i]) * inv;
      const uint32_t c = e2m1_sr(y, u[i]) | ((as_u(v[i]) >> 31) << 3);
      packed |= c << (4 * i);
    }
  } else {
    packed = fp4x8_from_f32(v, e8m0_operand(min(byte, 254u)));
  }
  return byte == 255u ? 0u : packed;
}

// MXFP4 round-to-nearest-even of 8 raw bf16 values (4 dwords): integer amax on the
// magnitude halves, then four hardware conversions.
__device__ __forceinline__ uint32_t mx_encode8_bf16(const uint4& r, uint32_t& byte) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  m = max(m, dpp<kQuadSwap1>(m));
  m = max(m, dpp<kQuadSwap2>(m));
  const uint32_t ea = m >> 7;  // bf16 exponent field of the block amax; 255: NaN/Inf
  byte = ea >= 255u ? 255u : (ea > 2u ? ea - 2u : 0u);
  const uint32_t packed = fp4x8_from_bf16(w, e8m0_operand(min(byte, 254u)));
  return byte == 255u ? 0u : packed;
}

// NVFP4: 8 values of one lane (half a 16-block) -> 8 codes, block byte.
template <bool SR>
__device__ __forceinline__ uint32_t nv_encode8(const float v[8], const uint32_t u[8],
                                               const NvTensor& t, uint32_t& byte) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = max(am, as_u(v[i]) & 0x7FFFFFFFu);
  am = max(am, dpp<kQuadSwap1>(am));
  uint32_t signs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) signs |= (as_u(v[i]) >> 31) << (4 * i + 3);
  if (t.mode == 2 || am >= 0x7F800000u) {
    byte = 0x7Fu;
    return 0u;
  }
  if (t.mode == 1) {
    byte = 0u;
    return signs;
  }
  const float a_n = ldexpf(as_f(am), -t.et);
  const uint32_t k = nv_block_scale(a_n, t.st_n);
  byte = k;
  if (k == 0u) return signs;
  if constexpr (SR) return nv_codes8_sr(v, u, t, k);
  return nv_codes8_rne(v, t, k);
}

}  // namespace mxq
