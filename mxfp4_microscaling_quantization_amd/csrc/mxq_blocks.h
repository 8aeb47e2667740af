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

// One 8-element chunk, by default with nontemporal loads: on inputs that come from
// HBM (not from the 256 MB MALL) they stream measurably faster than plain loads.
template <bool NT = true>
__device__ __forceinline__ void load_raw(const uint16_t* x, size_t off, Raw<uint16_t>& r) {
  if constexpr (NT) r.w = load_nt(reinterpret_cast<const uint4*>(x + off));
  else r.w = *reinterpret_cast<const uint4*>(x + off);
}
template <bool NT = true>
__device__ __forceinline__ void load_raw(const float* x, size_t off, Raw<float>& r) {
  if constexpr (NT) {
    r.a = load_nt(reinterpret_cast<const float4*>(x + off));
    r.b = load_nt(reinterpret_cast<const float4*>(x + off + 4));
  } else {
    r.a = *reinterpret_cast<const float4*>(x + off);
    r.b = *reinterpret_cast<const float4*>(x + off + 4);
  }
}
__device__ __forceinline__ void zero_raw(Raw<uint16_t>& r) { r.w = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_raw(Raw<float>& r) {
  r.a = make_float4(0, 0, 0, 0);
  r.b = r.a;
}

// Element j (0..7) of a chunk as fp32.
__device__ __forceinline__ float raw_elem(const Raw<uint16_t>& r, int j) {
  const uint32_t w = j < 2 ? r.w.x : (j < 4 ? r.w.y : (j < 6 ? r.w.z : r.w.w));
  return as_f((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
__device__ __forceinline__ float raw_elem(const Raw<float>& r, int j) {
  const float4& q = j < 4 ? r.a : r.b;
  const int k = j & 3;
  return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
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

// Sign flips of the Hadamard transform applied to raw inputs. For bf16 a lane's
// 8 values are 4 dwords, so the flips are 4 XOR masks precomputed per lane.
struct SignFlips {
  uint32_t d[4];  // bf16: per dword; fp32: bits 0..7 of d[0] hold the 8 flags
};

template <typename T>
__device__ __forceinline__ SignFlips make_flips(uint32_t sign_mask, uint32_t half) {
  SignFlips f;
  const uint32_t bits = (sign_mask >> (half * 8)) & 0xFFu;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      f.d[k] = (((bits >> (2 * k)) & 1u) << 15) | (((bits >> (2 * k + 1)) & 1u) << 31);
  } else {
    f.d[0] = bits;
    f.d[1] = f.d[2] = f.d[3] = 0;
  }
  return f;
}

__device__ __forceinline__ void flip(Raw<uint16_t>& r, const SignFlips& f) {
  r.w.x ^= f.d[0]; r.w.y ^= f.d[1]; r.w.z ^= f.d[2]; r.w.w ^= f.d[3];
}
__device__ __forceinline__ void flip(Raw<float>& r, const SignFlips& f) {
  float* p = reinterpret_cast<float*>(&r);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = as_f(as_u(p[i]) ^ (((f.d[0] >> i) & 1u) << 31));
}

// Negates all 8 values of a chunk when bit is 1 (a sign shared by the chunk).
__device__ __forceinline__ void flip_all(Raw<uint16_t>& r, uint32_t bit) {
  const uint32_t m = bit * 0x80008000u;
  r.w.x ^= m; r.w.y ^= m; r.w.z ^= m; r.w.w ^= m;
}
__device__ __forceinline__ void flip_all(Raw<float>& r, uint32_t bit) {
  const uint32_t m = bit << 31;
  float* p = reinterpret_cast<float*>(&r);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = as_f(as_u(p[i]) ^ m);
}

// z = H16 (s * x) over the 16 elements held by a lane pair (this lane holds
// positions half*8 .. half*8+7; the signs are already applied). Stages h = 1, 2, 4
// inside the lane, h = 8 across the pair; fp32. The transform's factor 1/4 is
// left to the caller (an exact power of two, folded into the block scale).
__device__ __forceinline__ void h16_pair(float v[8], uint32_t half) {
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
  // stage 8: lane 2j (holding a) keeps a + b, lane 2j+1 (holding b) keeps a + (-b)
  const uint32_t neg = half << 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dppf<kQuadSwap1>(v[i]);
    v[i] = o + as_f(as_u(v[i]) ^ neg);
  }
}

// In-thread Hadamard of 16 values (signs already applied): stages 1, 2, 4, 8 in
// fp32; the factor 1/4 is folded into the block scale by the caller.
__device__ __forceinline__ void h16_local(float* v) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}


// NaN-propagating max of |v| over 8 values (v_maximum3_f32 with abs modifiers).
__device__ __forceinline__ float absmax8(const float* v) {
  float m = __builtin_elementwise_maximum(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
#pragma unroll
  for (int i = 2; i < 8; ++i) m = __builtin_elementwise_maximum(m, __builtin_fabsf(v[i]));
  return m;
}

// E8M0 byte of a block from its amax bits (exponent field ea of max|z|), where the
// values z are the real values times 2^kShift (kShift = 2 when the Hadamard
// transform's 1/4 is still to be applied). 255: NaN or Inf in the block.
template <int kShift>
__device__ __forceinline__ uint32_t mx_byte(uint32_t amax_bits) {
  const uint32_t ea = (amax_bits & 0x7FFFFFFFu) >> 23;
  return ea >= 255u ? 255u : (ea > 2u + kShift ? ea - 2u - kShift : 0u);
}

// MXFP4 stochastic rounding of 8 values that are bf16 numbers (no transform) by the
// hardware conversion: for such values the position F inside an interval is a whole
// number of units unless |x| / 2^E < 2^-16, where F < 128 and only r <= 1 can meet
// a threshold: chunks holding such an r return false and take the carry path.
__device__ __forceinline__ bool mx_sr_hw8(const float v[8], const uint32_t u[8], uint32_t b, uint32_t& packed) {
  if (min_u8(u) < 0x20000u) return false;
  uint32_t sd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sd[i] = sr_hw_seed(u[i], kSrHwExact);
  packed = fp4x8_sr_hw(v, sd, e8m0_operand(b));
  return true;
}

// MXFP4: 8 values of one lane (a quarter of a 32-block) -> 8 codes, block byte.
// kBf16: the values are bf16 numbers (stochastic rounding may use the hardware).
template <bool SR, int kShift, bool kBf16 = false>
__device__ __forceinline__ uint32_t mx_encode8(const float v[8], const uint32_t u[8],
                                               uint32_t& byte) {
  float am = absmax8(v);
  am = __builtin_elementwise_maximum(am, dppf<kQuadSwap1>(am));
  am = __builtin_elementwise_maximum(am, dppf<kQuadSwap2>(am));
  byte = mx_byte<kShift>(as_u(am));
  const uint32_t b = min(byte, 252u);
  uint32_t packed = 0;
  if constexpr (SR && kBf16 && kShift == 0) {
    if (mx_sr_hw8(v, u, b, packed)) return byte == 255u ? 0u : packed;
  }
  if constexpr (SR) {
    const float inv = as_f((254u - b - kShift) << 23);  // 2^-(E + kShift), exact
    // y is exact; only the rounding of y + 1 (half a unit of F) can mislead the
    // carry, so a window of K = 1 suffices
    float q[8];
    uint32_t low = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float q0, q1;
      e2m1_sr_carry2<1>(fabsf(v[i]) * inv, fabsf(v[i + 1]) * inv, u[i], u[i + 1], low, q0, q1);
      q[i] = with_sign_of(q0, v[i]);
      q[i + 1] = with_sign_of(q1, v[i + 1]);
    }
    if (low < 2u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = with_sign_of(e2m1_sr_value(fabsf(v[i]) * inv, u[i]), v[i]);
    }
    packed = fp4x8_from_f32(q, 1.0f);
  } else {
    packed = fp4x8_from_f32(v, e8m0_operand(b + kShift));
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
  float am = absmax8(v);
  am = __builtin_elementwise_maximum(am, dppf<kQuadSwap1>(am));
  if (t.mode != 0) {  // uniform: s_t NaN, or s_t == 0 (sign-only codes)
    byte = t.mode == 2 ? 0x7Fu : 0u;
    return t.mode == 2 ? 0u : fp4x8_from_f32(v, 0.0f) & 0x88888888u;
  }
  const uint32_t amb = as_u(am) & 0x7FFFFFFFu;
  const bool nanb = amb >= 0x7F800000u;
  const uint32_t k = nv_block_scale_fast(ldexpf(as_f(nanb ? 0u : amb), -t.et), t.st_n);
  uint32_t packed;
  if constexpr (SR) packed = nv_codes8_sr(v, u, t, max(k, 1u));
  else packed = nv_codes8_rne(v, t, max(k, 1u));
  if (k == 0u) packed &= 0x88888888u;  // the block scale underflowed: sign bits only
  byte = nanb ? 0x7Fu : k;
  return nanb ? 0u : packed;
}

}  // namespace mxq
