// Device-side building blocks shared by the gfx950 kernels: bit views, wave-level
// reductions, E2M1/E4M3 rounding, Philox4x32-10 and 32-bit division by invariants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// Streaming loads: data is read exactly once, so it is marked non-temporal.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 load_nt(const float4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Nontemporal vector stores, for outputs whose every store instruction writes whole
// contiguous lines (measured faster on data that does not fit the caches). Pieces
// of a line written by different instructions or workgroups, and single scale
// bytes, stay plain stores so that the L2 can merge them.
__device__ __forceinline__ void store_nt(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(uint8_t* p, uint8_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
  __builtin_nontemporal_store(nt_u32x2{v.x, v.y}, reinterpret_cast<nt_u32x2*>(p));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}
__device__ __forceinline__ void store_nt(float4* p, float4 v) {
  store_nt(reinterpret_cast<uint4*>(p), make_uint4(__float_as_uint(v.x), __float_as_uint(v.y),
                                                    __float_as_uint(v.z), __float_as_uint(v.w)));
}

// DPP quad permutations (64-wide waves are split into quads of 4 lanes).
constexpr int kQuadSwap1 = 0xB1;  // [1,0,3,2]: exchange with the neighbouring lane
constexpr int kQuadSwap2 = 0x4E;  // [2,3,0,1]: exchange with the lane two away

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
}
template <int Ctrl>
__device__ __forceinline__ float dppf(float v) {
  return as_f(dpp<Ctrl>(as_u(v)));
}

// ---------------------------------------------------------------------------
// gfx950 scaled FP4 conversions. With the scale operand holding an E8M0 byte b in
// its exponent field (as_f(b << 23); b = 0 stands for 2^-127), the down-conversion
// returns sign | nearest-even E2M1 of |x| / 2^(b-127), saturating at 6, and the
// up-conversion returns v(code) * 2^(b-127) rounded to the output type. Checked
// against the oracle for every bf16 input and every b in 0..254; non-finite
// inputs are never passed (NaN blocks are overwritten by the callers).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));  // two E4M3 pairs per dword

__device__ __forceinline__ float e8m0_operand(uint32_t byte) { return as_f(byte << 23); }

// Four bf16 pairs (dwords) -> 8 codes in one dword, element 2j in the low nibble.
__device__ __forceinline__ uint32_t fp4x8_from_bf16(const uint32_t w[4], float scale) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, w[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[3]), scale, 3);
  return r;
}

// Eight fp32 values -> 8 codes in one dword.
__device__ __forceinline__ uint32_t fp4x8_from_f32(const float* v, float scale) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], scale, 3);
  return r;
}

// ---------------------------------------------------------------------------
// E2M1 rounding of a non-negative fp32 magnitude y (exact input, any size).
// Codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
//
// Nearest, ties to even, saturating at 6:
//  * y >= 1: the E2M1 normal range keeps one mantissa bit, so the fp32 mantissa
//    is rounded at bit 22 (add 0x1FFFFF plus the kept bit, then truncate); the
//    biased exponent/mantissa pair (t >> 22) is then 254 + code - 2, and anything
//    past 6.0 (8.0 and up, Inf) clamps to code 7;
//  * y < 1: E2M1 steps by 0.5 there, which is the fp32 ulp in [2^22, 2^23), so
//    y + 2^22 is rounded to a multiple of 0.5 by the FPU itself (round to nearest
//    even), and the distance from 2^22 in ulps is the code (0, 1 or 2).
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const uint32_t b = as_u(y);
  const uint32_t t = b + 0x1FFFFFu + ((b >> 22) & 1u);
  const uint32_t hi = min(t >> 22, 259u) - 252u;
  const uint32_t lo = as_u(y + 4194304.0f) - 0x4A800000u;
  return b >= 0x3F800000u ? hi : lo;
}

// Largest E2M1 magnitude code whose value is <= y (round toward zero; y >= 0).
__device__ __forceinline__ uint32_t e2m1_floor(float y) {
  const uint32_t b = as_u(y);
  const uint32_t hi = min(b >> 22, 259u) - 252u;
  const uint32_t lo = y >= 0.5f ? 1u : 0u;
  return b >= 0x3F800000u ? hi : lo;
}

// E2M1 magnitude of a code 0..7 as fp32 (0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  const uint32_t normal = (m << 22) + 0x3F000000u;  // m >= 2: exponent/mantissa fields
  return m >= 2u ? as_f(normal) : (m == 1u ? 0.5f : 0.0f);
}

// ---------------------------------------------------------------------------
// E4M3 ("fn") magnitude code k (0..126) -> fp32 value, and nearest-even encoding.
__device__ __forceinline__ float e4m3_value(uint32_t k) {
  const uint32_t e = k >> 3, m = k & 7u;
  return e ? as_f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;  // m * 2^-9
}

// E4M3 magnitude code of RNE(v) for a finite v >= 0 (exact input), saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = as_u(v);
  if (b >= 0x3C800000u) {  // v >= 2^-6: normal range, keep 3 mantissa bits
    const uint32_t t = b + 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t k = (t >> 20) - (120u << 3);  // (exp - 120) << 3 | mantissa
    return min(k, 126u);
  }
  // subnormal range: multiples of 2^-9; 2^14 has an fp32 ulp of 2^-9
  return as_u(v + 16384.0f) - 0x46800000u;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): multipliers 0xD2511F53 / 0xCD9E8D57,
// Weyl key increments 0x9E3779B9 / 0xBB67AE85, ten rounds.
struct u32x4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ c in one VALU instruction (v_bitop3_b32, truth table 0x96 = odd parity)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;  // v_mad_u64_u32
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = u32x4{xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1, xor3((uint32_t)(p0 >> 32), c.w, k1),
              (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Random words of elements n .. n+3 for n a multiple of 4 (one Philox call).
__device__ __forceinline__ u32x4 philox_words4(uint64_t n, uint64_t seed) {
  const uint64_t ctr = n >> 2;
  return philox4x32_10(u32x4{(uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u}, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// Random words of elements n .. n+K-1 for any n (K a multiple of 4): K/4 Philox
// calls when n is a multiple of 4, one more otherwise. n mod 4 is the same for
// every lane of a launch, so the shift below is a uniform branch.
template <int K>
__device__ __forceinline__ void philox_words(uint64_t n, uint64_t seed, uint32_t* u) {
  const uint32_t s = (uint32_t)(n & 3u);
  const uint64_t b = n - s;
  uint32_t w[K + 4];
#pragma unroll
  for (int i = 0; i < K; i += 4) {
    const u32x4 a = philox_words4(b + i, seed);
    w[i] = a.x; w[i + 1] = a.y; w[i + 2] = a.z; w[i + 3] = a.w;
  }
  if (s == 0) {
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = w[i];
    return;
  }
  const u32x4 a = philox_words4(b + K, seed);
  w[K] = a.x; w[K + 1] = a.y; w[K + 2] = a.z; w[K + 3] = a.w;
  if (s == 1) {
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = w[i + 1];
  } else if (s == 2) {
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = w[i + 2];
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) u[i] = w[i + 3];
  }
}

// Word of one element n (any n).
__device__ __forceinline__ uint32_t philox_word(uint64_t n, uint64_t seed) {
  const u32x4 w = philox_words4(n & ~3ull, seed);
  const uint32_t s = (uint32_t)(n & 3u);
  return s == 0 ? w.x : (s == 1 ? w.y : (s == 2 ? w.z : w.w));
}

// The E2M1 grid value at or below y >= 0 (as fp32) and the gap to the next one,
// from the bits of y: for y >= 1 the grid keeps one mantissa bit, on [0.5, 1) it
// is 0.5, below 0.5 it is 0. The gap is 2^(max(e, 0) - 1) for y in [2^e, 2^(e+1)).
__device__ __forceinline__ void e2m1_floor_step(float y, float& lo, float& step) {
  const uint32_t b = as_u(y);
  const uint32_t e = b >> 23;  // biased exponent (y >= 0)
  const uint32_t mask = e >= 127u ? 0xFFC00000u : (e == 126u ? 0xFF800000u : 0u);
  lo = as_f(b & mask);
  step = as_f((max(e, 127u) - 1u) << 23);
}

// (r + 1/2) / 2^16 with r the top 16 bits of the random word u (17 significant bits).
__device__ __forceinline__ float sr_offset16(uint32_t u) {
  return (float)((u >> 15) | 1u) * (1.0f / 131072.0f);
}

// 1 + (r + 1/2) / 2^16, built from bits: mantissa = r << 7 | 1 << 6.
__device__ __forceinline__ float sr_offset16_plus1(uint32_t u) {
  return as_f(((u >> 9) & 0x007FFF80u) | 0x3F800040u);
}

// |q| with the sign bit of s (one bitfield insert).
__device__ __forceinline__ float with_sign_of(float q, float s) {
  return __builtin_copysignf(q, s);
}

// Stochastic E2M1 rounding of an exact fp32 magnitude y with random word u:
// up iff y > lo + step * (r + 1/2) / 2^16, r = u >> 16; y >= 6 gives 6.
// lo + step * (r + 1/2) / 2^16 has at most 20 significant bits: exact in fp32.
// Returns the rounded grid value (<= 6) as fp32; the caller converts it (exactly).
__device__ __forceinline__ float e2m1_sr_value(float y, uint32_t u) {
  float lo, step;
  e2m1_floor_step(y, lo, step);
  // lo + step (r + 1/2) 2^-16, exact (at most 20 significant bits)
  const float thr = fmaf(step, sr_offset16_plus1(u), lo - step);
  return fminf(y > thr ? lo + step : lo, 6.0f);
}

__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) { return e2m1_rne(e2m1_sr_value(y, u)); }

// The same stochastic rounding decided by a carry. Adding 1 to y < 1 moves the grid
// 0, 0.5, 1 onto 1, 1.5, 2, so every grid interval is one fp32 mantissa bit wide.
// F, the 22 bits under that bit, is the position inside the interval in units of
// 2^-22 of the gap, and T = 64 r + 32 is the threshold (r + 1/2) / 2^16 in the same
// units. Adding 2^22 - 1 - T + K to the bits carries into the kept bit iff
// F >= T + 1 - K. For F in [T + 1 - K, T + 1 + K) the low 22 bits of the sum are
// below 2K: there an error of F below K units (y inexact, or the rounding of y + 1)
// could flip the decision, so the caller keeps the running minimum `low` of those
// bits and decides the elements exactly when it ends below 2K. Result: the grid
// value; 8 stands for 6 (values of [6, 8) that round up), which the callers' scaled
// E2M1 conversion saturates to 6.
template <uint32_t K>
__device__ __forceinline__ float e2m1_sr_carry(float y, uint32_t u, uint32_t& low) {
  const float off = y < 1.0f ? 1.0f : 0.0f;
  // bits(y + off) - 64 r + 2^22 - 64 + 31 + K, r = u >> 16. The bits of y + off >= 1
  // exceed 64 r < 2^22, so this is |bits - 64 r| + const: one v_sad_u32 (LLVM has no
  // builtin for it).
  // 64 r: the high half of u shifted left by 6, one SDWA shift (written out, as the
  // compiler would otherwise share a bit-field extract with the exact fallback)
  uint32_t r64, s;
  asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=v"(r64) : "v"(6u), "v"(u));
  asm("v_sad_u32 %0, %1, %2, %3" : "=v"(s) : "v"(as_u(y + off)), "v"(r64), "v"(0x3FFFC0u + 31u + K));
  low = min(low, s & 0x3FFFFFu);
  return as_f(s & 0xFFC00000u) - off;
}

// ---------------------------------------------------------------------------
// Unsigned division of i < 2^30 by an invariant d >= 1: q = (i * m) >> s with
// l = ceil(log2 d), s = 30 + l, m = ceil(2^s / d) < 2^31 + 1.
struct FastDiv {
  uint32_t d, m, s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t i, FastDiv f) {
  return (uint32_t)(((uint64_t)i * f.m) >> f.s);
}

}  // namespace mxq

namespace mxq {

// ---------------------------------------------------------------------------
// NVFP4 two-level scaling with exact-real rounding decisions.
//
// The tensor scale s_t = RN_fp32(A / 2688) (IEEE division). All decisions
// compare an exact quotient with a threshold of few significant bits; they are
// taken on values normalised by 2^-et (et = floor(log2 s_t)) so that
// s_t_n = s_t * 2^-et lies in [1, 2) and nothing underflows. A comparison
// "a >= c * s_t_n" with c exact in fp32 is decided by the sign of
// fma(c, s_t_n, -a), which is exact.
struct NvTensor {
  int mode;     // 0 finite nonzero s_t, 1 s_t == 0, 2 s_t NaN
  float st;     // s_t as stored
  float st_n;   // s_t * 2^-et, in [1, 2)
  int et;
};

// With the Hadamard transform the kernels quantise z = H16 (s * x), four times the
// transformed values y = z / 4 whose amax sets s_t: quantising z against 4 s_t
// (exact) gives the same block scales and codes as y against s_t.
__device__ __forceinline__ void nv_tensor_times4(NvTensor& t) {
  if (t.mode == 0) {
    t.st *= 4.0f;
    t.et += 2;
  }
}

__device__ __forceinline__ NvTensor nv_tensor(float amax) {
  NvTensor t;
  const float a = fabsf(amax);
  t.st = a / 2688.0f;
  t.et = 0;
  t.st_n = 1.0f;
  if (!(a <= 3.40282347e38f)) {  // NaN or Inf
    t.mode = 2;
    t.st = __uint_as_float(0x7FC00000u);
    return t;
  }
  if (t.st == 0.0f) {
    t.mode = 1;
    return t;
  }
  t.mode = 0;
  int e;
  const float m = frexpf(t.st, &e);  // st = m * 2^e, m in [0.5, 1)
  t.st_n = m * 2.0f;
  t.et = e - 1;
  return t;
}

// The same from a tensor scale already computed by nv_tensor (and stored): NaN
// gives mode 2, zero mode 1, anything else the normalised form.
__device__ __forceinline__ NvTensor nv_tensor_from_st(float st) {
  NvTensor t;
  t.st = st;
  t.et = 0;
  t.st_n = 1.0f;
  if (st != st) {
    t.mode = 2;
    t.st = __uint_as_float(0x7FC00000u);
    return t;
  }
  if (st == 0.0f) {
    t.mode = 1;
    return t;
  }
  t.mode = 0;
  int e;
  const float m = frexpf(st, &e);
  t.st_n = m * 2.0f;
  t.et = e - 1;
  return t;
}

// The tensor scale of a kernel's launch: `src` holds the amax, or (st_given) the
// tensor scale itself.
__device__ __forceinline__ NvTensor nv_tensor_load(const float* src, bool st_given) {
  return st_given ? nv_tensor_from_st(*src) : nv_tensor(*src);
}

// Exact E4M3 (nearest even, saturating) code of a_n / (6 st_n); a_n >= 0 exact.
__device__ __forceinline__ uint32_t nv_block_scale(float a_n, float st_n) {
  const float q = a_n * __builtin_amdgcn_rcpf(6.0f * st_n);
  uint32_t k = e4m3_rne(q);
  bool moved = false;
  if (k < 126u) {
    const float mu6 = 3.0f * (e4m3_value(k) + e4m3_value(k + 1u));  // 6 * midpoint, exact
    const float r = fmaf(mu6, st_n, -a_n);
    if (r < 0.0f || (r == 0.0f && ((k + 1u) & 1u) == 0u)) {
      k += 1u;
      moved = true;
    }
  }
  if (!moved && k > 0u) {
    const float mu6 = 3.0f * (e4m3_value(k - 1u) + e4m3_value(k));
    const float r = fmaf(mu6, st_n, -a_n);
    if (r > 0.0f || (r == 0.0f && ((k - 1u) & 1u) == 0u)) k -= 1u;
  }
  return k;
}

// y_a is within a few ulps of a value with at most 3 significant bits (every
// E2M1 grid value and rounding midpoint is one), at or above 0.2.
__device__ __forceinline__ bool near_3bit(float y_a) {
  const uint32_t b = as_u(y_a);
  return b >= 0x3E4CCCCDu && ((b + 64u) & 0x1FFFFFu) <= 128u;
}

// Exact nearest-even E2M1 code of x_n / (sb * st_n) by threshold tests.
__device__ __forceinline__ uint32_t nv_code_exact(float x_n, float sb, float st_n) {
  uint32_t c = 0;
  c += fmaf(0.25f * sb, st_n, -x_n) < 0.0f;
  c += fmaf(0.75f * sb, st_n, -x_n) <= 0.0f;
  c += fmaf(1.25f * sb, st_n, -x_n) < 0.0f;
  c += fmaf(1.75f * sb, st_n, -x_n) <= 0.0f;
  c += fmaf(2.5f * sb, st_n, -x_n) < 0.0f;
  c += fmaf(3.5f * sb, st_n, -x_n) <= 0.0f;
  c += fmaf(5.0f * sb, st_n, -x_n) < 0.0f;
  return c;
}

// Exact largest code whose value is <= x_n / (sb * st_n).
__device__ __forceinline__ uint32_t nv_floor_exact(float x_n, float sb, float st_n) {
  uint32_t c = 0;
#pragma unroll
  for (uint32_t m = 1; m < 8; ++m) c += fmaf(e2m1_value(m) * sb, st_n, -x_n) <= 0.0f;
  return c;
}

// NVFP4 element code (magnitude) with round-to-nearest-even.
__device__ __forceinline__ uint32_t nv_code_rne(float x_n, float sb, float inv, float st_n) {
  const float y = x_n * inv;
  const uint32_t c = e2m1_rne(y);
  return near_3bit(y) ? nv_code_exact(x_n, sb, st_n) : c;
}

// NVFP4 element code (magnitude) with stochastic rounding (word u).
__device__ __forceinline__ uint32_t nv_code_sr(float x_n, float sb, float inv, float st_n,
                                               uint32_t u) {
  const float y = x_n * inv;
  uint32_t lo = e2m1_floor(y);
  if (near_3bit(y)) lo = nv_floor_exact(x_n, sb, st_n);
  if (lo >= 7u) return 7u;
  const float vlo = e2m1_value(lo);
  const float step = e2m1_value(lo + 1u) - vlo;
  const float thr = vlo + step * ((float)(u >> 16) + 0.5f) * (1.0f / 65536.0f);
  return fmaf(thr * sb, st_n, -x_n) < 0.0f ? lo + 1u : lo;
}

// Codes (sign included) of 8 values of an NVFP4 block with scale code k >= 1,
// nearest even. The quotient y = |x| / (s_b s_t) is approximated in fp32 to a few
// ulp and rounded twice by the hardware conversion, at y (1 - 2^-20) and
// y (1 + 2^-20). Equal codes bracket the exact quotient and are the answer; where
// they differ a single rounding midpoint m lies between them, and the sign of
// fma(m s_b, s_t, -|x|) (exact) picks the lower code, the upper one, or on an
// exact tie the even one. When s_t < 2^-80 the same tests run on values
// normalised by 2^-et.
__device__ __forceinline__ uint32_t nv_codes8_rne(const float* v, const NvTensor& t, uint32_t k) {
  const float sb = e4m3_value(k);
  const float r = __builtin_amdgcn_rcpf(sb * t.st_n);
  const bool fast = t.et >= -80;
  const float inv = fast ? ldexpf(r, -t.et) : r;
  const float sts = fast ? t.st : t.st_n;
  // the two roundings' factors folded into the reciprocal (one product per value
  // and rounding; y (1 -/+ 2^-20) keeps a margin of about 2^-21 over the few-ulp
  // error of the approximate quotient)
  const float invlo = inv * 0.99999905f, invhi = inv * 1.00000095f;
  float ylo[8], yhi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xs = fast ? v[i] : ldexpf(v[i], -t.et);
    ylo[i] = xs * invlo;
    yhi[i] = xs * invhi;
  }
  const uint32_t clo = fp4x8_from_f32(ylo, 1.0f);
  const uint32_t chi = fp4x8_from_f32(yhi, 1.0f);
  const uint32_t diff = clo ^ chi;
  if (diff == 0u) return clo;
  // Some element lies within 2^-20 of a midpoint: decide exactly the ones that do,
  // one per iteration (usually one; such elements are rare but can be structural,
  // e.g. bf16 data whose exact quotients hit midpoints up to the rounding of s_t).
  uint32_t out = clo;
  uint32_t pending = diff;
  while (pending) {
    const uint32_t sh = (uint32_t)__builtin_ctz(pending) & ~3u;  // bit offset of the nibble
    pending &= ~(0xFu << sh);
    const uint32_t lo = (clo >> sh) & 0xFu, hi = (chi >> sh) & 0xFu;
    float xv = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) xv = sh == 4u * j ? v[j] : xv;
    // the two neighbouring grid values, decoded together: m is their midpoint
    const f32x2_t g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((lo & 7u) | ((hi & 7u) << 4), 1.0f, 0);
    const float m = 0.5f * (g.x + g.y);
    const float xs = fast ? fabsf(xv) : ldexpf(fabsf(xv), -t.et);
    const float d = fmaf(m * sb, sts, -xs);  // > 0: the quotient is below m
    const uint32_t c = d > 0.0f ? lo : (d < 0.0f ? hi : ((lo & 1u) ? hi : lo));
    out = (out & ~(0xFu << sh)) | (c << sh);
  }
  return out;
}

// Codes (sign included) of 8 values of an NVFP4 block with scale code k >= 1,
// stochastic rounding with words u. With lo and step taken from an approximate
// quotient, the decision |x| > (lo + step (r + 1/2) 2^-16) s_b s_t is exact (one
// FMA; the coefficient has at most 23 significant bits). An approximate lo can
// only be wrong within a few ulp of a grid value, where both candidate decisions
// return that same grid value, so no correction is needed.
__device__ __forceinline__ uint32_t nv_codes8_sr(const float* v, const uint32_t* u, const NvTensor& t,
                                                 uint32_t k) {
  const float sb = e4m3_value(k);
  const float r = __builtin_amdgcn_rcpf(sb * t.st_n);
  float q[8];
  if (t.et >= -80) {
    const float inv = ldexpf(r, -t.et);
    // y carries a relative error below 2^-21 (reciprocal, two products): at most a
    // few units of F, well inside the window K = 16 of the carry decision
    uint32_t low = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = with_sign_of(e2m1_sr_carry<16>(fabsf(v[i]) * inv, u[i], low), v[i]);
    if (low < 32u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ax = fabsf(v[i]);
        const float y = ax * inv;
        float lo, step;
        e2m1_floor_step(y, lo, step);
        // threshold (lo + step (r + 1/2) 2^-16) s_b, exact (at most 23 significant
        // bits); the sign of c s_t - |x| decides
        const float c = fmaf(step, sr_offset16_plus1(u[i]), lo - step) * sb;
        const bool up = fmaf(c, t.st, -ax) < 0.0f;
        q[i] = with_sign_of(fminf(up ? lo + step : lo, 6.0f), v[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xs = ldexpf(fabsf(v[i]), -t.et);
      const float y = xs * r;
      float lo, step;
      e2m1_floor_step(y, lo, step);
      const float c = fmaf(step * sb, sr_offset16(u[i]), lo * sb);
      const bool up = fmaf(c, t.st_n, -xs) < 0.0f;
      q[i] = as_f(as_u(fminf(up ? lo + step : lo, 6.0f)) | (as_u(v[i]) & 0x80000000u));
    }
  }
  return fp4x8_from_f32(q, 1.0f);  // grid values: the conversion is exact
}

// E4M3 code of the block scale, nearest even of the exact quotient a_n / (6 st_n):
// the approximate quotient is converted twice, at q (1 -+ 2^-20); equal codes are
// the answer, else the exact test against the midpoint between them decides.
__device__ __forceinline__ uint32_t nv_block_scale_fast(float a_n, float st_n) {
  const float q = a_n * __builtin_amdgcn_rcpf(6.0f * st_n);
  const float qlo = fminf(q * 0.99999905f, 448.0f), qhi = fminf(q * 1.00000095f, 448.0f);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qlo, qhi, 0, false);
  const uint32_t klo = w & 0x7Fu, khi = (w >> 8) & 0x7Fu;
  if (klo == khi) return klo;
  const float mu6 = 3.0f * (e4m3_value(klo) + e4m3_value(khi));  // 6 * midpoint, exact
  const float d = fmaf(mu6, st_n, -a_n);
  return d > 0.0f ? klo : (d < 0.0f ? khi : ((klo & 1u) ? khi : klo));
}

}  // namespace mxq
