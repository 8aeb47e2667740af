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

// E2M1 magnitude of a code 0..7 as fp32 (0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  const uint32_t normal = (m << 22) + 0x3F000000u;  // m >= 2: exponent/mantissa fields
  return m >= 2u ? as_f(normal) : (m == 1u ? 0.5f : 0.0f);
}

// ---------------------------------------------------------------------------
// E4M3 ("fn") magnitude code k (0..126) -> fp32 value (gfx950's FP8 conversion
// decodes the OCP E4M3 byte exactly, subnormals included), and nearest-even encoding.
__device__ __forceinline__ float e4m3_value(uint32_t k) { return __builtin_amdgcn_cvt_f32_fp8((int)k, 0); }

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

// Random values of elements n .. n+K-1 in the 16-bit-halves stream (n and K
// multiples of 8): element m takes half (m mod 2), the low half for even m, of word
// (m mod 8) / 2 of Philox4x32-10(counter = (m/8 lo, m/8 hi, 0, 0)), so one call
// serves eight elements. Each value is returned in bits 16..31 of u[i], the bits
// the stochastic rounding reads (bits 0..15 are not used).
template <int K>
__device__ __forceinline__ void philox_halves(uint64_t n, uint64_t seed, uint32_t* u) {
  const uint64_t c0 = n >> 3;
#pragma unroll
  for (int i = 0; i < K / 8; ++i) {
    const uint64_t ctr = c0 + i;
    const u32x4 a = philox4x32_10(u32x4{(uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u}, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
    u[8 * i + 0] = a.x << 16; u[8 * i + 1] = a.x;
    u[8 * i + 2] = a.y << 16; u[8 * i + 3] = a.y;
    u[8 * i + 4] = a.z << 16; u[8 * i + 5] = a.z;
    u[8 * i + 6] = a.w << 16; u[8 * i + 7] = a.w;
  }
}

// The four words serving elements n .. n+7 of the halves stream (n a multiple of
// 8), and their expansion into per-element values as philox_halves returns them.
__device__ __forceinline__ u32x4 philox_halves_words(uint64_t n, uint64_t seed) {
  const uint64_t ctr = n >> 3;
  return philox4x32_10(u32x4{(uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u}, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}
__device__ __forceinline__ void expand_halves(const u32x4& a, uint32_t* u) {
  u[0] = a.x << 16; u[1] = a.x;
  u[2] = a.y << 16; u[3] = a.y;
  u[4] = a.z << 16; u[5] = a.z;
  u[6] = a.w << 16; u[7] = a.w;
}

// The random values of a stochastic-rounding mode: kSrWords (one Philox word per
// element, the top 16 bits used) or kSrHalves (one 16-bit half per element).
enum SrStream : int { kRne = 0, kSrWords = 1, kSrHalves = 2 };

template <int SR, int K>
__device__ __forceinline__ void sr_values(uint64_t n, uint64_t seed, uint32_t* u) {
  if constexpr (SR == kSrWords) philox_words<K>(n, seed, u);
  else if constexpr (SR == kSrHalves) philox_halves<K>(n, seed, u);
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
// Stochastic rounding by gfx950's scaled stochastic FP4 conversion
// (v_cvt_scalef32_sr_pk_fp4_f32), one value per instruction in its first slot (the
// second slot reads overlapping seed bits, so it cannot serve an independent
// element). Characterised on the chip over every E2M1 interval, both signs and
// power-of-two scales: with F the position of y = x / scale inside its E2M1
// interval in units of 2^-22 of the interval, rounded down, the conversion rounds
// |y| up iff F + (seed >> 10) >= 2^22; values of 6 and more give 6; the sign is
// kept. The rule of this library rounds up iff the exact position exceeds 64 r + 32
// units (r the element's 16 random bits). A seed with seed >> 10 = 2^22 - 64 r - c,
// i.e. (~r << 16) | (64 - c) << 10, makes the conversion round up iff F >= 64 r + c.
// u carries r in bits 16..31.
__device__ __forceinline__ uint32_t sr_hw_seed(uint32_t u, uint32_t low) { return (~u & 0xFFFF0000u) | low; }
constexpr uint32_t kSrHwExact = 31u << 10;  // c = 33: F >= 64 r + 33, the rule for integer F

// 8 signed values, each converted stochastically with its own seed under one scale:
// codes packed two per byte, element 2j in the low nibble. Every conversion writes
// byte 0 of its own result (the value's code in bits 0-3, the code of +0 in bits
// 4-7) and only that byte is used: chaining the byte selects through one register
// leaves the other bytes to the register allocator, which does not keep the chain
// in one register. v_perm_b32 then gathers the bytes.
__device__ __forceinline__ uint32_t fp4x8_sr_hw(const float* v, const uint32_t* seed, float scale) {
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2_t{v[i], 0.0f}, seed[i], scale, 0);
  // bytes (r_a.b0, r_b.b0, 0, 0) of two results
  constexpr uint32_t kLow2 = 0x0C0C0400u;
  const uint32_t e = __builtin_amdgcn_perm(r[2], r[0], kLow2) | (__builtin_amdgcn_perm(r[6], r[4], kLow2) << 16);
  const uint32_t o = __builtin_amdgcn_perm(r[3], r[1], kLow2) | (__builtin_amdgcn_perm(r[7], r[5], kLow2) << 16);
  return e | (o << 4);
}

// The smallest random value of 8 elements (r in bits 16..31 of u), as u bits.
__device__ __forceinline__ uint32_t min_u8(const uint32_t* u) {
  return min(min(min(u[0], u[1]), min(u[2], u[3])), min(min(u[4], u[5]), min(u[6], u[7])));
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

// The midpoint decision of one element whose two roundings differ (lo, hi: the
// E2M1 codes with sign, from y (1 - 2^-20) and y (1 + 2^-20)): with m the
// midpoint of their magnitudes, the sign of m s_b s_t - |x| (exact: m s_b has at
// most 7 significant bits) picks lo, hi or, on an exact tie, the even one. xs and
// sts are |x| and s_t, both normalised by 2^-et when s_t is tiny.
__device__ __forceinline__ uint32_t nv_midpoint_pick(uint32_t lo, uint32_t hi, float xs, float sb, float sts) {
  const f32x2_t g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((lo & 7u) | ((hi & 7u) << 4), 1.0f, 0);
  const float m = 0.5f * (g.x + g.y);
  const float d = fmaf(m * sb, sts, -xs);  // > 0: the quotient is below m
  return d > 0.0f ? lo : (d < 0.0f ? hi : ((lo & 1u) ? hi : lo));
}

// Codes of 8 values rounded twice (clo, chi differ where a midpoint lies between):
// the differing nibbles are decided exactly, one per iteration (such elements are
// rare but can be structural, e.g. bf16 data whose exact quotients hit midpoints up
// to the rounding of s_t). |v[j]| is taken times 2^sh, the domain of `sts`.
__device__ __forceinline__ uint32_t nv_resolve8(uint32_t clo, uint32_t chi, const float* v, int sh, float sb,
                                                float sts) {
  uint32_t out = clo;
  uint32_t pending = clo ^ chi;
  while (pending) {
    const uint32_t bit = (uint32_t)__builtin_ctz(pending) & ~3u;  // bit offset of the nibble
    pending &= ~(0xFu << bit);
    float xv = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) xv = bit == 4u * j ? v[j] : xv;
    const float xs = ldexpf(fabsf(xv), sh);
    const uint32_t c = nv_midpoint_pick((clo >> bit) & 0xFu, (chi >> bit) & 0xFu, xs, sb, sts);
    out = (out & ~(0xFu << bit)) | (c << bit);
  }
  return out;
}

// Codes (sign included) of 8 values of an NVFP4 block with scale code k >= 1,
// nearest even. The quotient y = |x| / (s_b s_t) is approximated in fp32 to a few
// ulp and rounded twice by the hardware conversion, at y (1 - 2^-20) and
// y (1 + 2^-20). Equal codes bracket the exact quotient and are the answer; where
// they differ a single rounding midpoint lies between them and nv_resolve8 decides
// exactly. When s_t < 2^-80 the same steps run on values normalised by 2^-et (a
// uniform branch: the common case carries no per-element selection).
__device__ __forceinline__ uint32_t nv_codes8_rne(const float* v, const NvTensor& t, uint32_t k) {
  const float sb = e4m3_value(k);
  const float r = __builtin_amdgcn_rcpf(sb * t.st_n);
  const bool fast = t.et >= -80;
  uint32_t clo, chi;
  if (fast) {
    const float inv = ldexpf(r, -t.et);
    // the two roundings' factors folded into the reciprocal (one product per value
    // and rounding; y (1 -/+ 2^-20) keeps a margin of about 2^-21 over the few-ulp
    // error of the approximate quotient)
    const float invlo = inv * 0.99999905f, invhi = inv * 1.00000095f;
    float ylo[8], yhi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ylo[i] = v[i] * invlo;
      yhi[i] = v[i] * invhi;
    }
    clo = fp4x8_from_f32(ylo, 1.0f);
    chi = fp4x8_from_f32(yhi, 1.0f);
  } else {
    const float invlo = r * 0.99999905f, invhi = r * 1.00000095f;
    float ylo[8], yhi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float vn = ldexpf(v[i], -t.et);
      ylo[i] = vn * invlo;
      yhi[i] = vn * invhi;
    }
    clo = fp4x8_from_f32(ylo, 1.0f);
    chi = fp4x8_from_f32(yhi, 1.0f);
  }
  if (clo == chi) return clo;
  return fast ? nv_resolve8(clo, chi, v, 0, sb, t.st) : nv_resolve8(clo, chi, v, -t.et, sb, t.st_n);
}

// Stochastic rounding of two magnitudes by the carry (e2m1_sr_carry), with the
// window bits of both folded into `low` by one three-way minimum.
template <uint32_t K>
__device__ __forceinline__ void e2m1_sr_carry2(float y0, float y1, uint32_t u0, uint32_t u1, uint32_t& low,
                                               float& q0, float& q1) {
  uint32_t l0 = 0xFFFFFFFFu, l1 = 0xFFFFFFFFu;
  q0 = e2m1_sr_carry<K>(y0, u0, l0);
  q1 = e2m1_sr_carry<K>(y1, u1, l1);
  low = min(low, min(l0, l1));
}

// Codes (sign included) of 8 values of an NVFP4 block with scale code k >= 1,
// stochastic rounding with random values u (r in bits 16..31): the carry decision on
// the approximate quotient, and where an element lies within its window an exact
// decision: with lo and step taken from the approximate quotient,
// |x| > (lo + step (r + 1/2) 2^-16) s_b s_t is exact (one FMA; the coefficient has
// at most 23 significant bits). An approximate lo can only be wrong within a few
// ulp of a grid value, where both candidate decisions return that same grid value,
// so no correction is needed.
__device__ __forceinline__ uint32_t nv_codes8_sr(const float* v, const uint32_t* u, const NvTensor& t,
                                                 uint32_t k) {
  const float sb = e4m3_value(k);
  const float r = __builtin_amdgcn_rcpf(sb * t.st_n);
  float q[8];
  if (t.et >= -80) {
    const float inv = ldexpf(r, -t.et);
    // y carries a relative error below 2^-21 (reciprocal, two products): at most a
    // few units of F, well inside the window K = 16 of the carry decision. (The
    // hardware stochastic conversion would need two conversions per element here, to
    // bracket the threshold, and costs more than the carry.)
    uint32_t low = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float q0, q1;
      e2m1_sr_carry2<16>(fabsf(v[i]) * inv, fabsf(v[i + 1]) * inv, u[i], u[i + 1], low, q0, q1);
      q[i] = with_sign_of(q0, v[i]);
      q[i + 1] = with_sign_of(q1, v[i + 1]);
    }
    if (low < 32u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ax = fabsf(v[i]);
        const float ya = ax * inv;
        float lo, step;
        e2m1_floor_step(ya, lo, step);
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
