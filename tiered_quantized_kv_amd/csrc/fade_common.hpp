// Device helpers shared by the libfade kernels (gfx950, wave64).
//
// Storage types are raw 16-bit patterns; arithmetic uses _Float16 / float /
// double. Every conversion to a 16-bit type rounds to nearest-even exactly
// once (float64 values go through a round-to-odd float32, which makes the
// second rounding exact because float32 carries more than 11 + 2 bits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fade {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 32;          // quantization group along head_dim
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (f16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float64 -> float32 rounding to odd: truncate toward zero, then set the last
// bit if anything was discarded.
__device__ __forceinline__ float d2f_odd(double d) {
  const float f = (float)d;
  const double back = (double)f;
  uint32_t u = __float_as_uint(f);
  u -= (uint32_t)(fabs(back) > fabs(d));   // rounded away from zero: step back
  u |= (uint32_t)(back != d);
  return __uint_as_float(u);
}
// The same for a float64 headed for fp16, on the bit pattern: clear the 29
// mantissa bits that float32 lacks (the conversion is then exact) and set the
// last bit if any of them was set. Magnitudes below float32's normal range
// land far below fp16's smallest subnormal and still round to a signed zero.
__device__ __forceinline__ float d2f_odd_h(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint32_t st = min((uint32_t)u & 0x1FFFFFFFu, 1u);   // 1 if any cleared bit was set
  const float f = (float)__longlong_as_double((long long)(u & ~(uint64_t)0x1FFFFFFFu));
  return __uint_as_float(__float_as_uint(f) | st);
}
__device__ __forceinline__ uint16_t d2h(double d) { return f2h(d2f_odd_h(d)); }
__device__ __forceinline__ uint16_t d2bf(double d) { return f2bf(d2f_odd(d)); }

// ---- wave reductions -------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128, kRowRor1 = 0x121;

// Full-wave reductions without LDS: DPP inside each 16-lane row, then
// row_bcast:15 / row_bcast:31 to fold the rows into lane 63, read back as a
// wave-uniform value.
__device__ __forceinline__ float wave_sum_u(float x) {
  x += dpp_f<kRowRor1>(x);
  x += dpp_f<kRowRor2>(x);
  x += dpp_f<kRowRor4>(x);
  x += dpp_f<kRowRor8>(x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_max_u(float x) {
  const int ninf = __builtin_bit_cast(int, -INFINITY);
  x = fmaxf(x, dpp_f<kRowRor1>(x));
  x = fmaxf(x, dpp_f<kRowRor2>(x));
  x = fmaxf(x, dpp_f<kRowRor4>(x));
  x = fmaxf(x, dpp_f<kRowRor8>(x));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// (x & mask) | bits; with mask and bits held in VGPRs this is one
// v_and_or_b32 (VOP3 on gfx9 takes no 32-bit literal and one scalar operand at
// most). Plain C, not inline asm: the hazard recognizer does not count an
// inline-asm definition as a VALU write, so an asm result placed in a
// register that an in-flight MFMA still writes (a dead accumulator row) was
// overwritten by that MFMA.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) { return (x & mask) | bits; }

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kRowRor1>(x);
  x += dpp_f<kRowRor2>(x);
  x += dpp_f<kRowRor4>(x);
  x += dpp_f<kRowRor8>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kRowRor1>(x));
  x = fmaxf(x, dpp_f<kRowRor2>(x));
  x = fmaxf(x, dpp_f<kRowRor4>(x));
  x = fmaxf(x, dpp_f<kRowRor8>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Sum over the lanes of a 16-lane row that share (lane % STRIDE); the result
// is in every such lane. STRIDE in {1, 2, 4, 8}.
template <int STRIDE>
__device__ __forceinline__ float row_sum_strided(float x) {
  if constexpr (STRIDE <= 1) x += dpp_f<kRowRor1>(x);
  if constexpr (STRIDE <= 2) x += dpp_f<kRowRor2>(x);
  if constexpr (STRIDE <= 4) x += dpp_f<kRowRor4>(x);
  if constexpr (STRIDE <= 8) x += dpp_f<kRowRor8>(x);
  return x;
}

// ---- symmetric group quantizer ---------------------------------------------
// s = fp16_RNE(amax / qmax), q = clamp(RNE(x / s), -qmax, qmax), s == 0 -> q = 0,
// stored as the field q + 2^(BITS-1); evaluated without a division:
//  * scale: for qmax = 7, amax * float32(1/7) rounded once to fp16 equals the
//    RNE of the exact quotient for every finite fp16 amax; for qmax = 1, s = amax.
//  * field: with r = rcp(s) (r = 0 when s == 0, which yields q = 0),
//    a = fma(x, r, 192) rounds x * r to the 2^-16 grid. x * r lies within
//    2^-21 of x / s, and a quotient of fp16 values is either a half-integer
//    or at least 2^-13 away from every half-integer, with |x / s| <= 10 (the
//    bound is reached only for subnormal scales); so a equals the quotient at
//    a tie and lies on the quotient's side of every half-integer otherwise.
//    Adding 1.5 * 2^23 + 2^(BITS-1) - 192 rounds that to an integer with
//    ties to even, leaving the field in the low mantissa bits; fmed3 clamps.
// All of it was checked exhaustively over fp16 operands against exact
// rational rounding, with the reciprocal off by one ulp either way.
constexpr float kFieldBase = 12582912.f;            // 1.5 * 2^23
constexpr uint32_t kFieldBaseBits = 0x4B400000u;    // its bit pattern

template <int BITS>
__device__ __forceinline__ uint16_t group_scale_bits(float amax) {
  if constexpr (BITS == 2) return f2h(amax);
  else return f2h(amax * (1.0f / 7.0f));
}
__device__ __forceinline__ float quant_recip(float s) { return s != 0.f ? __builtin_amdgcn_rcpf(s) : 0.f; }

// kFieldBaseBits + field of one value.
template <int BITS>
__device__ __forceinline__ uint32_t quant_field(float x, float r) {
  constexpr float kOff = (float)(1 << (BITS - 1));
  constexpr float kQmax = kOff - 1.f;
  const float a = __builtin_fmaf(x, r, 192.f);
  const float b = a + (kFieldBase + kOff - 192.f);
  return __float_as_uint(__builtin_amdgcn_fmed3f(b, kFieldBase + kOff - kQmax, kFieldBase + kOff + kQmax));
}
// Sum over k < N of kFieldBaseBits << (BITS * k), modulo 2^32: subtracting
// it from the sum of quant_field(x_k) << (BITS * k) leaves the packed fields.
template <int BITS, int N>
__device__ __forceinline__ constexpr uint32_t field_bias() {
  uint32_t c = 0u;
  for (int k = 0; k < N; ++k) c += kFieldBaseBits << (BITS * k);
  return c;
}

// 32 values of one group (exact float copies of fp16 values) -> packed codes
// (BITS 32-bit words, little-endian: channel c at bit (c*BITS) of the group's
// byte stream) and the fp16 scale.
template <int BITS>
__device__ __forceinline__ void quant_group32(const float* x, uint32_t* packed, uint16_t& scale) {
  constexpr int kPerWord = 32 / BITS;
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(x[c]));
  const uint16_t sb = group_scale_bits<BITS>(amax);
  const float r = quant_recip(h2f(sb));
#pragma unroll
  for (int w = 0; w < BITS; ++w) packed[w] = 0u - field_bias<BITS, kPerWord>();
#pragma unroll
  for (int c = 0; c < 32; ++c) packed[c / kPerWord] += quant_field<BITS>(x[c], r) << ((c % kPerWord) * BITS);
  scale = sb;
}

// Offset-removed code of channel c (0..31) of a packed group, as float.
// 32 fp16 values (64 bytes, 16-byte aligned) as floats
__device__ __forceinline__ void load_group32_f16(const uint16_t* p, float* x) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = v[i];
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = h2f((uint16_t)(words[j] & 0xFFFFu));
      x[8 * i + 2 * j + 1] = h2f((uint16_t)(words[j] >> 16));
    }
  }
}

// A group's packed code words (quant_group32's order) to their row bytes
template <int BITS>
__device__ __forceinline__ void store_group_codes(uint8_t* dst, const uint32_t* packed) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  }
}

template <int BITS>
__device__ __forceinline__ float code_at(const uint32_t* packed, int c) {
  constexpr int kPerWord = 32 / BITS;
  const uint32_t u = (packed[c / kPerWord] >> ((c % kPerWord) * BITS)) & ((1u << BITS) - 1u);
  return (float)((int)u - (1 << (BITS - 1)));
}

}  // namespace fade
