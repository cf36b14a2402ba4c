// dev_common.h -- device helpers shared by the ds4moe kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds4moe.h"

namespace ds4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kQ2kBytes = 84;
constexpr int kIq2Bytes = 66;
constexpr int kQ80Bytes = 34;
constexpr int kQ4kBytes = 144;

__host__ __device__ inline int block_bytes(int qt) {
  return qt == DS4MOE_Q2_K ? kQ2kBytes : qt == DS4MOE_IQ2_XXS ? kIq2Bytes : qt == DS4MOE_Q4_K ? kQ4kBytes : kQ80Bytes;
}
__host__ __device__ inline int block_values(int qt) { return qt == DS4MOE_Q8_0 ? 32 : 256; }

// ---- scalar formats --------------------------------------------------------
__device__ inline float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ inline double bf16_bits_to_f64(uint32_t b) { return (double)bf16_bits_to_f32(b); }
__device__ inline double f16_bits_to_f64(uint32_t h) { return (double)f16_bits_to_f32(h); }

// fp32 -> binary16 bits, round to nearest even (hardware conversion).
__device__ inline uint32_t f32_to_f16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

// Round a double to the nearest bfloat16 (ties to even) and return its bits.
// Works on the binary64 encoding so no intermediate binary32 rounding occurs.
__device__ __noinline__ uint32_t f64_to_bf16_bits_general(double v) {
  uint64_t b = __double_as_longlong(v);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & 0xFFFFFFFFFFFFFULL;
  if (e == 0x7FF) return sign | 0x7F80u | (m ? 0x40u : 0u);
  if (e == 0) return sign;  // binary64 subnormals round to zero in bfloat16
  int E = e - 1023;
  uint64_t mant = m | (1ULL << 52);
  int shift = 52 - 7;
  if (E < -126) shift += -126 - E;
  if (E > 127) return sign | 0x7F80u;
  if (shift > 62) return sign;
  uint64_t q = mant >> shift;
  uint64_t rem = mant & ((1ULL << shift) - 1);
  uint64_t half = 1ULL << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  if (E >= -126) {
    int ee = E + 127;
    if (q == 256) { q = 128; ee++; }
    if (ee >= 255) return sign | 0x7F80u;
    return sign | ((uint32_t)ee << 7) | (uint32_t)(q - 128);
  }
  return sign | (uint32_t)q;
}

// Same rounding for results in the normal bfloat16 range (a carry out of
// the mantissa moves into the exponent by itself); ok is false otherwise and
// the result must then come from f64_to_bf16_bits_general.
__device__ inline uint32_t f64_to_bf16_bits_fast(double v, bool& ok) {
  uint64_t b = __double_as_longlong(v);
  uint64_t r = b + 0x00000FFFFFFFFFFFULL + ((b >> 45) & 1);
  int e8 = (int)((r >> 52) & 0x7FF) - 1023 + 127;
  ok = e8 >= 1 && e8 <= 254 && (b & 0x7FFFFFFFFFFFFFFFULL) != 0;
  return (uint32_t)((b >> 48) & 0x8000u) | ((uint32_t)(e8 & 0xFF) << 7) | (uint32_t)((r >> 45) & 0x7Fu);
}

__device__ inline uint32_t f64_to_bf16_bits(double v) {
  bool ok;
  const uint32_t r = f64_to_bf16_bits_fast(v, ok);
  return ok ? r : f64_to_bf16_bits_general(v);
}

// ---- packed dot products ----------------------------------------------------
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ inline float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}
__device__ inline int sdot2(uint32_t a, uint32_t b, int c) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_sdot2(__builtin_bit_cast(s16x2_t, a), __builtin_bit_cast(s16x2_t, b), c,
                                false);
}
__device__ inline uint32_t vperm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// (hi:lo) >> (8*sh) for sh in 0..3 -- extracts an unaligned dword.
__device__ inline uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t sh) {
  return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// ---- wavefront reductions (DPP inside rows of 16, then the four rows) -----
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
// Sum over the 64 lanes of a wave; the result is returned in every lane.
__device__ inline float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}

template <int CTRL>
__device__ inline double dpp_f64(double v) {
  uint64_t u = __double_as_longlong(v);
  int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ inline double readlane_f64(double v, int lane) {
  uint64_t u = __double_as_longlong(v);
  uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
// Sum of 64 lanes in a fixed tree of depth 6; result in every lane.
__device__ inline double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ---- largest magnitude with a non-finite check --------------------------------
// A lane's largest |v| over many values, and whether any of them is NaN or
// infinite, from their bit patterns alone: the signed maximum of the
// patterns is the largest positive value (with NaN and +Inf above every
// finite one), the unsigned maximum the negative value of largest magnitude
// (NaN and -Inf above every finite one); each stands for the other sign's
// extreme when no value of its own sign is present.  Two max3 operations per
// three values.
struct AbsMax {
  int smax = (int)0x80000000;  // -0.0
  uint32_t umax = 0u;          // +0.0
  __device__ inline void add(float v) {
    const uint32_t b = __float_as_uint(v);
    smax = max(smax, (int)b);
    umax = max(umax, b);
  }
  // max |v|; `bad` is set when some value was NaN or infinite
  __device__ inline float value(bool& bad) const {
    const uint32_t sp = (uint32_t)smax & 0x7FFFFFFFu, up = umax & 0x7FFFFFFFu;
    bad = sp >= 0x7F800000u || up >= 0x7F800000u;
    return fmaxf(__uint_as_float(sp), __uint_as_float(up));
  }
};

// A wave-uniform int32 read through the scalar cache (the data must not be
// written while the kernel runs).
__device__ inline int load_scalar_i32(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// ---- device fault word -------------------------------------------------------
__device__ inline void raise_fault(uint32_t* status, uint32_t bit) { atomicOr(status, bit); }

__device__ inline float silu(float v) { return v / (1.0f + __expf(-v)); }

}  // namespace ds4
