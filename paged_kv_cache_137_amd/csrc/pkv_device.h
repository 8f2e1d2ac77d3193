// Device-side helpers shared by the gfx950 kernels of libpkv: element types,
// conversions, packed dot products and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Storage tags.  bf16 travels as raw 16-bit patterns.
struct f32_t { using storage = float; static constexpr int bytes = 4; };
struct f16_t { using storage = _Float16; static constexpr int bytes = 2; };
struct bf16_t { using storage = uint16_t; static constexpr int bytes = 2; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// float -> f16 bits, round to nearest even, from the float32 value as given.
// The empty asm makes the float32 value opaque.  Without it the compiler may
// fold a preceding multiply into a mixed-precision convert (one rounding of the
// exact product), and a 16-bit output would then not always equal the rounding
// of the float32 output.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  asm volatile("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Unpack a 16-byte chunk into floats.
template <typename E> struct Chunk;
template <> struct Chunk<f32_t> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void unpack(const uint4& c, float* o) {
    o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
    o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
  }
  // sum_i q_i * k_i over the chunk, fp32 accumulate
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k) {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    return s;
  }
};
template <> struct Chunk<bf16_t> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void unpack(const uint4& c, float* o) {
    o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x); o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
    o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z); o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
  }
  // Products of two bf16 are exact in fp32; v_dot2 adds them into an fp32 sum.
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), s, false);
    return s;
  }
};
template <> struct Chunk<f16_t> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void unpack(const uint4& c, float* o) {
    o[0] = f16_lo(c.x); o[1] = f16_hi(c.x); o[2] = f16_lo(c.y); o[3] = f16_hi(c.y);
    o[4] = f16_lo(c.z); o[5] = f16_hi(c.z); o[6] = f16_lo(c.w); o[7] = f16_hi(c.w);
  }
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k) {
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.x), __builtin_bit_cast(f16x2_t, k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.y), __builtin_bit_cast(f16x2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.z), __builtin_bit_cast(f16x2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.w), __builtin_bit_cast(f16x2_t, k.w), s, false);
    return s;
  }
};

// Output stores: float, or the input type rounded to nearest even.
template <typename O> struct Out;
template <> struct Out<f32_t> {
  using storage = float;
  __device__ __forceinline__ static void put(void* p, int64_t i, float x) { ((float*)p)[i] = x; }
};
template <> struct Out<f16_t> {
  using storage = uint16_t;
  __device__ __forceinline__ static void put(void* p, int64_t i, float x) { ((uint16_t*)p)[i] = f32_to_f16_bits(x); }
};
template <> struct Out<bf16_t> {
  using storage = uint16_t;
  __device__ __forceinline__ static void put(void* p, int64_t i, float x) { ((uint16_t*)p)[i] = f32_to_bf16(x); }
};

// DPP controls (CDNA data-parallel primitives, within a 16-lane row).
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of N lanes (N in 4, 8, 16, 32, 64); every lane of
// the group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_f<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float LOG2E = 1.4426950408889634f;
// Start value of a running maximum.  It is finite, so exp2(m_old - m_new) is 1
// and not NaN while nothing has been seen yet.
constexpr float NEG_BIG = -1.0e30f;

}  // namespace pkv
