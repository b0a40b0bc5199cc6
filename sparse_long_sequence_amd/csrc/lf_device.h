// Device helpers for the gfx950 kernels: element types, conversions, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

typedef _Float16 f16;
typedef __bf16 bf16;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element traits: widening to fp32 is exact; narrowing rounds to nearest even.
template <typename T> struct Elem;
template <> struct Elem<float> {
  typedef float vec8 __attribute__((ext_vector_type(8)));
  typedef f32x4 vec4;
  __device__ static inline float to_f(float x) { return x; }
  __device__ static inline float from_f(float x) { return x; }
};
template <> struct Elem<f16> {
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  typedef f16x2 vec2;
  __device__ static inline float to_f(f16 x) { return (float)x; }
  __device__ static inline f16 from_f(float x) { return (f16)x; }
};
template <> struct Elem<bf16> {
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  typedef bf16x2 vec2;
  __device__ static inline float to_f(bf16 x) { return (float)x; }
  __device__ static inline bf16 from_f(float x) { return (bf16)x; }
};

// D = A(32x16) * B(16x32) + C on the matrix cores, fp32 accumulation.
__device__ inline f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32: D = A(32x2) * B(2x32) + C four times, one k pair per element of the 16-byte
// fragments (lane (n, g) holds 4 consecutive k of row n; both operands pair the same
// k values, so the sum over k is complete).
__device__ inline f32x16 mfma32(const f32x4& a, const f32x4& b, const f32x16& c) {
  f32x16 d = c;
#pragma unroll
  for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], d, 0, 0, 0);
  return d;
}

// Sum of a pair of 16-bit values accumulated in fp32 (v_dot2 with a (1,1) vector).
__device__ inline float dot2_ones(const f16x2& p, float acc) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
  return __builtin_amdgcn_fdot2(p, one, acc, false);
}
__device__ inline float dot2_ones(const bf16x2& p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int lane_id() { return __lane_id(); }

// Wave-wide exclusive prefix sum of an int (64 lanes).
__device__ inline int wave_excl_scan(int x) {
  int lane = lane_id();
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  return incl - x;
}

}  // namespace lf
