// Device helpers shared by the gfx950 kernels of libgpt2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

#define WAVE 64

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Rounding is to nearest, ties to even; NaN stays NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: nearest-even, NaN kept
}

// two floats -> packed pair of bf16 (lo in the low half)
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Typed scalar load/store for the storage types of activations.
__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ void stf(float* p, float v) { *p = v; }
__device__ __forceinline__ void stf(bf16_t* p, float v) { *p = f2bf(v); }

// Four consecutive elements (address aligned to 4 elements).
__device__ __forceinline__ void ld4(const float* p, float v[4]) {
  float4 t = *reinterpret_cast<const float4*>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void ld4(const bf16_t* p, float v[4]) {
  uint2 t = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
  v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(bf16_t* p, const float v[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// device error flags (bit set by kernels, read back by the host at sync points)
enum : int { ERRF_IDX = 1, ERRF_TARGET = 2 };

// GELU, tanh form: 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)) =: s,
// with the hardware exp2 and reciprocal (a few ulp in fp32); -2u log2(e) is
// formed as x (k0 + k1 x^2) with the constants folded.
__device__ __forceinline__ float gelu_sig_f(float x, float x2) {
  const float a = 0.7978845608028654f;  // sqrt(2/pi)
  const float c = 0.044715f;
  const float k0 = -2.0f * 1.4426950408889634f * a, k1 = k0 * c;
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * fmaf(x2, k1, k0)));
}
__device__ __forceinline__ float gelu_tanh_f(float x) { return x * gelu_sig_f(x, x * x); }
// d/dx = s + 2 x s (1 - s) u'(x), u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2)
__device__ __forceinline__ float gelu_grad_from_sig(float x, float x2, float s) {
  const float a = 0.7978845608028654f;
  const float c = 0.044715f;
  const float q = x * fmaf(x2, 6.0f * a * c, 2.0f * a);  // 2 x u'(x)
  return fmaf(q, fmaf(-s, s, s), s);                      // s + q s (1 - s)
}
__device__ __forceinline__ float gelu_tanh_grad_f(float x) {
  const float x2 = x * x;
  return gelu_grad_from_sig(x, x2, gelu_sig_f(x, x2));
}
// Both at once (one exponential): returns gelu(x), stores gelu'(x).
__device__ __forceinline__ float gelu_tanh_and_grad_f(float x, float* grad) {
  const float x2 = x * x;
  const float s = gelu_sig_f(x, x2);
  *grad = gelu_grad_from_sig(x, x2, s);
  return x * s;
}
