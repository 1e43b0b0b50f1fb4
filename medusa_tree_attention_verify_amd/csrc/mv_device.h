// Device-side helpers shared by the gfx950 kernels of the tree-verification library:
// bf16 bit conversions, MFMA operand types, wave64 / workgroup reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even to bf16: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8, t);
}

// Two floats -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Ordering used by every top-k / argmax of the library: larger value first, equal values by
// lower index.  An empty slot is (-inf, INT_MAX).
__device__ __forceinline__ bool kv_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// (v, i) strictly after (pv, pi) in that order.
__device__ __forceinline__ bool kv_after(float v, int i, float pv, int pi) {
  return v < pv || (v == pv && i > pi);
}

__device__ __forceinline__ void wave_argbest(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (kv_better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Workgroup-wide best (value, index); every thread gets the result.  `sv`/`si` are LDS
// arrays with one slot per wave.  Contains __syncthreads().
__device__ __forceinline__ void block_argbest(float& v, int& i, float* sv, int* si) {
  wave_argbest(v, i);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int k = 1; k < nw; ++k)
    if (kv_better(sv[k], si[k], v, i)) { v = sv[k]; i = si[k]; }
}

__device__ __forceinline__ float block_max(float v, float* s) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) s[w] = v;
  __syncthreads();
  v = s[0];
  for (int k = 1; k < nw; ++k) v = fmaxf(v, s[k]);
  return v;
}

__device__ __forceinline__ float block_sum(float v, float* s) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) s[w] = v;
  __syncthreads();
  v = 0.f;
  for (int k = 0; k < nw; ++k) v += s[k];
  return v;
}

// Streaming (non-temporal) 16-byte loads of data that is read once.
__device__ __forceinline__ uint4 load_nt_u4(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 load_nt_f4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

}  // namespace mv
