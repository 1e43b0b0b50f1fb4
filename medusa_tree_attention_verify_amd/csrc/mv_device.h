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

// Raw buffer resource (gfx950): dword 3 selects 32-bit data format for untyped loads; an
// offset at or past the record count reads as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kBufferOutOfRange = 0x7fffffff;

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

// ---- wave64 butterfly reductions with vector-ALU cross-lane moves.  The six exchange steps
// pair lanes 1 and 2 apart (DPP quad permutations), then mirror 8- and 16-lane rows (DPP row
// mirrors: after the quad steps every lane of a quad holds the same value, so a mirror pairs
// distinct quads), then swap 16-lane rows and 32-lane halves (v_permlane16_swap /
// v_permlane32_swap, which hand each lane its own value and its partner's).  No LDS round
// trips; every lane ends with the same bits for a commutative operation.  All 64 lanes must be
// active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
struct LanePair {
  uint32_t a, b;  // this lane's value and its partner's, in either order
};
__device__ __forceinline__ LanePair swap16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppHalfMirror>(v));
  v = op(v, dpp_u32<kDppMirror>(v));
  LanePair t = swap16(v);
  v = op(t.a, t.b);
  t = swap32(v);
  return op(t.a, t.b);
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
}

__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  }));
}

__device__ __forceinline__ int wave_max_i(int v) {
  return static_cast<int>(wave_allreduce_u32(static_cast<uint32_t>(v), [](uint32_t x, uint32_t y) {
    return static_cast<uint32_t>(max(static_cast<int>(x), static_cast<int>(y)));
  }));
}

__device__ __forceinline__ int wave_min_i(int v) {
  return static_cast<int>(wave_allreduce_u32(static_cast<uint32_t>(v), [](uint32_t x, uint32_t y) {
    return static_cast<uint32_t>(min(static_cast<int>(x), static_cast<int>(y)));
  }));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  auto step = [](double x, uint32_t lo, uint32_t hi) {
    return x + __hiloint2double(static_cast<int>(hi), static_cast<int>(lo));
  };
  auto lo = [](double x) { return static_cast<uint32_t>(__double2loint(x)); };
  auto hi = [](double x) { return static_cast<uint32_t>(__double2hiint(x)); };
  v = step(v, dpp_u32<kDppXor1>(lo(v)), dpp_u32<kDppXor1>(hi(v)));
  v = step(v, dpp_u32<kDppXor2>(lo(v)), dpp_u32<kDppXor2>(hi(v)));
  v = step(v, dpp_u32<kDppHalfMirror>(lo(v)), dpp_u32<kDppHalfMirror>(hi(v)));
  v = step(v, dpp_u32<kDppMirror>(lo(v)), dpp_u32<kDppMirror>(hi(v)));
  LanePair l = swap16(lo(v)), h = swap16(hi(v));
  v = __hiloint2double(static_cast<int>(h.a), static_cast<int>(l.a)) + __hiloint2double(static_cast<int>(h.b), static_cast<int>(l.b));
  l = swap32(lo(v));
  h = swap32(hi(v));
  return __hiloint2double(static_cast<int>(h.a), static_cast<int>(l.a)) + __hiloint2double(static_cast<int>(h.b), static_cast<int>(l.b));
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
  auto take = [&](uint32_t ov, uint32_t oi) {
    if (kv_better(__uint_as_float(ov), static_cast<int>(oi), v, i)) {
      v = __uint_as_float(ov);
      i = static_cast<int>(oi);
    }
  };
  take(dpp_u32<kDppXor1>(__float_as_uint(v)), dpp_u32<kDppXor1>(static_cast<uint32_t>(i)));
  take(dpp_u32<kDppXor2>(__float_as_uint(v)), dpp_u32<kDppXor2>(static_cast<uint32_t>(i)));
  take(dpp_u32<kDppHalfMirror>(__float_as_uint(v)), dpp_u32<kDppHalfMirror>(static_cast<uint32_t>(i)));
  take(dpp_u32<kDppMirror>(__float_as_uint(v)), dpp_u32<kDppMirror>(static_cast<uint32_t>(i)));
  {
    const LanePair tv = swap16(__float_as_uint(v)), ti = swap16(static_cast<uint32_t>(i));
    v = __uint_as_float(tv.a);
    i = static_cast<int>(ti.a);
    take(tv.b, ti.b);
  }
  {
    const LanePair tv = swap32(__float_as_uint(v)), ti = swap32(static_cast<uint32_t>(i));
    v = __uint_as_float(tv.a);
    i = static_cast<int>(ti.a);
    take(tv.b, ti.b);
  }
}

// Log-sum-exp merge of two partial (max, sum of exp(x - max)) pairs; symmetric in its operands,
// so the butterfly below leaves the same bits in every lane.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    l = l2;
    return;
  }
  const float mn = fmaxf(m, m2);
  l = l * expf(m - mn) + l2 * expf(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void wave_ml_merge(float& m, float& l) {
  auto step = [&](uint32_t om, uint32_t ol) { ml_merge(m, l, __uint_as_float(om), __uint_as_float(ol)); };
  step(dpp_u32<kDppXor1>(__float_as_uint(m)), dpp_u32<kDppXor1>(__float_as_uint(l)));
  step(dpp_u32<kDppXor2>(__float_as_uint(m)), dpp_u32<kDppXor2>(__float_as_uint(l)));
  step(dpp_u32<kDppHalfMirror>(__float_as_uint(m)), dpp_u32<kDppHalfMirror>(__float_as_uint(l)));
  step(dpp_u32<kDppMirror>(__float_as_uint(m)), dpp_u32<kDppMirror>(__float_as_uint(l)));
  {
    const LanePair tm = swap16(__float_as_uint(m)), tl = swap16(__float_as_uint(l));
    m = __uint_as_float(tm.a);
    l = __uint_as_float(tl.a);
    step(tm.b, tl.b);
  }
  {
    const LanePair tm = swap32(__float_as_uint(m)), tl = swap32(__float_as_uint(l));
    m = __uint_as_float(tm.a);
    l = __uint_as_float(tl.a);
    step(tm.b, tl.b);
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
