// Device helpers for the libssd kernels (gfx950, wave64). Library-internal.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_launch.h"

namespace ssd {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWave = 64;

// ---- scalar conversions ------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(u16 v) { return __uint_as_float((uint32_t)v << 16); }

// Round to nearest even; NaN stays NaN (quiet), overflow rounds to infinity.
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// The effective dt of head h from the dt the caller passed (see Dims): + bias, softplus
// (log(1 + exp(v)); v itself above 20, where the two agree to fp32 precision), clamp.
__device__ __forceinline__ float dt_effective(float v, float bias, const Dims& d) {
  v += bias;
  if (d.dt_softplus) v = v <= 20.f ? log1pf(expf(v)) : v;
  if (d.dt_max > 0.f) v = fminf(fmaxf(v, d.dt_min), d.dt_max);
  return v;
}
__device__ __forceinline__ float dt_bias_of(const Dims& d, int h) {
  return d.dt_bias ? d.dt_bias[h] : 0.f;
}

// IO element access: fp32 io stores float, bf16 io stores raw bf16 bits.
template <typename IO> struct Io;
template <> struct Io<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Io<u16> {
  static __device__ __forceinline__ float load(const u16* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(u16* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Load 8 consecutive io elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
__device__ __forceinline__ void load8(const u16* p, float (&v)[8]) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ---- matrix-core tiles (16 x 16 fp32 outputs) ------------------------------------------------
// Lane l of a wave owns output column (l & 15) and rows 4*(l >> 4) + r, r = 0..3.
// Operand fragments: lane l supplies row (A) / column (B) (l & 15) and the K slice
// [KPL*(l >> 4), KPL*(l >> 4) + KPL) of one K step (K step = 4 * KPL).
template <typename T> struct Mma;
template <> struct Mma<f16> {
  static constexpr int KPL = 8, KSTEP = 32;
  typedef f16x8 Frag;
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag lds(const f16* p) {  // 8 contiguous values
    return *reinterpret_cast<const f16x8*>(p);
  }
};
template <> struct Mma<float> {
  static constexpr int KPL = 1, KSTEP = 4;
  typedef float Frag;
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag lds(const float* p) { return *p; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- wave-level inclusive prefix sum -----------------------------------------------------------
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

}  // namespace ssd
