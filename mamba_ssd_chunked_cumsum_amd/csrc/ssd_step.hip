// Single-token recurrent step (decode) of the SSD layer.
//
// One step of the selective state-space recurrence ("Why SSM and linear-RNN FLOPs do not convert
// into GPU FLOPs: the sequential scan bypasses the tensor cores", first paragraph), with the
// per-head scalar decay of SSD: for every (batch b, head h) with group g = h / (H / G),
//   a = exp(dt[b,h] A[h]);   S[p,n] <- a S[p,n] + dt[b,h] x[b,h,p] B[b,g,n];
//   y[b,h,p] = sum_n S[p,n] C[b,g,n] + D[h] x[b,h,p].
// Generation reads and writes the whole fp32 state once per token and does ~4 flops per state
// element, so the step is bound by HBM; its cost is linear in the number of tokens while the
// state stays O(P N) per head ("nitter.gq/da_be19" thread, post 5/6).
//
// Layout: lanes run along n, four consecutive n per lane (16-byte loads and stores), LPR lanes per
// state row (N / 4 rounded up to a power of two, so that the row sum C . S is a butterfly over
// xor-shuffles); a wave covers 64 / LPR rows and a block of four waves RB rows of one head. Every
// load of a thread is issued before its first store, and the state is read and written with
// nontemporal accesses (it is touched once per step): at the 2.7B-shaped layer (10.5 MB moved per
// step) the step runs at ~88% of a device copy of the same bytes.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

__device__ __forceinline__ float ld_io(const float* p) { return *p; }
__device__ __forceinline__ float ld_io(const u16* p) { return bf16_to_f32(*p); }

// Four consecutive io values, kept as loaded (16 or 8 bytes) until converted.
template <typename IO>
struct Raw4;
template <>
struct Raw4<float> {
  float4 v;
  static __device__ __forceinline__ Raw4 load(const float* p) {
    return Raw4{*reinterpret_cast<const float4*>(p)};
  }
  __device__ __forceinline__ void get(float (&o)[4]) const {
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
  }
};
template <>
struct Raw4<u16> {
  uint2 v;
  static __device__ __forceinline__ Raw4 load(const u16* p) {
    return Raw4{*reinterpret_cast<const uint2*>(p)};
  }
  __device__ __forceinline__ void get(float (&o)[4]) const {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

__device__ __forceinline__ void st_io(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_io(u16* p, float v) { *p = f32_to_bf16(v); }

// one pass (16 rows per block at N = 128): more, smaller blocks measured faster than two or more
// rows per thread
constexpr int kStepWaves = 4, kStepPasses = 1;

template <typename IO, int LPR>
__global__ __launch_bounds__(64 * kStepWaves) void k_step(
    const IO* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ D,
    const float* s_in, float* s_out, IO* __restrict__ y, Dims d) {
  constexpr int RPW = 64 / LPR, RB = kStepWaves * RPW * kStepPasses;  // rows per wave pass, block
  const int nrb = (d.P + RB - 1) / RB;
  const int bh = blockIdx.x / nrb, rb = blockIdx.x % nrb;  // (batch, head), row block
  const int b = bh / d.H, h = bh % d.H, g = h / (d.H / d.G);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % LPR, n0 = 4 * q;
  const bool nv = n0 < d.N;  // lanes past the row end (N / 4 not a power of two) idle
  const float dtv = dt[bh], a = __expf(dtv * A[h]), dh = D[h];
  // every load of the thread first (branch-free, on clamped addresses), then the stores:
  // state_out may be state_in, and each element is read and written by the same lane, so reading
  // all of them before any write keeps an in-place update correct, and all loads are in flight
  // together
  const int nc = nv ? n0 : d.N - 4;
  const int64_t bg = ((int64_t)b * d.G + g) * d.N + nc;
  const Raw4<IO> braw = Raw4<IO>::load(B + bg), craw = Raw4<IO>::load(C + bg);
  float4 sv[kStepPasses];
  IO xr[kStepPasses];
  int pr[kStepPasses];
#pragma unroll
  for (int pass = 0; pass < kStepPasses; ++pass) {
    pr[pass] = rb * RB + (pass * kStepWaves + wave) * RPW + lane / LPR;
    const int pc = min(pr[pass], d.P - 1);
    xr[pass] = x[(int64_t)bh * d.P + pc];
    {  // streamed once per step: nontemporal (no cache allocation for the state)
      const f32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(s_in + ((int64_t)bh * d.P + pc) * d.N + nc));
      sv[pass] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  float bv[4], cv[4];
  braw.get(bv);
  craw.get(cv);
#pragma unroll
  for (int pass = 0; pass < kStepPasses; ++pass) {
    const int p = pr[pass];
    const bool pv = p < d.P;
    const float xp = ld_io(&xr[pass]);
    float part = 0.f;
    if (pv && nv) {
      const float4 s = sv[pass];
      const float u = dtv * xp;
      const float4 t = make_float4(a * s.x + u * bv[0], a * s.y + u * bv[1], a * s.z + u * bv[2],
                                   a * s.w + u * bv[3]);
      __builtin_nontemporal_store(f32x4{t.x, t.y, t.z, t.w},
                                  reinterpret_cast<f32x4*>(s_out + ((int64_t)bh * d.P + p) * d.N +
                                                           n0));
      part = t.x * cv[0] + t.y * cv[1] + t.z * cv[2] + t.w * cv[3];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
    if (pv && q == 0) st_io(y + (int64_t)bh * d.P + p, part + dh * xp);
  }
}

template <typename IO, int LPR>
hipError_t launch(const Dims& d, const void* x, const float* dt, const float* A, const void* B,
                  const void* C, const float* D, const float* s_in, float* s_out, void* y,
                  hipStream_t s) {
  constexpr int RB = kStepWaves * (64 / LPR) * kStepPasses;
  const int nrb = (d.P + RB - 1) / RB;
  hipLaunchKernelGGL((k_step<IO, LPR>), dim3(d.Bt * d.H * nrb), dim3(64 * kStepWaves), 0, s,
                     (const IO*)x, dt, A, (const IO*)B, (const IO*)C, D, s_in, s_out, (IO*)y, d);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const Dims& d, const void* x, const float* dt, const float* A, const void* B,
                     const void* C, const float* D, const float* s_in, float* s_out, void* y,
                     hipStream_t s) {
  const int lanes = d.N / 4;  // N is a multiple of 16, at most 256
  if (lanes <= 4) return launch<IO, 4>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
  if (lanes <= 8) return launch<IO, 8>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
  if (lanes <= 16) return launch<IO, 16>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
  if (lanes <= 32) return launch<IO, 32>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
  return launch<IO, 64>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
}

}  // namespace

hipError_t launch_step(const Dims& d, int io, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* s_in,
                       float* s_out, void* y, hipStream_t s) {
  if (io == kIoBf16) return launch_io<u16>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
  return launch_io<float>(d, x, dt, A, B, C, D, s_in, s_out, y, s);
}

}  // namespace ssd
