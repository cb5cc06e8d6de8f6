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
// xor-shuffles); a wave covers 64 / LPR rows per pass and a block of four waves covers RB rows of
// one head in two passes. B and C of the head's group are loaded once per lane.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

__device__ __forceinline__ float ld_io(const float* p) { return *p; }
__device__ __forceinline__ float ld_io(const u16* p) { return bf16_to_f32(*p); }

// four consecutive io values -> floats
__device__ __forceinline__ void ld4_io(const float* p, float (&v)[4]) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x;
  v[1] = q.y;
  v[2] = q.z;
  v[3] = q.w;
}
__device__ __forceinline__ void ld4_io(const u16* p, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

__device__ __forceinline__ void st_io(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_io(u16* p, float v) { *p = f32_to_bf16(v); }

constexpr int kStepWaves = 4, kStepPasses = 2;

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
  float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {0.f, 0.f, 0.f, 0.f};
  if (nv) {
    ld4_io(B + ((int64_t)b * d.G + g) * d.N + n0, bv);
    ld4_io(C + ((int64_t)b * d.G + g) * d.N + n0, cv);
  }
#pragma unroll
  for (int pass = 0; pass < kStepPasses; ++pass) {
    const int p = rb * RB + (pass * kStepWaves + wave) * RPW + lane / LPR;
    const bool pv = p < d.P;
    float part = 0.f, xp = 0.f;
    if (pv) {
      xp = ld_io(x + (int64_t)bh * d.P + p);
      if (nv) {
        const int64_t o = ((int64_t)bh * d.P + p) * d.N + n0;
        const float4 s = *reinterpret_cast<const float4*>(s_in + o);
        const float u = dtv * xp;
        const float4 t = make_float4(a * s.x + u * bv[0], a * s.y + u * bv[1],
                                     a * s.z + u * bv[2], a * s.w + u * bv[3]);
        *reinterpret_cast<float4*>(s_out + o) = t;
        part = t.x * cv[0] + t.y * cv[1] + t.z * cv[2] + t.w * cv[3];
      }
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
