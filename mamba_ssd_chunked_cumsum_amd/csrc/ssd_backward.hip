// Helper kernels of the SSD backward (ssd_backward in ssd_api.cpp). Library-internal.
//
// The backward reuses the forward's chunked kernels on rearranged inputs (see ssd_api.cpp); what
// is here moves data between those calls (reversal in time, group -> head broadcast, state
// transposes, fp32 conversion) and combines their outputs into the gradients: elementwise terms,
// the reverse cumulative sum that gives the decay gradients, and sums over heads and batch. Every
// kernel is memory-bound and bounds-checked per element.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

__global__ __launch_bounds__(256) void k_dt_shift_rev(const float* __restrict__ dt,
                                                      float* __restrict__ dtr, int Bt, int L,
                                                      int H, int pad) {
  const int Lo = L + pad;
  const int64_t total = (int64_t)Bt * Lo * H;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int h = (int)(i % H);
    const int t = (int)((i / H) % Lo) - pad;
    const int b = (int)(i / ((int64_t)H * Lo));
    dtr[i] = t <= 0 ? 0.f : dt[((int64_t)b * L + (L - t)) * H + h];
  }
}

// Sum over the 64 lanes of a wave (every lane gets the total).
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum over the wave's lanes, in double.
__device__ __forceinline__ double wave_scan_f64(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// dx = D dy + dt u, and the per-(b, t, h) sums the decay gradients are built from.
template <typename IO>
__global__ __launch_bounds__(256) void k_bwd_pointwise(
    const IO* __restrict__ x, const IO* __restrict__ dy, const float* __restrict__ ur,
    const float* __restrict__ ys, const float* __restrict__ dt, const float* __restrict__ D,
    float* __restrict__ dx, float* __restrict__ q, float* __restrict__ xu,
    float* __restrict__ dyx, int Bt, int L, int H, int P, int pad) {
  // 16 lanes per (b, t, h) unit, four units per wave: lane k of a unit takes p = 4 k + 64 m
  // (16-byte accesses); headdim is a multiple of 16. Lanes of a unit past the last one compute on
  // a clamped unit and store nothing (all lanes take part in the reductions).
  const int64_t nunit = (int64_t)Bt * L * H;
  const int64_t unit_raw = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const bool valid = unit_raw < nunit;
  const int64_t unit = valid ? unit_raw : nunit - 1;
  const int sl = threadIdx.x & 15;
  const int h = (int)(unit % H);
  const int t = (int)((unit / H) % L);
  const int b = (int)(unit / ((int64_t)H * L));
  const float dtv = dt[unit], dh = D[h];
  const int64_t row = unit * P;                                          // [b, t, h, :]
  // reversed time, pad leading rows per batch entry
  const int64_t rrow = (((int64_t)b * (L + pad) + pad + (L - 1 - t)) * H + h) * P;
  float s_dyys = 0.f, s_xu = 0.f, s_dyx = 0.f;
  for (int p = 4 * sl; p < P; p += 64) {
    float xv[4], dyv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xv[k] = Io<IO>::load(x, row + p + k);
      dyv[k] = Io<IO>::load(dy, row + p + k);
    }
    const float4 u = *reinterpret_cast<const float4*>(ur + rrow + p);
    const float4 yv = *reinterpret_cast<const float4*>(ys + row + p);
    const float uu[4] = {u.x, u.y, u.z, u.w}, yy[4] = {yv.x, yv.y, yv.z, yv.w};
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[k] = dh * dyv[k] + dtv * uu[k];
      s_dyys += dyv[k] * yy[k];
      s_xu += xv[k] * uu[k];
      s_dyx += dyv[k] * xv[k];
    }
    if (valid) *reinterpret_cast<float4*>(dx + row + p) = make_float4(o[0], o[1], o[2], o[3]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    s_dyys += __shfl_xor(s_dyys, off, 16);
    s_xu += __shfl_xor(s_xu, off, 16);
    s_dyx += __shfl_xor(s_dyx, off, 16);
  }
  if (valid && sl == 0) {
    q[unit] = s_dyys - dtv * s_xu;
    xu[unit] = s_xu;
    dyx[unit] = s_dyx;
  }
}

// One 256-thread block per (b, h, tile k): the anchor <G_t, S_{t-1}> of the tile's first token
// t = 256 k, in double, from the state that the forward recurrence has entering its chunk t / Q
// (hf: [Bt, ncf, H, P, N]) and the adjoint G_t, which the adjoint recurrence, run in reversed
// time over Lp = L + pad tokens (Lp % Q == 0), has entering its chunk (Lp - t) / Q (hg:
// [Bt, ncg, H, P, N]) or, for t = 0, leaves as its final state (g0: [Bt, H, P, N]).
__global__ __launch_bounds__(256) void k_anchor_dot(const float* __restrict__ hf,
                                                    const float* __restrict__ hg,
                                                    const float* __restrict__ g0,
                                                    double* __restrict__ anch, int H, int PN,
                                                    int Q, int ncf, int ncg, int Lp, int ntile) {
  __shared__ double part[4];
  const int k = blockIdx.x % ntile, bh = blockIdx.x / ntile, h = bh % H, b = bh / H;
  const int t = 256 * k;
  const float* S = hf + (((int64_t)b * ncf + t / Q) * H + h) * PN;
  const float* G = k == 0 ? g0 + (int64_t)bh * PN
                          : hg + (((int64_t)b * ncg + (Lp - t) / Q) * H + h) * PN;
  double v = 0.0;
  for (int i = threadIdx.x; i < PN; i += 256) v += (double)S[i] * (double)G[i];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) anch[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

// One 256-thread block per (b, h): tiles of 256 tokens, each tile's suffix sums by a block
// scan. Every tile starts from the exact value at its first token t0,
// da_t0 = exp(dt_t0 A) <G_t0, S_t0-1> (anch, per (b, h, tile)), and forms
// da_t = da_t0 - sum_{t0 <= s < t} q_s: a sum over the rest of the sequence instead would carry
// the terms' fp32 rounding, which grows with its length while da_t does not. The sums run in
// double: dA sums dt_t da_t over batch and time.
__global__ __launch_bounds__(256) void k_bwd_scan(const float* __restrict__ q,
                                                  const float* __restrict__ xu,
                                                  const float* __restrict__ dyx,
                                                  const float* __restrict__ dt,
                                                  const float* __restrict__ A,
                                                  const double* __restrict__ anch,
                                                  float* __restrict__ ddt, double* __restrict__ pa,
                                                  double* __restrict__ pd, int L, int H) {
  __shared__ double wtot[4];
  __shared__ double red[2][4];
  const int bh = blockIdx.x, h = bh % H, b = bh / H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double a = A[h];
  double sa = 0.0, sd = 0.0;
  const int ntile = (L + 255) / 256;
  for (int k = ntile - 1; k >= 0; --k) {
    // thread j of the tile holds token t = 256 k + 255 - j (reversed, so a prefix scan over j
    // is the suffix sum over t)
    const int t = 256 * k + 255 - threadIdx.x;
    const int64_t i = ((int64_t)b * L + t) * H + h;
    const bool ok = t < L;
    const double v = ok ? (double)q[i] : 0.0;
    const double incl = wave_scan_f64(v);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    // before + incl = sum_{t <= s <= tile end} q_s; less the tile's total: -sum_{t0 <= s < t} q_s
    const double tile_total = (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
    const double da0 = exp((double)dt[((int64_t)b * L + 256 * k) * H + h] * a) *
                       anch[(int64_t)bh * ntile + k];
    const double da = da0 - tile_total + before + incl;
    if (ok) {
      ddt[i] = (float)(a * da + (double)xu[i]);
      sa += (double)dt[i] * da;
      sd += (double)dyx[i];
    }
    __syncthreads();  // wtot is rewritten by the next tile
  }
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  if (lane == 0) {
    red[0][wave] = sa;
    red[1][wave] = sd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    pa[bh] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    pd[bh] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

__global__ __launch_bounds__(256) void k_sum_batch(const double* __restrict__ pa,
                                                   const double* __restrict__ pd,
                                                   float* __restrict__ dA, float* __restrict__ dD,
                                                   int Bt, int H) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  double sa = 0.0, sd = 0.0;
  for (int b = 0; b < Bt; ++b) {
    sa += pa[b * H + h];
    sd += pd[b * H + h];
  }
  dA[h] = (float)sa;
  dD[h] = (float)sd;
}

__global__ __launch_bounds__(256) void k_group_sums(const float* __restrict__ vb,
                                                    const float* __restrict__ vc,
                                                    const float* __restrict__ dt,
                                                    float* __restrict__ dB, float* __restrict__ dC,
                                                    int Bt, int L, int H, int G, int N,
                                                    int pad) {
  const int64_t total = (int64_t)Bt * L * G * N;
  const int hpg = H / G;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int n = (int)(i % N);
    const int g = (int)((i / N) % G);
    const int t = (int)((i / ((int64_t)N * G)) % L);
    const int b = (int)(i / ((int64_t)N * G * L));
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < hpg; ++k) {
      const int h = g * hpg + k;
      const int64_t f = ((int64_t)b * L + t) * H + h;
      const int64_t r = ((int64_t)b * (L + pad) + pad + (L - 1 - t)) * H + h;
      sb += dt[f] * vb[r * N + n];
      sc += vc[f * N + n];
    }
    dB[i] = sb;
    dC[i] = sc;
  }
}

__global__ __launch_bounds__(256) void k_scale_state(const float* __restrict__ g0,
                                                     const float* __restrict__ dt,
                                                     const float* __restrict__ A,
                                                     float* __restrict__ out, int Bt, int L,
                                                     int H, int PN) {
  const int64_t total = (int64_t)Bt * H * PN;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t bh = i / PN;
    const int h = (int)(bh % H);
    const int b = (int)(bh / H);
    out[i] = __expf(dt[(int64_t)b * L * H + h] * A[h]) * g0[i];
  }
}

int grid_for(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

// out[b, pad + t] = in[b, L - 1 - t] (rows of E elements of type T), out[b, 0 .. pad - 1] = 0:
// a copy reversed in time, in the input's own type. One block per output row, 16-byte pieces
// (E * sizeof(T) is a multiple of 16).
template <typename T>
__global__ __launch_bounds__(256) void k_reverse_rows(const T* __restrict__ in, T* __restrict__ out,
                                                     int L, int E, int pad) {
  const int Lo = L + pad;
  const int row = blockIdx.x, tp = row % Lo, b = row / Lo;
  uint4* o = reinterpret_cast<uint4*>(out + (int64_t)row * E);
  const int n16 = E * (int)sizeof(T) / 16;
  if (tp < pad) {
    for (int f = threadIdx.x; f < n16; f += 256) o[f] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint4* src =
      reinterpret_cast<const uint4*>(in + ((int64_t)b * L + (L - 1 - (tp - pad))) * E);
  for (int f = threadIdx.x; f < n16; f += 256) o[f] = src[f];
}

hipError_t launch_reverse_rows(int io, const void* in, void* out, int Bt, int L, int E, int pad,
                               hipStream_t s) {
  const dim3 g((unsigned)Bt * (unsigned)(L + pad));
  if (io == kIoBf16)
    hipLaunchKernelGGL(k_reverse_rows<u16>, g, dim3(256), 0, s, (const u16*)in, (u16*)out, L, E,
                       pad);
  else
    hipLaunchKernelGGL(k_reverse_rows<float>, g, dim3(256), 0, s, (const float*)in, (float*)out,
                       L, E, pad);
  return hipGetLastError();
}

hipError_t launch_dt_shift_rev(const float* dt, float* dtr, int Bt, int L, int H, int pad,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_dt_shift_rev, dim3(grid_for((int64_t)Bt * (L + pad) * H)), dim3(256), 0, s,
                     dt, dtr, Bt, L, H, pad);
  return hipGetLastError();
}

hipError_t launch_bwd_pointwise(int io, const void* x, const void* dy, const float* ur,
                                const float* ys, const float* dt, const float* D, float* dx,
                                float* q, float* xu, float* dyx, int Bt, int L, int H, int P,
                                int pad, hipStream_t s) {
  const int64_t units = (int64_t)Bt * L * H;
  const dim3 grid((unsigned)((units + 15) / 16));  // 16 units per block
  if (io == kIoBf16)
    hipLaunchKernelGGL(k_bwd_pointwise<u16>, grid, dim3(256), 0, s, (const u16*)x,
                       (const u16*)dy, ur, ys, dt, D, dx, q, xu, dyx, Bt, L, H, P, pad);
  else
    hipLaunchKernelGGL(k_bwd_pointwise<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)dy, ur, ys, dt, D, dx, q, xu, dyx, Bt, L, H, P, pad);
  return hipGetLastError();
}

hipError_t launch_anchor_dot(const float* hf, const float* hg, const float* g0, double* anch,
                             int Bt, int H, int PN, int Q, int ncf, int ncg, int L, int Lp,
                             hipStream_t s) {
  const int ntile = (L + 255) / 256;
  hipLaunchKernelGGL(k_anchor_dot, dim3((unsigned)(Bt * H * ntile)), dim3(256), 0, s, hf, hg, g0,
                     anch, H, PN, Q, ncf, ncg, Lp, ntile);
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const float* q, const float* xu, const float* dyx, const float* dt,
                           const float* A, const double* anch, float* ddt, double* pa, double* pd,
                           int Bt, int L, int H, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_scan, dim3(Bt * H), dim3(256), 0, s, q, xu, dyx, dt, A, anch, ddt, pa,
                     pd, L, H);
  return hipGetLastError();
}

hipError_t launch_sum_batch(const double* pa, const double* pd, float* dA, float* dD, int Bt,
                            int H, hipStream_t s) {
  hipLaunchKernelGGL(k_sum_batch, dim3((H + 255) / 256), dim3(256), 0, s, pa, pd, dA, dD, Bt, H);
  return hipGetLastError();
}

hipError_t launch_group_sums(const float* vb, const float* vc, const float* dt, float* dB,
                             float* dC, int Bt, int L, int H, int G, int N, int pad,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_group_sums, dim3(grid_for((int64_t)Bt * L * G * N)), dim3(256), 0, s, vb,
                     vc, dt, dB, dC, Bt, L, H, G, N, pad);
  return hipGetLastError();
}

hipError_t launch_scale_state(const float* g0, const float* dt, const float* A, float* dh0,
                              int Bt, int L, int H, int PN, hipStream_t s) {
  hipLaunchKernelGGL(k_scale_state, dim3(grid_for((int64_t)Bt * H * PN)), dim3(256), 0, s, g0, dt,
                     A, dh0, Bt, L, H, PN);
  return hipGetLastError();
}

}  // namespace ssd
