// Fused SSD chunked forward (bf16 io): the intra-chunk C B^T block lives only in registers, and
// the state is carried on chip through a run of consecutive chunks.
//
// The chunked algorithm ("nitter.gq/da_be19" thread, post 5/6; stage order as in "Mamba-2 in
// NVIDIA cuTile: Faster Forward Kernels and What the Benchmark Means", section "Why Mamba-2 is a
// useful kernel example") needs, for every chunk, the state entering it. A chunk's fp32 state
// (P x N) is as large as or larger than its bf16 x tile (Q x P) for the usual shapes, so
// materialising it per chunk would double the HBM traffic. Here the sequence of each (batch,
// head) is cut into runs of S chunks:
//
//   F1 k_run_state    each run's own end state (zero entry state) and total log-decay
//   F2 k_state_pass   (shared with the unfused path) state entering each run; final state
//   F3 k_fused_scan   per run: for each chunk, cumulative decay, C B^T, the masked intra-chunk
//                     product, the inter-chunk readout from the carried state, the skip term,
//                     and the carried-state update -- all on chip; only y leaves the kernel.
//
// Only run-boundary states touch memory (1/S of the per-chunk volume).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---- F1: run states -------------------------------------------------------------------------
// state_r = sum_{t in run} exp(sum_{k in (t, end]} dt_k A) dt_t x_t B_t^T, computed with suffix
// sums (so the weights of the tokens near the run end, which dominate, are accurate), and
// logdecay_r = sum_{t in run} dt_t A. Grid (nr * ceil(P/64), H, batch), 256 threads; token slabs
// of 32 are taken from the run end backwards. The state operand w_t x_t is split into fp16 high
// and low parts (two matrix-core passes) so the chained run states keep fp32-level accuracy.
constexpr int RSJ = 32;

__global__ __launch_bounds__(256) void k_run_state(const u16* __restrict__ x,
                                                   const u16* __restrict__ Bm,
                                                   const float* __restrict__ dt,
                                                   const float* __restrict__ Av,
                                                   float* __restrict__ states,
                                                   float* __restrict__ logdecay, Dims d,
                                                   int run_len, int nr) {
  using M = Mma<f16>;
  constexpr int LD = RSJ + 8;
  __shared__ __align__(16) f16 Wh[64 * LD];
  __shared__ __align__(16) f16 Wl[64 * LD];
  __shared__ __align__(16) f16 Bt[256 * LD];
  __shared__ float w[RSJ];
  __shared__ float carry_s;
  const int npb = (d.P + 63) / 64;
  const int r = blockIdx.x / npb, pb = blockIdx.x % npb, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (d.H / d.G);
  const int p0 = pb * 64, np = min(64, d.P - p0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t_begin = r * run_len, t_end = min(d.L, t_begin + run_len);
  const float a_h = Av[h];
  const int npt = np / 16, nnt = d.N / 16;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
  if (threadIdx.x == 0) carry_s = 0.f;

  const int nslab = (t_end - t_begin + RSJ - 1) / RSJ;
  for (int sidx = nslab - 1; sidx >= 0; --sidx) {
    const int s0 = t_begin + sidx * RSJ;
    __syncthreads();  // previous slab's consumers are done; carry_s is current
    if (wave == 0) {
      // suffix sums inside the slab: lane l holds token s0 + l (lanes >= RSJ idle)
      const int t = s0 + lane;
      const bool valid = lane < RSJ && t < t_end;
      const float dtv = valid ? dt[((int64_t)b * d.L + t) * d.H + h] : 0.f;
      const float a = dtv * a_h;
      // reverse inclusive scan over the 32 lanes: sum of a over lanes >= l
      float v = a;
#pragma unroll
      for (int off = 1; off < RSJ; off <<= 1) {
        const float o = __shfl_down(v, off, kWave);
        if (lane + off < RSJ) v += o;
      }
      const float carry = carry_s;
      // exclusive suffix (tokens after t up to the run end) = carry + (v - a) re-associated as
      // carry + sum over lanes > l
      float excl = __shfl_down(v, 1, kWave);
      if (lane + 1 >= RSJ) excl = 0.f;
      if (lane < RSJ) w[lane] = valid ? __expf(carry + excl) * dtv : 0.f;
      const float total = __shfl(v, 0, kWave);
      if (lane == 0) carry_s = carry + total;
    }
    // W^T slab (hi + lo)
    for (int e = threadIdx.x; e < RSJ * (np / 8); e += 256) {
      const int jj = e / (np / 8), p8 = (e % (np / 8)) * 8;
      const int t = s0 + jj;
      float v[8];
      if (t < t_end) {
        load8(x + (((int64_t)b * d.L + t) * d.H + h) * d.P + p0 + p8, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) Wh[(p8 + k) * LD + jj] = (f16)v[k];  // raw x, scaled below
    }
    for (int e = threadIdx.x; e < RSJ * (d.N / 8); e += 256) {
      const int jj = e / (d.N / 8), n8 = (e % (d.N / 8)) * 8;
      const int t = s0 + jj;
      float v[8];
      if (t < t_end) {
        load8(Bm + (((int64_t)b * d.L + t) * d.G + g) * d.N + n8, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) Bt[(n8 + k) * LD + jj] = (f16)v[k];
    }
    __syncthreads();  // w[], raw x, B^T visible
    // scale x by the weights and split into hi + lo
    for (int e = threadIdx.x; e < RSJ * np; e += 256) {
      const int p = e / RSJ, jj = e % RSJ;
      const float val = (float)Wh[p * LD + jj] * w[jj];
      const f16 hi = (f16)val;
      Wh[p * LD + jj] = hi;
      Wl[p * LD + jj] = (f16)(val - (float)hi);
    }
    __syncthreads();
    const int kk = M::KPL * kg;
    f16x8 ah[4], al[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt < npt) {
        ah[pt] = M::lds(Wh + (pt * 16 + col) * LD + kk);
        al[pt] = M::lds(Wl + (pt * 16 + col) * LD + kk);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int nt = wave + 4 * u;
      if (nt < nnt) {
        const f16x8 bf = M::lds(Bt + (nt * 16 + col) * LD + kk);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          if (pt < npt) {
            acc[pt][u] = M::mma(ah[pt], bf, acc[pt][u]);
            acc[pt][u] = M::mma(al[pt], bf, acc[pt][u]);
          }
        }
      }
    }
  }
  __syncthreads();
  if (pb == 0 && threadIdx.x == 0)
    logdecay[((int64_t)b * d.H + h) * nr + r] = carry_s;
  float* out = states + (((int64_t)b * nr + r) * d.H + h) * d.P * d.N;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int nt = wave + 4 * u;
    if (nt >= nnt) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt >= npt) continue;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int p = p0 + pt * 16 + 4 * kg + rr;
        out[(int64_t)p * d.N + nt * 16 + col] = acc[pt][u][rr];
      }
    }
  }
}


// ---- F3: fused chunk scan over a run ------------------------------------------------------------
// Grid (nr, H, batch); NW waves. Wave w owns the 16-row output tiles w, w + NW, ... of a chunk
// (all P columns), and the carried-state tiles (n-tile, p-tile) w, w + NW, ... of S^T [N x P].
//
// Per chunk:
//   cumulative decay acs, dt and the state weights w_j = exp(acs_last - acs_j) dt_j (wave 0);
//   the carried state, rounded to fp16, is written to LDS as h^T [p][n] (readout operand);
//   the wave's C rows are loaded once into registers (they are the B operand of C B^T and the A
//   operand of the readout: the same fragment layout);
//   readout y_i = exp(acs_i) C_i . h (matrix cores, K = N) starts each output accumulator;
//   token slabs of SL: B (natural and transposed) and x (transposed) go to LDS; for every K step
//   of 32 tokens the two 16x16 blocks of (C B^T)^T are computed into registers and turned, lane
//   by lane, into the A fragment M[i][j] = CB[i][j] exp(acs_i - acs_j) dt_j (0 for j > i) of the
//   intra-chunk product -- the Q x Q block never leaves registers. The K slots of that fragment
//   follow the accumulator layout (j = jb + 4 kg + r, jb + 16 + 4 kg + r), and the x fragment is
//   read from LDS with the same order;
//   the carried state decays by exp(acs_last) and accumulates B^T (w x) (skipped after the last
//   chunk of the run: the state entering the next run comes from the run-state pass);
//   y = accumulator + D x, rounded once to bf16.
template <int P, int N, int NW, int SL>
__global__ __launch_bounds__(NW * 64) void k_fused_scan(
    const u16* __restrict__ x, const u16* __restrict__ Bm, const u16* __restrict__ Cm,
    const float* __restrict__ dt, const float* __restrict__ Av, const float* __restrict__ Dv,
    const float* __restrict__ h_run, u16* __restrict__ y, Dims d, int S, int nr) {
  using M = Mma<f16>;
  constexpr int NP = P / 16, NN = N / 16;
  constexpr int MAXI = 16 / NW;          // output row tiles per wave (Q <= 256)
  constexpr int TS = NP * NN / NW;       // carried-state tiles per wave
  constexpr int NK = N / 32;             // K steps over the state size
  static_assert(NW % NP == 0, "each wave's state tiles share one p-tile");
  static_assert(N % 32 == 0 && SL % 32 == 0, "tile shape");
  constexpr int LDH = N + 8, LDB = N + 8, LDT = SL + 8;
  __shared__ float acs[256], dts[256], wts[256];
  __shared__ __align__(16) f16 hT[P * LDH];
  __shared__ __align__(16) f16 Bn[SL * LDB];
  __shared__ __align__(16) f16 Bt[N * LDT];
  __shared__ __align__(16) f16 Xt[P * LDT];

  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (d.H / d.G);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int Q = d.Q, nti = Q / 16;
  const float a_h = Av[h], d_h = Dv[h];
  const int c_begin = r * S, c_end = min(d.nc, c_begin + S);
  const int spt = wave % NP;             // this wave's state p-tile
  // Entries past Q are read (as zeros) when Q is shorter than a slab or a 32-token K step.
  for (int i = threadIdx.x; i < 256; i += NW * 64) {
    acs[i] = 0.f;
    dts[i] = 0.f;
    wts[i] = 0.f;
  }

  // carried state S^T tiles: lane holds p = spt*16 + col, n = nt*16 + 4 kg + rr
  f32x4 Sacc[TS];
  {
    const float* hr = h_run + (((int64_t)b * nr + r) * d.H + h) * (int64_t)(P * N);
#pragma unroll
    for (int k = 0; k < TS; ++k) {
      const int nt = (wave + NW * k) / NP;
      const float4 v = *reinterpret_cast<const float4*>(hr + (spt * 16 + col) * N + nt * 16 +
                                                        4 * kg);
      Sacc[k] = f32x4{v.x, v.y, v.z, v.w};
    }
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * Q, q = min(Q, d.L - t0);
    const bool carry = (c + 1) < c_end;
    __syncthreads();  // LDS of the previous chunk fully consumed
    if (wave == 0) {
      const int E = Q >= 64 ? Q / 64 : 1;
      float loc[4], dv[4];
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = lane * E + e;
        float v = 0.f;
        if (e < E && i < q) v = dt[((int64_t)b * d.L + t0 + i) * d.H + h];
        dv[e] = v;
        s += v * a_h;
        loc[e] = s;
      }
      const float incl = wave_inclusive_scan(s);
      float excl = __shfl_up(incl, 1, kWave);
      if (lane == 0) excl = 0.f;
      const int eq = (q - 1) % E;
      float mine = excl + loc[0];
#pragma unroll
      for (int e = 1; e < 4; ++e)
        if (e == eq) mine = excl + loc[e];
      const float vlast = __shfl(mine, (q - 1) / E, kWave);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = lane * E + e;
        if (e < E && i < Q) {
          const float a = (i < q) ? excl + loc[e] : vlast;
          acs[i] = a;
          dts[i] = dv[e];
          wts[i] = (i < q) ? __expf(vlast - a) * dv[e] : 0.f;
        }
      }
    }
    // carried state -> h^T (fp16) for the readout
#pragma unroll
    for (int k = 0; k < TS; ++k) {
      const int nt = (wave + NW * k) / NP;
      f16x4 v4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v4[rr] = (f16)Sacc[k][rr];
      *reinterpret_cast<f16x4*>(hT + (spt * 16 + col) * LDH + nt * 16 + 4 * kg) = v4;
    }
    // this wave's C rows, as fragments (zero past the end of the sequence)
    f16x8 Cf[MAXI][NK];
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = wave + NW * m;
      const int i = ti * 16 + col;
      const bool valid = ti < nti && i < q;
      const u16* crow = Cm + (((int64_t)b * d.L + t0 + i) * d.G + g) * N;
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        f16x8 f = {};
        if (valid) {
          float v[8];
          load8(crow + kn * 32 + 8 * kg, v);
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) f[qq] = (f16)v[qq];
        }
        Cf[m][kn] = f;
      }
    }
    __syncthreads();  // acs, dts, wts, h^T ready

    // readout of the state entering this chunk
    f32x4 Y[MAXI][NP];
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = wave + NW * m;
#pragma unroll
      for (int pt = 0; pt < NP; ++pt) Y[m][pt] = zero4();
      if (ti >= nti) continue;
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
#pragma unroll
        for (int pt = 0; pt < NP; ++pt)
          Y[m][pt] = M::mma(Cf[m][kn], M::lds(hT + (pt * 16 + col) * LDH + kn * 32 + 8 * kg),
                            Y[m][pt]);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float e = __expf(acs[ti * 16 + 4 * kg + rr]);
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) Y[m][pt][rr] *= e;
      }
    }
    if (carry) {
      const float dec = __expf(acs[Q - 1]);
#pragma unroll
      for (int k = 0; k < TS; ++k) Sacc[k] *= dec;
    }

    for (int j0 = 0; j0 < q; j0 += SL) {
      __syncthreads();  // previous slab consumed
      for (int e = threadIdx.x; e < SL * (N / 8); e += NW * 64) {
        const int jj = e / (N / 8), n8 = (e % (N / 8)) * 8;
        const int j = j0 + jj;
        f16x8 f = {};
        if (j < q) {
          float v[8];
          load8(Bm + (((int64_t)b * d.L + t0 + j) * d.G + g) * N + n8, v);
#pragma unroll
          for (int k = 0; k < 8; ++k) f[k] = (f16)v[k];
        }
        *reinterpret_cast<f16x8*>(Bn + jj * LDB + n8) = f;
#pragma unroll
        for (int k = 0; k < 8; ++k) Bt[(n8 + k) * LDT + jj] = f[k];
      }
      for (int e = threadIdx.x; e < SL * (P / 8); e += NW * 64) {
        const int jj = e / (P / 8), p8 = (e % (P / 8)) * 8;
        const int j = j0 + jj;
        float v[8];
        if (j < q) {
          load8(x + (((int64_t)b * d.L + t0 + j) * d.H + h) * P + p8, v);
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) Xt[(p8 + k) * LDT + jj] = (f16)v[k];
      }
      __syncthreads();

      // intra-chunk masked product for this slab
#pragma unroll
      for (int m = 0; m < MAXI; ++m) {
        const int ti = wave + NW * m;
        if (ti >= nti) continue;
        const int imax = ti * 16 + 15;
        const int i = ti * 16 + col;
        const float acs_i = acs[i];
#pragma unroll
        for (int ks = 0; ks < SL / 32; ++ks) {
          const int jbase = j0 + ks * 32;
          if (jbase > imax) break;
          const bool second = jbase + 16 <= imax;
          f32x4 c0 = zero4(), c1 = zero4();
          const f16* b0 = Bn + (jbase - j0 + col) * LDB + 8 * kg;
#pragma unroll
          for (int kn = 0; kn < NK; ++kn) {
            c0 = M::mma(M::lds(b0 + kn * 32), Cf[m][kn], c0);
            if (second) c1 = M::mma(M::lds(b0 + 16 * LDB + kn * 32), Cf[m][kn], c1);
          }
          f16x8 mf;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int j = jbase + 4 * kg + rr;
            const float v = c0[rr] * __expf(acs_i - acs[j]) * dts[j];
            mf[rr] = (f16)((j <= i) ? v : 0.f);
            const int j2 = j + 16;
            const float v2 = c1[rr] * __expf(acs_i - acs[j2]) * dts[j2];
            mf[4 + rr] = (f16)((j2 <= i) ? v2 : 0.f);
          }
#pragma unroll
          for (int pt = 0; pt < NP; ++pt) {
            const f16* xp = Xt + (pt * 16 + col) * LDT + (jbase - j0) + 4 * kg;
            const f16x4 lo = *reinterpret_cast<const f16x4*>(xp);
            const f16x4 hi = *reinterpret_cast<const f16x4*>(xp + 16);
            const f16x8 xf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            Y[m][pt] = M::mma(mf, xf, Y[m][pt]);
          }
        }
      }
      // carried-state update with this slab
      if (carry) {
#pragma unroll
        for (int ks = 0; ks < SL / 32; ++ks) {
          const int jb = ks * 32 + 8 * kg;  // slab-local first token of this lane's K slice
          const f16x8 xv = M::lds(Xt + (spt * 16 + col) * LDT + jb);
          f16x8 wf;
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) wf[qq] = (f16)((float)xv[qq] * wts[j0 + jb + qq]);
#pragma unroll
          for (int k = 0; k < TS; ++k) {
            const int nt = (wave + NW * k) / NP;
            Sacc[k] = M::mma(M::lds(Bt + (nt * 16 + col) * LDT + jb), wf, Sacc[k]);
          }
        }
      }
    }

    // y = accumulator + D x, rounded once to bf16
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = wave + NW * m;
      if (ti >= nti) continue;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = ti * 16 + 4 * kg + rr;
        if (i >= q) continue;
        const int64_t row = (((int64_t)b * d.L + t0 + i) * d.H + h) * P;
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) {
          const int p = pt * 16 + col;
          y[row + p] = f32_to_bf16(Y[m][pt][rr] + d_h * bf16_to_f32(x[row + p]));
        }
      }
    }
  }
}

// ---- launchers ----------------------------------------------------------------------------------
hipError_t launch_run_state(const Dims& d, const void* x, const void* B, const float* dt,
                            const float* A, int run_len, int nr, float* states, float* logdecay,
                            hipStream_t s) {
  dim3 grid(nr * ((d.P + 63) / 64), d.H, d.Bt);
  hipLaunchKernelGGL(k_run_state, grid, dim3(256), 0, s, (const u16*)x, (const u16*)B, dt, A,
                     states, logdecay, d, run_len, nr);
  return hipGetLastError();
}

template <int P, int N, int NW, int SL>
static hipError_t fused_impl(const Dims& d, const void* x, const void* B, const void* C,
                             const float* dt, const float* A, const float* D, const float* h_run,
                             void* y, int S, int nr, hipStream_t s) {
  dim3 grid(nr, d.H, d.Bt);
  hipLaunchKernelGGL((k_fused_scan<P, N, NW, SL>), grid, dim3(NW * 64), 0, s, (const u16*)x,
                     (const u16*)B, (const u16*)C, dt, A, D, h_run, (u16*)y, d, S, nr);
  return hipGetLastError();
}

bool fused_supported(const Dims& d) {
  return (d.P == 64 && (d.N == 64 || d.N == 128)) || (d.P == 128 && (d.N == 128 || d.N == 256));
}

hipError_t launch_fused_scan(const Dims& d, const void* x, const void* B, const void* C,
                             const float* dt, const float* A, const float* D,
                             const float* h_run, void* y, int S, int nr, hipStream_t s) {
  if (d.P == 64 && d.N == 64)
    return fused_impl<64, 64, 4, 64>(d, x, B, C, dt, A, D, h_run, y, S, nr, s);
  if (d.P == 64 && d.N == 128)
    return fused_impl<64, 128, 4, 64>(d, x, B, C, dt, A, D, h_run, y, S, nr, s);
  if (d.P == 128 && d.N == 128)
    return fused_impl<128, 128, 8, 64>(d, x, B, C, dt, A, D, h_run, y, S, nr, s);
  if (d.P == 128 && d.N == 256)
    return fused_impl<128, 256, 8, 32>(d, x, B, C, dt, A, D, h_run, y, S, nr, s);
  return hipErrorInvalidValue;
}

}  // namespace ssd
