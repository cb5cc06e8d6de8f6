// Unfused SSD chunked forward: five kernels with their intermediates in workspace.
//
// The stages follow the chunked algorithm's order ("Mamba-2 in NVIDIA cuTile: Faster Forward
// Kernels and What the Benchmark Means", section "Why Mamba-2 is a useful kernel example"):
// cumulative decay per chunk, the state entering each chunk, then the outputs, with the
// quadratic masked form inside a chunk and a linear recurrence across chunks ("nitter.gq/da_be19"
// thread, post 5/6). Layouts of the intermediates are given in include/ssd.h.
//
// Matrix-core use: C B^T (contraction over the state size), the chunk states (over the tokens of
// a chunk), the masked intra-chunk product (over the tokens) and the inter-chunk readout (over
// the state size) run on 16x16 MFMA tiles; the cumulative sum, decays and masks run on VALU.
#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// =============================================================================================
// Stage 1: per-chunk inclusive cumulative sum of dt*A.
// Grid (nc, ceil(H/16), batch), 256 threads. A block stages dt[b, chunk, h0:h0+16] (coalesced
// 64-byte rows) in LDS; each wave then scans one head at a time, a lane holding Q/64 consecutive
// tokens (one token when Q < 64), with a wave-shuffle scan over lane totals.
// =============================================================================================
__global__ __launch_bounds__(256) void k_chunk_cumsum(const float* __restrict__ dt,
                                                      const float* __restrict__ A,
                                                      float* __restrict__ Acs,
                                                      float* __restrict__ dtc, Dims d) {
  __shared__ float tile[256][17];
  const int c = blockIdx.x, h0 = blockIdx.y * 16, b = blockIdx.z;
  const int t0 = c * d.Q;
  const int q = min(d.Q, d.L - t0);
  for (int e = threadIdx.x; e < d.Q * 16; e += 256) {
    const int i = e >> 4, hh = e & 15, h = h0 + hh;
    float v = 0.f;
    if (i < q && h < d.H)
      v = dt_effective(dt[((int64_t)b * d.L + t0 + i) * d.H + h], dt_bias_of(d, h), d);
    tile[i][hh] = v;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = d.Q >= 64 ? d.Q / 64 : 1;
  for (int hh = wave; hh < 16; hh += 4) {
    const int h = h0 + hh;
    if (h >= d.H) break;
    const float a = A[h];
    float loc[4];
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = lane * E + e;
      if (e < E && i < d.Q) s += tile[i][hh] * a;
      loc[e] = s;
    }
    const float incl = wave_inclusive_scan(s);
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.f;
    // Past a ragged end the value is an exact copy of the last valid one (the shuffle scan
    // would otherwise re-associate the same sum there).
    const int eq = (q - 1) % E;
    float mine = excl + loc[0];
#pragma unroll
    for (int e = 1; e < 4; ++e)
      if (e == eq) mine = excl + loc[e];
    const float vlast = __shfl(mine, (q - 1) / E, kWave);
    const int64_t base = (((int64_t)b * d.H + h) * d.nc + c) * d.Q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = lane * E + e;
      if (e < E && i < d.Q) {
        Acs[base + i] = (i < q) ? excl + loc[e] : vlast;
        dtc[base + i] = (d.unit_input && i < q) ? 1.f : tile[i][hh];
      }
    }
  }
}

// Load KPL consecutive io values starting at element `off` as a compute-type fragment; zero when
// `valid` is false.
template <typename IO, typename T> struct FragLoad;
template <> struct FragLoad<u16, f16> {
  static __device__ __forceinline__ f16x8 load(const u16* p, int64_t off, bool valid) {
    f16x8 r = {};
    if (valid) {
      float v[8];
      load8(p + off, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q] = (f16)v[q];
    }
    return r;
  }
};
template <> struct FragLoad<float, float> {
  static __device__ __forceinline__ float load(const float* p, int64_t off, bool valid) {
    return valid ? p[off] : 0.f;
  }
};
template <> struct FragLoad<u16, float> {
  static __device__ __forceinline__ float load(const u16* p, int64_t off, bool valid) {
    return valid ? bf16_to_f32(p[off]) : 0.f;
  }
};

// =============================================================================================
// Stage 2: CB[b, c, g, i, j] = C_i . B_j for the 16x16 blocks on or below the block diagonal.
// Grid (nc, G, batch), 256 threads; the blocks of the chunk's lower triangle are dealt to the
// four waves. Operands come straight from global memory (rows of C and B are contiguous along
// the contraction index, the layout the matrix-core fragments want).
// =============================================================================================
template <typename IO, typename T>
__global__ __launch_bounds__(256) void k_bmm_chunk(const IO* __restrict__ Bm,
                                                   const IO* __restrict__ Cm,
                                                   float* __restrict__ CB, Dims d) {
  using M = Mma<T>;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t0 = c * d.Q, q = min(d.Q, d.L - t0);
  const int nt = d.Q / 16, ntiles = nt * (nt + 1) / 2;
  const int64_t rowstride = (int64_t)d.G * d.N;
  const int64_t gbase = ((int64_t)b * d.L + t0) * rowstride + (int64_t)g * d.N;
  float* out = CB + (((int64_t)b * d.nc + c) * d.G + g) * d.Q * d.Q;
  for (int k = wave; k < ntiles; k += 4) {
    int ti = (int)((sqrtf(8.f * k + 1.f) - 1.f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= k) ++ti;
    while (ti * (ti + 1) / 2 > k) --ti;
    const int tj = k - ti * (ti + 1) / 2;
    const int ia = ti * 16 + col;  // row of C this lane feeds
    const int jb = tj * 16 + col;  // row of B this lane feeds
    f32x4 acc = zero4();
    if constexpr (sizeof(T) == 4) {
      // fp32: 8 K steps of operands loaded together from clamped rows, zeroed past the chunk
      constexpr int GK = 8;
      const int64_t arow = gbase + min(ia, q - 1) * rowstride;
      const int64_t brow = gbase + min(jb, q - 1) * rowstride;
      for (int k00 = 0; k00 < d.N; k00 += GK * M::KSTEP) {
        float av[GK], bv[GK];
#pragma unroll
        for (int s = 0; s < GK; ++s) {
          const int nc = min(k00 + s * M::KSTEP + kg, d.N - 1);
          av[s] = Io<IO>::load(Cm, arow + nc);
          bv[s] = Io<IO>::load(Bm, brow + nc);
        }
#pragma unroll
        for (int s = 0; s < GK; ++s) {
          const int n = k00 + s * M::KSTEP + kg;
          if (k00 + s * M::KSTEP < d.N)
            acc = M::mma(ia < q && n < d.N ? av[s] : 0.f, jb < q && n < d.N ? bv[s] : 0.f, acc);
        }
      }
    } else {
      for (int k0 = 0; k0 < d.N; k0 += M::KSTEP) {
        const int n = k0 + M::KPL * kg;
        // n < N also guards the 32-wide fp16 K step when N is a multiple of 16 only
        auto a = FragLoad<IO, T>::load(Cm, gbase + ia * rowstride + n, ia < q && n < d.N);
        auto bb = FragLoad<IO, T>::load(Bm, gbase + jb * rowstride + n, jb < q && n < d.N);
        acc = M::mma(a, bb, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ti * 16 + 4 * kg + r;
      out[(int64_t)i * d.Q + jb] = acc[r];
    }
  }
}

// Stage 2 for fp32 io with chunks of at most 64 tokens and dstate at most 128: the chunk's C and
// B rows are staged in LDS once per block ([Q][N + 4] floats each: 16-byte rows, and the 16 rows
// of a fragment fall in distinct banks; rows past the sequence are zero), then every 16x16 block
// is computed from LDS. Each row serves up to four blocks of the lower triangle, which the
// global-memory version reads once per block.
template <typename IO>
__global__ __launch_bounds__(256) void k_bmm_chunk_lds(const IO* __restrict__ Bm,
                                                       const IO* __restrict__ Cm,
                                                       float* __restrict__ CB, Dims d) {
  using M = Mma<float>;
  extern __shared__ __align__(16) float sm_bmm[];
  const int ldn = d.N + 4;
  float* Cs = sm_bmm;
  float* Bs = sm_bmm + d.Q * ldn;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t0 = c * d.Q, q = min(d.Q, d.L - t0);
  const int64_t rowstride = (int64_t)d.G * d.N;
  const int64_t gbase = ((int64_t)b * d.L + t0) * rowstride + (int64_t)g * d.N;
  {
    // up to 64 rows x 128 floats per operand: thread = (float4 column tid % 32, rows tid / 32
    // + 8 u), 8 float4 per operand, all loads issued first from clamped rows and columns
    const int nv4 = d.N / 4, c4 = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int c4c = min(c4, nv4 - 1);
    float4 vc[8], vb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t o = gbase + (int64_t)min(r0 + 8 * u, q - 1) * rowstride + 4 * c4c;
      if constexpr (sizeof(IO) == 2) {  // bf16: four values in 8 bytes, widened exactly
        const uint2 c2 = *reinterpret_cast<const uint2*>(Cm + o);
        const uint2 b2 = *reinterpret_cast<const uint2*>(Bm + o);
        vc[u] = make_float4(__uint_as_float(c2.x << 16), __uint_as_float(c2.x & 0xffff0000u),
                            __uint_as_float(c2.y << 16), __uint_as_float(c2.y & 0xffff0000u));
        vb[u] = make_float4(__uint_as_float(b2.x << 16), __uint_as_float(b2.x & 0xffff0000u),
                            __uint_as_float(b2.y << 16), __uint_as_float(b2.y & 0xffff0000u));
      } else {
        vc[u] = *reinterpret_cast<const float4*>(Cm + o);
        vb[u] = *reinterpret_cast<const float4*>(Bm + o);
      }
    }
    // rows past the sequence are zeroed component by component (a select between two float4
    // values would become a load through a selected pointer, which puts the arrays in scratch)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + 8 * u;
      if (c4 < nv4 && r < d.Q) {
        const bool in = r < q;
        const float4 c = vc[u], bv = vb[u];
        *reinterpret_cast<float4*>(Cs + r * ldn + 4 * c4) =
            make_float4(in ? c.x : 0.f, in ? c.y : 0.f, in ? c.z : 0.f, in ? c.w : 0.f);
        *reinterpret_cast<float4*>(Bs + r * ldn + 4 * c4) =
            make_float4(in ? bv.x : 0.f, in ? bv.y : 0.f, in ? bv.z : 0.f, in ? bv.w : 0.f);
      }
    }
  }
  __syncthreads();
  const int nt = d.Q / 16, ntiles = nt * (nt + 1) / 2;
  float* out = CB + (((int64_t)b * d.nc + c) * d.G + g) * d.Q * d.Q;
  for (int k = wave; k < ntiles; k += 4) {
    int ti = (int)((sqrtf(8.f * k + 1.f) - 1.f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= k) ++ti;
    while (ti * (ti + 1) / 2 > k) --ti;
    const int tj = k - ti * (ti + 1) / 2;
    const float* ca = Cs + (ti * 16 + col) * ldn + kg;
    const float* bb = Bs + (tj * 16 + col) * ldn + kg;
    f32x4 acc = zero4();
#pragma unroll 8
    for (int k0 = 0; k0 < d.N; k0 += M::KSTEP) acc = M::mma(ca[k0], bb[k0], acc);
    const int jb = tj * 16 + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(int64_t)(ti * 16 + 4 * kg + r) * d.Q + jb] = acc[r];
  }
}

// =============================================================================================
// Stage 3: states[b, c, h, p, n] = sum_j w_j x[j, p] B[j, n], w_j = exp(Acs_last - Acs_j) dt_j.
// Grid (nc * ceil(P/64), H, batch), 256 threads. Tokens are taken in slabs of SJ = 32; each slab
// stages W^T [p][j] (optionally split hi + lo) and B^T [n][j] in LDS so both fragments read
// contiguous K. Wave w owns the n-tiles w, w+4, ... of the block's (up to) four p-tiles.
// =============================================================================================
constexpr int SJ = 32;

// The x row of head h: one per head, or shared by the heads of a group when d.x_groups > 0.
struct XRow {
  int n, row;  // x rows per token, this head's row
  __device__ XRow(const Dims& d, int h)
      : n(d.x_groups ? d.x_groups : d.H), row(d.x_groups ? h / (d.H / d.x_groups) : h) {}
};

template <typename T> struct Pad { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 1; };

// NU: n-tile slots per wave (wave w takes n-tiles w, w + 4, ...; dstate <= 64 NU)
template <typename IO, typename T, bool HILO, int NU>
__global__ __launch_bounds__(256) void k_chunk_state(const IO* __restrict__ x,
                                                     const IO* __restrict__ Bm,
                                                     const float* __restrict__ Acs,
                                                     const float* __restrict__ dtc,
                                                     float* __restrict__ states, Dims d) {
  using M = Mma<T>;
  constexpr int LD = SJ + Pad<T>::v;
  extern __shared__ __align__(16) unsigned char smem[];
  const int npb = (d.P + 63) / 64;
  const int c = blockIdx.x / npb, pb = blockIdx.x % npb, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (d.H / d.G);
  const XRow xh(d, h);
  const int p0 = pb * 64, np = min(64, d.P - p0);
  T* Wh = reinterpret_cast<T*>(smem);
  T* Wl = Wh + 64 * LD;
  T* Bt = Wl + (HILO ? 64 * LD : 0);
  float* w = reinterpret_cast<float*>(Bt + d.N * LD);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t0 = c * d.Q, q = min(d.Q, d.L - t0);
  const int64_t abase = (((int64_t)b * d.H + h) * d.nc + c) * d.Q;
  const float alast = Acs[abase + d.Q - 1];
  const int npt = np / 16, nnt = d.N / 16;

  f32x4 acc[4][NU];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NU; ++j) acc[i][j] = zero4();

  for (int j0 = 0; j0 < d.Q; j0 += SJ) {
    if (threadIdx.x < SJ) {
      const int j = j0 + threadIdx.x;
      w[threadIdx.x] = (j < q) ? __expf(alast - Acs[abase + j]) * dtc[abase + j] : 0.f;
    }
    __syncthreads();
    // W^T slab: 8 consecutive p of one token per thread-iteration.
    for (int e = threadIdx.x; e < SJ * (np / 8); e += 256) {
      const int jj = e / (np / 8), p8 = (e % (np / 8)) * 8;
      const int j = j0 + jj;
      float v[8];
      if (j < q) {
        const int64_t off = ((((int64_t)b * d.L + t0 + j) * xh.n + xh.row) * d.P) + p0 + p8;
        if constexpr (sizeof(IO) == 2) load8(reinterpret_cast<const u16*>(x) + off, v);
        else load8(reinterpret_cast<const float*>(x) + off, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
      const float wj = w[jj];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float val = v[k] * wj;
        const T hi = (T)val;
        Wh[(p8 + k) * LD + jj] = hi;
        if constexpr (HILO) Wl[(p8 + k) * LD + jj] = (T)(val - (float)hi);
      }
    }
    // B^T slab.
    for (int e = threadIdx.x; e < SJ * (d.N / 8); e += 256) {
      const int jj = e / (d.N / 8), n8 = (e % (d.N / 8)) * 8;
      const int j = j0 + jj;
      float v[8];
      if (j < q) {
        const int64_t off = (((int64_t)b * d.L + t0 + j) * d.G + g) * d.N + n8;
        if constexpr (sizeof(IO) == 2) load8(reinterpret_cast<const u16*>(Bm) + off, v);
        else load8(reinterpret_cast<const float*>(Bm) + off, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) Bt[(n8 + k) * LD + jj] = (T)v[k];
    }
    __syncthreads();
    for (int k0 = 0; k0 < SJ; k0 += M::KSTEP) {
      const int kk = k0 + M::KPL * kg;
      typename M::Frag ah[4], al[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt < npt) {
          ah[pt] = M::lds(Wh + (pt * 16 + col) * LD + kk);
          if constexpr (HILO) al[pt] = M::lds(Wl + (pt * 16 + col) * LD + kk);
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int nt = wave + 4 * u;
        if (nt < nnt) {
          const typename M::Frag bf = M::lds(Bt + (nt * 16 + col) * LD + kk);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            if (pt < npt) {
              acc[pt][u] = M::mma(ah[pt], bf, acc[pt][u]);
              if constexpr (HILO) acc[pt][u] = M::mma(al[pt], bf, acc[pt][u]);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  float* out = states + (((int64_t)b * d.nc + c) * d.H + h) * d.P * d.N;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int nt = wave + 4 * u;
    if (nt >= nnt) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt >= npt) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = p0 + pt * 16 + 4 * kg + r;
        out[(int64_t)p * d.N + nt * 16 + col] = acc[pt][u][r];
      }
    }
  }
}

// =============================================================================================
// Stage 4: state entering each step of a chain of segments (chunks, or runs of chunks):
//   h_in[0] = h0 (or 0);  h_in[s+1] = exp(logdecay[s]) h_in[s] + states[s];  final = h_in[nsteps].
// logdecay of (b, h, step s) is read at ld[(b*H + h)*ld_bh + s*ld_step] (for chunks: the last
// element of each chunk's cumulative sum). Grid (ceil(P*N/1024), H, batch), 256 threads, 4
// consecutive state entries per thread; the step loop is sequential per entry, and the loads of
// later steps do not depend on the carry.
// =============================================================================================
__global__ __launch_bounds__(256) void k_state_passing(const float* __restrict__ states,
                                                       const float* __restrict__ ld,
                                                       int64_t ld_bh, int64_t ld_step,
                                                       const float* __restrict__ h0,
                                                       float* __restrict__ h_in,
                                                       float* __restrict__ fin, Dims d,
                                                       int nsteps) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int PN = d.P * d.N;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= PN) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t sb = ((int64_t)b * d.H + h) * PN + e;
  if (h0) s = *reinterpret_cast<const float4*>(h0 + sb);
  const float* ldp = ld + ((int64_t)b * d.H + h) * ld_bh;
  const int64_t cstride = (int64_t)d.H * PN;
  const int64_t off0 = ((int64_t)b * nsteps * d.H + h) * PN + e;
  // 8 steps' states and decays loaded together (clamped to the last step), then the chain: only
  // the multiply-adds depend on the step before
  constexpr int GS = 8;
  for (int c0 = 0; c0 < nsteps; c0 += GS) {
    float4 st[GS];
    float a[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int c = min(c0 + u, nsteps - 1);
      st[u] = *reinterpret_cast<const float4*>(states + off0 + c * cstride);
      a[u] = ldp[(int64_t)c * ld_step];
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      if (c0 + u < nsteps) {
        if (h_in) *reinterpret_cast<float4*>(h_in + off0 + (c0 + u) * cstride) = s;
        const float dec = __expf(a[u]);
        s.x = dec * s.x + st[u].x;
        s.y = dec * s.y + st[u].y;
        s.z = dec * s.z + st[u].z;
        s.w = dec * s.w + st[u].w;
      }
    }
  }
  if (fin) *reinterpret_cast<float4*>(fin + sb) = s;
}

// Whether the chunk scan stages the entering state in LDS (the block's rows, at most 64, of
// N + 4 floats within 96 KB).
__host__ __device__ inline bool scan_state_in_lds(const Dims& d) {
  return (int64_t)min(d.P, 64) * (d.N + 4) * 4 <= 96 * 1024;
}

// =============================================================================================
// Stage 5: y = intra + exp(Acs_i) * (C_i . h_in) + D x, fp16 operands (bf16 io; fp32 arithmetic
// is k_chunk_scan_f32 below).
// Grid (nc * ceil(Q/64) * ceil(P/64), H, batch), 256 threads; a block takes 64 rows and 64
// columns of headdim (wave w 16 rows of them: four 16x16 accumulator tiles for each of the
// intra and inter parts).
// intra: for each K step over j <= i, the A fragment M[i][j] = CB[i][j] exp(Acs_i - Acs_j) dt_j
// (selected to 0 for j > i) is formed in registers straight from CB; X^T slabs [p][j] are staged
// in LDS. inter: C rows and h_in rows are read from global memory (both contiguous along n).
// =============================================================================================
template <typename IO, typename T>
__global__ __launch_bounds__(256) void k_chunk_scan(
    const IO* __restrict__ x, const IO* __restrict__ Cm, const float* __restrict__ CB,
    const float* __restrict__ Acs, const float* __restrict__ dtc,
    const float* __restrict__ h_in, const float* __restrict__ Dv, IO* __restrict__ y, Dims d) {
  using M = Mma<T>;
  constexpr int SX = (sizeof(T) == 2) ? 64 : 32;  // tokens per staged X slab
  constexpr int LD = SX + Pad<T>::v;
  extern __shared__ __align__(16) unsigned char smem[];
  float* acs = reinterpret_cast<float*>(smem);
  float* dts = acs + 256;
  T* Xs = reinterpret_cast<T*>(dts + 256);

  constexpr int NPT = 4;  // 16-column tiles of the block's 64 columns
  const int nib = (d.Q + 63) / 64, npb = (d.P + 63) / 64;
  const int c = blockIdx.x / (nib * npb), ib = (blockIdx.x / npb) % nib, pb = blockIdx.x % npb;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (d.H / d.G);
  const XRow xh(d, h);
  const int p0 = pb * 64, np = min(64, d.P - p0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t0 = c * d.Q, q = min(d.Q, d.L - t0);
  const int i0 = ib * 64 + wave * 16;           // first row of this wave
  const bool active = i0 < d.Q;
  const int rowmax_blk = min(ib * 64 + 63, d.Q - 1);
  const int64_t abase = (((int64_t)b * d.H + h) * d.nc + c) * d.Q;
  for (int i = threadIdx.x; i < d.Q; i += 256) {
    acs[i] = Acs[abase + i];
    dts[i] = dtc[abase + i];
  }
  const int npt = np / 16;
  f32x4 acc[NPT], inter[NPT];
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) { acc[pt] = zero4(); inter[pt] = zero4(); }
  const float* cb = CB + (((int64_t)b * d.nc + c) * d.G + g) * d.Q * d.Q;
  const int ia = i0 + col;  // row this lane feeds into A fragments
  __syncthreads();

  for (int j0 = 0; j0 <= rowmax_blk; j0 += SX) {
    const int sx = min(SX, d.Q - j0);
    // Stage all SX columns: those past the chunk (or past Q when Q < one K step) are zeros, so
    // every fragment read below sees finite values.
    for (int e = threadIdx.x; e < SX * (np / 8); e += 256) {
      const int jj = e / (np / 8), p8 = (e % (np / 8)) * 8;
      const int j = j0 + jj;
      float v[8];
      if (j < q) {
        const int64_t off = (((int64_t)b * d.L + t0 + j) * xh.n + xh.row) * d.P + p0 + p8;
        if constexpr (sizeof(IO) == 2) load8(reinterpret_cast<const u16*>(x) + off, v);
        else load8(reinterpret_cast<const float*>(x) + off, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) Xs[(p8 + k) * LD + jj] = (T)v[k];
    }
    __syncthreads();
    static_assert(sizeof(T) == 2, "fp32 arithmetic: k_chunk_scan_f32");
    if (active) {
      for (int k0 = 0; k0 < sx && j0 + k0 <= i0 + 15; k0 += M::KSTEP) {
        const int jb = j0 + k0 + M::KPL * kg;  // first j of this lane's K slice
        typename M::Frag a;
        {
          float cv[8];
          if (jb < d.Q) {
            load8(cb + (int64_t)ia * d.Q + jb, cv);
          } else {
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) cv[qq] = 0.f;
          }
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) {
            const int j = jb + qq;
            const float m = cv[qq] * __expf(acs[ia] - acs[j]) * dts[j];
            a[qq] = (T)((j <= ia) ? m : 0.f);
          }
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          if (pt < npt) acc[pt] = M::mma(a, M::lds(Xs + (pt * 16 + col) * LD + k0 + M::KPL * kg),
                                         acc[pt]);
      }
    }
    __syncthreads();
  }
  // inter-chunk readout: C_i . h_in[p, :]
  const float* hb = h_in + ((((int64_t)b * d.nc + c) * d.H + h) * d.P + p0) * d.N;  // row p0
  // The chunk's entering state, staged once for the block's waves over the X slabs (no longer
  // read), rows p padded by 4 floats so the 16 rows of a fragment read fall in distinct banks.
  // Too large a state (P (N + 4) floats past the budget) is read from global memory instead.
  const bool hlds = scan_state_in_lds(d);
  const int ldh = d.N + 4;
  float* Hs = reinterpret_cast<float*>(Xs);
  if (hlds) {
    // 8 float4 loads per thread in flight at a time (clamped; the extra ones are not stored)
    const int nv = np * d.N / 4;
    for (int e0 = threadIdx.x; e0 < nv; e0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(hb + 4 * min(e0 + 256 * u, nv - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 4 * (e0 + 256 * u);
        if (e0 + 256 * u < nv) *reinterpret_cast<float4*>(Hs + (e / d.N) * ldh + e % d.N) = v[u];
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const int64_t crow = (((int64_t)b * d.L + t0 + ia) * d.G + g) * d.N;
  for (int k0 = 0; k0 < d.N; k0 += M::KSTEP) {
    const int n = k0 + M::KPL * kg;
    const bool nvalid = n < d.N;  // the fp16 K step is 32 wide, N only a multiple of 16
    const auto a = FragLoad<IO, T>::load(Cm, crow + n, ia < q && nvalid);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      if (pt < npt) {
        typename M::Frag bf;
        const float* hp = hlds ? Hs + (pt * 16 + col) * ldh + n
                               : hb + (int64_t)(pt * 16 + col) * d.N + n;
        {
          float hv[8];
          if (nvalid) {
            load8(hp, hv);
          } else {
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) hv[qq] = 0.f;
          }
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) bf[qq] = (T)hv[qq];
        }
        inter[pt] = M::mma(a, bf, inter[pt]);
      }
    }
  }
  const float dh = Dv[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * kg + r;
    if (i >= q) continue;
    const float e = __expf(acs[i]);
    const int64_t row = (((int64_t)b * d.L + t0 + i) * d.H + h) * d.P;
    const int64_t xrow = (((int64_t)b * d.L + t0 + i) * xh.n + xh.row) * d.P;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      if (pt < npt) {
        const int p = p0 + pt * 16 + col;
        const float xv = Io<IO>::load(x, xrow + p);
        Io<IO>::store(y, row + p, acc[pt][r] + e * inter[pt][r] + dh * xv);
      }
    }
  }
}

// Four consecutive io values as floats (16 bytes of fp32 or 8 of bf16, aligned).
__device__ __forceinline__ float4 load4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4f(const u16* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ float at4(const float4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Stage 5 in fp32 (fp32 matrix cores, 16 x 16 x 4): the same grid and tiles as k_chunk_scan, with
// the K index of every group of four matrix-core steps running over 16 consecutive positions, lane
// group kg taking positions 4 kg .. 4 kg + 3 (one per step): every operand a lane feeds is then 16
// contiguous bytes, one 16-byte load per group of four steps (C and C B^T rows from global memory,
// the decay arrays, the X^T slab and the entering state from LDS) instead of four scalar loads.
// The X slab is staged transposed ([p][j]) through registers, 4 tokens x 4 columns per thread.
template <typename IO>
__global__ __launch_bounds__(256) void k_chunk_scan_f32(
    const IO* __restrict__ x, const IO* __restrict__ Cm, const float* __restrict__ CB,
    const float* __restrict__ Acs, const float* __restrict__ dtc,
    const float* __restrict__ h_in, const float* __restrict__ Dv, IO* __restrict__ y, Dims d) {
  using M = Mma<float>;
  constexpr int SX = 32, LDX = SX + 4;  // tokens per staged X slab; its rows [p][j], 16-byte aligned
  extern __shared__ __align__(16) unsigned char smem[];
  float* acs = reinterpret_cast<float*>(smem);
  float* dts = acs + 256;
  float* Xs = dts + 256;

  constexpr int NPT = 4;
  const int nib = (d.Q + 63) / 64, npb = (d.P + 63) / 64;
  const int c = blockIdx.x / (nib * npb), ib = (blockIdx.x / npb) % nib, pb = blockIdx.x % npb;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (d.H / d.G);
  const XRow xh(d, h);
  const int p0 = pb * 64, np = min(64, d.P - p0), npt = np / 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int t0 = c * d.Q, q = min(d.Q, d.L - t0);
  const int i0 = ib * 64 + wave * 16;
  const bool active = i0 < d.Q;
  const int rowmax_blk = min(ib * 64 + 63, d.Q - 1);
  const int64_t abase = (((int64_t)b * d.H + h) * d.nc + c) * d.Q;
  for (int i = threadIdx.x; i < d.Q; i += 256) {
    acs[i] = Acs[abase + i];
    dts[i] = dtc[abase + i];
  }
  f32x4 acc[NPT], inter[NPT];
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) { acc[pt] = zero4(); inter[pt] = zero4(); }
  const float* cb = CB + (((int64_t)b * d.nc + c) * d.G + g) * d.Q * d.Q;
  const int ia = i0 + col;
  __syncthreads();

  for (int j0 = 0; j0 <= rowmax_blk; j0 += SX) {
    // stage X^T: thread e takes columns 4 (e % (np/4)) .. + 3 of tokens 4 (e / (np/4)) .. + 3
    // (zeros past the chunk)
    {
      const int e = threadIdx.x, nc4 = np / 4;
      if (e < nc4 * (SX / 4)) {
        const int pc = 4 * (e % nc4), jj = 4 * (e / nc4);
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = j0 + jj + k;
          v[k] = j < q ? load4f(x + (((int64_t)b * d.L + t0 + j) * xh.n + xh.row) * d.P + p0 + pc)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(Xs + (pc + r) * LDX + jj) =
              make_float4(at4(v[0], r), at4(v[1], r), at4(v[2], r), at4(v[3], r));
      }
    }
    __syncthreads();
    if (active) {
      const float acs_i = acs[ia];
#pragma unroll
      for (int u = 0; u < SX / 16; ++u) {
        const int jb = j0 + 16 * u;  // first position of the group (wave-uniform)
        if (jb > i0 + 15 || jb >= d.Q) break;
        const int j = jb + 4 * kg;   // this lane's four positions j .. j + 3
        float m[4];
        if (j < d.Q) {
          const float4 cv = *reinterpret_cast<const float4*>(cb + (int64_t)ia * d.Q + j);
          const float4 av = *reinterpret_cast<const float4*>(acs + j);
          const float4 dv = *reinterpret_cast<const float4*>(dts + j);
#pragma unroll
          for (int v = 0; v < 4; ++v)
            m[v] = (j + v <= ia) ? at4(cv, v) * __expf(acs_i - at4(av, v)) * at4(dv, v) : 0.f;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) m[v] = 0.f;
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          if (pt < npt) {
            const float4 xb =
                *reinterpret_cast<const float4*>(Xs + (pt * 16 + col) * LDX + 16 * u + 4 * kg);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[pt] = M::mma(m[v], at4(xb, v), acc[pt]);
          }
        }
      }
    }
    __syncthreads();
  }
  // inter-chunk readout: C_i . h_in[p, :], the state staged in LDS (rows padded by 4 floats) when
  // it fits the budget, else read from global memory
  const float* hb = h_in + ((((int64_t)b * d.nc + c) * d.H + h) * d.P + p0) * d.N;
  const bool hlds = scan_state_in_lds(d);
  const int ldh = d.N + 4;
  float* Hs = Xs;
  if (d.hin_transposed) {
    // rows p0 .. p0 + np - 1 of the state from its transpose [N][P]: 16-byte loads along p,
    // four rows' entries per load (the host guarantees the LDS staging)
    const float* ht = h_in + (((int64_t)b * d.nc + c) * d.H + h) * d.P * d.N;
    const int nq = np / 4, nv = nq * d.N;
    for (int e0 = threadIdx.x; e0 < nv; e0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = min(e0 + 256 * u, nv - 1);
        v[u] = *reinterpret_cast<const float4*>(ht + (int64_t)(e / nq) * d.P + p0 + 4 * (e % nq));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 256 * u;
        if (e < nv) {
          float* o = Hs + (4 * (e % nq)) * ldh + e / nq;
          o[0] = v[u].x;
          o[ldh] = v[u].y;
          o[2 * ldh] = v[u].z;
          o[3 * ldh] = v[u].w;
        }
      }
    }
    __syncthreads();
  } else if (hlds) {
    const int nv = np * d.N / 4;
    for (int e0 = threadIdx.x; e0 < nv; e0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(hb + 4 * min(e0 + 256 * u, nv - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 4 * (e0 + 256 * u);
        if (e0 + 256 * u < nv) *reinterpret_cast<float4*>(Hs + (e / d.N) * ldh + e % d.N) = v[u];
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const bool iv = ia < q;
  const IO* crow = Cm + (((int64_t)b * d.L + t0 + min(ia, q - 1)) * d.G + g) * d.N;
  auto readout = [&](const float* hs, int ldr) {
    for (int n0 = 0; n0 < d.N; n0 += 16) {
      const int n = n0 + 4 * kg;
      const float4 cv = iv ? load4f(crow + n) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        if (pt < npt) {
          const float4 hv = *reinterpret_cast<const float4*>(hs + (pt * 16 + col) * ldr + n);
#pragma unroll
          for (int v = 0; v < 4; ++v) inter[pt] = M::mma(at4(cv, v), at4(hv, v), inter[pt]);
        }
      }
    }
  };
  if (hlds || d.hin_transposed)
    readout(Hs, ldh);
  else
    readout(hb, d.N);
  // the skip term D x (none when Dv is null: x is then not read again)
  const bool skip = Dv != nullptr;
  const float dh = skip ? Dv[h] : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * kg + r;
    if (i >= q) continue;
    const float e = __expf(acs[i]);
    const int64_t row = (((int64_t)b * d.L + t0 + i) * d.H + h) * d.P;
    const int64_t xrow = (((int64_t)b * d.L + t0 + i) * xh.n + xh.row) * d.P;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      if (pt < npt) {
        const int p = p0 + pt * 16 + col;
        float v = acc[pt][r] + e * inter[pt][r];
        if (skip) v += dh * Io<IO>::load(x, xrow + p);
        if (d.f32_math)
          reinterpret_cast<float*>(y)[row + p] = v;
        else
          Io<IO>::store(y, row + p, v);
      }
    }
  }
}

// =============================================================================================
// Launchers
// =============================================================================================
hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* Acs,
                               float* dtc, hipStream_t s) {
  dim3 grid(d.nc, (d.H + 15) / 16, d.Bt);
  hipLaunchKernelGGL(k_chunk_cumsum, grid, dim3(256), 0, s, dt, A, Acs, dtc, d);
  return hipGetLastError();
}

hipError_t launch_bmm_chunk(const Dims& d, int io, const void* B, const void* C, float* CB,
                            hipStream_t s) {
  dim3 grid(d.nc, d.G, d.Bt);
  if (io == kIoBf16 && !d.f32_math) {
    hipLaunchKernelGGL((k_bmm_chunk<u16, f16>), grid, dim3(256), 0, s, (const u16*)B,
                       (const u16*)C, CB, d);
  } else if (d.Q <= 64 && d.N <= 128) {
    const size_t shm = (size_t)2 * d.Q * (d.N + 4) * 4;
    auto kern = io == kIoBf16 ? (const void*)k_bmm_chunk_lds<u16> : (const void*)k_bmm_chunk_lds<float>;
    if (shm > 64 * 1024) {
      hipError_t e =
          hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
    }
    if (io == kIoBf16)
      hipLaunchKernelGGL(k_bmm_chunk_lds<u16>, grid, dim3(256), shm, s, (const u16*)B,
                         (const u16*)C, CB, d);
    else
      hipLaunchKernelGGL(k_bmm_chunk_lds<float>, grid, dim3(256), shm, s, (const float*)B,
                         (const float*)C, CB, d);
  } else if (io == kIoBf16) {
    hipLaunchKernelGGL((k_bmm_chunk<u16, float>), grid, dim3(256), 0, s, (const u16*)B,
                       (const u16*)C, CB, d);
  } else {
    hipLaunchKernelGGL((k_bmm_chunk<float, float>), grid, dim3(256), 0, s, (const float*)B,
                       (const float*)C, CB, d);
  }
  return hipGetLastError();
}

template <typename IO, typename T, bool HILO>
static hipError_t state_impl(const Dims& d, const void* x, const void* B, const float* Acs,
                             const float* dtc, float* states, hipStream_t s) {
  constexpr int LD = SJ + Pad<T>::v;
  const size_t shm = (size_t)(64 * LD * (HILO ? 2 : 1) + d.N * LD) * sizeof(T) + SJ * 4;
  // n-tile slots per wave: 2 for dstate <= 128 (76 registers in fp32 instead of 140, so twice
  // the waves per SIMD), else 4 (a 1-slot build is larger than the 2-slot one: more hoisting)
  auto kern = d.N <= 128 ? k_chunk_state<IO, T, HILO, 2> : k_chunk_state<IO, T, HILO, 4>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  dim3 grid(d.nc * ((d.P + 63) / 64), d.H, d.Bt);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, (const IO*)x, (const IO*)B, Acs, dtc,
                     states, d);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Dims& d, int io, int prec, const void* x, const void* B,
                              const float* Acs, const float* dtc, float* states, hipStream_t s) {
  if (io == kIoF32) return state_impl<float, float, false>(d, x, B, Acs, dtc, states, s);
  if (prec == kPrecFp32) return state_impl<u16, float, false>(d, x, B, Acs, dtc, states, s);
  if (prec == kPrecFp16) return state_impl<u16, f16, false>(d, x, B, Acs, dtc, states, s);
  return state_impl<u16, f16, true>(d, x, B, Acs, dtc, states, s);
}

hipError_t launch_state_passing(const Dims& d, const float* states, const float* Acs,
                                const float* h0, float* h_in, float* fin, hipStream_t s) {
  return launch_chain_passing(d, d.nc, states, Acs + (d.Q - 1), (int64_t)d.nc * d.Q, d.Q, h0,
                              h_in, fin, s);
}

hipError_t launch_chain_passing(const Dims& d, int nsteps, const float* states,
                                const float* logdecay, int64_t ld_bh, int64_t ld_step,
                                const float* h0, float* h_in, float* fin, hipStream_t s) {
  dim3 grid((d.P * d.N + 1023) / 1024, d.H, d.Bt);
  hipLaunchKernelGGL(k_state_passing, grid, dim3(256), 0, s, states, logdecay, ld_bh, ld_step,
                     h0, h_in, fin, d, nsteps);
  return hipGetLastError();
}

template <typename IO, typename T>
static hipError_t scan_impl(const Dims& d, const void* x, const void* C, const float* CB,
                            const float* Acs, const float* dtc, const float* h_in,
                            const float* D, void* y, hipStream_t s) {
  constexpr int SX = (sizeof(T) == 2) ? 64 : 32;
  constexpr int LD = SX + Pad<T>::v;
  const int rows = std::min(d.P, 64);  // headdim columns per block
  size_t slab = (size_t)rows * LD * sizeof(T);
  if (scan_state_in_lds(d)) slab = std::max(slab, (size_t)rows * (d.N + 4) * 4);
  const size_t shm = 512 * 4 + slab;
  auto kern = k_chunk_scan<IO, T>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  dim3 grid(d.nc * ((d.Q + 63) / 64) * ((d.P + 63) / 64), d.H, d.Bt);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, (const IO*)x, (const IO*)C, CB, Acs, dtc,
                     h_in, D, (IO*)y, d);
  return hipGetLastError();
}

template <typename IO>
static hipError_t scan_f32_impl(const Dims& d, const void* x, const void* C, const float* CB,
                                const float* Acs, const float* dtc, const float* h_in,
                                const float* D, void* y, hipStream_t s) {
  const int rows = std::min(d.P, 64);
  size_t slab = (size_t)rows * (32 + 4) * 4;
  if (d.hin_transposed && !scan_state_in_lds(d)) return hipErrorInvalidValue;  // staged only
  if (scan_state_in_lds(d)) slab = std::max(slab, (size_t)rows * (d.N + 4) * 4);
  const size_t shm = 512 * 4 + slab;
  auto kern = k_chunk_scan_f32<IO>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  dim3 grid(d.nc * ((d.Q + 63) / 64) * ((d.P + 63) / 64), d.H, d.Bt);
  hipLaunchKernelGGL(kern, grid, dim3(256), shm, s, (const IO*)x, (const IO*)C, CB, Acs, dtc,
                     h_in, D, (IO*)y, d);
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const Dims& d, int io, int prec, const void* x, const void* C,
                             const float* CB, const float* Acs, const float* dtc,
                             const float* h_in, const float* D, void* y, hipStream_t s) {
  // a null D (no skip term) and the transposed entering state: fp32 arithmetic only
  if ((d.hin_transposed || !D) && io != kIoF32 && prec != kPrecFp32) return hipErrorInvalidValue;
  if (io == kIoF32) return scan_f32_impl<float>(d, x, C, CB, Acs, dtc, h_in, D, y, s);
  if (prec == kPrecFp32) return scan_f32_impl<u16>(d, x, C, CB, Acs, dtc, h_in, D, y, s);
  return scan_impl<u16, f16>(d, x, C, CB, Acs, dtc, h_in, D, y, s);
}

}  // namespace ssd
