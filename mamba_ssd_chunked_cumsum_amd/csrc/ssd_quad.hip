// Short-sequence forward in one kernel: the whole sequence as a single block of the quadratic
// (masked, attention-like) form, with no chunking and no state passed between chunks.
//
// The "nitter.gq/da_be19" thread (post 5/6) notes that for short sequences the chunked
// algorithm's constant overheads can make the naive quadratic form the cheaper one; the chunked
// algorithm's intra-chunk step is that form. Unrolling the recurrence S_t = exp(dt_t A) S_{t-1} +
// dt_t x_t B_t^T, y_t = S_t C_t + D x_t over the whole sequence gives, per head,
// y = (L o C B^T) (dt x) + D x with the decay mask L[t, s] = exp(sum of dt A over (s, t]) for
// s <= t, else 0. With an initial state h0 the readout adds exp(sum of dt A over [0, t]) C_t h0,
// and the final state is
//     h_L = sum_s exp(sum of dt A over (s, L-1]) dt_s x_s B_s^T + exp(sum of dt A over [0, L-1]) h0.
//
// One block (4 waves) per (p tile, row tile, head, batch), plus one per (p tile, head, batch) for
// the final state, so that a block's serial path is one row tile (the sizes this path serves are
// latency-bound). fp32 arithmetic throughout on the vector units. T is both the token tile and
// the p tile: T = 64 for dstate <= 128, else 32; NMAX, the dstate bound the tiles are staged for,
// is the next power of two from 32. The block's 256 threads form a 16 x 16 grid;
// each owns an M x M micro-tile (M = T / 16) of every T x T product, whose operands are M-vectors
// read from LDS (C and B are staged transposed, [n][token], for that). Every block:
//   1. dt (pre-processed) and the cumulative decay acs_t = sum of dt A over [0, t], a block scan.
// A row-tile block, tokens t0 .. t0 + T - 1:
//   2. for each token tile s0 <= t0: G = (C B^T) o exp(acs_t - acs_s) [s <= t], y += G (dt x);
//      then y += exp(acs_t) C h0^T (the micro-tile of C h0^T is the thread's y micro-tile), + D x.
// The final-state block:
//   3. F = sum over token tiles of (w x)^T B with w_s = exp(acs_end - acs_s) dt_s, + e^acs_end h0.
// Tiles are staged with compile-time trip counts, every load of a tile issued before its first LDS
// store, from clamped (always valid) addresses with out-of-range values selected away afterwards
// (a load under a condition would make each wait for the one before it).
#include <hip/hip_runtime.h>

#include "ssd_device.h"

namespace ssd {
namespace {

constexpr int kQuadThreads = 256;

template <int T, int NMAX_>
struct QuadTile {
  static constexpr int M = T / 16;                     // micro-tile edge
  static constexpr int LDT = T + 4;                    // row length of [.][T] tiles (16-byte rows)
  static constexpr int NMAX = NMAX_;                   // dstate bound
  static constexpr int NLD = T * NMAX / kQuadThreads;  // B or C tile: loads per thread
  static constexpr int NLX = T * T / kQuadThreads;     // x tile: loads per thread
  static constexpr int NG = NMAX / 16;                 // final state: n per thread (at most)
};

template <int M>
struct VecM;
template <>
struct VecM<4> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct VecM<2> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[2]) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[2]) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
};

// acc[a][b] = sum over n < N of Ut[n][ra + a] Vt[n][cb + b] (both tiles [n][T + 4])
template <class Q>
__device__ __forceinline__ void micro_dots(const float* Ut, const float* Vt, int N, int ra, int cb,
                                           float (&acc)[Q::M][Q::M]) {
#pragma unroll
  for (int a = 0; a < Q::M; ++a)
#pragma unroll
    for (int b = 0; b < Q::M; ++b) acc[a][b] = 0.f;
#pragma unroll 4
  for (int n = 0; n < N; ++n) {
    float u[Q::M], v[Q::M];
    VecM<Q::M>::load(Ut + n * Q::LDT + ra, u);
    VecM<Q::M>::load(Vt + n * Q::LDT + cb, v);
#pragma unroll
    for (int a = 0; a < Q::M; ++a)
#pragma unroll
      for (int b = 0; b < Q::M; ++b) acc[a][b] += u[a] * v[b];
  }
}

template <typename IO, int T, int NMAX>
__global__ __launch_bounds__(kQuadThreads) void k_quadratic(
    const IO* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Av,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dv,
    const float* __restrict__ h0, IO* __restrict__ y, float* __restrict__ fin, Dims d) {
  using Q = QuadTile<T, NMAX>;
  constexpr int M = Q::M, LDT = Q::LDT;
  extern __shared__ __align__(16) float sm[];
  const int L = d.L, N = d.N, P = d.P, H = d.H;
  float* acs = sm;               // [256]
  float* dts = acs + 256;        // [256]
  float* wsum = dts + 256;       // [4] (+ 12 to keep 16-byte alignment)
  float* Ct = wsum + 16;         // [N][T + 4]   C of the row tile, transposed
  float* Bt = Ct + N * LDT;      // [N][T + 4]   B of a token tile (or h0 of the p tile), transposed
  float* Xs = Bt + N * LDT;      // [T][T + 4]   weighted x of a token tile
  float* Gt = Xs + T * LDT;      // [T][T + 4]   masked, decayed C B^T, transposed ([s][t])
  float* Bn = Ct;                // final-state block: [T][N + 4] B rows (over Ct and Bt)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = (L + T - 1) / T;
  const int rt = blockIdx.x % (ntile + 1);  // row tile, or ntile: the final-state block
  const int p0 = (blockIdx.x / (ntile + 1)) * T, h = blockIdx.y, b = blockIdx.z;
  if (rt == ntile && fin == nullptr) return;
  const int g = h / (H / d.G);
  const float a = Av[h];
  const float bias = dt_bias_of(d, h);
  const int64_t xrow = (int64_t)H * P;    // x and y token stride
  const int64_t brow = (int64_t)d.G * N;  // B and C token stride
  const IO* xb = x + (int64_t)b * L * xrow + (int64_t)h * P;
  const IO* Bb = Bm + (int64_t)b * L * brow + (int64_t)g * N;
  const IO* Cb = Cm + (int64_t)b * L * brow + (int64_t)g * N;
  const float* hb = h0 ? h0 + ((int64_t)b * H + h) * P * N : nullptr;

  // 1. dt and the cumulative decay (one token per thread; L <= 256)
  {
    const float v = tid < L ? dt_effective(dt[((int64_t)b * L + tid) * H + h], bias, d) : 0.f;
    dts[tid] = v;
    const float incl = wave_inclusive_scan(v * a);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    float carry = 0.f;
    for (int w = 0; w < wave; ++w) carry += wsum[w];
    acs[tid] = incl + carry;
    __syncthreads();
  }

  // A token tile is loaded into registers (load_bc, load_x: every load issued, none waited for)
  // and stored to LDS later (store_bc, store_x), so that the next tile's loads are in flight
  // while the current one is computed. B or C: T rows (tokens s0 + j, zero past the sequence)
  // into dst[n][j] (transposed) or, with ROWS, dst[j][n] (row length N + 4).
  auto load_bc = [&](float (&v)[Q::NLD], const IO* src, int s0) {
#pragma unroll
    for (int c = 0; c < Q::NLD; ++c) {
      const int e = tid + kQuadThreads * c, j = e / Q::NMAX, n = e % Q::NMAX;
      v[c] = Io<IO>::load(src, (int64_t)min(s0 + j, L - 1) * brow + min(n, N - 1));
    }
  };
  auto store_bc = [&](const float (&v)[Q::NLD], float* dst, int s0, bool rows) {
#pragma unroll
    for (int c = 0; c < Q::NLD; ++c) {
      const int e = tid + kQuadThreads * c, j = e / Q::NMAX, n = e % Q::NMAX;
      if (n < N) dst[rows ? j * (N + 4) + n : n * LDT + j] = s0 + j < L ? v[c] : 0.f;
    }
  };
  // x of tokens s0 + j, columns p0 + p; stored weighted, w_s x_s, into Xs[j][p] (zero past the
  // sequence or headdim)
  auto load_x = [&](float (&v)[Q::NLX], int s0) {
#pragma unroll
    for (int c = 0; c < Q::NLX; ++c) {
      const int e = tid + kQuadThreads * c, j = e / T, p = e % T, s = s0 + j;
      v[c] = Io<IO>::load(xb, (int64_t)min(s, L - 1) * xrow + min(p0 + p, P - 1));
    }
  };
  auto store_x = [&](const float (&v)[Q::NLX], int s0, float acs_end, bool to_end) {
#pragma unroll
    for (int c = 0; c < Q::NLX; ++c) {
      const int e = tid + kQuadThreads * c, j = e / T, p = e % T, s = s0 + j;
      const float w = s < L ? (to_end ? __expf(acs_end - acs[s]) * dts[s] : dts[s]) : 0.f;
      Xs[j * LDT + p] = (s < L && p0 + p < P) ? w * v[c] : 0.f;
    }
  };
  float vb[Q::NLD], vx[Q::NLX];

  const int ty = tid >> 4, tx = tid & 15;  // micro-tile rows ty * M .., columns tx * M ..

  if (rt < ntile) {
    // 2. outputs of row tile rt
    const int t0 = rt * T;
    {
      float vc[Q::NLD];
      load_bc(vc, Cb, t0);
      load_bc(vb, Bb, 0);
      load_x(vx, 0);
      store_bc(vc, Ct, t0, false);
    }
    float yacc[M][M];
#pragma unroll
    for (int i = 0; i < M; ++i)
#pragma unroll
      for (int k = 0; k < M; ++k) yacc[i][k] = 0.f;
    float acs_t[M];
#pragma unroll
    for (int i = 0; i < M; ++i) acs_t[i] = acs[min(t0 + ty * M + i, L - 1)];
    for (int st = 0; st <= rt; ++st) {
      const int s0 = st * T;
      store_bc(vb, Bt, s0, false);
      store_x(vx, s0, 0.f, false);
      __syncthreads();  // C, B and x tiles staged
      if (st < rt) {  // the next token tile's loads, in flight during this tile's products
        load_bc(vb, Bb, s0 + T);
        load_x(vx, s0 + T);
      }
      float acc[M][M];
      micro_dots<Q>(Ct, Bt, N, ty * M, tx * M, acc);
      // mask and decay, stored transposed: Gt[j][i]
#pragma unroll
      for (int k = 0; k < M; ++k) {
        const int j = tx * M + k, s = s0 + j;
        const float acs_s = acs[min(s, 255)];
        float col[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const int t = t0 + ty * M + i;
          col[i] = (s <= t && s < L) ? acc[i][k] * __expf(acs_t[i] - acs_s) : 0.f;
        }
        VecM<M>::store(Gt + j * LDT + ty * M, col);
      }
      __syncthreads();  // G tile complete
#pragma unroll 4
      for (int j = 0; j < T; ++j) {
        float gv[M], xv[M];
        VecM<M>::load(Gt + j * LDT + ty * M, gv);
        VecM<M>::load(Xs + j * LDT + tx * M, xv);
#pragma unroll
        for (int i = 0; i < M; ++i)
#pragma unroll
          for (int k = 0; k < M; ++k) yacc[i][k] += gv[i] * xv[k];
      }
      __syncthreads();  // before the next tiles are staged over these
    }
    if (hb) {  // readout of the initial state: C h0^T, h0 of the p tile staged as Bt[n][p]
      float v[Q::NLD];
#pragma unroll
      for (int c = 0; c < Q::NLD; ++c) {
        const int e = tid + kQuadThreads * c, j = e / Q::NMAX, n = e % Q::NMAX;
        v[c] = hb[(int64_t)min(p0 + j, P - 1) * N + min(n, N - 1)];
      }
#pragma unroll
      for (int c = 0; c < Q::NLD; ++c) {
        const int e = tid + kQuadThreads * c, j = e / Q::NMAX, n = e % Q::NMAX;
        if (n < N) Bt[n * LDT + j] = p0 + j < P ? v[c] : 0.f;
      }
      __syncthreads();
      float acc[M][M];
      micro_dots<Q>(Ct, Bt, N, ty * M, tx * M, acc);
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float e_t = __expf(acs_t[i]);
#pragma unroll
        for (int k = 0; k < M; ++k) yacc[i][k] += e_t * acc[i][k];
      }
    }
    const float dh = Dv[h];
    IO* yb = y + (int64_t)b * L * xrow + (int64_t)h * P;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int t = t0 + ty * M + i;
      if (t >= L) continue;
#pragma unroll
      for (int k = 0; k < M; ++k) {
        const int p = p0 + tx * M + k;
        if (p < P) {
          const int64_t o = (int64_t)t * xrow + p;
          Io<IO>::store(yb, o, yacc[i][k] + dh * Io<IO>::load(xb, o));
        }
      }
    }
    return;
  }

  // 3. final state of the p tile: thread p = p0 + ty * M + i, n = tx + 16 c
  const float acs_end = acs[L - 1];
  const int ng = N / 16;  // dstate is a multiple of 16
  float facc[M][Q::NG];
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int c = 0; c < Q::NG; ++c) facc[i][c] = 0.f;
  load_bc(vb, Bb, 0);
  load_x(vx, 0);
  for (int st = 0; st < ntile; ++st) {
    const int s0 = st * T;
    store_bc(vb, Bn, s0, true);
    store_x(vx, s0, acs_end, true);
    __syncthreads();
    if (st + 1 < ntile) {
      load_bc(vb, Bb, s0 + T);
      load_x(vx, s0 + T);
    }
#pragma unroll 2
    for (int j = 0; j < T; ++j) {
      float xv[M];
      VecM<M>::load(Xs + j * LDT + ty * M, xv);
      const float* br = Bn + j * (N + 4) + tx;
#pragma unroll
      for (int c = 0; c < Q::NG; ++c) {
        if (c < ng) {
          const float bv = br[16 * c];
#pragma unroll
          for (int i = 0; i < M; ++i) facc[i][c] += xv[i] * bv;
        }
      }
    }
    __syncthreads();
  }
  const float e_end = __expf(acs_end);
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int p = p0 + ty * M + i;
    if (p >= P) continue;
    float* fo = fin + (((int64_t)b * H + h) * P + p) * N;
#pragma unroll
    for (int c = 0; c < Q::NG; ++c) {
      const int n = tx + 16 * c;
      if (c < ng) fo[n] = facc[i][c] + (hb ? e_end * hb[(int64_t)p * N + n] : 0.f);
    }
  }
}

template <typename IO, int T, int NMAX>
hipError_t quad_impl(const Dims& d, const void* x, const float* dt, const float* A, const void* B,
                     const void* C, const float* D, const float* h0, void* y, float* fin,
                     hipStream_t s) {
  using Q = QuadTile<T, NMAX>;
  const size_t shm = (size_t)(256 + 256 + 16 + 2 * d.N * Q::LDT + 2 * T * Q::LDT) * 4;
  auto kern = k_quadratic<IO, T, NMAX>;
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  const int ntile = (d.L + T - 1) / T;
  dim3 grid(((d.P + T - 1) / T) * (ntile + 1), d.H, d.Bt);
  hipLaunchKernelGGL(kern, grid, dim3(kQuadThreads), shm, s, (const IO*)x, dt, A, (const IO*)B,
                     (const IO*)C, D, h0, (IO*)y, fin, d);
  return hipGetLastError();
}

template <typename IO>
hipError_t quad_io(const Dims& d, const void* x, const float* dt, const float* A, const void* B,
                   const void* C, const float* D, const float* h0, void* y, float* fin,
                   hipStream_t s) {
  if (d.N <= 32) return quad_impl<IO, 64, 32>(d, x, dt, A, B, C, D, h0, y, fin, s);
  if (d.N <= 64) return quad_impl<IO, 64, 64>(d, x, dt, A, B, C, D, h0, y, fin, s);
  if (d.N <= 128) return quad_impl<IO, 64, 128>(d, x, dt, A, B, C, D, h0, y, fin, s);
  return quad_impl<IO, 32, 256>(d, x, dt, A, B, C, D, h0, y, fin, s);
}

}  // namespace

int64_t quadratic_blocks(const Dims& d) {
  const int T = d.N <= 128 ? 64 : 32;
  return (int64_t)((d.P + T - 1) / T) * ((d.L + T - 1) / T + 1) * d.H * d.Bt;
}

bool quadratic_covers(const Dims& d) {
  return d.L >= 1 && d.L <= kQuadMaxLen && d.N >= 16 && d.N <= 256 && d.N % 16 == 0 &&
         d.P % 16 == 0 && d.unit_input == 0;
}

hipError_t launch_quadratic(const Dims& d, int io, const void* x, const float* dt, const float* A,
                            const void* B, const void* C, const float* D, const float* h0,
                            void* y, float* fin, hipStream_t s) {
  if (!quadratic_covers(d)) return hipErrorInvalidValue;
  return io == kIoBf16 ? quad_io<u16>(d, x, dt, A, B, C, D, h0, y, fin, s)
                       : quad_io<float>(d, x, dt, A, B, C, D, h0, y, fin, s);
}

}  // namespace ssd
