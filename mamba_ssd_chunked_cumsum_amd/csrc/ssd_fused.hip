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
//
// Both kernels handle HB heads of one B/C group per block (so B and C are loaded, and C B^T is
// computed, once for HB heads) with NW = 4 * HB (P = 64) or 8 (P = 128) waves: wave w carries the
// state tiles of head w / (NW / HB), p-tile w % (NW / HB), all n-tiles. Tokens are staged through
// LDS in slabs of SL, double-buffered: the next slab's global loads are issued into registers
// before the current slab is computed. LDS tiles keep the natural row-major layout ([token][p],
// [token][n]); matrix-core fragments whose K index is the token are read with the gfx950
// transposing LDS load (ds_read_b64_tr_b16), so no transposed copy is ever made.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---- fragment helpers -----------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read: within each 16-lane group, lane i receives, in slot q, the (i % 4)-th of
// the four 16-bit values addressed by lane 4q + i / 4.
__device__ __forceinline__ f16x4 lds_tr4(const f16* p) {
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// K fragment of a 16-column tile (columns c0..c0+15, lane -> column c0 + lane % 16) of a
// row-major LDS tile whose rows are the K index: slot s of lane group g holds row r0 + 8 g + s
// (the standard K order of the 16x16x32 operands).
__device__ __forceinline__ f16x8 frag_k(const f16* base, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const f16* p = base + (r0 + 8 * g + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const f16x4 a = lds_tr4(p), b = lds_tr4(p + 4 * ld);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Same, in the order of a 16x16 accumulator pair: slots 0-3 hold rows r0 + 4 g + s, slots 4-7
// rows r0 + 16 + 4 g + s (g = lane group) -- the rows the two C B^T accumulators of a 32-token K
// step give each lane.
__device__ __forceinline__ f16x8 frag_k_acc(const f16* base, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const f16* p = base + (r0 + 4 * g + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const f16x4 a = lds_tr4(p), b = lds_tr4(p + 16 * ld);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> two fp16, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ f16x2 cvt_f16x2(float a, float b) {
  return __builtin_convertvector(f32x2{a, b}, f16x2);
}
// two fp32 -> two bf16 bit patterns packed in 32 bits, round to nearest even
// (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 8 bf16 (one 16-byte piece) -> 8 fp16 (exact for values in fp16's normal range)
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(uint4 r) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = cvt_f16x2(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u));
    o[2 * i] = h[0];
    o[2 * i + 1] = h[1];
  }
  return o;
}

// 8 fp32 -> 8 fp16
__device__ __forceinline__ f16x8 cvt_f16x8(const float (&v)[8]) {
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = cvt_f16x2(v[2 * i], v[2 * i + 1]);
    o[2 * i] = h[0];
    o[2 * i + 1] = h[1];
  }
  return o;
}

template <int P_, int N_, int HB_, int NW_, int SL_, int MT_>
struct Cfg {
  static constexpr int P = P_, N = N_, HB = HB_, NW = NW_, SL = SL_;
  static constexpr int NT = NW * 64;
  static constexpr int NP = P / 16, NN = N / 16, NK = N / 32;
  static constexpr int WPH = NW / HB;   // waves per head for the state tiles
  static_assert(WPH % NP == 0, "whole waves per (head, p-tile)");
  static constexpr int WPP = WPH / NP;  // waves per (head, p-tile)
  static_assert(NN % WPP == 0, "n-tiles split evenly over a (head, p-tile)'s waves");
  static constexpr int TS = NN / WPP;   // carried-state tiles per wave
  static_assert(SL % 32 == 0 && SL <= 64, "slab of whole 32-token K steps, one wave of tokens");
  static_assert(HB == 1 || HB == 2, "one or two heads per block");
  static constexpr int MAXI = MT_;      // 16-row output tiles per wave (Q <= 16 NW MT)
  static constexpr int LDX = P + 8, LDB = N + 8, LDH = N + 8;
  static constexpr int LDY = HB * P + 4;  // floats per row of a wave's 8-row output tile
  static constexpr int XS = HB * SL * LDX, BS = SL * LDB;   // halfs per stage
  static constexpr int XPIECES = HB * SL * P / 8, PIECES = XPIECES + SL * N / 8;
  static constexpr int PPT = (PIECES + NT - 1) / NT;       // 16-byte pieces per thread
  // h^T (fp16) and, later in each chunk, the waves' fp32 output tiles share one region (halfs)
  static constexpr int HREG = HB * P * LDH > NW * 8 * LDY * 2 ? HB * P * LDH : NW * 8 * LDY * 2;
};

// Global -> registers for one slab: x of the HB heads and B, token rows [j0, j0 + SL) of the
// chunk starting at t0 (q valid rows; later rows are zeros).
template <class K>
__device__ __forceinline__ void slab_load(uint4 (&v)[K::PPT], const u16* x, const u16* Bm,
                                          const Dims& d, int b, int h0, int g, int t0, int q,
                                          int j0) {
  // Rows past the end of the chunk read row j0 instead (always inside the sequence) and are
  // zeroed afterwards, so the loads carry no branches and can all be in flight together.
#pragma unroll
  for (int k = 0; k < K::PPT; ++k) {
    const int e = threadIdx.x + k * K::NT;
    if (k * K::NT >= K::PIECES) break;  // whole iteration past the slab (compile-time)
    const bool isx = e < K::XPIECES;
    const int e2 = isx ? e : e - K::XPIECES;
    const int j = isx ? e / (K::HB * K::P / 8) : e2 / (K::N / 8);
    const bool valid = (e < K::PIECES) && (j0 + j < q);
    const int jr = valid ? j : 0;
    const u16* src =
        isx ? x + (((int64_t)b * d.L + t0 + j0 + jr) * d.H + h0) * K::P + (e % (K::HB * K::P / 8)) * 8
            : Bm + (((int64_t)b * d.L + t0 + j0 + jr) * d.G + g) * K::N + (e2 % (K::N / 8)) * 8;
    const uint4 val = *reinterpret_cast<const uint4*>(src);
    v[k] = valid ? val : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Registers -> LDS stage (converted to fp16).
template <class K>
__device__ __forceinline__ void slab_store(const uint4 (&v)[K::PPT], f16* Xs, f16* Bs) {
#pragma unroll
  for (int k = 0; k < K::PPT; ++k) {
    const int e = threadIdx.x + k * K::NT;
    if (e < K::XPIECES) {
      const int j = e / (K::HB * K::P / 8), rem = e % (K::HB * K::P / 8);
      const int hh = rem / (K::P / 8), c8 = rem % (K::P / 8);
      *reinterpret_cast<f16x8*>(Xs + (hh * K::SL + j) * K::LDX + c8 * 8) = bf16x8_to_f16x8(v[k]);
    } else if (e < K::PIECES) {
      const int e2 = e - K::XPIECES;
      const int j = e2 / (K::N / 8), c8 = e2 % (K::N / 8);
      *reinterpret_cast<f16x8*>(Bs + j * K::LDB + c8 * 8) = bf16x8_to_f16x8(v[k]);
    }
  }
}

// ---- F1: run states -------------------------------------------------------------------------
// state_r = sum_{t in run} exp(sum_{k in (t, end]} dt_k A) dt_t x_t B_t^T (zero entry state) and
// logdecay_r = sum_{t in run} dt_t A. Grid (nr, H / HB, batch). Slabs are taken from the run end
// backwards so the weights are suffix sums (accurate where they matter most, near the end).
// The state operand w_t x_t is split into fp16 high and low parts (two matrix-core passes) so the
// chained run states keep near-fp32 accuracy.
template <class K>
__global__ __launch_bounds__(K::NT) void k_run_state(const u16* __restrict__ x,
                                                     const u16* __restrict__ Bm,
                                                     const float* __restrict__ dt,
                                                     const float* __restrict__ Av,
                                                     float* __restrict__ states,
                                                     float* __restrict__ logdecay, Dims d,
                                                     int run_len, int nr) {
  using M = Mma<f16>;
  constexpr int SL = K::SL;
  __shared__ __align__(16) f16 Xs[2][K::XS];
  __shared__ __align__(16) f16 Bs[2][K::BS];
  __shared__ __align__(16) float w[2][K::HB][SL];

  const int r = blockIdx.x, h0 = blockIdx.y * K::HB, b = blockIdx.z;
  const int g = h0 / (d.H / d.G);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kg = lane >> 4, col = lane & 15;
  const int sh = wave / K::WPH, spt = (wave % K::WPH) % K::NP;
  const int sn0 = ((wave % K::WPH) / K::NP) * K::TS;  // first n-tile carried by this wave
  const int t_begin = r * run_len, t_end = min(d.L, t_begin + run_len);
  const int nslab = (t_end - t_begin + SL - 1) / SL;
  // waves 0..HB-1 compute the weights of their head; lane l < SL holds token s0 + l
  const float a_h = wave < K::HB ? Av[h0 + wave] : 0.f;
  float carry = 0.f;  // sum of dt A over the tokens after the current slab (waves < HB)

  f32x4 S[K::TS];
#pragma unroll
  for (int k = 0; k < K::TS; ++k) S[k] = zero4();

  // weights of one slab from its dt (one value per lane), then move the carry past the slab
  auto weights = [&](float dtv, int stg) {
    if (wave < K::HB) {
      const float a = dtv * a_h;
      float v = a;  // suffix sum over lanes >= l within the slab
#pragma unroll
      for (int off = 1; off < SL; off <<= 1) {
        const float o = __shfl_down(v, off, kWave);
        if (lane + off < SL) v += o;
      }
      float after = __shfl_down(v, 1, kWave);  // sum over lanes > l
      if (lane + 1 >= SL) after = 0.f;
      if (lane < SL) w[stg][wave][lane] = __expf(carry + after) * dtv;
      carry += __shfl(v, 0, kWave);
    }
  };
  auto load_dt = [&](int s0) -> float {
    float v = 0.f;
    if (wave < K::HB && lane < SL && s0 + lane < t_end)
      v = dt[((int64_t)b * d.L + s0 + lane) * d.H + h0 + wave];
    return v;
  };

  uint4 pre[K::PPT];
  int stage = 0;
  {
    const int s0 = t_begin + (nslab - 1) * SL;
    slab_load<K>(pre, x, Bm, d, b, h0, g, s0, t_end - s0, 0);
    const float dtv = load_dt(s0);
    slab_store<K>(pre, Xs[0], Bs[0]);
    weights(dtv, 0);
  }
  __syncthreads();
  for (int s = nslab - 1; s >= 0; --s) {
    const bool next = s > 0;
    float dtn = 0.f;
    if (next) {
      const int s0 = t_begin + (s - 1) * SL;
      slab_load<K>(pre, x, Bm, d, b, h0, g, s0, t_end - s0, 0);
      dtn = load_dt(s0);
    }
    const f16* X = Xs[stage] + sh * SL * K::LDX;
    const f16* Bt = Bs[stage];
    const float* ws = w[stage][sh];
#pragma unroll
    for (int ks = 0; ks < SL / 32; ++ks) {
      const f16x8 xv = frag_k(X, K::LDX, ks * 32, spt * 16, lane);
      const float4 w0 = *reinterpret_cast<const float4*>(ws + ks * 32 + 8 * kg);
      const float4 w1 = *reinterpret_cast<const float4*>(ws + ks * 32 + 8 * kg + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float val[8], rem[8];
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) val[qq] = (float)xv[qq] * wv[qq];
      const f16x8 hi = cvt_f16x8(val);
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) rem[qq] = val[qq] - (float)hi[qq];  // exact in fp32
      const f16x8 lo = cvt_f16x8(rem);
#pragma unroll
      for (int k = 0; k < K::TS; ++k) {
        const f16x8 bf = frag_k(Bt, K::LDB, ks * 32, (sn0 + k) * 16, lane);
        S[k] = M::mma(bf, hi, S[k]);
        S[k] = M::mma(bf, lo, S[k]);
      }
    }
    if (next) {
      slab_store<K>(pre, Xs[stage ^ 1], Bs[stage ^ 1]);
      weights(dtn, stage ^ 1);
    }
    __syncthreads();
    stage ^= 1;
  }
  if (wave < K::HB && lane == 0) logdecay[((int64_t)b * d.H + h0 + wave) * nr + r] = carry;
  // S^T tile (n rows, p columns): lane holds p = spt*16 + col, n = nt*16 + 4 kg + rr
  float* out = states + (((int64_t)b * nr + r) * d.H + h0 + sh) * (int64_t)(K::P * K::N);
#pragma unroll
  for (int k = 0; k < K::TS; ++k)
    *reinterpret_cast<float4*>(out + (spt * 16 + col) * K::N + (sn0 + k) * 16 + 4 * kg) =
        make_float4(S[k][0], S[k][1], S[k][2], S[k][3]);
}

// ---- F3: fused chunk scan over a run ------------------------------------------------------------
// Grid (nr, H / HB, batch). Wave w owns MAXI 16-row output tiles of each chunk (for all HB heads
// and all P columns), chosen so every wave has the same causal work (tiles w, 2 NW - 1 - w, ...),
// and carries the state tiles of its (head, p-tile).
//
// Per chunk: C rows of the wave's tiles are loaded once into registers (the B operand of
// (C B^T)^T and the A operand of the readout share one fragment layout); waves 0..HB-1 form, for
// their head, the cumulative decay acs, dt, the state weights w_j = exp(acs_last - acs_j) dt_j and
// the column factors cf_j = exp(acs_e - acs_j) dt_j (e = last token of j's 32-token K step); the
// carried state is written to LDS in fp16 as h^T [p][n]; the readout y_i = exp(acs_i) C_i . h
// starts the output accumulators. Then, per slab, for each 32-token K step the two 16x16 blocks
// of (C B^T)^T are computed into registers and turned, lane by lane, into the A fragment
//   M[i][j] = CB[i][j] exp(acs_i - acs_j) dt_j   (0 for j > i)
// of each head -- the Q x Q block never leaves registers. Below the diagonal this is formed as
// CB[i][j] * exp(acs_i - acs_e) * cf_j: both factors are <= 1 and the exponential is per row, not
// per element; the one K step holding the tile's diagonal uses the direct form and the mask. The
// fragment's K slots follow the accumulator layout (j = jb + 4 kg + r, jb + 16 + 4 kg + r), and x
// is read from LDS in the same order. The carried state decays by exp(acs_last) and accumulates
// B^T (w x) (skipped after the run's last chunk: the next run's entry state comes from F1/F2).
// Finally y = accumulator + D x is rounded once to bf16 and written as whole rows.
template <class K>
__device__ __forceinline__ int row_tile(int wave, int m) {
  // m-th 16-row tile of a wave: w, 2 NW - 1 - w, 2 NW + w, 4 NW - 1 - w, ...
  return (m & 1) ? K::NW * (m + 1) - 1 - wave : K::NW * m + wave;
}

template <class K>
__global__ __launch_bounds__(K::NT) void k_fused_scan(
    const u16* __restrict__ x, const u16* __restrict__ Bm, const u16* __restrict__ Cm,
    const float* __restrict__ dt, const float* __restrict__ Av, const float* __restrict__ Dv,
    const float* __restrict__ h_run, u16* __restrict__ y, Dims d, int S, int nr) {
  using M = Mma<f16>;
  constexpr int SL = K::SL, HB = K::HB, NP = K::NP, NK = K::NK, MAXI = K::MAXI;
  __shared__ __align__(16) f16 Xs[2][K::XS];
  __shared__ __align__(16) f16 Bs[2][K::BS];
  __shared__ __align__(16) f16 hreg[K::HREG];  // h^T [HB][P][LDH], then per-wave y tiles
  __shared__ __align__(16) float acs[HB][256];
  __shared__ __align__(16) float dts[HB][256];
  __shared__ __align__(16) float wts[HB][256];
  __shared__ __align__(16) float cfs[HB][256];

  const int r = blockIdx.x, h0 = blockIdx.y * HB, b = blockIdx.z;
  const int g = h0 / (d.H / d.G);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int Q = d.Q, nti = Q / 16;
  const int sh = wave / K::WPH, spt = (wave % K::WPH) % K::NP;
  const int sn0 = ((wave % K::WPH) / K::NP) * K::TS;  // first n-tile carried by this wave
  const int c_begin = r * S, c_end = min(d.nc, c_begin + S);
  float Dh[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) Dh[hh] = Dv[h0 + hh];
  const float a_h = wave < HB ? Av[h0 + wave] : 0.f;
  // entries past Q are read (as zeros) when Q is shorter than a K step or a slab
  for (int i = threadIdx.x; i < 256; i += K::NT) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) acs[hh][i] = dts[hh][i] = wts[hh][i] = cfs[hh][i] = 0.f;
  }

  // carried state (S^T tiles): lane holds p = spt*16 + col, n = nt*16 + 4 kg + rr
  f32x4 Sacc[K::TS];
  {
    const float* hr = h_run + (((int64_t)b * nr + r) * d.H + h0 + sh) * (int64_t)(K::P * K::N);
#pragma unroll
    for (int k = 0; k < K::TS; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(hr + (spt * 16 + col) * K::N +
                                                        (sn0 + k) * 16 + 4 * kg);
      Sacc[k] = f32x4{v.x, v.y, v.z, v.w};
    }
  }

  uint4 pre[K::PPT];
  int stage = 0;
  {
    const int t0 = c_begin * Q;
    slab_load<K>(pre, x, Bm, d, b, h0, g, t0, min(Q, d.L - t0), 0);
    slab_store<K>(pre, Xs[0], Bs[0]);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * Q, q = min(Q, d.L - t0);
    const bool carry = (c + 1) < c_end;
    const int nslab = (q + SL - 1) / SL;
    // C rows of this wave's tiles (zero past the end of the sequence)
    f16x8 Cf[MAXI][NK];
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = row_tile<K>(wave, m);
      const int i = ti * 16 + col;
      const bool valid = ti < nti && i < q;
      const u16* crow = Cm + (((int64_t)b * d.L + t0 + (valid ? i : 0)) * d.G + g) * K::N;
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        const uint4 v = *reinterpret_cast<const uint4*>(crow + kn * 32 + 8 * kg);
        Cf[m][kn] = bf16x8_to_f16x8(valid ? v : make_uint4(0u, 0u, 0u, 0u));
      }
    }
    __syncthreads();  // previous chunk's y tiles (aliasing h^T) and slab buffers are done
    if (wave < HB) {
      const int E = Q >= 64 ? Q / 64 : 1;
      float loc[4], dv[4];
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = lane * E + e;
        float v = 0.f;
        if (e < E && i < q) v = dt[((int64_t)b * d.L + t0 + i) * d.H + h0 + wave];
        dv[e] = v;
        s += v * a_h;
        loc[e] = s;
      }
      const float incl = wave_inclusive_scan(s);
      float excl = __shfl_up(incl, 1, kWave);
      if (lane == 0) excl = 0.f;
      const int eq = (q - 1) % E;
      float mine = excl + loc[0], mylast = excl + loc[0];
#pragma unroll
      for (int e = 1; e < 4; ++e) {
        if (e == eq) mine = excl + loc[e];
        if (e == E - 1) mylast = excl + loc[e];
      }
      const float vlast = __shfl(mine, (q - 1) / E, kWave);
      if (lane * E + E - 1 >= q) mylast = vlast;
      // cumulative decay at the last token of this lane's 32-token K step (a lane's E tokens
      // never straddle two K steps); meaningful for Q >= 32
      const float aend = __shfl(mylast, ((lane * E) | 31) / E, kWave);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = lane * E + e;
        if (e < E && i < Q) {
          const float a = (i < q) ? excl + loc[e] : vlast;
          acs[wave][i] = a;
          dts[wave][i] = dv[e];
          wts[wave][i] = (i < q) ? __expf(vlast - a) * dv[e] : 0.f;
          cfs[wave][i] = (i < q) ? __expf(aend - a) * dv[e] : 0.f;
        }
      }
    }
    {  // carried state -> h^T (fp16) for the readout
      f16* ht = hreg + (sh * K::P + spt * 16 + col) * K::LDH;
#pragma unroll
      for (int k = 0; k < K::TS; ++k) {
        const f16x2 lo = cvt_f16x2(Sacc[k][0], Sacc[k][1]);
        const f16x2 hi = cvt_f16x2(Sacc[k][2], Sacc[k][3]);
        *reinterpret_cast<f16x4*>(ht + (sn0 + k) * 16 + 4 * kg) = f16x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
    __syncthreads();

    // readout of the state entering this chunk
    f32x4 Y[MAXI][HB][NP];
    float acs_i[MAXI][HB];
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = row_tile<K>(wave, m);
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        acs_i[m][hh] = ti < nti ? acs[hh][ti * 16 + col] : 0.f;
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) Y[m][hh][pt] = zero4();
      }
      if (ti >= nti) continue;
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
        for (int kn = 0; kn < NK; ++kn) {
#pragma unroll
          for (int pt = 0; pt < NP; ++pt)
            Y[m][hh][pt] = M::mma(
                Cf[m][kn], M::lds(hreg + (hh * K::P + pt * 16 + col) * K::LDH + kn * 32 + 8 * kg),
                Y[m][hh][pt]);
        }
        const float4 ar = *reinterpret_cast<const float4*>(&acs[hh][ti * 16 + 4 * kg]);
        const float e4[4] = {__expf(ar.x), __expf(ar.y), __expf(ar.z), __expf(ar.w)};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int pt = 0; pt < NP; ++pt) Y[m][hh][pt][rr] *= e4[rr];
      }
    }
    if (carry) {
      const float dec = __expf(acs[sh][Q - 1]);
#pragma unroll
      for (int k = 0; k < K::TS; ++k) Sacc[k] *= dec;
    }

    for (int s = 0; s < nslab; ++s) {
      const int j0 = s * SL;
      const bool more = (s + 1 < nslab) || (c + 1 < c_end);
      if (more) {
        if (s + 1 < nslab) {
          slab_load<K>(pre, x, Bm, d, b, h0, g, t0, q, j0 + SL);
        } else {
          const int t1 = t0 + Q;
          slab_load<K>(pre, x, Bm, d, b, h0, g, t1, min(Q, d.L - t1), 0);
        }
      }
      const f16* Xst = Xs[stage];
      const f16* Bst = Bs[stage];
      // intra-chunk masked product
#pragma unroll
      for (int ks = 0; ks < SL / 32; ++ks) {
        const int jb = j0 + ks * 32;  // chunk-local first token of this K step
        bool act[MAXI];
        bool any = false;
#pragma unroll
        for (int m = 0; m < MAXI; ++m) {
          const int ti = row_tile<K>(wave, m);
          act[m] = (ti < nti) && (ti * 16 + 15 >= jb);
          any |= act[m];
        }
        if (!any) continue;
        // (C B^T)^T for both 16-token halves of the K step and every active row tile; the B
        // fragments are loaded once and shared by the tiles. Both halves are always formed: the
        // second is wasted (and masked) only in the K step holding an even tile's diagonal.
        f32x4 c0[MAXI], c1[MAXI];
        {
          f16x8 b0[NK], b1[NK];
          const f16* brow = Bst + (ks * 32 + col) * K::LDB + 8 * kg;
#pragma unroll
          for (int kn = 0; kn < NK; ++kn) {
            b0[kn] = M::lds(brow + kn * 32);
            b1[kn] = M::lds(brow + 16 * K::LDB + kn * 32);
          }
#pragma unroll
          for (int m = 0; m < MAXI; ++m) {
            c0[m] = zero4();
            c1[m] = zero4();
            if (!act[m]) continue;
#pragma unroll
            for (int kn = 0; kn < NK; ++kn) {
              c0[m] = M::mma(b0[kn], Cf[m][kn], c0[m]);
              c1[m] = M::mma(b1[kn], Cf[m][kn], c1[m]);
            }
          }
        }
        const int ja = jb + 4 * kg;  // this lane's K slots: ja + rr and ja + 16 + rr
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
          f16x8 xf[NP];
#pragma unroll
          for (int pt = 0; pt < NP; ++pt)
            xf[pt] = frag_k_acc(Xst + hh * SL * K::LDX, K::LDX, ks * 32, pt * 16, lane);
          const float aend = acs[hh][jb + 31];
          const float4 f0 = *reinterpret_cast<const float4*>(&cfs[hh][ja]);
          const float4 f1 = *reinterpret_cast<const float4*>(&cfs[hh][ja + 16]);
          const float cf[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
          for (int m = 0; m < MAXI; ++m) {
            if (!act[m]) continue;
            const int ti = row_tile<K>(wave, m);
            const int i = ti * 16 + col;
            float v[8];
            if (ti * 16 >= jb + 32) {  // strictly below the diagonal: factorized decay
              const float rf = __expf(acs_i[m][hh] - aend);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                v[rr] = c0[m][rr] * rf * cf[rr];
                v[4 + rr] = c1[m][rr] * rf * cf[4 + rr];
              }
            } else {  // the K step holding this tile's diagonal: direct form and causal mask
              const float4 a0 = *reinterpret_cast<const float4*>(&acs[hh][ja]);
              const float4 a1 = *reinterpret_cast<const float4*>(&acs[hh][ja + 16]);
              const float4 d0 = *reinterpret_cast<const float4*>(&dts[hh][ja]);
              const float4 d1 = *reinterpret_cast<const float4*>(&dts[hh][ja + 16]);
              const float aj[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
              const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const float e0 = c0[m][rr] * __expf(acs_i[m][hh] - aj[rr]) * dj[rr];
                const float e1 = c1[m][rr] * __expf(acs_i[m][hh] - aj[4 + rr]) * dj[4 + rr];
                v[rr] = (ja + rr <= i) ? e0 : 0.f;
                v[4 + rr] = (ja + 16 + rr <= i) ? e1 : 0.f;
              }
            }
            const f16x8 mf = cvt_f16x8(v);
#pragma unroll
            for (int pt = 0; pt < NP; ++pt) Y[m][hh][pt] = M::mma(mf, xf[pt], Y[m][hh][pt]);
          }
        }
      }
      // carried-state update with this slab
      if (carry) {
        const f16* X = Xst + sh * SL * K::LDX;
#pragma unroll
        for (int ks = 0; ks < SL / 32; ++ks) {
          const f16x8 xv = frag_k(X, K::LDX, ks * 32, spt * 16, lane);
          const float4 w0 = *reinterpret_cast<const float4*>(&wts[sh][j0 + ks * 32 + 8 * kg]);
          const float4 w1 = *reinterpret_cast<const float4*>(&wts[sh][j0 + ks * 32 + 8 * kg + 4]);
          const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          float val[8];
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) val[qq] = (float)xv[qq] * wv[qq];
          const f16x8 wf = cvt_f16x8(val);
#pragma unroll
          for (int k = 0; k < K::TS; ++k)
            Sacc[k] = M::mma(frag_k(Bst, K::LDB, ks * 32, (sn0 + k) * 16, lane), wf, Sacc[k]);
        }
      }
      if (more) slab_store<K>(pre, Xs[stage ^ 1], Bs[stage ^ 1]);
      __syncthreads();
      stage ^= 1;
    }

    // y = accumulator + D x, rounded once to bf16. Each wave moves its 16-row tiles through an
    // fp32 LDS tile (8 rows at a time) so that y is written, and x read back exactly (bf16) for
    // the skip term, as whole 16-byte pieces of rows.
    float* yt = reinterpret_cast<float*>(hreg) + wave * 8 * K::LDY;
    constexpr int RP = HB * K::P / 8;  // 16-byte (8-value) pieces per row
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
      const int ti = row_tile<K>(wave, m);
      if (ti >= nti) continue;
      // x for the skip term of this tile, loaded up front (rows past the end read row 0)
      constexpr int PPL = (8 * RP + 63) / 64;  // pieces per lane per half
      uint4 xr[2][PPL];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const int e = lane + 64 * k;
          const int row = e / RP, c8 = e % RP;
          const int i = ti * 16 + 8 * half + row;
          const int ir = (e < 8 * RP && i < q) ? i : 0;
          xr[half][k] = *reinterpret_cast<const uint4*>(
              x + (((int64_t)b * d.L + t0 + ir) * d.H + h0) * K::P + c8 * 8);
        }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if ((kg >> 1) == half) {  // lanes holding rows 8*half .. 8*half + 7
#pragma unroll
          for (int hh = 0; hh < HB; ++hh)
#pragma unroll
            for (int pt = 0; pt < NP; ++pt)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                yt[(4 * (kg & 1) + rr) * K::LDY + hh * K::P + pt * 16 + col] = Y[m][hh][pt][rr];
        }
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const int e = lane + 64 * k;
          const int row = e / RP, c8 = e % RP;
          const int i = ti * 16 + 8 * half + row;
          if (e < 8 * RP && i < q) {
            const int64_t off = (((int64_t)b * d.L + t0 + i) * d.H + h0) * K::P + c8 * 8;
            const float dh = (c8 * 8 < K::P) ? Dh[0] : Dh[HB - 1];  // HB <= 2
            const uint4 xw = xr[half][k];
            const uint32_t xwv[4] = {xw.x, xw.y, xw.z, xw.w};
            float xv[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              xv[2 * t] = __uint_as_float(xwv[t] << 16);
              xv[2 * t + 1] = __uint_as_float(xwv[t] & 0xffff0000u);
            }
            const float4 lo = *reinterpret_cast<const float4*>(yt + row * K::LDY + c8 * 8);
            const float4 hi = *reinterpret_cast<const float4*>(yt + row * K::LDY + c8 * 8 + 4);
            const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            uint32_t packed[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              packed[k] = cvt_bf16x2(v[2 * k] + dh * xv[2 * k], v[2 * k + 1] + dh * xv[2 * k + 1]);
            *reinterpret_cast<uint4*>(y + off) =
                make_uint4(packed[0], packed[1], packed[2], packed[3]);
          }
        }
      }
    }
  }
}

// ---- launchers ----------------------------------------------------------------------------------
// One head per block, 8 waves; MT 16-row output tiles per wave: 2 for Q = 256, 1 for Q <= 128.
template <int P, int N, int SL>
using CfgQ256 = Cfg<P, N, 1, 8, SL, 2>;
template <int P, int N, int SL>
using CfgQ128 = Cfg<P, N, 1, 8, SL, 1>;

bool fused_supported(const Dims& d) {
  return (d.P == 64 && (d.N == 64 || d.N == 128)) || (d.P == 128 && (d.N == 128 || d.N == 256));
}

template <class K>
static hipError_t launch_phase(int phase, const Dims& d, const void* x, const void* B,
                               const void* C, const float* dt, const float* A, const float* D,
                               int S, int nr, float* states, float* logdecay,
                               const float* h_run, void* y, hipStream_t s) {
  dim3 grid(nr, d.H / K::HB, d.Bt);
  if (phase == 0)
    hipLaunchKernelGGL(k_run_state<K>, grid, dim3(K::NT), 0, s, (const u16*)x, (const u16*)B, dt,
                       A, states, logdecay, d, S * d.Q, nr);
  else
    hipLaunchKernelGGL(k_fused_scan<K>, grid, dim3(K::NT), 0, s, (const u16*)x, (const u16*)B,
                       (const u16*)C, dt, A, D, h_run, (u16*)y, d, S, nr);
  return hipGetLastError();
}

template <int P, int N, int SL>
static hipError_t dispatch_q(int phase, const Dims& d, const void* x, const void* B, const void* C,
                             const float* dt, const float* A, const float* D, int S, int nr,
                             float* states, float* logdecay, const float* h_run, void* y,
                             hipStream_t s) {
  if (d.Q > 128)
    return launch_phase<CfgQ256<P, N, SL>>(phase, d, x, B, C, dt, A, D, S, nr, states, logdecay,
                                           h_run, y, s);
  return launch_phase<CfgQ128<P, N, SL>>(phase, d, x, B, C, dt, A, D, S, nr, states, logdecay,
                                         h_run, y, s);
}

static hipError_t dispatch(int phase, const Dims& d, const void* x, const void* B, const void* C,
                           const float* dt, const float* A, const float* D, int S, int nr,
                           float* states, float* logdecay, const float* h_run, void* y,
                           hipStream_t s) {
#define SSD_PHASE(P, N, SL) \
  dispatch_q<P, N, SL>(phase, d, x, B, C, dt, A, D, S, nr, states, logdecay, h_run, y, s)
  if (d.P == 64 && d.N == 128) return SSD_PHASE(64, 128, 64);
  if (d.P == 64 && d.N == 64) return SSD_PHASE(64, 64, 64);
  if (d.P == 128 && d.N == 128) return SSD_PHASE(128, 128, 64);
  if (d.P == 128 && d.N == 256) return SSD_PHASE(128, 256, 32);
#undef SSD_PHASE
  return hipErrorInvalidValue;
}

hipError_t launch_run_state(const Dims& d, const void* x, const void* B, const float* dt,
                            const float* A, int S, int nr, float* states, float* logdecay,
                            hipStream_t s) {
  return dispatch(0, d, x, B, nullptr, dt, A, nullptr, S, nr, states, logdecay, nullptr, nullptr,
                  s);
}

hipError_t launch_fused_scan(const Dims& d, const void* x, const void* B, const void* C,
                             const float* dt, const float* A, const float* D,
                             const float* h_run, void* y, int S, int nr, hipStream_t s) {
  return dispatch(1, d, x, B, C, dt, A, D, S, nr, nullptr, nullptr, h_run, y, s);
}

}  // namespace ssd
