// Fused SSD chunked forward (bf16 io): three kernels for the whole forward.
//
// The chunked algorithm ("nitter.gq/da_be19" thread, post 5/6; stage order as in "Mamba-2 in
// NVIDIA cuTile: Faster Forward Kernels and What the Benchmark Means", section "Why Mamba-2 is a
// useful kernel example") needs the state entering every chunk. A (batch, head)'s fp32 state
// (P x N) is as large as its bf16 x tile of 256 tokens, so materialising one per chunk would
// double the HBM traffic. Here each sequence is cut into a few runs of consecutive tokens (about
// one block per compute unit in total; a chain is the runs of one batch entry and head block):
//
//   k_run_states  one block per (chain, run) whose state is needed: the run's own end state
//                 (zero entry state) and total log-decay. States handed to the chain are stored
//                 in fp16; the last run's state, computed only when a final state is wanted, is
//                 stored in fp32 straight into the final state.
//   k_state_chain one thread per 8 entries of a (batch, head) state walks its runs in fp32,
//                 h_in(r+1) = exp(logdecay_r) h_in(r) + state_r from h0 (or zero), overwriting
//                 each run's slot with the state entering the next run (fp16), and completes the
//                 final state.
//   k_fused_scan  one block per (chain, run), sub-chunk by sub-chunk from the state entering the
//                 run: cumulative decay, C B^T, the masked intra-sub-chunk product, the readout
//                 of the carried state, the skip term and the state update, all on chip; only y
//                 leaves.
//
// With one run per sequence there is no chain: k_run_states completes its state into the final
// state (S + exp(sum of dt A) h0; skipped when no final state is wanted) and k_fused_scan starts
// from the initial state itself.
//
// Inside the kernels a run is walked in sub-chunks of T = 32 tokens, whatever the caller's chunk
// length: the exact result does not depend on where the sequence is cut (the chunk length cancels
// out of the recurrence), so the kernels pick the cut that suits the chip's registers and LDS.
// The caller's chunk length still fixes the stage entry points' outputs.
//
// Work split (one 512-thread block per compute unit, two waves per SIMD): a wave owns one head's
// p-slice of PS columns (PS * N <= 8192, so its fp32 state is at most 128 registers per lane; at
// headdim 64 the whole head) and keeps that state in registers across the whole run. The HPB
// heads of a block belong to one B/C group, so B and C are staged once per block; each head's
// decay-masked C B^T blocks are built from C B^T products shared by the block's heads (one wave
// per head) or computed by that head's waves.
//
// Staging: x, B and C tiles are copied global -> LDS by the gfx950 LDS DMA (global_load_lds
// dwordx4), which needs no registers, so a whole sub-chunk is in flight while the previous one is
// computed (scan: two stages, run states: three). The DMA writes each wave instruction's 64 pieces
// of 16 bytes contiguously; the swizzle (16-byte piece c of row t stored at position c ^ key(t))
// is applied by choosing which global piece each lane fetches. B and C are converted to fp16 in
// place after arrival; x stays raw bf16 (the skip term D x uses it exactly) and is converted while
// its fragments are built. Fragments whose K index is the token are read with the gfx950
// transposing LDS load (ds_read_b64_tr_b16). Every fragment access reads at a lane offset
// computed once per kernel; where the registers allow, the fused scan's loop runs two
// sub-chunks per pass, one per stage buffer, so each LDS address is that offset plus an
// immediate.
//
// Matrix-core operand precision: x, B, C enter as exact fp16 copies of the bf16 inputs (inputs
// are assumed to lie in fp16's range); the decay-masked C B^T block, the carried state (for the
// readout) and the decay-weighted x (for the state update) are rounded to fp16; k_run_states
// splits the weighted x of the sequence's last 128 tokens into fp16 high and low parts (two
// passes) where the state is kept in fp32 (the final state). All accumulation is fp32.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- small helpers ------------------------------------------------------------------------------
__device__ __forceinline__ f16x2 cvt_f16x2(float a, float b) {  // v_cvt_pk_f16_f32, RNE
  return __builtin_convertvector(f32x2{a, b}, f16x2);
}
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {  // v_cvt_pk_bf16_f32, RNE
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
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
// 8 bf16 (one 16-byte piece) -> 8 fp16 (exact in fp16's normal range)
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 r) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = __builtin_bit_cast(
        uint32_t, cvt_f16x2(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u)));
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// two packed bf16 (one 32-bit word) -> two floats
__device__ __forceinline__ void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}

// Swizzle of staged tiles: 16-byte piece c of row t is stored at position c ^ key(t), key(t) a
// permutation of t's low bits chosen so that the fragment reads below touch every LDS bank once:
// 16 consecutive rows read at one piece (key injective on 16 rows), and the transposing reads of
// rows {0..3, 8..11} (+4) at a pair of pieces (key >> 1 distinct on those rows; for 128-byte rows,
// which share a bank line in pairs, distinct within each row parity).
template <int PPR>
__device__ __forceinline__ int swz_key(int t) {
  if (PPR >= 16)  // key bits (t2, t0, t1, t3)
    return ((t >> 2) & 1) | ((t & 3) << 1) | (((t >> 3) & 1) << 3);
  return ((t >> 2) & 1) | (((t >> 1) & 1) << 1) | (((t >> 3) & 1) << 2);  // (t2, t1, t3)
}

// Byte offset of 16-byte piece c of row t in a swizzled staged tile with rows of ROW bytes.
template <int ROW>
__device__ __forceinline__ int swz(int t, int c) {
  return t * ROW + ((c ^ swz_key<ROW / 16>(t)) << 4);
}

// LDS DMA (global_load_lds): lane l copies 16 (dma_x4) or 4 (dma_x1) bytes from sbase + voff to
// LDS address lds + 16 l (4 l); sbase and lds are wave-uniform. Issued as inline assembly so that
// the compiler neither counts them nor adds its own conservative waits before LDS reads (it
// treats any such DMA as possibly aliasing every LDS access); the kernels wait for them
// explicitly (wait_vm_*) and publish the data with a barrier. M0 holds the LDS address; the
// compiler reserves M0 and sets it right before its own uses, so it holds no live value here.
// No memory clobber: a DMA writes a stage that no LDS access between two barriers touches (every
// access of that stage lies before the barrier that precedes the DMA, or after the wait and the
// barrier that follow it, and the waits, being volatile with a memory clobber, and the barriers
// keep their order), and it reads only kernel inputs; so the compiler may move the block's other
// LDS accesses across it (measured: -0.7%).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_x4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(sbase), "s"(lds)
               : "m0");
}
__device__ __forceinline__ void dma_x1(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff),
               "s"(sbase), "s"(lds)
               : "m0");
}
#pragma clang diagnostic pop
// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p);
}
// Wait until all of this wave's vector memory operations (DMA included) have completed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// ... all but the most recent n; loads complete in issue order.
template <int n>
__device__ __forceinline__ void wait_vm_but() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// Transposing LDS read: lane i of each 16-lane group receives, in slot q, the (i % 4)-th of the
// four 16-bit values addressed by lane 4 q + i / 4.
__device__ __forceinline__ s16x4 tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// ---- configuration ----------------------------------------------------------------------------
template <int P_, int N_, int NW_ = 4, int PSMAX_ = 64, int T_ = (N_ >= 256 ? 32 : 64)>
struct Fz {
  static constexpr int P = P_, N = N_;
  static constexpr int T = T_;  // tokens per sub-chunk
  static constexpr int NW = NW_, NT = 64 * NW_;
  static constexpr int PS0 = 8192 / N < P ? 8192 / N : P;
  static constexpr int PS = PS0 < PSMAX_ ? PS0 : PSMAX_;  // p columns per wave
  static constexpr int WPH = P / PS, HPB = NW / WPH;  // waves per head, heads per block
  static constexpr int NPT = PS / 16, NNT = N / 16, NKN = N / 32, NIT = T / 16, NJS = T / 32;
  static constexpr int ROW_N = N * 2, ROW_P = P * 2;  // staged row bytes
  static constexpr int BC_BYTES = T * ROW_N, X_BYTES = HPB * T * ROW_P;
  static constexpr int BC_NI = BC_BYTES / 1024;       // DMA instructions per B (or C) tile
  static constexpr int X_NI = X_BYTES / 1024;         // ... per x tile of the block's heads
  static constexpr int DT_BYTES = NW * 256;           // per wave: dt of its head, 64 tokens
  // stage: [B][C (scan only)][x of the HPB heads][dt per wave]
  static constexpr int SCAN_NI = 2 * BC_NI + X_NI, RUN_NI = BC_NI + X_NI;
  static constexpr int SCAN_DT = SCAN_NI * 1024, RUN_DT = RUN_NI * 1024;  // dt offsets
  static constexpr int SCAN_STAGE = SCAN_DT + DT_BYTES, RUN_STAGE = RUN_DT + DT_BYTES;
  static constexpr int NMB = NIT * (NIT + 1) / 2;    // lower-triangle 16x16 blocks of M
  static constexpr int MT_HEAD = NMB * 512;           // a head's fp16 M blocks
  static constexpr int NWA = 5;                       // per-wave token arrays
  static constexpr int WA_BYTES = NW * NWA * T * 4;   // acs2, dt, w, cf, rdiag (phase A: per wave)
  static constexpr int WA_SCAN = HPB * NWA * T * 4;   // phase B: per head
  static constexpr int NSCAN = 2, NRUN = 3;           // stages
  static constexpr int NSPLIT = 128 / T;              // phase A: split sub-chunks (final state)
  // phase B at one wave per head: the sub-chunk's C B^T blocks, fp32, computed once for the block's
  // heads (they share one B/C group)
  static constexpr bool SHARED_CB = WPH == 1 && NMB <= NW;
  static constexpr int CB_SHARED = SHARED_CB ? NMB * 1024 : 0;
  // phase B runs two sub-chunks per loop pass with the stage buffer fixed at compile time (no
  // stage-base additions on LDS addresses) where that fits in the registers: dstate <= 128 at one
  // wave per head
  static constexpr bool UNROLL2 = SHARED_CB && N <= 128;
  static constexpr int SCAN_LDS = NSCAN * SCAN_STAGE + HPB * MT_HEAD + WA_SCAN + CB_SHARED;
  static constexpr int RUN_LDS = NRUN * RUN_STAGE + WA_BYTES;
  static_assert(P % PS == 0 && NW % WPH == 0, "whole waves per head");
  static_assert(N / 8 >= 8 && P / 8 >= 8, "swizzle needs 8 pieces per row");
  static_assert(BC_BYTES % 1024 == 0 && X_BYTES % 1024 == 0, "whole DMA instructions");
  static_assert(BC_BYTES >= 1024, "whole DMA instructions");
};

// Block / wave coordinates shared by both phases: run r, head block hbi (over every group's head
// blocks) and batch entry b.
struct Coord {
  int b, r, grp, hbase, hlast;  // block: batch, run, group, first head, last head of the group
  int wave, lane, g, c16;       // wave, lane, lane group, lane % 16
  int h, p0;                    // this wave's head and first p column
  bool active;                  // this wave's head exists
};

template <class K>
__device__ __forceinline__ Coord coords(const Dims& d, int r, int hbi, int b) {
  Coord c;
  const int hpg = d.H / d.G, hbg = (hpg + K::HPB - 1) / K::HPB;
  c.r = r;
  c.b = b;
  c.grp = hbi / hbg;
  const int first = (hbi % hbg) * K::HPB;
  c.hbase = c.grp * hpg + first;
  c.hlast = c.grp * hpg + hpg - 1;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
  c.lane = threadIdx.x & 63;
  c.g = c.lane >> 4;
  c.c16 = c.lane & 15;
  const int hh = c.wave / K::WPH;
  c.active = first + hh < hpg;
  c.h = c.active ? c.hbase + hh : c.hlast;
  c.p0 = (c.wave % K::WPH) * K::PS;
  return c;
}

// This lane's byte offsets of its DMA pieces, relative to wave-uniform bases. Instruction kk of a
// region with PPR 16-byte pieces per row covers rows kk * RPI .. + RPI - 1 (RPI = 64 / PPR); lane
// l fetches piece (l % PPR) ^ key(t) of row t = kk * RPI + l / PPR. The key depends on t mod 16,
// i.e. on kk mod NPAT = 16 / RPI; a wave's instructions of a region all have kk = wave (mod
// NPAT) (region starts and the wave count are multiples of NPAT), so one offset per region does.
template <int PPR>
struct DmaGeo {
  static constexpr int RPI = 64 / PPR, NPAT = RPI >= 16 ? 1 : 16 / RPI;
  static __device__ __forceinline__ uint32_t lane_off(int wave, int lane, uint32_t ld) {
    const int r = lane / PPR, t = (wave % NPAT) * RPI + r;
    return (uint32_t)r * ld + (uint32_t)(((lane % PPR) ^ swz_key<PPR>(t)) << 4);
  }
};

template <class K, bool WITH_C>
struct DmaLanes {
  using GN = DmaGeo<K::N / 8>;
  using GP = DmaGeo<K::P / 8>;
  static_assert(K::NW % GN::NPAT == 0 && K::BC_NI % GN::NPAT == 0, "B/C pattern per wave");
  static_assert(K::NW % GP::NPAT == 0 && (K::T / GP::RPI) % GP::NPAT == 0 &&
                    K::BC_NI % GP::NPAT == 0,
                "x pattern per wave");
  static constexpr int NBC = (WITH_C ? 2 : 1) * K::BC_NI;  // B (and C) instructions per stage
  static constexpr int NI = NBC + K::X_NI;                  // tile instructions per stage
  static constexpr int XI = K::T / GP::RPI;                 // x instructions per head
  // Direct form: every round of NW instructions (one per wave) lies inside one region (B, C or
  // x) and a round of x instructions covers whole heads (used by the fused scan only at one wave
  // per head: with several waves per head it costs that kernel more registers than it has). A wave's instructions of a stage then
  // read rows at one lane offset per region (wbc, wx: the wave's rows and, for x, its head within
  // the round, folded in), from bases that differ by compile-time multiples of the row strides.
  static constexpr bool DIRECT =
      K::BC_NI % K::NW == 0 && NI % K::NW == 0 && K::NW % XI == 0 && (!WITH_C || K::WPH == 1);
  static constexpr int NPW_DIRECT = NI / K::NW;  // instructions per wave and stage
  uint32_t bc, x;      // generic form: lane offsets of rows 0.. of an instruction
  uint32_t wbc, wx;    // direct form
  __device__ __forceinline__ void init(const Dims& d, const Coord& c) {
    const uint32_t ldbc = (uint32_t)d.G * K::N * 2, ldx = (uint32_t)d.H * K::P * 2;
    bc = GN::lane_off(c.wave, c.lane, ldbc);
    x = GP::lane_off(c.wave, c.lane, ldx);
    if constexpr (DIRECT) {
      constexpr int PPR_N = K::N / 8, PPR_P = K::P / 8;
      const int tb = c.wave * GN::RPI + c.lane / PPR_N;
      wbc = (uint32_t)tb * ldbc + (uint32_t)(((c.lane % PPR_N) ^ swz_key<PPR_N>(tb)) << 4);
      const int tx = (c.wave % XI) * GP::RPI + c.lane / PPR_P;
      wx = (uint32_t)((c.wave / XI) * (K::P * 2)) + (uint32_t)tx * ldx +
           (uint32_t)(((c.lane % PPR_P) ^ swz_key<PPR_P>(tx)) << 4);
    }
  }
  // Opaque copies at the top of every sub-chunk: the offsets stay in registers instead of being
  // recomputed from the lane index where they are used.
  __device__ __forceinline__ void pin() {
    if constexpr (DIRECT) asm volatile("" : "+v"(wbc), "+v"(wx));
  }
};

// Re-derive the lane coordinates through an opaque copy at the top of every sub-chunk, so that the
// compiler recomputes lane-dependent addresses and masks where they are used instead of hoisting
// all of them out of the loop (which costs more registers than the loop body has).
__device__ __forceinline__ void refresh_lane(Coord& c) {
  asm volatile("" : "+v"(c.lane));
  c.g = c.lane >> 4;
  c.c16 = c.lane & 15;
}

// Issue one stage's DMA: [B][C if WITH_C][x of the block's heads], tokens tok0 .. tok0 + T - 1,
// then one instruction per wave for the dt of its own head. In the last, partial sub-chunk rows
// past the sequence end re-read its last row; heads past the group re-read its last head (their
// results are never used). Per wave: NI / NW (+1 for the first NI % NW waves) + 1 instructions,
// in rounds of one instruction per wave; only rounds r0 .. r1 - 1 (and the dt instruction if
// with_dt) are issued here, so that a caller can spread a stage's instructions over its work
// (a wave stalls when it issues more than the memory pipeline accepts). After full unrolling
// the round tests are compile-time.
template <class K, bool WITH_C>
__device__ __forceinline__ void issue_stage(char* st, const u16* x, const u16* Bm, const u16* Cm,
                                            const float* dt, const Dims& d, const Coord& c,
                                            const DmaLanes<K, WITH_C>& dl, int tok0, int r0 = 0,
                                            int r1 = 1 << 20, bool with_dt = true) {
  constexpr int NBC = (WITH_C ? 2 : 1) * K::BC_NI;
  constexpr int NI = NBC + K::X_NI;
  constexpr int PPR_N = K::N / 8, PPR_P = K::P / 8;
  constexpr int RPI_N = 64 / PPR_N, RPI_P = 64 / PPR_P;
  constexpr int XI = K::T / RPI_P;  // x instructions per head
  const int64_t ldbc = (int64_t)d.G * K::N * 2, ldx = (int64_t)d.H * K::P * 2;  // row bytes
  const int64_t row0 = (int64_t)c.b * d.L + tok0;
  const char* bbase = reinterpret_cast<const char*>(Bm) + (row0 * d.G + c.grp) * (K::N * 2);
  const char* cbase = reinterpret_cast<const char*>(Cm) + (row0 * d.G + c.grp) * (K::N * 2);
  const char* xbase = reinterpret_cast<const char*>(x) + (row0 * d.H + c.hbase) * (K::P * 2);
  const char* dbase = reinterpret_cast<const char*>(dt) + (row0 * d.H + c.h) * 4;
  const uint32_t l0 = lds_addr(st);
  const uint32_t ldt = l0 + NI * 1024 + c.wave * 256;
  using DL = DmaLanes<K, WITH_C>;
  if constexpr (DL::DIRECT) {
    if (tok0 + K::T <= d.L) {
      // full stage: round m is this wave's instruction m; x rows of heads past the group re-read
      // its last head (their results are never used)
      const uint32_t lw = l0 + c.wave * 1024;
      const int hw = c.wave / DL::XI, hmax = c.hlast - c.hbase;
      constexpr int BSTEP = K::NW * RPI_N;  // rows between a wave's B (C) instructions
      constexpr int XSTEP = K::NW / DL::XI;  // heads between a wave's x instructions
#pragma unroll
      for (int m = 0; m < DL::NPW_DIRECT; ++m) {
        if (m < r0 || m >= r1) continue;
        const int k0 = K::NW * m;
        if (k0 < NBC) {
          const bool isC = WITH_C && k0 >= K::BC_NI;
          const int j = (isC ? k0 - K::BC_NI : k0) / K::NW;
          dma_x4((isC ? cbase : bbase) + (int64_t)(j * BSTEP) * ldbc, dl.wbc, lw + k0 * 1024);
        } else {
          const int hh = (k0 - NBC) / K::NW * XSTEP + hw;
          dma_x4(xbase + (min(hh, hmax) - hw) * (K::P * 2), dl.wx, lw + k0 * 1024);
        }
      }
      if (with_dt) dma_x1(dbase, (uint32_t)min(c.lane, K::T - 1) * (uint32_t)d.H * 4, ldt);
      return;
    }
  }
  if (!DL::DIRECT && tok0 + K::T <= d.L) {
    // row strides as opaque scalars: their per-instruction multiples are recomputed (scalar ALU)
    // each call rather than held in scalar registers across the loop
    uint32_t lb = (uint32_t)ldbc, lx = (uint32_t)ldx;
    asm volatile("" : "+s"(lb), "+s"(lx));
    // every round of NW instructions lies inside one region: the region tests are compile-time
    constexpr bool EVEN = K::BC_NI % K::NW == 0 && NI % K::NW == 0;
#pragma unroll
    for (int k0 = 0; k0 < NI; k0 += K::NW) {
      if (k0 < r0 * K::NW || k0 >= r1 * K::NW) continue;
      const int k = k0 + c.wave;  // wave-uniform
      if (!EVEN && k >= NI) break;
      const bool bc = EVEN ? k0 < NBC : k < NBC;
      if (bc) {  // B or C
        const bool isC = WITH_C && (EVEN ? k0 >= K::BC_NI : k >= K::BC_NI);
        const int kk = isC ? k - K::BC_NI : k;
        dma_x4((isC ? cbase : bbase) + (uint32_t)(kk * RPI_N) * lb, dl.bc, l0 + k * 1024);
      } else {
        const int kk = k - NBC;
        const int hh = kk / XI, kr = kk % XI;
        const int hoff = min(hh, c.hlast - c.hbase) * (K::P * 2);
        dma_x4(xbase + hoff + (uint32_t)(kr * RPI_P) * lx, dl.x, l0 + k * 1024);
      }
    }
    if (with_dt) dma_x1(dbase, (uint32_t)min(c.lane, K::T - 1) * (uint32_t)d.H * 4, ldt);
  } else {
    const int last = d.L - 1 - tok0;  // last valid row of the sub-chunk
#pragma unroll
    for (int k0 = 0; k0 < NI; k0 += K::NW) {
      if (k0 < r0 * K::NW || k0 >= r1 * K::NW) continue;
      const int k = k0 + c.wave;
      if (k >= NI) break;
      if (k < NBC) {
        const bool isC = WITH_C && k >= K::BC_NI;
        const int kk = isC ? k - K::BC_NI : k;
        const int t = kk * RPI_N + c.lane / PPR_N, cp = c.lane % PPR_N;
        const uint32_t o =
            (uint32_t)(min(t, last) * ldbc) + (uint32_t)((cp ^ swz_key<PPR_N>(t)) << 4);
        dma_x4(isC ? cbase : bbase, o, l0 + k * 1024);
      } else {
        const int kk = k - NBC;
        const int hh = kk / XI, kr = kk % XI;
        const int hoff = min(hh, c.hlast - c.hbase) * (K::P * 2);
        const int t = kr * RPI_P + c.lane / PPR_P, cp = c.lane % PPR_P;
        const uint32_t o = (uint32_t)(hoff + min(t, last) * ldx) +
                           (uint32_t)((cp ^ swz_key<PPR_P>(t)) << 4);
        dma_x4(xbase, o, l0 + k * 1024);
      }
    }
    if (with_dt) dma_x1(dbase, (uint32_t)min(c.lane, last) * (uint32_t)d.H * 4, ldt);
  }
}

// Convert this wave's own DMA'd B (and C) pieces of a stage from bf16 to fp16 in place.
template <class K, bool WITH_C>
__device__ __forceinline__ void convert_stage(char* st, const Coord& c) {
  constexpr int NBC = (WITH_C ? 2 : 1) * K::BC_NI;
#pragma unroll
  for (int k0 = 0; k0 < NBC; k0 += K::NW) {
    if (k0 + c.wave >= NBC) break;
    uint4* p = reinterpret_cast<uint4*>(st + (k0 + c.wave) * 1024 + c.lane * 16);
    *p = bf16x8_to_f16x8(*p);
  }
}

// Effective dt of this wave's head for the tokens of a staged sub-chunk (lane l: token tok0 + l),
// 0 past the sequence end; dts is the stage's dt region (this wave's own DMA: readable after its
// own wait), dtb the head's dt bias.
template <class K>
__device__ __forceinline__ float stage_dt(const char* dts, const Dims& d, const Coord& c, int tok0,
                                          float dtb) {
  const float v = dt_effective(reinterpret_cast<const float*>(dts + c.wave * 256)[c.lane], dtb, d);
  return (c.lane < K::T && tok0 + c.lane < d.L && c.active) ? v : 0.f;
}

// DPP lane moves (VALU, no LDS round trip); lanes whose source is outside the pattern read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}
// Inclusive prefix sum over the wave's 64 lanes: within rows of 16 by shifts of 1, 2, 4, 8, then
// row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then rows 0-1's total into rows
// 2-3 (row_bcast:31).
__device__ __forceinline__ float wave_scan(float v) {
  v += dpp_mov<0x111, 0xf>(v);
  v += dpp_mov<0x112, 0xf>(v);
  v += dpp_mov<0x114, 0xf>(v);
  v += dpp_mov<0x118, 0xf>(v);
  v += dpp_mov<0x142, 0xa>(v);
  v += dpp_mov<0x143, 0xc>(v);
  return v;
}
// Lane 15 of each row of 16, broadcast to the row (row_newbcast:15).
__device__ __forceinline__ float row_last(float v) { return dpp_mov<0x15f, 0xf>(v); }

// Per-sub-chunk decay bookkeeping of one wave (lane l = token l, acs = inclusive cumulative
// log-decay from the sub-chunk start, e(l) the last token of l's 16-token block). Into the wave's
// LDS arrays (only w when WEIGHTS_ONLY):
//   acs2 = acs log2(e);  dt;  w = exp(shift + acs_end - acs) dt (state weights, anchored shift
//   (<= 0) past the sub-chunk end);
//   cf = exp(acs_e - acs) dt (column factor of the decay mask through the end of the token's
//   block; both of its factors are <= 1);  rdiag = exp(acs - acs_e) >= 1 (its row factor inside
//   the token's own block).
// Returns acs_end; *fast tells whether every block's decay span acs - acs_e stays below 2^100 in
// base 2, so that rdiag and cf stay inside fp32's normal range and the factored diagonal is exact
// up to rounding.
template <class K, bool WEIGHTS_ONLY = false>
__device__ __forceinline__ float decay_terms(float dv, float a_h, float* wa, const Coord& c,
                                             bool* fast = nullptr, float shift = 0.f) {
  const float acs = wave_scan(a_h * dv);
  const float acs_end = __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acs), K::T - 1));
  const float span = acs - row_last(acs);  // >= 0
  if (c.lane < K::T) {
    wa[2 * K::T + c.lane] = __expf(shift + (acs_end - acs)) * dv;
    if constexpr (!WEIGHTS_ONLY) {
      wa[c.lane] = acs * kLog2e;
      wa[K::T + c.lane] = dv;
      wa[3 * K::T + c.lane] = __expf(-span) * dv;
      if (fast) wa[4 * K::T + c.lane] = __expf(span);
    }
  }
  if (fast) *fast = __ballot(span * kLog2e >= 100.f) == 0;
  return acs_end;
}

// Lane-constant byte offsets of the LDS fragment accesses of both phases, relative to the tile they read,
// computed once per kernel. The swizzle key sees only a row's low 4 bits and a piece's low bits,
// so the unrolled loop indices it does not see (token-tile rows, high piece bits) enter as
// immediates on top of these.

template <class K>
struct ScanLane {
  static constexpr int PPR_N = K::N / 8;
  static constexpr int KP = PPR_N >= 16 ? 4 : 2;   // K steps over n with distinct patterns
  static constexpr int NP = PPR_N >= 16 ? 8 : 4;   // n tiles with distinct patterns
  uint32_t cro[KP][2];      // readout C^T fragment: row c16, piece 4 kn + 2 h + g/2, half g&1
  // B^T fragment (transposing read) of n tile 0: rows 8 g + j/4 (+4), pieces 0..1; n tile b < NP
  // reads at btr0 ^ (b << 5) (its pieces 2 b, 2 b + 1: the swizzle key flips bits of the piece
  // index, and the row's own offset has no bits in 5..7 below the NP tiles)
  uint32_t btr0[2];
  uint32_t xtr[K::NPT][2];  // x fragment (transposing read)
  uint32_t cbr[KP];         // C B^T inputs: row c16, piece 4 kn + g
  uint32_t epi[K::NPT];     // y write into the x tile: row c16, piece (p0 + 16 pt) / 8 + g/2
  uint32_t mwr;             // M block write: row c16, columns 4 g .. 4 g + 3
  uint32_t mrd;             // M fragment read: block + g/2, row c16, columns 8 (g&1) .. + 7
  __device__ __forceinline__ void init(const Coord& c) {
    const int g = c.g, c16 = c.c16, j = c.lane & 15;
    const int sw = (c16 >> 3) & 1;  // M rows 8..15 of a block hold their two pieces swapped
    mwr = c16 * 32 + (((g >> 1) ^ sw) << 4) + ((g & 1) << 3);
    mrd = (g >> 1) * 512 + c16 * 32 + (((g & 1) ^ sw) << 4);
#pragma unroll
    for (int b = 0; b < KP; ++b) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        cro[b][h] = swz<K::ROW_N>(c16, 4 * b + 2 * h + (g >> 1)) + ((g & 1) << 3);
      cbr[b] = swz<K::ROW_N>(c16, 4 * b + g);
    }
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int t = 8 * g + (j >> 2) + 4 * hi;
      btr0[hi] = swz<K::ROW_N>(t, (j & 3) >> 1) + ((j & 1) << 3);
#pragma unroll
      for (int pt = 0; pt < K::NPT; ++pt)
        xtr[pt][hi] = swz<K::ROW_P>(t, ((c.p0 + 16 * pt) >> 3) + ((j & 3) >> 1)) + ((j & 1) << 3);
    }
#pragma unroll
    for (int pt = 0; pt < K::NPT; ++pt)
      epi[pt] = swz<K::ROW_P>(c16, ((c.p0 + 16 * pt) >> 3) + (g >> 1)) + ((g & 1) << 3);
  }
};

// Two transposing reads at precomputed lane offsets -> one 8-value K fragment.
__device__ __forceinline__ s16x8 tr8(const char* base, uint32_t lo, uint32_t hi) {
  const s16x4 a = tr4(base + lo), b = tr4(base + hi);
  return s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <bool V>
struct Flag {
  static constexpr bool value = V;
};

// ---- phase A: run states ------------------------------------------------------------------------
// state_r = sum_{t in run} exp(sum_{k in (t, end]} dt_k A) dt_t x_t B_t^T (zero entry state) and
// logdecay_r = sum_{t in run} dt_t A. Walked backwards: per sub-chunk, S += B^T (w x) with the
// weights anchored at the run end. The weighted x of the first `nsplit` sub-chunks walked (the
// last tokens of the run) is split into fp16 high and low parts (two passes), the rest rounded
// once: a token's rounding error scales with its weight, and the weights are largest at the run
// end (dt itself there; a single such term can dominate an entry of the state), while earlier
// tokens carry decayed weights or, in slowly decaying heads, many comparable terms whose
// independent roundings average out. Leaves the state in S (lane: p = p0 + 16 pt + c16,
// n = 16 nt + 4 g + 0..3) and returns the log-decay.
template <class K>
__device__ __forceinline__ float run_state(char* smem, const Coord& c, const u16* __restrict__ x,
                                           const u16* __restrict__ Bm,
                                           const float* __restrict__ dt, float a_h, float dtb,
                                           const Dims& d, int s_begin, int s_end, int nsplit,
                                           f32x4 (&S)[K::NNT][K::NPT]) {
  using M = Mma<f16>;
  DmaLanes<K, false> dl;
  dl.init(d, c);
  ScanLane<K> sl;
  sl.init(c);
  using SL = ScanLane<K>;
  constexpr int T = K::T;
  float* wa = reinterpret_cast<float*>(smem + K::NRUN * K::RUN_STAGE) + c.wave * K::NWA * T;
  const int xoff = K::BC_BYTES + (c.wave / K::WPH) * (T * K::ROW_P);

#pragma unroll
  for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < K::NPT; ++pt) S[nt][pt] = zero4();
  // The run is walked backwards, last sub-chunk first, with token weights anchored at the run
  // end: w_t = exp(sum of a over (t, run end]) dt_t. The state then never needs decaying.
  float rem = 0.f;  // log-decay from the end of the current sub-chunk to the run end

  // prologue: stages of the last two sub-chunks
  issue_stage<K, false>(smem, x, Bm, nullptr, dt, d, c, dl, (s_end - 1) * T);
  if (s_end - 2 >= s_begin)
    issue_stage<K, false>(smem + K::RUN_STAGE, x, Bm, nullptr, dt, d, c, dl, (s_end - 2) * T);
  // DMA instructions this wave issues per stage: NLO or NLO + 1 tile pieces, and its dt
  constexpr int NLO = K::RUN_NI / K::NW + 1;
  const bool hi = c.wave < K::RUN_NI % K::NW;

  auto body = [&](int s, auto split_c) {
    constexpr bool SPL = decltype(split_c)::value;
    dl.pin();
    const int cur = (s_end - 1 - s) % K::NRUN;
    char* st = smem + cur * K::RUN_STAGE;
    // this stage's DMA done; the next stage's (this wave's instructions for it were issued after
    // this stage's) may still be in flight
    if (s - 1 < s_begin)
      wait_vm_all();
    else if (hi)
      wait_vm_but<NLO + 1>();
    else
      wait_vm_but<NLO>();
    const float dv = stage_dt<K>(st + K::RUN_DT, d, c, s * T, dtb);
    convert_stage<K, false>(st, c);
    __syncthreads();  // stage visible to all waves; every wave is done with sub-chunk s + 1
    // the DMA of sub-chunk s - 2 (into the stage of s + 1), spread over the K steps below
    const bool more = s - 2 >= s_begin;
    constexpr int NRND = (K::RUN_NI + K::NW - 1) / K::NW, RPJ = (NRND + K::NJS - 1) / K::NJS;
    const uint32_t bt0 = sl.btr0[0], bt1 = sl.btr0[1];
    rem += decay_terms<K, true>(dv, a_h, wa, c, nullptr, rem);
#pragma unroll
    for (int js = 0; js < K::NJS; ++js) {
      if (more)
        issue_stage<K, false>(smem + ((cur + 2) % K::NRUN) * K::RUN_STAGE, x, Bm, nullptr, dt, d,
                              c, dl, (s - 2) * T, js * RPJ, (js + 1) * RPJ, js == K::NJS - 1);
      const float4 w0 = *reinterpret_cast<const float4*>(wa + 2 * T + 32 * js + 8 * c.g);
      const float4 w1 = *reinterpret_cast<const float4*>(wa + 2 * T + 32 * js + 8 * c.g + 4);
      const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      f16x8 xhi[K::NPT], xlo[K::NPT];
#pragma unroll
      for (int pt = 0; pt < K::NPT; ++pt) {
        float v[8], lo[8];
        const s16x8 r = tr8(st + xoff + 32 * js * K::ROW_P, sl.xtr[pt][0], sl.xtr[pt][1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float((uint32_t)(uint16_t)r[e] << 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= wj[e];
        xhi[pt] = cvt_f16x8(v);
        if constexpr (SPL) {
#pragma unroll
          for (int e = 0; e < 8; ++e) lo[e] = v[e] - (float)xhi[pt][e];
          xlo[pt] = cvt_f16x8(lo);
        }
      }
#pragma unroll
      for (int nt = 0; nt < K::NNT; ++nt) {
        const char* bb = st + 32 * js * K::ROW_N + (nt / SL::NP) * (16 * 2 * SL::NP);
        const f16x8 bt = __builtin_bit_cast(
            f16x8, tr8(bb, bt0 ^ ((nt % SL::NP) << 5), bt1 ^ ((nt % SL::NP) << 5)));
#pragma unroll
        for (int pt = 0; pt < K::NPT; ++pt) {
          S[nt][pt] = M::mma(bt, xhi[pt], S[nt][pt]);
          if constexpr (SPL) S[nt][pt] = M::mma(bt, xlo[pt], S[nt][pt]);
        }
      }
    }
  };
  int s = s_end - 1;
  for (const int s_lo = max(s_begin, s_end - nsplit); s >= s_lo; --s) body(s, Flag<true>{});
  for (; s >= s_begin; --s) body(s, Flag<false>{});
  return rem;
}

// Store this wave's state slice S (layout of run_state) to the [P, N] state at `so` (the head's
// state, row-major), plus e0 times the matching slice of h (when not null).
template <class K>
__device__ __forceinline__ void store_state(const f32x4 (&S)[K::NNT][K::NPT], const Coord& c,
                                            float* __restrict__ so, const float* __restrict__ h,
                                            float e0) {
#pragma unroll
  for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < K::NPT; ++pt) {
      const int o = (c.p0 + 16 * pt + c.c16) * K::N + 16 * nt + 4 * c.g;
      f32x4 v = S[nt][pt];
      if (h) {
        const float4 q = *reinterpret_cast<const float4*>(h + o);
        v += e0 * f32x4{q.x, q.y, q.z, q.w};
      }
      *reinterpret_cast<float4*>(so + o) = make_float4(v[0], v[1], v[2], v[3]);
    }
}


// The same slice rounded to fp16 (a run's state handed to the chain).
template <class K>
__device__ __forceinline__ void store_state_h(const f32x4 (&S)[K::NNT][K::NPT], const Coord& c,
                                              u16* __restrict__ so) {
#pragma unroll
  for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < K::NPT; ++pt) {
      const int o = (c.p0 + 16 * pt + c.c16) * K::N + 16 * nt + 4 * c.g;
      const f32x4 v = S[nt][pt];
      *reinterpret_cast<uint2*>(so + o) =
          make_uint2(__builtin_bit_cast(uint32_t, cvt_f16x2(v[0], v[1])),
                     __builtin_bit_cast(uint32_t, cvt_f16x2(v[2], v[3])));
    }
}

// Store the bf16 y tile that phase B left in the x tile of a stage: this wave's p-slice of its head,
// rows tok0 .. tok0 + T - 1 (rows past the sequence end skipped), 16 bytes per lane. Round k
// covers rows k * RPR .. + RPR - 1; the swizzle key repeats every 16 rows, so the LDS lane offset
// takes 16 / RPR values (at least one).
template <class K>
__device__ __forceinline__ void store_y(const char* xt, u16* y, const Dims& d, const Coord& c,
                                        int tok0) {
  if (!c.active) return;
  constexpr int PPR = K::PS / 8;  // pieces per row of the wave's slice
  constexpr int RPR = 64 / PPR;   // rows per round
  constexpr int ROUNDS = K::T / RPR;
  constexpr int NPAT = RPR >= 16 ? 1 : 16 / RPR;
  static_assert(K::T % RPR == 0 && (RPR % 16 == 0 || 16 % RPR == 0), "whole store rounds");
  const int r = c.lane / PPR, cp = (c.p0 >> 3) + c.lane % PPR;
  const int64_t ld = (int64_t)d.H * K::P;  // y row stride (elements)
  u16* yb = y + (((int64_t)c.b * d.L + tok0) * d.H + c.h) * K::P + (cp << 3) + r * ld;
  int xl[NPAT];
#pragma unroll
  for (int q = 0; q < NPAT; ++q) xl[q] = swz<K::ROW_P>(q * RPR + r, cp);
  const int nrow = d.L - tok0;  // valid rows
#pragma unroll
  for (int k = 0; k < ROUNDS; ++k) {
    const int row0 = k * RPR;
    const uint4 v = *reinterpret_cast<const uint4*>(xt + xl[k % NPAT] + (row0 / (NPAT * RPR)) *
                                                                          (NPAT * RPR) * K::ROW_P);
    if (nrow >= K::T || row0 + r < nrow) {  // y is not read again: nontemporal
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                  reinterpret_cast<u32x4*>(yb + (int64_t)row0 * ld));
    }
  }
}

// ---- phase B helpers: the fused scan -------------------------------------------------------------
// Per sub-chunk (tokens i, j), with acs the inclusive cumulative log-decay from its start:
//   y_i = sum_{j <= i} M_ij x_j + exp(acs_i) C_i . S,
//   M_ij = (C_i . B_j) exp(acs_i - acs_j) dt_j (j <= i), plus D on the diagonal (skip term)
//   S  <- exp(acs_end) S + sum_j exp(acs_end - acs_j) dt_j x_j B_j^T
// The lower-triangle 16x16 blocks of a head's M are built from C B^T accumulators and left in LDS
// in fp16: at one wave per head the C B^T blocks are computed once for the block's heads (which
// share one B/C group) and each wave applies its head's decay; with several waves per head those
// waves split the head's blocks. Each wave then computes y^T for its p-slice
// (rows p, columns i), so every accumulator lane holds four consecutive p of one token: the
// readout's A operand comes straight from the state accumulators (K index n in accumulator
// order), and y leaves in 8-byte row pieces.

// Byte offset of M block (row block it, column block jt <= it) in a head's M area.
__device__ __forceinline__ constexpr int mblk(int it, int jt) {
  return (it * (it + 1) / 2 + jt) * 512;
}

// One M block from its C B^T accumulators (transposed: lane (g, c16) holds tokens
// j = 16 jt + 4 g + rr, rr = 0..3, of row i = 16 it + c16), written to the head's M area in fp16.
// Blocks below the diagonal factor the decay through the end of column block jt (both factors
// <= 1); diagonal blocks through the end of their own block (rdiag >= 1, cf <= dt) when the
// sub-chunk's block spans allow it (fast), else directly.
template <class K>
__device__ __forceinline__ void put_m(f32x4 acc, int it, int jt, const float* wa, float d_h,
                                      bool fast, char* mh, const ScanLane<K>& sl, const Coord& c) {
  constexpr int T = K::T;
  const int i = 16 * it + c.c16, jb = 16 * jt + 4 * c.g;
  const float4 cf = *reinterpret_cast<const float4*>(wa + 3 * T + jb);
  const float cfv[4] = {cf.x, cf.y, cf.z, cf.w};
  float m[4];
  if (jt < it) {
    const float r = __builtin_amdgcn_exp2f(wa[i] - wa[16 * jt + 15]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) m[rr] = acc[rr] * cfv[rr] * r;
  } else if (fast) {
    const float r = wa[4 * T + i];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float v = acc[rr] * cfv[rr] * r;
      m[rr] = (jb + rr < i) ? v : ((jb + rr == i) ? v + d_h : 0.f);
    }
  } else {
    const float acs2_i = wa[i];
    const float4 aj = *reinterpret_cast<const float4*>(wa + jb);
    const float4 dj = *reinterpret_cast<const float4*>(wa + T + jb);
    const float ajv[4] = {aj.x, aj.y, aj.z, aj.w}, djv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float v = acc[rr] * __builtin_amdgcn_exp2f(fminf(acs2_i - ajv[rr], 0.f)) * djv[rr];
      m[rr] = (jb + rr < i) ? v : ((jb + rr == i) ? v + d_h : 0.f);
    }
  }
  const f16x2 lo = cvt_f16x2(m[0], m[1]), hi = cvt_f16x2(m[2], m[3]);
  *reinterpret_cast<uint2*>(mh + mblk(it, jt) + sl.mwr) =
      make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// C B^T fragment (rows r0 .. r0 + 15 of a converted B or C tile, K step kn over n).
template <class K>
__device__ __forceinline__ f16x8 bc_frag(const char* tile, int r0, int kn, const ScanLane<K>& sl) {
  using SL = ScanLane<K>;
  return *reinterpret_cast<const f16x8*>(tile + r0 * K::ROW_N + sl.cbr[kn % SL::KP] +
                                         (kn / SL::KP) * (16 * SL::KP * 4));
}

// This wave's share of its head's M blocks for the staged sub-chunk (several waves per head; at
// one wave per head the C B^T blocks are shared by the block's heads, see shared_cb).
// dma(kn) issues the next stage's share for K step kn (0 .. NKN - 1), spread over the work.
template <class K, class Dma>
__device__ __forceinline__ void build_m(const char* Bh, const char* Ch, const float* wa, float d_h,
                                        bool fast, char* mh, const ScanLane<K>& sl,
                                        const Coord& c, Dma&& dma) {
  using M = Mma<f16>;
  constexpr int NIT = K::NIT;
  const int hw = c.wave % K::WPH;  // wave within the head (wave-uniform)
  if constexpr (NIT == 4 && K::WPH == 2) {
    // row blocks {0, 3} or {1, 2}: five blocks each, C fragments of two row blocks and B
    // fragments of (up to) four column blocks per K step
    const int ia = hw, ib = 3 - hw;
    f32x4 a0 = zero4(), a1 = zero4(), b0 = zero4(), b1 = zero4(), b2 = zero4(), b3 = zero4();
#pragma unroll
    for (int kn = 0; kn < K::NKN; ++kn) {
      dma(kn);
      const f16x8 ca = bc_frag<K>(Ch, 16 * ia, kn, sl), cb = bc_frag<K>(Ch, 16 * ib, kn, sl);
      f16x8 bf[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) bf[jt] = bc_frag<K>(Bh, 16 * jt, kn, sl);
      a0 = M::mma(bf[0], ca, a0);
      b0 = M::mma(bf[0], cb, b0);
      b1 = M::mma(bf[1], cb, b1);
      b2 = M::mma(bf[2], cb, b2);
      if (hw) {
        a1 = M::mma(bf[1], ca, a1);
      } else {
        b3 = M::mma(bf[3], cb, b3);
      }
    }
    put_m<K>(a0, ia, 0, wa, d_h, fast, mh, sl, c);
    put_m<K>(b0, ib, 0, wa, d_h, fast, mh, sl, c);
    put_m<K>(b1, ib, 1, wa, d_h, fast, mh, sl, c);
    put_m<K>(b2, ib, 2, wa, d_h, fast, mh, sl, c);
    if (hw)
      put_m<K>(a1, 1, 1, wa, d_h, fast, mh, sl, c);
    else
      put_m<K>(b3, 3, 3, wa, d_h, fast, mh, sl, c);
  } else {
    // blocks in row-major order over the lower triangle, block q to the head's wave q % WPH
#pragma unroll
    for (int kn = 0; kn < K::NKN; ++kn) dma(kn);
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int jt = 0; jt <= it; ++jt) {
        if ((it * (it + 1) / 2 + jt) % K::WPH != hw) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int kn = 0; kn < K::NKN; ++kn)
          acc = M::mma(bc_frag<K>(Bh, 16 * jt, kn, sl), bc_frag<K>(Ch, 16 * it, kn, sl), acc);
        put_m<K>(acc, it, jt, wa, d_h, fast, mh, sl, c);
      }
  }
}

// Shared C B^T blocks (one wave per head): block q of the lower triangle (row-major) is computed
// by wave q for the whole block and left in LDS in fp32, in the lane layout put_m takes; every
// wave issues the next stage's DMA share for K steps 0 .. NKN - 1 meanwhile.
template <class K, class Dma>
__device__ __forceinline__ void shared_cb(const char* Bh, const char* Ch, char* cbs,
                                          const ScanLane<K>& sl, const Coord& c, Dma&& dma) {
  using M = Mma<f16>;
  const bool mine = c.wave < K::NMB;  // wave-uniform
  const int q = mine ? c.wave : 0;
  const int it = (q >= 1) + (q >= 3) + (q >= 6), jt = q - it * (it + 1) / 2;
  static_assert(K::NMB <= 10, "blocks of at most four row blocks");
  f32x4 acc = zero4();
#pragma unroll
  for (int kn = 0; kn < K::NKN; ++kn) {
    dma(kn);
    if (mine) acc = M::mma(bc_frag<K>(Bh, 16 * jt, kn, sl), bc_frag<K>(Ch, 16 * it, kn, sl), acc);
  }
  if (mine) *reinterpret_cast<f32x4*>(cbs + q * 1024 + c.lane * 16) = acc;
}

// This wave's head's M blocks from the shared C B^T blocks.
template <class K>
__device__ __forceinline__ void m_from_shared(const char* cbs, const float* wa, float d_h, bool fast,
                                              char* mh, const ScanLane<K>& sl, const Coord& c) {
#pragma unroll
  for (int it = 0; it < K::NIT; ++it)
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      const int q = it * (it + 1) / 2 + jt;
      const f32x4 acc = *reinterpret_cast<const f32x4*>(cbs + q * 1024 + c.lane * 16);
      put_m<K>(acc, it, jt, wa, d_h, fast, mh, sl, c);
    }
}

// ---- phase B: fused scan ------------------------------------------------------------------------
// The state entering the run for this wave's head ([P, N], row-major): h0_head (fp32) or
// hin_head (fp16, from the chain), at most one of them not null; both null: zero.
template <class K>
__device__ __forceinline__ void fused_scan(char* smem, Coord c, const u16* __restrict__ x,
                                           const u16* __restrict__ Bm, const u16* __restrict__ Cm,
                                           const float* __restrict__ dt,
                                           const float* __restrict__ Av,
                                           const float* __restrict__ Dv,
                                           const float* __restrict__ h0_head,
                                           const u16* __restrict__ hin_head, u16* __restrict__ y,
                                           const Dims& d, int s_begin, int s_end) {
  using M = Mma<f16>;
  DmaLanes<K, true> dl;
  dl.init(d, c);
  ScanLane<K> sl;
  sl.init(c);
  using SL = ScanLane<K>;
  constexpr int T = K::T, NPT = K::NPT, NIT = K::NIT;
  const int hb = c.wave / K::WPH;  // head within the block
  char* mh = smem + K::NSCAN * K::SCAN_STAGE + hb * K::MT_HEAD;
  // token arrays of the head: both of its waves compute and write identical values; they are
  // read only between the two barriers of a sub-chunk
  float* wa =
      reinterpret_cast<float*>(smem + K::NSCAN * K::SCAN_STAGE + K::HPB * K::MT_HEAD) +
      hb * K::NWA * T;
  const int xoff = 2 * K::BC_BYTES + hb * (T * K::ROW_P);
  const float a_h = Av[c.h], d_h = Dv[c.h], dtb = dt_bias_of(d, c.h);
  char* cbs = smem + K::NSCAN * K::SCAN_STAGE + K::HPB * K::MT_HEAD + K::WA_SCAN;

  // the first stage's DMA first: it and the entry state below are then in flight together
  issue_stage<K, true>(smem, x, Bm, Cm, dt, d, c, dl, s_begin * T);

  // carried state S^T tiles (rows n, columns p): lane holds p = p0 + 16 pt + c16,
  // n = 16 nt + 4 g + 0..3
  f32x4 S[K::NNT][NPT];
  if (h0_head != nullptr) {
    const float* hr = h0_head + (int64_t)c.p0 * K::N;
#pragma unroll
    for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const float4 v =
            *reinterpret_cast<const float4*>(hr + (16 * pt + c.c16) * K::N + 16 * nt + 4 * c.g);
        S[nt][pt] = f32x4{v.x, v.y, v.z, v.w};
      }
  } else if (hin_head != nullptr) {
    const u16* hr = hin_head + (int64_t)c.p0 * K::N;
#pragma unroll
    for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint2 v =
            *reinterpret_cast<const uint2*>(hr + (16 * pt + c.c16) * K::N + 16 * nt + 4 * c.g);
        const f16x2 lo = __builtin_bit_cast(f16x2, v.x), hi = __builtin_bit_cast(f16x2, v.y);
        S[nt][pt] = f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) S[nt][pt] = zero4();
  }
  {
    // the compiler's own wait for these loads (it does not see the DMA waits, which are inline
    // assembly), here rather than at the state's first use inside the loop; it also covers the
    // first stage's DMA, which the loop waits for anyway
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }

  int ytok = -1;  // first token of the sub-chunk whose y waits in the previous stage's x tile

  // Sub-chunks in pairs where that fits in the registers: two unrolled copies, one per stage
  // buffer, so that in each the stage is a compile-time constant and every LDS address a lane
  // offset plus an immediate.
  constexpr int UN = K::UNROLL2 ? 2 : 1;
  for (int s0 = s_begin; s0 < s_end; s0 += UN) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int s = s0 + u;
      if (UN > 1 && s >= s_end) break;
      const int cur = UN > 1 ? u : (s - s_begin) & 1;
      refresh_lane(c);
      dl.pin();
      char* st = smem + cur * K::SCAN_STAGE;
      const char* Bh = st;
      const char* Ch = st + K::BC_BYTES;
      const char* xt = st + xoff;
      wait_vm_all();  // this stage's DMA and the y stores of the previous round
      if (ytok >= 0) store_y<K>(smem + (cur ^ 1) * K::SCAN_STAGE + xoff, y, d, c, ytok);
      const float dv = stage_dt<K>(st + K::SCAN_DT, d, c, s * T, dtb);
      convert_stage<K, true>(st, c);
      // the head's decay bookkeeping needs only its dt: done while other waves finish converting
      bool fast;
      const float acs_end = decay_terms<K>(dv, a_h, wa, c, &fast);
      // A: stage and token arrays visible; every wave is done with sub-chunk s - 1
      __syncthreads();
      // the next stage's DMA (into the stage every wave is done with), spread over the work:
      // slots 0 .. NKN - 1 are the K steps of the C B^T / M blocks, slot NKN follows the M
      // blocks, slots NKN + 1 .. 2 NKN are the readout's K steps (the dt goes with the last).
      // With the C B^T blocks shared (one wave per head) one round goes into the C B^T step, one
      // after the M blocks and the rest over the readout (a wave issuing several rounds back to
      // back waits for the memory pipeline; measured -1% at the headline shape, -1.6% at 65536
      // tokens); otherwise the rounds are spread evenly over the C B^T and readout steps (at
      // headdim 128, dstate 256 the other spread measured 1.7% slower).
      const bool more = s + 1 < s_end;
      constexpr int NSLOT = 2 * K::NKN + 1;
      constexpr int NRND = (K::SCAN_NI + K::NW - 1) / K::NW;
      constexpr int RR = NRND > 2 ? (NRND - 2 + K::NKN - 1) / K::NKN : 0;  // per readout step
      constexpr int RPS = (NRND + 2 * K::NKN - 1) / (2 * K::NKN);         // even spread
      auto dma = [&](int slot) {
        int r0 = 0, r1 = 0;
        if constexpr (K::SHARED_CB) {
          if (slot == 0) {
            r1 = 1;
          } else if (slot == K::NKN) {
            r0 = 1;
            r1 = 2;
          } else if (slot > K::NKN) {
            r0 = 2 + (slot - K::NKN - 1) * RR;
            r1 = r0 + RR;
          }
        } else if (slot != K::NKN) {
          const int k = slot < K::NKN ? slot : slot - 1;
          r0 = k * RPS;
          r1 = r0 + RPS;
        }
        if (more && (r1 > r0 || slot == NSLOT - 1))
          issue_stage<K, true>(smem + (cur ^ 1) * K::SCAN_STAGE, x, Bm, Cm, dt, d, c, dl,
                               (s + 1) * T, r0, r1, slot == NSLOT - 1);
      };

      f32x4 Y[NPT][NIT];
      f16x8 w16[K::NJS];  // state weights of the lane's 8 tokens per K step
      if constexpr (K::SHARED_CB) {
        shared_cb<K>(Bh, Ch, cbs, sl, c, dma);
        __syncthreads();  // the shared C B^T blocks visible to every wave
        if (c.active) m_from_shared<K>(cbs, wa, d_h, fast, mh, sl, c);
      }
      if (!c.active) {
#pragma unroll
        for (int slot = K::SHARED_CB ? K::NKN : 0; slot < NSLOT; ++slot) dma(slot);
      } else {
        if constexpr (!K::SHARED_CB) build_m<K>(Bh, Ch, wa, d_h, fast, mh, sl, c, dma);
        dma(K::NKN);

        // readout of the carried state: Y^T = S C^T (K index n in accumulator order)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
          for (int it = 0; it < NIT; ++it) Y[pt][it] = zero4();
#pragma unroll
        for (int kn = 0; kn < K::NKN; ++kn) {
          dma(K::NKN + 1 + kn);
          f16x8 sa[NPT];
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            const float v[8] = {S[2 * kn][pt][0],     S[2 * kn][pt][1],     S[2 * kn][pt][2],
                                S[2 * kn][pt][3],     S[2 * kn + 1][pt][0], S[2 * kn + 1][pt][1],
                                S[2 * kn + 1][pt][2], S[2 * kn + 1][pt][3]};
            sa[pt] = cvt_f16x8(v);
          }
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const char* crow = Ch + 16 * it * K::ROW_N + (kn / SL::KP) * (16 * SL::KP * 4);
            uint32_t o0 = sl.cro[kn % SL::KP][0], o1 = sl.cro[kn % SL::KP][1];
            // later row blocks read at offsets the compiler cannot relate to the first's: it
            // would merge the row blocks' reads at one offset into one instruction whose halves
            // then need register moves into the fragments
            if (it > 0) asm volatile("" : "+v"(o0), "+v"(o1));
            const uint2 lo = *reinterpret_cast<const uint2*>(crow + o0);
            const uint2 hi = *reinterpret_cast<const uint2*>(crow + o1);
            const f16x8 cf = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) Y[pt][it] = M::mma(sa[pt], cf, Y[pt][it]);
          }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const float e = __builtin_amdgcn_exp2f(wa[16 * it + c.c16]);
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) Y[pt][it] *= e;
        }
#pragma unroll
        for (int js = 0; js < K::NJS; ++js) {
          const float4 w0 = *reinterpret_cast<const float4*>(wa + 2 * T + 32 * js + 8 * c.g);
          const float4 w1 = *reinterpret_cast<const float4*>(wa + 2 * T + 32 * js + 8 * c.g + 4);
          const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          w16[js] = cvt_f16x8(wv);
        }
      }
      if constexpr (K::WPH > 1) {
        __syncthreads();  // B: every M block of the head visible to both of its waves
      } else {
        // one wave per head: it alone writes and reads its M blocks and token arrays (the shared
        // C B^T blocks were published by the barrier before them), and a wave's LDS accesses
        // complete in order, so only the compiler must keep them in program order
        asm volatile("" ::: "memory");
      }
      if (!c.active) continue;

      // Raised wave priority from here to the y tile: the SIMD's other wave is then usually in
      // its readout or bookkeeping, and the state update's matrix-core chain is the longer one
      // (measured: fused scan -2.5%).
      __builtin_amdgcn_s_setprio(1);
      // with two sub-chunks per pass the B^T fragment offsets of the n tiles are formed here, per
      // sub-chunk (held across the loop they would take 16 registers, more than are left; with one
      // per pass they are held: measured faster there)
      uint32_t bt0 = sl.btr0[0], bt1 = sl.btr0[1];
      if constexpr (K::UNROLL2) asm volatile("" : "+v"(bt0), "+v"(bt1));
      // state decay (the readout above used the entry state)
      const float dec = __expf(acs_end);
#pragma unroll
      for (int nt = 0; nt < K::NNT; ++nt)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) S[nt][pt] *= dec;

#pragma unroll
      for (int js = 0; js < K::NJS; ++js) {
        f16x8 xh[NPT], xs[NPT];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const s16x8 r = tr8(xt + 32 * js * K::ROW_P, sl.xtr[pt][0], sl.xtr[pt][1]);
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = __uint_as_float((uint32_t)(uint16_t)r[e] << 16);
          xh[pt] = cvt_f16x8(v);
          xs[pt] = xh[pt] * w16[js];  // packed fp16 multiply
        }
        // intra-sub-chunk product: Y^T += x^T M^T over the K step's 32 tokens; in the block row
        // on the diagonal, lanes g >= 2 hold tokens after the row block (zero)
#pragma unroll
        for (int it = 2 * js; it < NIT; ++it) {
          f16x8 mf = *reinterpret_cast<const f16x8*>(mh + mblk(it, 2 * js) + sl.mrd);
          if (it == 2 * js) mf = c.g >= 2 ? f16x8{} : mf;
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) Y[pt][it] = M::mma(xh[pt], mf, Y[pt][it]);
        }
        // state update: S^T += B^T (w x)
#pragma unroll
        for (int nt = 0; nt < K::NNT; ++nt) {
          const char* bb = Bh + 32 * js * K::ROW_N + (nt / SL::NP) * (16 * 2 * SL::NP);
          const f16x8 bt = __builtin_bit_cast(
              f16x8, tr8(bb, bt0 ^ ((nt % SL::NP) << 5), bt1 ^ ((nt % SL::NP) << 5)));
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) S[nt][pt] = M::mma(bt, xs[pt], S[nt][pt]);
        }
      }

      __builtin_amdgcn_s_setprio(0);
      // y = Y, written over x in the stage (each lane's 8-byte pieces are its own and x is no
      // longer needed); stored to memory after the next wait
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const f32x4 v = Y[pt][it];
          *reinterpret_cast<uint2*>(st + xoff + 16 * it * K::ROW_P + sl.epi[pt]) =
              make_uint2(cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]));
        }
      }
      ytok = s * T;
    }
  }
  if (ytok >= 0) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's y tile writes have landed
    store_y<K>(smem + ((s_end - 1 - s_begin) & 1) * K::SCAN_STAGE + xoff, y, d, c, ytok);
  }
}


// ---- chain between runs -------------------------------------------------------------------------
// One thread per 8 consecutive entries of one (batch, head) state: walk the runs,
// h <- exp(logdecay_q) h + state_q starting from h0 (or 0), in fp32, writing the state entering
// run q + 1 over slot q (fp16). When a final state is wanted, the last run's state is already in
// it (fp32, from phase A): final = exp(logdecay_last) h + that. Only the multiply-adds depend on
// the run before: the loads of GS runs are issued together (16: -0.5 us against 8 at 12 and 64
// runs per sequence; 32 slower).
struct ChainArgs {
  u16* states;              // [Bt, nr - 1, H, P, N] fp16
  const float* logdecay;    // [Bt, H, nr]
  const float* h0;          // [Bt, H, P, N] or null
  float* fin;               // [Bt, H, P, N] or null; holds the last run's state on entry
  int64_t pieces;           // Bt * H * P * N / 8
  int PN8, H, nr;
};

__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    f[2 * i] = (float)h[0];
    f[2 * i + 1] = (float)h[1];
  }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, cvt_f16x2(f[2 * i], f[2 * i + 1]));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void k_state_chain(ChainArgs a) {
  constexpr int GS = 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.pieces) return;
  const int64_t bh = i / a.PN8;        // batch * H + head
  const int64_t e = (i % a.PN8) * 8;   // entry within the state
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t PN = (int64_t)a.PN8 * 8;
  const int64_t slot = (int64_t)a.H * PN;  // elements between runs' slots
  u16* sp = a.states + (b * (a.nr - 1) * a.H + h) * PN + e;
  const float* ld = a.logdecay + bh * a.nr;
  float acc[8];
  if (a.h0) {
    const float4 u = *reinterpret_cast<const float4*>(a.h0 + bh * PN + e);
    const float4 v = *reinterpret_cast<const float4*>(a.h0 + bh * PN + e + 4);
    acc[0] = u.x; acc[1] = u.y; acc[2] = u.z; acc[3] = u.w;
    acc[4] = v.x; acc[5] = v.y; acc[6] = v.z; acc[7] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  }
  const int nsteps = a.nr - 1;
  for (int q0 = 0; q0 < nsteps; q0 += GS) {
    uint4 st[GS];
    float dec[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int q = min(q0 + u, nsteps - 1);
      st[u] = *reinterpret_cast<const uint4*>(sp + q * slot);
      dec[u] = __expf(ld[q]);
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      if (q0 + u < nsteps) {
        float f[8];
        unpack8(st[u], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = dec[u] * acc[k] + f[k];
        *reinterpret_cast<uint4*>(sp + (q0 + u) * slot) = pack8(acc);
      }
    }
  }
  if (a.fin) {
    const float dl = __expf(ld[a.nr - 1]);
    float4* fo = reinterpret_cast<float4*>(a.fin + bh * PN + e);
    const float4 u = fo[0], v = fo[1];
    fo[0] = make_float4(dl * acc[0] + u.x, dl * acc[1] + u.y, dl * acc[2] + u.z, dl * acc[3] + u.w);
    fo[1] = make_float4(dl * acc[4] + v.x, dl * acc[5] + v.y, dl * acc[6] + v.z, dl * acc[7] + v.w);
  }
}

// ---- the three kernels ---------------------------------------------------------------------------
struct FwdArgs {
  const u16 *x, *B, *C;
  const float *dt, *A, *D, *h0;
  u16* y;
  float* fin;       // final state [Bt, H, P, N]; null: not written
  u16* states;      // [Bt, nr - 1, H, P, N] fp16: run states (all runs but the last), then the
                    // state entering the next run
  float* logdecay;  // [Bt, H, nr]
  Dims d;
  int run_len, nr, hb;  // run length (tokens), runs per sequence, head blocks per batch entry
  int na;               // runs per sequence whose state phase A computes
  int nsplit, nsplit_last;  // phase A sub-chunks with split operands, per run / in the last run
};

// A block's (batch, head block, run) and sub-chunk range from its item index: chains (batch,
// head block) one after another, nper runs per chain.
struct Item {
  int chain, r, b, s_begin, s_end;
};
template <class K>
__device__ __forceinline__ Item item_of(const FwdArgs& a, int item, int nper) {
  Item it;
  it.chain = item / nper;
  it.r = item % nper;
  it.b = it.chain / a.hb;
  const int nsub = (a.d.L + K::T - 1) / K::T;
  const int RS = a.run_len / K::T;  // sub-chunks per run (run_len is a multiple of T)
  it.s_begin = it.r * RS;
  it.s_end = min(nsub, it.s_begin + RS);  // never empty (the plan)
  return it;
}

// Phase A, one block per (chain, run) whose state is needed: the runs before the last (for the
// chain, stored fp16) and, when a final state is wanted, the last one too, stored fp32 into the
// final state (the chain adds the decayed entry state to it). With one run per sequence the state
// is completed into the final state here: S + exp(sum of dt A) h0. a.nsplit_last sub-chunks at the
// end of the last run, and a.nsplit of every other, take the split operands.
template <class K>
__global__ __launch_bounds__(K::NT, 1) void k_run_states(FwdArgs a) {
  static_assert(K::RUN_LDS <= 160 * 1024, "LDS budget");
  __shared__ __align__(1024) char smem[K::RUN_LDS];
  const Dims& d = a.d;
  const Item it = item_of<K>(a, blockIdx.x, a.na);
  const Coord c = coords<K>(d, it.r, it.chain % a.hb, it.b);
  const int64_t PN = (int64_t)K::P * K::N;
  f32x4 S[K::NNT][K::NPT];
  const bool last = it.r == a.nr - 1;
  const float ld = run_state<K>(smem, c, a.x, a.B, a.dt, a.A[c.h], dt_bias_of(d, c.h), d,
                                it.s_begin, it.s_end, last ? a.nsplit_last : a.nsplit, S);
  if (!c.active) return;
  if (last) {  // only launched when a final state is wanted
    const int64_t o = ((int64_t)it.b * d.H + c.h) * PN;
    store_state<K>(S, c, a.fin + o, a.nr == 1 && a.h0 ? a.h0 + o : nullptr, __expf(ld));
    if (a.nr > 1 && c.lane == 0 && c.p0 == 0)
      a.logdecay[((int64_t)it.b * d.H + c.h) * a.nr + it.r] = ld;
  } else {
    store_state_h<K>(S, c, a.states + (((int64_t)it.b * (a.nr - 1) + it.r) * d.H + c.h) * PN);
    if (c.lane == 0 && c.p0 == 0) a.logdecay[((int64_t)it.b * d.H + c.h) * a.nr + it.r] = ld;
  }
}

// Phase B, one block per (chain, run), from the state entering the run.
template <class K>
__global__ __launch_bounds__(K::NT, 1) void k_fused_scan(FwdArgs a) {
  static_assert(K::SCAN_LDS <= 160 * 1024, "LDS budget");
  __shared__ __align__(1024) char smem[K::SCAN_LDS];
  const Dims& d = a.d;
  const Item it = item_of<K>(a, blockIdx.x, a.nr);
  const Coord c = coords<K>(d, it.r, it.chain % a.hb, it.b);
  const int64_t PN = (int64_t)K::P * K::N;
  const float* h0 = it.r == 0 && a.h0 ? a.h0 + ((int64_t)it.b * d.H + c.h) * PN : nullptr;
  const u16* hin =
      it.r > 0 ? a.states + (((int64_t)it.b * (a.nr - 1) + (it.r - 1)) * d.H + c.h) * PN : nullptr;
  fused_scan<K>(smem, c, a.x, a.B, a.C, a.dt, a.A, a.D, h0, hin, a.y, d, it.s_begin, it.s_end);
}

// ---- plan and launch ----------------------------------------------------------------------------
// Both phases run 8 waves per block, two per SIMD (one wave's memory and matrix-core latencies
// hide behind the other's work), with 64-column slices (one wave per head at headdim 64) over
// sub-chunks of 32 tokens, so each wave keeps its fp32 state slice (64 x N) and the rest of its
// working set within 256 registers. One wave per head halves, per token, the B and C fragments
// read from LDS and the decay-mask work (a head's M blocks are built by its own wave), at the
// price of twice as many runs (twice the run-state traffic); measured with separate kernels at the
// headline workload: fused scan 145 -> 126 us, the forward -3%. The run-state phase reads its B^T
// fragments one K step at a time (holding a whole step's would spill at this width).
template <int P, int N>
using Cfg = Fz<P, N, 8, 64, 32>;

template <class K>
static int head_blocks(const Dims& d) {
  const int hpg = d.H / d.G;
  return d.G * ((hpg + K::HPB - 1) / K::HPB);
}

// Runs are planned in tokens, as whole multiples of 64 (so of the sub-chunk): by default about one
// block per compute unit in each of the two phases.
template <class K>
static void plan_for(const Dims& d, int run_tokens, int n_cu, FusedPlan* fp) {
  constexpr int U = 64;
  const int nunit = (d.L + U - 1) / U;
  fp->head_blocks = head_blocks<K>(d);
  const int units = d.Bt * fp->head_blocks;
  int RU;
  if (run_tokens > 0) {
    RU = (run_tokens + U - 1) / U;
  } else {
    int want = n_cu / units;  // runs per sequence: about one block per compute unit
    if (want < 1) want = 1;
    RU = (nunit + want - 1) / want;
  }
  if (RU < 1) RU = 1;
  if (RU > nunit) RU = nunit;
  fp->run_len = RU * U;
  fp->nr = (nunit + RU - 1) / RU;
}

#define SSD_FUSED_SHAPES(X) X(64, 64) X(64, 128) X(64, 256) X(128, 64) X(128, 128) X(128, 256)

bool fused_plan(const Dims& d, int run_tokens, int n_cu, FusedPlan* fp) {
#define SSD_PLAN(P_, N_)                                 \
  if (d.P == P_ && d.N == N_) {                          \
    plan_for<Cfg<P_, N_>>(d, run_tokens, n_cu, fp);      \
    return true;                                         \
  }
  SSD_FUSED_SHAPES(SSD_PLAN)
#undef SSD_PLAN
  return false;
}

int64_t fused_workspace_bytes(const Dims& d, const FusedPlan& fp) {
  if (fp.nr <= 1) return 0;
  const int64_t st = (int64_t)d.Bt * (fp.nr - 1) * d.H * d.P * d.N * 2;
  const int64_t ld = (int64_t)d.Bt * d.H * fp.nr * 4;
  return ((st + 255) & ~int64_t(255)) + ld;
}

template <class K>
static hipError_t launch_k(const Dims& d, const FusedPlan& fp, const void* x, const void* B,
                           const void* C, const float* dt, const float* A, const float* D,
                           const float* h0, void* y, float* fin, void* ws, FusedTimer* tm,
                           hipStream_t s) {
  FwdArgs a{};
  a.x = (const u16*)x;
  a.B = (const u16*)B;
  a.C = (const u16*)C;
  a.dt = dt;
  a.A = A;
  a.D = D;
  a.h0 = h0;
  a.y = (u16*)y;
  a.fin = fin;
  a.d = d;
  a.run_len = fp.run_len;
  a.nr = fp.nr;
  a.hb = fp.head_blocks;
  a.na = fin ? fp.nr : fp.nr - 1;  // phase A: every run but the last, unless a final state
  // split operands: where the run state is kept in fp32 (the final state), over the whole run at
  // one run per sequence, else over its last K::NSPLIT sub-chunks; states handed on in fp16 are
  // rounded anyway
  a.nsplit = 0;
  a.nsplit_last = !fp.split ? 0 : fp.nr == 1 ? fp.run_len / K::T : K::NSPLIT;
  if (fp.nr > 1) {
    const int64_t st = (int64_t)d.Bt * (fp.nr - 1) * d.H * d.P * d.N * 2;
    a.states = static_cast<u16*>(ws);
    a.logdecay = reinterpret_cast<float*>(static_cast<char*>(ws) + ((st + 255) & ~int64_t(255)));
  }
  const int chains = d.Bt * fp.head_blocks;
  hipError_t e = tm ? tm->mark(s) : hipSuccess;
  if (e == hipSuccess && a.na > 0) {
    hipLaunchKernelGGL((k_run_states<K>), dim3(chains * a.na), dim3(K::NT), 0, s, a);
    e = hipGetLastError();
    if (e == hipSuccess && tm) e = tm->mark(s);
  }
  if (e == hipSuccess && fp.nr > 1) {
    ChainArgs ca{a.states, a.logdecay, h0, fin, (int64_t)d.Bt * d.H * d.P * d.N / 8,
                 (int)(d.P * d.N / 8), (int)d.H, fp.nr};
    hipLaunchKernelGGL(k_state_chain, dim3((unsigned)((ca.pieces + 255) / 256)), dim3(256), 0, s,
                       ca);
    e = hipGetLastError();
    if (e == hipSuccess && tm) e = tm->mark(s);
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_fused_scan<K>), dim3(chains * fp.nr), dim3(K::NT), 0, s, a);
    e = hipGetLastError();
    if (e == hipSuccess && tm) e = tm->mark(s);
  }
  return e;
}

hipError_t launch_fused(const Dims& d, const FusedPlan& fp, const void* x, const void* B,
                        const void* C, const float* dt, const float* A, const float* D,
                        const float* h0, void* y, float* fin, void* ws, FusedTimer* tm,
                        hipStream_t s) {
#define SSD_LAUNCH(P_, N_)                                                                    \
  if (d.P == P_ && d.N == N_)                                                                 \
    return launch_k<Cfg<P_, N_>>(d, fp, x, B, C, dt, A, D, h0, y, fin, ws, tm, s);
  SSD_FUSED_SHAPES(SSD_LAUNCH)
#undef SSD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssd
