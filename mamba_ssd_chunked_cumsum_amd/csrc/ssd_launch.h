// Kernel launchers of libssd (library-internal). Every launcher assumes the host checks of
// ssd_api.cpp have passed: positive sizes, nheads % ngroups == 0, chunk size a power of two in
// [16, 256], headdim and dstate multiples of 16 up to 256, 16-byte aligned pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Dims {
  int Bt, L, H, P, N, G, Q, nc;
  // dt pre-processing where the kernels read dt: dt + dt_bias[h] (no bias when null), then
  // softplus when dt_softplus != 0, then clamped to [dt_min, dt_max] when dt_max > 0
  const float* dt_bias = nullptr;
  int dt_softplus = 0;
  float dt_min = 0.f, dt_max = 0.f;
  // unfused path only (the backward's adjoint recurrences): the input term is x B^T instead of
  // dt x B^T, while dt still sets the decay exp(dt A)
  int unit_input = 0;
  // unfused path only (the backward's transposed recurrences): 0 = x has one row per head; else x
  // has x_groups rows per token and head h reads row h / (H / x_groups) (x shared like B and C)
  int x_groups = 0;
  // fp32 chunk scan only (the backward's transposed recurrences): h_in holds, per (batch, chunk,
  // head), the transposed states [N][P] that the untransposed problem left, read transposed
  int hin_transposed = 0;
  // unfused path, bf16 io (the backward's recurrences): every stage computes in fp32 (C B^T
  // included) and the chunk scan stores y in fp32
  int f32_math = 0;
};

constexpr int kIoF32 = 0, kIoBf16 = 1;
constexpr int kPrecAuto = 0, kPrecFp16 = 1, kPrecFp32 = 3;

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* Acs,
                               float* dtc, hipStream_t s);
hipError_t launch_bmm_chunk(const Dims& d, int io, const void* B, const void* C, float* CB,
                            hipStream_t s);
hipError_t launch_chunk_state(const Dims& d, int io, int prec, const void* x, const void* B,
                              const float* Acs, const float* dtc, float* states, hipStream_t s);
hipError_t launch_state_passing(const Dims& d, const float* states, const float* Acs,
                                const float* h0, float* h_in, float* fin, hipStream_t s);
hipError_t launch_chain_passing(const Dims& d, int nsteps, const float* states,
                                const float* logdecay, int64_t ld_bh, int64_t ld_step,
                                const float* h0, float* h_in, float* fin, hipStream_t s);
hipError_t launch_chunk_scan(const Dims& d, int io, int prec, const void* x, const void* C,
                             const float* CB, const float* Acs, const float* dtc,
                             const float* h_in, const float* D, void* y, hipStream_t s);


// fused path (bf16 io)
// Run plan of one fused forward: runs of run_len tokens (a multiple of 64), nr runs per sequence,
// head_blocks blocks per (batch, run).
// split: where phase A keeps a run state in fp32 (the final state), it feeds the weighted x of the
// run's last 128 tokens (of the whole run at one run per sequence) to the matrix cores as fp16
// high + low parts; false: high parts only everywhere.
struct FusedPlan {
  int run_len, nr, head_blocks;
  bool split = true;
};
// Optional timing events: ev[k++] recorded on the stream before the first launch and after each.
struct KernelMarks {
  void** ev = nullptr;
  int n = 0, k = 0;
  hipError_t mark(hipStream_t s) {
    if (!ev || k >= n) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[k++]), s);
  }
};
using FusedTimer = KernelMarks;
// False when the fused kernels do not cover (P, N). run_tokens > 0 asks for runs of at least that
// many tokens (rounded up to 64); 0 lets the plan aim at about one block per compute unit (n_cu of
// them).
bool fused_plan(const Dims& d, int run_tokens, int n_cu, FusedPlan* fp);
// Workspace bytes of a plan (0 for one run per sequence): the states of every run but the last,
// [Bt, nr - 1, H, P, N] fp16 (padded to 256 bytes), then run log-decays [Bt, H, nr] f32.
int64_t fused_workspace_bytes(const Dims& d, const FusedPlan& fp);
// The whole fused forward, up to three kernels: run states (skipped with one run per sequence and
// no final state), the chain over runs (nr > 1) and the fused scan. h0 and fin nullable;
// ws: fused_workspace_bytes(d, fp) bytes of device memory (unused when nr == 1).
hipError_t launch_fused(const Dims& d, const FusedPlan& fp, const void* x, const void* B,
                        const void* C, const float* dt, const float* A, const float* D,
                        const float* h0, void* y, float* fin, void* ws, FusedTimer* tm,
                        hipStream_t s);
// Short sequences (L <= kQuadMaxLen, dstate <= 256): the whole forward in one kernel, the
// sequence as a single block of the quadratic (masked) form, fp32 arithmetic; h0 and fin
// nullable. quadratic_covers() tells whether a problem qualifies.
constexpr int kQuadMaxLen = 256;
bool quadratic_covers(const Dims& d);
int64_t quadratic_blocks(const Dims& d);  // blocks of its launch
hipError_t launch_quadratic(const Dims& d, int io, const void* x, const float* dt, const float* A,
                            const void* B, const void* C, const float* D, const float* h0,
                            void* y, float* fin, hipStream_t s);

// No-allocation forward: the per-device static scratch (ssd_scratch.hip), kScratchBytes long,
// shared by every call on a device. *out = this device's copy (looked up once per device).
constexpr int64_t kScratchBytes = int64_t(64) << 20;
hipError_t scratch_address(void** out);

// backward helpers (ssd_backward.hip); outputs fp32 unless stated, layouts row-major.
// out[b, pad + t, :] = in[b, L - 1 - t, :] (rows of E elements of the io type), out[b, 0 .. pad - 1]
// = 0; E times the element size a multiple of 16 bytes
hipError_t launch_reverse_rows(int io, const void* in, void* out, int Bt, int L, int E, int pad,
                               hipStream_t s);
// dtr[b, pad + t, h] = t == 0 ? 0 : dt[b, L - t, h], dtr[b, 0 .. pad - 1] = 0
hipError_t launch_dt_shift_rev(const float* dt, float* dtr, int Bt, int L, int H, int pad,
                               hipStream_t s);
// per (b, t, h): dx = D dy + dt u; q = dy . ys - dt x . u; xu = x . u; dyx = dy . x, where
// u = ur[b, pad + L - 1 - t, h, :] (the adjoint readout, stored in reversed time after pad rows)
hipError_t launch_bwd_pointwise(int io, const void* x, const void* dy, const float* ur,
                                const float* ys, const float* dt, const float* D, float* dx,
                                float* q, float* xu, float* dyx, int Bt, int L, int H, int P,
                                int pad, hipStream_t s);
// anch[b, h, k] = <G_t, S_{t-1}> at t = 256 k, k < ceil(L / 256), from the forward recurrence's
// chunk-entry states hf [Bt, ncf, H, P, N] (chunk t / Q) and the reversed-time adjoint's hg
// [Bt, ncg, H, P, N] over Lp tokens (chunk (Lp - t) / Q; Lp = L + pad, Lp % Q == 0), or its final
// state g0 [Bt, H, P, N] for t = 0; double
hipError_t launch_anchor_dot(const float* hf, const float* hg, const float* g0, double* anch,
                             int Bt, int H, int PN, int Q, int ncf, int ncg, int L, int Lp,
                             hipStream_t s);
// per (b, h): da_t = exp(dt_t0 A) anch[b, h, k] - sum_{t0 <= s < t} q_s over each 256-token tile k
// (first token t0); ddt = A da + xu; per-(b, h) partial sums of dt da (for dA) and of dyx (for
// dD) (sums in double)
hipError_t launch_bwd_scan(const float* q, const float* xu, const float* dyx, const float* dt,
                           const float* A, const double* anch, float* ddt, double* pa, double* pd,
                           int Bt, int L, int H, hipStream_t s);
// dA[h] = sum_b pa[b, h]; dD[h] = sum_b pd[b, h]
hipError_t launch_sum_batch(const double* pa, const double* pd, float* dA, float* dD, int Bt,
                            int H, hipStream_t s);
// dB[b, t, g, n] = sum_{h in g} dt[b, t, h] vb[b, pad + L - 1 - t, h, n];
// dC[b, t, g, n] = sum_{h in g} vc[b, t, h, n]
hipError_t launch_group_sums(const float* vb, const float* vc, const float* dt, float* dB,
                             float* dC, int Bt, int L, int H, int G, int N, int pad,
                             hipStream_t s);
// dh0[b, h] = exp(dt[b, 0, h] A[h]) g0[b, h]
hipError_t launch_scale_state(const float* g0, const float* dt, const float* A, float* dh0,
                              int Bt, int L, int H, int PN, hipStream_t s);

// single-token step: state [Bt, H, P, N] fp32 (s_out may equal s_in); x, y [Bt, H, P];
// dt [Bt, H]; B, C [Bt, G, N]
hipError_t launch_step(const Dims& d, int io, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* s_in,
                       float* s_out, void* y, hipStream_t s);

}  // namespace ssd
