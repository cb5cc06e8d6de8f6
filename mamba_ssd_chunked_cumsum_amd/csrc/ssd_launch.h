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
// head_blocks fused-scan blocks per (batch, run).
// split: F1 feeds the weighted x to the matrix cores as fp16 high + low parts (else high only).
struct FusedPlan {
  int run_len, nr, head_blocks;
  bool split = true;
};
// False when the fused kernels do not cover (P, N). run_tokens > 0 asks for runs of at least that
// many tokens; 0 lets the plan aim at about one block per compute unit (n_cu of them).
bool fused_plan(const Dims& d, int run_tokens, int n_cu, FusedPlan* fp);
// states [Bt, nr, H, P, N] (each run's end state from a zero entry state), logdecay [Bt, H, nr]
hipError_t launch_run_state(const Dims& d, const FusedPlan& fp, const void* x, const void* B,
                            const float* dt, const float* A, float* states, float* logdecay,
                            hipStream_t s);
// h_run [Bt, nr, H, P, N]: the state entering each run
hipError_t launch_fused_scan(const Dims& d, const FusedPlan& fp, const void* x, const void* B,
                             const void* C, const float* dt, const float* A, const float* D,
                             const float* h_run, void* y, hipStream_t s);

// single-token step: state [Bt, H, P, N] fp32 (s_out may equal s_in); x, y [Bt, H, P];
// dt [Bt, H]; B, C [Bt, G, N]
hipError_t launch_step(const Dims& d, int io, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* s_in,
                       float* s_out, void* y, hipStream_t s);

}  // namespace ssd
