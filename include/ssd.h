/*
 * libssd -- Mamba-2 SSD (state-space duality) chunked selective-scan forward on AMD Instinct
 * MI355X (gfx950). C ABI: plain pointers and sizes only.
 *
 * The operation (per batch b and head h, state S of shape [P, N]):
 *     S_t    = exp(dt[t,h] * A[h]) * S_{t-1} + dt[t,h] * outer(x[t,h,:], B[t,g(h),:])
 *     y[t,h] = S_t @ C[t,g(h),:] + D[h] * x[t,h,:]
 * with S_{-1} = initial_state (zeros when NULL), final_state = S_{L-1}, and g(h) = h / (H / G).
 * This is the selective state-space step of "Why SSM and linear-RNN FLOPs do not convert into GPU
 * FLOPs" (first paragraph) with one decay shared by every state entry of a head, in the Mamba-2
 * SSD form. It is evaluated with the chunked algorithm ("nitter.gq/da_be19" thread, post 5/6):
 * the sequence is cut into chunks of `chunk_size` tokens; inside a chunk the quadratic masked form
 * (C B^T masked by the decay) is used, across chunks a linear recurrence over chunk states; the
 * stages are the per-chunk cumulative decay, the state entering each chunk, and the outputs
 * ("Mamba-2 in NVIDIA cuTile: Faster Forward Kernels and What the Benchmark Means", section
 * "Why Mamba-2 is a useful kernel example").
 *
 * Layouts: every tensor is dense, row-major (last index fastest), in device memory:
 *     x, y            [batch, seqlen, nheads, headdim]     io dtype (fp32 or bf16)
 *     dt              [batch, seqlen, nheads]              fp32, the final positive step sizes
 *     A, D            [nheads]                             fp32 (A <= 0 is the decay regime)
 *     B, C            [batch, seqlen, ngroups, dstate]     io dtype
 *     initial_state,
 *     final_state     [batch, nheads, headdim, dstate]     fp32
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer after a call returns.
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the null stream):
 * device faults surface at the caller's next synchronisation. Workspace (unfused path, and the
 * run states and run decays of the fused path) is allocated stream-ordered on `stream` and
 * released the same way.
 *
 * Errors: every argument check runs on the host before any HIP call; on failure nothing is
 * launched and nothing is written. Status codes are never thrown across the ABI.
 *
 * Precision (bf16 io): x, B, C are converted exactly to fp16 for the matrix cores; operands that
 * carry fp32 values (the masked C B^T block, the chunk states fed to the readout) are rounded to
 * fp16 once, and the chunk-state operand is split into fp16 high + low parts. All accumulation is
 * fp32; y is rounded once to bf16 (nearest-even). Inputs must stay within fp16 range
 * (|v| < 65504). fp32 io uses fp32 matrix-core instructions throughout.
 * Results are bitwise reproducible run to run on one GPU (fixed reduction order, no atomics on
 * data).
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, nheads % ngroups != 0,
                                     misaligned pointer, overlapping output, bad enum value */
    SSD_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels implement: chunk_size
                                     not a power of two in [16, 256], headdim or dstate not a
                                     multiple of 16 or above 256, sizes beyond 32-bit indexing */
    SSD_ERR_NO_DEVICE = 3,        /* no HIP device visible */
    SSD_ERR_OUT_OF_MEMORY = 4,    /* workspace allocation failed */
    SSD_ERR_HIP = 5,              /* a HIP call or kernel launch failed */
    SSD_ERR_WORKSPACE_LIMIT = 6   /* ssd_forward_noalloc: the request's workspace does not fit the
                                     library's static scratch (SSD_SCRATCH_BYTES) */
} ssd_status;

typedef enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype; /* dtype of x, B, C, y */

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
    int32_t io_dtype; /* ssd_dtype */
    int32_t reserved; /* must be 0 */
} ssd_problem;

typedef enum {
    SSD_VARIANT_AUTO = 0,
    SSD_VARIANT_UNFUSED = 1, /* cumsum, C B^T, chunk states, state passing, chunk scan: five
                                kernels, intermediates in workspace */
    SSD_VARIANT_FUSED = 2,   /* bf16 io, headdim 64 or 128, dstate 64, 128 or 256: up to three
                                kernels. The sequence is cut into runs (about one block per compute
                                unit); one kernel computes each run's own end state (skipped with
                                one run per sequence and no final state), one chains those states
                                into the state entering each run and the final state (skipped with
                                one run per sequence), and one walks every run in sub-chunks of 32
                                tokens with the state on chip: C B^T block, decay mask, readout and
                                state update never leave the compute unit. The exact result does
                                not depend on the chunk length, so chunk_size only sets the run
                                length when run_chunks is given. Assumes A <= 0 and dt >= 0
                                (decays at most 1); D enters through the fp16 diagonal of the
                                masked block (exact for D = 1) */
    SSD_VARIANT_QUADRATIC = 3 /* seqlen <= 256, dstate <= 256, either io: one kernel, the whole
                                sequence as a single block of the quadratic (masked,
                                attention-like) form y = (L o C B^T)(dt x) + D x plus the
                                initial state's readout, and the final state, in fp32 arithmetic
                                whatever the precision option (the naive quadratic form that
                                the "nitter.gq/da_be19" thread, post 5/6, finds cheaper for
                                short sequences). chunk_size is checked but not used. Assumes A <= 0
                                and dt >= 0. AUTO takes it for problems the fused kernels do not
                                cover with seqlen * dstate <= 8192 and a launch of at most two
                                blocks per compute unit; otherwise the unfused kernels */
} ssd_variant;

typedef enum {
    SSD_PRECISION_AUTO = 0, /* bf16 io: fp16 operands, with the chunk-state operand split hi + lo
                               where a state is kept in fp32 (the unfused chunk states; the fused
                               path's last run state, which goes into the final state: over the
                               run's last 128 tokens, or the whole run at one run per sequence);
                               the fused path hands the other run states to its chain in fp16.
                               fp32 io: fp32 */
    SSD_PRECISION_FP16 = 1, /* bf16 io: every fp32-carrying operand rounded once to fp16 */
    SSD_PRECISION_FP32 = 3  /* fp32 matrix-core instructions for every contraction */
} ssd_precision;

typedef struct {
    int32_t variant;    /* ssd_variant */
    int32_t precision;  /* ssd_precision */
    int32_t run_chunks; /* fused variant: runs of run_chunks * chunk_size tokens (rounded up to
                           64 tokens); 0 = chosen from the problem size and the device's compute
                           units; must be >= 0 */
    int32_t n_events;   /* capacity of `events`; 0 = no timing events */
    void** events;      /* optional hipEvent_t[n_events], created by the caller: events[0] is
                           recorded on `stream` before the first kernel and events[k] after the
                           k-th kernel, so the caller can time each kernel. Needs n_events >=
                           kernels + 1 (6 covers every variant), else SSD_ERR_INVALID_ARGUMENT. */
    int32_t* n_kernels; /* optional out: number of kernels the call launched */
    /* dt pre-processing, applied by the kernels where they read dt (no separate pass), in this
     * order: dt + dt_bias[h]; softplus, log(1 + exp(v)) (v itself above 20, where the two agree
     * to fp32 precision); clamp to [dt_min, dt_max]. The recurrence then runs on that dt. With
     * every field zero (or opts NULL) dt is used as given. */
    const float* dt_bias; /* optional [nheads] f32, 16-byte aligned; NULL = no bias */
    int32_t dt_softplus;  /* nonzero: apply softplus */
    float dt_min, dt_max; /* dt_max > 0: clamp to [dt_min, dt_max] (needs dt_min <= dt_max);
                             dt_max == 0: no clamp; dt_max < 0 is invalid */
    int32_t* kernel_mask; /* optional out: the ssd_kernel bits of the kernels the call launched;
                             they were launched in increasing bit order */
} ssd_options;

/* Kernels of a forward, as reported in ssd_options.kernel_mask. */
typedef enum {
    SSD_KERNEL_QUADRATIC = 1,       /* quadratic variant: the whole forward */
    SSD_KERNEL_CHUNK_CUMSUM = 2,    /* unfused: stage 1 */
    SSD_KERNEL_BMM_CHUNK = 4,       /* unfused: stage 2 */
    SSD_KERNEL_CHUNK_STATE = 8,     /* unfused: stage 3 */
    SSD_KERNEL_STATE_PASSING = 16,  /* unfused: stage 4 */
    SSD_KERNEL_CHUNK_SCAN = 32,     /* unfused: stage 5 */
    SSD_KERNEL_FUSED_RUN_STATES = 64, /* fused: each run's own end state (several runs per
                                         sequence, or a final state wanted) */
    SSD_KERNEL_FUSED_CHAIN = 128,     /* fused, several runs per sequence: the chain over runs */
    SSD_KERNEL_FUSED_SCAN = 256       /* fused: the outputs, run by run */
} ssd_kernel;

/* Full forward. initial_state may be NULL (zeros); final_state may be NULL (not written).
 * Alignment: every pointer 16-byte aligned. y must not overlap any input; final_state must not
 * overlap initial_state or any other argument. chunk_size: power of two in [16, 256]; the last
 * chunk may be shorter. */
ssd_status ssd_forward(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, int64_t chunk_size,
                       const float* initial_state, void* y, float* final_state, void* stream);

/* Same, with explicit variant / precision (opts may be NULL = auto). */
ssd_status ssd_forward_ex(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                          const void* B, const void* C, const float* D, int64_t chunk_size,
                          const float* initial_state, void* y, float* final_state, void* stream,
                          const ssd_options* opts);

/* ---- Forward without device allocation. ---------------------------------------------------
 * For callers that cannot allocate device memory during the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, checks and results as
 * ssd_forward_ex, but the call allocates nothing: its workspace is a static array of
 * SSD_SCRATCH_BYTES in device memory, one per device, held from the library's load until the
 * process ends (the first call on a device looks up that device's copy). The fused variant plans
 * its runs so that their states fit (longer runs, down to one run per sequence, which needs no
 * workspace); the quadratic variant needs none; the unfused variant's intermediates must fit as
 * they are, else SSD_ERR_WORKSPACE_LIMIT and nothing is launched. Every call on a device shares its
 * scratch, which keeps the last call's contents (no kernel reads what it did not write in the same
 * call), and calls that overlap on one device (other streams, other host threads) race and must
 * not be issued. Results may differ from ssd_forward_ex within the stated tolerance where the fitted
 * plan's run boundaries differ; with the same plan they are bitwise equal. */
#define SSD_SCRATCH_BYTES (64ll << 20)
ssd_status ssd_forward_noalloc(const ssd_problem* prob, const void* x, const float* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               int64_t chunk_size, const float* initial_state, void* y,
                               float* final_state, void* stream, const ssd_options* opts);

/* ---- Stages of the unfused path, exposed so each can be checked on its own. -----------------
 * nc = ceil(seqlen / chunk_size), Q = chunk_size. Workspace layouts (fp32, row-major):
 *     Acs      [batch, nheads, nc, Q]   inclusive cumulative sum of dt*A inside each chunk; past
 *                                       the end of a ragged last chunk it repeats the last value
 *     dtc      [batch, nheads, nc, Q]   dt regrouped per (head, chunk); 0 past the end
 *     CB       [batch, nc, ngroups, Q, Q]  C_i . B_j; only 16x16 blocks on or below the block
 *                                       diagonal are written, and in them only j <= i is
 *                                       meaningful
 *     states   [batch, nc, nheads, headdim, dstate]  each chunk's own end state (zero entry state)
 *     h_in     [batch, nc, nheads, headdim, dstate]  state entering each chunk
 */

/* Stage 1 (per-chunk cumulative decay): writes Acs and dtc. */
ssd_status ssd_chunk_cumsum(const ssd_problem* prob, const float* dt, const float* A,
                            int64_t chunk_size, float* Acs, float* dtc, void* stream);

/* Stage 2 (C B^T inside each chunk, shared by the heads of a group): writes CB. */
ssd_status ssd_bmm_chunk(const ssd_problem* prob, const void* B, const void* C,
                         int64_t chunk_size, float* CB, void* stream);

/* Stage 3 (each chunk's own end state): states = sum_j exp(Acs_last - Acs_j) dt_j x_j B_j^T. */
ssd_status ssd_chunk_state(const ssd_problem* prob, const void* x, const void* B,
                           const float* Acs, const float* dtc, int64_t chunk_size,
                           float* states, void* stream, const ssd_options* opts);

/* Stage 4 (state entering each chunk): h_in[0] = initial_state (or 0),
 * h_in[c+1] = exp(Acs_last[c]) h_in[c] + states[c]; final_state = h_in[nc] (may be NULL). */
ssd_status ssd_state_passing(const ssd_problem* prob, const float* states, const float* Acs,
                             int64_t chunk_size, const float* initial_state, float* h_in,
                             float* final_state, void* stream);

/* Stage 5 (outputs): y = (CB * exp(Acs_i - Acs_j) * dt_j, j <= i) x + exp(Acs_i) C_i h_in^T
 * + D x. */
ssd_status ssd_chunk_scan(const ssd_problem* prob, const void* x, const void* C, const float* CB,
                          const float* Acs, const float* dtc, const float* h_in, const float* D,
                          int64_t chunk_size, void* y, void* stream, const ssd_options* opts);

/* Bytes of each unfused workspace tensor, in the order Acs, dtc, CB, states, h_in. */
ssd_status ssd_workspace_sizes(const ssd_problem* prob, int64_t chunk_size, int64_t sizes[5]);

/* ---- Single-token recurrent step (decode): continue a sequence from its state. --------------
 * One step of the selective state-space recurrence ("Why SSM and linear-RNN FLOPs do not convert
 * into GPU FLOPs: the sequential scan bypasses the tensor cores", first paragraph) with SSD's
 * scalar decay per head; per token it costs one pass over the fixed-size state ("nitter.gq/
 * da_be19" thread, post 5/6). For every batch entry b and head h, with g = h / (nheads / ngroups):
 *     a = exp(dt[b,h] A[h]);  state[b,h,p,n] <- a state[b,h,p,n] + dt[b,h] x[b,h,p] B[b,g,n];
 *     y[b,h,p] = sum_n state[b,h,p,n] C[b,g,n] + D[h] x[b,h,p]          (the updated state)
 * This is the recurrence ssd_forward evaluates by chunks: after ssd_forward over tokens 0..L-1
 * with final_state S, ssd_step from S with token L gives token L's output.
 * prob->seqlen must be 1. Layouts (row-major): x, y [batch, nheads, headdim] io dtype;
 * dt [batch, nheads] f32; A, D [nheads] f32; B, C [batch, ngroups, dstate] io dtype;
 * state_in, state_out [batch, nheads, headdim, dstate] f32. state_out may be state_in (updated
 * in place); otherwise the two must not overlap. y must not overlap any other argument, nor
 * state_out any input. headdim and dstate: multiples of 16 up to 256, as for the forward.
 * Arithmetic is fp32; y is rounded once to the io dtype (nearest even for bf16). Every pointer
 * 16-byte aligned. Errors as for ssd_forward: all checks on the host before any HIP call. */
ssd_status ssd_step(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* state_in,
                    float* state_out, void* y, void* stream);

/* ---- Backward: gradients of the forward with respect to every input. ----------------------
 * Training depends on the backward pass as well as the forward ("Mamba-2 in NVIDIA cuTile: Faster
 * Forward Kernels and What the Benchmark Means", section "What the speedup does and does not
 * establish"). Given dy = dL/dy and dfinal = dL/dfinal_state (NULL: zero), for the recurrence of
 * ssd_forward (dt as given: no dt pre-processing options) this computes, with G_t = dL/dS_t:
 *     G_t = dy_t C_t^T + exp(dt_{t+1} A) G_{t+1},  G_{L-1} = dy_{L-1} C_{L-1}^T + dfinal
 *     dx_t = D dy_t + dt_t G_t B_t;   dB_t = sum over the group's heads of dt_t G_t^T x_t;
 *     dC_t = sum over the group's heads of S_t^T dy_t;
 *     ddt_t = A dlog_t + x_t . (G_t B_t) with dlog_t = <G_t, exp(dt_t A) S_{t-1}>;
 *     dA = sum over batch and time of dt_t dlog_t;  dD = sum over batch and time of dy_t . x_t;
 *     dinitial_state = exp(dt_0 A) G_0.
 * It runs the chunked forward machinery four times in fp32 (the state part of y and the final
 * state; the adjoint G in reversed time; the transposed state for dC; the transposed adjoint for
 * dB) plus elementwise and reduction kernels; dlog is formed from the product of the forward's
 * and the adjoint's states at the first token of every 256-token tile and from per-token terms
 * within the tile (sums in double). Inputs as for ssd_forward (io dtype for x, B, C and
 * dy; initial_state and dfinal [batch, nheads, headdim, dstate] f32, both nullable). Outputs, all
 * f32 and overwritten (not accumulated into): dx [batch, seqlen, nheads, headdim], ddt [batch,
 * seqlen, nheads], dA and dD [nheads], dB and dC [batch, seqlen, ngroups, dstate],
 * dinitial_state [batch, nheads, headdim, dstate] (nullable: not computed). No output may overlap
 * an input or another output; every pointer 16-byte aligned. Shapes as for the forward, and the
 * transposed problem (headdim and dstate swapped, one group per head) must pass the same checks.
 * Workspace: 2 fp32 and 2 io-typed x-sized tensors, 2 fp32 tensors of [batch, seqlen, nheads,
 * dstate] and the chunk states of two recurrences (4 fp32 tensors of [batch, ceil(seqlen / 64),
 * nheads, headdim, dstate]), allocated and released stream-ordered on `stream`. Errors as for
 * ssd_forward. */
ssd_status ssd_backward(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                        const void* B, const void* C, const float* D, int64_t chunk_size,
                        const float* initial_state, const void* dy, const float* dfinal,
                        float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD,
                        float* dinitial_state, void* stream);

/* Static text for a status code. */
const char* ssd_status_string(ssd_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
