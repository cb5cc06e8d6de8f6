// libssd C ABI: argument checks, workspace, and the sequence of kernel launches.
// Every check runs on the host before the first HIP call, so invalid requests return without
// touching the device (and the checks work on machines without a GPU).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/ssd.h"
#include "ssd_launch.h"

namespace {

using ssd::Dims;

constexpr int kVersion = 1 * 10000 + 5 * 100 + 0;  // 1.2: ssd_backward; 1.3: quadratic variant;
                                                   // 1.4: kernel_mask; 1.5: fused forward as run
                                                   // states, chain and fused scan
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Shape checks shared by every entry point.
ssd_status check_problem(const ssd_problem* p, int64_t chunk_size) {
  if (!p) return SSD_ERR_INVALID_ARGUMENT;
  if (p->batch <= 0 || p->seqlen <= 0 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 ||
      p->ngroups <= 0)
    return SSD_ERR_INVALID_ARGUMENT;
  if (p->nheads % p->ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (p->io_dtype != SSD_DTYPE_F32 && p->io_dtype != SSD_DTYPE_BF16)
    return SSD_ERR_INVALID_ARGUMENT;
  if (p->reserved != 0) return SSD_ERR_INVALID_ARGUMENT;
  if (chunk_size <= 0) return SSD_ERR_INVALID_ARGUMENT;
  if (!pow2(chunk_size) || chunk_size < 16 || chunk_size > 256) return SSD_ERR_UNSUPPORTED;
  if (p->headdim % 16 || p->headdim > 256 || p->dstate % 16 || p->dstate > 256)
    return SSD_ERR_UNSUPPORTED;
  // Every tensor (inputs, outputs, workspace) must be indexable with 31-bit element counts
  // inside one (batch) slice and 63-bit overall; keep whole tensors below 2^31 elements.
  const int64_t nc = (p->seqlen + chunk_size - 1) / chunk_size;
  const double big = static_cast<double>(kMaxIndex);
  const double x_el = double(p->batch) * p->seqlen * p->nheads * p->headdim;
  const double bc_el = double(p->batch) * p->seqlen * p->ngroups * p->dstate;
  const double st_el = double(p->batch) * nc * p->nheads * p->headdim * p->dstate;
  const double cb_el = double(p->batch) * nc * p->ngroups * chunk_size * chunk_size;
  if (x_el > big || bc_el > big || st_el > big || cb_el > big) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

Dims make_dims(const ssd_problem* p, int64_t Q) {
  Dims d;
  d.Bt = (int)p->batch;
  d.L = (int)p->seqlen;
  d.H = (int)p->nheads;
  d.P = (int)p->headdim;
  d.N = (int)p->dstate;
  d.G = (int)p->ngroups;
  d.Q = (int)Q;
  d.nc = (int)((p->seqlen + Q - 1) / Q);
  return d;
}

int64_t io_bytes(const ssd_problem* p) { return p->io_dtype == SSD_DTYPE_BF16 ? 2 : 4; }

struct Sizes {
  int64_t x, dt, hd, bc, state;  // bytes of x/y, dt, A/D, B/C, initial/final state
};

Sizes sizes_of(const ssd_problem* p) {
  Sizes s;
  const int64_t e = io_bytes(p);
  s.x = p->batch * p->seqlen * p->nheads * p->headdim * e;
  s.dt = p->batch * p->seqlen * p->nheads * 4;
  s.hd = p->nheads * 4;
  s.bc = p->batch * p->seqlen * p->ngroups * p->dstate * e;
  s.state = p->batch * p->nheads * p->headdim * p->dstate * 4;
  return s;
}

ssd_status check_options(const ssd_options* o) {
  if (!o) return SSD_OK;
  if (o->variant < SSD_VARIANT_AUTO || o->variant > SSD_VARIANT_QUADRATIC)
    return SSD_ERR_INVALID_ARGUMENT;
  if (o->precision != SSD_PRECISION_AUTO && o->precision != SSD_PRECISION_FP16 &&
      o->precision != SSD_PRECISION_FP32)
    return SSD_ERR_INVALID_ARGUMENT;
  if (o->run_chunks < 0) return SSD_ERR_INVALID_ARGUMENT;
  if (o->n_events < 0 || (o->n_events > 0 && !o->events)) return SSD_ERR_INVALID_ARGUMENT;
  if (o->n_events > 0 && o->n_events < 6) return SSD_ERR_INVALID_ARGUMENT;
  if (o->dt_bias && !aligned16(o->dt_bias)) return SSD_ERR_INVALID_ARGUMENT;
  if (!(o->dt_max >= 0.f) || !(o->dt_min == o->dt_min) ||
      (o->dt_max > 0.f && !(o->dt_min <= o->dt_max)))  // also rejects NaN
    return SSD_ERR_INVALID_ARGUMENT;
  return SSD_OK;
}

ssd_status device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return SSD_ERR_NO_DEVICE;
  return SSD_OK;
}

ssd_status from_hip(hipError_t e) {
  if (e == hipSuccess) return SSD_OK;
  if (e == hipErrorOutOfMemory) return SSD_ERR_OUT_OF_MEMORY;
  return SSD_ERR_HIP;
}

ssd_status check_forward_args(const ssd_problem* prob, const void* x, const float* dt,
                              const float* A, const void* B, const void* C, const float* D,
                              int64_t chunk_size, const float* h0, void* y, float* fin) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, dt, A, B, C, D, h0, y, fin};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SSD_ERR_INVALID_ARGUMENT;
  const Sizes s = sizes_of(prob);
  const Range ry = range_of(y, s.x);
  const Range inputs[] = {range_of(x, s.x),  range_of(dt, s.dt), range_of(A, s.hd),
                          range_of(B, s.bc), range_of(C, s.bc),  range_of(D, s.hd)};
  for (const Range& r : inputs)
    if (overlap(ry, r)) return SSD_ERR_INVALID_ARGUMENT;
  if (h0 && overlap(ry, range_of(h0, s.state))) return SSD_ERR_INVALID_ARGUMENT;
  if (fin) {
    const Range rf = range_of(fin, s.state);
    if (overlap(rf, ry)) return SSD_ERR_INVALID_ARGUMENT;
    for (const Range& r : inputs)
      if (overlap(rf, r)) return SSD_ERR_INVALID_ARGUMENT;
    if (h0 && overlap(rf, range_of(h0, s.state))) return SSD_ERR_INVALID_ARGUMENT;
  }
  return SSD_OK;
}

// Optional timing events around each kernel (caller-owned hipEvent_t's).
using Timer = ssd::KernelMarks;

struct Workspace {
  float *Acs, *dtc, *CB, *states, *h_in;
};

void workspace_sizes(const Dims& d, int64_t out[5]) {
  const int64_t aq = (int64_t)d.Bt * d.H * d.nc * d.Q * 4;
  out[0] = aq;
  out[1] = aq;
  out[2] = (int64_t)d.Bt * d.nc * d.G * d.Q * d.Q * 4;
  out[3] = (int64_t)d.Bt * d.nc * d.H * d.P * d.N * 4;
  out[4] = out[3];
}

int resolve_precision(int io, int prec) {
  if (io == ssd::kIoF32) return ssd::kPrecFp32;
  return prec;  // auto, fp16 or fp32 for bf16 io
}

int64_t unfused_workspace_bytes(const Dims& d, int64_t off[5]) {
  int64_t sz[5];
  workspace_sizes(d, sz);
  int64_t total = 0;
  for (int i = 0; i < 5; ++i) {
    off[i] = total;
    total += (sz[i] + 255) & ~int64_t(255);
  }
  return total;
}

// ws: unfused_workspace_bytes(d) bytes of device memory, or null to allocate them stream-ordered.
ssd_status run_unfused(const ssd_problem* prob, const Dims& d, int prec, const void* x,
                       const float* dt, const float* A, const void* B, const void* C,
                       const float* D, const float* h0, void* y, float* fin, hipStream_t s,
                       Timer& t, void* ws) {
  int64_t off[5];
  const int64_t total = unfused_workspace_bytes(d, off);
  void* base = ws;
  if (!base && hipMallocAsync(&base, (size_t)total, s) != hipSuccess) return SSD_ERR_OUT_OF_MEMORY;
  char* b = static_cast<char*>(base);
  Workspace w{reinterpret_cast<float*>(b + off[0]), reinterpret_cast<float*>(b + off[1]),
              reinterpret_cast<float*>(b + off[2]), reinterpret_cast<float*>(b + off[3]),
              reinterpret_cast<float*>(b + off[4])};
  const int io = prob->io_dtype;
  hipError_t e = t.mark(s);
  if (e == hipSuccess) e = ssd::launch_chunk_cumsum(d, dt, A, w.Acs, w.dtc, s);
  if (e == hipSuccess) e = t.mark(s);
  if (e == hipSuccess) e = ssd::launch_bmm_chunk(d, io, B, C, w.CB, s);
  if (e == hipSuccess) e = t.mark(s);
  if (e == hipSuccess) e = ssd::launch_chunk_state(d, io, prec, x, B, w.Acs, w.dtc, w.states, s);
  if (e == hipSuccess) e = t.mark(s);
  if (e == hipSuccess) e = ssd::launch_state_passing(d, w.states, w.Acs, h0, w.h_in, fin, s);
  if (e == hipSuccess) e = t.mark(s);
  if (e == hipSuccess)
    e = ssd::launch_chunk_scan(d, io, prec, x, C, w.CB, w.Acs, w.dtc, w.h_in, D, y, s);
  if (e == hipSuccess) e = t.mark(s);
  hipError_t ef = ws ? hipSuccess : hipFreeAsync(base, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(ef);
}

// The unfused path's S1, S2 and S5 only, with the entering state of every chunk read from h_in
// (the backward's transposed recurrences read, transposed, those of the untransposed ones: see
// Dims::hin_transposed); fp32 arithmetic.
ssd_status run_unfused_scan(const ssd_problem* prob, const Dims& d, const void* x,
                            const float* dt, const float* A, const void* B, const void* C,
                            const float* D, const float* h_in, void* y, hipStream_t s) {
  int64_t sz[5];
  workspace_sizes(d, sz);
  const int64_t od = (sz[0] + 255) & ~int64_t(255), oc = od + ((sz[1] + 255) & ~int64_t(255));
  void* base = nullptr;
  if (hipMallocAsync(&base, (size_t)(oc + sz[2]), s) != hipSuccess) return SSD_ERR_OUT_OF_MEMORY;
  char* b = static_cast<char*>(base);
  float *Acs = reinterpret_cast<float*>(b), *dtc = reinterpret_cast<float*>(b + od),
        *CB = reinterpret_cast<float*>(b + oc);
  const int io = prob->io_dtype;
  hipError_t e = ssd::launch_chunk_cumsum(d, dt, A, Acs, dtc, s);
  if (e == hipSuccess) e = ssd::launch_bmm_chunk(d, io, B, C, CB, s);
  if (e == hipSuccess)
    e = ssd::launch_chunk_scan(d, io, ssd::kPrecFp32, x, C, CB, Acs, dtc, h_in, D, y, s);
  const hipError_t ef = hipFreeAsync(base, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(ef);
}

// Compute units of the current device (cached per device).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

// Fused forward: run states, the chain over runs (several runs per sequence) and the fused scan.
// Runs are run_chunks chunks long when run_chunks > 0, else planned to give about one block per
// compute unit (each run boundary costs one fp16 state write and read, twice). ws: the workspace
// (fp16 run states and decays; none with one run per sequence), or null to allocate it
// stream-ordered.
ssd_status run_fused(const Dims& d, const ssd::FusedPlan& fp, const void* x, const float* dt,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* h0, void* y, float* fin, hipStream_t s, Timer& t, void* ws) {
  const int64_t bytes = ssd::fused_workspace_bytes(d, fp);
  void* w = ws;
  const bool own = bytes > 0 && !ws;
  if (own && hipMallocAsync(&w, (size_t)bytes, s) != hipSuccess) return SSD_ERR_OUT_OF_MEMORY;
  hipError_t e = ssd::launch_fused(d, fp, x, B, C, dt, A, D, h0, y, fin, w, &t, s);
  hipError_t ef = own ? hipFreeAsync(w, s) : hipSuccess;
  if (e != hipSuccess) return from_hip(e);
  return from_hip(ef);
}

// The kernels a forward launches, for the caller's optional out fields.
void report_kernels(const ssd_options* o, int mask) {
  if (!o) return;
  if (o->n_kernels) *o->n_kernels = __builtin_popcount((unsigned)mask);
  if (o->kernel_mask) *o->kernel_mask = mask;
}

// The forward behind ssd_forward_ex (noalloc false: workspace allocated stream-ordered) and
// ssd_forward_noalloc (noalloc true: workspace from the device's static scratch, plans fitted to it).
ssd_status forward_impl(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                        const void* B, const void* C, const float* D, int64_t chunk_size,
                        const float* initial_state, void* y, float* final_state, void* stream,
                        const ssd_options* opts, bool noalloc) {
  ssd_status st = check_forward_args(prob, x, dt, A, B, C, D, chunk_size, initial_state, y,
                                     final_state);
  if (st != SSD_OK) return st;
  st = check_options(opts);
  if (st != SSD_OK) return st;
  if (opts && opts->dt_bias) {  // an input too: no output may overlap it
    const Sizes sz = sizes_of(prob);
    const Range rb = range_of(opts->dt_bias, sz.hd);
    if (overlap(rb, range_of(y, sz.x)) ||
        (final_state && overlap(rb, range_of(final_state, sz.state))))
      return SSD_ERR_INVALID_ARGUMENT;
  }
  st = device_ready();
  if (st != SSD_OK) return st;
  Dims d = make_dims(prob, chunk_size);
  if (opts) {
    d.dt_bias = opts->dt_bias;
    d.dt_softplus = opts->dt_softplus;
    d.dt_min = opts->dt_min;
    d.dt_max = opts->dt_max;
  }
  const int prec = resolve_precision(prob->io_dtype, opts ? opts->precision : 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int variant = opts ? opts->variant : SSD_VARIANT_AUTO;
  // The fused kernels cover bf16 io with fp16 operands for headdim 64 or 128 and dstate 64,
  // 128 or 256.
  ssd::FusedPlan fp{};
  const int64_t run_tokens = opts && opts->run_chunks > 0 ? (int64_t)opts->run_chunks * chunk_size : 0;
  const bool fusable = prob->io_dtype == SSD_DTYPE_BF16 && prec != ssd::kPrecFp32 &&
                       ssd::fused_plan(d, (int)(run_tokens < (1 << 30) ? run_tokens : (1 << 30)),
                                       compute_units(), &fp);
  if (variant == SSD_VARIANT_FUSED && !fusable) return SSD_ERR_UNSUPPORTED;
  // auto: the last run's state, which goes into the final state, takes the hi + lo split over
  // the sequence's last 128 tokens; fp16: every operand rounded once
  fp.split = prec != ssd::kPrecFp16;
  Timer t;
  if (opts && opts->n_events > 0) {
    t.ev = opts->events;
    t.n = opts->n_events;
  }
  const bool quad = ssd::quadratic_covers(d);
  if (variant == SSD_VARIANT_QUADRATIC && !quad) return SSD_ERR_UNSUPPORTED;
  // auto: problems the fused kernels do not cover, short and small enough that the one-kernel
  // quadratic form stays latency-bound (at most 8192 token x dstate products per row of its
  // masked block, at most two blocks per compute unit), take it instead of the five unfused
  // kernels (measured: 256 tokens, dstate 16, 2 heads: 32 vs 51 us; it loses beyond these bounds)
  const bool quad_auto = variant == SSD_VARIANT_AUTO && !fusable && quad &&
                         (int64_t)d.L * d.N <= 8192 &&
                         ssd::quadratic_blocks(d) <= 2 * (int64_t)compute_units();
  if (variant == SSD_VARIANT_QUADRATIC || quad_auto) {
    report_kernels(opts, SSD_KERNEL_QUADRATIC);
    hipError_t e = t.mark(s);
    if (e == hipSuccess)
      e = ssd::launch_quadratic(d, prob->io_dtype, x, dt, A, B, C, D, initial_state, y,
                                final_state, s);
    if (e == hipSuccess) e = t.mark(s);
    return from_hip(e);
  }
  const bool fused = variant != SSD_VARIANT_UNFUSED && fusable;
  void* ws = nullptr;
  if (noalloc) {
    // the fused plan's runs are lengthened until its workspace fits the scratch (one run per
    // sequence needs none); the unfused workspace must fit as it is
    if (fused) {
      while (ssd::fused_workspace_bytes(d, fp) > ssd::kScratchBytes && fp.nr > 1) {
        const bool split = fp.split;
        ssd::fused_plan(d, fp.run_len * 2, compute_units(), &fp);
        fp.split = split;
      }
    } else {
      int64_t off[5];
      if (unfused_workspace_bytes(d, off) > ssd::kScratchBytes) return SSD_ERR_WORKSPACE_LIMIT;
    }
    const hipError_t e = ssd::scratch_address(&ws);
    if (e != hipSuccess) return from_hip(e);
  }
  if (fused)
    report_kernels(opts, ((fp.nr > 1 || final_state) ? SSD_KERNEL_FUSED_RUN_STATES : 0) |
                             (fp.nr > 1 ? SSD_KERNEL_FUSED_CHAIN : 0) | SSD_KERNEL_FUSED_SCAN);
  else
    report_kernels(opts, SSD_KERNEL_CHUNK_CUMSUM | SSD_KERNEL_BMM_CHUNK |
                             SSD_KERNEL_CHUNK_STATE | SSD_KERNEL_STATE_PASSING |
                             SSD_KERNEL_CHUNK_SCAN);
  if (fused)
    return run_fused(d, fp, x, dt, A, B, C, D, initial_state, y, final_state, s, t, ws);
  return run_unfused(prob, d, prec, x, dt, A, B, C, D, initial_state, y, final_state, s, t, ws);
}

}  // namespace

extern "C" {

ssd_status ssd_forward_ex(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                          const void* B, const void* C, const float* D, int64_t chunk_size,
                          const float* initial_state, void* y, float* final_state, void* stream,
                          const ssd_options* opts) {
  return forward_impl(prob, x, dt, A, B, C, D, chunk_size, initial_state, y, final_state, stream,
                      opts, false);
}

ssd_status ssd_forward_noalloc(const ssd_problem* prob, const void* x, const float* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               int64_t chunk_size, const float* initial_state, void* y,
                               float* final_state, void* stream, const ssd_options* opts) {
  return forward_impl(prob, x, dt, A, B, C, D, chunk_size, initial_state, y, final_state, stream,
                      opts, true);
}

ssd_status ssd_forward(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, int64_t chunk_size,
                       const float* initial_state, void* y, float* final_state, void* stream) {
  return ssd_forward_ex(prob, x, dt, A, B, C, D, chunk_size, initial_state, y, final_state,
                        stream, nullptr);
}

ssd_status ssd_workspace_sizes(const ssd_problem* prob, int64_t chunk_size, int64_t sizes[5]) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  if (!sizes) return SSD_ERR_INVALID_ARGUMENT;
  workspace_sizes(make_dims(prob, chunk_size), sizes);
  return SSD_OK;
}

ssd_status ssd_chunk_cumsum(const ssd_problem* prob, const float* dt, const float* A,
                            int64_t chunk_size, float* Acs, float* dtc, void* stream) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  if (!dt || !A || !Acs || !dtc) return SSD_ERR_INVALID_ARGUMENT;
  const Dims d = make_dims(prob, chunk_size);
  int64_t ws[5];
  workspace_sizes(d, ws);
  const Sizes s = sizes_of(prob);
  const Range ra = range_of(Acs, ws[0]), rd = range_of(dtc, ws[1]);
  if (overlap(ra, rd) || overlap(ra, range_of(dt, s.dt)) || overlap(rd, range_of(dt, s.dt)))
    return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  return from_hip(ssd::launch_chunk_cumsum(d, dt, A, Acs, dtc, static_cast<hipStream_t>(stream)));
}

ssd_status ssd_bmm_chunk(const ssd_problem* prob, const void* B, const void* C,
                         int64_t chunk_size, float* CB, void* stream) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  if (!B || !C || !CB || !aligned16(B) || !aligned16(C) || !aligned16(CB))
    return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  const Dims d = make_dims(prob, chunk_size);
  return from_hip(
      ssd::launch_bmm_chunk(d, prob->io_dtype, B, C, CB, static_cast<hipStream_t>(stream)));
}

ssd_status ssd_chunk_state(const ssd_problem* prob, const void* x, const void* B,
                           const float* Acs, const float* dtc, int64_t chunk_size, float* states,
                           void* stream, const ssd_options* opts) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  st = check_options(opts);
  if (st != SSD_OK) return st;
  if (!x || !B || !Acs || !dtc || !states || !aligned16(x) || !aligned16(B) ||
      !aligned16(states))
    return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  const Dims d = make_dims(prob, chunk_size);
  const int prec = resolve_precision(prob->io_dtype, opts ? opts->precision : 0);
  return from_hip(ssd::launch_chunk_state(d, prob->io_dtype, prec, x, B, Acs, dtc, states,
                                          static_cast<hipStream_t>(stream)));
}

// The backward's own chunk length: its fp32 recurrences cost least with short chunks (the
// quadratic intra-chunk work shrinks with the chunk, the chunk states it adds are cheap), and the
// result does not depend on where the chunks start.
constexpr int64_t kBackwardChunk = 64;

ssd_status ssd_backward(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                        const void* B, const void* C, const float* D, int64_t chunk_size,
                        const float* initial_state, const void* dy, const float* dfinal,
                        float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD,
                        float* dinitial_state, void* stream) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  st = check_problem(prob, kBackwardChunk);  // the backward's own chunking must fit too
  if (st != SSD_OK) return st;
  // the transposed problems (head dim and state dim swapped, one group per head) must fit too
  ssd_problem tp = *prob;
  tp.headdim = prob->dstate;
  tp.dstate = prob->headdim;
  tp.ngroups = prob->nheads;
  tp.io_dtype = SSD_DTYPE_F32;
  st = check_problem(&tp, kBackwardChunk);
  if (st != SSD_OK) return st;
  // The reversed-time recurrences run over pad leading tokens of no input and no decay, so that
  // their chunk boundaries fall on the forward recurrence's (Lp % Q == 0): the states both hold
  // there give the decay gradient's exact value at the first token of every 256-token tile.
  const int64_t pad = (kBackwardChunk - prob->seqlen % kBackwardChunk) % kBackwardChunk;
  const int64_t Lp = prob->seqlen + pad;
  ssd_problem pp = *prob, tpp = tp;
  pp.seqlen = Lp;
  tpp.seqlen = Lp;
  st = check_problem(&pp, kBackwardChunk);
  if (st == SSD_OK) st = check_problem(&tpp, kBackwardChunk);
  if (st != SSD_OK) return st;
  if (!x || !dt || !A || !B || !C || !D || !dy || !dx || !ddt || !dA || !dB || !dC || !dD)
    return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x,  dt, A,  B,  C,  D,  initial_state, dy, dfinal,
                        dx, ddt, dA, dB, dC, dD, dinitial_state};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SSD_ERR_INVALID_ARGUMENT;
  const Sizes s = sizes_of(prob);
  const int64_t Bt = prob->batch, L = prob->seqlen, H = prob->nheads, P = prob->headdim,
                N = prob->dstate, G = prob->ngroups;
  const int64_t nx = Bt * L * H * P, nb = Bt * L * G * N, nt = Bt * L * H * N, nd = Bt * L * H,
                ns = Bt * H * P * N;
  const Range ins[] = {range_of(x, s.x),        range_of(dt, s.dt),  range_of(A, s.hd),
                       range_of(B, s.bc),       range_of(C, s.bc),   range_of(D, s.hd),
                       range_of(dy, s.x),       initial_state ? range_of(initial_state, s.state)
                                                              : Range{0, 0},
                       dfinal ? range_of(dfinal, s.state) : Range{0, 0}};
  const Range outs[] = {range_of(dx, nx * 4),  range_of(ddt, nd * 4), range_of(dA, H * 4),
                        range_of(dB, nb * 4),  range_of(dC, nb * 4),  range_of(dD, H * 4),
                        dinitial_state ? range_of(dinitial_state, ns * 4) : Range{0, 0}};
  for (int i = 0; i < 7; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSD_ERR_INVALID_ARGUMENT;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return SSD_ERR_INVALID_ARGUMENT;
  }
  st = device_ready();
  if (st != SSD_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  // the forward-time recurrences (1, 3) read the caller's x, B, C and dy in place, bf16 ones
  // widened exactly and computed in fp32 (f32_math)
  Dims d = make_dims(prob, kBackwardChunk);
  d.f32_math = 1;
  Dims dup = make_dims(&pp, kBackwardChunk);  // the adjoint: reversed, padded, unit input weight
  dup.unit_input = 1;
  dup.f32_math = 1;
  // the transposed problems' input is B (or C) per head: read in place, shared by each group
  ssd_problem tpio = tp;
  tpio.io_dtype = prob->io_dtype;
  Dims dT = make_dims(&tp, kBackwardChunk);
  dT.x_groups = (int)G;
  dT.f32_math = 1;
  ssd_problem tppio = tpp;
  tppio.io_dtype = prob->io_dtype;
  Dims dTup = make_dims(&tpp, kBackwardChunk);
  dTup.x_groups = (int)G;
  dTup.unit_input = 1;
  dTup.f32_math = 1;
  int64_t off1[5], off2[5];
  const int64_t ws1 = unfused_workspace_bytes(d, off1), ws2 = unfused_workspace_bytes(dup, off2);
  const int64_t ntile = (L + 255) / 256;
  const int64_t nxp = Bt * Lp * H * P, nbp = Bt * Lp * G * N, ntp = Bt * Lp * H * N,
                ndp = Bt * Lp * H;
  // workspace (fp32): see the steps below for what each holds; WS1 and WS2 are the unfused
  // workspaces of steps 1 and 2 (kept for their chunk-entry states), ANCH doubles
  enum { Y0, XR, BR, CR, DTR, UR, G0, YT, CTR, YTR, Q, XU, DYX, PA, PD, WS1, WS2, ANCH, NBUF };
  // (XR, BR, CR and CTR hold reversed copies in the io type)
  const int64_t eb = io_bytes(prob);
  const int64_t rx = (nxp * eb + 3) / 4, rb = (nbp * eb + 3) / 4;
  const int64_t el[NBUF] = {nx, rx, rb, rb, ndp, nxp, ns, nt, rx, ntp, nd, nd, nd,
                            2 * Bt * H, 2 * Bt * H, (ws1 + 3) / 4, (ws2 + 3) / 4,
                            2 * Bt * H * ntile};
  int64_t off[NBUF], total = 0;
  for (int i = 0; i < NBUF; ++i) {
    off[i] = total;
    total += (el[i] * 4 + 255) & ~int64_t(255);
  }
  void* base = nullptr;
  if (hipMallocAsync(&base, (size_t)total, hs) != hipSuccess) return SSD_ERR_OUT_OF_MEMORY;
  float* w[NBUF];
  for (int i = 0; i < NBUF; ++i) w[i] = reinterpret_cast<float*>(static_cast<char*>(base) + off[i]);

  const int io = prob->io_dtype;
  const int iBt = (int)Bt, iL = (int)L, iH = (int)H, iP = (int)P, iN = (int)N, iG = (int)G,
            ipad = (int)pad;
  Timer none;
  ssd_status r = SSD_OK;
  auto hip = [&](hipError_t e) {
    if (r == SSD_OK && e != hipSuccess) r = from_hip(e);
  };
  auto fwd = [&](const ssd_problem* pr, const Dims& dd, const void* xx, const float* dtt,
                 const void* bb, const void* cc, const float* h0, float* yy, float* fin,
                 float* ws) {
    if (r == SSD_OK)
      r = run_unfused(pr, dd, ssd::kPrecFp32, xx, dtt, A, bb, cc, nullptr, h0, yy, fin, hs, none,
                      ws);
  };
  // (the recurrences below compute state terms only: no skip term D)
  // 1. forward: the state part of y (ys = y - D x); its chunk-entry states stay in WS1
  fwd(prob, d, x, dt, B, C, initial_state, w[Y0], nullptr, w[WS1]);
  // 2. adjoint G_t = dy_t C_t^T + exp(dt_{t+1} A) G_{t+1} as a forward recurrence in reversed
  //    time (decay of the next token, unit input weight) from dfinal, after pad tokens of zero
  //    input and zero dt (the state passes them unchanged); its readout with B gives u_t = G_t B_t,
  //    its final state G_0, its chunk-entry states (in WS2) G_t at the forward chunks' starts
  // (reversed copies of the caller's tensors in their own type, widened to fp32 where read)
  hip(ssd::launch_reverse_rows(io, dy, w[XR], iBt, iL, iH * iP, ipad, hs));
  hip(ssd::launch_reverse_rows(io, C, w[BR], iBt, iL, iG * iN, ipad, hs));
  hip(ssd::launch_reverse_rows(io, B, w[CR], iBt, iL, iG * iN, ipad, hs));
  hip(ssd::launch_dt_shift_rev(dt, w[DTR], iBt, iL, iH, ipad, hs));
  fwd(&pp, dup, w[XR], w[DTR], w[BR], w[CR], dfinal, w[UR], w[G0], w[WS2]);
  // chunk-entry states of steps 1 and 2 ([Bt, nc, H, P, N]): the anchors of the decay gradient,
  // and, transposed, the entering states of steps 3 and 4
  const float* hf = reinterpret_cast<const float*>(reinterpret_cast<const char*>(w[WS1]) + off1[4]);
  const float* hg = reinterpret_cast<const float*>(reinterpret_cast<const char*>(w[WS2]) + off2[4]);
  auto scan = [&](const ssd_problem* pr, const Dims& dd, const void* xx, const float* dtt,
                  const void* bb, const void* cc, const float* h_in, float* yy) {
    if (r == SSD_OK)
      r = run_unfused_scan(pr, dd, xx, dtt, A, bb, cc, nullptr, h_in, yy, hs);
  };
  // 3. dC: the transposed state S_t^T (state dim N, head dim P) read out with dy; its input is
  //    B of the head's group. Its chunk-entry states are those of step 1, transposed (the same
  //    chunks), so only its cumulative decay, C B^T and chunk scan run.
  dT.hin_transposed = 1;
  scan(&tpio, dT, B, dt, x, dy, hf, w[YT]);
  // 4. dB: the transposed adjoint G_t^T in reversed time (padded as step 2), read out with x; its
  //    input is C of the head's group in reversed time (step 2's BR); entering states: step 2's,
  //    transposed
  hip(ssd::launch_reverse_rows(io, x, w[CTR], iBt, iL, iH * iP, ipad, hs));
  dTup.hin_transposed = 1;
  scan(&tppio, dTup, w[BR], w[DTR], w[XR], w[CTR], hg, w[YTR]);
  // 5. the gradients
  hip(ssd::launch_bwd_pointwise(io, x, dy, w[UR], w[Y0], dt, D, dx, w[Q], w[XU], w[DYX], iBt, iL,
                                iH, iP, ipad, hs));
  double* pa = reinterpret_cast<double*>(w[PA]);
  double* pd = reinterpret_cast<double*>(w[PD]);
  double* anch = reinterpret_cast<double*>(w[ANCH]);
  hip(ssd::launch_anchor_dot(hf, hg, w[G0], anch, iBt, iH, iP * iN, (int)kBackwardChunk, d.nc,
                             dup.nc, iL, (int)Lp, hs));
  hip(ssd::launch_bwd_scan(w[Q], w[XU], w[DYX], dt, A, anch, ddt, pa, pd, iBt, iL, iH, hs));
  hip(ssd::launch_sum_batch(pa, pd, dA, dD, iBt, iH, hs));
  hip(ssd::launch_group_sums(w[YTR], w[YT], dt, dB, dC, iBt, iL, iH, iG, iN, ipad, hs));
  if (dinitial_state)
    hip(ssd::launch_scale_state(w[G0], dt, A, dinitial_state, iBt, iL, iH, iP * iN, hs));
  const hipError_t ef = hipFreeAsync(base, hs);
  if (r != SSD_OK) return r;
  return from_hip(ef);
}

ssd_status ssd_step(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* state_in,
                    float* state_out, void* y, void* stream) {
  ssd_status st = check_problem(prob, 16);  // the chunk length plays no part in a step
  if (st != SSD_OK) return st;
  if (prob->seqlen != 1) return SSD_ERR_INVALID_ARGUMENT;
  if (!x || !dt || !A || !B || !C || !D || !state_in || !state_out || !y)
    return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, dt, A, B, C, D, state_in, state_out, y};
  for (const void* q : ptrs)
    if (!aligned16(q)) return SSD_ERR_INVALID_ARGUMENT;
  const Sizes s = sizes_of(prob);  // seqlen 1: x and y [batch, nheads, headdim], B/C per group
  const Range ry = range_of(y, s.x), rso = range_of(state_out, s.state),
              rsi = range_of(state_in, s.state);
  const Range inputs[] = {range_of(x, s.x),  range_of(dt, s.dt), range_of(A, s.hd),
                          range_of(B, s.bc), range_of(C, s.bc),  range_of(D, s.hd)};
  for (const Range& r : inputs)
    if (overlap(ry, r) || overlap(rso, r)) return SSD_ERR_INVALID_ARGUMENT;
  if (overlap(ry, rsi) || overlap(ry, rso)) return SSD_ERR_INVALID_ARGUMENT;
  if (state_out != state_in && overlap(rso, rsi)) return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  const Dims d = make_dims(prob, 16);
  return from_hip(ssd::launch_step(d, prob->io_dtype, x, dt, A, B, C, D, state_in, state_out, y,
                                   static_cast<hipStream_t>(stream)));
}

ssd_status ssd_state_passing(const ssd_problem* prob, const float* states, const float* Acs,
                             int64_t chunk_size, const float* initial_state, float* h_in,
                             float* final_state, void* stream) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  if (!states || !Acs || !h_in) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {states, h_in, initial_state, final_state};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SSD_ERR_INVALID_ARGUMENT;
  const Dims d = make_dims(prob, chunk_size);
  int64_t ws[5];
  workspace_sizes(d, ws);
  if (overlap(range_of(states, ws[3]), range_of(h_in, ws[4]))) return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  return from_hip(ssd::launch_state_passing(d, states, Acs, initial_state, h_in, final_state,
                                            static_cast<hipStream_t>(stream)));
}

ssd_status ssd_chunk_scan(const ssd_problem* prob, const void* x, const void* C, const float* CB,
                          const float* Acs, const float* dtc, const float* h_in, const float* D,
                          int64_t chunk_size, void* y, void* stream, const ssd_options* opts) {
  ssd_status st = check_problem(prob, chunk_size);
  if (st != SSD_OK) return st;
  st = check_options(opts);
  if (st != SSD_OK) return st;
  if (!x || !C || !CB || !Acs || !dtc || !h_in || !D || !y) return SSD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, C, CB, h_in, y};
  for (const void* q : ptrs)
    if (!aligned16(q)) return SSD_ERR_INVALID_ARGUMENT;
  const Sizes s = sizes_of(prob);
  if (overlap(range_of(y, s.x), range_of(x, s.x)) || overlap(range_of(y, s.x), range_of(C, s.bc)))
    return SSD_ERR_INVALID_ARGUMENT;
  st = device_ready();
  if (st != SSD_OK) return st;
  const Dims d = make_dims(prob, chunk_size);
  const int prec = resolve_precision(prob->io_dtype, opts ? opts->precision : 0);
  return from_hip(ssd::launch_chunk_scan(d, prob->io_dtype, prec, x, C, CB, Acs, dtc, h_in, D,
                                         y, static_cast<hipStream_t>(stream)));
}

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported problem";
    case SSD_ERR_NO_DEVICE: return "no HIP device";
    case SSD_ERR_OUT_OF_MEMORY: return "out of device memory";
    case SSD_ERR_HIP: return "HIP error";
    case SSD_ERR_WORKSPACE_LIMIT: return "workspace beyond the no-allocation scratch";
  }
  return "unknown status";
}

int ssd_version(void) { return kVersion; }

}  // extern "C"
