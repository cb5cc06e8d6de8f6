"""CPU oracle for the Mamba-2 SSD chunked forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import, call, link
or execute anything in this package. The GPU library never depends on it, and it shares no code
with the GPU library (no kernels, headers, helpers or constants). Both sides read the same seeded
input arrays, drawn by a generator module that holds none of the method's arithmetic.

What it computes (float64 throughout, from exactly widened inputs):

* ``recurrence.ssd_recurrence`` -- the definition: the selective state-space recurrence run token
  by token, with one scalar decay per head (the selective-SSM step of "Why SSM and linear-RNN FLOPs
  do not convert into GPU FLOPs", first paragraph, in the Mamba-2 SSD form: decay exp(dt*A_h),
  input dt*B_t*x_t, readout C_t*h_t plus the skip D*x_t).
* ``quadratic.ssd_quadratic`` -- the naive quadratic (masked, attention-like) form that the
  chunked algorithm's intra-chunk part uses, over the whole sequence ("nitter.gq/da_be19" thread,
  post 5/6). Its decay mask is built from running products, not from cumulative sums, so it is an
  independent formulation.
* ``chunked.ssd_chunked`` -- the chunked algorithm's steps in the order the cuTile walkthrough
  gives them ("Mamba-2 in NVIDIA cuTile: Faster Forward Kernels and What the Benchmark Means",
  section "Why Mamba-2 is a useful kernel example"): per-chunk cumulative decay, the state entering
  each chunk, then the outputs. It also returns every intermediate for per-stage checks.
* ``native`` -- the token-by-token recurrence again, in plain C with OpenMP over (batch, head), for
  full-size workloads and the timed CPU baseline.
* ``backward.ssd_backward`` -- the gradients of the recurrence with respect to every input, by
  reverse-mode differentiation of its steps (the backward pass training needs).
* ``dt.dt_effective`` -- the dt pre-processing (bias, softplus, clamp) written out from its
  definition; the recurrence then runs on its output.
* ``metrics`` -- the error measures the parity tests apply.

Pins: every function here is checked by the ``-m "not gpu"`` tests against values fixed outside
the oracle (hand-worked examples, closed forms, brute force on tiny inputs, invariants); none is
"parity unpinned".
"""

from .recurrence import ssd_recurrence, ssd_step
from .quadratic import ssd_quadratic
from .chunked import ssd_chunked
from .dt import dt_effective
from .backward import ssd_backward

__all__ = ["ssd_recurrence", "ssd_step", "ssd_quadratic", "ssd_chunked", "dt_effective",
           "ssd_backward"]
