"""Reverse-mode gradients of the SSD recurrence in float64 -- test infrastructure (package header).

Training "also depends on the backward pass" ("Mamba-2 in NVIDIA cuTile: Faster Forward Kernels
and What the Benchmark Means", section "What the speedup does and does not establish"). This is
the plain definition of that pass: the recurrence of ``recurrence.ssd_recurrence`` run forwards
token by token with every state kept, then differentiated in reverse order, step by step. For one
(batch, head) with state S_t of shape [P, N], decay a_t = exp(dt_t A), and a loss whose gradients
with respect to y and the final state are dy and dfinal:

    G_t   = dy_t C_t^T + a_{t+1} G_{t+1},   G_{L-1} = dy_{L-1} C_{L-1}^T + dfinal   (dL/dS_t)
    dx_t  = D dy_t + dt_t G_t B_t           dB_t += dt_t G_t^T x_t      dC_t += S_t^T dy_t
    dlog a_t = <G_t, a_t S_{t-1}>           ddt_t = A dlog a_t + x_t . (G_t B_t)
    dA    = sum_t dt_t dlog a_t             dD = sum_t dy_t . x_t        dS_{-1} = a_0 G_0

(B and C gradients summed over the heads of their group; dA and dD over batch and time.)
"""

from __future__ import annotations

import numpy as np

from .recurrence import _as64, _group_of_heads


def ssd_backward(x, dt, A, B, C, D, dy, initial_state=None, dfinal=None):
    """Gradients of sum(dy * y) + sum(dfinal * final_state) with respect to every input.

    Shapes as in ``ssd_recurrence``; dy [Bt, L, H, P], dfinal [Bt, H, P, N] or None.
    Returns a dict of float64 arrays: dx, ddt, dA, dB, dC, dD, dinitial_state, dlog_decay
    [Bt, L, H] = dL/d(dt_t A), the per-token terms that dA and ddt are built from, and
    dlog_decay_abs [Bt, L, H], the sum of the absolute values of the products that dlog_decay
    sums (a scale for rounding-error bounds; no gradient).
    """
    x, dt, A, B, C, D, dy = (_as64(v) for v in (x, dt, A, B, C, D, dy))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = _group_of_heads(H, G)
    S0 = np.zeros((Bt, H, P, N)) if initial_state is None else _as64(initial_state)

    # forward, keeping the state entering and leaving every step
    a = np.exp(dt * A[None, None, :])                               # [Bt, L, H]
    states = np.empty((L + 1, Bt, H, P, N))                         # states[t + 1] = S_t
    states[0] = S0
    for t in range(L):
        Bh = B[:, t][:, grp]                                        # [Bt, H, N]
        states[t + 1] = (a[:, t, :, None, None] * states[t]
                         + (dt[:, t, :, None] * x[:, t])[..., None] * Bh[:, :, None, :])

    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dlog = np.empty_like(dt)
    dlog_abs = np.empty_like(dt)
    dA = np.zeros(H)
    dBh = np.zeros((Bt, L, H, N))
    dCh = np.zeros((Bt, L, H, N))
    Gs = np.zeros((Bt, H, P, N)) if dfinal is None else _as64(dfinal).copy()
    for t in range(L - 1, -1, -1):
        Bh = B[:, t][:, grp]
        Ch = C[:, t][:, grp]
        # dL/dS_t: the readout of step t plus what flows back from step t + 1 (already decayed)
        Gs = Gs + dy[:, t][..., None] * Ch[:, :, None, :]
        GB = (Gs @ Bh[..., None])[..., 0]                           # G_t B_t       [Bt, H, P]
        dx[:, t] = D[None, :, None] * dy[:, t] + dt[:, t, :, None] * GB
        dBh[:, t] = dt[:, t, :, None] * (np.swapaxes(Gs, 2, 3) @ x[:, t][..., None])[..., 0]
        dCh[:, t] = (np.swapaxes(states[t + 1], 2, 3) @ dy[:, t][..., None])[..., 0]
        dloga = np.einsum("bhpn,bhpn->bh", Gs, a[:, t, :, None, None] * states[t])
        dlog[:, t] = dloga
        dlog_abs[:, t] = np.einsum("bhpn,bhpn->bh", np.abs(Gs),
                                   a[:, t, :, None, None] * np.abs(states[t]))
        ddt[:, t] = A[None, :] * dloga + np.einsum("bhp,bhp->bh", x[:, t], GB)
        dA += np.sum(dt[:, t] * dloga, axis=0)
        Gs = a[:, t, :, None, None] * Gs                            # into dL/dS_{t-1}
    dB = np.zeros((Bt, L, G, N))
    dC = np.zeros((Bt, L, G, N))
    for h in range(H):
        dB[:, :, grp[h]] += dBh[:, :, h]
        dC[:, :, grp[h]] += dCh[:, :, h]
    dD = np.einsum("blhp,blhp->h", dy, x)
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dinitial_state=Gs, dlog_decay=dlog,
                dlog_decay_abs=dlog_abs)
