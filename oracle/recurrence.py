"""Token-by-token SSD recurrence in float64 -- test infrastructure, see the package header.

The selective state-space step is h_t = a_t * h_{t-1} + b_t * x_t, a multiplicative chain over t
("Why SSM and linear-RNN FLOPs do not convert into GPU FLOPs", first paragraph). In SSD (Mamba-2)
the decay is one scalar per head, shared by every state entry of that head (same page, both
paragraphs). Written out for head h with state S of shape [P, N]:

    a_t      = exp(dt[t, h] * A[h])                       scalar decay of step t
    S_t      = a_t * S_{t-1} + dt[t, h] * outer(x[t, h, :], B[t, g(h), :])
    y[t, h]  = S_t @ C[t, g(h), :] + D[h] * x[t, h, :]

with S_{-1} the initial state (zeros when absent), g(h) = h // (H / G) the B/C group of head h, and
the final state S_{L-1}. The state is stored [P, N] (head-dim rows, state columns).
"""

from __future__ import annotations

import numpy as np


def _as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _group_of_heads(nheads: int, ngroups: int) -> np.ndarray:
    if nheads % ngroups:
        raise ValueError("nheads must be a multiple of ngroups")
    return np.arange(nheads) // (nheads // ngroups)


def ssd_recurrence(x, dt, A, B, C, D, initial_state=None):
    """Run the recurrence over the whole sequence.

    x [Bt, L, H, P], dt [Bt, L, H], A [H], B and C [Bt, L, G, N], D [H],
    initial_state [Bt, H, P, N] or None.  Returns (y [Bt, L, H, P], final_state [Bt, H, P, N]),
    both float64.
    """
    x, dt, A, B, C, D = (_as64(v) for v in (x, dt, A, B, C, D))
    Bt, L, H, P = x.shape
    N = B.shape[3]
    grp = _group_of_heads(H, B.shape[2])
    S = np.zeros((Bt, H, P, N)) if initial_state is None else _as64(initial_state).copy()
    y = np.empty((Bt, L, H, P))
    for t in range(L):
        decay = np.exp(dt[:, t, :] * A[None, :])                  # [Bt, H]
        u = dt[:, t, :, None] * x[:, t]                            # [Bt, H, P]
        Bh = B[:, t][:, grp]                                       # [Bt, H, N]
        Ch = C[:, t][:, grp]                                       # [Bt, H, N]
        S = decay[:, :, None, None] * S + u[:, :, :, None] * Bh[:, :, None, :]
        y[:, t] = (S @ Ch[:, :, :, None])[..., 0] + D[None, :, None] * x[:, t]
    return y, S


def ssd_step(state, x, dt, A, B, C, D):
    """One recurrent (decode) step from `state`.

    state [Bt, H, P, N], x [Bt, H, P], dt [Bt, H], A [H], B and C [Bt, G, N], D [H].
    Returns (y [Bt, H, P], new_state [Bt, H, P, N]) in float64.
    """
    y, S = ssd_recurrence(_as64(x)[:, None], _as64(dt)[:, None], A, _as64(B)[:, None],
                          _as64(C)[:, None], D, initial_state=state)
    return y[:, 0], S
