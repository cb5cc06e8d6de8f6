"""Naive quadratic (masked, attention-like) form of SSD in float64 -- test infrastructure.

Unrolling the recurrence gives, for head h of group g and tokens s <= t,

    y[t] = sum_{s<=t} Lam[t, s] * (C[t] . B[s]) * dt[s] * x[s]  +  D * x[t]
           + (prod_{k<=t} a_k) * h0 @ C[t]
    Lam[t, s] = prod_{k=s+1..t} a_k      (1 on the diagonal, 0 above it)

which is the L x L masked form that the chunked algorithm applies inside each chunk ("nitter.gq/
da_be19" thread, post 5/6: the quadratic form, cheaper for short sequences). Lam is built row by
row from running products of the per-step decays a_k = exp(dt_k * A), never from differences of a
cumulative sum, so this file is an independent check of both the recurrence and the chunked
decomposition.  Cost is O(L^2) per head: meant for L up to a few hundred.
"""

from __future__ import annotations

import numpy as np


def decay_mask(a: np.ndarray) -> np.ndarray:
    """Lam[t, s] = prod_{k=s+1..t} a[k] for s <= t, else 0, by running products."""
    L = a.shape[0]
    lam = np.zeros((L, L))
    row = np.zeros(0)
    for t in range(L):
        row = np.append(row * a[t], 1.0)
        lam[t, : t + 1] = row
    return lam


def ssd_quadratic(x, dt, A, B, C, D, initial_state=None):
    """Same signature and result as recurrence.ssd_recurrence, via the L x L masked form."""
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    per_group = H // G
    y = np.empty((Bt, L, H, P))
    final = np.empty((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = h // per_group
            a = np.exp(dt[b, :, h] * A[h])                  # [L]
            lam = decay_mask(a)                             # [L, L]
            scores = C[b, :, g, :] @ B[b, :, g, :].T        # [L, L]: C_t . B_s
            u = dt[b, :, h, None] * x[b, :, h, :]           # [L, P]
            y[b, :, h, :] = (lam * scores) @ u + D[h] * x[b, :, h, :]
            final[b, h] = (lam[L - 1, :, None] * u).T @ B[b, :, g, :]
            if initial_state is not None:
                h0 = np.asarray(initial_state[b, h], dtype=np.float64)   # [P, N]
                from_start = np.empty(L)                    # prod_{k<=t} a_k, running product
                run = 1.0
                for t in range(L):
                    run *= a[t]
                    from_start[t] = run
                y[b, :, h, :] += from_start[:, None] * (C[b, :, g, :] @ h0.T)
                final[b, h] += from_start[L - 1] * h0
    return y, final
