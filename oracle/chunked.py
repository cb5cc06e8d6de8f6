"""Chunked SSD forward in float64, with every intermediate -- test infrastructure.

The sequence is cut into chunks of Q tokens (the last one may be shorter). The steps follow the
order the cuTile walkthrough describes ("Mamba-2 in NVIDIA cuTile: Faster Forward Kernels and What
the Benchmark Means", section "Why Mamba-2 is a useful kernel example"): first the cumulative decay
inside each chunk, then the state entering each chunk, then the outputs; inside a chunk the
quadratic masked form, across chunks the linear recurrence ("nitter.gq/da_be19" thread, post 5/6).

For chunk c (tokens cQ .. cQ+q_c-1, local index i or j) and head h of group g:

    S1  Acs[i]         = sum_{k<=i} dt[k] * A[h]                          (inclusive, per chunk)
    S2  CB[i, j]       = C[i] . B[j]                                      (shared by the group)
    S3  states[c]      = sum_j exp(Acs[last] - Acs[j]) * dt[j] * outer(x[j], B[j])
    S4  h_in[0]        = h0 (or 0);   h_in[c+1] = exp(Acs[last]) * h_in[c] + states[c]
    S5  y[i]           = sum_{j<=i} CB[i, j] * exp(Acs[i] - Acs[j]) * dt[j] * x[j]
                         + exp(Acs[i]) * h_in[c] @ C[i]  +  D * x[i]

and final_state = h_in[nc].  Only differences Acs[i] - Acs[j] with j <= i (never positive for
A <= 0, dt >= 0) are exponentiated, so no term overflows.
"""

from __future__ import annotations

import numpy as np


def ssd_chunked(x, dt, A, B, C, D, chunk_size, initial_state=None):
    """Chunked forward.  Returns (y, final_state, intermediates).

    intermediates holds
      "Acs"    [Bt, H, nc, Q]        inclusive cumulative decay per chunk; entries past the end of
                                     a ragged last chunk repeat its last value
      "CB"     [Bt, nc, G, Q, Q]     C_i . B_j for every (i, j) of the chunk (zero past its end)
      "states" [Bt, nc, H, P, N]     each chunk's own end state (zero state on entry)
      "h_in"   [Bt, nc + 1, H, P, N] state entering chunk c; h_in[:, nc] is the final state
    """
    x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Q = int(chunk_size)
    if Q < 1:
        raise ValueError("chunk_size must be positive")
    nc = -(-L // Q)
    Lp = nc * Q
    grp = np.arange(H) // (H // G)

    def pad(a):  # zero-pad the token axis (axis 1) to nc * Q
        w = [(0, 0)] * a.ndim
        w[1] = (0, Lp - L)
        return np.pad(a, w)

    # A padded token has dt = 0: it adds nothing to any state and does not decay it.
    xc = pad(x).reshape(Bt, nc, Q, H, P)
    dtc = pad(dt).reshape(Bt, nc, Q, H)
    Bc = pad(B).reshape(Bt, nc, Q, G, N)
    Cc = pad(C).reshape(Bt, nc, Q, G, N)

    # S1: per-chunk inclusive cumulative sum of dt * A.
    Acs = np.cumsum(dtc * A[None, None, None, :], axis=2)            # [Bt, nc, Q, H]
    Acs = np.transpose(Acs, (0, 3, 1, 2)).copy()                      # [Bt, H, nc, Q]
    # S2: C . B inside each chunk, per group.
    CB = np.einsum("bcign,bcjgn->bcgij", Cc, Bc)                      # [Bt, nc, G, Q, Q]

    states = np.empty((Bt, nc, H, P, N))
    y = np.empty((Bt, nc, Q, H, P))
    h_in = np.empty((Bt, nc + 1, H, P, N))
    h_in[:, 0] = 0.0 if initial_state is None else np.asarray(initial_state, dtype=np.float64)
    causal = np.tril(np.ones((Q, Q), dtype=bool))
    for b in range(Bt):
        for c in range(nc):
            acs = Acs[b, :, c, :]                                     # [H, Q]
            last = acs[:, Q - 1]                                      # [H]
            u = dtc[b, c, :, :, None] * xc[b, c]                      # [Q, H, P] = dt_j * x_j
            Bh = Bc[b, c][:, grp, :]                                  # [Q, H, N]
            Ch = Cc[b, c][:, grp, :]                                  # [Q, H, N]
            # S3: this chunk's own end state.
            w = np.exp(last[None, :] - acs.T)                         # [Q, H]
            states[b, c] = np.einsum("jh,jhp,jhn->hpn", w, u, Bh)
            # S4: state entering the next chunk.
            h_in[b, c + 1] = np.exp(last)[:, None, None] * h_in[b, c] + states[b, c]
            # S5: outputs -- intra-chunk masked form, inter-chunk readout, skip term.
            seg = acs[:, :, None] - acs[:, None, :]                   # [H, Q, Q]: Acs_i - Acs_j
            decay = np.where(causal[None], np.exp(np.where(causal[None], seg, 0.0)), 0.0)
            cb = CB[b, c][grp]                                        # [H, Q, Q]
            intra = np.einsum("hij,jhp->ihp", cb * decay, u)
            inter = np.exp(acs.T)[:, :, None] * np.einsum("ihn,hpn->ihp", Ch, h_in[b, c])
            y[b, c] = intra + inter + D[None, :, None] * xc[b, c]
    y = y.reshape(Bt, Lp, H, P)[:, :L]
    inter_out = {"Acs": Acs, "CB": CB, "states": states, "h_in": h_in}
    return y, h_in[:, nc].copy(), inter_out
