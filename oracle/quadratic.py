"""Quadratic ("masked attention") form of the SSD forward, NumPy fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It exists to pin the
C recurrence: it reaches the same result by a different route, so a dropped
term, a wrong sign or a transposed operand in either one shows up as a
mismatch.  Cost is O(L^2) per head, so it is for tiny inputs only.

Written from the duality the flash-linear-attention PR #49 page relies on when
it swaps the mamba2 chunk-scan kernel for simple_gla (its list of differences
between the two kernels): the SSD output is gated linear attention with
query C, key B, value dt*x, log-gate dt*A (constant A per head), no
1/sqrt(d) scaling, and keys/queries shared by a group of heads.  Unrolling
h_t = a_t h_{t-1} + dt_t x_t B_t^T gives, with c_t = sum_{r<=t} dt_r A:

  y_t  = sum_{s<=t} exp(c_t - c_s) (C_t . B_s) dt_s x_s
         + exp(c_t) C_t . h_{-1} + D x_t
  h_{L-1} = exp(c_{L-1}) h_{-1} + sum_s exp(c_{L-1} - c_s) dt_s x_s B_s^T

and out = y * silu(z) when a gate is given.

With seq_idx (several sequences packed along a batch row; the state restarts
from zero where the label changes) a pair (t, s) interacts only when no
sequence starts in (s, t]: with k_t the number of sequence starts up to t,
the decay mask keeps s <= t with k_s = k_t, the initial state reaches only
the steps with k_t = 0, and the final state sums only over the steps of the
row's last sequence (plus the initial state if the row holds one sequence).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def _segment_sums(dA: np.ndarray) -> np.ndarray:
    """seg[t, s] = sum_{r=s+1..t} dA[r] for s <= t, -inf above the diagonal.

    Each entry is summed over its own segment (a masked cumulative sum down
    the columns) rather than taken as a difference of two long prefix sums."""
    T = dA.shape[0]
    r = np.arange(T)
    # rep[r, s] = dA[r] where r > s, else 0; its running sum down r gives seg.
    rep = np.where(r[:, None] > r[None, :], dA[:, None], 0.0)
    seg = np.cumsum(rep, axis=0)
    seg[np.triu_indices(T, 1)] = -np.inf
    return seg


def _sequence_counts(seq_row) -> np.ndarray:
    """k_t = number of steps r <= t (r > 0) whose label differs from step r-1's."""
    seq_row = np.asarray(seq_row)
    starts = np.concatenate([[0], (seq_row[1:] != seq_row[:-1]).astype(np.int64)])
    return np.cumsum(starts)


def ssd_fwd_quadratic(x, dt, A, B, C, D=None, z=None, dt_bias=None,
                      dt_limit=(0.0, float("inf")), initial_states=None, seq_idx=None):
    """Same arguments and layouts as ``oracle.ssd_fwd``; returns (out, final)."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    u = dt + (0.0 if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)[None, None, :])
    dtv = np.clip(np.logaddexp(0.0, u), dt_limit[0], dt_limit[1])  # softplus, then dt_limit
    out = np.zeros((b, L, H, P))
    final = np.zeros((b, H, P, N))
    for bi in range(b):
        k = _sequence_counts(seq_idx[bi]) if seq_idx is not None else np.zeros(L, np.int64)
        same = k[:, None] == k[None, :]                  # [t, s]: same packed sequence
        first = (k == 0).astype(np.float64)              # steps the initial state reaches
        last = (k == k[-1]).astype(np.float64) if L else k.astype(np.float64)
        for h in range(H):
            g = h // hpg
            dA = dtv[bi, :, h] * A[h]
            seg = _segment_sums(dA)                      # [t, s]
            decay = np.exp(seg) * same                   # 0 above the diagonal
            scores = C[bi, :, g, :] @ B[bi, :, g, :].T   # [t, s] = C_t . B_s
            v = dtv[bi, :, h][:, None] * x[bi, :, h, :]  # [s, p]
            y = (decay * scores) @ v
            c = np.cumsum(dA)
            fin = ((np.exp(c[-1] - c) * last)[:, None] * v).T @ B[bi, :, g, :]  # [p, n]
            if initial_states is not None:
                h0 = np.asarray(initial_states, dtype=np.float64)[bi, h]  # [p, n]
                y += (np.exp(c) * first)[:, None] * (C[bi, :, g, :] @ h0.T)
                if L == 0 or k[-1] == 0:
                    fin += (np.exp(c[-1]) if L else 1.0) * h0
            if D is not None:
                y += float(D[h]) * x[bi, :, h, :]
            if z is not None:
                zz = np.asarray(z, dtype=np.float64)[bi, :, h, :]
                y *= zz * expit(zz)
            out[bi, :, h, :] = y
            final[bi, h] = fin
    return out, final
