"""Chunked two-algorithm SSD forward in fp64 numpy (test infrastructure only).

This is the decomposition the aiwiki "State Space Duality" page describes in "Two
algorithms for one operator" and prints as a PyTorch sketch, and that llms.blog "State Space
Models and Mamba" lays out in "The Chunk-Wise SSD Algorithm" and the chunk pipeline figure:

  1. inside a chunk of Q tokens, the quadratic (attention) form with the decaying causal
     mask:  Y_intra = (L o (C B^T)) X,  L_ij = exp(cum_i - cum_j) for i >= j, else 0,
     where cum is the within-chunk running sum of log a;
  2. between chunks, one recurrent step on an N x P state:
     H_k = exp(cum_last) H_{k-1} + B^T (X o exp(cum_last - cum));
  3. the carried state enters each chunk's output:  Y += exp(cum_i) C_i H_{k-1};
  plus the skip D x.

Readings applied where the printed sketch is silent or wrong (each one follows the plain
recurrence h_t = a_t h_{t-1} + B_t x_t^T, y_t = C_t^T h_t + D x_t):
  * the carried-state term needs the decay from the chunk start to token i, exp(cum_i);
    the sketch and the pipeline figure omit it (they are only right for a = 1);
  * the state decay exp(cum_last) is one scalar per (batch, head) (the sketch's broadcast
    would mix batch entries);
  * the mask is selected (i >= j) before the exponential, so that the upper triangle,
    where cum_i - cum_j > 0, never produces inf (and inf * 0 = NaN);
  * the decay input is log a (the sketch takes cumsum and then exp of it);
  * a final chunk shorter than Q (T not a multiple of Q) is processed with its own length;
  * the per-state-dimension (diagonal) decay of "On Structured State-Space Duality" (ICML
    2026 poster, abstract item (i)) replaces the scalar mask by
    M_ij = sum_n C_in B_jn exp(cum_in - cum_jn) and the state decay by diag(exp(cum_last,n)).

No blocking beyond the chunk and no fusion: a reader can check each line against the steps.
"""
from __future__ import annotations

import numpy as np


def chunked_forward(x, log_a, Bm, Cm, D=None, init_state=None, chunk=64, return_states=False):
    """Chunked SSD forward.  Shapes as for ``oracle.forward``; all arithmetic in float64.

    Returns (y, final_state) or, with ``return_states``, (y, final_state, prev_states)
    where prev_states[b, h, k] is the state entering chunk k (H_{k-1}).
    """
    x = np.asarray(x, dtype=np.float64)
    log_a = np.asarray(log_a, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    Cm = np.asarray(Cm, dtype=np.float64)
    nb, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    diag = log_a.ndim == 4
    heads_per_group = H // G
    nchunks = -(-T // chunk) if T > 0 else 0
    y = np.zeros((nb, T, H, P))
    final = np.zeros((nb, H, N, P))
    prev_states = np.zeros((nb, H, nchunks, N, P))
    for b in range(nb):
        for h in range(H):
            g = h // heads_per_group
            state = np.zeros((N, P)) if init_state is None else np.array(init_state[b, h], dtype=np.float64)
            for k in range(nchunks):
                sl = slice(k * chunk, min((k + 1) * chunk, T))
                X = x[b, sl, h, :]            # [q, P]
                Bc = Bm[b, sl, g, :]          # [q, N]
                Cc = Cm[b, sl, g, :]          # [q, N]
                q = X.shape[0]
                causal = np.tril(np.ones((q, q), dtype=bool))
                prev_states[b, h, k] = state
                if not diag:
                    cum = np.cumsum(log_a[b, sl, h])                       # [q]
                    diff = np.where(causal, cum[:, None] - cum[None, :], 0.0)
                    L = np.where(causal, np.exp(diff), 0.0)                # [q, q]
                    scores = Cc @ Bc.T                                     # [q, q]
                    Y = (scores * L) @ X
                    Y += np.exp(cum)[:, None] * (Cc @ state)
                    decay_to_end = np.exp(cum[-1] - cum)                   # [q]
                    state = np.exp(cum[-1]) * state + Bc.T @ (X * decay_to_end[:, None])
                else:
                    cum = np.cumsum(log_a[b, sl, h, :], axis=0)            # [q, N]
                    diff = np.where(causal[:, :, None], cum[:, None, :] - cum[None, :, :], 0.0)
                    L = np.where(causal[:, :, None], np.exp(diff), 0.0)    # [q, q, N]
                    M = np.einsum("in,jn,ijn->ij", Cc, Bc, L)
                    Y = M @ X
                    Y += (Cc * np.exp(cum)) @ state
                    decay_to_end = np.exp(cum[-1][None, :] - cum)          # [q, N]
                    state = np.exp(cum[-1])[:, None] * state + (Bc * decay_to_end).T @ X
                if D is not None:
                    Y += D[h] * X
                y[b, sl, h, :] = Y
            final[b, h] = state
    if return_states:
        return y, final, prev_states
    return y, final
