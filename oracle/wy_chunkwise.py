"""Chunkwise (WY) forms of the gated delta rule, in float64 numpy.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).  The oracle
of record for prefill is the token-by-token recurrence in ``gdn_oracle.c``.
This module writes out the chunked algebra so that tests can pin it to that
recurrence by brute force on tiny shapes:

* ``page_chunk`` follows the pymllm ``gdn_chunkwise`` page, "Algorithm (per
  chunk of C tokens with initial state S_0)", steps 1-3, in that page's
  column notation: K, Q, W are Dk x C, U~ is Dv x C, the state S is Dv x Dk
  (the storage orientation [Dv, Dk]).  Two readings of the garbled step-1
  ``w`` recursion are available: ``printed_w=True`` takes the text literally
  (``w_i = b_i k_i - K_<i (W_<i^T (b_i k_i))``); the default swaps K and W
  (``w_i = b_i k_i - W_<i (K_<i^T (b_i k_i))``), which is what expanding the
  product of the factors (I - b_i k_i k_i^T) gives.  The ``u~`` recursion and
  gamma_i = prod_{j<=i} alpha_j (inclusive) are as printed.
* ``ratio_chunk`` is the same chunk rescaled so that no 1/gamma appears:
  A_ij = b_i exp(G_i - G_j) k_i.k_j (j < i), T = (I + A)^-1,
  Delta = T (diag(b) V - diag(b gamma) K S0^T), then
  O = diag(gamma) Q S0^T + (Gamma o tril(Q K^T)) Delta and
  S_C^T = gamma_C S0^T + (diag(exp(G_C - G)) K)^T Delta.
  Here rows are tokens (C x Dk, C x Dv) and S0 is Dv x Dk as stored.
"""
from __future__ import annotations

import numpy as np


def page_chunk(S0, Q, K, V, g, beta, printed_w=False):
    """One chunk by the page's WY steps.  S0 [Dv,Dk]; Q,K [C,Dk]; V [C,Dv];
    g (log-space) and beta [C].  Returns (O [C,Dv], S_new [Dv,Dk])."""
    S0 = np.asarray(S0, np.float64)
    Kc = np.asarray(K, np.float64).T          # Dk x C, column i is k_i
    Qc = np.asarray(Q, np.float64).T          # Dk x C
    Vc = np.asarray(V, np.float64).T          # Dv x C
    beta = np.asarray(beta, np.float64)
    C = Kc.shape[1]
    gamma = np.exp(np.cumsum(np.asarray(g, np.float64)))   # inclusive product of alphas
    W = np.zeros_like(Kc)
    U = np.zeros_like(Vc)
    for i in range(C):
        bk = beta[i] * Kc[:, i]
        if printed_w:
            W[:, i] = bk - Kc[:, :i] @ (W[:, :i].T @ bk)
        else:
            W[:, i] = bk - W[:, :i] @ (Kc[:, :i].T @ bk)
        U[:, i] = (beta[i] / gamma[i]) * Vc[:, i] - U[:, :i] @ (Kc[:, :i].T @ bk)
    M = np.triu(Kc.T @ Qc)                      # (i, r) = k_i . q_r for i <= r
    O = (S0 @ Qc - (S0 @ W) @ M + U @ M) * gamma[None, :]
    S_new = gamma[-1] * (S0 - (S0 @ W) @ Kc.T + U @ Kc.T)
    return O.T, S_new


def ratio_chunk(S0, Q, K, V, g, beta):
    """Division-free chunk form (see module doc).  Same arguments and results
    as ``page_chunk``."""
    S0 = np.asarray(S0, np.float64)
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    beta = np.asarray(beta, np.float64)
    C = K.shape[0]
    G = np.cumsum(np.asarray(g, np.float64))
    diff = G[:, None] - G[None, :]
    low = np.tril(np.ones((C, C), dtype=bool))
    Gam = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)   # exp(G_i - G_j), j <= i
    A = np.tril(beta[:, None] * Gam * (K @ K.T), -1)
    T = np.linalg.inv(np.eye(C) + A)
    gamma = np.exp(G)
    R = beta[:, None] * V - (beta * gamma)[:, None] * (K @ S0.T)
    Delta = T @ R
    O = gamma[:, None] * (Q @ S0.T) + (Gam * (Q @ K.T)) @ Delta
    decay_to_end = np.exp(G[-1] - G)
    S_new_T = gamma[-1] * S0.T + (decay_to_end[:, None] * K).T @ Delta
    return O, S_new_T.T


def chunked_head(S0, Q, K, V, g, beta, chunk, form="ratio", printed_w=False):
    """Run one head over T tokens in chunks of ``chunk`` (last one partial),
    carrying the state.  Returns (O [T,Dv], S_T [Dv,Dk])."""
    T = Q.shape[0]
    S = np.asarray(S0, np.float64).copy()
    outs = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        sl = slice(c0, c1)
        if form == "ratio":
            O, S = ratio_chunk(S, Q[sl], K[sl], V[sl], g[sl], beta[sl])
        else:
            O, S = page_chunk(S, Q[sl], K[sl], V[sl], g[sl], beta[sl], printed_w=printed_w)
        outs.append(O)
    O = np.concatenate(outs, axis=0) if outs else np.zeros((0, S.shape[0]))
    return O, S
