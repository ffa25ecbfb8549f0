"""Independent fp64 derivation of the KDA forward in chunked (WY / UT) form.

TEST INFRASTRUCTURE: used only to cross-check the token recurrence in
kda_oracle.c (the two must agree to rounding), and as a readable statement of
the chunk algebra.  It shares nothing with the GPU library.

The pages (vLLM PR #55737's report, "Features and motivation") say the kernel
computes the same bounded-gate KDA recurrence as the Triton "chunk" path it
replaces; the chunked form below follows from unrolling

    S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = scale S_t^T q_t

over a block of C tokens.  With G_t = sum_{s<=t} log a_s (inclusive, per
channel, restarting at each chunk) and S the state entering the chunk, every
state inside the chunk is S_t = Diag(e^{G_t}) S + sum_{i<=t} (e^{G_t - G_i} * k_i) n_i^T
for pseudo-values n_i that solve a unit lower-triangular system:

    A[t, i] = b_t * sum_c k_t[c] k_i[c] e^{G_t[c] - G_i[c]}          (i < t)
    (I + A) N = diag(b) (V - (e^{G} * K) S)
    O = scale ((e^{G} * Q) S + Mq N),  Mq[t, i] = sum_c q_t[c] k_i[c] e^{G_t[c] - G_i[c]}  (i <= t)
    S_next = Diag(e^{G_last}) S + (e^{G_last - G} * K)^T N

Everything here is evaluated literally: pairwise exponentials e^{G_t - G_i}
(no factoring), and the triangular system solved by explicit forward
substitution, one row at a time.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def preprocess(q, k, g, beta_logits, A_log, dt_bias, lower_bound, h):
    """Per-token quantities for head h (float64 arrays over the token axis)."""
    qh = q[:, h, :]
    kh = k[:, h, :]
    qn = qh / np.sqrt((qh * qh).sum(-1, keepdims=True) + EPS)
    kn = kh / np.sqrt((kh * kh).sum(-1, keepdims=True) + EPS)
    beta = 1.0 / (1.0 + np.exp(-beta_logits[:, h]))
    x = np.exp(np.float64(A_log[h])) * (g[:, h, :] + dt_bias[h][None, :])
    lam = lower_bound / (1.0 + np.exp(-x))  # log of the per-channel decay
    return qn, kn, beta, lam


def forward_substitution(L, R):
    """Solve (I + L) X = R for X with L strictly lower triangular, row by row."""
    X = np.zeros_like(R)
    for t in range(R.shape[0]):
        X[t] = R[t] - L[t, :t] @ X[:t]
    return X


def chunk_step(S, qn, kn, v, beta, lam, scale):
    """Advance one chunk (C tokens, C = len(qn)).  Returns (O, S_next)."""
    C = qn.shape[0]
    G = np.cumsum(lam, axis=0)  # inclusive cumulative log-decay per channel
    # pairwise decays e^{G_t - G_i}, shape [t, i, c]; only i <= t is used
    dec = np.exp(G[:, None, :] - G[None, :, :])
    A = np.zeros((C, C))
    Mq = np.zeros((C, C))
    for t in range(C):
        for i in range(t + 1):
            if i < t:
                A[t, i] = beta[t] * np.sum(kn[t] * kn[i] * dec[t, i])
            Mq[t, i] = np.sum(qn[t] * kn[i] * dec[t, i])
    R = beta[:, None] * (v - (np.exp(G) * kn) @ S)
    Npv = forward_substitution(A, R)
    O = scale * ((np.exp(G) * qn) @ S + Mq @ Npv)
    S_next = np.exp(G[-1])[:, None] * S + (np.exp(G[-1][None, :] - G) * kn).T @ Npv
    return O, S_next


def kda_chunked_fwd(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale,
                    initial_state, cu_seqlens, chunk=64):
    """Same contract as oracle.kda_oracle_fwd, but all inputs already float64.

    q, k, v, g [T, H, D]; beta_logits [T, H]; A_log [H]; dt_bias [H, D];
    initial_state [N, H, D, D] float64 or None; cu_seqlens int [N + 1].
    """
    T, H, D = q.shape
    N = len(cu_seqlens) - 1
    out = np.zeros((T, H, D))
    fin = np.zeros((N, H, D, D))
    for h in range(H):
        qn, kn, beta, lam = preprocess(q, k, g, beta_logits, A_log, dt_bias, lower_bound, h)
        for n in range(N):
            S = np.zeros((D, D)) if initial_state is None else initial_state[n, h].copy()
            lo, hi = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
            for s0 in range(lo, hi, chunk):
                s1 = min(s0 + chunk, hi)
                O, S = chunk_step(S, qn[s0:s1], kn[s0:s1], v[s0:s1, h, :], beta[s0:s1],
                                  lam[s0:s1], scale)
                out[s0:s1, h, :] = O
            fin[n, h] = S
    return out, fin
