"""fp64 chunk (WY / UT) form of the gated delta rule replay.

TEST INFRASTRUCTURE ONLY. It pins, against the token-by-token recurrence, the
algebra a chunked kernel can use to replay a block of T tokens at once. It is
written from the derivation below, not from any kernel.

Derivation (per value head; S is d_v x d_k, tokens t = 1..T from S_0)
--------------------------------------------------------------------
The gated delta rule (Yang et al., "Gated Delta Networks", 2025) in rank-1
form is S_t = alpha_t S_{t-1} + w_t k_t^T with
    w_t = beta_t (v_t - alpha_t S_{t-1} k_t).
With gamma_t = alpha_1 ... alpha_t (gamma_0 = 1) this unrolls to
    S_t = gamma_t S_0 + sum_{i<=t} (gamma_t / gamma_i) w_i k_i^T.
Substituting S_{t-1} into w_t:
    w_t + beta_t sum_{i<t} (gamma_t / gamma_i) (k_t . k_i) w_i
        = beta_t (v_t - gamma_t S_0 k_t),
i.e. (I + A) W = X with the strictly lower-triangular
    A_ti = beta_t (gamma_t / gamma_i) (k_t . k_i),  i < t,
    X_t  = beta_t (v_t - gamma_t Y_t),  Y_t = S_0 k_t.
Then
    S_T = gamma_T S_0 + sum_i (gamma_T / gamma_i) w_i k_i^T
    o_t = S_t q_t = gamma_t S_0 q_t + sum_{i<=t} (gamma_t / gamma_i) (k_i . q_t) w_i.
The only contractions with the state are Y = K S_0^T and Z = Q S_0^T; the rest
works on T x T matrices and T x d_v blocks. The ratios gamma_t / gamma_i are
formed here as direct products of the alphas between i and t.
"""
from __future__ import annotations

import numpy as np


def _decay_ratio(alpha: np.ndarray) -> np.ndarray:
    """L[t, i] = prod_{s=i+1..t} alpha_s for i <= t (1 on the diagonal), else 0."""
    T = alpha.shape[0]
    L = np.zeros((T, T))
    for t in range(T):
        L[t, t] = 1.0
        for i in range(t - 1, -1, -1):
            L[t, i] = L[t, i + 1] * alpha[i + 1]
    return L


def chunk_replay(S0, K, V, alpha, beta, Q=None):
    """Replay T tokens from S0 in chunk form.

    S0 [dv, dk]; K [T, dk]; V [T, dv]; alpha, beta [T]; Q [T, dk] or None.
    Returns (S_T, W, O) where O [T, dv] are the outputs S_t q_t (or None)."""
    T = K.shape[0]
    L = _decay_ratio(alpha)                      # gamma_t / gamma_i
    gamma = np.cumprod(alpha)                    # gamma_t (1-based t -> index t-1)
    G = K @ K.T
    A = np.tril(beta[:, None] * L * G, -1)
    Y = K @ S0.T                                 # [T, dv], Y_t = S0 k_t
    X = beta[:, None] * (V - gamma[:, None] * Y)
    W = np.linalg.solve(np.eye(T) + A, X)        # unit lower-triangular system
    S_T = gamma[-1] * S0 + (L[-1][:, None] * W).T @ K
    O = None
    if Q is not None:
        Z = Q @ S0.T                             # [T, dv]
        P = np.tril(L * (Q @ K.T))               # (gamma_t/gamma_i)(q_t . k_i), i <= t
        O = gamma[:, None] * Z + P @ W
    return S_T, W, O


def chunk_replay_subchunks(S0, K, V, alpha, beta, Q, chunk: int):
    """Same replay cut into sub-chunks of `chunk` tokens, with the state carried
    between them; returns (S_T, O)."""
    T = K.shape[0]
    S = S0
    outs = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        S, _, O = chunk_replay(S, K[c0:c1], V[c0:c1], alpha[c0:c1], beta[c0:c1], Q[c0:c1])
        outs.append(O)
    return S, np.concatenate(outs, axis=0)
