"""Chunked (WY / UT-transform) form of the KDA recurrence in fp64 NumPy.

TEST INFRASTRUCTURE ONLY.  This is the chunk-parallel refactoring of the gated
delta rule with per-channel decay, written from its algebra, and is used only
to pin the token-by-token oracle: on small inputs both must agree to rounding.

For a chunk of n tokens entered with state S (dk x dv), with
  Gam[t]   = g[0] + ... + g[t]                    (per key channel)
  M[t, s]  = sum_i k[t,i] k[s,i] exp(Gam[t,i] - Gam[s,i])   s <  t
  P[t, s]  = sum_i q[t,i] k[s,i] exp(Gam[t,i] - Gam[s,i])   s <= t
  T        = (I + Diag(beta) M)^{-1} Diag(beta)
the per-token updates u_t of the delta rule solve
  U = T (V - (k * exp(Gam)) S),
the outputs are O = (q * exp(Gam)) S + P U, and the chunk leaves the state
  exp(Gam[n-1]) * S + (k * exp(Gam[n-1] - Gam))^T U.
The pairwise exponentials are evaluated directly (no reference-point
factorisation), which is slow but has no range limit.

The preprocessing (causal conv + SiLU, L2 norm) and the gated RMSNorm are the
same per-token maps as in the oracle; they are written out again here so that
this module does not depend on the C oracle.
"""
from __future__ import annotations

import numpy as np


def _silu(y):
    return y / (1.0 + np.exp(-y))


def _sigmoid(y):
    return 1.0 / (1.0 + np.exp(-y))


def preprocess(xq, xk, xv, conv_w, X0, l2_eps):
    """Conv + SiLU + L2 norm for one sequence and one head.

    xq, xk: [L][dk]; xv: [L][dv]; conv_w: [C][W]; X0: [C][W-1] (oldest first).
    Returns q_hat, k_hat, v_hat and the final conv state.
    """
    L = xq.shape[0]
    dk = xq.shape[1]
    x = np.concatenate([xq, xk, xv], axis=1)           # [L][C]
    W = conv_w.shape[1]
    full = np.concatenate([X0.T, x], axis=0)            # [W-1+L][C]
    y = np.zeros_like(x)
    for m in range(W):
        # tap m multiplies the input m-(W-1) tokens back
        y += conv_w[:, m][None, :] * full[m:m + L]
    a = _silu(y)
    aq, ak, av = a[:, :dk], a[:, dk:2 * dk], a[:, 2 * dk:]
    qh = aq / np.sqrt((aq * aq).sum(1, keepdims=True) + l2_eps)
    kh = ak / np.sqrt((ak * ak).sum(1, keepdims=True) + l2_eps)
    Xn = full[L:].T.copy() if W > 1 else X0.copy()
    return qh, kh, av, Xn


def chunk_step(S, qh, kh, vh, g, beta):
    """Advance state S over one chunk; return (O, S_next)."""
    n, dk = kh.shape
    Gam = np.cumsum(g, axis=0)                           # [n][dk]
    D = Gam[:, None, :] - Gam[None, :, :]               # [t][s][i]
    tri_strict = np.tril(np.ones((n, n)), -1)
    tri = np.tril(np.ones((n, n)))
    # entries above the diagonal have D > 0 and are masked before use
    E = np.exp(np.where(tri[:, :, None] > 0, D, 0.0))
    M = np.einsum("ti,si,tsi->ts", kh, kh, E) * tri_strict
    P = np.einsum("ti,si,tsi->ts", qh, kh, E) * tri
    A = np.eye(n) + beta[:, None] * M
    T = np.linalg.solve(A, np.diag(beta))
    Kg = kh * np.exp(Gam)
    Qg = qh * np.exp(Gam)
    U = T @ (vh - Kg @ S)
    O = Qg @ S + P @ U
    last = Gam[n - 1]
    Kc = kh * np.exp(last[None, :] - Gam)
    S_next = np.exp(last)[:, None] * S + Kc.T @ U
    return O, S_next


def run_sequence(xq, xk, xv, z, g, beta, conv_w, norm_w, S0, X0, *, chunk=64,
                 start_pos=0, l2_eps=1e-6, rms_eps=1e-6):
    """One sequence, one head.  Chunks are aligned to absolute multiples of
    `chunk` counted from position 0, so a sequence that starts at an unaligned
    start_pos begins with a short chunk.  Returns (y [L][dv], S, X)."""
    L = xq.shape[0]
    qh, kh, vh, X = preprocess(xq, xk, xv, conv_w, X0, l2_eps)
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((L, vh.shape[1]))
    t = 0
    while t < L:
        pos = start_pos + t
        n = min(L - t, chunk - (pos % chunk))
        sl = slice(t, t + n)
        O[sl], S = chunk_step(S, qh[sl], kh[sl], vh[sl], g[sl], beta[sl])
        t += n
    ms = (O * O).mean(1, keepdims=True)
    y = O / np.sqrt(ms + rms_eps) * norm_w[None, :] * _sigmoid(z)
    return y, S, X
