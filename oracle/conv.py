"""The KDA layer's short causal convolution and SiLU in fp64 NumPy, over
packed sequences, on its own: the activations a fused front end (input
projections with the conv in their epilogue) hands to the recurrence.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check and the CPU-baseline leg of
bench.py may use it; the GPU library never does).

[vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
 "KDA prefill and decode": a short causal convolution on q, k and v is fused
 in front of the recurrence; section "The Hardest Part: Prefix Caching for
 KDA": its state (the last raw inputs) lives beside the recurrent state.]

For channel c of a head and token t of a sequence (window oldest first):
  y[t][c] = w[c][0] x[t-3][c] + w[c][1] x[t-2][c] + w[c][2] x[t-1][c] + w[c][3] x[t][c]
  a[t][c] = y / (1 + exp(-y))                                        (SiLU)
where rows before the sequence's first token come from its initial conv
state X0[c][m], m = 0 the token three before the start and m = 2 the one just
before (zero when there is none).  These are the conventions of the
recurrence oracle (kda_oracle.c), whose conv state holds raw inputs; the
pages fix none of them (parity unpinned as the pages' convention, pinned
here by closed forms in tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np


def preactivation(x, conv_w, cu_seqlens, X0=None):
    """x [T][H][C] raw channels (q | k | v per head), conv_w [H][C][4],
    cu_seqlens [N+1], X0 [N][H][C][3] or None -> y [T][H][C] in fp64."""
    x = np.asarray(x, np.float64)
    w = np.asarray(conv_w, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, H, C = x.shape
    assert w.shape == (H, C, 4) and cu[0] == 0 and cu[-1] == T
    y = np.zeros((T, H, C))
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        x0 = np.zeros((H, C, 3)) if X0 is None else np.asarray(X0[n], np.float64)
        # the sequence's rows with its left context in front: [3 + L][H][C]
        ext = np.concatenate([np.transpose(x0, (2, 0, 1)), x[a:b]], axis=0)
        for t in range(b - a):
            for m in range(4):
                y[a + t] += w[:, :, m] * ext[t + m]
    return y


def silu(y):
    y = np.asarray(y, np.float64)
    return y / (1.0 + np.exp(-y))


def activations(q, k, v, conv_w, cu_seqlens, X0=None):
    """SiLU(conv) of q [T][H][dk], k [T][H][dk], v [T][H][dv] with the layer's
    channel order (per head: q, then k, then v) -> (a_q, a_k, a_v) in fp64."""
    dk = np.asarray(q).shape[2]
    x = np.concatenate([np.asarray(q, np.float64), np.asarray(k, np.float64), np.asarray(v, np.float64)], axis=2)
    a = silu(preactivation(x, conv_w, cu_seqlens, X0))
    return a[:, :, :dk], a[:, :, dk:2 * dk], a[:, :, 2 * dk:]
