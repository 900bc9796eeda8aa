"""Input projections of the KDA layer in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check and the CPU-baseline leg of
bench.py may use it; the GPU library never does).

The layer's per-token inputs come from one hidden vector x (model width Dm)
through linear maps: q, k (H x dk), v, z (H x dv), the decay gate's
pre-activation (H x dk) and beta's pre-activation (H), with
  g    = -softplus(pre_g)      (log decay, <= 0)
  beta = sigmoid(pre_beta)
[vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
 "KDA prefill and decode": the input projections and the causal convolution
 are fused around the recurrence.  The pages give neither the model width nor
 the gate parameterisation; a linear pre-activation followed by -softplus and
 the logistic function is the plainest reading that yields a log decay <= 0
 and a beta in (0, 1), and matches the workloads' synthetic distributions.]

The output projection maps the layer's gated, normalised output o (H x dv
per token) back to the model width: y = o W_o^T with W_o [Dm][H dv].  [The
pages name no output projection; a linear map back to the model width is
the plainest reading of a layer that sits in the model's residual stream.]

Packed weight layout (one row per output channel, Dm contiguous):
  rows [0, H dk)              q      rows [H dk, 2 H dk)            k
  rows [2 H dk, 2 H dk + H dv) v     then H dv rows of z, H dk rows of the
  gate pre-activation and H rows of beta's pre-activation:
  N = H (3 dk + 2 dv) + H rows in all.
"""
from __future__ import annotations

import numpy as np


def rows(H: int, dk: int, dv: int) -> int:
    return H * (3 * dk + 2 * dv) + H


def softplus(x):
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """The logistic function 1 / (1 + e^-x), written with e = e^-|x| so that
    no exponential overflows and small values keep their relative precision."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def project(x, w, H: int, dk: int, dv: int):
    """x [T][Dm], w [N][Dm] -> dict of q, k [T][H][dk], v, z [T][H][dv],
    g [T][H][dk], beta [T][H] in fp64 (the matmul is NumPy's, in fp64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T = x.shape[0]
    assert w.shape == (rows(H, dk, dv), x.shape[1])
    y = x @ w.T
    o = 0
    out = {}
    for name, width in (("q", dk), ("k", dk), ("v", dv), ("z", dv), ("g", dk)):
        out[name] = y[:, o:o + H * width].reshape(T, H, width)
        o += H * width
    out["g"] = -softplus(out["g"])
    out["beta"] = sigmoid(y[:, o:o + H])
    return out


def output(o, w_o):
    """o [T][H][dv] (or [T][H dv]), w_o [Dm][H dv] -> y [T][Dm] = o W_o^T in
    fp64 (the matmul is NumPy's, in fp64)."""
    o = np.asarray(o, np.float64)
    o = o.reshape(o.shape[0], -1)
    w = np.asarray(w_o, np.float64)
    assert w.shape[1] == o.shape[1]
    return o @ w.T
