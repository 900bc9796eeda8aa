"""Seeded synthetic inputs for the Kimi Delta Attention (KDA) layer.

This module is shared by the oracle's tests, the GPU parity tests and
``bench.py``. It holds random draws and nothing of the method's arithmetic:
the input distributions are the ones the workloads define (q, k, v, z ~ N(0,1),
g = -softplus(N(0,1)) per key channel, beta = sigmoid(N(0,1)) per head),
followed by round-to-nearest-even to the activation dtype where the workload
asks for bf16 inputs.

Every token-indexed tensor is drawn in blocks of ``BLOCK_TOKENS`` tokens with
``numpy.random.default_rng([seed, tensor_id, block])``, so a tensor's values do
not depend on how many blocks are generated at once or in which order.

Arrays come back as numpy float32 (bf16 activations are float32 arrays whose
values are exactly representable in bf16), int32 or int64. Layouts:
  q, k, g   [T][H][dk]        v, z   [T][H][dv]        beta [T][H]
  conv_w    [H][2*dk+dv][W]   (per head: q channels, then k, then v)
  norm_w    [dv]
  state     [S][H][dk][dv]    conv_state [S][H][2*dk+dv][W-1] (index 0 = oldest)
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_TOKENS = 4096

# Tensor ids for the seed sequence; fixed forever so stored inputs stay valid.
TID = {
    "q": 1, "k": 2, "v": 3, "z": 4, "g": 5, "beta": 6,
    "conv_w": 7, "norm_w": 8, "state": 9, "conv_state": 10,
    "lengths": 11, "slots": 12, "resume": 13, "hidden": 14, "proj_w": 15,
    "layer_out": 16, "out_proj_w": 17,
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bf16 (ties to even); return
    float32.  Works in place on a float32 array (a copy of anything else)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> 16) & 1
    b += np.uint32(0x7FFF)
    b += lsb
    b &= np.uint32(0xFFFF0000)
    return x


def _softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + exp(x)) in float32, as max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float32)
    return (np.maximum(x, np.float32(0.0)) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw_tokens(seed: int, tid: int, T: int, inner: tuple, std: float = 1.0,
                transform=None) -> np.ndarray:
    """Draw a [T, *inner] float32 tensor block by block (see module docstring);
    `transform`, if given, maps each drawn block (in the worker threads)."""
    out = np.empty((T,) + tuple(inner), dtype=np.float32)
    nblk = (T + BLOCK_TOKENS - 1) // BLOCK_TOKENS

    def one(b):
        lo, hi = b * BLOCK_TOKENS, min(T, (b + 1) * BLOCK_TOKENS)
        rng = np.random.default_rng([seed, tid, b])
        blk = rng.standard_normal((hi - lo,) + tuple(inner), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if transform is not None:
            blk = transform(blk)
        out[lo:hi] = blk

    if nblk <= 1:
        for b in range(nblk):
            one(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nblk)))
    return out


def draw_plain(seed: int, tid: int, shape: tuple, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, 0])
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclass
class LayerShape:
    """Head geometry of one KDA layer on one GPU."""
    H: int
    dk: int
    dv: int
    W: int = 4
    act: str = "bf16"            # dtype of q, k, v, z, out and the conv state

    @property
    def C(self) -> int:          # conv channels per head
        return 2 * self.dk + self.dv


@dataclass
class Inputs:
    shape: LayerShape
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    conv_w: np.ndarray
    norm_w: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.q.shape[0]


def token_inputs(seed: int, shape: LayerShape, T: int, *, g_scale: float = 1.0,
                 norm_w: str = "ones", conv_w_std: float = 0.5) -> Inputs:
    """Per-token activations and gates for T tokens, plus conv and norm weights.

    g_scale multiplies the drawn log-decay (1.0 is the workloads' gate; small
    values give the weak-decay stress inputs, 0.0 gives the pure delta rule).
    norm_w is "ones" (the workloads' RMSNorm weight) or "random" (a positive
    non-unit weight that exposes indexing mistakes).
    """
    H, dk, dv = shape.H, shape.dk, shape.dv
    rnd = round_bf16 if shape.act == "bf16" else None
    q = draw_tokens(seed, TID["q"], T, (H, dk), transform=rnd)
    k = draw_tokens(seed, TID["k"], T, (H, dk), transform=rnd)
    v = draw_tokens(seed, TID["v"], T, (H, dv), transform=rnd)
    z = draw_tokens(seed, TID["z"], T, (H, dv), transform=rnd)
    gs = np.float32(g_scale)
    g = draw_tokens(seed, TID["g"], T, (H, dk),
                    transform=lambda a: (-_softplus(a) * gs).astype(np.float32) if g_scale != 1.0
                    else -_softplus(a))
    beta = draw_tokens(seed, TID["beta"], T, (H,), transform=_sigmoid)
    conv_w = draw_plain(seed, TID["conv_w"], (H, shape.C, shape.W), std=conv_w_std)
    if norm_w == "ones":
        nw = np.ones((dv,), np.float32)
    else:
        nw = (0.5 + np.abs(draw_plain(seed, TID["norm_w"], (dv,)))).astype(np.float32)
    return Inputs(shape, q, k, v, z, g, beta, conv_w, nw)


def token_rows(seed: int, shape: LayerShape, rows, *, g_scale: float = 1.0, norm_w: str = "ones",
               conv_w_std: float = 0.5) -> Inputs:
    """The inputs token_inputs(seed, shape, T, ...) holds at the packed token
    indices `rows` (any T beyond max(rows)), drawing only the blocks that
    contain them: each block is its own seeded stream and a shorter draw from
    a stream gives its first values, so the rows are the same values."""
    rows = np.asarray(rows, np.int64)
    H, dk, dv = shape.H, shape.dk, shape.dv
    rnd = round_bf16 if shape.act == "bf16" else None
    gs = np.float32(g_scale)
    specs = {"q": ((H, dk), rnd), "k": ((H, dk), rnd), "v": ((H, dv), rnd), "z": ((H, dv), rnd),
             "g": ((H, dk), (lambda a: (-_softplus(a) * gs).astype(np.float32)) if g_scale != 1.0
                   else (lambda a: -_softplus(a))),
             "beta": ((H,), _sigmoid)}
    blocks = rows // BLOCK_TOKENS
    out = {}
    for name, (inner, tf) in specs.items():
        arr = np.empty((len(rows),) + inner, np.float32)
        for b in np.unique(blocks):
            sel = np.nonzero(blocks == b)[0]
            lo = int(b) * BLOCK_TOKENS
            n = int(rows[sel].max()) - lo + 1
            rng = np.random.default_rng([seed, TID[name], int(b)])
            blk = rng.standard_normal((n,) + inner, dtype=np.float32)
            if tf is not None:
                blk = tf(blk)
            arr[sel] = blk[rows[sel] - lo]
        out[name] = arr
    conv_w = draw_plain(seed, TID["conv_w"], (H, shape.C, shape.W), std=conv_w_std)
    if norm_w == "ones":
        nw = np.ones((dv,), np.float32)
    else:
        nw = (0.5 + np.abs(draw_plain(seed, TID["norm_w"], (dv,)))).astype(np.float32)
    return Inputs(shape, out["q"], out["k"], out["v"], out["z"], out["g"], out["beta"], conv_w, nw)


def states(seed: int, shape: LayerShape, nslots: int, state_std: float = 0.02,
           conv_std: float = 1.0):
    """Random recurrent state (fp32) and conv state (activation dtype) pools."""
    S = draw_plain(seed, TID["state"], (nslots, shape.H, shape.dk, shape.dv), std=state_std)
    X = draw_plain(seed, TID["conv_state"], (nslots, shape.H, shape.C, shape.W - 1), std=conv_std)
    if shape.act == "bf16":
        X = round_bf16(X)
    return S, X


def loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n lengths floor(exp(U(ln lo, ln hi))) (the varlen workload's length mix)."""
    rng = np.random.default_rng([seed, TID["lengths"], 0])
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.floor(np.exp(u)).astype(np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu


def slot_permutation(seed: int, nslots: int, n: int) -> np.ndarray:
    """n distinct slot ids drawn from a pool of nslots."""
    rng = np.random.default_rng([seed, TID["slots"], 0])
    return rng.permutation(nslots)[:n].astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads (tiny recurrent, batched decode, chunked prefill, varlen
# prefill with checkpoints, long context).  Each returns a plain description;
# the inputs themselves come from the functions above.
# ---------------------------------------------------------------------------

WORKLOADS = {
    "tiny_f32": dict(seed=0, shape=LayerShape(H=2, dk=32, dv=32, act="f32"), B=1, T=64),
    "decode_b64": dict(seed=1, shape=LayerShape(H=32, dk=128, dv=128, act="bf16"),
                       B=64, steps=256, pool=80, state_std=0.02, conv_std=1.0),
    "prefill_4x8k": dict(seed=2, shape=LayerShape(H=32, dk=128, dv=128, act="bf16"),
                         lengths=[8192] * 4),
    # seed 6: the first seed from 3 on whose 16 lengths total within 1% of the
    # workload's 256Ki tokens (262,990 tokens, longest 51,782); seed 3 drew
    # 165,069 tokens with none above 29,637
    "varlen_ckpt": dict(seed=6, shape=LayerShape(H=32, dk=128, dv=128, act="bf16"),
                        n=16, lo=1024, hi=65536, interval=4096),
    "long_1m": dict(seed=4, shape=LayerShape(H=8, dk=128, dv=128, act="bf16"),
                    lengths=[1 << 20], interval=32768, decode_B=256, decode_steps=512),
    # input projections of the 4 x 8192 prefill: model width 7168 is a synthetic
    # choice (the pages give none)
    "project_4x8k": dict(seed=5, shape=LayerShape(H=32, dk=128, dv=128, act="bf16"), T=32768, Dm=7168),
}


def projection_inputs(seed: int, shape: LayerShape, T: int, Dm: int):
    """Hidden states x ~ N(0, 1) [T][Dm] and packed projection weights
    W ~ N(0, 1/Dm) [N][Dm] (so every pre-activation is about N(0, 1), as the
    token inputs of token_inputs are), both rounded to bf16 and held as
    float32.  N = H (3 dk + 2 dv) + H."""
    N = shape.H * (3 * shape.dk + 2 * shape.dv) + shape.H
    x = draw_tokens(seed, TID["hidden"], T, (Dm,), transform=round_bf16)
    w = draw_tokens(seed, TID["proj_w"], N, (Dm,), std=float(Dm) ** -0.5, transform=round_bf16)
    return x, w


def output_projection_inputs(seed: int, shape: LayerShape, T: int, Dm: int):
    """The layer's output o ~ N(0, 1) [T][H][dv] (the scale of a gated RMSNorm
    output with unit weight) and output-projection weights W_o ~ N(0, 1/(H dv))
    [Dm][H dv], both rounded to bf16 and held as float32."""
    K = shape.H * shape.dv
    o = draw_tokens(seed, TID["layer_out"], T, (shape.H, shape.dv), transform=round_bf16)
    w = draw_tokens(seed, TID["out_proj_w"], Dm, (K,), std=float(K) ** -0.5, transform=round_bf16)
    return o, w
