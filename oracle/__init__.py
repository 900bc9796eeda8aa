"""fp64 CPU oracle for the Kimi Delta Attention (KDA) layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  It shares no code with
the GPU library: ``kda_oracle.c`` is a plain token-by-token recurrence in
double precision (see its header for the steps and the passages of the pages
each one follows) and ``chunked.py`` is the chunked (WY/UT) refactoring of the
same recurrence in NumPy, kept as an independent check of the recurrence.

``run`` is the entry point: it widens the inputs to float64 (exactly), calls
the C recurrence with OpenMP over (sequence, head) chains and returns float64
outputs, final states and checkpoints.

Parity status of the parts (the pins live in tests/test_oracle_pins.py):
  recurrence (decay, delta rule, readout)   pinned: closed forms + chunked form
  conv + SiLU, tap order, conv-state shift  pinned: unit-tap closed forms
  L2 norm, gated RMSNorm                    pinned: closed forms
  checkpoint positions and contents         pinned: brute-force split runs
  bf16 state storage (rounding, where)      pinned: library bf16 conversion,
                                            single rounding at the end, splits
  eps values, unit query scale, logistic output gate, conv tap orientation
  as a convention of the pages               parity unpinned (readings)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.kda_oracle_run.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_double,
            ctypes.c_int, P, P,
            P, P, P, P, P, P, P, P,
            P, P,
            ctypes.c_int64, P, P, P, ctypes.c_int,
            P, ctypes.c_int]
        lib.kda_oracle_run.restype = ctypes.c_int
        lib.kda_oracle_num_checkpoints.argtypes = [ctypes.c_int64] * 3
        lib.kda_oracle_num_checkpoints.restype = ctypes.c_int64
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        lib.kda_oracle_round_bf16.argtypes = [P, P, ctypes.c_int64]
        _lib = lib
    return _lib


def num_checkpoints(start: int, length: int, interval: int) -> int:
    return int(_load().kda_oracle_num_checkpoints(int(start), int(length), int(interval)))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def round_bf16(x) -> np.ndarray:
    """The oracle's rounding of values to the nearest bf16 value (ties to even)."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().kda_oracle_round_bf16(_ptr(x), _ptr(y), x.size)
    return y


@dataclass
class Result:
    out: np.ndarray        # [T][H][dv]
    S: np.ndarray          # [N][H][dk][dv] final states
    X: np.ndarray          # [N][H][2dk+dv][W-1] final conv states
    ckpt_S: np.ndarray     # [K][H][dk][dv]
    ckpt_X: np.ndarray     # [K][H][2dk+dv][W-1]
    ckpt_base: np.ndarray  # [N] first checkpoint slot of each sequence
    ckpt_pos: list         # absolute position of every checkpoint slot


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run(q, k, v, z, g, beta, conv_w, norm_w, cu_seqlens, *, start_pos=None,
        S0=None, X0=None, ckpt_interval: int = 0, l2_eps: float = 1e-6,
        rms_eps: float = 1e-6, threads: int = 0, state_round: bool = False) -> Result:
    """Run the recurrence over packed sequences.

    q, k, g: [T][H][dk]; v, z: [T][H][dv]; beta: [T][H]; conv_w: [H][2dk+dv][W];
    norm_w: [dv]; cu_seqlens: [N+1]; start_pos: [N] absolute position of each
    sequence's first token (default 0); S0: [N][H][dk][dv] and X0:
    [N][H][2dk+dv][W-1] initial states (default zero).  state_round: bf16 state
    storage, the state rounded to bf16 wherever it is stored (checkpoints and
    sequence ends).
    """
    q, k, v, z, g, beta = map(_f64, (q, k, v, z, g, beta))
    conv_w, norm_w = _f64(conv_w), _f64(norm_w)
    T, H, dk = q.shape
    dv = v.shape[2]
    W = conv_w.shape[2]
    C = 2 * dk + dv
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and z.shape == (T, H, dv) and beta.shape == (T, H)
    assert conv_w.shape == (H, C, W) and norm_w.shape == (dv,)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    sp = np.zeros(N, np.int64) if start_pos is None else np.ascontiguousarray(start_pos, dtype=np.int64)
    S = np.zeros((N, H, dk, dv)) if S0 is None else _f64(S0).copy()
    X = np.zeros((N, H, C, W - 1)) if X0 is None else _f64(X0).copy()
    assert S.shape == (N, H, dk, dv) and X.shape == (N, H, C, W - 1)
    counts = [num_checkpoints(sp[n], cu[n + 1] - cu[n], ckpt_interval) for n in range(N)]
    base = np.zeros(N, np.int64)
    if N:
        base[1:] = np.cumsum(counts)[:-1]
    K = int(sum(counts))
    cS = np.zeros((max(K, 1), H, dk, dv))
    cX = np.zeros((max(K, 1), H, C, W - 1))
    out = np.zeros((T, H, dv))
    rc = _load().kda_oracle_run(H, dk, dv, W, l2_eps, rms_eps, N, _ptr(cu), _ptr(sp),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(g), _ptr(beta),
                                _ptr(conv_w), _ptr(norm_w), _ptr(S), _ptr(X),
                                int(ckpt_interval), _ptr(base), _ptr(cS), _ptr(cX),
                                int(bool(state_round)), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_run failed with {rc}")
    pos = []
    for n in range(N):
        L = int(cu[n + 1] - cu[n])
        if ckpt_interval > 0 and L > 0:
            s0 = int(sp[n])
            for p in range(s0 + 1, s0 + L + 1):
                if p % ckpt_interval == 0 or p == s0 + L:
                    pos.append(p)
    return Result(out, S, X, cS[:K], cX[:K], base, pos)


def decode_steps(q, k, v, z, g, beta, conv_w, norm_w, S0, X0, *, l2_eps=1e-6,
                 rms_eps=1e-6, threads: int = 0, state_round: bool = False):
    """Run `steps` single-token decode steps for B sequences.

    q, k, g: [steps][B][H][dk]; v, z: [steps][B][H][dv]; beta: [steps][B][H];
    S0: [B][H][dk][dv]; X0: [B][H][2dk+dv][W-1].  Returns (out [steps][B][H][dv],
    S [B][H][dk][dv], X).  Each step is one call of the recurrence with every
    sequence one token long, carrying the state between calls (with
    state_round, rounded to bf16 after every step: the state is stored every
    step).
    """
    steps, B = q.shape[0], q.shape[1]
    S, X = _f64(S0), _f64(X0)
    outs = []
    cu = np.arange(B + 1, dtype=np.int64)
    for s in range(steps):
        r = run(q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, cu,
                S0=S, X0=X, l2_eps=l2_eps, rms_eps=rms_eps, threads=threads, state_round=state_round)
        S, X = r.S, r.X
        outs.append(r.out)
    return np.stack(outs), S, X
