"""Python binding of libkda, the gfx950 KDA layer library (include/kda.h).

The functions here carry the C-ABI names and only marshal arguments: they
check that torch tensors have the expected device, dtype, shape and
contiguity, pass their device pointers and the current HIP stream to the
library, and raise KdaError when the library returns an error.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  If
libkda.so has not been built, importing this package works but every call
raises KdaLibraryMissing.

Build with ``python -m linear_attention_recurrence_decode_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_PREFILL_SPLIT = 1
KDA_PREFILL_PAIRED = 2
KDA_PREFILL_PAIRED_POLL_ONCE = 4
KDA_PREFILL_CONV_DONE = 8

# every symbol include/kda.h declares
EXPORTS = (
    "kda_decode_step", "kda_decode_multi", "kda_prefill_varlen", "kda_prefill_varlen_static",
    "kda_state_checkpoint", "kda_resume",
    "kda_project_inputs", "kda_project_inputs_conv", "kda_project_output", "kda_prefill_workspace_bytes",
    "kda_num_checkpoints", "kda_last_error",
    # host-side prefix cache (include/kda_prefix_cache.h)
    "kda_pcache_create", "kda_pcache_destroy", "kda_pcache_lookup", "kda_pcache_release",
    "kda_pcache_reserve", "kda_pcache_insert", "kda_pcache_insert_many", "kda_pcache_unreserve",
    "kda_pcache_commit",
    "kda_pcache_stats", "kda_pcache_last_error",
)
KDA_PCACHE_KEEP_ALL, KDA_PCACHE_SECOND_HIT = 0, 1


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kda status {status}: {message}")
        self.status = status


class KdaLibraryMissing(RuntimeError):
    pass


class _Config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_k", ctypes.c_int32),
                ("head_v", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("l2_eps", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("state_dtype", ctypes.c_int32)]


@dataclass
class Config:
    num_heads: int
    head_k: int
    head_v: int
    act_dtype: int = KDA_BF16
    conv_width: int = 4
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6
    state_dtype: int = KDA_F32

    @property
    def torch_act(self):
        return torch.bfloat16 if self.act_dtype == KDA_BF16 else torch.float32

    @property
    def torch_state(self):
        return torch.bfloat16 if self.state_dtype == KDA_BF16 else torch.float32

    @property
    def conv_channels(self):
        return 2 * self.head_k + self.head_v

    def c(self) -> _Config:
        return _Config(self.num_heads, self.head_k, self.head_v, self.conv_width,
                       self.act_dtype, self.l2_eps, self.rms_eps, self.state_dtype)


_lib = None


def lib():
    """The loaded libkda.so (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KdaLibraryMissing(f"{LIB_PATH} is not built; run "
                                "`python -m linear_attention_recurrence_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    CP = ctypes.POINTER(_Config)
    L.kda_decode_step.argtypes = [CP, I32] + [P] * 8 + [P, P, I32, P, P, P]
    L.kda_decode_multi.argtypes = [CP, I32, I32] + [P] * 8 + [P, P, I32, P, P, P, P, P]
    L.kda_project_inputs.argtypes = [CP, I32, I32] + [P] * 9
    L.kda_project_output.argtypes = [CP, I32, I32, P, P, P, P]
    L.kda_project_inputs_conv.argtypes = [CP, I32, I32, I32, P, P, P, P, P, I32, P] + [P] * 6 + [P]
    L.kda_prefill_varlen.argtypes = ([CP, I32, I64, P, P] + [P] * 8 + [P, P, I32, P, P, I32, P, P, I32, P,
                                     I32, P, P, ctypes.c_size_t, P])
    L.kda_prefill_varlen_static.argtypes = ([CP, I32, I64, P, P] + [P] * 8 + [P, P, I32, P, P, I32, P, P, I32, P,
                                            I32, P, P])
    L.kda_state_checkpoint.argtypes = [CP, I32, P, P, I32, P, P, P, I32, P, P]
    L.kda_resume.argtypes = [CP, I32, P, P, I32, P, P, P, I32, P, P]
    L.kda_prefill_workspace_bytes.argtypes = [CP, I32, I64, I32, I32]
    L.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.kda_num_checkpoints.argtypes = [I64, I64, I32]
    L.kda_num_checkpoints.restype = I64
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_pcache_create.argtypes = [I32, I32, I32, I32]
    L.kda_pcache_create.restype = P
    L.kda_pcache_destroy.argtypes = [P]
    L.kda_pcache_lookup.argtypes = [P, P, I64, P]
    L.kda_pcache_lookup.restype = I64
    L.kda_pcache_release.argtypes = [P, I32]
    L.kda_pcache_reserve.argtypes = [P, I32, P]
    L.kda_pcache_insert.argtypes = [P, P, I64, I32, I64]
    L.kda_pcache_insert_many.argtypes = [P, P, I32, P, P, I64, P]
    L.kda_pcache_unreserve.argtypes = [P, I32]
    L.kda_pcache_commit.argtypes = [P, I64]
    L.kda_pcache_stats.argtypes = [P, P, I32]
    L.kda_pcache_last_error.restype = ctypes.c_char_p
    for f in ("kda_pcache_release", "kda_pcache_reserve", "kda_pcache_insert", "kda_pcache_insert_many",
              "kda_pcache_unreserve"):
        getattr(L, f).restype = I32
    for f in ("kda_decode_step", "kda_decode_multi", "kda_prefill_varlen", "kda_prefill_varlen_static",
              "kda_state_checkpoint", "kda_resume", "kda_project_inputs", "kda_project_inputs_conv",
              "kda_project_output"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().kda_last_error().decode()


def _check(status: int):
    if status != KDA_OK:
        raise KdaError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t, name, dtype, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device's stream
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def kda_num_checkpoints(start: int, length: int, interval: int) -> int:
    return int(lib().kda_num_checkpoints(int(start), int(length), int(interval)))


def kda_prefill_workspace_bytes(cfg: Config, num_seqs: int, total_tokens: int, ckpt_interval: int = 0,
                                flags: int = 0) -> int:
    n = int(lib().kda_prefill_workspace_bytes(ctypes.byref(cfg.c()), int(num_seqs), int(total_tokens),
                                              int(ckpt_interval), int(flags)))
    if n == 0 and last_error():
        raise KdaError(KDA_ERR_INVALID_ARG, last_error())
    return n


def kda_decode_step(cfg: Config, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool,
                    slot, out, stream=None):
    """One fused decode step for B = slot.numel() sequences (see include/kda.h)."""
    B, H, dk, dv, C = slot.numel(), cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    act = cfg.torch_act
    S = state_pool.shape[0]
    _want(q, "q", act, (B, H, dk)); _want(k, "k", act, (B, H, dk))
    _want(v, "v", act, (B, H, dv)); _want(z, "z", act, (B, H, dv))
    _want(g, "g", torch.float32, (B, H, dk)); _want(beta, "beta", torch.float32, (B, H))
    _want(conv_w, "conv_w", torch.float32, (H, C, 4)); _want(norm_w, "norm_w", torch.float32, (dv,))
    _want(state_pool, "state_pool", cfg.torch_state, (S, H, dk, dv))
    _want(conv_pool, "conv_pool", act, (S, H, C, 3))
    _want(slot, "slot", torch.int32, (B,)); _want(out, "out", act, (B, H, dv))
    _check(lib().kda_decode_step(ctypes.byref(cfg.c()), B, _ptr(q), _ptr(k), _ptr(v), _ptr(z),
                                 _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(norm_w), _ptr(state_pool),
                                 _ptr(conv_pool), S, _ptr(slot), _ptr(out), _stream(stream)))
    return out


def kda_decode_multi(cfg: Config, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool,
                     slot, out, token_state=None, token_conv=None, stream=None):
    """T decode tokens per sequence in one launch (see include/kda.h)."""
    T, B = q.shape[0], slot.numel()
    H, dk, dv, C = cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    act = cfg.torch_act
    S = state_pool.shape[0]
    _want(q, "q", act, (T, B, H, dk)); _want(k, "k", act, (T, B, H, dk))
    _want(v, "v", act, (T, B, H, dv)); _want(z, "z", act, (T, B, H, dv))
    _want(g, "g", torch.float32, (T, B, H, dk)); _want(beta, "beta", torch.float32, (T, B, H))
    _want(conv_w, "conv_w", torch.float32, (H, C, 4)); _want(norm_w, "norm_w", torch.float32, (dv,))
    _want(state_pool, "state_pool", cfg.torch_state, (S, H, dk, dv))
    _want(conv_pool, "conv_pool", act, (S, H, C, 3))
    _want(slot, "slot", torch.int32, (B,)); _want(out, "out", act, (T, B, H, dv))
    if token_state is not None:
        _want(token_state, "token_state", cfg.torch_state, (B, T, H, dk, dv))
    if token_conv is not None:
        _want(token_conv, "token_conv", act, (B, T, H, C, 3))
    _check(lib().kda_decode_multi(ctypes.byref(cfg.c()), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(z),
                                  _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(norm_w), _ptr(state_pool),
                                  _ptr(conv_pool), S, _ptr(slot), _ptr(out), _ptr(token_state),
                                  _ptr(token_conv), _stream(stream)))
    return out


def projection_rows(cfg: Config) -> int:
    return cfg.num_heads * (3 * cfg.head_k + 2 * cfg.head_v) + cfg.num_heads


def kda_project_inputs(cfg: Config, x, w, q, k, v, z, g, beta, stream=None):
    """Input projections y = x W^T routed to q, k, v, z, g, beta (see include/kda.h)."""
    T, Dm = x.shape
    H, dk, dv = cfg.num_heads, cfg.head_k, cfg.head_v
    _want(x, "x", torch.bfloat16, (T, Dm)); _want(w, "w", torch.bfloat16, (projection_rows(cfg), Dm))
    _want(q, "q", torch.bfloat16, (T, H, dk)); _want(k, "k", torch.bfloat16, (T, H, dk))
    _want(v, "v", torch.bfloat16, (T, H, dv)); _want(z, "z", torch.bfloat16, (T, H, dv))
    _want(g, "g", torch.float32, (T, H, dk)); _want(beta, "beta", torch.float32, (T, H))
    _check(lib().kda_project_inputs(ctypes.byref(cfg.c()), T, Dm, _ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(z), _ptr(g), _ptr(beta), _stream(stream)))


def kda_project_inputs_conv(cfg: Config, cu_seqlens, x, w, conv_w, conv_pool, init_slot, q, k, v, z, g, beta,
                            stream=None):
    """Input projections with the causal conv fused (see include/kda.h): q, k
    [2][T][H][dk] and v [2][T][H][dv] bf16 receive the post-conv activations
    and then the raw projections; z, g, beta as kda_project_inputs."""
    T, Dm = x.shape
    N = cu_seqlens.numel() - 1
    H, dk, dv, C = cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    S = conv_pool.shape[0]
    _want(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _want(x, "x", torch.bfloat16, (T, Dm)); _want(w, "w", torch.bfloat16, (projection_rows(cfg), Dm))
    _want(conv_w, "conv_w", torch.float32, (H, C, 4)); _want(conv_pool, "conv_pool", torch.bfloat16, (S, H, C, 3))
    _want(init_slot, "init_slot", torch.int32, (N,))
    _want(q, "q", torch.bfloat16, (2, T, H, dk)); _want(k, "k", torch.bfloat16, (2, T, H, dk))
    _want(v, "v", torch.bfloat16, (2, T, H, dv)); _want(z, "z", torch.bfloat16, (T, H, dv))
    _want(g, "g", torch.float32, (T, H, dk)); _want(beta, "beta", torch.float32, (T, H))
    _check(lib().kda_project_inputs_conv(ctypes.byref(cfg.c()), N, T, Dm, _ptr(cu_seqlens), _ptr(x), _ptr(w),
                                         _ptr(conv_w), _ptr(conv_pool), S, _ptr(init_slot), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(z), _ptr(g), _ptr(beta), _stream(stream)))


def kda_project_output(cfg: Config, o, w_o, y, stream=None):
    """Output projection y = o W_o^T (see include/kda.h): o [T][H][dv] bf16,
    w_o [Dm][H dv] bf16, y [T][Dm] bf16."""
    T = o.shape[0]
    H, dv = cfg.num_heads, cfg.head_v
    Dm = w_o.shape[0]
    _want(o, "o", torch.bfloat16, (T, H, dv)); _want(w_o, "w_o", torch.bfloat16, (Dm, H * dv))
    _want(y, "y", torch.bfloat16, (T, Dm))
    _check(lib().kda_project_output(ctypes.byref(cfg.c()), T, Dm, _ptr(o), _ptr(w_o), _ptr(y), _stream(stream)))


STATIC_WORKSPACE_BYTES = 64 << 20      # KDA_STATIC_WORKSPACE_BYTES


def kda_prefill_varlen(cfg: Config, cu_seqlens, q, k, v, z, g, beta, conv_w, norm_w,
                       state_pool, conv_pool, init_slot, final_slot, out, workspace,
                       start_pos=None, ckpt_interval: int = 0, ckpt_state=None, ckpt_conv=None,
                       ckpt_base=None, flags: int = 0, stream=None):
    """Chunked varlen prefill (see include/kda.h)."""
    a = _prefill_args(cfg, cu_seqlens, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool,
                      init_slot, final_slot, out, start_pos, ckpt_interval, ckpt_state, ckpt_conv, ckpt_base,
                      conv_done=bool(int(flags) & KDA_PREFILL_CONV_DONE))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None:
        _want(workspace, "workspace", workspace.dtype)
    _check(lib().kda_prefill_varlen(*a, int(flags), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kda_prefill_varlen_static(cfg: Config, cu_seqlens, q, k, v, z, g, beta, conv_w, norm_w,
                              state_pool, conv_pool, init_slot, final_slot, out,
                              start_pos=None, ckpt_interval: int = 0, ckpt_state=None, ckpt_conv=None,
                              ckpt_base=None, flags: int = 0, stream=None):
    """kda_prefill_varlen with the library's static device workspace: allocates
    nothing (see include/kda.h)."""
    a = _prefill_args(cfg, cu_seqlens, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool,
                      init_slot, final_slot, out, start_pos, ckpt_interval, ckpt_state, ckpt_conv, ckpt_base,
                      conv_done=bool(int(flags) & KDA_PREFILL_CONV_DONE))
    _check(lib().kda_prefill_varlen_static(*a, int(flags), _ptr(out), _stream(stream)))
    return out


def _prefill_args(cfg, cu_seqlens, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool,
                  init_slot, final_slot, out, start_pos, ckpt_interval, ckpt_state, ckpt_conv, ckpt_base,
                  conv_done=False):
    """Checked leading arguments shared by the two prefill entry points, up to
    ckpt_base."""
    N = cu_seqlens.numel() - 1
    T = z.shape[0]
    H, dk, dv, C = cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    act = cfg.torch_act
    S = state_pool.shape[0]
    lead = (2, T) if conv_done else (T,)           # KDA_PREFILL_CONV_DONE: post-conv then raw
    _want(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _want(start_pos, "start_pos", torch.int64, (N,))
    _want(q, "q", act, lead + (H, dk)); _want(k, "k", act, lead + (H, dk))
    _want(v, "v", act, lead + (H, dv)); _want(z, "z", act, (T, H, dv))
    _want(g, "g", torch.float32, (T, H, dk)); _want(beta, "beta", torch.float32, (T, H))
    _want(conv_w, "conv_w", torch.float32, (H, C, 4)); _want(norm_w, "norm_w", torch.float32, (dv,))
    _want(state_pool, "state_pool", cfg.torch_state, (S, H, dk, dv))
    _want(conv_pool, "conv_pool", act, (S, H, C, 3))
    _want(init_slot, "init_slot", torch.int32, (N,)); _want(final_slot, "final_slot", torch.int32, (N,))
    _want(out, "out", act, (T, H, dv))
    nck = 0
    if ckpt_interval:
        nck = ckpt_state.shape[0]
        _want(ckpt_state, "ckpt_state", cfg.torch_state, (nck, H, dk, dv))
        _want(ckpt_conv, "ckpt_conv", act, (nck, H, C, 3))
        _want(ckpt_base, "ckpt_base", torch.int32, (N,))
    return (ctypes.byref(cfg.c()), N, T, _ptr(cu_seqlens), _ptr(start_pos),
            _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(g), _ptr(beta),
            _ptr(conv_w), _ptr(norm_w), _ptr(state_pool), _ptr(conv_pool), S,
            _ptr(init_slot), _ptr(final_slot), int(ckpt_interval),
            _ptr(ckpt_state), _ptr(ckpt_conv), nck, _ptr(ckpt_base))


def prefill_status(workspace) -> int:
    """The status word of the last kda_prefill_varlen call on this workspace
    (bytes 0..3, int32): waits between paired workgroups that gave up.  Read
    after the call has completed on its stream (this synchronises)."""
    return int(workspace[:4].view(torch.int32).item())


def _copy(fn, cfg, src_state, src_conv, src_idx, dst_state, dst_conv, dst_idx, stream):
    H, dk, dv, C = cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    act = cfg.torch_act
    n = src_idx.numel()
    for nm, t, shape in (("src_state", src_state, (src_state.shape[0], H, dk, dv)),
                         ("dst_state", dst_state, (dst_state.shape[0], H, dk, dv))):
        _want(t, nm, cfg.torch_state, shape)
    _want(src_conv, "src_conv", act, (src_state.shape[0], H, C, 3))
    _want(dst_conv, "dst_conv", act, (dst_state.shape[0], H, C, 3))
    _want(src_idx, "src ids", torch.int32, (n,)); _want(dst_idx, "dst ids", torch.int32, (n,))
    _check(fn(ctypes.byref(cfg.c()), n, _ptr(src_state), _ptr(src_conv), src_state.shape[0],
              _ptr(src_idx), _ptr(dst_state), _ptr(dst_conv), dst_state.shape[0], _ptr(dst_idx),
              _stream(stream)))


def kda_state_checkpoint(cfg: Config, state_pool, conv_pool, src_slot, ckpt_state, ckpt_conv,
                         dst_ckpt, stream=None):
    """ckpt[dst_ckpt[i]] = pool[src_slot[i]] (bitwise copy)."""
    _copy(lib().kda_state_checkpoint, cfg, state_pool, conv_pool, src_slot, ckpt_state,
          ckpt_conv, dst_ckpt, stream)


def kda_resume(cfg: Config, ckpt_state, ckpt_conv, src_ckpt, state_pool, conv_pool, dst_slot,
               stream=None):
    """pool[dst_slot[i]] = ckpt[src_ckpt[i]] (copy-on-write resume)."""
    _copy(lib().kda_resume, cfg, ckpt_state, ckpt_conv, src_ckpt, state_pool, conv_pool,
          dst_slot, stream)


class PrefixCache:
    """Host-side prefix cache of KDA states over the slots of a state pool
    (see include/kda_prefix_cache.h).  Token sequences are int32 arrays."""

    STATS = ("entries", "free_slots", "pinned_slots", "hits", "misses", "evictions", "declined", "first_sightings")

    def __init__(self, num_slots: int, unit: int, policy: int = KDA_PCACHE_KEEP_ALL, ghost_capacity: int = 0):
        self._h = lib().kda_pcache_create(int(num_slots), int(unit), int(policy), int(ghost_capacity))
        if not self._h:
            raise KdaError(KDA_ERR_INVALID_ARG, lib().kda_pcache_last_error().decode())

    def close(self):
        if self._h:
            lib().kda_pcache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _toks(tokens):
        import numpy as np
        return np.ascontiguousarray(tokens, dtype=np.int32)

    def _err(self, rc):
        if rc < 0:
            raise KdaError(KDA_ERR_INVALID_ARG, lib().kda_pcache_last_error().decode())
        return rc

    def lookup(self, tokens, max_len=None):
        """(p, slot) of the longest visible cached prefix of tokens with p <= max_len
        (default len(tokens)); (0, -1) on a miss.  A hit stays pinned until release()."""
        t = self._toks(tokens)
        n = len(t) if max_len is None else min(int(max_len), len(t))
        slot = ctypes.c_int32(-1)
        p = self._err(lib().kda_pcache_lookup(self._h, t.ctypes.data_as(ctypes.c_void_p), n, ctypes.byref(slot)))
        return int(p), int(slot.value)

    def release(self, slot: int):
        self._err(lib().kda_pcache_release(self._h, int(slot)))

    def reserve(self, n: int):
        import numpy as np
        out = np.zeros(max(int(n), 1), np.int32)
        self._err(lib().kda_pcache_reserve(self._h, int(n), out.ctypes.data_as(ctypes.c_void_p)))
        return out[:int(n)]

    def unreserve(self, slot: int):
        self._err(lib().kda_pcache_unreserve(self._h, int(slot)))

    def insert(self, tokens, pos: int, slot: int, step: int) -> bool:
        t = self._toks(tokens)
        assert 1 <= pos <= len(t)
        return bool(self._err(lib().kda_pcache_insert(self._h, t.ctypes.data_as(ctypes.c_void_p), int(pos), int(slot),
                                                      int(step))))

    def insert_many(self, tokens, positions, slots, step: int):
        """Register the states after tokens[0:p] for every p in positions (increasing)
        held in the reserved slots; returns a bool array (kept or declined)."""
        import numpy as np
        t = self._toks(tokens)
        pos = np.ascontiguousarray(positions, dtype=np.int64)
        sl = np.ascontiguousarray(slots, dtype=np.int32)
        assert len(pos) == len(sl) and (len(pos) == 0 or pos[-1] <= len(t))
        kept = np.zeros(max(len(pos), 1), np.int32)
        self._err(lib().kda_pcache_insert_many(self._h, t.ctypes.data_as(ctypes.c_void_p), len(pos),
                                               pos.ctypes.data_as(ctypes.c_void_p), sl.ctypes.data_as(ctypes.c_void_p),
                                               int(step), kept.ctypes.data_as(ctypes.c_void_p)))
        return kept[:len(pos)].astype(bool)

    def commit(self, step: int):
        lib().kda_pcache_commit(self._h, int(step))

    def stats(self) -> dict:
        import numpy as np
        out = np.zeros(8, np.int64)
        lib().kda_pcache_stats(self._h, out.ctypes.data_as(ctypes.c_void_p), 8)
        return dict(zip(self.STATS, (int(x) for x in out)))
