"""C-ABI checks that need no GPU: libkda.so loads, exports every symbol that
include/kda.h declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes.  Fake, aligned, non-NULL addresses
stand in for device pointers: every call here fails validation or is a no-op,
so nothing is dereferenced or launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_recurrence_decode_amd as kda
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("kda.h", "kda_prefix_cache.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH), reason="libkda.so not built")

FAKE = 0x10000          # 16-byte aligned stand-in for a device address
MISALIGNED = 0x10008


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(kda.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def cfg(**kw):
    base = dict(num_heads=4, head_k=128, head_v=128, act_dtype=kda.KDA_BF16)
    base.update(kw)
    return kda.Config(**base)


def decode_call(c, B=2, num_slots=8, **ptrs):
    P = {n: FAKE for n in ("q", "k", "v", "z", "g", "beta", "conv_w", "norm_w", "state", "conv",
                           "slot", "out")}
    P.update(ptrs)
    cp = ctypes.byref(c.c()) if c is not None else None
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.lib().kda_decode_step(cp, B, vp(P["q"]), vp(P["k"]), vp(P["v"]), vp(P["z"]),
                                     vp(P["g"]), vp(P["beta"]), vp(P["conv_w"]), vp(P["norm_w"]),
                                     vp(P["state"]), vp(P["conv"]), num_slots, vp(P["slot"]),
                                     vp(P["out"]), None)


def test_decode_validation():
    assert decode_call(None) == kda.KDA_ERR_INVALID_ARG
    assert "cfg" in kda.last_error()
    assert decode_call(cfg(head_k=96, head_v=96)) == kda.KDA_ERR_UNSUPPORTED
    assert decode_call(cfg(head_k=128, head_v=64)) == kda.KDA_ERR_UNSUPPORTED
    assert decode_call(cfg(conv_width=3)) == kda.KDA_ERR_UNSUPPORTED
    assert decode_call(cfg(act_dtype=7)) == kda.KDA_ERR_INVALID_ARG
    assert decode_call(cfg(num_heads=0)) == kda.KDA_ERR_INVALID_ARG
    assert decode_call(cfg(state_dtype=2)) == kda.KDA_ERR_INVALID_ARG
    assert "state_dtype" in kda.last_error()
    assert decode_call(cfg(l2_eps=float("nan"))) == kda.KDA_ERR_INVALID_ARG
    assert decode_call(cfg(), B=-1) == kda.KDA_ERR_INVALID_ARG
    assert decode_call(cfg(), num_slots=0) == kda.KDA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "z", "g", "beta", "conv_w", "norm_w", "state", "conv", "slot", "out"):
        assert decode_call(cfg(), **{name: None}) == kda.KDA_ERR_INVALID_ARG, name
    assert decode_call(cfg(), q=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert "aligned" in kda.last_error()
    assert decode_call(cfg(), B=1 << 30) == kda.KDA_ERR_INVALID_ARG      # grid overflow
    # B == 0 is a no-op that touches no pointer
    assert decode_call(cfg(), B=0, q=None) == kda.KDA_OK
    assert kda.last_error() == ""


def copy_call(fn, c, n=3, src_slots=4, dst_slots=4, **ptrs):
    P = {n_: FAKE for n_ in ("ss", "sc", "si", "ds", "dc", "di")}
    P.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return fn(ctypes.byref(c.c()), n, vp(P["ss"]), vp(P["sc"]), src_slots, vp(P["si"]),
              vp(P["ds"]), vp(P["dc"]), dst_slots, vp(P["di"]), None)


@pytest.mark.parametrize("name", ["kda_state_checkpoint", "kda_resume"])
def test_copy_validation(name):
    fn = getattr(kda.lib(), name)
    assert copy_call(fn, cfg(), n=-1) == kda.KDA_ERR_INVALID_ARG
    assert copy_call(fn, cfg(), src_slots=0) == kda.KDA_ERR_INVALID_ARG
    for p in ("ss", "sc", "si", "ds", "dc", "di"):
        assert copy_call(fn, cfg(), **{p: None}) == kda.KDA_ERR_INVALID_ARG, p
    assert copy_call(fn, cfg(), ss=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert copy_call(fn, cfg(head_k=48, head_v=48)) == kda.KDA_ERR_UNSUPPORTED
    assert copy_call(fn, cfg(), n=0, ss=None) == kda.KDA_OK
    # one workgroup per 4 KiB piece of every (pair, head): 17 per head at d=128 with an fp32 state
    c = cfg()
    pieces = (c.head_k * c.head_v * 4 + 4095) // 4096 + ((2 * c.head_k + c.head_v) * 3 * 2 + 4095) // 4096
    n_max = (2 ** 31 - 1) // (c.num_heads * pieces)
    assert copy_call(fn, c, n=n_max + 1) == kda.KDA_ERR_INVALID_ARG
    assert "launch grid" in kda.lib().kda_last_error().decode()


def prefill_call(c, N=2, T=100, interval=0, ws_bytes=1 << 20, nck=4, flags=0, **ptrs):
    names = ("cu", "sp", "q", "k", "v", "z", "g", "beta", "conv_w", "norm_w", "state", "conv",
             "init", "final", "cks", "ckc", "ckb", "out", "ws")
    P = {n: FAKE for n in names}
    P.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.lib().kda_prefill_varlen(
        ctypes.byref(c.c()), N, T, vp(P["cu"]), vp(P["sp"]), vp(P["q"]), vp(P["k"]), vp(P["v"]),
        vp(P["z"]), vp(P["g"]), vp(P["beta"]), vp(P["conv_w"]), vp(P["norm_w"]), vp(P["state"]),
        vp(P["conv"]), 8, vp(P["init"]), vp(P["final"]), interval, vp(P["cks"]), vp(P["ckc"]),
        nck, vp(P["ckb"]), flags, vp(P["out"]), vp(P["ws"]), ws_bytes, None)


def test_prefill_validation():
    assert prefill_call(cfg(), N=-1) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), T=-5) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), T=1 << 31) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), interval=100) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), interval=-64) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(head_k=96, head_v=96)) == kda.KDA_ERR_UNSUPPORTED
    assert prefill_call(cfg(act_dtype=kda.KDA_F32)) == kda.KDA_ERR_UNSUPPORTED   # fp32 with dk=128
    assert prefill_call(cfg(), ws_bytes=0) == kda.KDA_ERR_WORKSPACE
    assert "workspace" in kda.last_error()
    assert prefill_call(cfg(), cu=None) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), q=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), interval=64, ckb=None) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), interval=64, nck=0) == kda.KDA_ERR_INVALID_ARG
    assert prefill_call(cfg(), N=0, cu=None) == kda.KDA_OK                      # nothing to do
    assert prefill_call(cfg(), flags=16) == kda.KDA_ERR_INVALID_ARG                # unknown flag
    assert "unknown" in kda.last_error()
    assert prefill_call(cfg(head_k=64, head_v=64, act_dtype=kda.KDA_F32),
                        flags=kda.KDA_PREFILL_CONV_DONE) == kda.KDA_ERR_UNSUPPORTED  # the front end is bf16 only
    assert "CONV_DONE" in kda.last_error()
    assert prefill_call(cfg(), flags=kda.KDA_PREFILL_PAIRED_POLL_ONCE) == kda.KDA_ERR_INVALID_ARG
    assert "needs KDA_PREFILL_PAIRED" in kda.last_error()
    both = kda.KDA_PREFILL_SPLIT | kda.KDA_PREFILL_PAIRED
    assert prefill_call(cfg(), interval=64, flags=both) == kda.KDA_ERR_INVALID_ARG   # exclusive modes
    assert "exclude" in kda.last_error()
    assert prefill_call(cfg(), flags=kda.KDA_PREFILL_SPLIT) == kda.KDA_ERR_INVALID_ARG   # split without interval
    assert "interval" in kda.last_error()
    assert prefill_call(cfg(), interval=64, flags=kda.KDA_PREFILL_SPLIT, ws_bytes=1 << 20) == kda.KDA_ERR_WORKSPACE
    ws = kda.kda_prefill_workspace_bytes(cfg(), 16, 1 << 18)
    assert ws >= 256 + 16 * 32 and ws % 256 == 0          # status word block, then the work items
    assert kda.kda_prefill_workspace_bytes(cfg(), 0, 0) == 256
    # split: room for 2N + T/interval segments, three dk x dv fp32 matrices per segment and head
    ws_split = kda.kda_prefill_workspace_bytes(cfg(), 16, 1 << 18, 4096, kda.KDA_PREFILL_SPLIT)
    segs = 2 * 16 + (1 << 18) // 4096
    assert ws_split >= segs * 4 * 3 * 128 * 128 * 4 and ws_split % 256 == 0
    # paired: a ring of three slots per pair of workgroups, each slot holding a chunk's planes (at
    # least K+ and K-^T as bf16 hi/lo pairs and Q+ hi); up to min(chains, 256) pairs
    ws_pair = kda.kda_prefill_workspace_bytes(cfg(), 16, 1 << 18, 0, kda.KDA_PREFILL_PAIRED)
    slot_min = 2 * 2 * 64 * 128 * 2 + 64 * 128 * 2
    assert ws_pair >= ws + 16 * 4 * 3 * slot_min and ws_pair % 256 == 0
    ws_big = kda.kda_prefill_workspace_bytes(cfg(), 512, 1 << 18)
    ws_big_pair = kda.kda_prefill_workspace_bytes(cfg(), 512, 1 << 18, 0, kda.KDA_PREFILL_PAIRED)
    assert ws_big + 256 * 3 * slot_min <= ws_big_pair < ws_big + 257 * 3 * 2 * slot_min
    with pytest.raises(kda.KdaError):
        kda.kda_prefill_workspace_bytes(cfg(), 16, 1 << 18, 0, kda.KDA_PREFILL_SPLIT)


def test_num_checkpoints_matches_oracle_rule():
    rng = np.random.default_rng(5)
    for _ in range(500):
        start = int(rng.integers(0, 1 << 20))
        length = int(rng.integers(0, 1 << 16))
        interval = int(rng.choice([0, 64, 128, 4096, 32768]))
        assert kda.kda_num_checkpoints(start, length, interval) == oracle.num_checkpoints(start, length, interval)


def project_in_call(c, T=4, Dm=256, **ptrs):
    P = {n: FAKE for n in ("x", "w", "q", "k", "v", "z", "g", "beta")}
    P.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.lib().kda_project_inputs(ctypes.byref(c.c()), T, Dm, *(vp(P[n]) for n in
                                        ("x", "w", "q", "k", "v", "z", "g", "beta")), None)


def project_out_call(c, T=4, Dm=7168, **ptrs):
    P = {n: FAKE for n in ("o", "w_o", "y")}
    P.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.lib().kda_project_output(ctypes.byref(c.c()), T, Dm, vp(P["o"]), vp(P["w_o"]), vp(P["y"]), None)


def test_projection_validation():
    assert project_in_call(cfg(act_dtype=kda.KDA_F32)) == kda.KDA_ERR_UNSUPPORTED
    assert project_in_call(cfg(), Dm=100) == kda.KDA_ERR_INVALID_ARG
    assert project_in_call(cfg(), Dm=0) == kda.KDA_ERR_INVALID_ARG
    assert project_in_call(cfg(), Dm=(1 << 22) + 64) == kda.KDA_ERR_INVALID_ARG
    assert project_in_call(cfg(), T=-1) == kda.KDA_ERR_INVALID_ARG
    for name in ("x", "w", "q", "k", "v", "z", "g", "beta"):
        assert project_in_call(cfg(), **{name: None}) == kda.KDA_ERR_INVALID_ARG, name
    assert project_in_call(cfg(), w=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert project_in_call(cfg(), T=0, x=None) == kda.KDA_OK

    assert project_out_call(cfg(act_dtype=kda.KDA_F32)) == kda.KDA_ERR_UNSUPPORTED
    assert project_out_call(cfg(num_heads=1, head_k=32, head_v=32)) == kda.KDA_ERR_UNSUPPORTED   # H dv = 32
    assert "multiple of 64" in kda.last_error()
    assert project_out_call(cfg(), Dm=0) == kda.KDA_ERR_INVALID_ARG
    assert project_out_call(cfg(), T=-1) == kda.KDA_ERR_INVALID_ARG
    for name in ("o", "w_o", "y"):
        assert project_out_call(cfg(), **{name: None}) == kda.KDA_ERR_INVALID_ARG, name
    assert project_out_call(cfg(), o=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert project_out_call(cfg(), y=FAKE + 1) == kda.KDA_ERR_INVALID_ARG
    assert project_out_call(cfg(), T=0, o=None) == kda.KDA_OK
    assert kda.last_error() == ""


def test_project_inputs_conv_validation():
    """The conv front end checks its arguments on the host (no GPU needed)."""
    P = ctypes.c_void_p
    L = kda.lib()

    def call(c, N=2, T=8, Dm=128, **ptrs):
        names = ("cu", "x", "w", "cw", "pool", "init", "q", "k", "v", "z", "g", "beta")
        a = {n: FAKE for n in names}
        a.update(ptrs)
        vp = lambda x: None if x is None else P(x)
        return L.kda_project_inputs_conv(ctypes.byref(c.c()), N, T, Dm, vp(a["cu"]), vp(a["x"]), vp(a["w"]),
                                         vp(a["cw"]), vp(a["pool"]), 4, vp(a["init"]), vp(a["q"]), vp(a["k"]),
                                         vp(a["v"]), vp(a["z"]), vp(a["g"]), vp(a["beta"]), None)

    assert call(cfg(act_dtype=kda.KDA_F32, head_k=64, head_v=64)) == kda.KDA_ERR_UNSUPPORTED
    assert call(cfg(), N=0) == kda.KDA_ERR_INVALID_ARG
    assert call(cfg(), Dm=100) == kda.KDA_ERR_INVALID_ARG
    assert call(cfg(), cu=None) == kda.KDA_ERR_INVALID_ARG
    assert call(cfg(), q=MISALIGNED) == kda.KDA_ERR_INVALID_ARG
    assert call(cfg(), T=0, cu=None) == kda.KDA_OK                     # nothing to do
