"""GPU integration of the prefix cache: a second request that shares a prefix
resumes from the cached state (copy-on-write into a private slot) and
prefills only the rest.

Token ids select per-token layer inputs from a seeded table, so equal token
prefixes give equal inputs.  A hit on an interval checkpoint (a multiple of
64) reproduces the straight run of the second request bit for bit; a hit on
a prompt end between chunk boundaries agrees to rounding.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import TOL_STATE_PER_CHAIN, bits, dev, host, per_chain_max, per_row_max, rel_l2, say, tol_row

pytestmark = pytest.mark.gpu

SHAPE = wl.LayerShape(2, 64, 64)
VOCAB, INTERVAL = 64, 128


class Layer:
    def __init__(self, seed):
        self.cfg = kda.Config(SHAPE.H, SHAPE.dk, SHAPE.dv, kda.KDA_BF16)
        self.table = wl.token_inputs(seed, SHAPE, VOCAB, g_scale=0.1, norm_w="random")   # one row per token id
        act = self.cfg.torch_act
        t = self.table
        self.q, self.k, self.v, self.z = (dev(a, act) for a in (t.q, t.k, t.v, t.z))
        self.g, self.beta = dev(t.g), dev(t.beta)
        self.cw, self.nw = dev(t.conv_w), dev(t.norm_w)

    def prefill(self, ids, start, S, X, init, final, ckS=None, ckX=None, ckbase=0):
        """One sequence: tokens ids (absolute positions start..) from slot init
        (-1: zero) into slot final; checkpoints every INTERVAL if ckS given."""
        idx = torch.from_numpy(np.asarray(ids, np.int64)).cuda()
        T = len(ids)
        H, dv = SHAPE.H, SHAPE.dv
        out = torch.empty((T, H, dv), dtype=self.cfg.torch_act, device="cuda")
        iv = INTERVAL if ckS is not None else 0
        ws = torch.empty(max(kda.kda_prefill_workspace_bytes(self.cfg, 1, T, iv, 0), 1), dtype=torch.uint8,
                         device="cuda")
        kda.kda_prefill_varlen(self.cfg, dev(np.array([0, T], np.int32)), self.q[idx], self.k[idx], self.v[idx],
                               self.z[idx], self.g[idx], self.beta[idx], self.cw, self.nw, S, X,
                               dev(np.array([init], np.int32)), dev(np.array([final], np.int32)), out, ws,
                               start_pos=dev(np.array([start], np.int64)), ckpt_interval=iv, ckpt_state=ckS,
                               ckpt_conv=ckX, ckpt_base=dev(np.array([ckbase], np.int32)) if iv else None)
        return out


def check_hit_against_oracle(layer, ids, p, out_hit, S_hit, X_hit):
    """The fp64 oracle over the whole request ids from a zero state: the
    outputs the hit prefilled (tokens p..) and the final state and conv
    state, within the bf16 tolerances (outputs 1e-2 whole and 5e-2 per row,
    states 5e-3 whole and 1e-4 per head)."""
    t = layer.table
    idx = np.asarray(ids, np.int64)
    r = oracle.run(t.q[idx], t.k[idx], t.v[idx], t.z[idx], t.g[idx], t.beta[idx], t.conv_w, t.norm_w,
                   [0, len(ids)])
    o = host(out_hit)
    e_o, e_r = rel_l2(o, r.out[p:]), per_row_max(o, r.out[p:])
    S = host(S_hit)[None]
    e_s, e_c = rel_l2(S, r.S), per_chain_max(S, r.S)
    say(f"  hit at {p} vs oracle: out {e_o:.3e} (worst row {e_r:.3e}), state {e_s:.3e} (worst head {e_c:.3e})")
    assert e_o <= 1e-2 and e_r <= tol_row("bf16") and e_s <= 5e-3 and e_c <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(host(X_hit)[None], r.X)


def pools(n):
    H, dk, dv, C = SHAPE.H, SHAPE.dk, SHAPE.dv, SHAPE.C
    return (torch.zeros((n, H, dk, dv), device="cuda"), torch.zeros((n, H, C, 3), dtype=torch.bfloat16, device="cuda"))


def test_prefix_hit_resumes_and_matches_straight_runs():
    rng = np.random.default_rng(90)
    layer = Layer(90)
    cfg = layer.cfg
    live_S, live_X = pools(8)
    cache_S, cache_X = pools(16)
    stage_S, stage_X = pools(8)
    cache = kda.PrefixCache(16, unit=INTERVAL)

    # request A: 700 tokens, checkpoints at 128..640 and the prompt end 700
    A = rng.integers(0, VOCAB, 700)
    layer.prefill(A, 0, live_S, live_X, -1, 0, stage_S, stage_X, 0)
    positions = [128, 256, 384, 512, 640, 700]
    slots = cache.reserve(len(positions))
    kda.kda_resume(cfg, stage_S, stage_X, dev(np.arange(len(positions), dtype=np.int32)), cache_S, cache_X,
                   dev(slots))
    for j, p in enumerate(positions):
        assert cache.insert(A, p, int(slots[j]), step=1)
    assert cache.lookup(A)[0] == 0                  # not visible before the step commits
    torch.cuda.synchronize()
    cache.commit(1)

    # request B shares A's first 520 tokens: hit at 512
    B = np.concatenate([A[:520], rng.integers(0, VOCAB, 380)])
    p, slot = cache.lookup(B, max_len=len(B) - 1)
    assert p == 512 and slot == int(slots[3])
    kda.kda_resume(cfg, cache_S, cache_X, dev(np.array([slot], np.int32)), live_S, live_X, dev(np.array([1], np.int32)))
    cache.release(slot)
    out_hit = layer.prefill(B[p:], p, live_S, live_X, 1, 1)
    out_ref = layer.prefill(B, 0, live_S, live_X, -1, 2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_hit), bits(out_ref[p:]))
    assert np.array_equal(bits(live_S[1]), bits(live_S[2])) and np.array_equal(bits(live_X[1]), bits(live_X[2]))
    say(f"  hit at {p}: {len(B) - p} of {len(B)} tokens prefilled, bitwise equal to the straight run")
    check_hit_against_oracle(layer, B, p, out_hit, live_S[1], live_X[1])

    # request C extends the whole prompt A: hit at the prompt end 700
    Cq = np.concatenate([A, rng.integers(0, VOCAB, 100)])
    p, slot = cache.lookup(Cq, max_len=len(Cq) - 1)
    assert p == 700 and slot == int(slots[5])
    kda.kda_resume(cfg, cache_S, cache_X, dev(np.array([slot], np.int32)), live_S, live_X, dev(np.array([3], np.int32)))
    cache.release(slot)
    out_hit = layer.prefill(Cq[p:], p, live_S, live_X, 3, 3)
    out_ref = layer.prefill(Cq, 0, live_S, live_X, -1, 4)
    torch.cuda.synchronize()
    e_o = rel_l2(host(out_hit), host(out_ref[p:]))
    e_s = per_chain_max(host(live_S[3:4]), host(live_S[4:5]))
    say(f"  hit at prompt end {p}: outputs {e_o:.3e}, state {e_s:.3e} from the straight run")
    assert e_o <= 1e-2 and e_s <= TOL_STATE_PER_CHAIN
    check_hit_against_oracle(layer, Cq, p, out_hit, live_S[3], live_X[3])
    # the cached states were never written by the requests that extended them
    assert np.array_equal(bits(cache_S[torch.from_numpy(slots.astype(np.int64)).cuda()]),
                          bits(stage_S[:len(positions)]))
    st = cache.stats()
    assert st["hits"] == 2 and st["pinned_slots"] == 0
