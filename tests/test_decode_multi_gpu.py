"""GPU tests of kda_decode_multi: T decode tokens per sequence in one launch.

The contract is bitwise: T tokens in one launch equal T successive
kda_decode_step calls (outputs, final states, conv states), the per-token
states equal the states after each single step, and rolling a sequence back
to its first a tokens with kda_resume from slot b*T + a - 1 of the per-token
pools gives the state of a single steps.  One case is also checked against
the oracle directly.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import TOL_STATE_PER_CHAIN, bits, dev, host, per_chain_max, per_row_max, rel_l2, say, tol_row, tols

pytestmark = pytest.mark.gpu


def setup(shape, seed, B, T, pool, state_dtype, g_scale=0.2):
    cfg = kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16 if shape.act == "bf16" else kda.KDA_F32,
                     state_dtype=state_dtype)
    act, st = cfg.torch_act, cfg.torch_state
    inp = wl.token_inputs(seed, shape, B * T, g_scale=g_scale, norm_w="random")
    S, X = wl.states(seed, shape, pool, state_std=0.1, conv_std=1.0)
    S = torch.from_numpy(S).to(st).double().numpy()             # values the pool dtype holds
    slots = wl.slot_permutation(seed, pool, B)
    r = lambda a: a.reshape((T, B) + a.shape[1:])
    t = dict(q=dev(r(inp.q), act), k=dev(r(inp.k), act), v=dev(r(inp.v), act), z=dev(r(inp.z), act),
             g=dev(r(inp.g)), beta=dev(r(inp.beta)), cw=dev(inp.conv_w), nw=dev(inp.norm_w))
    return cfg, inp, S, X, slots, t


def single_steps(cfg, S, X, slots, t, T):
    Sd, Xd = dev(S, cfg.torch_state), dev(X, cfg.torch_act)
    slot = dev(slots)
    B = len(slots)
    out = torch.empty((T, B, cfg.num_heads, cfg.head_v), dtype=cfg.torch_act, device="cuda")
    after = []
    for s in range(T):
        kda.kda_decode_step(cfg, t["q"][s], t["k"][s], t["v"][s], t["z"][s], t["g"][s], t["beta"][s], t["cw"], t["nw"],
                            Sd, Xd, slot, out[s])
        after.append((Sd[slot.long()].clone(), Xd[slot.long()].clone()))
    torch.cuda.synchronize()
    return out, Sd, Xd, after


def multi(cfg, S, X, slots, t, T, keep=True):
    Sd, Xd = dev(S, cfg.torch_state), dev(X, cfg.torch_act)
    slot = dev(slots)
    B, H, dk, dv, C = len(slots), cfg.num_heads, cfg.head_k, cfg.head_v, cfg.conv_channels
    out = torch.full((T, B, H, dv), float("nan"), dtype=cfg.torch_act, device="cuda")
    ts = torch.zeros((B, T, H, dk, dv), dtype=cfg.torch_state, device="cuda") if keep else None
    tc = torch.zeros((B, T, H, C, 3), dtype=cfg.torch_act, device="cuda") if keep else None
    kda.kda_decode_multi(cfg, t["q"], t["k"], t["v"], t["z"], t["g"], t["beta"], t["cw"], t["nw"], Sd, Xd, slot, out,
                         token_state=ts, token_conv=tc)
    torch.cuda.synchronize()
    return out, Sd, Xd, ts, tc


CASES = {
    # name: (shape, B, T, pool, state dtype)
    "bf16_d128_T5": (wl.LayerShape(4, 128, 128), 8, 5, 12, kda.KDA_F32),
    "bf16_d128_T5_bf16state": (wl.LayerShape(4, 128, 128), 8, 5, 12, kda.KDA_BF16),
    "bf16_d64_T8": (wl.LayerShape(3, 64, 64), 5, 8, 9, kda.KDA_F32),
    "f32_d64_T3": (wl.LayerShape(2, 64, 64, act="f32"), 4, 3, 6, kda.KDA_F32),
    "f32_d32_T2_bf16state": (wl.LayerShape(2, 32, 32, act="f32"), 3, 2, 5, kda.KDA_BF16),
    "bf16_d32_T1": (wl.LayerShape(4, 32, 32), 6, 1, 8, kda.KDA_F32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_multi_equals_single_steps_bitwise(name):
    shape, B, T, pool, sdt = CASES[name]
    say(f"decode multi {name}: B={B} T={T}")
    cfg, inp, S, X, slots, t = setup(shape, 80, B, T, pool, sdt)
    o1, S1, X1, after = single_steps(cfg, S, X, slots, t, T)
    o2, S2, X2, ts, tc = multi(cfg, S, X, slots, t, T)
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(S1), bits(S2)) and np.array_equal(bits(X1), bits(X2))
    for s in range(T):
        assert np.array_equal(bits(ts[:, s]), bits(after[s][0])), f"token state {s}"
        assert np.array_equal(bits(tc[:, s]), bits(after[s][1])), f"token conv state {s}"


def test_multi_rollback_by_resume():
    """Roll every sequence back to a seeded number of accepted tokens."""
    shape, B, T, pool = wl.LayerShape(4, 128, 128), 8, 5, 20
    cfg, inp, S, X, slots, t = setup(shape, 81, B, T, pool, kda.KDA_F32)
    _, _, _, after = single_steps(cfg, S, X, slots, t, T)
    _, Sd, Xd, ts, tc = multi(cfg, S, X, slots, t, T)
    acc = np.random.default_rng(81).integers(1, T + 1, B)
    src = dev((np.arange(B) * T + acc - 1).astype(np.int32))
    kda.kda_resume(cfg, ts.reshape(B * T, *ts.shape[2:]), tc.reshape(B * T, *tc.shape[2:]), src, Sd, Xd,
                   dev(slots))
    torch.cuda.synchronize()
    for b in range(B):
        a = int(acc[b])
        assert np.array_equal(bits(Sd[int(slots[b])]), bits(after[a - 1][0][b])), f"sequence {b}, {a} accepted"
        assert np.array_equal(bits(Xd[int(slots[b])]), bits(after[a - 1][1][b]))


def test_multi_matches_oracle_and_no_token_buffers():
    shape, B, T, pool = wl.LayerShape(4, 128, 128), 8, 7, 12
    cfg, inp, S, X, slots, t = setup(shape, 82, B, T, pool, kda.KDA_F32)
    out, Sd, Xd, _, _ = multi(cfg, S, X, slots, t, T, keep=False)
    r = lambda a: a.reshape((T, B) + a.shape[1:])
    o_ref, S_ref, X_ref = oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                                              inp.conv_w, inp.norm_w, S[slots], X[slots])
    tol_o, tol_s = tols("bf16")
    e_o, e_s = rel_l2(host(out), o_ref), rel_l2(host(Sd)[slots], S_ref)
    e_c = per_chain_max(host(Sd)[slots], S_ref)
    e_r = per_row_max(host(out), o_ref, 3)
    say(f"  multi vs oracle: out {e_o:.3e} state {e_s:.3e} worst chain {e_c:.3e} worst row {e_r:.3e}")
    assert e_o <= tol_o and e_s <= tol_s and e_c <= TOL_STATE_PER_CHAIN and e_r <= tol_row("bf16")
    np.testing.assert_array_equal(host(Xd)[slots], X_ref)


def test_multi_invalid_slot_gives_nan_and_writes_nothing():
    shape, B, T = wl.LayerShape(2, 64, 64), 3, 4
    cfg, inp, S, X, _, t = setup(shape, 83, B, T, 4, kda.KDA_F32)
    slots = np.array([1, -1, 9], np.int32)
    Sd, Xd = dev(S, torch.float32), dev(X, cfg.torch_act)
    before = (bits(Sd), bits(Xd))
    out = torch.zeros((T, B, 2, 64), dtype=cfg.torch_act, device="cuda")
    ts = torch.zeros((B, T, 2, 64, 64), device="cuda")
    kda.kda_decode_multi(cfg, t["q"], t["k"], t["v"], t["z"], t["g"], t["beta"], t["cw"], t["nw"], Sd, Xd,
                         dev(slots), out, token_state=ts)
    torch.cuda.synchronize()
    o = host(out)
    assert np.isfinite(o[:, 0]).all() and np.isnan(o[:, 1:]).all()
    Sh, Xh = bits(Sd), bits(Xd)
    assert not np.array_equal(Sh, before[0])                          # slot 1 advanced
    keep = [i for i in range(4) if i != 1]
    assert np.array_equal(bits(Sd[keep]), bits(dev(S, torch.float32)[keep]))
    assert np.array_equal(bits(Xd[keep]), bits(dev(X, cfg.torch_act)[keep]))
    assert torch.count_nonzero(ts[1:]) == 0
