"""GPU parity of the fused decode step (kda_decode_step) against the fp64 oracle.

Each case steps B sequences through `steps` single-token decode launches on
slots drawn from a larger pool, then compares every step's outputs and the
final states and conv states with the oracle stepped the same way.  The pool's
unused slots are filled with a NaN pattern and must come back untouched.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import TOL_STATE_PER_CHAIN, bits, dev, host, per_chain_max, per_row_max, rel_l2, say, tol_row, tols

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0DEAD


def make_case(seed, shape: wl.LayerShape, B, steps, pool, g_scale=1.0, norm_w="ones",
              state_std=0.02, conv_std=1.0, zero_state=False):
    T = B * steps
    inp = wl.token_inputs(seed, shape, T, g_scale=g_scale, norm_w=norm_w)
    S, X = wl.states(seed, shape, pool, state_std=state_std, conv_std=conv_std)
    if zero_state:
        S[:] = 0.0
        X[:] = 0.0
    slots = wl.slot_permutation(seed, pool, B)
    return inp, S, X, slots


def run_gpu(inp, S, X, slots, shape, steps, B):
    cfg = kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16 if shape.act == "bf16" else kda.KDA_F32)
    act = cfg.torch_act
    H, dk, dv = shape.H, shape.dk, shape.dv
    r = lambda a, d: a.reshape((steps, B) + a.shape[1:])
    q, k, v, z = (dev(r(a, 0), act) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = dev(r(inp.g, 0)), dev(r(inp.beta, 0))
    conv_w, norm_w = dev(inp.conv_w), dev(inp.norm_w)
    Sd = dev(S)
    Xd = dev(X, act)
    # NaN-fill the slots no sequence uses (guards)
    used = np.zeros(S.shape[0], bool)
    used[slots] = True
    guard = torch.from_numpy(~used).cuda()
    Sd.view(torch.int32)[guard] = NAN_BITS
    Xd.view(torch.int16 if act == torch.bfloat16 else torch.int32)[guard] = -1
    guard_before = (bits(Sd[guard]), bits(Xd[guard]))
    slot_d = dev(slots)
    out = torch.empty((steps, B, H, dv), dtype=act, device="cuda")
    for s in range(steps):
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, Sd, Xd,
                            slot_d, out[s])
    torch.cuda.synchronize()
    assert np.array_equal(bits(Sd[guard]), guard_before[0]), "guard state slots were written"
    assert np.array_equal(bits(Xd[guard]), guard_before[1]), "guard conv slots were written"
    return out, Sd, Xd


def run_oracle(inp, S, X, slots, steps, B):
    r = lambda a: a.reshape((steps, B) + a.shape[1:])
    return oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                               inp.conv_w, inp.norm_w, S[slots], X[slots])


CASES = {
    # name: (seed, shape, B, steps, pool, kwargs)
    "tiny_f32_d32": (0, wl.LayerShape(2, 32, 32, act="f32"), 1, 64, 1, dict(zero_state=True)),
    "f32_d64": (5, wl.LayerShape(3, 64, 64, act="f32"), 5, 20, 9, {}),
    "f32_d128_weakdecay": (6, wl.LayerShape(2, 128, 128, act="f32"), 3, 40, 4,
                           dict(g_scale=0.01, norm_w="random", state_std=0.5)),
    "bf16_d32": (7, wl.LayerShape(4, 32, 32), 6, 30, 8, {}),
    "bf16_d64_nodecay": (8, wl.LayerShape(2, 64, 64), 4, 30, 6, dict(g_scale=0.0, norm_w="random")),
    "bf16_d128_weakdecay": (9, wl.LayerShape(4, 128, 128), 8, 48, 12, dict(g_scale=0.01, norm_w="random")),
    "bf16_d128_strongdecay": (10, wl.LayerShape(4, 128, 128), 8, 48, 12, dict(g_scale=4.0, norm_w="random")),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    seed, shape, B, steps, pool, kw = CASES[name]
    say(f"decode case {name}: H={shape.H} d={shape.dk} act={shape.act} B={B} steps={steps}")
    inp, S, X, slots = make_case(seed, shape, B, steps, pool, **kw)
    out, Sd, Xd = run_gpu(inp, S, X, slots, shape, steps, B)
    o_ref, S_ref, X_ref = run_oracle(inp, S, X, slots, steps, B)
    tol_o, tol_s = tols(shape.act)
    e_out = rel_l2(host(out), o_ref)
    e_s = rel_l2(host(Sd)[slots], S_ref)
    e_c = per_chain_max(host(Sd)[slots], S_ref)
    e_r = per_row_max(host(out), o_ref, 3)
    say(f"  rel-L2 out {e_out:.3e}  state {e_s:.3e}  worst chain {e_c:.3e}  worst row {e_r:.3e}")
    assert e_out <= tol_o and e_s <= tol_s and e_c <= TOL_STATE_PER_CHAIN and e_r <= tol_row(shape.act)
    # the conv state holds raw inputs: exact
    np.testing.assert_array_equal(host(Xd)[slots], X_ref)


def test_decode_batched_b64_full_size():
    """The batched decode workload at full size: 64 sequences x 256 steps,
    H=32, dk=dv=128, bf16 activations, fp32 state ~ N(0, 0.02^2), bf16 conv
    state ~ N(0,1), slots drawn from an 80-slot pool (16 NaN guards)."""
    w = wl.WORKLOADS["decode_b64"]
    shape, B, steps, pool = w["shape"], w["B"], w["steps"], w["pool"]
    say(f"decode full size: B={B} steps={steps} H={shape.H}")
    inp, S, X, slots = make_case(w["seed"], shape, B, steps, pool, state_std=w["state_std"],
                                 conv_std=w["conv_std"])
    out, Sd, Xd = run_gpu(inp, S, X, slots, shape, steps, B)
    o_ref, S_ref, X_ref = run_oracle(inp, S, X, slots, steps, B)
    e_out = rel_l2(host(out), o_ref)
    e_s = rel_l2(host(Sd)[slots], S_ref)
    e_c = per_chain_max(host(Sd)[slots], S_ref)
    e_r = per_row_max(host(out), o_ref, 3)
    say(f"  rel-L2 out {e_out:.3e}  state {e_s:.3e}  worst chain {e_c:.3e}  worst row {e_r:.3e}")
    assert e_out <= 1e-2 and e_s <= 5e-3 and e_c <= TOL_STATE_PER_CHAIN and e_r <= tol_row("bf16")
    np.testing.assert_array_equal(host(Xd)[slots], X_ref)


def test_decode_invalid_slot_writes_nan_and_skips():
    shape = wl.LayerShape(2, 32, 32)
    inp, S, X, _ = make_case(11, shape, 3, 1, 4)
    cfg = kda.Config(2, 32, 32)
    act = cfg.torch_act
    Sd, Xd = dev(S), dev(X, act)
    before = (bits(Sd), bits(Xd))
    slot = dev(np.array([-1, 4, 1000], np.int32))
    out = torch.zeros((3, 2, 32), dtype=act, device="cuda")
    kda.kda_decode_step(cfg, dev(inp.q, act), dev(inp.k, act), dev(inp.v, act), dev(inp.z, act),
                        dev(inp.g), dev(inp.beta), dev(inp.conv_w), dev(inp.norm_w), Sd, Xd, slot, out)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    assert np.array_equal(bits(Sd), before[0]) and np.array_equal(bits(Xd), before[1])


def test_decode_deterministic():
    shape = wl.LayerShape(4, 128, 128)
    inp, S, X, slots = make_case(12, shape, 8, 6, 8)
    a = run_gpu(inp, S, X, slots, shape, 6, 8)
    b = run_gpu(inp, S, X, slots, shape, 6, 8)
    for x, y in zip(a, b):
        assert np.array_equal(bits(x), bits(y))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_checkpoint_resume_decode_bitwise(act):
    """Checkpoint the live slots after some steps, keep stepping; resume the
    checkpoint into fresh slots (copy-on-write) and step the same inputs: the
    results equal the straight run bit for bit, and the checkpoint is left
    untouched."""
    shape = wl.LayerShape(3, 64, 64, act=act)
    B, steps, p = 4, 12, 5
    inp, S, X, slots = make_case(13, shape, B, steps, 16)
    cfg = kda.Config(3, 64, 64, kda.KDA_BF16 if act == "bf16" else kda.KDA_F32)
    tact = cfg.torch_act
    r = lambda a: a.reshape((steps, B) + a.shape[1:])
    q, k, v, z = (dev(r(a), tact) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = dev(r(inp.g)), dev(r(inp.beta))
    cw, nw = dev(inp.conv_w), dev(inp.norm_w)
    Sd, Xd = dev(S), dev(X, tact)
    ckS = torch.zeros((6,) + S.shape[1:], device="cuda")
    ckX = torch.zeros((6,) + X.shape[1:], dtype=tact, device="cuda")
    live = dev(slots)
    ck_ids = dev(np.array([5, 0, 3, 1], np.int32))
    outA = torch.empty((steps, B, 3, 64), dtype=tact, device="cuda")
    for s in range(steps):
        if s == p:
            kda.kda_state_checkpoint(cfg, Sd, Xd, live, ckS, ckX, ck_ids)
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], cw, nw, Sd, Xd, live, outA[s])
    torch.cuda.synchronize()
    ck_before = (bits(ckS), bits(ckX))
    # resume into the other slots of the pool, enqueued right before the steps
    free = np.setdiff1d(np.arange(16), slots)[:B].astype(np.int32)
    fresh = dev(free)
    kda.kda_resume(cfg, ckS, ckX, ck_ids, Sd, Xd, fresh)
    outB = torch.empty((steps - p, B, 3, 64), dtype=tact, device="cuda")
    for s in range(p, steps):
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], cw, nw, Sd, Xd, fresh, outB[s - p])
    torch.cuda.synchronize()
    assert np.array_equal(bits(outA[p:]), bits(outB))
    assert np.array_equal(bits(Sd[live.long()]), bits(Sd[fresh.long()]))
    assert np.array_equal(bits(Xd[live.long()]), bits(Xd[fresh.long()]))
    assert np.array_equal(bits(ckS), ck_before[0]) and np.array_equal(bits(ckX), ck_before[1])


def test_copy_skips_out_of_range_ids():
    cfg = kda.Config(2, 32, 32)
    S = torch.randn(4, 2, 32, 32, device="cuda")
    X = torch.randn(4, 2, 96, 3, device="cuda").to(torch.bfloat16)
    cS = torch.zeros(2, 2, 32, 32, device="cuda")
    cX = torch.zeros(2, 2, 96, 3, device="cuda", dtype=torch.bfloat16)
    kda.kda_state_checkpoint(cfg, S, X, dev(np.array([1, 7, -1], np.int32)), cS, cX,
                             dev(np.array([0, 1, 1], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(cS[0], S[1]) and torch.equal(cX[0], X[1])
    assert torch.count_nonzero(cS[1]) == 0 and torch.count_nonzero(cX[1].float()) == 0
