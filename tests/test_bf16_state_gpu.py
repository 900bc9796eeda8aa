"""GPU tests of bf16 state storage (kda_config.state_dtype = KDA_BF16).

The state pools and checkpoints hold bf16; the kernels compute in fp32, round
to nearest bf16 wherever the state is stored (every decode step, every prefill
checkpoint, the prefill end) and continue from the stored value.  The oracle
runs with the same storage rule (state_round), so GPU and oracle differ only
where fp32 and fp64 values fall on different sides of a bf16 rounding
boundary.  Tolerances (relative L2, fp64): outputs 1e-2, states 5e-3 over the
whole tensor and 2e-3 per (sequence, head) (measured up to 6.5e-4, with weak
decay, where a flipped rounding persists longest); conv states exact;
checkpoints and resumes bit for bit in the stored dtype.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import bits, dev, host, per_chain_max, rel_l2, say
from tests.prefill_runner import Run, check_against_oracle, oracle_for, resume_and_finish, states_for

pytestmark = pytest.mark.gpu

BF = kda.KDA_BF16
TOL_OUT, TOL_STATE, TOL_CHAIN = 1e-2, 5e-3, 2e-3


def bf16_values(a):
    """The nearest bf16 values of a (the initial states a bf16 pool can hold)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).double().numpy()


def decode_run(shape, seed, B, steps, pool, g_scale=1.0, state_std=0.05):
    cfg = kda.Config(shape.H, shape.dk, shape.dv, BF if shape.act == "bf16" else kda.KDA_F32, state_dtype=BF)
    act = cfg.torch_act
    inp = wl.token_inputs(seed, shape, B * steps, g_scale=g_scale, norm_w="random")
    S, X = wl.states(seed, shape, pool, state_std=state_std, conv_std=1.0)
    S = bf16_values(S)
    slots = wl.slot_permutation(seed, pool, B)
    r = lambda a: a.reshape((steps, B) + a.shape[1:])
    q, k, v, z = (dev(r(a), act) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = dev(r(inp.g)), dev(r(inp.beta))
    Sd, Xd = dev(S, torch.bfloat16), dev(X, act)
    assert Sd.dtype == torch.bfloat16
    out = torch.empty((steps, B, shape.H, shape.dv), dtype=act, device="cuda")
    slot_d = dev(slots)
    for s in range(steps):
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], dev(inp.conv_w), dev(inp.norm_w),
                            Sd, Xd, slot_d, out[s])
    torch.cuda.synchronize()
    o_ref, S_ref, X_ref = oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                                              inp.conv_w, inp.norm_w, S[slots], X[slots], state_round=True)
    return out, Sd, Xd, slots, o_ref, S_ref, X_ref


@pytest.mark.parametrize("name,shape,B,steps,pool,g_scale", [
    ("bf16_d128", wl.LayerShape(4, 128, 128), 8, 48, 12, 1.0),
    ("bf16_d128_weak", wl.LayerShape(2, 128, 128), 4, 64, 6, 0.02),
    ("f32_d64", wl.LayerShape(3, 64, 64, act="f32"), 5, 30, 9, 0.1),
    ("bf16_d32", wl.LayerShape(4, 32, 32), 6, 30, 8, 1.0),
])
def test_decode_bf16_state_matches_oracle(name, shape, B, steps, pool, g_scale):
    say(f"decode, bf16 state: {name} B={B} steps={steps}")
    out, Sd, Xd, slots, o_ref, S_ref, X_ref = decode_run(shape, 70, B, steps, pool, g_scale)
    e_o = rel_l2(host(out), o_ref)
    Sg = host(Sd)[slots]
    e_s, e_c = rel_l2(Sg, S_ref), per_chain_max(Sg, S_ref)
    say(f"  rel-L2 out {e_o:.3e}  state {e_s:.3e}  worst chain {e_c:.3e}")
    assert e_o <= TOL_OUT and e_s <= TOL_STATE and e_c <= TOL_CHAIN
    np.testing.assert_array_equal(host(Xd)[slots], X_ref)


def test_decode_bf16_state_full_size():
    """The batched decode workload (64 x 256 steps, H=32, d=128) with a bf16 state pool."""
    w = wl.WORKLOADS["decode_b64"]
    shape, B, steps, pool = w["shape"], w["B"], w["steps"], w["pool"]
    out, Sd, Xd, slots, o_ref, S_ref, X_ref = decode_run(shape, w["seed"], B, steps, pool,
                                                         state_std=w["state_std"])
    e_o = rel_l2(host(out), o_ref)
    Sg = host(Sd)[slots]
    e_s, e_c = rel_l2(Sg, S_ref), per_chain_max(Sg, S_ref)
    say(f"  full size, bf16 state: out {e_o:.3e}  state {e_s:.3e}  worst chain {e_c:.3e}")
    assert e_o <= TOL_OUT and e_s <= TOL_STATE and e_c <= TOL_CHAIN


def check_bf16_prefill(run, r):
    Sf, Xf = run.final_state()
    e_o, e_s, e_c = rel_l2(host(run.out), r.out), rel_l2(Sf, r.S), per_chain_max(Sf, r.S)
    ck = host(run.ckS)[:run.nck] if run.nck else np.zeros(0)
    e_k = per_chain_max(ck, r.ckpt_S) if run.nck else 0.0
    say(f"  rel-L2 out {e_o:.3e}  state {e_s:.3e}  worst chain {e_c:.3e}  worst checkpoint chain {e_k:.3e}")
    assert e_o <= TOL_OUT and e_s <= TOL_STATE and e_c <= TOL_CHAIN and e_k <= TOL_CHAIN
    np.testing.assert_array_equal(Xf, r.X)
    if run.nck:
        np.testing.assert_array_equal(host(run.ckX)[:run.nck], r.ckpt_X)


@pytest.mark.parametrize("flags", [0, kda.KDA_PREFILL_SPLIT, kda.KDA_PREFILL_PAIRED])
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_prefill_bf16_state_matches_oracle(act, flags):
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [400, 1, 0, 190, 129], [0, 5, 3, 64, 128]
    inp = wl.token_inputs(71, shape, sum(lengths), g_scale=0.05, norm_w="random")
    S0, X0 = states_for(71, shape, len(lengths))
    S0 = bf16_values(S0)
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=64, flags=flags, state_dtype=BF).launch()
    assert run.Sd.dtype == torch.bfloat16 and run.ckS.dtype == torch.bfloat16
    check_bf16_prefill(run, oracle_for(run, S0, X0))
    for n, L in enumerate(lengths):
        if L:
            last = run.base[n] + oracle.num_checkpoints(starts[n], L, 64) - 1
            assert np.array_equal(bits(run.ckS[last]), bits(run.Sd[int(run.final[n])]))


def test_prefill_bf16_state_d128_no_checkpoints():
    shape = wl.LayerShape(4, 128, 128)
    lengths, starts = [300, 64, 17, 128], [0, 100, 7, 64]
    inp = wl.token_inputs(72, shape, sum(lengths))
    S0, X0 = states_for(72, shape, len(lengths))
    S0 = bf16_values(S0)
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, state_dtype=BF).launch()
    check_bf16_prefill(run, oracle_for(run, S0, X0))


@pytest.mark.parametrize("flags", [0, kda.KDA_PREFILL_SPLIT, kda.KDA_PREFILL_PAIRED])
def test_prefill_bf16_state_resume_is_bitwise(flags):
    shape = wl.LayerShape(2, 64, 64)
    lengths, starts = [700, 450, 300], [0, 128, 64]
    inp = wl.token_inputs(73, shape, sum(lengths), g_scale=0.05, norm_w="random")
    S0, X0 = states_for(73, shape, len(lengths))
    S0 = bf16_values(S0)
    straight = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=flags,
                   state_dtype=BF).launch()
    resumed, seqs, res_pos, src_ck, idx = resume_and_finish(straight, [2, 0, 1])
    say(f"  resumed at {res_pos}")
    assert np.array_equal(bits(resumed.out), bits(straight.out[torch.from_numpy(idx).cuda()]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))
        later = oracle.num_checkpoints(res_pos[j], resumed.lengths[j], 128)
        assert np.array_equal(bits(resumed.ckS[int(resumed.base[j]):int(resumed.base[j]) + later]),
                              bits(straight.ckS[src_ck[j] + 1:src_ck[j] + 1 + later]))


def test_bf16_state_copies_are_bitwise():
    cfg = kda.Config(2, 64, 64, state_dtype=BF)
    S = torch.randn(5, 2, 64, 64, device="cuda").to(torch.bfloat16)
    X = torch.randn(5, 2, 192, 3, device="cuda").to(torch.bfloat16)
    cS = torch.zeros(3, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    cX = torch.zeros(3, 2, 192, 3, device="cuda", dtype=torch.bfloat16)
    kda.kda_state_checkpoint(cfg, S, X, dev(np.array([4, 0, 2], np.int32)), cS, cX, dev(np.array([1, 2, 0], np.int32)))
    S2 = torch.zeros_like(S)
    X2 = torch.zeros_like(X)
    kda.kda_resume(cfg, cS, cX, dev(np.array([0, 1], np.int32)), S2, X2, dev(np.array([3, 1], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(cS[1].view(torch.int16), S[4].view(torch.int16)) and torch.equal(cS[0], S[2])
    assert torch.equal(S2[3].view(torch.int16), S[2].view(torch.int16))
    assert torch.equal(S2[1].view(torch.int16), S[4].view(torch.int16)) and torch.equal(X2[1], X[4])
    assert torch.count_nonzero(S2[0].float()) == 0
