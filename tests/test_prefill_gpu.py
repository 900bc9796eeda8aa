"""GPU parity of the chunked prefill (kda_prefill_varlen) against the fp64
oracle, plus its checkpoint and resume contracts.

Inputs come from the seeded generator; sequences are packed by cu_seqlens and
may start at unaligned absolute positions with nonzero initial states.  The
full-size 4 x 8192 workload is compared on sampled heads (the oracle runs only
those) and against the decode kernel stepped token by token.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import bits, dev, host, rel_l2, say, tols
from tests.prefill_runner import Run, check_against_oracle, oracle_for, resume_and_finish, states_for

pytestmark = pytest.mark.gpu


def test_prefill_tiny_f32_workload():
    """The tiny recurrent workload: B=1, T=64, H=2, dk=dv=32, fp32, zero state, seed 0."""
    w = wl.WORKLOADS["tiny_f32"]
    shape = w["shape"]
    inp = wl.token_inputs(w["seed"], shape, w["T"])
    run = Run(shape, inp, [w["T"]]).launch()
    check_against_oracle(run, oracle_for(run))


CASES = {
    # name: (seed, shape, lengths, starts, with_state, g_scale, norm_w)
    "f32_d32_ragged": (20, wl.LayerShape(2, 32, 32, act="f32"), [150, 1, 64, 0, 77], [0, 5, 64, 9, 30], True, 1.0, "random"),
    "f32_d64_weak": (21, wl.LayerShape(3, 64, 64, act="f32"), [200, 129], [13, 0], True, 0.02, "random"),
    "bf16_d64_nodecay": (22, wl.LayerShape(2, 64, 64), [190, 65, 3], [0, 63, 2], True, 0.0, "random"),
    "bf16_d128": (23, wl.LayerShape(4, 128, 128), [300, 64, 17, 128], [0, 100, 7, 64], True, 1.0, "ones"),
    "bf16_d128_weak": (24, wl.LayerShape(2, 128, 128), [256, 333], [0, 31], True, 0.01, "random"),
    "bf16_d128_zero_state": (25, wl.LayerShape(2, 128, 128), [257, 2], [0, 0], False, 1.0, "ones"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    seed, shape, lengths, starts, with_state, g_scale, norm_w = CASES[name]
    say(f"prefill case {name}: H={shape.H} d={shape.dk} act={shape.act} lengths={lengths} starts={starts}")
    inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=g_scale, norm_w=norm_w)
    S0 = X0 = None
    if with_state:
        S0, X0 = states_for(seed, shape, len(lengths))
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0).launch()
    check_against_oracle(run, oracle_for(run, S0, X0))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_prefill_checkpoints(act):
    """Checkpoint count and positions follow the rule; contents match the
    oracle's; the last checkpoint of a sequence equals its final state bit for
    bit."""
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [300, 64, 129, 0, 5], [0, 64, 100, 3, 128]
    inp = wl.token_inputs(30, shape, sum(lengths), g_scale=0.1, norm_w="random")
    S0, X0 = states_for(30, shape, len(lengths))
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=64).launch()
    r = oracle_for(run, S0, X0)
    assert run.nck == len(r.ckpt_S) and list(run.base) == list(r.ckpt_base)
    check_against_oracle(run, r)
    tol_o, tol_s = tols(act)
    ckS = host(run.ckS)[:run.nck]
    ckX = host(run.ckX)[:run.nck]
    e = rel_l2(ckS, r.ckpt_S)
    say(f"  checkpoints: {run.nck}, rel-L2 {e:.3e}")
    assert e <= tol_s
    np.testing.assert_array_equal(ckX, r.ckpt_X)
    Sf, Xf = run.final_state()
    for n, L in enumerate(lengths):
        if L == 0:
            continue
        last = run.base[n] + oracle.num_checkpoints(starts[n], L, 64) - 1
        assert np.array_equal(bits(run.ckS[last]), bits(run.Sd[int(run.final[n])]))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_resume_is_bitwise_identical(act):
    """Resume from interval checkpoints (copy-on-write into fresh slots) and
    prefill the remainder: every output from the resume point on, every later
    checkpoint and the final state equal the straight-through run bit for bit."""
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [400, 250, 193], [0, 128, 64]
    N = len(lengths)
    inp = wl.token_inputs(31, shape, sum(lengths), g_scale=0.05, norm_w="random")
    S0, X0 = states_for(31, shape, N)
    straight = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128).launch()
    ck_before = bits(straight.ckS)
    resumed, seqs, res_pos, src_ck, idx = resume_and_finish(straight, [1, 0, 1])
    assert np.array_equal(bits(straight.ckS), ck_before)          # copy-on-write source untouched
    assert np.array_equal(bits(resumed.out), bits(straight.out[torch.from_numpy(idx).cuda()]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))
        assert np.array_equal(bits(resumed.Xd[int(resumed.final[j])]), bits(straight.Xd[int(straight.final[n])]))
        later = oracle.num_checkpoints(res_pos[j], resumed.lengths[j], 128)
        for i in range(later):
            assert np.array_equal(bits(resumed.ckS[int(resumed.base[j]) + i]), bits(straight.ckS[src_ck[j] + 1 + i]))


def test_prefill_deterministic_and_packing_invariant():
    """Two identical calls give identical bits, and reordering the sequences in
    the packed batch leaves each sequence's outputs and states unchanged."""
    shape = wl.LayerShape(4, 128, 128)
    lengths, starts = [130, 64, 300, 1], [0, 64, 5, 0]
    inp = wl.token_inputs(32, shape, sum(lengths))
    S0, X0 = states_for(32, shape, len(lengths))
    a = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0).launch()
    b = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0).launch()
    assert np.array_equal(bits(a.out), bits(b.out)) and np.array_equal(bits(a.Sd), bits(b.Sd))
    perm = [2, 0, 3, 1]
    cu = a.cu
    idx = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in perm])
    sub = wl.Inputs(shape, inp.q[idx], inp.k[idx], inp.v[idx], inp.z[idx], inp.g[idx], inp.beta[idx],
                    inp.conv_w, inp.norm_w)
    c = Run(shape, sub, [lengths[n] for n in perm], starts=[starts[n] for n in perm],
            S0=S0[perm], X0=X0[perm]).launch()
    assert np.array_equal(bits(c.out), bits(a.out[torch.from_numpy(idx).cuda()]))
    for j, n in enumerate(perm):
        assert np.array_equal(bits(c.Sd[int(c.final[j])]), bits(a.Sd[int(a.final[n])]))


def test_prefill_invalid_slot_gives_nan_and_writes_nothing():
    shape = wl.LayerShape(2, 64, 64)
    lengths = [70, 20]
    inp = wl.token_inputs(33, shape, sum(lengths))
    run = Run(shape, inp, lengths)
    run.init = np.array([-1, 999], np.int32)
    before = bits(run.Sd[int(run.final[1])])
    run.launch()
    out = host(run.out)
    assert np.isfinite(out[:70]).all() and np.isnan(out[70:]).all()
    # sequence 0 wrote its final slot; sequence 1 (invalid init) wrote nothing
    assert np.array_equal(bits(run.Sd[int(run.final[1])]), before)
    assert np.isfinite(host(run.Sd)[int(run.final[0])]).all()


def test_prefill_4x8192_full_size():
    """The chunked prefill workload at full size (4 x 8192 tokens, H=32,
    dk=dv=128, bf16, zero initial state): outputs and final states on sampled
    heads against the oracle, and every head against the decode kernel stepped
    token by token (the GPU recurrent path)."""
    w = wl.WORKLOADS["prefill_4x8k"]
    shape, lengths = w["shape"], w["lengths"]
    say(f"prefill full size: lengths={lengths} H={shape.H}")
    inp = wl.token_inputs(w["seed"], shape, sum(lengths))
    run = Run(shape, inp, lengths).launch()
    heads = [0, 17, 31]
    r = oracle_for(run, heads=heads)
    check_against_oracle(run, r, heads=heads)
    # recurrent path: the decode kernel, one launch per token position, B = 4
    cfg = run.cfg
    N, T, H, dv = len(lengths), lengths[0], shape.H, shape.dv
    Sp = torch.zeros((N, H, shape.dk, dv), device="cuda")
    Xp = torch.zeros((N, H, shape.C, 3), dtype=cfg.torch_act, device="cuda")
    slot = torch.arange(N, dtype=torch.int32, device="cuda")
    rec = torch.empty((T, N, H, dv), dtype=cfg.torch_act, device="cuda")
    seqmaj = lambda t: t.view((N, T) + t.shape[1:]).transpose(0, 1).contiguous()
    q, k, v, z, g, beta = (seqmaj(t) for t in (run.q, run.k, run.v, run.z, run.g, run.beta))
    for t in range(T):
        kda.kda_decode_step(cfg, q[t], k[t], v[t], z[t], g[t], beta[t], run.conv_w, run.norm_w, Sp, Xp,
                            slot, rec[t])
    torch.cuda.synchronize()
    e_rec = rel_l2(host(rec.transpose(0, 1).reshape(N * T, H, dv)), host(run.out))
    e_rec_s = rel_l2(host(Sp), run.final_state()[0])
    say(f"  vs decode-kernel recurrence: out {e_rec:.3e}  state {e_rec_s:.3e}")
    assert e_rec <= 1e-2 and e_rec_s <= 5e-3
