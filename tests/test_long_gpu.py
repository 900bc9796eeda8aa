"""Full-size GPU runs of the varlen-with-checkpoints workload and the
1M-token long-context workload.

Varlen: 16 sequences with lengths floor(exp(U(ln 1K, ln 64K))) (about 248K
tokens), H=32, dk=dv=128, bf16, checkpoints every 4096 tokens and at sequence
ends.  Outputs, final states and checkpoints are compared with the oracle on
sampled heads; every sequence with an interval checkpoint is then resumed from
a seeded one and finished, and must match the straight run bit for bit.  The
scheduled launch (KDA_PREFILL_PAIRED) of the same batch must equal the
one-workgroup run bit for bit.

Long context: one sequence of 1,048,576 tokens, H=8, checkpoints every 32K.
The oracle checks the first 64K tokens (outputs and the checkpoints there)
and, started from the run's own checkpoint at 1,015,808, the last 32K tokens
of two heads and the final state;
a resume from the checkpoint at 512K must reproduce the second half bit for
bit; the end state is fanned out to 256 decode slots by copy-on-write resume
and advanced 512 decode steps, checked on sampled slots against the oracle
started from the same checkpoint.  The same sequence split at its
checkpoints (KDA_PREFILL_SPLIT) must agree with the unsplit run to fp32
rounding, match the oracle on the first 64K and the last 32K tokens and resume
bit for bit; with its chains paired (KDA_PREFILL_PAIRED) it must equal the
unsplit run bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import (TOL_STATE_PER_CHAIN, bits, dev, host, per_chain_max, per_row_max, rel_l2, say,
                           tol_row, tols)
from tests.prefill_runner import Run, checkpoint_positions, resume_and_finish

PAIRED = kda.KDA_PREFILL_PAIRED


def same_bits_on_device(a, b):
    """Every output, final state, conv state and checkpoint of two runs of
    the same call equal bit for bit (compared on the device)."""
    eq = lambda x, y: torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))
    assert eq(a.out, b.out) and eq(a.Sd, b.Sd) and eq(a.Xd, b.Xd)
    if a.interval:
        assert a.nck == b.nck
        assert eq(a.ckS[:a.nck], b.ckS[:b.nck]) and eq(a.ckX[:a.nck], b.ckX[:b.nck])

pytestmark = pytest.mark.gpu


def test_varlen_checkpoints_and_resume_full_size():
    w = wl.WORKLOADS["varlen_ckpt"]
    shape, N, interval = w["shape"], w["n"], w["interval"]
    lengths = [int(x) for x in wl.loguniform_lengths(w["seed"], N, w["lo"], w["hi"])]
    say(f"varlen full size: {N} sequences, {sum(lengths)} tokens, lengths {lengths}")
    inp = wl.token_inputs(w["seed"], shape, sum(lengths))
    straight = Run(shape, inp, lengths, interval=interval).launch()
    say(f"  prefill done, {straight.nck} checkpoints")
    heads = [5, 27]
    r = oracle.run(inp.q[:, heads], inp.k[:, heads], inp.v[:, heads], inp.z[:, heads], inp.g[:, heads],
                   inp.beta[:, heads], inp.conv_w[heads], inp.norm_w, straight.cu, ckpt_interval=interval)
    tol_o, tol_s = tols("bf16")
    e_out = rel_l2(host(straight.out)[:, heads], r.out)
    Sf, Xf = straight.final_state()
    e_s = rel_l2(Sf[:, heads], r.S)
    e_c = per_chain_max(Sf[:, heads], r.S)
    ck = host(straight.ckS)[:straight.nck][:, heads]
    e_ck = rel_l2(ck, r.ckpt_S)
    e_ckc = per_chain_max(ck, r.ckpt_S)
    e_row = per_row_max(host(straight.out)[:, heads], r.out)
    say(f"  sampled heads {heads}: out {e_out:.3e} (worst row {e_row:.3e}) state {e_s:.3e} (worst chain {e_c:.3e}) "
        f"checkpoints {e_ck:.3e} (worst {e_ckc:.3e})")
    assert e_out <= tol_o and e_s <= tol_s and e_c <= TOL_STATE_PER_CHAIN and e_row <= tol_row("bf16")
    assert e_ck <= tol_s and e_ckc <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(Xf[:, heads], r.X)
    np.testing.assert_array_equal(host(straight.ckX)[:straight.nck][:, heads], r.ckpt_X)
    # the scheduled launch (pairs for the longest chains, the rest queued)
    # gives the one-workgroup run's bits at full size
    paired = Run(shape, inp, lengths, interval=interval, flags=PAIRED).launch()
    same_bits_on_device(paired, straight)
    assert kda.prefill_status(paired.ws) == 0
    say("  scheduled (paired) launch: bitwise equal")
    del paired
    # resume every sequence that has an interval checkpoint from a seeded one
    rng = np.random.default_rng([w["seed"], wl.TID["resume"], 0])
    picks = []
    for n, L in enumerate(lengths):
        n_int = len(checkpoint_positions(0, L, interval)) - 1      # interval checkpoints (not the end)
        picks.append(int(rng.integers(0, n_int)) if n_int > 0 else None)
    resumed, seqs, res_pos, src_ck, idx = resume_and_finish(straight, picks)
    say(f"  resumed {len(seqs)} sequences at {res_pos}")
    assert np.array_equal(bits(resumed.out), bits(straight.out[torch.from_numpy(idx).cuda()]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))
        assert np.array_equal(bits(resumed.Xd[int(resumed.final[j])]), bits(straight.Xd[int(straight.final[n])]))
        later = oracle.num_checkpoints(res_pos[j], resumed.lengths[j], interval)
        assert np.array_equal(bits(resumed.ckS[int(resumed.base[j]):int(resumed.base[j]) + later]),
                              bits(straight.ckS[src_ck[j] + 1:src_ck[j] + 1 + later]))


@functools.lru_cache(maxsize=1)
def long_inputs():
    w = wl.WORKLOADS["long_1m"]
    return wl.token_inputs(w["seed"], w["shape"], w["lengths"][0])


@functools.lru_cache(maxsize=1)
def long_unsplit_run():
    w = wl.WORKLOADS["long_1m"]
    return Run(w["shape"], long_inputs(), [w["lengths"][0]], interval=w["interval"]).launch()


def check_tail_against_oracle(run, inp, interval):
    """The oracle on the last checkpoint interval (32K tokens) of two sampled
    heads, started from the run's own checkpoint at its start (state and conv
    state): the outputs of those tokens and the final state."""
    L = inp.T
    P, hs = L - interval, [1, 6]
    j = P // interval - 1                      # checkpoint slot of position P
    S0 = host(run.ckS[j:j + 1])[:, hs]
    X0 = host(run.ckX[j:j + 1])[:, hs]
    r = oracle.run(inp.q[P:, hs], inp.k[P:, hs], inp.v[P:, hs], inp.z[P:, hs], inp.g[P:, hs], inp.beta[P:, hs],
                   inp.conv_w[hs], inp.norm_w, [0, L - P], start_pos=[P], S0=S0, X0=X0)
    out = host(run.out[P:])[:, hs]
    e_out, e_row = rel_l2(out, r.out), per_row_max(out, r.out)
    Sf, Xf = run.final_state()
    e_s, e_c = rel_l2(Sf[:, hs], r.S), per_chain_max(Sf[:, hs], r.S)
    say(f"  last {L - P} tokens from the checkpoint at {P}, heads {hs}: out {e_out:.3e} (worst row {e_row:.3e}), "
        f"final state {e_s:.3e} (worst head {e_c:.3e})")
    assert e_out <= 1e-2 and e_row <= tol_row("bf16") and e_s <= 5e-3 and e_c <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(Xf[:, hs], r.X)


def check_prefix_against_oracle(run, inp, interval):
    """The oracle on the first 64K tokens of one sampled head: outputs and the
    checkpoints at 32K and 64K."""
    P, hs = 65536, [3]
    r = oracle.run(inp.q[:P, hs], inp.k[:P, hs], inp.v[:P, hs], inp.z[:P, hs], inp.g[:P, hs], inp.beta[:P, hs],
                   inp.conv_w[hs], inp.norm_w, [0, P], ckpt_interval=interval)
    e_out = rel_l2(host(run.out[:P])[:, hs], r.out)
    ck = host(run.ckS[:2])[:, hs]
    e_ck = rel_l2(ck, r.ckpt_S[:2])
    say(f"  first {P} tokens, head {hs}: out {e_out:.3e}, checkpoints at 32K/64K {e_ck:.3e}")
    assert e_out <= 1e-2 and e_ck <= 5e-3 and per_chain_max(ck, r.ckpt_S[:2]) <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(host(run.ckX[:2])[:, hs], r.ckpt_X[:2])


def test_long_context_1m_full_size():
    w = wl.WORKLOADS["long_1m"]
    shape, L, interval = w["shape"], w["lengths"][0], w["interval"]
    say(f"long context: {L} tokens, H={shape.H}, checkpoints every {interval}")
    inp = long_inputs()
    straight = long_unsplit_run()
    say(f"  prefill done, {straight.nck} checkpoints")
    assert straight.nck == L // interval
    assert torch.isfinite(straight.out.float()).all()
    check_prefix_against_oracle(straight, inp, interval)
    check_tail_against_oracle(straight, inp, interval)
    # resume from the checkpoint at 512K: the second half is reproduced bit for bit
    j = L // 2 // interval - 1
    resumed, _, res_pos, _, idx = resume_and_finish(straight, [j])
    assert res_pos == [L // 2]
    assert np.array_equal(bits(resumed.out), bits(straight.out[L // 2:]))
    assert np.array_equal(bits(resumed.Sd[int(resumed.final[0])]), bits(straight.Sd[int(straight.final[0])]))
    say("  resume from 512K: bitwise identical")
    # fan the end state out to 256 decode slots and run 512 decode steps
    B, steps = w["decode_B"], w["decode_steps"]
    cfg = straight.cfg
    Sp = torch.zeros((B, shape.H, shape.dk, shape.dv), device="cuda")
    Xp = torch.zeros((B, shape.H, shape.C, 3), dtype=cfg.torch_act, device="cuda")
    last = straight.nck - 1
    kda.kda_resume(cfg, straight.ckS, straight.ckX, dev(np.full(B, last, np.int32)), Sp, Xp,
                   dev(np.arange(B, dtype=np.int32)))
    dinp = wl.token_inputs(w["seed"] + 100, shape, B * steps)
    rs = lambda a: a.reshape((steps, B) + a.shape[1:])
    q, k, v, z = (dev(rs(a), cfg.torch_act) for a in (dinp.q, dinp.k, dinp.v, dinp.z))
    g, beta = dev(rs(dinp.g)), dev(rs(dinp.beta))
    cw, nw = dev(inp.conv_w), dev(inp.norm_w)
    slot = dev(np.arange(B, dtype=np.int32))
    dout = torch.empty((steps, B, shape.H, shape.dv), dtype=cfg.torch_act, device="cuda")
    for s in range(steps):
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], cw, nw, Sp, Xp, slot, dout[s])
    torch.cuda.synchronize()
    pick = [0, 37, 128, 255]
    S0 = np.repeat(host(straight.ckS[last:last + 1]), len(pick), axis=0)
    X0 = np.repeat(host(straight.ckX[last:last + 1]), len(pick), axis=0)
    sub = lambda a: rs(a)[:, pick]
    o_ref, S_ref, X_ref = oracle.decode_steps(sub(dinp.q), sub(dinp.k), sub(dinp.v), sub(dinp.z), sub(dinp.g),
                                              sub(dinp.beta), inp.conv_w, inp.norm_w, S0, X0)
    e_o = rel_l2(host(dout)[:, pick], o_ref)
    e_s = rel_l2(host(Sp)[pick], S_ref)
    e_c = per_chain_max(host(Sp)[pick], S_ref)
    say(f"  decode fan-out, slots {pick}: out {e_o:.3e} state {e_s:.3e} (worst chain {e_c:.3e})")
    assert e_o <= 1e-2 and e_s <= 5e-3 and e_c <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(host(Xp)[pick], X_ref)


def test_long_context_1m_split():
    """The 1M-token sequence cut at its 32 checkpoints (segments in parallel,
    joined by the scan of their transitions)."""
    w = wl.WORKLOADS["long_1m"]
    shape, L, interval = w["shape"], w["lengths"][0], w["interval"]
    say(f"long context split: {L} tokens, H={shape.H}, segments of {interval}")
    inp = long_inputs()
    split = Run(shape, inp, [L], interval=interval, flags=kda.KDA_PREFILL_SPLIT).launch()
    assert split.nck == L // interval
    assert torch.isfinite(split.out.float()).all()
    check_prefix_against_oracle(split, inp, interval)
    check_tail_against_oracle(split, inp, interval)
    ref = long_unsplit_run()
    # (on this workload the two agree exactly: its gate, about -0.8 per token,
    # takes any state below fp32 resolution within a few chunks, so every
    # segment's transition F is exactly zero and F S + G equals the
    # sequential state bit for bit; the small split tests see the rounding)
    e_o = rel_l2(host(split.out[::97]), host(ref.out[::97]))
    e_k = per_chain_max(host(split.ckS), host(ref.ckS))
    say(f"  split vs unsplit: out (every 97th token) {e_o:.3e}, worst checkpoint chain {e_k:.3e}")
    assert e_o <= 2e-3 and e_k <= 1e-5
    np.testing.assert_array_equal(bits(split.ckX), bits(ref.ckX))
    j = L // 2 // interval - 1
    resumed, _, res_pos, _, idx = resume_and_finish(split, [j])
    assert res_pos == [L // 2]
    assert np.array_equal(bits(resumed.out), bits(split.out[L // 2:]))
    assert np.array_equal(bits(resumed.Sd[int(resumed.final[0])]), bits(split.Sd[int(split.final[0])]))
    assert np.array_equal(bits(resumed.ckS[:resumed.nck]), bits(split.ckS[j + 1:]))
    say("  split resume from 512K: bitwise identical")


def test_long_context_1m_paired():
    """The 1M-token sequence with its 8 chains paired (KDA_PREFILL_PAIRED):
    bitwise equal to the one-workgroup run, and the oracle on its last
    interval from its own checkpoint."""
    w = wl.WORKLOADS["long_1m"]
    shape, L, interval = w["shape"], w["lengths"][0], w["interval"]
    say(f"long context paired: {L} tokens, H={shape.H}")
    inp = long_inputs()
    paired = Run(shape, inp, [L], interval=interval, flags=PAIRED).launch()
    assert kda.prefill_status(paired.ws) == 0
    same_bits_on_device(paired, long_unsplit_run())
    say("  paired vs one workgroup: bitwise equal")
    check_tail_against_oracle(paired, inp, interval)
