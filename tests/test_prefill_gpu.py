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
from tests.helpers import TOL_STATE_PER_CHAIN, bits, dev, host, per_chain_max, rel_l2, say, tols

pytestmark = pytest.mark.gpu


def cfg_for(shape):
    return kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16 if shape.act == "bf16" else kda.KDA_F32)


class Run:
    """One prefill call on the GPU with pools, slots and checkpoint buffers."""

    def __init__(self, shape, inp, lengths, *, starts=None, S0=None, X0=None, interval=0,
                 pool_extra=3, seq_order=None):
        self.shape, self.inp = shape, inp
        H, dk, dv, C = shape.H, shape.dk, shape.dv, shape.C
        N = len(lengths)
        self.N, self.lengths = N, list(lengths)
        self.starts = [0] * N if starts is None else list(starts)
        self.cfg = cfg_for(shape)
        act = self.cfg.torch_act
        cu = wl.cu_seqlens(lengths)
        self.cu = cu
        nslots = 2 * N + pool_extra
        S = np.zeros((nslots, H, dk, dv), np.float32)
        X = np.zeros((nslots, H, C, 3), np.float32)
        init = np.full(N, -1, np.int32)
        if S0 is not None:
            init = np.arange(N, dtype=np.int32)
            S[:N] = S0
            X[:N] = X0
        final = np.arange(N, 2 * N, dtype=np.int32)
        self.init, self.final = init, final
        self.Sd, self.Xd = dev(S), dev(X, act)
        counts = [oracle.num_checkpoints(s, L, interval) for s, L in zip(self.starts, lengths)]
        base = np.zeros(N, np.int32)
        if N:
            base[1:] = np.cumsum(counts)[:-1]
        self.base, self.nck = base, int(sum(counts))
        self.interval = interval
        self.ckS = torch.full((max(self.nck, 1), H, dk, dv), float("nan"), device="cuda")
        self.ckX = torch.zeros((max(self.nck, 1), H, C, 3), dtype=act, device="cuda")
        T = int(cu[-1])
        self.q, self.k, self.v, self.z = (dev(a, act) for a in (inp.q, inp.k, inp.v, inp.z))
        self.g, self.beta = dev(inp.g), dev(inp.beta)
        self.conv_w, self.norm_w = dev(inp.conv_w), dev(inp.norm_w)
        self.out = torch.full((T, H, dv), float("nan"), dtype=act, device="cuda")
        nbytes = kda.kda_prefill_workspace_bytes(self.cfg, N, T)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def launch(self):
        kda.kda_prefill_varlen(self.cfg, dev(self.cu.astype(np.int32)), self.q, self.k, self.v, self.z,
                               self.g, self.beta, self.conv_w, self.norm_w, self.Sd, self.Xd,
                               dev(self.init), dev(self.final), self.out, self.ws,
                               start_pos=dev(np.asarray(self.starts, np.int64)),
                               ckpt_interval=self.interval,
                               ckpt_state=self.ckS if self.interval else None,
                               ckpt_conv=self.ckX if self.interval else None,
                               ckpt_base=dev(self.base) if self.interval else None)
        torch.cuda.synchronize()
        return self

    def final_state(self):
        return host(self.Sd)[self.final], host(self.Xd)[self.final]


def oracle_for(run, S0=None, X0=None, heads=None):
    inp = run.inp
    sl = (slice(None),) if heads is None else (slice(None), heads)
    hs = slice(None) if heads is None else heads
    return oracle.run(inp.q[sl], inp.k[sl], inp.v[sl], inp.z[sl], inp.g[sl], inp.beta[sl],
                      inp.conv_w[hs], inp.norm_w, run.cu, start_pos=run.starts,
                      S0=None if S0 is None else S0[:, hs], X0=None if X0 is None else X0[:, hs],
                      ckpt_interval=run.interval)


def states_for(seed, shape, N, scale=0.3):
    S, X = wl.states(seed + 100, shape, N, state_std=scale, conv_std=1.0)
    return S, X


def check_against_oracle(run, r, heads=None):
    tol_o, tol_s = tols(run.shape.act)
    hs = slice(None) if heads is None else heads
    out = host(run.out)[:, hs]
    Sf, Xf = run.final_state()
    e_out = rel_l2(out, r.out)
    e_s = rel_l2(Sf[:, hs], r.S)
    e_c = per_chain_max(Sf[:, hs], r.S)
    say(f"  rel-L2 out {e_out:.3e} (tol {tol_o})  state {e_s:.3e} (tol {tol_s})  worst chain {e_c:.3e}")
    assert np.isfinite(out).all()
    assert e_out <= tol_o and e_s <= tol_s and e_c <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(Xf[:, hs], r.X)
    return e_out, e_s


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
    # resume sequence n from its j-th checkpoint (an interval boundary, not the end)
    picks = [1, 0, 1]
    cfg = straight.cfg
    res_pos, src_ck = [], []
    for n in range(N):
        ps = [p for p in range(starts[n] + 1, starts[n] + lengths[n] + 1)
              if p % 128 == 0 or p == starts[n] + lengths[n]]
        res_pos.append(ps[picks[n]])
        src_ck.append(int(straight.base[n]) + picks[n])
    # second batch: the remainders, packed, starting at the resume positions
    rem = [starts[n] + lengths[n] - res_pos[n] for n in range(N)]
    offs = [int(straight.cu[n]) + (res_pos[n] - starts[n]) for n in range(N)]
    idx = np.concatenate([np.arange(o, o + r) for o, r in zip(offs, rem)])
    sub = wl.Inputs(shape, inp.q[idx], inp.k[idx], inp.v[idx], inp.z[idx], inp.g[idx], inp.beta[idx],
                    inp.conv_w, inp.norm_w)
    resumed = Run(shape, sub, rem, starts=res_pos, interval=128)
    # seed its initial slots from the straight run's checkpoints
    resumed.init = np.arange(N, dtype=np.int32)
    kda.kda_resume(cfg, straight.ckS, straight.ckX, dev(np.asarray(src_ck, np.int32)),
                   resumed.Sd, resumed.Xd, dev(resumed.init))
    ck_before = bits(straight.ckS)
    resumed.launch()
    assert np.array_equal(bits(straight.ckS), ck_before)          # copy-on-write source untouched
    out_s = bits(straight.out[torch.from_numpy(idx).cuda()])
    assert np.array_equal(bits(resumed.out), out_s)
    for n in range(N):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[n])]), bits(straight.Sd[int(straight.final[n])]))
        assert np.array_equal(bits(resumed.Xd[int(resumed.final[n])]), bits(straight.Xd[int(straight.final[n])]))
        later = oracle.num_checkpoints(res_pos[n], rem[n], 128)
        for j in range(later):
            a = resumed.ckS[int(resumed.base[n]) + j]
            b = straight.ckS[src_ck[n] + 1 + j]
            assert np.array_equal(bits(a), bits(b))


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
