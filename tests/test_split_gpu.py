"""GPU tests of the prefill with sequences split at checkpoint positions
(KDA_PREFILL_SPLIT): parity with the oracle, agreement with the unsplit run,
bit-identical resume from interval checkpoints, in-place slots, determinism
and the invalid-slot path.

Split mode forms the state at every interval position inside a sequence as
F S + G from the segment transitions, so it agrees with the unsplit run to
fp32 rounding, not bit for bit; bit-identity holds between split runs.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import TOL_STATE_PER_CHAIN, bits, host, per_chain_max, rel_l2, say, tols
from tests.prefill_runner import Run, check_against_oracle, oracle_for, resume_and_finish, states_for

pytestmark = pytest.mark.gpu

SPLIT = kda.KDA_PREFILL_SPLIT

CASES = {
    # name: (seed, shape, lengths, starts, interval, g_scale)
    "bf16_d128": (40, wl.LayerShape(2, 128, 128), [700, 1, 0, 450, 129, 64], [0, 5, 3, 70, 128, 1000], 128, 0.1),
    "bf16_d64_nodecay": (41, wl.LayerShape(3, 64, 64), [520, 63, 300], [64, 0, 127], 128, 0.0),
    "f32_d64": (42, wl.LayerShape(2, 64, 64, act="f32"), [640, 200, 2], [0, 191, 255], 64, 0.05),
    "f32_d32": (43, wl.LayerShape(2, 32, 32, act="f32"), [1000, 130], [3, 0], 192, 0.2),
}


def check_checkpoints(run, r):
    _, tol_s = tols(run.shape.act)
    assert run.nck == len(r.ckpt_S) and list(run.base) == list(r.ckpt_base)
    ckS = host(run.ckS)[:run.nck]
    e = rel_l2(ckS, r.ckpt_S)
    e_c = per_chain_max(ckS, r.ckpt_S)
    say(f"  checkpoints: {run.nck}, rel-L2 {e:.3e} (worst chain {e_c:.3e})")
    assert e <= tol_s and e_c <= TOL_STATE_PER_CHAIN
    np.testing.assert_array_equal(host(run.ckX)[:run.nck], r.ckpt_X)


@pytest.mark.parametrize("name", list(CASES))
def test_split_matches_oracle(name):
    seed, shape, lengths, starts, interval, g_scale = CASES[name]
    say(f"split case {name}: H={shape.H} d={shape.dk} act={shape.act} lengths={lengths} starts={starts} "
        f"interval={interval}")
    inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=g_scale, norm_w="random")
    S0, X0 = states_for(seed, shape, len(lengths))
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=SPLIT).launch()
    r = oracle_for(run, S0, X0)
    check_against_oracle(run, r)
    check_checkpoints(run, r)
    # a sequence's last checkpoint is its final state
    for n, L in enumerate(lengths):
        if L:
            last = run.base[n] + oracle.num_checkpoints(starts[n], L, interval) - 1
            assert np.array_equal(bits(run.ckS[last]), bits(run.Sd[int(run.final[n])]))


@pytest.mark.parametrize("name", ["bf16_d128", "f32_d64"])
def test_split_agrees_with_unsplit(name):
    seed, shape, lengths, starts, interval, g_scale = CASES[name]
    inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=g_scale, norm_w="random")
    S0, X0 = states_for(seed, shape, len(lengths))
    a = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval).launch()
    b = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=SPLIT).launch()
    e_o = rel_l2(host(b.out), host(a.out))
    e_s = per_chain_max(b.final_state()[0], a.final_state()[0])
    e_k = per_chain_max(host(b.ckS)[:b.nck], host(a.ckS)[:a.nck])
    say(f"  split vs unsplit: out {e_o:.3e}, worst final chain {e_s:.3e}, worst checkpoint {e_k:.3e}")
    # fp32 rounding of the scan; bf16 outputs may differ by one rounding step
    assert e_o <= (2e-3 if shape.act == "bf16" else 1e-5)
    assert e_s <= 1e-5 and e_k <= 1e-5
    np.testing.assert_array_equal(bits(b.ckX), bits(a.ckX))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_split_resume_is_bitwise_identical(act):
    """Resume from interval checkpoints of a split run, split again: outputs
    from the resume point, later checkpoints and final states are identical."""
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [700, 450, 300], [0, 128, 64]
    inp = wl.token_inputs(44, shape, sum(lengths), g_scale=0.05, norm_w="random")
    S0, X0 = states_for(44, shape, len(lengths))
    straight = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=SPLIT).launch()
    ck_before = bits(straight.ckS)
    resumed, seqs, res_pos, src_ck, idx = resume_and_finish(straight, [2, 0, 1])
    say(f"  resumed at {res_pos}")
    assert np.array_equal(bits(straight.ckS), ck_before)
    assert np.array_equal(bits(resumed.out), bits(straight.out[torch.from_numpy(idx).cuda()]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))
        assert np.array_equal(bits(resumed.Xd[int(resumed.final[j])]), bits(straight.Xd[int(straight.final[n])]))
        later = oracle.num_checkpoints(res_pos[j], resumed.lengths[j], 128)
        assert np.array_equal(bits(resumed.ckS[int(resumed.base[j]):int(resumed.base[j]) + later]),
                              bits(straight.ckS[src_ck[j] + 1:src_ck[j] + 1 + later]))


def test_split_in_place_and_deterministic():
    """Final slot == initial slot gives the same bits as distinct slots, and
    two identical split calls give identical bits."""
    seed, shape, lengths, starts, interval, g_scale = CASES["bf16_d128"]
    inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=g_scale, norm_w="random")
    S0, X0 = states_for(seed, shape, len(lengths))
    a = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=SPLIT).launch()
    b = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=SPLIT).launch()
    assert np.array_equal(bits(a.out), bits(b.out)) and np.array_equal(bits(a.ckS), bits(b.ckS))
    c = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=SPLIT)
    c.final = c.init.copy()
    c.launch()
    assert np.array_equal(bits(c.out), bits(a.out)) and np.array_equal(bits(c.ckS), bits(a.ckS))
    for n in range(len(lengths)):
        assert np.array_equal(bits(c.Sd[int(c.init[n])]), bits(a.Sd[int(a.final[n])]))
        assert np.array_equal(bits(c.Xd[int(c.init[n])]), bits(a.Xd[int(a.final[n])]))


def test_split_invalid_slot_gives_nan_and_writes_nothing():
    shape = wl.LayerShape(2, 64, 64)
    lengths = [300, 260]
    inp = wl.token_inputs(45, shape, sum(lengths))
    run = Run(shape, inp, lengths, interval=64, flags=SPLIT)
    run.init = np.array([-1, 999], np.int32)
    before = bits(run.Sd[int(run.final[1])])
    run.launch()
    out = host(run.out)
    assert np.isfinite(out[:300]).all() and np.isnan(out[300:]).all()
    assert np.array_equal(bits(run.Sd[int(run.final[1])]), before)
    ck1 = slice(int(run.base[1]), run.nck)
    assert torch.isnan(run.ckS[ck1]).all()                  # no checkpoint of sequence 1 was written
    r = oracle_for(run, None, None)
    e = rel_l2(out[:300], r.out[:300])
    say(f"  valid sequence: out rel-L2 {e:.3e}")
    assert e <= tols("bf16")[0]
