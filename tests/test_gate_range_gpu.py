"""GPU parity of the chunked prefill over the whole gate domain g <= 0.

The recurrence multiplies the state by Diag(exp g_t) for any log-decay
g_t <= 0, including g = -inf (the channel forgets everything).  Inside a
chunk the prefill forms the pairwise decays exp(Gam_t - Gam_s) either through
the chunk's middle row (when every channel's decay over each half of the chunk
stays above -80) or from sums over 16-row blocks (any other chunk).  These
tests drive both forms with strong gates and compare against the fp64 oracle
(whole tensor, per chain, per output row), in the one-workgroup, paired and
split launches, for bf16 and fp32 activations, and check that no NaN or inf
appears:

  g_x4        the workloads' gate times 4 (mean about -3.3 per token: nearly
              every chunk leaves the middle-row range)
  minus20     g = -20 on a tenth of the (head, channel) pairs, for all tokens
  minus_inf   g = -inf at 3% of the (token, head, channel) entries and on
              every channel of a few whole tokens
  at_bound    per-chunk decays placed at the middle-row range's edge: a chunk
              whose first half sums to exactly -80 on some channels (block
              path), one at -79.68 (middle-row path, factors up to e^79.7),
              one mixing -inf and -2.4, then ordinary chunks

[vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
"KDA prefill and decode": the chunked prefill runs the same recurrence as the
decode, whose per-channel decay gate may take any value g <= 0.]
"""
import numpy as np
import pytest

import linear_attention_recurrence_decode_amd as kda
import workloads as wl
from tests.helpers import bits, host, say
from tests.prefill_runner import Run, check_against_oracle, oracle_for, resume_and_finish, states_for

pytestmark = pytest.mark.gpu

PAIRED, SPLIT = kda.KDA_PREFILL_PAIRED, kda.KDA_PREFILL_SPLIT
MODES = {"one_workgroup": 0, "paired": PAIRED, "split": SPLIT}


def strong_gate_inputs(kind: str, seed: int, shape, lengths):
    """Seeded inputs with the gate of `kind` (see the module docstring)."""
    T = sum(lengths)
    inp = wl.token_inputs(seed, shape, T, g_scale=4.0 if kind == "g_x4" else 1.0, norm_w="random")
    g = inp.g
    rng = np.random.default_rng([seed, 99, 0])
    if kind == "minus20":
        sel = rng.random((shape.H, shape.dk)) < 0.1
        g[:, sel] = -20.0
    elif kind == "minus_inf":
        g[rng.random(g.shape) < 0.03] = -np.inf
        for t in (5, 70, 200, T - 1):
            if t < T:
                g[t, 0, :] = -np.inf
    elif kind == "at_bound":
        # per-chunk patterns on the first sequence (chunks aligned to its start)
        sel = rng.random((shape.H, shape.dk)) < 0.25
        pats = [np.float32(-2.5), np.float32(-2.49), None]
        for c, v in enumerate(pats):
            lo, hi = 64 * c, min(64 * c + 64, lengths[0])
            if lo >= hi:
                break
            blk = g[lo:hi]
            if v is None:
                blk[:, sel] = -2.4
                blk[10, sel] = -np.inf
            else:
                blk[:, sel] = v
    else:
        assert kind == "g_x4"
    return inp


KINDS = ["g_x4", "minus20", "minus_inf", "at_bound"]
SHAPES = {
    "bf16_d128": wl.LayerShape(3, 128, 128),
    "f32_d64": wl.LayerShape(2, 64, 64, act="f32"),
}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape_name", list(SHAPES))
@pytest.mark.parametrize("kind", KINDS)
def test_strong_gates_match_oracle(kind, shape_name, mode):
    shape = SHAPES[shape_name]
    lengths, starts = [300, 129, 64, 7], [0, 64, 30, 0]
    seed = 70 + KINDS.index(kind)
    say(f"gate case {kind} {shape_name} {mode}: lengths={lengths} starts={starts}")
    inp = strong_gate_inputs(kind, seed, shape, lengths)
    S0, X0 = states_for(seed, shape, len(lengths))
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=MODES[mode]).launch()
    check_against_oracle(run, oracle_for(run, S0, X0))
    assert np.isfinite(host(run.ckS[:run.nck])).all()


@pytest.mark.parametrize("kind", KINDS)
def test_strong_gates_paired_equals_one_workgroup(kind):
    """The paired launch reproduces the one-workgroup launch bit for bit on
    both decay paths (their arithmetic is the same code)."""
    shape = SHAPES["bf16_d128"]
    lengths, starts = [300, 129, 64, 7], [0, 64, 30, 0]
    seed = 70 + KINDS.index(kind)
    inp = strong_gate_inputs(kind, seed, shape, lengths)
    S0, X0 = states_for(seed, shape, len(lengths))
    a = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=PAIRED).launch()
    b = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128).launch()
    for x, y in ((a.out, b.out), (a.Sd, b.Sd), (a.Xd, b.Xd), (a.ckS[:a.nck], b.ckS[:b.nck])):
        assert np.array_equal(bits(x), bits(y))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_strong_gates_resume_is_bitwise_identical(act):
    """Resume at interval checkpoints inside chains whose chunks alternate
    between the two decay paths reproduces the straight run bit for bit."""
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [640, 384], [0, 128]
    inp = wl.token_inputs(80, shape, sum(lengths), norm_w="random")
    # odd chunks of each sequence (by absolute position) strongly gated
    pos = np.concatenate([np.arange(s, s + L) for s, L in zip(starts, lengths)])
    strong = (pos // 64) % 2 == 1
    inp.g[strong] *= 6.0
    inp.g[pos % 97 == 0, :, :3] = -np.inf
    S0, X0 = states_for(80, shape, len(lengths))
    straight = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128).launch()
    check_against_oracle(straight, oracle_for(straight, S0, X0))
    resumed, seqs, res_pos, src_ck, idx = resume_and_finish(straight, [2, 1])
    say(f"  resumed {seqs} at {res_pos}")
    assert np.array_equal(bits(resumed.out), bits(straight.out[idx]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))


@pytest.mark.parametrize("d", [32, 64])
def test_strong_gates_small_heads(d):
    """Head sizes 32 and 64 (fewer waves per chain) under -inf and x4 gates."""
    shape = wl.LayerShape(2, d, d)
    lengths, starts = [200, 77], [0, 5]
    inp = strong_gate_inputs("minus_inf", 90 + d, shape, lengths)
    inp.g *= 4.0
    S0, X0 = states_for(90 + d, shape, len(lengths))
    run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0).launch()
    check_against_oracle(run, oracle_for(run, S0, X0))
