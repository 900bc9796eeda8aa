"""Seeded random sweeps of small prefill and decode calls against the fp64 oracle.

Each case draws its own head size (32, 64, 128), activation dtype (fp32 at
d <= 64), head count, packed sequences (empty, one to three tokens, one
chunk and a token either side of it, or up to 420 tokens), absolute start
positions (aligned and unaligned), initial states, gate strength (none,
weak, the workloads' own, and strong enough to send chunks to the
block-local decay path), checkpoint interval, state storage dtype and
launch mode (one workgroup per chain, paired, split at checkpoints).  The
draws are fixed by the sweep's seed, so the list of cases never changes.

Checks, per case: outputs, final states and every checkpoint against the
oracle (the parity bars of the other prefill tests; bf16-stored states to
the bf16-state bars), conv states and conv checkpoints exactly, and for the
paired launch the one-workgroup launch's results bit for bit.  The decode
sweep draws head size, dtypes, batch, tokens per launch (1 to 8), pool size
and gate strength, checks T single-token steps against the oracle and one
T-token launch against those steps bit for bit.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.test_decode_multi_gpu import multi, setup, single_steps
from tests.helpers import TOL_STATE_PER_CHAIN, bits, host, per_chain_max, per_row_max, rel_l2, say, tol_row, tols
from tests.prefill_runner import Run, oracle_for, states_for

pytestmark = pytest.mark.gpu

SWEEP_SEED = 20261203
N_CASES = 96
# bf16-stored states: the bars of the bf16-state tests
TOL_BF16_STATE_OUT, TOL_BF16_STATE, TOL_BF16_STATE_CHAIN = 1e-2, 5e-3, 2e-3


def draw_case(i):
    rng = np.random.default_rng([SWEEP_SEED, i])
    d = int(rng.choice([32, 64, 128]))
    act = "f32" if d <= 64 and rng.random() < 0.5 else "bf16"
    H = int(rng.integers(1, 4))
    while True:
        N = int(rng.integers(1, 6))
        lengths = []
        for _ in range(N):
            kind = rng.random()
            if kind < 0.15:
                lengths.append(0)
            elif kind < 0.3:
                lengths.append(int(rng.integers(1, 4)))
            elif kind < 0.45:
                lengths.append(int(rng.choice([63, 64, 65])))
            else:
                lengths.append(int(rng.integers(4, 421)))
        if 0 < sum(lengths) <= 1200:
            break
    starts = []
    for _ in range(N):
        kind = rng.random()
        starts.append(0 if kind < 0.35 else (64 * int(rng.integers(1, 5)) if kind < 0.6 else int(rng.integers(1, 301))))
    c = dict(
        idx=i, d=d, act=act, H=H, lengths=lengths, starts=starts,
        with_state=bool(rng.random() < 0.7),
        g_scale=float(rng.choice([0.0, 0.05, 1.0, 6.0])),
        norm_w=str(rng.choice(["ones", "random"])),
        interval=int(rng.choice([0, 64, 128, 192])),
        bf16_state=bool(rng.random() < 0.25),
        mode=str(rng.choice(["one_workgroup", "paired", "split"])),
    )
    if c["mode"] == "split" and c["interval"] == 0:
        c["interval"] = 128                     # the split launch cuts at checkpoint positions
    return c


CASES = [draw_case(i) for i in range(N_CASES)]
FLAGS = {"one_workgroup": 0, "paired": kda.KDA_PREFILL_PAIRED, "split": kda.KDA_PREFILL_SPLIT}


def case_id(c):
    return (f"{c['idx']:02d}-d{c['d']}-{c['act']}-{c['mode']}-g{c['g_scale']}-i{c['interval']}"
            f"{'-bf16state' if c['bf16_state'] else ''}")


def run_case(c, flags):
    shape = wl.LayerShape(c["H"], c["d"], c["d"], act=c["act"])
    seed = SWEEP_SEED % 100000 + c["idx"]
    inp = wl.token_inputs(seed, shape, sum(c["lengths"]), g_scale=c["g_scale"], norm_w=c["norm_w"])
    S0 = X0 = None
    if c["with_state"]:
        S0, X0 = states_for(seed, shape, len(c["lengths"]))
        if c["bf16_state"]:
            # the nearest bf16 values: what a bf16 pool can hold
            S0 = torch.from_numpy(np.ascontiguousarray(S0, np.float32)).to(torch.bfloat16).double().numpy()
    state_dtype = kda.KDA_BF16 if c["bf16_state"] else kda.KDA_F32
    run = Run(shape, inp, c["lengths"], starts=c["starts"], S0=S0, X0=X0, interval=c["interval"], flags=flags,
              state_dtype=state_dtype).launch()
    return run, S0, X0


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_sweep_case_matches_oracle(c):
    say(f"sweep case {case_id(c)}: H={c['H']} lengths={c['lengths']} starts={c['starts']} "
        f"state={c['with_state']} norm_w={c['norm_w']}")
    run, S0, X0 = run_case(c, FLAGS[c["mode"]])
    if c["mode"] == "paired":
        assert int(run.ws[:4].view(torch.int32).item()) == 0       # no wait between the pair ran out
    r = oracle_for(run, S0, X0)
    out = host(run.out)
    Sf, Xf = run.final_state()
    if c["bf16_state"]:
        tol_o, tol_s, tol_c = TOL_BF16_STATE_OUT, TOL_BF16_STATE, TOL_BF16_STATE_CHAIN
    else:
        tol_o, tol_s = tols(c["act"])
        tol_c = TOL_STATE_PER_CHAIN
    e_o, e_r = rel_l2(out, r.out), per_row_max(out, r.out)
    e_s, e_c = rel_l2(Sf, r.S), per_chain_max(Sf, r.S)
    say(f"  out {e_o:.3e} (worst row {e_r:.3e})  state {e_s:.3e} (worst chain {e_c:.3e})")
    assert np.isfinite(out).all() and np.isfinite(Sf).all()
    assert e_o <= tol_o and e_r <= tol_row(c["act"]) and e_s <= tol_s and e_c <= tol_c
    np.testing.assert_array_equal(Xf, r.X)
    assert run.nck == len(r.ckpt_S)
    if run.nck:
        ck = host(run.ckS)[:run.nck]
        e_k, e_kc = rel_l2(ck, r.ckpt_S), per_chain_max(ck, r.ckpt_S)
        say(f"  {run.nck} checkpoints: {e_k:.3e} (worst chain {e_kc:.3e})")
        assert e_k <= tol_s and e_kc <= tol_c
        np.testing.assert_array_equal(host(run.ckX)[:run.nck], r.ckpt_X)
    if c["mode"] == "paired":
        one, _, _ = run_case(c, 0)
        assert np.array_equal(bits(run.out), bits(one.out))
        assert np.array_equal(bits(run.Sd), bits(one.Sd)) and np.array_equal(bits(run.Xd), bits(one.Xd))
        if run.nck:
            assert np.array_equal(bits(run.ckS[:run.nck]), bits(one.ckS[:run.nck]))


# ---- decode: single steps and multi-token launches over random configurations

def draw_decode_case(i):
    rng = np.random.default_rng([SWEEP_SEED, 1000 + i])
    d = int(rng.choice([32, 64, 128]))
    act = "f32" if d <= 64 and rng.random() < 0.5 else "bf16"
    B = int(rng.integers(1, 13))
    return dict(idx=i, d=d, act=act, H=int(rng.integers(1, 5)), B=B, T=int(rng.integers(1, 9)),
                pool=B + int(rng.integers(0, 7)), bf16_state=bool(rng.random() < 0.3),
                g_scale=float(rng.choice([0.0, 0.05, 0.2, 1.0, 6.0])))


DECODE_CASES = [draw_decode_case(i) for i in range(48)]


def decode_case_id(c):
    return (f"{c['idx']:02d}-d{c['d']}-{c['act']}-B{c['B']}-T{c['T']}-g{c['g_scale']}"
            f"{'-bf16state' if c['bf16_state'] else ''}")


@pytest.mark.parametrize("c", DECODE_CASES, ids=[decode_case_id(c) for c in DECODE_CASES])
def test_sweep_decode_matches_oracle(c):
    """T single-token steps against the oracle, and one T-token launch against
    those steps bit for bit (outputs, states, conv states, per-token states)."""
    shape = wl.LayerShape(c["H"], c["d"], c["d"], act=c["act"])
    B, T = c["B"], c["T"]
    say(f"sweep decode {decode_case_id(c)}: H={c['H']} pool={c['pool']}")
    sdt = kda.KDA_BF16 if c["bf16_state"] else kda.KDA_F32
    cfg, inp, S, X, slots, t = setup(shape, SWEEP_SEED % 100000 + 500 + c["idx"], B, T, c["pool"], sdt,
                                     g_scale=c["g_scale"])
    o1, S1, X1, after = single_steps(cfg, S, X, slots, t, T)
    r = lambda a: a.reshape((T, B) + a.shape[1:])
    o_ref, S_ref, X_ref = oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                                              inp.conv_w, inp.norm_w, S[slots], X[slots],
                                              state_round=c["bf16_state"])
    if c["bf16_state"]:
        tol_o, tol_s, tol_c = TOL_BF16_STATE_OUT, TOL_BF16_STATE, TOL_BF16_STATE_CHAIN
    else:
        tol_o, tol_s = tols(c["act"])
        tol_c = TOL_STATE_PER_CHAIN
    out, Sg = host(o1), host(S1)[slots]
    e_o, e_r = rel_l2(out, o_ref), per_row_max(out, o_ref, 3)
    e_s, e_c = rel_l2(Sg, S_ref), per_chain_max(Sg, S_ref)
    say(f"  steps vs oracle: out {e_o:.3e} (worst row {e_r:.3e})  state {e_s:.3e} (worst chain {e_c:.3e})")
    assert np.isfinite(out).all() and np.isfinite(Sg).all()
    assert e_o <= tol_o and e_r <= tol_row(c["act"]) and e_s <= tol_s and e_c <= tol_c
    np.testing.assert_array_equal(host(X1)[slots], X_ref)
    o2, S2, X2, ts, tc = multi(cfg, S, X, slots, t, T)
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(S1), bits(S2)) and np.array_equal(bits(X1), bits(X2))
    for s in range(T):
        assert np.array_equal(bits(ts[:, s]), bits(after[s][0])), f"token state {s}"
        assert np.array_equal(bits(tc[:, s]), bits(after[s][1])), f"token conv state {s}"
