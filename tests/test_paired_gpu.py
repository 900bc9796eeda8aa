"""GPU tests of the paired prefill (KDA_PREFILL_PAIRED): two workgroups per
(sequence, head) chain, one for the state-independent phase of every chunk
and one for the state phase, joined by a ring in the workspace.

Both workgroups run the one-workgroup kernel's own arithmetic, so a paired
call must reproduce the one-workgroup call bit for bit (outputs, final
states, conv states, checkpoints), and through it the oracle.  In a batch
with more chains than the device holds as resident pairs, the launch pairs
the longest chains and runs the others one workgroup each from a queue, with
the same results.
"""
import numpy as np
import pytest

import linear_attention_recurrence_decode_amd as kda
import workloads as wl
from tests.helpers import bits, host, say
from tests.prefill_runner import Run, check_against_oracle, oracle_for, resume_and_finish, states_for
from tests.test_prefill_gpu import CASES

pytestmark = pytest.mark.gpu

PAIRED = kda.KDA_PREFILL_PAIRED


def assert_same_bits(a, b):
    assert np.array_equal(bits(a.out), bits(b.out))
    assert np.array_equal(bits(a.Sd), bits(b.Sd))
    assert np.array_equal(bits(a.Xd), bits(b.Xd))
    if a.interval:
        assert np.array_equal(bits(a.ckS[:a.nck]), bits(b.ckS[:b.nck]))
        assert np.array_equal(bits(a.ckX[:a.nck]), bits(b.ckX[:b.nck]))


@pytest.mark.parametrize("name", list(CASES))
def test_paired_matches_oracle_and_one_workgroup_bits(name):
    seed, shape, lengths, starts, with_state, g_scale, norm_w = CASES[name]
    say(f"paired case {name}: H={shape.H} d={shape.dk} act={shape.act} lengths={lengths} starts={starts}")
    inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=g_scale, norm_w=norm_w)
    S0 = X0 = None
    if with_state:
        S0, X0 = states_for(seed, shape, len(lengths))
    interval = 128
    paired = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval, flags=PAIRED).launch()
    check_against_oracle(paired, oracle_for(paired, S0, X0))
    single = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=interval).launch()
    assert_same_bits(paired, single)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_paired_resume_is_bitwise_identical(act):
    """Resume at an interval checkpoint, paired on both sides, reproduces the
    straight paired run's later outputs and final states bit for bit."""
    shape = wl.LayerShape(2, 64, 64, act=act)
    lengths, starts = [700, 300, 129], [0, 64, 3]
    inp = wl.token_inputs(60, shape, sum(lengths))
    S0, X0 = states_for(60, shape, len(lengths))
    straight = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=PAIRED).launch()
    resumed, seqs, res_pos, _, idx = resume_and_finish(straight, [2, 1, 0])
    say(f"  resumed {seqs} at {res_pos}")
    assert np.array_equal(bits(resumed.out), bits(straight.out[idx]))
    for j, n in enumerate(seqs):
        assert np.array_equal(bits(resumed.Sd[int(resumed.final[j])]), bits(straight.Sd[int(straight.final[n])]))


def test_paired_4x8192_full_size_equals_one_workgroup():
    """The 4 x 8192-token workload (128 chains, the shape the paired launch is
    for): every output, final state and conv state equals the one-workgroup
    run bit for bit (that run is checked against the oracle and the decode
    kernel in the prefill tests)."""
    w = wl.WORKLOADS["prefill_4x8k"]
    shape, lengths = w["shape"], w["lengths"]
    inp = wl.token_inputs(w["seed"], shape, sum(lengths))
    say(f"paired full size: lengths={lengths} H={shape.H}")
    paired = Run(shape, inp, lengths, flags=PAIRED).launch()
    single = Run(shape, inp, lengths).launch()
    assert np.isfinite(host(paired.out)).all()
    assert_same_bits(paired, single)


@pytest.mark.parametrize("case", ["uniform_160_chains", "skewed_lengths"])
def test_paired_schedule_mixes_pairs_and_singles(case):
    """More chains than pairs fit: the scheduled launch pairs the longest
    chains and runs the rest one workgroup each from a queue.  Same bits as
    the one-workgroup kernel, and the oracle on one head."""
    shape = wl.LayerShape(4, 128, 128)
    rng = np.random.default_rng(61)
    if case == "uniform_160_chains":
        lengths = [int(x) for x in rng.integers(1, 90, 40)]
    else:
        # a few long sequences among many short ones (the shape of a varlen batch)
        lengths = [1500, 900] + [int(x) for x in rng.integers(1, 200, 70)] + [0, 3]
    inp = wl.token_inputs(61, shape, sum(lengths))
    say(f"paired schedule {case}: {len(lengths)} sequences x {shape.H} heads, {sum(lengths)} tokens")
    paired = Run(shape, inp, lengths, interval=64, flags=PAIRED).launch()
    single = Run(shape, inp, lengths, interval=64).launch()
    assert_same_bits(paired, single)
    check_against_oracle(paired, oracle_for(paired, heads=[1]), heads=[1])


def test_paired_invalid_slot_gives_nan_and_writes_nothing():
    shape = wl.LayerShape(2, 64, 64)
    lengths = [70, 200]
    inp = wl.token_inputs(62, shape, sum(lengths))
    run = Run(shape, inp, lengths, flags=PAIRED)
    run.init = np.array([-1, 999], np.int32)
    before = bits(run.Sd[int(run.final[1])])
    run.launch()
    out = host(run.out)
    assert np.isfinite(out[:70]).all() and np.isnan(out[70:]).all()
    assert np.array_equal(bits(run.Sd[int(run.final[1])]), before)
    assert np.isfinite(host(run.Sd)[int(run.final[0])]).all()


def schedule_pairs_model(lengths, starts, H, G, max_pairs):
    """Host statement of the launch's choice of K (pairs for the leading
    chains, longest first): every chain when the grid holds a pair for each;
    otherwise, in chunk steps of one workgroup, a paired chain at 0.72 per
    chunk, the unpaired chains spread over the G - 2K other workgroups, and K
    minimises the largest of the three times."""
    order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    chunks = [0 if lengths[i] <= 0 else (starts[i] % 64 + lengths[i] + 63) // 64 for i in order]
    NH = len(lengths) * H
    if 2 * NH <= G and NH <= max_pairs:
        return NH                                             # a pair for every chain fits: all paired
    W = float(sum(chunks) * H)
    kmax = min(max_pairs, G // 2, NH)
    best, bestk, paired = float("inf"), 0, 0.0
    for k in range(kmax + 1):
        lu = float(chunks[k // H]) if k < NH else 0.0
        workers = G - 2 * k
        if k == NH or workers > 0:
            mk = max(0.72 * chunks[0] if k > 0 else 0.0, lu, (W - paired) / workers if workers > 0 else 0.0)
            if mk < best * (1.0 - 1e-9):
                best, bestk = mk, k
        if k < NH:
            paired += lu
    return bestk


@pytest.mark.parametrize("case", ["equal", "one_long", "skewed"])
def test_paired_schedule_choice_matches_model(case):
    """The number of paired chains the metadata kernel writes into the
    workspace equals the host statement of the cost model."""
    import torch
    shape = wl.LayerShape(4, 128, 128)
    rng = np.random.default_rng(63)
    lengths = {"equal": [256] * 8,
               "one_long": [2000] + [int(x) for x in rng.integers(1, 60, 90)],
               "skewed": [1500, 900] + [int(x) for x in rng.integers(1, 200, 70)] + [0, 3]}[case]
    inp = wl.token_inputs(63, shape, sum(lengths))
    run = Run(shape, inp, lengths, flags=PAIRED).launch()
    NH = len(lengths) * shape.H
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G = min(cus // 16 * 16, 16 * ((NH + 7) // 8))          # one 512-thread workgroup per CU at d = 128
    max_pairs = min(NH, 256)
    ctr_off = 256 + (len(lengths) * 32 + 255) // 256 * 256  # after the status block and the work items (32 B each)
    ws = run.ws.cpu().numpy()
    k_dev = int(ws[ctr_off + max_pairs * 128: ctr_off + max_pairs * 128 + 4].view(np.int32)[0])
    k_host = schedule_pairs_model(lengths, [0] * len(lengths), shape.H, G, max_pairs)
    say(f"  {case}: {NH} chains, grid {G}: pairs {k_dev} (model {k_host})")
    assert k_dev == k_host
    if case == "equal":
        assert k_dev == NH                                    # every chain paired


def test_paired_many_short_sequences():
    """More than 1024 sequences (work items then keep their input order):
    the scheduled launch still equals the one-workgroup kernel bit for bit."""
    shape = wl.LayerShape(1, 32, 32, act="f32")
    rng = np.random.default_rng(64)
    lengths = [int(x) for x in rng.integers(0, 70, 1100)]
    lengths[500] = 400                                        # one long sequence in the middle
    inp = wl.token_inputs(64, shape, sum(lengths))
    say(f"paired many short: {len(lengths)} sequences, {sum(lengths)} tokens")
    paired = Run(shape, inp, lengths, interval=64, flags=PAIRED).launch()
    single = Run(shape, inp, lengths, interval=64).launch()
    assert_same_bits(paired, single)


def test_paired_wait_gives_up_with_status_and_nan():
    """Every wait between paired workgroups limited to one poll (the test-only
    flag), so waits give up although both workgroups run and every kernel
    exits normally.  The workspace status word counts the waits that gave up;
    a chain whose state-phase workgroup gave up has NaN outputs from a chunk
    boundary on, a NaN final state and NaN in its later checkpoints, and its
    rows before that chunk, like every chain that completed, equal the
    one-workgroup run bit for bit."""
    shape = wl.LayerShape(4, 128, 128)
    lengths, starts = [640, 513, 300, 64], [0, 64, 7, 0]
    inp = wl.token_inputs(61, shape, sum(lengths))
    ref = Run(shape, inp, lengths, starts=starts, interval=128).launch()
    assert kda.prefill_status(ref.ws) == 0
    run = Run(shape, inp, lengths, starts=starts, interval=128,
              flags=PAIRED | kda.KDA_PREFILL_PAIRED_POLL_ONCE).launch()
    status = kda.prefill_status(run.ws)
    out, ro = host(run.out), host(ref.out)
    Sf, Sr = host(run.Sd), host(ref.Sd)
    ck = host(run.ckS)
    failed = 0
    for n, L in enumerate(lengths):
        a = int(ref.cu[n])
        fin = int(run.final[n])
        for h in range(shape.H):
            rows, rrows = out[a:a + L, h], ro[a:a + L, h]
            nan_rows = np.isnan(rows).any(axis=1)
            if not nan_rows.any():
                assert np.array_equal(rows, rrows)
                assert np.array_equal(Sf[fin, h], Sr[fin, h])
                continue
            failed += 1
            first = int(np.argmax(nan_rows))
            assert np.isnan(rows[first:]).all() and not np.isnan(rows[:first]).any()
            assert first == 0 or (starts[n] + first) % 64 == 0
            assert np.array_equal(rows[:first], rrows[:first])
            assert np.isnan(Sf[fin, h]).all()
            last = int(run.base[n]) + kda.kda_num_checkpoints(starts[n], L, 128) - 1
            assert np.isnan(ck[last, h]).all()
    say(f"  status word {status}, chains with NaN tails {failed} of {len(lengths) * shape.H}")
    assert status > 0 and status >= failed
