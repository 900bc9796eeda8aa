"""kda_prefill_varlen_static, the prefill entry point that allocates nothing
(its workspace is the library's static device buffer), against
kda_prefill_varlen with an allocated workspace: the same kernels, so every
output, final state, conv state and checkpoint must agree bit for bit.  Two
calls in a row per launch form, the second smaller, since the buffer keeps
the previous call's contents; and a call too large for the buffer is refused
without touching its outputs."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import workloads as wl
from tests.helpers import bits, host, say
from tests.prefill_runner import Run, states_for

pytestmark = pytest.mark.gpu

MODES = {"one_workgroup": 0, "paired": kda.KDA_PREFILL_PAIRED, "split": kda.KDA_PREFILL_SPLIT}
CALLS = [  # (seed, shape, lengths, starts): the second call of each mode is the smaller one
    (110, wl.LayerShape(4, 128, 128), [700, 129, 300, 64], [0, 64, 5, 0]),
    (111, wl.LayerShape(2, 128, 128), [150, 3], [64, 0]),
]


def same_bits(a, b):
    for x, y in ((a.out, b.out), (a.Sd, b.Sd), (a.Xd, b.Xd)):
        assert np.array_equal(bits(x), bits(y))
    if a.interval:
        assert np.array_equal(bits(a.ckS[:a.nck]), bits(b.ckS[:b.nck]))
        assert np.array_equal(bits(a.ckX[:a.nck]), bits(b.ckX[:b.nck]))


@pytest.mark.parametrize("mode", list(MODES))
def test_static_workspace_equals_allocated_workspace(mode):
    for i, (seed, shape, lengths, starts) in enumerate(CALLS):
        say(f"static workspace {mode} call {i}: H={shape.H} lengths={lengths}")
        inp = wl.token_inputs(seed, shape, sum(lengths), g_scale=3.0 if i else 1.0, norm_w="random")
        S0, X0 = states_for(seed, shape, len(lengths))
        ref = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=MODES[mode]).launch()
        run = Run(shape, inp, lengths, starts=starts, S0=S0, X0=X0, interval=128, flags=MODES[mode])
        run.launch(static=True)
        assert np.isfinite(host(run.out)).all()
        same_bits(run, ref)
        # again: torch now serves the small index tensors of the call from its
        # cache, so any change in free device memory would be the library's
        free0 = torch.cuda.mem_get_info()[0]
        run.launch(static=True)
        assert torch.cuda.mem_get_info()[0] == free0
        same_bits(run, ref)


def test_static_workspace_refuses_a_call_it_cannot_hold():
    # a paired ring for 160 chains at dk = dv = 128 needs about 70 MB
    shape = wl.LayerShape(32, 128, 128)
    lengths = [64] * 5
    assert kda.kda_prefill_workspace_bytes(kda.Config(32, 128, 128), 5, 320, 0,
                                           kda.KDA_PREFILL_PAIRED) > kda.STATIC_WORKSPACE_BYTES
    inp = wl.token_inputs(112, shape, sum(lengths))
    run = Run(shape, inp, lengths, flags=kda.KDA_PREFILL_PAIRED)
    with pytest.raises(kda.KdaError) as e:
        run.launch(static=True)
    assert e.value.status == kda.KDA_ERR_WORKSPACE and "static workspace" in str(e.value)
    assert np.isnan(host(run.out)).all()                    # nothing was launched
