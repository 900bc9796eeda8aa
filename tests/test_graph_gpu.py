"""Library calls captured in a HIP graph: every replay must equal the same
calls made eagerly, bit for bit.  The library allocates nothing and issues no
memset or copy of its own, so its launches are all a graph records.  Between
replays the test does eager work of its own (restoring the initial states and
filling the outputs with NaN) and synchronizes, and each of several replays is
checked."""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import workloads as wl
from tests.helpers import dev, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def test_decode_steps_in_a_graph():
    shape = wl.LayerShape(H=4, dk=128, dv=128, act="bf16")
    cfg = kda.Config(4, 128, 128, kda.KDA_BF16)
    B, steps, pool = 8, 4, 12
    inp = wl.token_inputs(30, shape, B * steps)
    S0, X0 = wl.states(30, shape, pool)
    slots = dev(wl.slot_permutation(30, pool, B))
    r = lambda a, dt=None: dev(a.reshape((steps, B) + a.shape[1:]), dt)
    q, k, v, z = (r(a, torch.bfloat16) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = r(inp.g), r(inp.beta)
    cw, nw = dev(inp.conv_w), dev(inp.norm_w)
    S0d, X0d = dev(S0), dev(X0, torch.bfloat16)

    def run(S, X, out, stream):
        for s in range(steps):
            kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], cw, nw, S, X, slots, out[s],
                                stream=stream)

    Se, Xe = S0d.clone(), X0d.clone()
    oute = torch.empty((steps, B, 4, 128), dtype=torch.bfloat16, device="cuda")
    run(Se, Xe, oute, torch.cuda.current_stream())
    torch.cuda.synchronize()

    Sg, Xg = S0d.clone(), X0d.clone()
    outg = torch.empty_like(oute)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(Sg, Xg, outg, torch.cuda.current_stream())
    for rep in range(REPLAYS):
        Sg.copy_(S0d)
        Xg.copy_(X0d)
        outg.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"decode graph replay {rep}")
        assert torch.equal(outg, oute) and torch.equal(Sg, Se) and torch.equal(Xg, Xe), rep


@pytest.mark.parametrize("flags", [0, kda.KDA_PREFILL_PAIRED])
def test_prefill_call_in_a_graph(flags):
    shape = wl.LayerShape(H=2, dk=64, dv=64, act="bf16")
    cfg = kda.Config(2, 64, 64, kda.KDA_BF16)
    lengths = [300, 77, 129]
    N, T = len(lengths), sum(lengths)
    inp = wl.token_inputs(31, shape, T)
    q, k, v, z = (dev(a, torch.bfloat16) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta, cw, nw = dev(inp.g), dev(inp.beta), dev(inp.conv_w), dev(inp.norm_w)
    S0, X0 = wl.states(31, shape, 2 * N)
    S0d, X0d = dev(S0), dev(X0, torch.bfloat16)
    cu = dev(wl.cu_seqlens(lengths).astype(np.int32))
    init = dev(np.arange(N, dtype=np.int32))
    fin = dev(np.arange(N, 2 * N, dtype=np.int32))
    counts = [kda.kda_num_checkpoints(0, L, 64) for L in lengths]
    nck = sum(counts)
    ck_S = torch.empty((nck, 2, 64, 64), device="cuda")
    ck_X = torch.empty((nck, 2, 2 * 64 + 64, 3), dtype=torch.bfloat16, device="cuda")
    based = dev(np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32))
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, N, T, 64, flags), dtype=torch.uint8, device="cuda")

    def run(S, X, out, cS, cX, stream):
        kda.kda_prefill_varlen(cfg, cu, q, k, v, z, g, beta, cw, nw, S, X, init, fin, out, ws, ckpt_interval=64,
                               ckpt_state=cS, ckpt_conv=cX, ckpt_base=based, flags=flags, stream=stream)

    Se, Xe, oute = S0d.clone(), X0d.clone(), torch.empty((T, 2, 64), dtype=torch.bfloat16, device="cuda")
    cSe, cXe = torch.full_like(ck_S, float("nan")), torch.zeros_like(ck_X)
    run(Se, Xe, oute, cSe, cXe, torch.cuda.current_stream())
    torch.cuda.synchronize()

    Sg, Xg, outg = S0d.clone(), X0d.clone(), torch.empty_like(oute)
    cSg, cXg = torch.empty_like(ck_S), torch.empty_like(ck_X)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(Sg, Xg, outg, cSg, cXg, torch.cuda.current_stream())
    for rep in range(REPLAYS):
        Sg.copy_(S0d)
        Xg.copy_(X0d)
        outg.fill_(float("nan"))
        cSg.fill_(float("nan"))
        cXg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"prefill graph replay {rep}: {nck} checkpoints")
        assert torch.equal(outg, oute) and torch.equal(Sg, Se) and torch.equal(Xg, Xe), rep
        assert torch.equal(cSg, cSe) and torch.equal(cXg, cXe), rep
