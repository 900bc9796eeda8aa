"""Library calls captured in a HIP graph: every replay must equal the same
calls made eagerly, bit for bit.  The library allocates nothing and issues no
memset or copy of its own, so its launches are all a graph records.  Between
replays the test does eager work of its own (restoring the initial states and
filling the outputs with NaN) and synchronizes, and each of several replays is
checked.  Every entry point that launches work is covered: decode steps,
multi-token decode with per-token states, the prefill in its three launch
forms and with the static workspace, the slot copies, and the projections
with the conv front end."""
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


def replays(reset, graph, got, want, what):
    """Replay a captured graph REPLAYS times, resetting its buffers eagerly
    before each replay, and check that every replay leaves the buffers `got`
    bit-equal to the eager run's `want`."""
    for rep in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"{what} graph replay {rep}")
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}, buffer {i}"


@pytest.mark.parametrize("flags", [0, kda.KDA_PREFILL_PAIRED, kda.KDA_PREFILL_SPLIT, "static"],
                         ids=["one_workgroup", "paired", "split", "static"])
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
    static = flags == "static"
    if static:
        flags = 0
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, N, T, 64, flags), dtype=torch.uint8, device="cuda")

    def run(S, X, out, cS, cX, stream):
        if static:
            kda.kda_prefill_varlen_static(cfg, cu, q, k, v, z, g, beta, cw, nw, S, X, init, fin, out,
                                          ckpt_interval=64, ckpt_state=cS, ckpt_conv=cX, ckpt_base=based,
                                          stream=stream)
            return
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


def test_decode_multi_in_a_graph():
    """Multi-token launches with per-token states, two in a row in one graph."""
    shape = wl.LayerShape(H=3, dk=64, dv=64, act="bf16")
    cfg = kda.Config(3, 64, 64, kda.KDA_BF16, state_dtype=kda.KDA_BF16)
    B, T, pool, C = 5, 3, 8, shape.C
    inp = wl.token_inputs(32, shape, 2 * B * T)
    S0, X0 = wl.states(32, shape, pool)
    slots = dev(wl.slot_permutation(32, pool, B))
    r = lambda a, dt=None: dev(a.reshape((2, T, B) + a.shape[1:]), dt)
    q, k, v, z = (r(a, torch.bfloat16) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = r(inp.g), r(inp.beta)
    cw, nw = dev(inp.conv_w), dev(inp.norm_w)
    S0d, X0d = dev(S0, torch.bfloat16), dev(X0, torch.bfloat16)

    def buffers():
        return (S0d.clone(), X0d.clone(), torch.empty((2, T, B, 3, 64), dtype=torch.bfloat16, device="cuda"),
                torch.empty((2, B, T, 3, 64, 64), dtype=torch.bfloat16, device="cuda"),
                torch.empty((2, B, T, 3, C, 3), dtype=torch.bfloat16, device="cuda"))

    def run(S, X, out, ts, tc):
        for i in range(2):
            kda.kda_decode_multi(cfg, q[i], k[i], v[i], z[i], g[i], beta[i], cw, nw, S, X, slots, out[i],
                                 token_state=ts[i], token_conv=tc[i], stream=torch.cuda.current_stream())

    e = buffers()
    run(*e)
    torch.cuda.synchronize()
    gb = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*gb)

    def reset():
        gb[0].copy_(S0d)
        gb[1].copy_(X0d)
        for t in gb[2:]:
            t.fill_(float("nan"))

    replays(reset, graph, gb, e, "decode multi")


def test_slot_copies_in_a_graph():
    """Checkpoint then resume in one graph (the copy-on-write round trip)."""
    shape = wl.LayerShape(H=2, dk=128, dv=128, act="bf16")
    cfg = kda.Config(2, 128, 128, kda.KDA_BF16)
    S0, X0 = wl.states(33, shape, 6)
    S0d, X0d = dev(S0), dev(X0, torch.bfloat16)
    src = dev(np.array([4, 0, 2], np.int32))
    ck = dev(np.array([1, 2, 0], np.int32))
    back = dev(np.array([5, 3, 1], np.int32))

    def run(S, X, cS, cX):
        kda.kda_state_checkpoint(cfg, S, X, src, cS, cX, ck, stream=torch.cuda.current_stream())
        kda.kda_resume(cfg, cS, cX, ck, S, X, back, stream=torch.cuda.current_stream())

    def buffers():
        return (S0d.clone(), X0d.clone(), torch.empty((3, 2, 128, 128), device="cuda"),
                torch.empty((3, 2, 3 * 128, 3), dtype=torch.bfloat16, device="cuda"))

    e = buffers()
    run(*e)
    torch.cuda.synchronize()
    assert torch.equal(e[0][[5, 3, 1]], S0d[[4, 0, 2]]) and torch.equal(e[1][[5, 3, 1]], X0d[[4, 0, 2]])
    gb = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*gb)

    def reset():
        gb[0].copy_(S0d)
        gb[1].copy_(X0d)
        gb[2].fill_(float("nan"))
        gb[3].fill_(float("nan"))

    replays(reset, graph, gb, e, "slot copies")


def test_projections_in_a_graph():
    """The conv front end (GEMM plus its tile-top pass) and the output
    projection, captured together."""
    H, d, Dm = 2, 64, 256
    shape = wl.LayerShape(H, d, d)
    cfg = kda.Config(H, d, d, kda.KDA_BF16)
    lengths = [300, 1, 260]
    N, T, C = len(lengths), sum(lengths), shape.C
    x, w = wl.projection_inputs(34, shape, T, Dm)
    base = wl.token_inputs(34, shape, 1)
    _, X0 = wl.states(35, shape, N, conv_std=1.0)
    bf = torch.bfloat16
    xd, wd, cw, Xd = dev(x, bf), dev(w, bf), dev(base.conv_w), dev(X0, bf)
    cu = dev(wl.cu_seqlens(lengths).astype(np.int32))
    init = dev(np.arange(N, dtype=np.int32))
    w_o = dev(np.random.default_rng(36).standard_normal((Dm, H * d)) * 0.05, bf)

    def buffers():
        return [torch.empty((2, T, H, d), dtype=bf, device="cuda"), torch.empty((2, T, H, d), dtype=bf, device="cuda"),
                torch.empty((2, T, H, d), dtype=bf, device="cuda"), torch.empty((T, H, d), dtype=bf, device="cuda"),
                torch.empty((T, H, d), device="cuda"), torch.empty((T, H), device="cuda"),
                torch.empty((T, Dm), dtype=bf, device="cuda")]

    def run(q, k, v, z, g, beta, y):
        st = torch.cuda.current_stream()
        kda.kda_project_inputs_conv(cfg, cu, xd, wd, cw, Xd, init, q, k, v, z, g, beta, stream=st)
        kda.kda_project_output(cfg, v[0], w_o, y, stream=st)       # any [T][H][dv] bf16 operand will do

    e = buffers()
    run(*e)
    torch.cuda.synchronize()
    gb = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*gb)

    def reset():
        for t in gb:
            t.fill_(float("nan"))

    replays(reset, graph, gb, e, "projections")
