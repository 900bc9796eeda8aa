"""Maximum sizes: tensors and pools past 4 GiB.

The kernels address memory through 32-bit buffer offsets from 64-bit bases
(per (slot, head), per chunk, per output tile).  These cases put the data that
is checked beyond 4 GiB into large device tensors whose leading part is zero
(filled on the device, so the host only generates the checked part), and
compare it with the fp64 oracle:
  - decode on slots of a 4.4 GB state pool (slot, head offsets past 2^32 bytes);
  - a prefill whose second sequence starts past 2^31 elements of q, k, v, z
    (4 GiB of bf16) and 8 GiB of g;
  - input projections whose last row tiles start past 4 GiB of x.
About 40 GB of device memory at most.
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from oracle import projection
from tests.helpers import dev, host, rel_l2, say

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def test_decode_slots_past_4gib():
    shape = wl.LayerShape(H=32, dk=128, dv=128, act="bf16")
    cfg = kda.Config(32, 128, 128, kda.KDA_BF16)
    B, steps, pool = 8, 2, 2112                     # 2112 x 32 x 64 KiB = 4.43e9 bytes of state
    lo = 2048                                       # the slots used lie past 2048 x 2 MiB = 4 GiB
    inp = wl.token_inputs(40, shape, B * steps)
    S, X = wl.states(40, shape, B)                  # states of the used slots only
    slots = (lo + wl.slot_permutation(40, pool - lo, B)).astype(np.int32)
    Sd = torch.zeros((pool, 32, 128, 128), device="cuda")
    Xd = torch.zeros((pool, 32, 384, 3), dtype=torch.bfloat16, device="cuda")
    sl = torch.from_numpy(slots.astype(np.int64)).cuda()
    Sd[sl] = dev(S)
    Xd[sl] = dev(X, torch.bfloat16)
    say(f"decode: pool {Sd.numel() * 4 / GIB:.2f} GiB, slots {sorted(slots.tolist())}")
    r = lambda a: a.reshape((steps, B) + a.shape[1:])
    q, k, v, z = (dev(r(a), torch.bfloat16) for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = dev(r(inp.g)), dev(r(inp.beta))
    cw, nw = dev(inp.conv_w), dev(inp.norm_w)
    out = torch.empty((steps, B, 32, 128), dtype=torch.bfloat16, device="cuda")
    slot_d = dev(slots)
    for s in range(steps):
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], cw, nw, Sd, Xd, slot_d, out[s])
    torch.cuda.synchronize()
    o_ref, S_ref, X_ref = oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                                              inp.conv_w, inp.norm_w, S, X)
    e_o = rel_l2(host(out), o_ref)
    e_s = rel_l2(host(Sd[sl]), S_ref)
    say(f"  out {e_o:.2e} state {e_s:.2e}")
    assert e_o <= 1e-2 and e_s <= 5e-3
    assert np.array_equal(host(Xd[sl]), np.asarray(torch.from_numpy(X_ref.astype(np.float32)).to(torch.bfloat16).float()))
    del Sd, Xd
    torch.cuda.empty_cache()


def test_prefill_sequence_past_4gib():
    shape = wl.LayerShape(H=32, dk=128, dv=128, act="bf16")
    cfg = kda.Config(32, 128, 128, kda.KDA_BF16)
    H, D = 32, 128
    lead = (1 << 31) // (H * D) + 64                # 524,352 tokens: 2^31 + 2^18 elements before the tail
    L = 300                                         # the checked sequence
    T = lead + L
    inp = wl.token_inputs(41, shape, L)
    act = torch.bfloat16
    q, k, v, z = (torch.zeros((T, H, D), dtype=act, device="cuda") for _ in range(4))
    g = torch.zeros((T, H, D), device="cuda")
    beta = torch.zeros((T, H), device="cuda")
    for t, a in ((q, inp.q), (k, inp.k), (v, inp.v), (z, inp.z)):
        t[lead:] = dev(a, act)
    g[lead:] = dev(inp.g)
    beta[lead:] = dev(inp.beta)
    say(f"prefill: {T} tokens, q {q.numel() * 2 / GIB:.2f} GiB, g {g.numel() * 4 / GIB:.2f} GiB; "
        f"checked sequence starts at element {lead * H * D}")
    S = torch.zeros((2, H, D, D), device="cuda")
    X = torch.zeros((2, H, 3 * D, 3), dtype=act, device="cuda")
    out = torch.empty((T, H, D), dtype=act, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, 2, T), dtype=torch.uint8, device="cuda")
    kda.kda_prefill_varlen(cfg, dev(np.array([0, lead, T], np.int32)), q, k, v, z, g, beta, dev(inp.conv_w),
                           dev(inp.norm_w), S, X, dev(np.array([-1, -1], np.int32)), dev(np.array([0, 1], np.int32)),
                           out, ws)
    torch.cuda.synchronize()
    ref = oracle.run(inp.q, inp.k, inp.v, inp.z, inp.g, inp.beta, inp.conv_w, inp.norm_w, wl.cu_seqlens([L]))
    e_o = rel_l2(host(out[lead:]), ref.out)
    e_s = rel_l2(host(S[1]), ref.S[0])
    say(f"  tail sequence: out {e_o:.2e} state {e_s:.2e}")
    assert e_o <= 1e-2 and e_s <= 5e-3
    # the all-zero leading sequence: zero inputs keep a zero state and give zero outputs
    assert float(out[:lead].abs().max()) == 0.0 and float(S[0].abs().max()) == 0.0
    del q, k, v, z, g, out
    torch.cuda.empty_cache()


def test_projection_rows_past_4gib():
    shape = wl.LayerShape(H=4, dk=128, dv=128)
    cfg = kda.Config(4, 128, 128, kda.KDA_BF16)
    Dm = 7168
    lead = (1 << 31) // Dm + 256                    # x rows before the checked ones: > 2^31 elements
    Tc = 300
    T = lead + Tc
    xs, w = wl.projection_inputs(42, shape, Tc, Dm)
    x = torch.zeros((T, Dm), dtype=torch.bfloat16, device="cuda")
    x[lead:] = dev(xs, torch.bfloat16)
    say(f"projection: x {x.numel() * 2 / GIB:.2f} GiB, checked rows from {lead}")
    H, d = 4, 128
    o = dict(q=torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda"),
             k=torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda"),
             v=torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda"),
             z=torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda"),
             g=torch.empty((T, H, d), device="cuda"), beta=torch.empty((T, H), device="cuda"))
    kda.kda_project_inputs(cfg, x, dev(w, torch.bfloat16), o["q"], o["k"], o["v"], o["z"], o["g"], o["beta"])
    torch.cuda.synchronize()
    ref = projection.project(xs, w, H, d, d)
    for name in ("q", "k", "v", "z", "g", "beta"):
        e = rel_l2(host(o[name][lead:]), ref[name])
        tol = 1e-2 if name in "qkvz" else 1e-5
        say(f"  {name}: {e:.2e}")
        assert e <= tol, name
    # zero rows: q..z zero, g = -ln 2, beta = 1/2
    assert float(o["q"][:lead].abs().max()) == 0.0
    assert torch.allclose(o["beta"][:lead], torch.full_like(o["beta"][:lead], 0.5))
    del x, o
    torch.cuda.empty_cache()
