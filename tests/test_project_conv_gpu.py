"""GPU parity of the conv front end (kda_project_inputs_conv: the input
projections with the causal conv + SiLU fused into the GEMM epilogue) and of
the prefill that takes its activations (KDA_PREFILL_CONV_DONE).

The front end writes, for q, k and v, the post-conv activations and the raw
projections back to back.  Its raw projections are the GEMM kda_project_inputs
runs (bit for bit); its activations are checked against the conv oracle
(oracle/conv.py) applied to the projection oracle's q, k, v rounded to bf16,
with each sequence's left context from its initial conv state.  The prefill
on those activations is checked against the recurrence oracle on the same
bf16-rounded projections (the layer's inputs): the post-conv activations are
rounded to bf16 once more than in the unfused pipeline, so the whole-tensor
bf16 bounds apply (outputs 1e-2, states 5e-3; measured about 3e-3 and 2e-3).
Per output row the bound is 1e-1 instead of the unfused 5e-2: the rounding of
q^ (about 2^-9 per element) reaches o = S^T q^ as 2^-9 |S| |q^|, so a row whose
|o| is small against |S| |q^| carries it amplified (the RMSNorm removes the
row's scale, not its relative error); measured worst rows 1.5e-2 to 4.8e-2.
Its conv states and checkpoints' conv states hold raw inputs and equal those
of the unfused pipeline bit for bit.

[vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
"KDA prefill and decode": the input projections and the causal convolution
are fused around the recurrence.]
"""
import numpy as np
import pytest
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from oracle import conv, projection
from tests.helpers import bits, dev, host, per_row_max, rel_l2, say, tol_row

pytestmark = pytest.mark.gpu

CD = kda.KDA_PREFILL_CONV_DONE

CASES = {
    # name: (seed, H, d, Dm, lengths, initial states)
    "d64_tiles": (120, 2, 64, 256, [300, 1, 2, 0, 260], True),   # sequences across the 253-row tile steps
    "d128": (121, 4, 128, 512, [1000, 129], False),
    "d32_short": (122, 3, 32, 64, [129, 77, 3], True),
}


def r16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()


class Case:
    def __init__(self, name):
        seed, H, d, Dm, lengths, with_state = CASES[name]
        self.shape = shape = wl.LayerShape(H, d, d)
        self.lengths, self.N, self.T = lengths, len(lengths), sum(lengths)
        self.cfg = kda.Config(H, d, d, kda.KDA_BF16)
        self.x, self.w = wl.projection_inputs(seed, shape, self.T, Dm)
        base = wl.token_inputs(seed, shape, 1, norm_w="random")          # conv and norm weights
        self.conv_w, self.norm_w = base.conv_w, base.norm_w
        self.cu = wl.cu_seqlens(lengths)
        N, C = self.N, shape.C
        self.S0 = self.X0 = None
        if with_state:
            self.S0, self.X0 = wl.states(seed + 1, shape, N, state_std=0.3, conv_std=1.0)
        # slots 0..N-1 hold the initial states (zero without them), N..2N-1 receive the final ones
        S = np.zeros((2 * N + 1, H, d, d), np.float32)
        X = np.zeros((2 * N + 1, H, C, 3), np.float32)
        if with_state:
            S[:N], X[:N] = self.S0, self.X0
        self.S_init, self.X_init = S, X
        self.init = np.arange(N, dtype=np.int32) if with_state else np.full(N, -1, np.int32)
        self.p = projection.project(self.x, self.w, H, d, d)

    def front_end(self):
        H, d, T = self.shape.H, self.shape.dk, self.T
        bf = torch.bfloat16
        o = dict(q=torch.full((2, T, H, d), float("nan"), dtype=bf, device="cuda"),
                 k=torch.full((2, T, H, d), float("nan"), dtype=bf, device="cuda"),
                 v=torch.full((2, T, H, d), float("nan"), dtype=bf, device="cuda"),
                 z=torch.full((T, H, d), float("nan"), dtype=bf, device="cuda"),
                 g=torch.full((T, H, d), float("nan"), device="cuda"),
                 beta=torch.full((T, H), float("nan"), device="cuda"))
        kda.kda_project_inputs_conv(self.cfg, dev(self.cu.astype(np.int32)), dev(self.x, bf), dev(self.w, bf),
                                    dev(self.conv_w), dev(self.X_init, bf), dev(self.init), o["q"], o["k"], o["v"],
                                    o["z"], o["g"], o["beta"])
        torch.cuda.synchronize()
        return o

    def unfused_projections(self):
        H, d, T = self.shape.H, self.shape.dk, self.T
        bf = torch.bfloat16
        o = dict(q=torch.empty((T, H, d), dtype=bf, device="cuda"), k=torch.empty((T, H, d), dtype=bf, device="cuda"),
                 v=torch.empty((T, H, d), dtype=bf, device="cuda"), z=torch.empty((T, H, d), dtype=bf, device="cuda"),
                 g=torch.empty((T, H, d), device="cuda"), beta=torch.empty((T, H), device="cuda"))
        kda.kda_project_inputs(self.cfg, dev(self.x, bf), dev(self.w, bf), o["q"], o["k"], o["v"], o["z"], o["g"],
                               o["beta"])
        torch.cuda.synchronize()
        return o

    def prefill(self, o, flags, interval=64):
        """One prefill call on projections o (CD flag: the front end's pairs)."""
        H, d, T, N, C = self.shape.H, self.shape.dk, self.T, self.N, self.shape.C
        bf = torch.bfloat16
        S, X = dev(self.S_init), dev(self.X_init, bf)
        counts = [oracle.num_checkpoints(0, L, interval) for L in self.lengths]
        base = np.zeros(N, np.int32)
        base[1:] = np.cumsum(counts)[:-1]
        nck = max(int(sum(counts)), 1)
        ckS = torch.full((nck, H, d, d), float("nan"), device="cuda")
        ckX = torch.zeros((nck, H, C, 3), dtype=bf, device="cuda")
        out = torch.full((T, H, d), float("nan"), dtype=bf, device="cuda")
        ws = torch.empty(kda.kda_prefill_workspace_bytes(self.cfg, N, T, interval, flags & ~CD), dtype=torch.uint8,
                         device="cuda")
        kda.kda_prefill_varlen(self.cfg, dev(self.cu.astype(np.int32)), o["q"], o["k"], o["v"], o["z"], o["g"],
                               o["beta"], dev(self.conv_w), dev(self.norm_w), S, X, dev(self.init),
                               dev(np.arange(N, 2 * N, dtype=np.int32)), out, ws, ckpt_interval=interval,
                               ckpt_state=ckS, ckpt_conv=ckX, ckpt_base=dev(base), flags=flags)
        torch.cuda.synchronize()
        return out, S[N:2 * N], X[N:2 * N], ckS[:int(sum(counts))], ckX[:int(sum(counts))]


@pytest.mark.parametrize("name", list(CASES))
def test_front_end_matches_oracles(name):
    c = Case(name)
    say(f"conv front end {name}: H={c.shape.H} d={c.shape.dk} lengths={c.lengths}")
    o = c.front_end()
    ref = c.unfused_projections()
    # raw projections: the same GEMM as kda_project_inputs, bit for bit
    for t in ("q", "k", "v"):
        assert np.array_equal(bits(o[t][1]), bits(ref[t])), t
    for t in ("z", "g", "beta"):
        assert np.array_equal(bits(o[t]), bits(ref[t])), t
    # post-conv activations against the conv oracle on the bf16-rounded projections
    X0 = None if c.X0 is None else c.X0
    aq, ak, av = conv.activations(r16(c.p["q"]), r16(c.p["k"]), r16(c.p["v"]), c.conv_w, c.cu, X0)
    for t, a in (("q", aq), ("k", ak), ("v", av)):
        got = host(o[t][0])
        e, e_r = rel_l2(got, a), per_row_max(got, a)
        say(f"  {t} post-conv: rel-L2 {e:.3e}, worst row {e_r:.3e}")
        assert np.isfinite(got).all() and e <= 1e-2 and e_r <= tol_row("bf16")


@pytest.mark.parametrize("mode", ["one_workgroup", "paired", "split"])
@pytest.mark.parametrize("name", list(CASES))
def test_conv_done_prefill_matches_oracle_and_unfused(name, mode):
    flags = {"one_workgroup": 0, "paired": kda.KDA_PREFILL_PAIRED, "split": kda.KDA_PREFILL_SPLIT}[mode]
    c = Case(name)
    say(f"conv-done prefill {name} {mode}: lengths={c.lengths}")
    out, S, X, ckS, ckX = c.prefill(c.front_end(), flags | CD)
    p = c.p
    r = oracle.run(r16(p["q"]), r16(p["k"]), r16(p["v"]), r16(p["z"]), p["g"], p["beta"], c.conv_w, c.norm_w, c.cu,
                   S0=c.S0, X0=c.X0, ckpt_interval=64)
    o_h = host(out)
    e_o, e_r = rel_l2(o_h, r.out), per_row_max(o_h, r.out)
    e_s, e_ck = rel_l2(host(S), r.S), rel_l2(host(ckS), r.ckpt_S)
    say(f"  vs oracle: out {e_o:.3e} (worst row {e_r:.3e}) state {e_s:.3e} checkpoints {e_ck:.3e}")
    assert np.isfinite(o_h).all() and e_o <= 1e-2 and e_r <= 1e-1 and e_s <= 5e-3 and e_ck <= 5e-3
    # the unfused pipeline: the same but for one bf16 rounding of the activations;
    # conv states hold raw inputs, which both pipelines take from the same GEMM
    out_u, S_u, X_u, ckS_u, ckX_u = c.prefill(c.unfused_projections(), flags)
    e_u, e_us = rel_l2(o_h, host(out_u)), rel_l2(host(S), host(S_u))
    say(f"  vs unfused pipeline: out {e_u:.3e} state {e_us:.3e}")
    assert e_u <= 1e-2 and e_us <= 5e-3
    assert np.array_equal(bits(X), bits(X_u)) and np.array_equal(bits(ckX), bits(ckX_u))


def test_front_end_full_size_sampled_rows():
    """The conv front end on the 4 x 8192 token projections (Dm 7168, H=32,
    d=128) as four packed sequences: one starting from an initial conv state,
    one with none, one from a second state, one whose slot is out of range
    (zero context, as in the prefill).  Raw halves bit-equal to
    kda_project_inputs on every row; activations of sampled rows (the first
    three rows of tiles, where the tile-top pass computes them, sequence
    starts and random rows) against the conv oracle on the projection
    oracle's rows, rounded to bf16.  Each sampled row's window is the oracle
    run over the rows from max(start, m - 3) to m, from the sequence's
    initial conv state when that range begins at its start."""
    wk = wl.WORKLOADS["project_4x8k"]
    shape, T, Dm = wk["shape"], wk["T"], wk["Dm"]
    H, d = shape.H, shape.dk
    bf = torch.bfloat16
    x, w = wl.projection_inputs(wk["seed"], shape, T, Dm)
    lengths = [T // 4] * 4
    cu = wl.cu_seqlens(lengths)
    conv_w = wl.token_inputs(wk["seed"], shape, 1).conv_w
    _, X = wl.states(wk["seed"] + 1, shape, 2, conv_std=1.0)     # two slots of conv state
    init = np.array([0, -1, 1, 7], np.int32)                       # 7 >= 2 slots: zero context
    cfg = kda.Config(H, d, d, kda.KDA_BF16)
    q2, k2, v2 = (torch.empty((2, T, H, d), dtype=bf, device="cuda") for _ in range(3))
    z = torch.empty((T, H, d), dtype=bf, device="cuda")
    g = torch.empty((T, H, d), device="cuda")
    beta = torch.empty((T, H), device="cuda")
    xd, wd = dev(x, bf), dev(w, bf)
    kda.kda_project_inputs_conv(cfg, dev(cu.astype(np.int32)), xd, wd, dev(conv_w), dev(X, bf), dev(init),
                                q2, k2, v2, z, g, beta)
    torch.cuda.synchronize()
    say(f"conv front end full size: T={T} Dm={Dm} H={H}; raw halves against kda_project_inputs")
    q1, k1, v1 = (torch.empty((T, H, d), dtype=bf, device="cuda") for _ in range(3))
    z1 = torch.empty_like(z)
    g1, b1 = torch.empty_like(g), torch.empty_like(beta)
    kda.kda_project_inputs(cfg, xd, wd, q1, k1, v1, z1, g1, b1)
    torch.cuda.synchronize()
    for name, a, b in (("q", q2[1], q1), ("k", k2[1], k1), ("v", v2[1], v1), ("z", z, z1), ("g", g, g1),
                       ("beta", beta, b1)):
        assert torch.equal(a.view(torch.int16) if a.dtype == bf else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == bf else b.view(torch.int32)), name
    del q1, k1, v1, z1, g1, b1
    starts = [int(s) for s in cu[:-1]]
    rng = np.random.default_rng(wk["seed"] + 2)
    tops = [t + j for t in (256, 512, 8192 + 256, 3 * 8192 - 256, T - 256) for j in range(3)]
    rows = sorted(set(tops + [s + j for s in starts for j in range(4)] + list(rng.choice(T, 24, replace=False))))
    sel = torch.tensor(rows, device="cuda")
    got = {n: host(t[0][sel]) for n, t in (("q", q2), ("k", k2), ("v", v2))}
    want = {n: [] for n in got}
    for m in rows:
        n = int(np.searchsorted(cu, m, side="right")) - 1
        s = starts[n]
        lo = max(s, m - 3)
        p = projection.project(x[lo:m + 1], w, H, d, d)
        X0 = None
        if lo == s and 0 <= init[n] < 2:
            X0 = X[init[n]:init[n] + 1]
        aq, ak, av = conv.activations(r16(p["q"]), r16(p["k"]), r16(p["v"]), conv_w, np.array([0, m + 1 - lo]), X0)
        for name, a in (("q", aq), ("k", ak), ("v", av)):
            want[name].append(a[-1])
    for name in ("q", "k", "v"):
        ref = np.stack(want[name])
        e, e_r = rel_l2(got[name], ref), per_row_max(got[name], ref)
        say(f"  {name}: {len(rows)} rows, rel-L2 {e:.3e}, worst row {e_r:.3e}")
        assert np.isfinite(got[name]).all() and e <= 1e-2 and e_r <= tol_row("bf16"), name
