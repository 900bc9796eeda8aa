"""GPU parity of the fused input projections (kda_project_inputs) and the
output projection (kda_project_output) against the fp64 projection oracle,
and of both composed with the prefill.

Tolerances (relative L2, fp64): q, k, v, z and y are stored in bf16 (their
rounding dominates: about 1e-3 to 2e-3), bound 1e-2; g and beta are fp32 from
an fp32-accumulated GEMM, bound 1e-5.  The composed path must match the
oracle's projections rounded to bf16 and run through the oracle recurrence
within the bf16 prefill tolerances.
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


def run_gpu(shape, x, w):
    cfg = kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16)
    T = x.shape[0]
    H, dk, dv = shape.H, shape.dk, shape.dv
    xd, wd = dev(x, torch.bfloat16), dev(w, torch.bfloat16)
    o = dict(q=torch.full((T, H, dk), float("nan"), dtype=torch.bfloat16, device="cuda"),
             k=torch.full((T, H, dk), float("nan"), dtype=torch.bfloat16, device="cuda"),
             v=torch.full((T, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda"),
             z=torch.full((T, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda"),
             g=torch.full((T, H, dk), float("nan"), device="cuda"),
             beta=torch.full((T, H), float("nan"), device="cuda"))
    kda.kda_project_inputs(cfg, xd, wd, o["q"], o["k"], o["v"], o["z"], o["g"], o["beta"])
    torch.cuda.synchronize()
    return o


def run_output_gpu(shape, o, w):
    cfg = kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16)
    y = torch.full((o.shape[0], w.shape[0]), float("nan"), dtype=torch.bfloat16, device="cuda")
    kda.kda_project_output(cfg, dev(o, torch.bfloat16), dev(w, torch.bfloat16), y)
    torch.cuda.synchronize()
    return y


def check(o, ref, rows=None):
    sel = slice(None) if rows is None else rows
    for name in ("q", "k", "v", "z", "g", "beta"):
        got = host(o[name])[sel]
        e = rel_l2(got, ref[name])
        tol = 1e-2 if name in "qkvz" else 1e-5
        say(f"  {name}: rel-L2 {e:.3e} (tol {tol})")
        assert np.isfinite(got).all() and e <= tol, name


@pytest.mark.parametrize("H,d,T,Dm", [(2, 64, 300, 256), (4, 128, 1000, 1024), (3, 32, 129, 64), (1, 32, 1, 128),
                                       (2, 64, 257, 64)])
def test_project_matches_oracle(H, d, T, Dm):
    shape = wl.LayerShape(H, d, d)
    say(f"projection H={H} d={d} T={T} Dm={Dm}")
    x, w = wl.projection_inputs(50 + H, shape, T, Dm)
    o = run_gpu(shape, x, w)
    check(o, projection.project(x, w, H, d, d))


def test_project_full_size_sampled_rows():
    """The 4 x 8192 token projections (Dm 7168, H=32, d=128), every row on the
    GPU, 96 sampled rows through the oracle."""
    wk = wl.WORKLOADS["project_4x8k"]
    shape, T, Dm = wk["shape"], wk["T"], wk["Dm"]
    x, w = wl.projection_inputs(wk["seed"], shape, T, Dm)
    o = run_gpu(shape, x, w)
    rows = np.sort(np.random.default_rng(wk["seed"]).choice(T, 96, replace=False))
    check(o, projection.project(x[rows], w, shape.H, shape.dk, shape.dv), rows)


@pytest.mark.parametrize("H,dv,T,Dm", [(2, 64, 300, 200), (4, 128, 1000, 1024), (1, 64, 129, 7), (3, 64, 257, 513),
                                        (1, 64, 1, 256)])
def test_output_projection_matches_oracle(H, dv, T, Dm):
    shape = wl.LayerShape(H, dv, dv)
    say(f"output projection H={H} dv={dv} T={T} Dm={Dm}")
    o, w = wl.output_projection_inputs(70 + H, shape, T, Dm)
    y = host(run_output_gpu(shape, o, w))
    e = rel_l2(y, projection.output(o, w))
    say(f"  y: rel-L2 {e:.3e} (tol 1e-2)")
    assert np.isfinite(y).all() and e <= 1e-2


def test_output_projection_full_size_sampled_rows():
    """The 4 x 8192 token output projection (H=32, dv=128 -> Dm 7168), every
    row on the GPU, 96 sampled rows through the oracle."""
    wk = wl.WORKLOADS["project_4x8k"]
    shape, T, Dm = wk["shape"], wk["T"], wk["Dm"]
    o, w = wl.output_projection_inputs(wk["seed"], shape, T, Dm)
    y = host(run_output_gpu(shape, o, w))
    rows = np.sort(np.random.default_rng(wk["seed"] + 1).choice(T, 96, replace=False))
    e = rel_l2(y[rows], projection.output(o[rows], w))
    say(f"  y (96 rows): rel-L2 {e:.3e} (tol 1e-2); all rows finite: {np.isfinite(y).all()}")
    assert np.isfinite(y).all() and e <= 1e-2


def test_projections_feed_the_prefill():
    shape = wl.LayerShape(2, 64, 64)
    lengths = [200, 77]
    T, Dm = sum(lengths), 256
    x, w = wl.projection_inputs(60, shape, T, Dm)
    o = run_gpu(shape, x, w)
    base = wl.token_inputs(60, shape, 1, norm_w="random")          # conv and norm weights
    cfg = kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16)
    N = len(lengths)
    S = torch.zeros((2 * N, shape.H, shape.dk, shape.dv), device="cuda")
    X = torch.zeros((2 * N, shape.H, shape.C, 3), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, shape.H, shape.dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, N, T), dtype=torch.uint8, device="cuda")
    kda.kda_prefill_varlen(cfg, dev(wl.cu_seqlens(lengths).astype(np.int32)), o["q"], o["k"], o["v"], o["z"], o["g"],
                           o["beta"], dev(base.conv_w), dev(base.norm_w), S, X, dev(np.full(N, -1, np.int32)),
                           dev(np.arange(N, 2 * N, dtype=np.int32)), out, ws)
    torch.cuda.synchronize()
    p = projection.project(x, w, shape.H, shape.dk, shape.dv)
    r16 = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
    r = oracle.run(r16(p["q"]), r16(p["k"]), r16(p["v"]), r16(p["z"]), p["g"], p["beta"], base.conv_w, base.norm_w,
                   wl.cu_seqlens(lengths))
    e_o = rel_l2(host(out), r.out)
    e_s = rel_l2(host(S)[N:], r.S)
    # and on to the model width through the output projection
    _, w_o = wl.output_projection_inputs(61, shape, 1, 192)
    y = host(run_output_gpu(shape, host(out).astype(np.float32), w_o))
    e_y = rel_l2(y, projection.output(r.out, w_o))
    say(f"  projections -> prefill -> output projection: out {e_o:.3e} state {e_s:.3e} y {e_y:.3e}")
    assert e_o <= 1e-2 and e_s <= 5e-3 and e_y <= 1e-2


def test_routing_and_gate_maps_elementwise():
    """One-hot rows of x make the GEMM exact: y[m][n] = W[n][m mod Dm], one
    bf16 product.  q, k, v and z must then equal those weights bit for bit
    (which pins the column routing), and g and beta are checked element by
    element against the oracle's -softplus and logistic function of exactly
    those pre-activations.  Bound: the fp32 maps evaluate exp(-|y|) as
    exp2(-|y| log2 e); rounding the product costs the result up to |y| 2^-24
    relative and the fp32 constant log2 e (0.22 2^-24 off) another
    0.22 |y| 2^-24, to which exp2, the reciprocal and the log1p series add a
    few ulp: |got - ref| <= (1.25 |y| + 8) 2^-24 |ref|."""
    H, d, Dm, T = 2, 32, 64, 320
    shape = wl.LayerShape(H, d, d)
    N = projection.rows(H, d, d)
    rng = np.random.default_rng(31)
    w = np.concatenate([rng.uniform(-60.0, 40.0, (N, Dm // 2)), 3.0 * rng.standard_normal((N, Dm // 2))], 1)
    w[:, 0] = 0.0
    w = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).double().numpy()   # exact bf16 values
    x = np.zeros((T, Dm))
    x[np.arange(T), np.arange(T) % Dm] = 1.0
    o = run_gpu(shape, x, w)
    ref = projection.project(x, w, H, d, d)
    for name in ("q", "k", "v", "z"):
        got = host(o[name])
        assert np.array_equal(got, ref[name]), name
    y_g = x @ w[2 * H * d + 2 * H * d:3 * H * d + 2 * H * d].T                 # gate pre-activations [T][H d]
    y_b = x @ w[3 * H * d + 2 * H * d:].T                                      # beta pre-activations [T][H]
    for name, y in (("g", y_g.reshape(T, H, d)), ("beta", y_b)):
        got, r = host(o[name]), ref[name]
        err = np.abs(got - r)
        bound = (1.25 * np.abs(y) + 8.0) * 2.0 ** -24 * np.abs(r)
        worst = float(np.max(err / np.maximum(np.abs(r), 1e-300)))
        say(f"  {name}: worst relative error {worst:.3e}, worst error / bound {float(np.max(err / bound)):.3f}")
        assert np.isfinite(got).all() and (err <= bound).all(), name
