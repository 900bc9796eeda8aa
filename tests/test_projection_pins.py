"""Pins for the projection oracle (oracle/projection.py): brute-force loops,
the packed row order, the gate activations' closed forms, and the output
projection's loops and selection weights."""
import math

import numpy as np
from scipy.special import expit, log_expit

from oracle import projection


def test_brute_force_tiny():
    rng = np.random.default_rng(100)
    T, Dm, H, dk, dv = 3, 5, 2, 2, 3
    N = projection.rows(H, dk, dv)
    x = rng.standard_normal((T, Dm))
    w = rng.standard_normal((N, Dm))
    o = projection.project(x, w, H, dk, dv)
    for t in range(T):
        y = [sum(x[t][i] * w[n][i] for i in range(Dm)) for n in range(N)]
        r = 0
        for name, width in (("q", dk), ("k", dk), ("v", dv), ("z", dv), ("g", dk)):
            for h in range(H):
                for j in range(width):
                    want = y[r]
                    if name == "g":
                        want = -math.log1p(math.exp(want))
                    assert abs(o[name][t, h, j] - want) <= 1e-12 * (1 + abs(want)), (name, t, h, j)
                    r += 1
        for h in range(H):
            assert abs(o["beta"][t, h] - 1.0 / (1.0 + math.exp(-y[r]))) <= 1e-14
            r += 1
        assert r == N


def test_selection_rows_and_gate_closed_forms():
    H, dk, dv = 2, 3, 4
    N = projection.rows(H, dk, dv)
    Dm = N
    w = np.eye(N)                                   # row n picks x[:, n]
    x = np.zeros((2, Dm))
    x[1] = np.arange(Dm) * 0.25 - 3.0
    o = projection.project(x, w, H, dk, dv)
    np.testing.assert_array_equal(o["q"][1].ravel(), x[1, :H * dk])
    np.testing.assert_array_equal(o["z"][1].ravel(), x[1, 2 * H * dk + H * dv:2 * H * dk + 2 * H * dv])
    # x = 0: g = -ln 2, beta = 1/2 exactly
    np.testing.assert_allclose(o["g"][0], -math.log(2.0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(o["beta"][0], 0.5, rtol=0, atol=1e-15)
    # large pre-activations: -softplus(a) -> -a, softplus(-a) -> exp(-a)
    big = projection.softplus(np.array([40.0, -40.0]))
    assert abs(big[0] - 40.0) < 1e-15 and abs(big[1] - math.exp(-40.0)) < 1e-30


def test_output_projection_brute_force_and_selection():
    rng = np.random.default_rng(101)
    T, H, dv, Dm = 3, 2, 3, 4
    o = rng.standard_normal((T, H, dv))
    w = rng.standard_normal((Dm, H * dv))
    y = projection.output(o, w)
    assert y.shape == (T, Dm)
    for t in range(T):
        for m in range(Dm):
            want = sum(o[t, h, j] * w[m, h * dv + j] for h in range(H) for j in range(dv))
            assert abs(y[t, m] - want) <= 1e-12 * (1 + abs(want)), (t, m)
    # one-hot rows: output m reads head h, channel j (head-major flattening of o)
    sel = np.zeros((H * dv, H * dv))
    for h in range(H):
        for j in range(dv):
            sel[j * H + h, h * dv + j] = 1.0         # output j*H+h <- (h, j)
    ys = projection.output(o, sel)
    for h in range(H):
        for j in range(dv):
            np.testing.assert_array_equal(ys[:, j * H + h], o[:, h, j])



def test_projection_gate_maps_against_scipy_and_definitions():
    """softplus against its definition log(1 + e^y) (written with log1p,
    accurate in fp64 up to y = 30) and against scipy's log-sigmoid
    (softplus(y) = -log_expit(-y)) over a wide range; sigmoid against
    scipy's expit."""
    y = np.linspace(-700.0, 700.0, 20001)
    np.testing.assert_allclose(projection.softplus(y), -log_expit(-y), rtol=1e-14, atol=1e-300)
    mid = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(projection.softplus(mid), np.log1p(np.exp(mid)), rtol=1e-13)
    np.testing.assert_allclose(projection.sigmoid(y), expit(y), rtol=1e-13, atol=1e-300)
    # softplus(y) - softplus(-y) = y, softplus(0) = log 2
    np.testing.assert_allclose(projection.softplus(mid) - projection.softplus(-mid), mid, rtol=0, atol=1e-12)
    assert projection.softplus(0.0) == np.log(2.0)


def test_projection_routes_weight_rows_to_tensors():
    """With x the identity, y = W^T, so every output element is one weight:
    the rows of W are q (H dk), k (H dk), v (H dv), z (H dv), g (H dk) and
    beta (H), each block head-major."""
    H, dk, dv = 2, 3, 4
    N = projection.rows(H, dk, dv)
    assert N == H * (3 * dk + 2 * dv) + H
    w = np.arange(N * N, dtype=np.float64).reshape(N, N) / (N * N) - 0.5
    out = projection.project(np.eye(N), w, H, dk, dv)
    o = 0
    for name, width in (("q", dk), ("k", dk), ("v", dv), ("z", dv)):
        for h in range(H):
            for c in range(width):
                np.testing.assert_array_equal(out[name][:, h, c], w[o + h * width + c])
        o += H * width
    for h in range(H):
        for c in range(dk):
            np.testing.assert_allclose(out["g"][:, h, c], -np.logaddexp(0.0, w[o + h * dk + c]), rtol=1e-14)
    o += H * dk
    for h in range(H):
        np.testing.assert_allclose(out["beta"][:, h], expit(w[o + h]), rtol=1e-14)
    assert (out["g"] < 0).all() and ((out["beta"] > 0) & (out["beta"] < 1)).all()
