"""Pins for the projection oracle (oracle/projection.py): brute-force loops,
the packed row order, the gate activations' closed forms, and the output
projection's loops and selection weights."""
import math

import numpy as np

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
