"""Pins for the fp64 oracle: closed forms, invariants and brute-force checks.

The pages print no equation and no worked example for the KDA layer, so every
pin here comes from the mathematics of the gated delta rule with per-channel
decay (S_t = (I - b k k^T) Diag(exp g) S_{t-1} + b k v^T, o_t = S_t^T q_t) and
of the maps around it.  Each one is chosen so that a plausible mistake in the
oracle fails it: a dropped decay, decay applied after the delta instead of
before, reading the state before the update, a transposed state, a wrong conv
tap order or conv-state shift, a missing eps, a wrong checkpoint position.

SiLU and the logistic function come from scipy.special here, not from the
oracle.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def silu(x):
    return x * expit(x)


def ident_conv(H, dk, dv, W=4):
    """Conv weights that pass the current raw input through (tap W-1 = 1)."""
    w = np.zeros((H, 2 * dk + dv, W))
    w[:, :, W - 1] = 1.0
    return w


def rand_inputs(rng, T, H, dk, dv, W=4, g_scale=1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    z = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, H, dk))) * g_scale
    beta = expit(rng.standard_normal((T, H)))
    conv_w = rng.standard_normal((H, 2 * dk + dv, W)) * 0.5
    norm_w = 0.5 + np.abs(rng.standard_normal(dv))
    return q, k, v, z, g, beta, conv_w, norm_w


def basis(dim, idx, scale=2.0):
    e = np.zeros(dim)
    e[idx] = scale
    return e


# ---------------------------------------------------------------- recurrence

def test_beta_zero_is_pure_decay():
    """beta = 0: the delta term vanishes and S_T = Diag(exp(sum_t g_t)) S_0."""
    rng = np.random.default_rng(10)
    T, H, dk, dv = 37, 2, 8, 5
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, dk, dv))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0)
    expect = np.exp(g.sum(0))[:, :, None] * S0[0]
    np.testing.assert_allclose(r.S[0], expect, rtol=1e-13, atol=0)


def test_basis_keys_reduce_to_rowwise_ema():
    """With keys and queries on the standard basis, row i of S evolves as
    r <- exp(g_i) r, then r <- (1-b) r + b v_hat on the tokens whose key is e_i;
    the readout is the row picked by the query, after the update.  This pins
    the decay-before-delta order, the state orientation and the post-update
    readout."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 1, 6, 4
    _, _, v, z, g, beta, _, nw = rand_inputs(rng, T, H, dk, dv, g_scale=0.4)
    ki = rng.integers(0, dk, T)
    qi = rng.integers(0, dk, T)
    q = np.stack([basis(dk, i) for i in qi])[:, None, :]
    k = np.stack([basis(dk, i, 3.0) for i in ki])[:, None, :]
    cw = ident_conv(H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0, l2_eps=0.0, rms_eps=0.0)
    rows = S0[0, 0].copy()
    vh = silu(v[:, 0])
    for t in range(T):
        rows *= np.exp(g[t, 0])[:, None]
        i = ki[t]
        rows[i] = (1 - beta[t, 0]) * rows[i] + beta[t, 0] * vh[t]
        o = rows[qi[t]]
        y = o / np.sqrt(np.mean(o * o)) * nw * expit(z[t, 0])
        np.testing.assert_allclose(r.out[t, 0], y, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r.S[0, 0], rows, rtol=1e-12, atol=1e-15)


def test_unit_write_recalls_value():
    """g = 0, b = 1 and a unit key: after the write S_t^T k_t = v_hat_t.  With
    q = k the readout therefore returns v_hat_t at every token."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 30, 2, 16, 8
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    g[:] = 0.0
    beta[:] = 1.0
    cw[:, :dk] = cw[:, dk:2 * dk]          # q channels convolve like k channels
    q = k.copy()
    S0 = rng.standard_normal((1, H, dk, dv))
    X0 = rng.standard_normal((1, H, 2 * dk + dv, 3))
    X0[:, :, :dk] = X0[:, :, dk:2 * dk]
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0, X0=X0, l2_eps=0.0, rms_eps=0.0)
    # v_hat from an independent evaluation of the conv with scipy's SiLU
    xs = np.concatenate([X0[0].transpose(2, 0, 1), np.concatenate([q, k, v], 2)], 0)
    for h in range(H):
        for t in range(T):
            yconv = np.einsum("cm,mc->c", cw[h], xs[t:t + 4, h])
            vh = silu(yconv[2 * dk:])
            y = vh / np.sqrt(np.mean(vh * vh)) * nw * expit(z[t, h])
            np.testing.assert_allclose(r.out[t, h], y, rtol=1e-10, atol=1e-13)
        kh = silu(np.einsum("cm,mc->c", cw[h], xs[T - 1:T + 3, h])[dk:2 * dk])
        kh /= np.linalg.norm(kh)
        np.testing.assert_allclose(r.S[0, h].T @ kh, vh, rtol=1e-10, atol=1e-13)


def test_householder_preserves_gram():
    """b = 2, g = 0, v = 0: each step is the reflection I - 2 k k^T, so
    S^T S is preserved (and ||S||_F with it)."""
    rng = np.random.default_rng(13)
    T, H, dk, dv = 50, 2, 12, 7
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    v[:] = 0.0
    g[:] = 0.0
    beta[:] = 2.0
    S0 = rng.standard_normal((1, H, dk, dv))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0, l2_eps=0.0)
    for h in range(H):
        np.testing.assert_allclose(r.S[0, h].T @ r.S[0, h], S0[0, h].T @ S0[0, h],
                                   rtol=1e-11, atol=1e-12)
    assert not np.allclose(r.S, S0)     # the state did move


def test_full_forget_keeps_last_write():
    """exp(g) = 0 (g = -inf) wipes the state before each write: S_T = b k_hat v_hat^T."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 9, 2, 8, 6
    q, k, v, z, g, beta, _, nw = rand_inputs(rng, T, H, dk, dv)
    g[:] = -np.inf
    cw = ident_conv(H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0, l2_eps=0.0)
    for h in range(H):
        kh = silu(k[-1, h]) / np.linalg.norm(silu(k[-1, h]))
        np.testing.assert_allclose(r.S[0, h], beta[-1, h] * np.outer(kh, silu(v[-1, h])),
                                   rtol=1e-12, atol=1e-15)


def test_one_token_closed_form_with_eps():
    """One token from a zero state: o = b (q_hat . k_hat) v_hat.  With q = k,
    q_hat . k_hat = s / (s + eps_l2) (s = sum of squares after SiLU), and the
    gated RMSNorm gives y = o / sqrt(mean(o^2) + eps_rms) * w * sigmoid(z).
    Large eps values make both eps terms visible."""
    rng = np.random.default_rng(15)
    H, dk, dv = 3, 16, 8
    q, k, v, z, g, beta, _, nw = rand_inputs(rng, 1, H, dk, dv)
    q = k.copy()
    cw = ident_conv(H, dk, dv)
    l2e, rmse = 0.7, 0.05
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, 1], l2_eps=l2e, rms_eps=rmse)
    for h in range(H):
        a = silu(k[0, h])
        s = np.sum(a * a)
        o = beta[0, h] * s / (s + l2e) * silu(v[0, h])
        y = o / np.sqrt(np.mean(o * o) + rmse) * nw * expit(z[0, h])
        np.testing.assert_allclose(r.out[0, h], y, rtol=1e-13)


def test_scalar_head_closed_form():
    """dk = dv = 1: the state is a scalar s; with l2_eps = 0 the normalised key
    and query are the signs of their SiLU outputs, and with rms_eps = 0 the
    RMSNorm of a scalar is its sign: y = sign(s q_hat) w sigmoid(z)."""
    rng = np.random.default_rng(16)
    T = 25
    q, k, v, z, g, beta, _, nw = rand_inputs(rng, T, 1, 1, 1)
    cw = ident_conv(1, 1, 1)
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], l2_eps=0.0, rms_eps=0.0)
    s = 0.0
    for t in range(T):
        kh = np.sign(silu(k[t, 0, 0]))
        qh = np.sign(silu(q[t, 0, 0]))
        s = np.exp(g[t, 0, 0]) * s
        s = s + kh * beta[t, 0] * (silu(v[t, 0, 0]) - s * kh)
        assert r.out[t, 0, 0] == pytest.approx(np.sign(s * qh) * nw[0] * expit(z[t, 0, 0]), rel=1e-13)
    assert r.S[0, 0, 0, 0] == pytest.approx(s, rel=1e-12)


# ---------------------------------------------------------------- conv

@pytest.mark.parametrize("tap", [0, 1, 2, 3])
def test_conv_tap_order_and_state_shift(tap):
    """Single-tap conv weights pick one input of the window: tap m reads the
    raw input m-3 tokens back (tap 3 is the current token), and for the first
    tokens that input comes from the conv state, oldest first.  The final conv
    state holds the last W-1 raw inputs, oldest first.  The value path is
    observed through a full-forget, unit-write readout that returns v_hat."""
    rng = np.random.default_rng(20 + tap)
    T, H, dk, dv = 10, 1, 4, 6
    _, _, v, z, g, beta, _, nw = rand_inputs(rng, T, H, dk, dv)
    kq = np.stack([basis(dk, t % dk) for t in range(T)])[:, None, :]
    q, k = kq.copy(), kq.copy()
    cw = ident_conv(H, dk, dv)
    cw[:, 2 * dk:, :] = 0.0
    cw[:, 2 * dk:, tap] = 1.0
    g[:] = -np.inf
    beta[:] = 1.0
    z[:] = 40.0                                    # sigmoid(z) == 1.0 in double
    nw[:] = 1.0
    X0 = rng.standard_normal((1, H, 2 * dk + dv, 3))
    X0[:, :, :2 * dk] = 0.0
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], X0=X0, l2_eps=0.0, rms_eps=0.0)
    hist = np.concatenate([X0[0, 0, 2 * dk:].T, v[:, 0]], 0)   # [3+T][dv], oldest first
    for t in range(T):
        src = hist[t + tap]                        # window of token t starts at hist[t]
        vh = silu(src)
        np.testing.assert_allclose(r.out[t, 0], vh / np.sqrt(np.mean(vh * vh)), rtol=1e-12)
    np.testing.assert_array_equal(r.X[0, 0, 2 * dk:], hist[-3:].T)
    np.testing.assert_array_equal(r.X[0, 0, :dk], q[-3:, 0].T)
    np.testing.assert_array_equal(r.X[0, 0, dk:2 * dk], k[-3:, 0].T)


def test_conv_state_shorter_than_window():
    """A sequence of 2 tokens keeps one old conv-state entry and the 2 new
    raw inputs."""
    rng = np.random.default_rng(30)
    T, H, dk, dv = 2, 2, 4, 4
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    X0 = rng.standard_normal((1, H, 2 * dk + dv, 3))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], X0=X0)
    x = np.concatenate([q, k, v], 2)               # [T][H][C]
    np.testing.assert_array_equal(r.X[0][:, :, 0], X0[0][:, :, 2])
    np.testing.assert_array_equal(r.X[0][:, :, 1], x[0])
    np.testing.assert_array_equal(r.X[0][:, :, 2], x[1])


# ---------------------------------------------------------------- chunked form

@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
@pytest.mark.parametrize("start", [0, 45])
def test_chunked_form_equals_recurrence(chunk, start):
    """The chunked WY/UT form (independent NumPy code) reproduces the
    token-by-token recurrence, from a nonzero state, with chunks aligned to
    absolute position."""
    rng = np.random.default_rng(40 + chunk)
    T, H, dk, dv = 200, 2, 16, 12
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv, g_scale=0.05)
    S0 = rng.standard_normal((1, H, dk, dv)) * 0.3
    X0 = rng.standard_normal((1, H, 2 * dk + dv, 3))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], start_pos=[start], S0=S0, X0=X0)
    for h in range(H):
        y, S, X = chunked.run_sequence(q[:, h], k[:, h], v[:, h], z[:, h], g[:, h], beta[:, h],
                                       cw[h], nw, S0[0, h], X0[0, h], chunk=chunk, start_pos=start)
        np.testing.assert_allclose(r.out[:, h], y, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r.S[0, h], S, rtol=1e-10, atol=1e-12)
        np.testing.assert_array_equal(r.X[0, h], X)


def test_chunked_form_strong_decay():
    """Same check with the workloads' gate (mean log-decay about -0.8 per
    token per channel), where a chunk forgets almost everything."""
    rng = np.random.default_rng(50)
    T, H, dk, dv = 130, 1, 16, 16
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    r = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0)
    y, S, X = chunked.run_sequence(q[:, 0], k[:, 0], v[:, 0], z[:, 0], g[:, 0], beta[:, 0],
                                   cw[0], nw, S0[0, 0], np.zeros((2 * dk + dv, 3)), chunk=64)
    np.testing.assert_allclose(r.out[:, 0], y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r.S[0, 0], S, rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- split / checkpoints

def test_split_invariance_bitwise():
    """Running L tokens equals running p tokens and then the remaining L-p from
    the resulting state and conv state, bit for bit (same order of operations)."""
    rng = np.random.default_rng(60)
    T, H, dk, dv = 90, 3, 8, 8
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    whole = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T])
    for p in (1, 33, 64, 89):
        a = oracle.run(q[:p], k[:p], v[:p], z[:p], g[:p], beta[:p], cw, nw, [0, p])
        b = oracle.run(q[p:], k[p:], v[p:], z[p:], g[p:], beta[p:], cw, nw, [0, T - p],
                       start_pos=[p], S0=a.S, X0=a.X)
        np.testing.assert_array_equal(np.concatenate([a.out, b.out]), whole.out)
        np.testing.assert_array_equal(b.S, whole.S)
        np.testing.assert_array_equal(b.X, whole.X)


def test_checkpoints_positions_and_contents():
    """Checkpoints land at the multiples of the interval strictly inside the
    sequence plus its end, in order, and each holds the state after exactly
    that many tokens (compared with split runs)."""
    rng = np.random.default_rng(61)
    lens = [50, 7, 0, 64, 33]
    starts = [10, 60, 5, 0, 127]
    T = sum(lens)
    H, dk, dv = 2, 8, 4
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    X0 = rng.standard_normal((len(lens), H, 2 * dk + dv, 3))
    N = 16
    r = oracle.run(q, k, v, z, g, beta, cw, nw, cu, start_pos=starts, S0=S0, X0=X0, ckpt_interval=N)
    expect_pos = []
    for L, s in zip(lens, starts):
        ps = [p for p in range(s + 1, s + L + 1) if p % N == 0 or p == s + L]
        expect_pos += ps
        assert oracle.num_checkpoints(s, L, N) == len(ps)
    assert r.ckpt_pos == expect_pos
    slot = 0
    for n, (L, s) in enumerate(zip(lens, starts)):
        assert r.ckpt_base[n] == slot
        for p in range(s + 1, s + L + 1):
            if p % N == 0 or p == s + L:
                m = p - s
                t0 = cu[n]
                sl = slice(t0, t0 + m)
                a = oracle.run(q[sl], k[sl], v[sl], z[sl], g[sl], beta[sl], cw, nw, [0, m],
                               start_pos=[s], S0=S0[n:n + 1], X0=X0[n:n + 1])
                np.testing.assert_array_equal(r.ckpt_S[slot], a.S[0])
                np.testing.assert_array_equal(r.ckpt_X[slot], a.X[0])
                slot += 1
    assert slot == len(r.ckpt_S)
    # the empty sequence leaves its state untouched
    np.testing.assert_array_equal(r.S[2], S0[2])
    np.testing.assert_array_equal(r.X[2], X0[2])


@pytest.mark.parametrize("start,length,interval", [
    (0, 64, 64), (0, 65, 64), (1, 63, 64), (63, 1, 64), (64, 0, 64), (0, 100, 0),
    (4095, 8193, 4096), (32768 * 3, 1 << 20, 32768), (5, 3, 4),
])
def test_num_checkpoints_brute_force(start, length, interval):
    expect = 0
    if interval > 0 and length > 0:
        expect = sum(1 for p in range(start + 1, start + length) if p % interval == 0) + 1
    assert oracle.num_checkpoints(start, length, interval) == expect


def test_decode_steps_equal_packed_run():
    """Stepping B sequences one token at a time equals running each sequence
    whole, bitwise."""
    rng = np.random.default_rng(62)
    steps, B, H, dk, dv = 12, 3, 2, 8, 8
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, steps * B, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    X0 = rng.standard_normal((B, H, 2 * dk + dv, 3))
    shp = lambda a: a.reshape((steps, B) + a.shape[1:])
    out, S, X = oracle.decode_steps(shp(q), shp(k), shp(v), shp(z), shp(g), shp(beta), cw, nw, S0, X0)
    pk = lambda a: shp(a).swapaxes(0, 1).reshape(a.shape)   # sequence-major packing
    r = oracle.run(pk(q), pk(k), pk(v), pk(z), pk(g), pk(beta), cw, nw,
                   np.arange(B + 1) * steps, S0=S0, X0=X0)
    np.testing.assert_array_equal(out.swapaxes(0, 1).reshape(r.out.shape), r.out)
    np.testing.assert_array_equal(S, r.S)
    np.testing.assert_array_equal(X, r.X)


def test_golden_hand_worked_example():
    """A 2x2 example worked by hand (tests/golden/hand_2x2.json)."""
    with open(os.path.join(GOLDEN, "hand_2x2.json")) as f:
        ex = json.load(f)
    T = len(ex["key_index"])
    dk = dv = 2
    rng = np.random.default_rng(ex["v_seed"])
    v = rng.standard_normal((T, 1, dv))
    vh = silu(v[:, 0])
    k = np.stack([basis(dk, i) for i in ex["key_index"]])[:, None, :]
    q = np.stack([basis(dk, i) for i in ex["query_index"]])[:, None, :]
    g = np.tile(np.log(np.array(ex["decay"]))[None, None, :], (T, 1, 1))
    beta = np.full((T, 1), ex["beta"])
    z = np.full((T, 1, dv), 40.0)
    r = oracle.run(q, k, v, z, g, beta, ident_conv(1, dk, dv), np.ones(dv), [0, T],
                   l2_eps=0.0, rms_eps=0.0)
    # expected state rows and outputs as combinations of the v_hat_t
    Sx = np.array(ex["final_state_coeffs"]) @ vh        # [dk][dv]
    np.testing.assert_allclose(r.S[0, 0], Sx, rtol=1e-14, atol=1e-15)
    for t, coeffs in enumerate(ex["output_coeffs"]):
        o = np.array(coeffs) @ vh
        np.testing.assert_allclose(r.out[t, 0], o / np.sqrt(np.mean(o * o)), rtol=1e-13)


# ---------------------------------------------------------------- bf16 state storage

def test_round_bf16_matches_library_conversion():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even) on random values, exact ties, values next
    to ties, bf16 subnormals and large magnitudes."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(90)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000)
    b = rng.standard_normal(4000).astype(np.float32)
    bits = b.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)                 # exactly halfway
    near = np.concatenate([(bits | np.uint32(0x7FFF)).view(np.float32),
                           (bits | np.uint32(0x8001)).view(np.float32)])
    sub = (rng.standard_normal(2000) * 2.0 ** -128).astype(np.float32)   # bf16 subnormal range
    for arr in (x, ties, near, sub):
        ref = torch.from_numpy(arr).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(oracle.round_bf16(arr), ref)


def test_state_round_only_at_the_end_without_checkpoints():
    """Without checkpoints the state is stored once, at the end: the outputs are
    those of the unrounded run and the final state is its rounding."""
    rng = np.random.default_rng(91)
    T, H, dk, dv = 70, 2, 8, 8
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv, g_scale=0.1)
    S0 = oracle.round_bf16(rng.standard_normal((1, H, dk, dv)) * 0.3)
    a = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0)
    b = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], S0=S0, state_round=True)
    np.testing.assert_array_equal(b.out, a.out)
    np.testing.assert_array_equal(b.S, oracle.round_bf16(a.S))
    assert not np.array_equal(b.S, a.S)


def test_state_round_continues_from_each_checkpoint():
    """With bf16 storage a run with checkpoints equals, bit for bit, the runs
    between consecutive checkpoint positions chained through their (rounded)
    final states; every checkpoint is bf16-representable."""
    rng = np.random.default_rng(92)
    T, H, dk, dv, I = 150, 2, 8, 8, 40
    q, k, v, z, g, beta, cw, nw = rand_inputs(rng, T, H, dk, dv, g_scale=0.1)
    whole = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], start_pos=[7], ckpt_interval=I, state_round=True)
    cuts = [0] + [p - 7 for p in whole.ckpt_pos]                      # 33, 73, 113, 150
    S, X, outs = None, None, []
    for j in range(len(cuts) - 1):
        a, b = cuts[j], cuts[j + 1]
        r = oracle.run(q[a:b], k[a:b], v[a:b], z[a:b], g[a:b], beta[a:b], cw, nw, [0, b - a],
                       start_pos=[7 + a], S0=S, X0=X, state_round=True)
        np.testing.assert_array_equal(whole.ckpt_S[j], r.S[0])
        S, X = r.S, r.X
        outs.append(r.out)
    np.testing.assert_array_equal(np.concatenate(outs), whole.out)
    np.testing.assert_array_equal(whole.S, S)
    np.testing.assert_array_equal(whole.ckpt_S, oracle.round_bf16(whole.ckpt_S))
    # and the unrounded run differs after the first checkpoint
    plain = oracle.run(q, k, v, z, g, beta, cw, nw, [0, T], start_pos=[7], ckpt_interval=I)
    np.testing.assert_array_equal(plain.out[:cuts[1]], whole.out[:cuts[1]])
    assert not np.array_equal(plain.out[cuts[1]:], whole.out[cuts[1]:])


# ---------------------------------------------------------------------------
# The stand-alone conv oracle (oracle/conv.py), the reference for a fused
# front end's post-conv activations.

def _conv_case(seed=7):
    rng = np.random.default_rng(seed)
    H, C = 2, 6
    lengths = [5, 1, 0, 9, 2]
    T = sum(lengths)
    x = rng.standard_normal((T, H, C))
    X0 = rng.standard_normal((len(lengths), H, C, 3))
    return x, X0, np.concatenate([[0], np.cumsum(lengths)]), H, C


def test_conv_oracle_current_tap_is_identity():
    """w = e3 (only the current token's tap): the pre-activation is the raw
    input, at sequence starts too."""
    from oracle import conv
    x, X0, cu, H, C = _conv_case()
    w = np.zeros((H, C, 4))
    w[:, :, 3] = 1.0
    np.testing.assert_array_equal(conv.preactivation(x, w, cu, X0), x)


def test_conv_oracle_oldest_tap_reads_the_conv_state():
    """w = e0 (the token three back): inside a sequence the raw input three
    rows up; for its first three tokens the initial conv state, index 0 for
    the first token, 1 for the second, 2 for the third (pins the tap order and
    the conv-state order against a shift or a reversal)."""
    from oracle import conv
    x, X0, cu, H, C = _conv_case()
    w = np.zeros((H, C, 4))
    w[:, :, 0] = 1.0
    y = conv.preactivation(x, w, cu, X0)
    for n in range(len(cu) - 1):
        for t in range(int(cu[n]), int(cu[n + 1])):
            r = t - int(cu[n])
            want = X0[n][:, :, r] if r < 3 else x[t - 3]
            np.testing.assert_array_equal(y[t], want)


def test_conv_oracle_is_linear_in_the_weights_and_silu_closed_form():
    from oracle import conv
    x, X0, cu, H, C = _conv_case(8)
    rng = np.random.default_rng(9)
    w1, w2 = rng.standard_normal((H, C, 4)), rng.standard_normal((H, C, 4))
    y12 = conv.preactivation(x, w1 + w2, cu, X0)
    np.testing.assert_allclose(y12, conv.preactivation(x, w1, cu, X0) + conv.preactivation(x, w2, cu, X0),
                               rtol=0, atol=1e-12)
    assert conv.silu(0.0) == 0.0
    assert abs(conv.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert abs(conv.silu(-40.0)) < 1e-15 and abs(conv.silu(40.0) - 40.0) < 1e-12
    # the layer's channel order: q, then k, then v per head
    q, k, v = x[:, :, :2], x[:, :, 2:4], x[:, :, 4:]
    w = np.zeros((H, C, 4))
    w[:, :, 3] = 1.0
    aq, ak, av = conv.activations(q, k, v, w, cu, X0)
    np.testing.assert_allclose(np.concatenate([aq, ak, av], axis=2), conv.silu(x), rtol=0, atol=0)



def test_conv_oracle_brute_force_every_tap():
    """Random weights on all four taps against scalar loops: tap j multiplies
    the raw input 3 - j tokens back; a token before the sequence's first one
    comes from the initial conv state, slot 3 - (start - token) (slot 2 is the
    token just before the start)."""
    from oracle import conv
    x, X0, cu, H, C = _conv_case(11)
    w = np.random.default_rng(12).standard_normal((H, C, 4))
    y = conv.preactivation(x, w, cu, X0)
    for n in range(len(cu) - 1):
        s0 = int(cu[n])
        for t in range(s0, int(cu[n + 1])):
            for h in range(H):
                for c in range(C):
                    acc = 0.0
                    for j in range(4):
                        src = t - 3 + j                       # token feeding tap j
                        val = x[src, h, c] if src >= s0 else X0[n, h, c, 3 - (s0 - src)]
                        acc += w[h, c, j] * val
                    assert abs(y[t, h, c] - acc) <= 1e-12, (n, t, h, c)


def test_conv_oracle_split_sequence_invariance():
    """A sequence cut in two gives the same pre-activations when the second
    part starts from a conv state holding the first part's last three raw
    inputs (the state a checkpoint at the cut stores)."""
    from oracle import conv
    rng = np.random.default_rng(13)
    H, C, T, cut = 2, 5, 17, 7
    x = rng.standard_normal((T, H, C))
    X0 = rng.standard_normal((1, H, C, 3))
    w = rng.standard_normal((H, C, 4))
    whole = conv.preactivation(x, w, np.array([0, T]), X0)
    X1 = np.transpose(x[cut - 3:cut], (1, 2, 0))[None]          # [1][H][C][3], oldest first
    tail = conv.preactivation(x[cut:], w, np.array([0, T - cut]), X1)
    np.testing.assert_allclose(tail, whole[cut:], rtol=0, atol=1e-13)
