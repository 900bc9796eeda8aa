"""Shared harness for the prefill GPU tests: one kda_prefill_varlen call with
its pools, slots and checkpoint buffers, and the matching oracle run."""
import numpy as np
import torch

import linear_attention_recurrence_decode_amd as kda
import oracle
import workloads as wl
from tests.helpers import TOL_STATE_PER_CHAIN, dev, host, per_chain_max, per_row_max, rel_l2, say, tol_row, tols


def cfg_for(shape, state_dtype=kda.KDA_F32):
    return kda.Config(shape.H, shape.dk, shape.dv, kda.KDA_BF16 if shape.act == "bf16" else kda.KDA_F32,
                      state_dtype=state_dtype)


class Run:
    """One prefill call on the GPU with pools, slots and checkpoint buffers."""

    def __init__(self, shape, inp, lengths, *, starts=None, S0=None, X0=None, interval=0,
                 pool_extra=3, seq_order=None, flags=0, state_dtype=kda.KDA_F32):
        self.shape, self.inp = shape, inp
        H, dk, dv, C = shape.H, shape.dk, shape.dv, shape.C
        N = len(lengths)
        self.N, self.lengths = N, list(lengths)
        self.starts = [0] * N if starts is None else list(starts)
        self.cfg = cfg_for(shape, state_dtype)
        act = self.cfg.torch_act
        cu = wl.cu_seqlens(lengths)
        self.cu = cu
        nslots = 2 * N + pool_extra
        S = np.zeros((nslots, H, dk, dv), np.float32)
        X = np.zeros((nslots, H, C, 3), np.float32)
        init = np.full(N, -1, np.int32)
        if S0 is not None:
            init = np.arange(N, dtype=np.int32)
            S[:N] = S0
            X[:N] = X0
        final = np.arange(N, 2 * N, dtype=np.int32)
        self.init, self.final = init, final
        self.Sd, self.Xd = dev(S, self.cfg.torch_state), dev(X, act)
        counts = [oracle.num_checkpoints(s, L, interval) for s, L in zip(self.starts, lengths)]
        base = np.zeros(N, np.int32)
        if N:
            base[1:] = np.cumsum(counts)[:-1]
        self.base, self.nck = base, int(sum(counts))
        self.interval = interval
        self.ckS = torch.full((max(self.nck, 1), H, dk, dv), float("nan"), dtype=self.cfg.torch_state, device="cuda")
        self.ckX = torch.zeros((max(self.nck, 1), H, C, 3), dtype=act, device="cuda")
        T = int(cu[-1])
        self.q, self.k, self.v, self.z = (dev(a, act) for a in (inp.q, inp.k, inp.v, inp.z))
        self.g, self.beta = dev(inp.g), dev(inp.beta)
        self.conv_w, self.norm_w = dev(inp.conv_w), dev(inp.norm_w)
        self.out = torch.full((T, H, dv), float("nan"), dtype=act, device="cuda")
        self.flags = flags
        nbytes = kda.kda_prefill_workspace_bytes(self.cfg, N, T, interval, flags)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def launch(self, static: bool = False):
        """Run the call; static=True goes through kda_prefill_varlen_static
        (the library's static workspace) instead of the allocated one."""
        args = (self.cfg, dev(self.cu.astype(np.int32)), self.q, self.k, self.v, self.z,
                self.g, self.beta, self.conv_w, self.norm_w, self.Sd, self.Xd,
                dev(self.init), dev(self.final), self.out)
        kw = dict(start_pos=dev(np.asarray(self.starts, np.int64)), ckpt_interval=self.interval,
                  ckpt_state=self.ckS if self.interval else None,
                  ckpt_conv=self.ckX if self.interval else None,
                  ckpt_base=dev(self.base) if self.interval else None, flags=self.flags)
        if static:
            kda.kda_prefill_varlen_static(*args, **kw)
        else:
            kda.kda_prefill_varlen(*args, self.ws, **kw)
        torch.cuda.synchronize()
        return self

    def final_state(self):
        return host(self.Sd)[self.final], host(self.Xd)[self.final]


def oracle_for(run, S0=None, X0=None, heads=None):
    inp = run.inp
    sl = (slice(None),) if heads is None else (slice(None), heads)
    hs = slice(None) if heads is None else heads
    return oracle.run(inp.q[sl], inp.k[sl], inp.v[sl], inp.z[sl], inp.g[sl], inp.beta[sl],
                      inp.conv_w[hs], inp.norm_w, run.cu, start_pos=run.starts,
                      S0=None if S0 is None else S0[:, hs], X0=None if X0 is None else X0[:, hs],
                      ckpt_interval=run.interval, state_round=run.cfg.state_dtype == kda.KDA_BF16)


def states_for(seed, shape, N, scale=0.3):
    S, X = wl.states(seed + 100, shape, N, state_std=scale, conv_std=1.0)
    return S, X


def check_against_oracle(run, r, heads=None):
    tol_o, tol_s = tols(run.shape.act)
    hs = slice(None) if heads is None else heads
    out = host(run.out)[:, hs]
    Sf, Xf = run.final_state()
    e_out = rel_l2(out, r.out)
    e_s = rel_l2(Sf[:, hs], r.S)
    e_c = per_chain_max(Sf[:, hs], r.S)
    e_r = per_row_max(out, r.out)
    say(f"  rel-L2 out {e_out:.3e} (tol {tol_o})  state {e_s:.3e} (tol {tol_s})  worst chain {e_c:.3e}"
        f"  worst row {e_r:.3e} (tol {tol_row(run.shape.act)})")
    assert np.isfinite(out).all() and np.isfinite(Sf[:, hs]).all()
    assert e_out <= tol_o and e_s <= tol_s and e_c <= TOL_STATE_PER_CHAIN
    assert e_r <= tol_row(run.shape.act)
    np.testing.assert_array_equal(Xf[:, hs], r.X)
    return e_out, e_s


def checkpoint_positions(start, length, interval):
    """Absolute positions of a sequence's checkpoints, in slot order."""
    return [p for p in range(start + 1, start + length + 1) if p % interval == 0 or p == start + length]


def resume_and_finish(straight, picks):
    """Resume every sequence n with picks[n] is not None from its picks[n]-th
    checkpoint of `straight` (copy-on-write into fresh slots) and prefill the
    rest of it as one packed batch.  Returns (resumed Run, resume positions,
    source checkpoint slots, packed token indices of the remainders)."""
    shape, inp, cfg = straight.shape, straight.inp, straight.cfg
    seqs = [n for n, j in enumerate(picks) if j is not None]
    res_pos, src_ck, rem, idx = [], [], [], []
    for n in seqs:
        s0, L = straight.starts[n], straight.lengths[n]
        p = checkpoint_positions(s0, L, straight.interval)[picks[n]]
        res_pos.append(p)
        src_ck.append(int(straight.base[n]) + picks[n])
        rem.append(s0 + L - p)
        off = int(straight.cu[n]) + (p - s0)
        idx.append(np.arange(off, off + rem[-1]))
    idx = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    sub = wl.Inputs(shape, inp.q[idx], inp.k[idx], inp.v[idx], inp.z[idx], inp.g[idx], inp.beta[idx],
                    inp.conv_w, inp.norm_w)
    resumed = Run(shape, sub, rem, starts=res_pos, interval=straight.interval, flags=straight.flags,
                  state_dtype=straight.cfg.state_dtype)
    resumed.init = np.arange(len(seqs), dtype=np.int32)
    kda.kda_resume(cfg, straight.ckS, straight.ckX, dev(np.asarray(src_ck, np.int32)),
                   resumed.Sd, resumed.Xd, dev(resumed.init))
    resumed.launch()
    return resumed, seqs, res_pos, src_ck, idx
