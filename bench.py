"""Benchmark of the KDA layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload varlen_ckpt|long_1m [--steps K] [--warmup W]

A step is one pass of the batched decode workload: 64 sequences advanced by
256 single-token decode steps (H=32, dk=dv=128, bf16 activations, fp32
state), i.e. 256 launches of the fused decode kernel over inputs that are
already resident in HBM.  `value` is decode tokens/s (64*256 tokens per
step).  The line also carries:
  roofline      the decode kernel's achieved algorithmic HBM bandwidth
                (bytes per launch / mean launch duration from HIP events)
                against the 8 TB/s peak, and the HBM traffic measured by
                rocprofv3 counters when those were taken on this kernel source
  slot_copies   the checkpoint and resume copies of the 64 live slots (all
                heads): microseconds per call and the HBM fraction by the
                bytes read and written
  cold_state    the same decode step cycled over 4 distinct state pools (640
                MiB, standing in for consecutive layers, so each launch reads
                its state from HBM, not from the 256 MB Infinity Cache), and a
                2 GiB read+write copy for the streaming rate this box attains
  next_rows     the same decode workload with a bf16-stored state, and as
                4-token launches keeping every token's state (fp32 and bf16
                pools): tokens/s and the HBM fraction by the bytes each moves
  prefill       the chunked prefill workload (4 x 8192 tokens, one call per
                pass): tokens/s and the algorithmic HBM and bf16-MFMA fractions
  varlen_ckpt   the varlen prefill with checkpoints (16 sequences, 262,990
                tokens), one workgroup per chain and scheduled
  long_1m       the 1M-token prefill split at its checkpoints, and with its 8
                chains paired
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the
                decode workload, and (prefill_workloads) on samples of the
                three prefill workloads
--no-paired leaves out every KDA_PREFILL_PAIRED (cooperative) launch; --no-next-rows the
next_rows legs.
With --workload the line instead reports one of the larger prefill
workloads (inputs resident in HBM, one call per pass):
  varlen_ckpt   16 sequences of log-uniform length in [1K, 64K] (262,990
                tokens in the seeded draw), H=32, checkpoints every 4096 tokens and at
                the ends, unsplit (the reported value) and split at the
                checkpoints; then a resume batch (each sequence restarted from a seeded
                interval checkpoint) timed on its own
  long_1m       one sequence of 1,048,576 tokens, H=8, checkpoints every 32K,
                unsplit and split at the checkpoints; then 512 decode steps of
                256 sequences fanned out from the end state
Only one GPU is supported: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA decode tok/s @B=64 (% HBM peak); prefill tok/s (% bf16 MFMA peak)"
HBM_PEAK = 8.0e12            # bytes/s
BF16_PEAK = 2.5e15           # dense FLOP/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_b64_traffic.json")
DECODE_SOURCES = ["linear_attention_recurrence_decode_amd/csrc/decode.hip",
                  "linear_attention_recurrence_decode_amd/csrc/kda_device.h"]
PROJECT_TRAFFIC = os.path.join(ROOT, "profiles", "project_4x8k_traffic.json")
PROJECT_SOURCES = ["linear_attention_recurrence_decode_amd/csrc/project.hip",
                   "linear_attention_recurrence_decode_amd/csrc/kda_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes_per_launch(B, H, dk, dv, act_bytes=2, state_bytes=4):
    """Algorithmic HBM bytes of one decode launch: per (sequence, head) the
    state read + written (fp32 or bf16), the conv state read + written,
    q/k/v/z in, g and beta in, out; plus the conv and norm weights and the
    slot ids."""
    C = 2 * dk + dv
    per = (2 * dk * dv * state_bytes + 2 * C * 3 * act_bytes + (2 * dk + 2 * dv) * act_bytes
           + dk * 4 + 4 + dv * act_bytes)
    return B * H * per + H * C * 4 * 4 + dv * 4 + B * 4


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path=PROFILE_TRAFFIC, sources=DECODE_SOURCES):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel code."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != source_sha(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


_DECODE_INPUTS = {}


def decode_inputs(w):
    """The decode workload's host inputs, drawn once per process."""
    import workloads as wl
    key = w["seed"]
    if key not in _DECODE_INPUTS:
        shape, B, nsteps, pool = w["shape"], w["B"], w["steps"], w["pool"]
        log(f"[bench] generating decode inputs B={B} steps={nsteps} H={shape.H} d={shape.dk}")
        inp = wl.token_inputs(w["seed"], shape, B * nsteps)
        S, X = wl.states(w["seed"], shape, pool, state_std=w["state_std"], conv_std=w["conv_std"])
        _DECODE_INPUTS[key] = (inp, S, X, wl.slot_permutation(w["seed"], pool, B))
    return _DECODE_INPUTS[key]


def bench_decode(args, extras=True):
    import torch
    import linear_attention_recurrence_decode_amd as kda
    import workloads as wl

    w = wl.WORKLOADS["decode_b64"]
    shape, B, nsteps, pool = w["shape"], w["B"], w["steps"], w["pool"]
    H, dk, dv = shape.H, shape.dk, shape.dv
    bf16_state = args.state_dtype == "bf16"
    cfg = kda.Config(H, dk, dv, kda.KDA_BF16, state_dtype=kda.KDA_BF16 if bf16_state else kda.KDA_F32)
    act = cfg.torch_act
    inp, S, X, slots = decode_inputs(w)
    r = lambda a: torch.from_numpy(a.reshape((nsteps, B) + a.shape[1:]))
    q, k, v, z = (r(a).to(act).cuda() for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = r(inp.g).cuda(), r(inp.beta).cuda()
    conv_w, norm_w = torch.from_numpy(inp.conv_w).cuda(), torch.from_numpy(inp.norm_w).cuda()
    Sd = torch.from_numpy(S).to(cfg.torch_state).cuda()
    Xd = torch.from_numpy(X).to(act).cuda()
    slot_d = torch.from_numpy(slots).cuda()
    out = torch.empty((nsteps, B, H, dv), dtype=act, device="cuda")
    stream = torch.cuda.current_stream()

    T = args.multi_token
    if T > 1:
        # speculative verify: nsteps/T launches of T tokens, per-token states kept for rollback
        assert nsteps % T == 0, "--multi-token must divide the step count"
        mq, mk, mv, mz = (a.reshape((nsteps // T, T) + a.shape[1:]) for a in (q, k, v, z))
        mg, mb = g.reshape((nsteps // T, T) + g.shape[1:]), beta.reshape((nsteps // T, T) + beta.shape[1:])
        mout = out.reshape((nsteps // T, T) + out.shape[1:])
        tstate = torch.empty((B, T, H, dk, dv), dtype=cfg.torch_state, device="cuda")
        tconv = torch.empty((B, T, H, 2 * dk + dv, 3), dtype=act, device="cuda")

    def one_pass():
        if T > 1:
            for s in range(nsteps // T):
                kda.kda_decode_multi(cfg, mq[s], mk[s], mv[s], mz[s], mg[s], mb[s], conv_w, norm_w, Sd, Xd,
                                     slot_d, mout[s], token_state=tstate, token_conv=tconv, stream=stream)
            return
        for s in range(nsteps):
            kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, Sd, Xd,
                                slot_d, out[s], stream=stream)

    log(f"[bench] warmup {args.warmup} passes")
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    # timed region: exactly K passes, bracketed by synchronisation
    log(f"[bench] timing {args.steps} passes")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        one_pass()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # mean duration of one decode launch: the timed region's HIP-event time on
    # the launch stream divided by the number of launches (the launches are
    # back to back, so this is the kernel's own duration plus dispatch gaps)
    launch_s = total_ms * 1e-3 / (args.steps * nsteps // T)

    tokens = B * nsteps * args.steps
    ms_per_step = total_ms / args.steps
    sb = 2 if bf16_state else 4
    nbytes = decode_bytes_per_launch(B, H, dk, dv, state_bytes=sb)
    if T > 1:
        # per launch: state read once, written to the pool and to T per-token slots,
        # conv state likewise, and T tokens of inputs and outputs
        one = decode_bytes_per_launch(B, H, dk, dv, state_bytes=sb)
        st_b, cv_b = B * H * dk * dv * sb, B * H * (2 * dk + dv) * 3 * 2
        tok_b = one - 2 * st_b - 2 * cv_b - (H * (2 * dk + dv) * 4 * 4 + dv * 4 + B * 4)
        nbytes = (2 + T) * st_b + (2 + T) * cv_b + T * tok_b + (H * (2 * dk + dv) * 4 * 4 + dv * 4 + B * 4)
    achieved = nbytes / launch_s
    traffic = None if (bf16_state or T > 1) else measured_traffic()
    variants = decode_variants(kda, cfg, q, k, v, z, g, beta, conv_w, norm_w, Sd, Xd, slot_d, out, nbytes, B, args) \
        if (args.variants and T == 1) else None
    res = {
        "value": tokens / (total_ms * 1e-3),
        "ms_per_step": ms_per_step,
        "wall_s": wall,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": traffic,
                     "kernel": ("decode_multi_kernel<128,128,bf16,%s,256>, T=%d" % ("bf16" if bf16_state else "f32", T)
                                if T > 1 else "decode_kernel<128,128,bf16,%s,256>" % ("bf16" if bf16_state else "f32")),
                     "bytes_per_launch": nbytes, "mean_launch_us": launch_s * 1e6},
    }
    if variants is not None:
        res["variants"] = variants
    if T == 1 and extras:
        res["slot_copies"] = slot_copies(kda, cfg, Sd, Xd, slot_d, B, H, dk, dv, sb, args)
        res["cold_state"] = cold_state_decode(kda, cfg, q, k, v, z, g, beta, conv_w, norm_w, S, X, slot_d,
                                              nbytes, B, args)
    return res


def bench_next_rows(args):
    """The decode workload in the forms the next rows of the design add: a
    bf16-stored state (one token per launch) and 4-token launches with
    per-token states kept for rollback, with an fp32 and with a bf16 pool.
    Same inputs, passes and warm-up as the headline leg."""
    import copy
    import torch
    out = {}
    for sd, T in (("bf16", 1), ("f32", 4), ("bf16", 4)):
        a = copy.copy(args)
        a.state_dtype, a.multi_token, a.variants = sd, T, False
        log(f"[bench] decode with a {sd} state pool, {T} token(s) per launch")
        r = bench_decode(a, extras=False)
        rf = r["roofline"]
        out[f"{sd}_state_T{T}"] = {"value": r["value"], "unit": "tok/s", "ms_per_step": r["ms_per_step"],
                                   "hbm_frac": rf["frac"], "kernel": rf["kernel"],
                                   "bytes_per_launch": rf["bytes_per_launch"], "mean_launch_us": rf["mean_launch_us"],
                                   "steps": a.steps}
        torch.cuda.empty_cache()
    return out


def cold_state_decode(kda, cfg, q, k, v, z, g, beta, conv_w, norm_w, S, X, slot_d, nbytes, B, args, layers=4):
    """The decode step with its state coming from HBM: `layers` distinct state
    pools (standing in for consecutive KDA layers of a model, 160 MiB each
    with fp32 states, 640 MiB in all, beyond the 256 MB Infinity Cache) are
    stepped in turn, launch after launch, so each launch finds its pool last
    touched three launches (480 MiB of other states) ago.  Beside it, a
    plain 1 GiB device-to-device copy (2 GiB read and written) gives the
    streaming rate this box attains."""
    import torch
    stream = torch.cuda.current_stream()
    pools = [(torch.from_numpy(S).to(cfg.torch_state).cuda(), torch.from_numpy(X).to(cfg.torch_act).cuda())
             for _ in range(layers)]
    out = torch.empty((B,) + tuple(q.shape[2:]), dtype=cfg.torch_act, device="cuda")
    nsteps = min(q.shape[0], 64)

    def one_pass():
        for s in range(nsteps):
            for Sl, Xl in pools:
                kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, Sl, Xl,
                                    slot_d, out, stream=stream)

    t = _time_calls(one_pass, max(1, args.steps // 4), 1, stream) / (nsteps * layers)
    src = torch.ones(1 << 28, device="cuda")
    dst = torch.empty_like(src)
    t_copy = _time_calls(lambda: dst.copy_(src), max(3, args.steps // 2), 2, stream)
    copy_bytes = 2 * src.numel() * 4
    del pools, src, dst
    return {"what": f"{layers} state pools of {S.nbytes >> 20} MiB stepped in turn ({nsteps} steps x {layers} "
                    f"launches); each launch's state last touched {layers - 1} launches earlier",
            "us_per_launch": t * 1e6, "tok_s_per_layer": B / t, "achieved_GBs": nbytes / t / 1e9,
            "hbm_frac": nbytes / t / HBM_PEAK,
            "streaming_copy": {"what": "torch copy_ of 1 GiB fp32 (2 GiB read and written)",
                               "achieved_GBs": copy_bytes / t_copy / 1e9, "hbm_frac": copy_bytes / t_copy / HBM_PEAK},
            "frac_of_streaming": (nbytes / t) / (copy_bytes / t_copy)}


def slot_copies(kda, cfg, Sd, Xd, slot_d, B, H, dk, dv, sb, args):
    """The checkpoint and resume copies at the decode workload's size: the
    state and conv state of its 64 live slots (all heads) copied into a
    64-slot checkpoint pool (kda_state_checkpoint) and back (kda_resume), each
    timed over `steps` calls after `warmup`.  Algorithmic bytes per call: every
    copied byte read once and written once."""
    import torch
    stream = torch.cuda.current_stream()
    ckS = torch.empty((B,) + tuple(Sd.shape[1:]), dtype=Sd.dtype, device="cuda")
    ckX = torch.empty((B,) + tuple(Xd.shape[1:]), dtype=Xd.dtype, device="cuda")
    ck_ids = torch.arange(B, dtype=torch.int32, device="cuda")
    nbytes = 2 * B * H * (dk * dv * sb + (2 * dk + dv) * 3 * Xd.element_size())
    calls = {"checkpoint": lambda: kda.kda_state_checkpoint(cfg, Sd, Xd, slot_d, ckS, ckX, ck_ids, stream=stream),
             "resume": lambda: kda.kda_resume(cfg, ckS, ckX, ck_ids, Sd, Xd, slot_d, stream=stream)}
    res = {"what": f"{B} slots x {H} heads per call, live pool <-> checkpoint pool", "bytes_per_call": nbytes}
    for name in ("checkpoint", "resume"):
        for _ in range(max(1, args.warmup)):
            calls[name]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            calls[name]()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / args.steps
        res[name] = {"us_per_call": t * 1e6, "achieved_GBs": nbytes / t / 1e9, "hbm_frac": nbytes / t / HBM_PEAK}
    return res


def decode_variants(kda, cfg, q, k, v, z, g, beta, conv_w, norm_w, Sd, Xd, slot_d, out, nbytes, B, args):
    """Two more timings of the same decode launches, outside the main timed
    region: (1) one pass of the launches captured once in a HIP graph and
    replayed; (2) each launch timed alone with the Infinity Cache flushed
    first by a 1 GiB read-modify-write sweep (not timed), so the state comes
    from HBM rather than from the 256 MB memory-side cache."""
    import torch
    nsteps = q.shape[0]
    res = {}

    # (1) HIP graph of one pass
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = torch.cuda.current_stream()
        for s in range(nsteps):
            kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, Sd, Xd,
                                slot_d, out[s], stream=st)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (args.steps * nsteps)
    res["hip_graph"] = {"us_per_launch": t * 1e6, "tok_s": B / t, "hbm_frac": nbytes / t / HBM_PEAK,
                        "what": f"{args.steps} replays of a graph holding one pass ({nsteps} launches)"}
    del graph

    # (2) Infinity Cache flushed before every launch
    n = min(nsteps, 64)
    scratch = torch.zeros(1 << 28, device="cuda")            # 1 GiB
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s in range(n):
        scratch.add_(1.0)
        ev[s][0].record(stream)
        kda.kda_decode_step(cfg, q[s], k[s], v[s], z[s], g[s], beta[s], conv_w, norm_w, Sd, Xd,
                            slot_d, out[s], stream=stream)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in ev) * 1e-3 / n
    res["mall_flushed"] = {"us_per_launch": t * 1e6, "tok_s": B / t, "hbm_frac": nbytes / t / HBM_PEAK,
                           "what": f"{n} launches, each after a 1 GiB read-modify-write sweep (untimed)"}
    del scratch
    return res


def prefill_flops_per_token_head(dk, dv, chunk=64):
    """Algorithmic FLOPs of the chunked form per token and head: the state
    products (K_g S, Q_g S, K^T U: 2*dk*dv each), the intra-chunk products
    (M and P: 2*C*dk/2 each on their triangles, W-like and U-like solves:
    C*(dk+dv)), and the triangular solve (C^2/3); masked triangles are not
    counted."""
    return 6 * dk * dv + chunk * (3 * dk + 2 * dv) + chunk * chunk // 3


def prefill_bytes_per_token_head(dk, dv, act_bytes=2):
    """Unavoidable HBM bytes per token and head: q, k, v, z in (activation
    dtype), g (fp32, per key channel) and beta (fp32) in, out (activation
    dtype)."""
    return (2 * dk + 2 * dv) * act_bytes + dk * 4 + 4 + dv * act_bytes


def bench_prefill(steps, warmup, paired_leg=True):
    import torch
    import linear_attention_recurrence_decode_amd as kda
    import workloads as wl

    w = wl.WORKLOADS["prefill_4x8k"]
    shape, lengths = w["shape"], w["lengths"]
    H, dk, dv, C = shape.H, shape.dk, shape.dv, shape.C
    N, T = len(lengths), sum(lengths)
    cfg = kda.Config(H, dk, dv, kda.KDA_BF16)
    act = cfg.torch_act
    log(f"[bench] generating prefill inputs {N} x {lengths[0]} tokens, H={H}")
    inp = wl.token_inputs(w["seed"], shape, T)
    q, k, v, z = (torch.from_numpy(a).to(act).cuda() for a in (inp.q, inp.k, inp.v, inp.z))
    g, beta = torch.from_numpy(inp.g).cuda(), torch.from_numpy(inp.beta).cuda()
    conv_w, norm_w = torch.from_numpy(inp.conv_w).cuda(), torch.from_numpy(inp.norm_w).cuda()
    cu = torch.from_numpy(wl.cu_seqlens(lengths).astype(np.int32)).cuda()
    Sd = torch.zeros((N, H, dk, dv), device="cuda")
    Xd = torch.zeros((N, H, C, 3), dtype=act, device="cuda")
    init = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    final = torch.arange(N, dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, dv), dtype=act, device="cuda")
    paired = kda.KDA_PREFILL_PAIRED
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, N, T, 0, paired), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(flags):
        def one():
            kda.kda_prefill_varlen(cfg, cu, q, k, v, z, g, beta, conv_w, norm_w, Sd, Xd, init, final, out, ws,
                                   flags=flags, stream=stream)
        return _time_calls(one, steps, warmup, stream)

    # the paired launch (two workgroups per chain) is the headline: this
    # workload has 128 chains for 256 compute units
    t1 = timed(0)
    t = timed(paired) if paired_leg else t1
    th = T * H
    flops = prefill_flops_per_token_head(dk, dv) * th
    nbytes = prefill_bytes_per_token_head(dk, dv) * th
    return {"workload": f"prefill_4x8k: {N} x {lengths[0]} tokens, H={H}, dk=dv={dk}, bf16, chunk 64",
            "mode": "paired (KDA_PREFILL_PAIRED)" if paired_leg else "one workgroup per chain",
            "value": T / t, "unit": "tok/s", "ms_per_call": t * 1e3,
            "mfma_frac": flops / t / BF16_PEAK, "hbm_frac": nbytes / t / HBM_PEAK,
            "alg_flops": flops, "alg_bytes": nbytes,
            "attainable_frac": max(flops / BF16_PEAK, nbytes / HBM_PEAK) / t,
            "one_workgroup": {"value": T / t1, "ms_per_call": t1 * 1e3, "mfma_frac": flops / t1 / BF16_PEAK,
                              "hbm_frac": nbytes / t1 / HBM_PEAK}}


def _time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


class PrefillSetup:
    """Device buffers of one packed prefill batch with checkpoints."""

    def __init__(self, kda, wl, shape, inp, lengths, starts, interval, flags_list):
        import torch
        H, dk, dv, C = shape.H, shape.dk, shape.dv, shape.C
        N, T = len(lengths), int(sum(lengths))
        self.cfg = cfg = kda.Config(H, dk, dv, kda.KDA_BF16)
        act = cfg.torch_act
        self.kda, self.N, self.T, self.interval = kda, N, T, interval
        self.q, self.k, self.v, self.z = (torch.from_numpy(a).to(act).cuda() for a in (inp.q, inp.k, inp.v, inp.z))
        self.g, self.beta = torch.from_numpy(inp.g).cuda(), torch.from_numpy(inp.beta).cuda()
        self.conv_w, self.norm_w = torch.from_numpy(inp.conv_w).cuda(), torch.from_numpy(inp.norm_w).cuda()
        self.cu = torch.from_numpy(wl.cu_seqlens(lengths).astype(np.int32)).cuda()
        self.sp = torch.tensor(starts, dtype=torch.int64).cuda()
        self.S = torch.zeros((2 * N, H, dk, dv), device="cuda")
        self.X = torch.zeros((2 * N, H, C, 3), dtype=act, device="cuda")
        self.init = torch.full((N,), -1, dtype=torch.int32).cuda()
        self.final = torch.arange(N, 2 * N, dtype=torch.int32).cuda()
        counts = [kda.kda_num_checkpoints(s0, L, interval) for s0, L in zip(starts, lengths)]
        base = np.zeros(N, np.int32)
        base[1:] = np.cumsum(counts)[:-1]
        self.base_h, self.nck = base, int(sum(counts))
        self.base = torch.from_numpy(base).cuda()
        self.ckS = torch.zeros((max(self.nck, 1), H, dk, dv), device="cuda")
        self.ckX = torch.zeros((max(self.nck, 1), H, C, 3), dtype=act, device="cuda")
        self.out = torch.empty((T, H, dv), dtype=act, device="cuda")
        nbytes = max(kda.kda_prefill_workspace_bytes(cfg, N, T, interval, f) for f in flags_list)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def call(self, flags, stream):
        self.kda.kda_prefill_varlen(self.cfg, self.cu, self.q, self.k, self.v, self.z, self.g, self.beta,
                                    self.conv_w, self.norm_w, self.S, self.X, self.init, self.final, self.out,
                                    self.ws, start_pos=self.sp, ckpt_interval=self.interval, ckpt_state=self.ckS,
                                    ckpt_conv=self.ckX, ckpt_base=self.base, flags=flags, stream=stream)


def prefill_rates(T, H, dk, dv, t):
    th = T * H
    flops = prefill_flops_per_token_head(dk, dv) * th
    nbytes = prefill_bytes_per_token_head(dk, dv) * th
    return {"value": T / t, "unit": "tok/s", "ms_per_call": t * 1e3, "mfma_frac": flops / t / BF16_PEAK,
            "hbm_frac": nbytes / t / HBM_PEAK, "attainable_frac": max(flops / BF16_PEAK, nbytes / HBM_PEAK) / t}


def bench_varlen(steps, warmup, paired_leg=True, full=True):
    """Varlen prefill with checkpoints (one workgroup per chain, the
    scheduled launch and, with `full`, the split launch), then with `full` the
    resume batch."""
    import torch
    import linear_attention_recurrence_decode_amd as kda
    import workloads as wl

    w = wl.WORKLOADS["varlen_ckpt"]
    shape, N, interval = w["shape"], w["n"], w["interval"]
    lengths = [int(x) for x in wl.loguniform_lengths(w["seed"], N, w["lo"], w["hi"])]
    log(f"[bench] varlen: {N} sequences, {sum(lengths)} tokens")
    inp = wl.token_inputs(w["seed"], shape, sum(lengths))
    stream = torch.cuda.current_stream()
    split, paired = kda.KDA_PREFILL_SPLIT, kda.KDA_PREFILL_PAIRED
    st = PrefillSetup(kda, wl, shape, inp, lengths, [0] * N, interval, [0, split, paired])
    del inp
    t = _time_calls(lambda: st.call(0, stream), steps, warmup, stream)
    res = {"workload": f"varlen_ckpt: {N} sequences, {sum(lengths)} tokens (lengths log-uniform in [1K, 64K]), "
                       f"H={shape.H}, dk=dv={shape.dk}, bf16, checkpoints every {interval} and at ends "
                       f"({st.nck} checkpoints)",
           "straight": prefill_rates(st.T, shape.H, shape.dk, shape.dv, t)}
    if full:
        t_s = _time_calls(lambda: st.call(split, stream), steps, warmup, stream)
        res["straight_split"] = prefill_rates(st.T, shape.H, shape.dk, shape.dv, t_s)
    if paired_leg:
        t_p = _time_calls(lambda: st.call(paired, stream), steps, warmup, stream)
        res["straight_paired"] = prefill_rates(st.T, shape.H, shape.dk, shape.dv, t_p)
    res["value"] = max(r["value"] for key, r in res.items() if key.startswith("straight") and key != "straight_split")
    if not full:
        del st
        return res
    inp = wl.token_inputs(w["seed"], shape, sum(lengths))
    # resume batch: each sequence with an interval checkpoint restarts from a seeded one
    rng = np.random.default_rng([w["seed"], wl.TID["resume"], 0])
    rem, pos, src, idx = [], [], [], []
    cu = wl.cu_seqlens(lengths)
    for n, L in enumerate(lengths):
        n_int = kda.kda_num_checkpoints(0, L, interval) - 1
        if n_int <= 0:
            continue
        j = int(rng.integers(0, n_int))
        p = (j + 1) * interval
        rem.append(L - p)
        pos.append(p)
        src.append(int(st.base_h[n]) + j)
        idx.append(np.arange(cu[n] + p, cu[n] + L))
    idx = np.concatenate(idx)
    sub = wl.Inputs(shape, inp.q[idx], inp.k[idx], inp.v[idx], inp.z[idx], inp.g[idx], inp.beta[idx],
                    inp.conv_w, inp.norm_w)
    rs = PrefillSetup(kda, wl, shape, sub, rem, pos, interval, [0, paired])
    n_r = len(rem)
    rs.init = torch.arange(n_r, dtype=torch.int32).cuda()
    kda.kda_resume(st.cfg, st.ckS, st.ckX, torch.tensor(src, dtype=torch.int32).cuda(), rs.S, rs.X, rs.init,
                   stream=stream)
    # every pass restarts from the resumed slots (the final slots are distinct)
    t_r = _time_calls(lambda: rs.call(0, stream), steps, warmup, stream)
    res["resume"] = dict(prefill_rates(rs.T, shape.H, shape.dk, shape.dv, t_r),
                         sequences=n_r, tokens=int(rs.T))
    if paired_leg:
        t_rp = _time_calls(lambda: rs.call(paired, stream), steps, warmup, stream)
        res["resume_paired"] = prefill_rates(rs.T, shape.H, shape.dk, shape.dv, t_rp)
    # the headline (value, set above) is the faster of the straight
    # one-workgroup and scheduled calls
    return res


def bench_long(steps, warmup, paired_leg=True, full=True):
    """The 1M-token sequence split at its checkpoints (the value) and with
    its 8 chains paired; with `full` also unsplit in one workgroup per chain,
    and the 256-sequence decode fanned out from its end state."""
    import torch
    import linear_attention_recurrence_decode_amd as kda
    import workloads as wl

    w = wl.WORKLOADS["long_1m"]
    shape, L, interval = w["shape"], w["lengths"][0], w["interval"]
    log(f"[bench] long context: {L} tokens, H={shape.H}")
    inp = wl.token_inputs(w["seed"], shape, L)
    stream = torch.cuda.current_stream()
    split, paired = kda.KDA_PREFILL_SPLIT, kda.KDA_PREFILL_PAIRED
    st = PrefillSetup(kda, wl, shape, inp, [L], [0], interval, [0, split, paired])
    conv_w, norm_w = st.conv_w, st.norm_w
    del inp
    res = {"workload": f"long_1m: 1 sequence of {L} tokens, H={shape.H}, dk=dv={shape.dk}, bf16, checkpoints "
                       f"every {interval}"}
    if full:
        t_u = _time_calls(lambda: st.call(0, stream), max(1, steps // 4), min(warmup, 1), stream)
        res["unsplit"] = prefill_rates(L, shape.H, shape.dk, shape.dv, t_u)
    if paired_leg:
        # the 8 chains paired (producer and consumer workgroups), not split
        t_p = _time_calls(lambda: st.call(paired, stream), max(1, steps // 4), min(warmup, 1), stream)
        res["unsplit_paired"] = prefill_rates(L, shape.H, shape.dk, shape.dv, t_p)
    t_s = _time_calls(lambda: st.call(split, stream), steps, warmup, stream)
    res["split"] = prefill_rates(L, shape.H, shape.dk, shape.dv, t_s)
    res["value"] = res["split"]["value"]
    if not full:
        del st
        return res
    # decode fan-out: 256 slots from the end state, 512 steps
    B, nsteps = w["decode_B"], w["decode_steps"]
    cfg = st.cfg
    Sp = torch.zeros((B, shape.H, shape.dk, shape.dv), device="cuda")
    Xp = torch.zeros((B, shape.H, shape.C, 3), dtype=cfg.torch_act, device="cuda")
    slot = torch.arange(B, dtype=torch.int32).cuda()
    kda.kda_resume(cfg, st.ckS, st.ckX, torch.full((B,), st.nck - 1, dtype=torch.int32).cuda(), Sp, Xp, slot,
                   stream=stream)
    dinp = wl.token_inputs(w["seed"] + 100, shape, B * nsteps)
    r = lambda a: torch.from_numpy(a.reshape((nsteps, B) + a.shape[1:]))
    q, k, v, z = (r(a).to(cfg.torch_act).cuda() for a in (dinp.q, dinp.k, dinp.v, dinp.z))
    g, beta = r(dinp.g).cuda(), r(dinp.beta).cuda()
    dout = torch.empty((nsteps, B, shape.H, shape.dv), dtype=cfg.torch_act, device="cuda")

    def decode_pass():
        for s2 in range(nsteps):
            kda.kda_decode_step(cfg, q[s2], k[s2], v[s2], z[s2], g[s2], beta[s2], conv_w, norm_w, Sp, Xp,
                                slot, dout[s2], stream=stream)

    t_d = _time_calls(decode_pass, max(1, steps // 4), 1, stream)
    nbytes = decode_bytes_per_launch(B, shape.H, shape.dk, shape.dv)
    res["decode"] = {"value": B * nsteps / t_d, "unit": "tok/s", "ms_per_pass": t_d * 1e3,
                     "hbm_frac": nbytes * nsteps / t_d / HBM_PEAK, "B": B, "steps": nsteps}
    return res


def bench_project(steps, warmup, paired_leg=True):
    """The input projections of the 4 x 8192 prefill: one bf16 GEMM per call
    (the line's value); the output projection of the same tokens is timed
    after it and reported beside it."""
    import torch
    import linear_attention_recurrence_decode_amd as kda
    import workloads as wl

    w = wl.WORKLOADS["project_4x8k"]
    shape, T, Dm = w["shape"], w["T"], w["Dm"]
    H, dk, dv = shape.H, shape.dk, shape.dv
    log(f"[bench] projection inputs T={T} Dm={Dm}")
    x, wt = wl.projection_inputs(w["seed"], shape, T, Dm)
    cfg = kda.Config(H, dk, dv, kda.KDA_BF16)
    xd, wd = torch.from_numpy(x).to(torch.bfloat16).cuda(), torch.from_numpy(wt).to(torch.bfloat16).cuda()
    del x, wt
    q, k = (torch.empty((T, H, dk), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    v, z = (torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    g, beta = torch.empty((T, H, dk), device="cuda"), torch.empty((T, H), device="cuda")
    stream = torch.cuda.current_stream()
    t = _time_calls(lambda: kda.kda_project_inputs(cfg, xd, wd, q, k, v, z, g, beta, stream=stream), steps, warmup,
                    stream)
    N = kda.projection_rows(cfg)
    flops = 2.0 * T * Dm * N
    nbytes = (T * Dm + N * Dm) * 2 + T * H * (2 * dk + 2 * dv) * 2 + T * H * (dk + 1) * 4
    # context only: the library GEMM (torch.matmul) on the same bf16 product, without the routing and gate maps
    wcol = wd.t().contiguous()
    t_lib = _time_calls(lambda: torch.matmul(xd, wcol), steps, warmup, stream)
    del wcol
    # the conv front end (the causal conv + SiLU on q, k, v in the epilogue), and the
    # prefill of these tokens (4 sequences of 8192) after each front end
    conv_res = conv_front_end(kda, wl, cfg, shape, xd, wd, q, k, v, z, g, beta, T, flops, steps, warmup, stream,
                              paired_leg)
    del xd, wd, q, k, v, z, g, beta
    # the output projection of the same tokens: o [T][H][dv] -> y [T][Dm]
    o, wo = wl.output_projection_inputs(w["seed"], shape, T, Dm)
    od, wod = torch.from_numpy(o).to(torch.bfloat16).cuda(), torch.from_numpy(wo).to(torch.bfloat16).cuda()
    del o, wo
    y = torch.empty((T, Dm), dtype=torch.bfloat16, device="cuda")
    t_out = _time_calls(lambda: kda.kda_project_output(cfg, od, wod, y, stream=stream), steps, warmup, stream)
    flops_out = 2.0 * T * (H * dv) * Dm
    return {"workload": f"project_4x8k: x [{T}][{Dm}] bf16 times W [{N}][{Dm}] bf16 (q, k, v, z, g, beta of "
                        f"H={H}, dk=dv={dk})",
            "value": flops / t / 1e12, "unit": "TFLOP/s", "ms_per_call": t * 1e3,
            "roofline": {"bound": "mfma", "achieved": flops / t / 1e12, "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": flops / t / BF16_PEAK, "traffic": measured_traffic(PROJECT_TRAFFIC, PROJECT_SOURCES),
                         "alg_flops": flops, "alg_bytes": nbytes},
            "tokens_per_s": T / t,
            "library_matmul": {"TFLOP/s": flops / t_lib / 1e12, "ms_per_call": t_lib * 1e3,
                               "what": "torch.matmul of the same bf16 x and W^T (plain product, no epilogue)"},
            "output_projection": {"TFLOP/s": flops_out / t_out / 1e12, "ms_per_call": t_out * 1e3,
                                  "frac": flops_out / t_out / BF16_PEAK,
                                  "what": f"kda_project_output: o [{T}][{H * dv}] bf16 times W_o [{Dm}][{H * dv}] bf16"},
            "conv_front_end": conv_res}


def conv_front_end(kda, wl, cfg, shape, xd, wd, q, k, v, z, g, beta, T, flops, steps, warmup, stream, paired_leg=True):
    """kda_project_inputs_conv on the same x and W (the GEMM plus the causal
    conv and SiLU of q, k, v in its epilogue, post-conv and raw tensors
    written), then the 4 x 8192 prefill on each front end's outputs: the
    unfused pair (kda_project_inputs + kda_prefill_varlen) against the fused
    one (kda_project_inputs_conv + kda_prefill_varlen with
    KDA_PREFILL_CONV_DONE), one workgroup per chain and paired."""
    import torch
    H, dk, dv, C = shape.H, shape.dk, shape.dv, shape.C
    N = 4
    lengths = [T // N] * N
    cu = torch.from_numpy(wl.cu_seqlens(lengths).astype(np.int32)).cuda()
    pool = torch.zeros((1, H, C, 3), dtype=torch.bfloat16, device="cuda")
    init = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    q2, k2 = (torch.empty((2, T, H, dk), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    v2 = torch.empty((2, T, H, dv), dtype=torch.bfloat16, device="cuda")
    cw = torch.from_numpy(wl.token_inputs(5, shape, 1).conv_w).cuda()
    nw = torch.ones((dv,), device="cuda")
    t_fe = _time_calls(lambda: kda.kda_project_inputs_conv(cfg, cu, xd, wd, cw, pool, init, q2, k2, v2, z, g, beta,
                                                           stream=stream), steps, warmup, stream)
    S = torch.zeros((N, H, dk, dv), device="cuda")
    X = torch.zeros((N, H, C, 3), dtype=torch.bfloat16, device="cuda")
    fin = torch.arange(N, dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, N, T, 0, kda.KDA_PREFILL_PAIRED), dtype=torch.uint8,
                     device="cuda")
    res = {"what": "kda_project_inputs_conv: the input projections with the causal conv + SiLU of q, k, v in the "
                   "epilogue (post-conv and raw tensors written); prefill_ms: the 4 x 8192 prefill after it "
                   "(KDA_PREFILL_CONV_DONE) and after kda_project_inputs (unfused)",
           "ms_per_call": t_fe * 1e3, "TFLOP/s": flops / t_fe / 1e12, "prefill_ms": {}}
    for label, (qq, kk, vv), cd in (("unfused", (q, k, v), 0), ("conv_done", (q2, k2, v2), kda.KDA_PREFILL_CONV_DONE)):
        for mode, fl in (("one_workgroup", 0), ("paired", kda.KDA_PREFILL_PAIRED))[:2 if paired_leg else 1]:
            t = _time_calls(lambda: kda.kda_prefill_varlen(cfg, cu, qq, kk, vv, z, g, beta, cw, nw, S, X, init, fin,
                                                           out, ws, flags=fl | cd, stream=stream),
                            max(3, steps // 2), max(1, warmup), stream)
            res["prefill_ms"][f"{label}_{mode}"] = t * 1e3
    return res


def cpu_baseline(sample_steps: int):
    """The fp64 oracle on the first `sample_steps` steps of the decode
    workload (all 64 sequences, all 32 heads), timed on this host."""
    import oracle
    import workloads as wl

    w = wl.WORKLOADS["decode_b64"]
    shape, B, pool = w["shape"], w["B"], w["pool"]
    inp = wl.token_inputs(w["seed"], shape, B * sample_steps)
    S, X = wl.states(w["seed"], shape, pool, state_std=w["state_std"], conv_std=w["conv_std"])
    slots = wl.slot_permutation(w["seed"], pool, B)
    r = lambda a: a.reshape((sample_steps, B) + a.shape[1:])
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.decode_steps(r(inp.q), r(inp.k), r(inp.v), r(inp.z), r(inp.g), r(inp.beta),
                        inp.conv_w, inp.norm_w, S[slots], X[slots])
    dt = time.perf_counter() - t0
    # the same oracle on one thread, over the first 48 steps
    n1 = min(48, sample_steps)
    t1 = time.perf_counter()
    oracle.decode_steps(r(inp.q)[:n1], r(inp.k)[:n1], r(inp.v)[:n1], r(inp.z)[:n1], r(inp.g)[:n1],
                        r(inp.beta)[:n1], inp.conv_w, inp.norm_w, S[slots], X[slots], threads=1)
    dt1 = time.perf_counter() - t1
    # the oracle keeps a thread count it is given: restore all of them
    oracle.decode_steps(r(inp.q)[:1], r(inp.k)[:1], r(inp.v)[:1], r(inp.z)[:1], r(inp.g)[:1],
                        r(inp.beta)[:1], inp.conv_w, inp.norm_w, S[slots], X[slots], threads=threads)
    return {"value": B * sample_steps / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"decode workload, {sample_steps} of 256 steps, 64 sequences x 32 heads, "
                      f"fp64 token-by-token, {dt:.1f} s",
            "single_thread": {"value": B * n1 / dt1, "unit": "tok/s",
                              "sample": f"first {n1} steps of the same workload on one thread, {dt1:.1f} s"},
            "cpu": cpu_model()}


def cpu_baseline_prefill(threads: int):
    """The fp64 oracle on bounded samples of the three prefill workloads
    (the first tokens of every sequence, all heads, checkpoints as in the
    workload), timed on this host with `threads` threads (given explicitly:
    a thread count passed to the oracle stays set for later calls).  The
    oracle runs one (sequence, head) chain per thread, so the 1M-token sample
    uses 8 threads (its 8 heads)."""
    import oracle
    import workloads as wl

    res = {}

    def sample(name, seed, shape, lengths, take, interval, what):
        cu = wl.cu_seqlens(lengths)
        sub = [min(take, int(L)) for L in lengths]
        rows = np.concatenate([np.arange(cu[n], cu[n] + m) for n, m in enumerate(sub)])
        inp = wl.token_rows(seed, shape, rows)
        t0 = time.perf_counter()
        oracle.run(inp.q, inp.k, inp.v, inp.z, inp.g, inp.beta, inp.conv_w, inp.norm_w, wl.cu_seqlens(sub),
                   ckpt_interval=interval, threads=threads)
        dt = time.perf_counter() - t0
        tokens = int(sum(sub))
        res[name] = {"value": tokens / dt, "unit": "tok/s", "cores": min(threads, len(sub) * shape.H),
                     "kind": "oracle", "seconds": dt, "token_heads": tokens * shape.H,
                     "sample": f"{what}: first {take} tokens of each of {len(sub)} sequences ({tokens} tokens), "
                               f"all {shape.H} heads, fp64 token-by-token, {dt:.1f} s"}

    w = wl.WORKLOADS["prefill_4x8k"]
    sample("prefill_4x8k", w["seed"], w["shape"], w["lengths"], 2048, 0, "prefill_4x8k")
    w = wl.WORKLOADS["varlen_ckpt"]
    lengths = [int(x) for x in wl.loguniform_lengths(w["seed"], w["n"], w["lo"], w["hi"])]
    sample("varlen_ckpt", w["seed"], w["shape"], lengths, 1024, w["interval"], "varlen_ckpt")
    w = wl.WORKLOADS["long_1m"]
    sample("long_1m", w["seed"], w["shape"], w["lengths"], 16384, w["interval"], "long_1m")
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip() + f", {os.cpu_count()} logical CPUs visible"
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="leave out the bf16-state and multi-token decode legs of the default line")
    ap.add_argument("--no-paired", action="store_true",
                    help="leave out every KDA_PREFILL_PAIRED launch (a cooperative launch), e.g. under a profiler")
    ap.add_argument("--multi-token", type=int, default=1,
                    help="decode T tokens per launch with per-token states kept (speculative verify); 1 = one step")
    ap.add_argument("--state-dtype", choices=["f32", "bf16"], default="f32",
                    help="stored state dtype of the decode workload (the workload is defined with f32)")
    ap.add_argument("--workload", choices=["decode_b64", "varlen_ckpt", "long_1m", "project_4x8k"],
                    default="decode_b64",
                    help="decode_b64 (default): the headline line; the others report a larger prefill workload")
    ap.add_argument("--variants", action="store_true",
                    help="decode workload: also time the launches replayed from a HIP graph and with the "
                         "Infinity Cache flushed before each launch (outside the main timed region)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a kernel of "
                         "known traffic, used to scale memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the KDA layer shards by heads or by sequences with no exchange between GPUs, "
              "so one GPU's throughput is the figure that matters here)", file=sys.stderr)
        sys.exit(2)

    if args.calibration_copy_mib > 0:
        import torch
        n = args.calibration_copy_mib << 18          # float32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload != "decode_b64":
        if args.workload == "project_4x8k":
            res = bench_project(args.steps, args.warmup, paired_leg=not args.no_paired)
        else:
            res = bench_varlen(args.steps, args.warmup, paired_leg=not args.no_paired) \
                if args.workload == "varlen_ckpt" else bench_long(args.steps, args.warmup, paired_leg=not args.no_paired)
        metric = ("KDA input projections TFLOP/s (" if args.workload == "project_4x8k" else "KDA prefill tok/s (")
        line = {"metric": metric + args.workload + ")", "value": res["value"], "unit": res.get("unit", "tok/s"),
                "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16" if args.workload == "project_4x8k" else "f32", "data": "synthetic",
                "config": {"workload": res.pop("workload"), "parallelism": "single GPU"}}
        line.update({k: v for k, v in res.items() if k != "value"})
        print(json.dumps(line), flush=True)
        return
    res = bench_decode(args)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_b64: 64 seqs x 256 single-token steps, H=32, dk=dv=128, "
                               "bf16 activations, %s state%s" % ("bf16-stored" if args.state_dtype == "bf16" else "fp32",
                                                                   ", %d tokens per launch with per-token states" % args.multi_token
                                                                   if args.multi_token > 1 else ""),
                   "global_batch": 64, "seq_len": 256, "parallelism": "single GPU"},
        "roofline": res["roofline"],
    }
    if "variants" in res:
        line["variants"] = res["variants"]
    if "slot_copies" in res:
        line["slot_copies"] = res["slot_copies"]
    if "cold_state" in res:
        line["cold_state"] = res["cold_state"]
    if not args.no_next_rows and args.state_dtype == "f32" and args.multi_token == 1:
        line["next_rows"] = bench_next_rows(args)
    if not args.no_prefill:
        import torch
        line["prefill"] = bench_prefill(max(3, args.steps // 2), max(1, args.warmup), paired_leg=not args.no_paired)
        torch.cuda.empty_cache()
        line["varlen_ckpt"] = bench_varlen(max(3, args.steps // 2), max(1, args.warmup),
                                           paired_leg=not args.no_paired, full=False)
        torch.cuda.empty_cache()
        line["long_1m"] = bench_long(max(3, args.steps // 4), 1, paired_leg=not args.no_paired, full=False)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_sample_steps} decode steps")
        line["cpu_baseline"] = cpu_baseline(args.cpu_sample_steps)
        if not args.no_prefill:
            log("[bench] cpu baseline: oracle on samples of the prefill workloads")
            line["cpu_baseline"]["prefill_workloads"] = cpu_baseline_prefill(line["cpu_baseline"]["cores"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
