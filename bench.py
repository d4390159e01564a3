"""Benchmark of the Gated DeltaNet mixer on one MI355X.

Headline: chunked prefill throughput (tokens/s) on the Qwen3-Next layer shape at long
context, B=1, T=32768, 16 QK heads shared by 32 V heads, head dim 128, bf16 q/k/v/o, fp32
initial state S0 ~ N(0, 0.02) in and fp32 final state out. A step is one gdn_chunk_prefill
call over the whole batch: its launches (the chunk-parallel prep and the sequential state
pass) run every step of the chunked method. Alongside: the same prefill at T=4096 with S0 =
0; the packed variable-length batch (64 sequences, lengths uniform in [128, 8192]) through
the front end and the prefill; the decode step on a 256-sequence fp32 state pool (HBM-bound,
no matrix cores), with the decode-time front end (two calls and one launch); the
multi-token verify step; the per-channel decay form (decode and token-sequential prefill);
and the output epilogue. The fp64 oracle is timed on the host cores on the headline
workload as a CPU baseline.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps K2]
                  [--workload prefill,decode,frontend,epilogue] [--no-cpu-baseline]
      prints one JSON line (prefill_t32768 or prefill_t4096 alone for one prefill workload)
  python bench.py --workload copy
      a plain 1 GiB device copy, the calibration run for hardware byte counters
  python bench.py --pmc-summary DIR
      per-kernel averages of the counters in rocprofv3 --pmc output under DIR
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s/GPU (H_v=32,d=128) + decode state GB/s vs HBM peak"
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published (packed issue), TFLOP/s
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s

D = 128
C = 64
H_QK, H_V = 16, 32
CSRC = os.path.join(ROOT, "linear_attention_recurrence_amd", "csrc")

# Hardware counters of one call, from rocprofv3 --pmc runs of `python bench.py --workload
# prefill_t32768,frontend,decode,copy` and `--workload prefill_t4096` (with `--steps 5
# --warmup 1 --decode-steps 20 --no-cpu-baseline`; the commands and the per-kernel figures
# are kept in profiles/hbm_mfma_counters.md):
#  * "bytes": HBM bytes per call, FETCH_SIZE plus WRITE_SIZE (KiB per dispatch, summed over
#    the call's kernels) in two passes, each scaled by what the same counter reads for a
#    plain 1 GiB device copy;
#  * "mfma_busy": the fraction of the matrix cores' cycles spent busy over the call,
#    sum(SQ_VALU_MFMA_BUSY_CYCLES) / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) per kernel, weighted by
#    each kernel's share of the call's time.
# `sources` fingerprints the kernel sources the figures were taken on: once they change,
# the figures no longer describe the kernels and are reported as null.
COUNTERS = {
    "prefill_t32768": {"bytes": 2019556243, "mfma_busy": 0.1429, "sources": "aa289cfee5e4dc67"},
    "prefill_t4096": {"bytes": 250348481, "mfma_busy": 0.1426, "sources": "aa289cfee5e4dc67"},
    "prefill_packed64": {"bytes": 12458583064, "mfma_busy": 0.2553, "sources": "aa289cfee5e4dc67"},
    "prefill_conv_packed64": {"bytes": 22514586491, "sources": "ee640ee8469c140d"},
    "decode": {"bytes": 1083356788, "sources": "1cbcbd1979d4176c"},
}


def _sources_sha(names):
    """Fingerprint of kernel sources: their code with comments and blank space removed, so
    that edits to comments alone leave recorded figures in force."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ("chunk_prefill.hip", "gdn_device.h")
PREFILL_CONV_SOURCES = ("chunk_prefill.hip", "conv_prep.hip", "conv_device.h", "gdn_device.h")
DECODE_SOURCES = ("recurrent.hip", "gdn_device.h")


def counter(name, field, sources):
    """A counter figure recorded for `name`, or None when not measured on these kernel
    sources."""
    rec = COUNTERS.get(name)
    if rec is None or rec.get(field) is None or rec["sources"] != _sources_sha(sources):
        return None
    return rec[field]


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must compute and move, not what a kernel happens to do)
# ---------------------------------------------------------------------------------------

def prefill_flops(tokens: int, h_v: int = H_V) -> float:
    """Matrix-product FLOPs of the chunked form per token and V head, as derived from the
    update: five C x C x d products (K K^T, Q K^T, T diag(beta gam) K, T diag(beta) V, P U)
    = 10 C d, and three C x d x d products (W S^T, Q S^T, U^T K) = 6 d^2: 180,224 at C = 64,
    d = 128. (The kernels apply T to the residual V - diag(gam) K S^T instead, one C x C x d
    product fewer, 8 C d + 6 d^2; the figure here is the method's, not the kernels'.)"""
    return float(tokens) * h_v * (10 * C * D + 6 * D * D)


def prefill_bytes(tokens: int, num_seqs: int, with_s0: bool, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes: q, k (bf16, per QK head), v and o (bf16, per V head), g and beta (fp32),
    the final states (fp32) and the initial states when given."""
    per_tok = 2 * h_qk * D * 2 + 2 * h_v * D * 2 + 2 * h_v * 4
    states = num_seqs * h_v * D * D * 4 * (2 if with_s0 else 1)
    return float(tokens) * per_tok + states


def decode_bytes(num_seqs: int, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes of one decode step: every state read and written (fp32), q, k, v, o
    (bf16), g and beta (fp32)."""
    state = num_seqs * h_v * D * D * 4 * 2
    io = num_seqs * (2 * h_qk * D * 2 + 2 * h_v * D * 2 + 2 * h_v * 4)
    return float(state + io)


def conv_prep_bytes(tokens: int, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes of the front end: the mixed input read and q, k, v written (bf16)."""
    ch = 2 * h_qk * D + h_v * D
    return float(tokens) * ch * 2 * 2


# ---------------------------------------------------------------------------------------

def _dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _timed(fn, steps, warmup):
    """W untimed calls, then exactly `steps` calls between two device synchronisations.
    HIP events around every call, recorded on torch's current stream (the stream the
    binding launches on), give the per-call device durations. Returns (wall seconds of the
    timed region, mean per-call device ms)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, float(np.mean(per))


def _timed_batch(fn, steps, warmup):
    """Like _timed, for kernels of a few microseconds: one HIP event pair around all `steps`
    back-to-back calls (events around every call would add their own gaps). Returns the
    mean device ms per call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _timed_graph(fn, calls, replays, warmup):
    """For kernels shorter than a host launch: `calls` calls (fn(0) .. fn(calls - 1)) captured
    once in a HIP graph on the binding's stream (torch's current stream during capture; the
    graph holds kernel launches only), then `replays` replays between one HIP event pair, so
    the device runs the launches back to back without host gaps. Returns the mean device ms
    per call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(calls):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * calls)


def _workspace(total_tokens, num_seqs):
    import torch
    import linear_attention_recurrence_amd as gdn
    need = gdn.gdn_chunk_prefill_workspace_bytes(total_tokens, num_seqs, H_QK, H_V, D, D)
    return torch.empty(need, dtype=torch.uint8, device="cuda")


PREFILL_KERNELS = "gdn_chunk_prefill call: prep_kernel + state pass"

PREFILL_WORKLOADS = {
    # name: (input generator, seed, input sets rotated, with initial state, description)
    "t32768": ("config2", 1002, 2, True,
               "gated delta rule chunked prefill, B=1, T=32768, 16 QK / 32 V heads, d=128, "
               "chunk 64, bf16 q/k/v/o, fp32 state, S0 ~ N(0, 0.02) in, final state out"),
    "t4096": ("config1", 1001, 4, False,
              "gated delta rule chunked prefill, B=1, T=4096, 16 QK / 32 V heads, d=128, "
              "chunk 64, bf16 q/k/v/o, fp32 state, S0=0, final state out"),
}


def bench_prefill(name, steps, warmup):
    """One B=1 prefill workload of PREFILL_WORKLOADS; its input sets rotate so the 256 MB
    last-level cache cannot hold the working set across steps (one T=32768 set alone is
    about 0.8 GB). Returns (tokens, wall seconds, mean device ms per call)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    gen, seed, copies, with_s0, _ = PREFILL_WORKLOADS[name]
    sets = []
    T = None
    for c in range(copies):
        x = getattr(workloads, gen)(seed=seed + 97 * c)
        T = x.total_tokens
        sets.append(dict(q=_dev(x.q), k=_dev(x.k), v=_dev(x.v), g=_dev(x.g), b=_dev(x.beta),
                         cu=_dev(x.cu_seqlens), s0=_dev(x.initial_state),
                         o=torch.empty((T, H_V, D), dtype=torch.bfloat16, device="cuda"),
                         fin=torch.empty((1, H_V, D, D), dtype=torch.float32, device="cuda")))
        del x
    ws = _workspace(T, 1)
    scale = D ** -0.5

    def step(i):
        s = sets[i % copies]
        gdn.gdn_chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["b"], s["cu"], scale,
                              initial_state=s["s0"], final_state=s["fin"], o=s["o"], workspace=ws)

    wall, ms = _timed(step, steps, warmup)
    return T, wall, ms


def prefill_rooflines(tokens, num_seqs, with_s0, call_ms, counter_name, kernel):
    """HBM and matrix-core roofline objects of one prefill call: algorithmic bytes and FLOPs
    over the call's mean device time, with the counter figures when they describe the
    current kernels."""
    flops = prefill_flops(tokens)
    nbytes = prefill_bytes(tokens, num_seqs, with_s0)
    achieved = nbytes / (call_ms / 1e3) / 1e9
    tf = flops / (call_ms / 1e3) / 1e12
    hbm = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": achieved / HBM_PEAK_GBS,
           "traffic": counter(counter_name, "bytes", PREFILL_SOURCES),
           "kernel": kernel, "call_ms": call_ms, "algorithmic_bytes": nbytes}
    mfma = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": flops,
            "mfma_busy_counter": counter(counter_name, "mfma_busy", PREFILL_SOURCES)}
    return hbm, mfma


def bench_decode(steps, warmup):
    """256 sequences x 1 token over the 512 MiB fp32 pool, ring of 16 input sets."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    d = workloads.config3()
    pool = _dev(d.pool)
    q, k, v, g, b = _dev(d.q), _dev(d.k), _dev(d.v), _dev(d.g), _dev(d.beta)
    o = torch.empty((256, H_V, D), dtype=torch.bfloat16, device="cuda")

    def step(i):
        r = i % 16
        gdn.gdn_decode_step(q[r], k[r], v[r], g[r], b[r], pool, d.scale, o=o)

    return _timed(step, steps, warmup)


def conv_decode_bytes(num_seqs: int, K=4, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes the decode-time front end must move: each sequence's input row read, its
    K - 1 earlier inputs read, the new input kept (one row written) and q, k, v written
    (bf16), plus the conv weights (fp32) once."""
    ch = 2 * h_qk * D + h_v * D
    return float(num_seqs * ch * 2 * (1 + (K - 1) + 1 + 1) + ch * K * 4)


def bench_decode_front_end(steps, warmup):
    """256 sequences x 1 token: gdn_conv_decode_step over a [256][3][8192] bf16 window pool,
    then gdn_decode_step on its q, k and v over the 512 MiB state pool; a ring of 16 input
    sets; and gdn_decode_step_with_conv, the two in one launch. Returns (conv ms per call,
    wall seconds and ms per step of the two calls, the same for the one-launch form)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    d = workloads.config3()
    fe = workloads.make_frontend([16] * 256, with_initial_state=False, seed=1005)
    C = fe.mixed.shape[1]
    mixed = _dev(fe.mixed).view(256, 16, C).transpose(0, 1).contiguous()   # [ring][seq][C]
    w = _dev(fe.conv_weight)
    win = torch.zeros((256, 3, C), dtype=torch.bfloat16, device="cuda")
    pool = _dev(d.pool)
    g, b = _dev(d.g), _dev(d.beta)
    q = torch.empty((256, H_QK, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((256, H_V, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(v)

    def conv(i):
        gdn.gdn_conv_decode_step(mixed[i % 16], w, win, H_QK, H_V, D, D, fe.q_scale, q=q, k=k, v=v)

    def both(i):
        conv(i)
        gdn.gdn_decode_step(q, k, v, g[i % 16], b[i % 16], pool, 1.0, o=o)

    def fused(i):
        gdn.gdn_decode_step_with_conv(mixed[i % 16], w, win, g[i % 16], b[i % 16], pool, H_QK, H_V,
                                      D, D, fe.q_scale, 1.0, o=o)

    conv_ms = _timed_graph(conv, 16, max(1, steps // 16), warmup)
    wall, both_ms = _timed(both, steps, warmup)
    fwall, fused_ms = _timed(fused, steps, warmup)
    return conv_ms, wall, both_ms, fwall, fused_ms


def verify_bytes(num_seqs: int, n_tok: int, snapshots: bool, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes of one verify call: every state read and written once (fp32), the state
    after every token when snapshots are kept, and q, k, v, o (bf16), g and beta (fp32) of
    every token."""
    state = num_seqs * h_v * D * D * 4 * (2 + (n_tok if snapshots else 0))
    io = num_seqs * n_tok * (2 * h_qk * D * 2 + 2 * h_v * D * 2 + 2 * h_v * 4)
    return float(state + io)


def bench_verify(steps, warmup, n_tok=4):
    """256 sequences x n_tok draft tokens over the 512 MiB pool, with and without per-token
    snapshots (2 GiB at n_tok = 4). Returns {snapshots: (wall s, ms per call)}."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    d = workloads.make_decode(num_seqs=256, ring=n_tok, seed=1006)
    sm = lambda a: _dev(np.ascontiguousarray(np.swapaxes(a, 0, 1)))
    q, k, v, g, b = sm(d.q), sm(d.k), sm(d.v), sm(d.g), sm(d.beta)
    pool = _dev(d.pool)
    o = torch.empty((256, n_tok, H_V, D), dtype=torch.bfloat16, device="cuda")
    snaps = torch.empty((256, n_tok, H_V, D, D), dtype=torch.float32, device="cuda")
    out = {}
    for keep in (True, False):
        def call(i):
            gdn.gdn_verify_step(q, k, v, g, b, pool, d.scale, snapshots=snaps if keep else None, o=o)
        out[keep] = _timed(call, steps, warmup)
    return out


def bench_channel_decay(steps, warmup, prefill_reps=5):
    """The per-channel form: one decode step at 256 sequences over the 512 MiB pool (a ring of
    16 input sets, per-channel log-decays [256][32][128]), and the token-sequential prefill
    at B = 1, T = 4096 and at B = 16, T = 1024. Returns (decode wall s, decode ms, B = 1
    prefill ms, B = 16 prefill ms)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    d = workloads.config3()
    pool = _dev(d.pool)
    q, k, v, b = _dev(d.q), _dev(d.k), _dev(d.v), _dev(d.beta)
    g = _dev(workloads.channel_log_alpha(16 * 256, seed=1008).reshape(16, 256, H_V, D))
    o = torch.empty((256, H_V, D), dtype=torch.bfloat16, device="cuda")

    def step(i):
        r = i % 16
        gdn.gdn_channel_decay_decode_step(q[r], k[r], v[r], g[r], b[r], pool, d.scale, o=o)

    dwall, dms = _timed(step, steps, warmup)
    x = workloads.config1()
    xq, xk, xv, xb, cu = _dev(x.q), _dev(x.k), _dev(x.v), _dev(x.beta), _dev(x.cu_seqlens)
    xg = _dev(workloads.channel_log_alpha(4096, seed=1009))
    xo = torch.empty((4096, H_V, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, H_V, D, D), dtype=torch.float32, device="cuda")

    def prefill(i):
        gdn.gdn_channel_decay_prefill(xq, xk, xv, xg, xb, cu, x.scale, final_state=fin, o=xo)

    _, pms = _timed(prefill, prefill_reps, 1)
    y = workloads.make_prefill([1024] * 16, seed=1010)
    yq, yk, yv, yb, ycu = _dev(y.q), _dev(y.k), _dev(y.v), _dev(y.beta), _dev(y.cu_seqlens)
    yg = _dev(workloads.channel_log_alpha(16 * 1024, seed=1011))
    yo = torch.empty((16 * 1024, H_V, D), dtype=torch.bfloat16, device="cuda")
    yfin = torch.empty((16, H_V, D, D), dtype=torch.float32, device="cuda")

    def prefill16(i):
        gdn.gdn_channel_decay_prefill(yq, yk, yv, yg, yb, ycu, y.scale, final_state=yfin, o=yo)

    _, pms16 = _timed(prefill16, prefill_reps, 1)
    return dwall, dms, pms, pms16


def bench_epilogue(reps, warmup):
    """The output epilogue on the prefill's read-out shape (B = 1, T = 4096, 32 V heads,
    bf16, sigmoid gate): gdn_gated_rmsnorm back to back over four input sets in turn (400
    MB, more than the last-level cache holds). Returns (vectors, device ms per call)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    sets = []
    for s in range(4):
        o, z, w = workloads.epilogue_inputs(4096, H_V, seed=1012 + s)
        od = _dev(o)
        sets.append((od, _dev(z), _dev(w), torch.empty_like(od)))

    gdn.gdn_gated_rmsnorm(*sets[0][:3], out=sets[0][3])     # argument checks once
    # The timed loop calls the C entry point with its arguments prepared: a 20 us kernel is
    # shorter than the binding's per-call checks, which would otherwise set the pace.
    lib = gdn.load()
    args = [(od.data_ptr(), zd.data_ptr(), 0, wd.data_ptr(), 4096, H_V, D, 1e-6, 0, out.data_ptr(),
             torch.cuda.current_stream().cuda_stream) for od, zd, wd, out in sets]
    fn = lib.gdn_gated_rmsnorm

    def call(i):
        fn(*args[i % 4])

    return 4096 * H_V, _timed_batch(call, reps, warmup)


def bench_frontend(reps, warmup):
    """64 packed sequences (lengths uniform in [128, 8192]): gdn_conv_prep then
    gdn_chunk_prefill with per-sequence initial and final states, and the same through
    gdn_chunk_prefill_conv (the two in one call, through its workspace). Returns (tokens,
    sequences, conv ms, prefill ms, one-call ms)."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    fe = workloads.config4()
    T = fe.total_tokens
    N = fe.num_seqs
    mixed, w, cu = _dev(fe.mixed), _dev(fe.conv_weight), _dev(fe.cu_seqlens)
    g, b, s0 = _dev(fe.g), _dev(fe.beta), _dev(fe.initial_state)
    q = torch.empty((T, H_QK, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, H_V, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(v)
    fin = torch.empty_like(s0)
    ws = _workspace(T, N)
    wsc = torch.empty(gdn.gdn_chunk_prefill_conv_workspace_bytes(T, N, H_QK, H_V, D, D), dtype=torch.uint8,
                      device="cuda")

    def conv(i):
        gdn.gdn_conv_prep(mixed, w, cu, H_QK, H_V, D, D, fe.q_scale, q=q, k=k, v=v)

    def prefill(i):
        gdn.gdn_chunk_prefill(q, k, v, g, b, cu, 1.0, initial_state=s0, final_state=fin, o=o,
                              workspace=ws)

    def fused(i):
        gdn.gdn_chunk_prefill_conv(mixed, w, g, b, cu, H_QK, H_V, D, D, fe.q_scale, 1.0, initial_state=s0,
                                   final_state=fin, o=o, workspace=wsc)

    _, conv_ms = _timed(conv, reps, warmup)
    _, pre_ms = _timed(prefill, reps, warmup)
    _, fused_ms = _timed(fused, reps, warmup)
    return T, N, conv_ms, pre_ms, fused_ms


def fused_bytes(tokens: int, num_seqs: int, h_qk=H_QK, h_v=H_V) -> float:
    """HBM bytes of the prefill with the front end inside: the mixed input (bf16), o (bf16),
    g and beta (fp32), the initial and final states (fp32)."""
    ch = 2 * h_qk * D + h_v * D
    per_tok = ch * 2 + h_v * D * 2 + 2 * h_v * 4
    return float(tokens) * per_tok + num_seqs * h_v * D * D * 4 * 2


def bench_copy(steps, warmup, nbytes=1 << 30):
    """A plain device-to-device copy of `nbytes`: reads and writes exactly nbytes each."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    wall, ms = _timed(lambda i: dst.copy_(src), steps, warmup)
    return nbytes, ms


def cpu_baseline(min_core_seconds=10.0):
    """The fp64 oracle, as it stands, on the headline workload (B=1, T=32768, all 32 heads,
    S0 ~ N(0, 0.02)), run whole and repeated until about `min_core_seconds` of CPU work has
    been done."""
    import oracle
    import workloads
    x = workloads.config2()
    args = [x.as_f64(n) for n in ("q", "k", "v", "g", "beta")]
    s0 = x.as_f64("initial_state")
    threads = oracle.default_threads()
    reps, t = 0, time.perf_counter()
    while True:
        oracle.recurrence(*args, x.cu_seqlens, x.scale, initial_state=s0, n_threads=threads)
        reps += 1
        dt = time.perf_counter() - t
        if dt * threads >= min_core_seconds:
            break
    return {"value": reps * x.total_tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole headline workload (B=1, T=32768, 32 V heads, S0 given, fp64 "
                      "token loop) run %d times, %.2f s wall on %d threads" % (reps, dt, threads)}


def pmc_summary(root):
    """Per-kernel average counter values per dispatch from rocprofv3 --pmc CSV output."""
    lines = []
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        disp = collections.defaultdict(set)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = r.get("Kernel_Name", "")
                agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
                disp[k].add(r.get("Dispatch_Id", ""))
        lines.append("== %s" % os.path.relpath(f, root))
        for k, d in agg.items():
            nd = max(1, len(disp[k]))
            lines.append("  %-60s dispatches=%-4d %s" % (
                k[:60], nd, " ".join("%s=%.6g" % (c, v / nd) for c, v in sorted(d.items()))))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--workload", default="prefill,decode,frontend,epilogue",
                    help="comma list of prefill (both prefill_t32768 and prefill_t4096), decode, "
                         "frontend, epilogue, copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-summary", metavar="DIR")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the Gated DeltaNet path here has no multi-GPU "
              "mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    work = [w.strip() for w in args.workload.split(",") if w.strip()]
    import torch
    torch.cuda.set_device(0)
    out = {}

    if "prefill" in work or "prefill_t32768" in work:
        T, wall, call_ms = bench_prefill("t32768", args.steps, args.warmup)
        hbm, mfma = prefill_rooflines(T, 1, True, call_ms, "prefill_t32768", PREFILL_KERNELS)
        out.update({
            "metric": METRIC,
            "value": T * args.steps / wall,
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": wall * 1e3 / args.steps,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": PREFILL_WORKLOADS["t32768"][4],
                       "global_batch": 1, "seq_len": T, "parallelism": "none (1 GPU)"},
            "roofline": hbm,
            "roofline_mfma": mfma,
            # context only: the whole-model claim the pages make, which names no hardware and
            # measures a different thing than this mixer's tokens/s
            "pages_claim": "whole Qwen3-Next model: about 10x the inference throughput of "
                           "Qwen3-32B at contexts beyond 32K tokens; no hardware named",
        })
    if "prefill" in work or "prefill_t4096" in work:
        psteps = max(20, args.steps)
        T1, wall1, ms1 = bench_prefill("t4096", psteps, args.warmup)
        hbm1, mfma1 = prefill_rooflines(T1, 1, False, ms1, "prefill_t4096", PREFILL_KERNELS)
        out["prefill_b1_t4096"] = {"workload": PREFILL_WORKLOADS["t4096"][4], "steps": psteps,
                                   "ms_per_step": wall1 * 1e3 / psteps,
                                   "tokens_per_s": T1 * psteps / wall1,
                                   "roofline": hbm1, "roofline_mfma": mfma1}
    if "decode" in work:
        dsteps = args.decode_steps
        wall, dms = bench_decode(dsteps, args.warmup)
        dbytes = decode_bytes(256)
        achieved = dbytes / (dms / 1e3) / 1e9
        out["decode"] = {
            "workload": "decode step, 256 sequences x 1 token, 16 QK / 32 V heads, fp32 state "
                        "pool 512 MiB updated in place, ring of 16 input sets",
            "steps": dsteps, "ms_per_step": wall * 1e3 / dsteps,
            "tokens_per_s": 256 * dsteps / wall,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "traffic": counter("decode", "bytes", DECODE_SOURCES),
                         "kernel": "decode_kernel<bf16>", "kernel_ms": dms,
                         "algorithmic_bytes": dbytes}}
    if "decode" in work:
        dsteps = args.decode_steps
        cms, fwall, fms, uwall, ums = bench_decode_front_end(dsteps, args.warmup)
        ubytes = decode_bytes(256) + conv_decode_bytes(256) - 256 * (2 * H_QK + H_V) * D * 2 * 2
        cbytes = conv_decode_bytes(256)
        out["decode_front_end"] = {
            "workload": "decode step with the front end, 256 sequences x 1 token: conv k=4 over "
                        "a bf16 window pool of the last 3 inputs, then the decode step; ring of "
                        "16 input sets",
            "steps": dsteps, "ms_per_step": fwall * 1e3 / dsteps,
            "tokens_per_s": 256 * dsteps / fwall,
            "conv_decode": {"kernel": "conv_decode_kernel", "kernel_ms_graph_replay": cms,
                            "algorithmic_bytes": cbytes,
                            "achieved_GBs": cbytes / (cms / 1e3) / 1e9},
            "one_launch": {"entry_point": "gdn_decode_step_with_conv", "ms_per_step": uwall * 1e3 / dsteps,
                           "tokens_per_s": 256 * dsteps / uwall, "kernel": "decode_conv_kernel<2>",
                           "kernel_ms": ums,
                           "roofline": {"bound": "hbm", "achieved": ubytes / (ums / 1e3) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": ubytes / (ums / 1e3) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes": ubytes}}}
    if "decode" in work:
        vsteps = max(20, args.decode_steps // 10)
        res = bench_verify(vsteps, args.warmup)
        out["verify"] = {
            "workload": "verify step, 256 sequences x 4 draft tokens, 16 QK / 32 V heads, fp32 "
                        "state pool 512 MiB updated in place",
            "steps": vsteps}
        for keep, (vwall, vms) in res.items():
            vb = verify_bytes(256, 4, keep)
            achieved = vb / (vms / 1e3) / 1e9
            out["verify"]["with_snapshots" if keep else "without_snapshots"] = {
                "ms_per_call": vms, "tokens_per_s": 256 * 4 * vsteps / vwall,
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                             "kernel": "seq_kernel<bf16>", "algorithmic_bytes": vb}}
    if "decode" in work:
        csteps = max(20, args.decode_steps // 10)
        cwall, cms, cpms, cpms16 = bench_channel_decay(csteps, args.warmup)
        # 7 d^2 flops per (token, V head): S k and S q (2 d^2 each), the decay and the rank-1
        # update (3 d^2)
        cflops = 16 * 1024 * H_V * 7 * D * D
        ctf = cflops / (cpms16 / 1e3) / 1e12
        cb = decode_bytes(256) + 256 * H_V * D * 4 - 256 * H_V * 4   # g per channel
        achieved = cb / (cms / 1e3) / 1e9
        out["channel_decay"] = {
            "workload": "per-channel decay form (one decay per value channel, correction from the "
                        "state before the decay): decode step at 256 sequences x 1 token over the "
                        "512 MiB pool; token-sequential prefill at B=1, T=4096 and at "
                        "B=16, T=1024, 32 V heads",
            "decode": {"steps": csteps, "ms_per_step": cwall * 1e3 / csteps,
                       "tokens_per_s": 256 * csteps / cwall,
                       "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                                    "kernel": "decode_kernel<bf16, true>", "kernel_ms": cms,
                                    "algorithmic_bytes": cb}},
            "prefill_b1_t4096": {"ms_per_call": cpms, "tokens_per_s": 4096 / (cpms / 1e3),
                                 "bound": "latency: one chain of 4096 dependent tokens per V head"},
            "prefill_b16_t1024": {"ms_per_call": cpms16, "tokens_per_s": 16 * 1024 / (cpms16 / 1e3),
                                  "roofline": {"bound": "alu", "achieved": ctf,
                                               "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                               "frac": ctf / FP32_PEAK_TFLOPS,
                                               "kernel": "rows_kernel<bf16, true, 8, 4>",
                                               "algorithmic_flops": cflops}}}
    if "frontend" in work:
        T4, N4, conv_ms, pre_ms, fused_ms = bench_frontend(10, 2)
        hbm4, mfma4 = prefill_rooflines(T4, N4, True, pre_ms, "prefill_packed64", PREFILL_KERNELS)
        cb = conv_prep_bytes(T4)
        fb = fused_bytes(T4, N4)
        out["frontend_prefill"] = {
            "workload": "64 packed sequences, lengths uniform in [128, 8192], conv k=4 front end "
                        "then prefill with S0 and final states",
            "total_tokens": T4, "conv_prep_ms": conv_ms, "prefill_ms": pre_ms,
            "tokens_per_s_with_front_end": T4 / ((conv_ms + pre_ms) / 1e3),
            "tokens_per_s_prefill_only": T4 / (pre_ms / 1e3),
            "conv_prep_roofline": {"bound": "hbm", "achieved": cb / (conv_ms / 1e3) / 1e9,
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": cb / (conv_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                   "kernel": "conv_prep_kernel", "kernel_ms": conv_ms,
                                   "algorithmic_bytes": cb},
            "prefill_roofline": hbm4, "prefill_roofline_mfma": mfma4,
            "one_call": {"entry_point": "gdn_chunk_prefill_conv (the front end and the prefill in one call)",
                         "ms_per_call": fused_ms, "tokens_per_s": T4 / (fused_ms / 1e3),
                         "roofline": {"bound": "hbm", "achieved": fb / (fused_ms / 1e3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": fb / (fused_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                      "traffic": counter("prefill_conv_packed64", "bytes", PREFILL_CONV_SOURCES),
                                      "kernel": "gdn_chunk_prefill_conv call: conv_prep_kernel + "
                                                "prep_kernel<false, 2> + state_kernel<8, true>",
                                      "call_ms": fused_ms, "algorithmic_bytes": fb}}}
    if "epilogue" in work:
        nvec, ems = bench_epilogue(200, 10)
        eb = nvec * D * 2 * 3          # o and z read, out written, bf16
        achieved = eb / (ems / 1e3) / 1e9
        out["epilogue"] = {
            "workload": "output epilogue (per-head RMS norm with the zero-centred scale, then "
                        "the sigmoid output gate) on the read-out of B=1, T=4096, 32 V heads, bf16; "
                        "four input sets in turn",
            "ms_per_call": ems, "tokens_per_s": 4096 / (ems / 1e3),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "kernel": "gated_rmsnorm_kernel<bf16, false>",
                         "algorithmic_bytes": eb}}
    if "copy" in work:
        nb, cms = bench_copy(max(5, args.steps), args.warmup)
        out["copy"] = {"bytes_each_way": nb, "ms": cms, "GBs_read_plus_write": 2 * nb / (cms / 1e3) / 1e9}
    if ("prefill" in work or "prefill_t32768" in work) and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
