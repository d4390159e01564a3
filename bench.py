"""Benchmark of the Gated DeltaNet mixer on one MI355X.

Headline: chunked prefill throughput (tokens/s) on the Qwen3-Next layer shape, B=1, T=4096,
16 QK heads shared by 32 V heads, head dim 128, bf16 q/k/v, S0 = 0, fp32 final states. A
step is one gdn_chunk_prefill call over the whole batch (every step of the chunked method
runs inside it). Alongside: decode-step HBM bandwidth on a 256-sequence fp32 state pool,
and the packed variable-length front end + prefill. The fp64 oracle is timed on the host
cores on the headline workload as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s/GPU (H_v=32,d=128) + decode state GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s

D = 128
C = 64
H_QK, H_V = 16, 32


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must compute and move, not what a kernel happens to do)
# ---------------------------------------------------------------------------------------

def prefill_flops(tokens: int, h_v: int = H_V) -> float:
    """Matrix-product FLOPs of the chunked form per token and V head: five C x C x d
    products (K K^T, Q K^T, T(beta gam)K, T(beta)V, P U) = 10 C d, and three C x d x d
    products (W S^T, Q S^T, U^T K) = 6 d^2."""
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


def _time_launches(fn, n_launches, warmup):
    """Runs fn(i) warmup times, then n_launches times between HIP events on torch's current
    stream (the stream libgdn launches on). Returns (total_ms, per-launch ms list)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_launches)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_launches)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n_launches):
        starts[i].record()
        fn(i)
        ends[i].record()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), [s.elapsed_time(e) for s, e in zip(starts, ends)]


def bench_prefill_config1(steps, warmup, copies=4):
    """B=1, T=4096 prefill; `copies` input sets rotate so the 256 MB last-level cache cannot
    hold the working set across steps."""
    import torch
    import linear_attention_recurrence_amd as gdn
    import workloads
    sets = []
    for c in range(copies):
        x = workloads.config1(seed=1001 + 97 * c)
        sets.append(dict(q=_dev(x.q), k=_dev(x.k), v=_dev(x.v), g=_dev(x.g), b=_dev(x.beta),
                         cu=_dev(x.cu_seqlens),
                         o=torch.empty((4096, H_V, D), dtype=torch.bfloat16, device="cuda"),
                         fin=torch.empty((1, H_V, D, D), dtype=torch.float32, device="cuda")))
    scale = D ** -0.5

    def step(i):
        s = sets[i % copies]
        gdn.gdn_chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["b"], s["cu"], scale,
                              final_state=s["fin"], o=s["o"])

    total_ms, per = _time_launches(step, steps, warmup)
    return total_ms, per


def bench_decode_config3(steps, warmup):
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

    total_ms, per = _time_launches(step, steps, warmup)
    return total_ms, per


def bench_frontend_config4(reps, warmup):
    """64 packed sequences (lengths uniform in [128, 8192]): gdn_conv_prep then
    gdn_chunk_prefill with per-sequence initial and final states."""
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

    def conv(i):
        gdn.gdn_conv_prep(mixed, w, cu, H_QK, H_V, D, D, fe.q_scale, q=q, k=k, v=v)

    def prefill(i):
        gdn.gdn_chunk_prefill(q, k, v, g, b, cu, 1.0, initial_state=s0, final_state=fin, o=o)

    conv_ms, _ = _time_launches(conv, reps, warmup)
    pre_ms, _ = _time_launches(prefill, reps, warmup)
    return T, N, conv_ms / reps, pre_ms / reps


def cpu_baseline():
    """The fp64 oracle, as it stands, on the headline workload (all 32 heads, T = 4096)."""
    import oracle
    import workloads
    x = workloads.config1()
    args = [x.as_f64(n) for n in ("q", "k", "v", "g", "beta")]
    threads = oracle.default_threads()
    t = time.perf_counter()
    oracle.recurrence(*args, x.cu_seqlens, x.scale, n_threads=threads)
    dt = time.perf_counter() - t
    return {"value": x.total_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "whole workload: B=1, T=4096, 32 V heads, fp64 token loop, %.2f s wall" % dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true", help="headline prefill only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)

    total_ms, per = bench_prefill_config1(args.steps, args.warmup)
    kernel_ms = float(np.mean(per))
    tokens = 4096
    value = tokens * args.steps / (total_ms / 1e3)
    flops = prefill_flops(tokens)
    nbytes = prefill_bytes(tokens, 1, with_s0=False)
    achieved_gbs = nbytes / (kernel_ms / 1e3) / 1e9
    achieved_tf = flops / (kernel_ms / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta rule chunked prefill, B=1, T=4096, 16 QK / 32 V heads, "
                               "d=128, chunk 64, bf16 q/k/v/o, fp32 state, S0=0, final state out",
                   "global_batch": 1, "seq_len": tokens, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "chunk_prefill_kernel", "kernel_ms": kernel_ms,
                     "algorithmic_bytes": nbytes},
        "roofline_mfma": {"achieved": achieved_tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": achieved_tf / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": flops},
    }
    if not args.no_extras:
        dsteps = 1000
        dtot, dper = bench_decode_config3(dsteps, 20)
        dms = float(np.mean(dper))
        dbytes = decode_bytes(256)
        out["decode"] = {"workload": "decode step, 256 sequences x 1 token, 16 QK / 32 V heads, "
                                     "fp32 state pool 512 MiB in place, 1000 steps",
                         "ms_per_step": dtot / dsteps, "kernel_ms": dms,
                         "tokens_per_s": 256 * dsteps / (dtot / 1e3),
                         "achieved_GBs": dbytes / (dms / 1e3) / 1e9,
                         "frac_of_hbm_peak": dbytes / (dms / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": dbytes}
        T4, N4, conv_ms, pre_ms = bench_frontend_config4(10, 2)
        out["frontend_prefill"] = {
            "workload": "64 packed sequences, lengths uniform in [128, 8192], conv k=4 front end "
                        "then prefill with S0 and final states",
            "total_tokens": T4, "conv_prep_ms": conv_ms, "prefill_ms": pre_ms,
            "tokens_per_s_with_front_end": T4 / ((conv_ms + pre_ms) / 1e3),
            "tokens_per_s_prefill_only": T4 / (pre_ms / 1e3),
            "conv_prep_GBs": conv_prep_bytes(T4) / (conv_ms / 1e3) / 1e9,
            "prefill_GBs": prefill_bytes(T4, N4, True) / (pre_ms / 1e3) / 1e9,
            "prefill_TFLOPs": prefill_flops(T4) / (pre_ms / 1e3) / 1e12}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
