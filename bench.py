#!/usr/bin/env python3
"""Benchmark of the fused RoPE causal prefill attention on one MI355X.

A step is one full pass of the hot path -- one prefill_attn_run call: RoPE of
Q and K, causal Q.K^T, blocked online softmax and P.V for every (batch, head)
-- over a synthetic batch already resident in HBM.  The default workload is
the long-prompt case (batch 1, 32 heads, seq 4096, head_dim 96, bf16 inputs
with per-head scales, RoPE theta 1e4, causal).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--cpu-budget SECONDS | --no-cpu-baseline] [--calib-copy]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RoPE causal prefill attention: tokens/s and TFLOP/s (% bf16 MFMA peak)"
PEAK_TFLOPS = 2516.6       # MI355X dense fp16/bf16 matrix-core peak (256 CU x 4096 FLOP/clk x 2.4 GHz)
DEFAULT_WORKLOAD = "mha_bf16_h32_s4096_d96"
KERNEL_SOURCE = os.path.join(ROOT, "rope_causal_attention_amd", "csrc", "attn_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def algorithmic_bytes(w):
    """Q, K, V read once, O (fp32) written once, RoPE table rows read once."""
    el = {"f32": 4, "bf16": 2, "i16": 2}[w.dtype]
    q = w.batch * w.seq_len * w.n_heads * w.head_dim * el
    kv = 2 * w.batch * w.seq_len * w.n_kv_heads * w.head_dim * (el if w.dtype != "i16" else 2)
    o = w.batch * w.seq_len * w.n_heads * w.head_dim * 4
    tab = w.seq_len * w.head_dim * (4 if w.dtype != "i16" else 2)
    return q + kv + o + tab


def traffic_record(w):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle on whole heads of batch element 0 until the budget
    is spent; scale to the full workload."""
    import numpy as np

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    q, k, v = synth.make_inputs(w)
    g = w.n_heads // w.n_kv_heads
    one = synth.workload(w.name, batch=1, n_heads=1, n_kv_heads=1)
    heads, t_total = 0, 0.0
    for h in range(w.n_heads):
        qs, ks, vs = q[:1, :, h:h + 1], k[:1, :, h // g:h // g + 1], v[:1, :, h // g:h // g + 1]
        t0 = time.perf_counter()
        if w.dtype == "i16":
            oracle.attention_i16(synth.to_f64(qs), synth.to_f64(ks), synth.to_f64(vs), rope_theta=w.rope_theta,
                                 score_scale=one.score_scale)
        else:
            oracle.attention(synth.to_f64(qs), synth.to_f64(ks), synth.to_f64(vs), rope_theta=w.rope_theta,
                             scale=one.score_scale or None)
        t_total += time.perf_counter() - t0
        heads += 1
        if t_total >= budget_s:
            break
    per_head = t_total / heads
    full = per_head * w.batch * w.n_heads
    return {
        "value": w.batch * w.seq_len / full,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} of {w.batch * w.n_heads} (batch, head) slices, full sequence, "
                  f"{t_total:.1f} s; scaled to the whole workload",
        "tflops": w.flops() / full / 1e12,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path "
            "(heads or sequence shards would each run this kernel at their own shape). Use --gpus 1.")
        sys.exit(2)

    import torch

    import rope_causal_attention_amd as pa
    import synth

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    q, k, v = synth.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty((w.batch, w.seq_len, w.n_heads, w.head_dim), dtype=torch.float32, device="cuda")
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.max_seq or w.seq_len, w.rope_theta)
    stream = torch.cuda.current_stream()

    def step():
        attn(qd, kd, vd, score_scale=w.score_scale, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if attn.status() != pa.PA_OK:
        raise RuntimeError("status word set during warm-up")

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    if attn.status() != pa.PA_OK:
        raise RuntimeError("status word set during the timed steps")
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{w.name}: {ms * 1e3:.1f} us/step (host wall {t_host / args.steps * 1e6:.1f} us/step)")

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = w.tokens / (ms * 1e-3)
    log(f"{tflops:.1f} TFLOP/s = {100 * tflops / PEAK_TFLOPS:.1f}% of {PEAK_TFLOPS} ; {tokens_s:.4g} tokens/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"cpu oracle: {cpu['value']:.4g} tokens/s on {cpu['cores']} BLAS threads ({cpu['sample']})")

    result = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == "bf16" else {"f32": "f32", "i16": "i8"}[w.dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "seq_len": w.seq_len,
            "n_heads": w.n_heads,
            "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim,
            "input_dtype": w.dtype,
            "rope_theta": w.rope_theta,
            "causal": True,
            "tflops": tflops,
            "pct_bf16_peak": 100 * tflops / PEAK_TFLOPS,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / PEAK_TFLOPS,
            "traffic": traffic_record(w),
            "algorithmic_bytes": algorithmic_bytes(w),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    attn.close()


if __name__ == "__main__":
    main()
