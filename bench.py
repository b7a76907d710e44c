#!/usr/bin/env python3
"""Benchmark of the fused RoPE causal prefill attention on one MI355X.

A step is one full pass of the hot path -- one prefill_attn_run call: RoPE of
Q and K, causal Q.K^T, blocked online softmax and P.V for every (batch, head)
-- over a synthetic batch already resident in HBM.  The default workload is
the long-prompt case (batch 1, 32 heads, seq 4096, head_dim 96, bf16 inputs
with per-head scales, RoPE theta 1e4, causal).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--cpu-budget SECONDS | --no-cpu-baseline] [--calib-copy]
                    [--mode prefill|chunked|decode] [--chunk N]

--mode chunked prefills the same prompt in chunks of N tokens through a KV
cache (a ring of seq_len slots): each chunk's K/V is written to the cache and
its queries attend to every cached key in one launch
(prefill_attn_run_cached_update, which splits the cached keys over several
workgroups; --no-split keeps one workgroup per query block;
--separate-update runs prefill_attn_kv_cache_update, then
prefill_attn_run_cached_splitk).  A step is the whole prompt, all chunks.

--mode decode times decode attention (prefill_attn_decode): 16 sequences each
with one new token at position 4095 against a paged bf16 KV cache of 4096
tokens, 32 query / 8 KV heads of dimension 128.  A step is one new token for
every sequence; the roofline is HBM bandwidth (every cached K and V row read
once).
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
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
BALANCE = PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte where the two bounds meet
DEFAULT_WORKLOAD = "mha_bf16_h32_s4096_d96"
KERNEL_SOURCE = os.path.join(ROOT, "rope_causal_attention_amd", "csrc", "attn_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def algorithmic_bytes(w):
    """Q, K, V read once, O (fp32) written once, RoPE table rows read once."""
    el = {"f32": 4, "bf16": 2, "i16": 2, "bf16q": 2}[w.dtype]
    q = w.batch * w.seq_len * w.n_heads * w.head_dim * el
    kv = 2 * w.batch * w.seq_len * w.n_kv_heads * w.head_dim * (el if w.dtype != "i16" else 2)
    o = w.batch * w.seq_len * w.n_heads * w.head_dim * 4
    # (cos, sin) pairs per position: fp32 for the float paths, Q1.14 int16 for the integer ones
    tab = w.seq_len * w.head_dim * (4 if w.dtype in ("f32", "bf16") else 2)
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
        if w.dtype == "bf16q":
            oracle.attention_i16_quantized(qs.float().numpy(), ks.float().numpy(), synth.to_f64(vs),
                                           rope_theta=w.rope_theta, score_scale=w.score_scale or None)
        elif w.dtype == "i16":
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


DECODE = dict(batch=16, ctx=4096, n_heads=32, n_kv_heads=8, head_dim=128, rope_theta=1e4, block=64, seed=2024)


def calib_copy(torch):
    """A plain 256 MiB elementwise copy: what the HBM byte counters read for known traffic."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_decode(args, torch, pa):
    """Decode attention over a paged bf16 cache; prints one JSON line."""
    import numpy as np

    c = DECODE
    B, T, Hq, Hkv, D = c["batch"], c["ctx"], c["n_heads"], c["n_kv_heads"], c["head_dim"]
    g = torch.Generator().manual_seed(c["seed"])
    n_blocks = B * T // c["block"]
    kc = torch.randn((n_blocks * c["block"], Hkv, D), generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn((n_blocks * c["block"], Hkv, D), generator=g).to(torch.bfloat16).cuda()
    q = torch.randn((B, Hq, D), generator=g).to(torch.bfloat16).cuda()
    perm = np.random.default_rng(c["seed"]).permutation(n_blocks)
    per = T // c["block"]
    rows = [pa.prefill_attn_paged_map(perm[b * per:(b + 1) * per], c["block"], T) for b in range(B)]
    kv_map = torch.from_numpy(np.stack(rows)).cuda()
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    attn = pa.PrefillAttention(Hq, Hkv, D, T, c["rope_theta"])
    ws = torch.empty(pa.prefill_attn_decode_workspace_size(attn.handle, B, 64), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        attn.decode(q, kc, vc, kv_map, pos_offsets=pos, workspace=ws, out=out, stream=stream, n_split=args.n_split)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if attn.status() != pa.PA_OK:
        raise RuntimeError("status word set during warm-up")
    if args.calib_copy:
        calib_copy(torch)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # K and V rows read once, q read, O written, the map row read.
    algo = 2 * B * T * Hkv * D * 2 + B * Hq * D * 2 + B * Hq * D * 4 + B * T * 4
    gbs = algo / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s = {100 * gbs / 8000:.1f}% of 8 TB/s")
    print(json.dumps({
        "metric": "decode attention over a KV cache: new tokens/s (HBM GB/s)",
        "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode_bf16_b{B}_h{Hq}kv{Hkv}_ctx{T}_d{D}", "batch": B, "context": T,
                   "n_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "input_dtype": "bf16", "cache": "paged, 64"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": 8000.0, "unit": "GB/s", "frac": gbs / 8000.0,
                     "traffic": None, "algorithmic_bytes": algo},
        "cpu_baseline": None,
    }), flush=True)
    attn.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=70)
    ap.add_argument("--samples", type=int, default=7,
                    help="the timed steps are split into this many equal samples; the median sample is reported")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (HBM counter calibration)")
    ap.add_argument("--mode", choices=["prefill", "chunked", "decode"], default="prefill")
    ap.add_argument("--chunk", type=int, default=1024, help="chunk length for --mode chunked")
    ap.add_argument("--pwl-softmax", action="store_true",
                    help="int16 workload with the piecewise-linear softmax (PA_IN_I16_PWL)")
    ap.add_argument("--split", dest="n_split", type=int, default=0,
                    help="split count for --mode chunked / decode (0 = chosen by the library)")
    ap.add_argument("--no-split", dest="split", action="store_false",
                    help="--mode chunked without split-K over the cached keys")
    ap.add_argument("--separate-update", dest="fuse", action="store_false",
                    help="--mode chunked with the cache update as its own launch (kv_cache_update, then "
                         "run_cached) instead of prefill_attn_run_cached_update")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(heads or sequence shards would each run this kernel at their own shape). Use --gpus 1.")
        sys.exit(2)

    import torch

    import rope_causal_attention_amd as pa
    import synth

    torch.cuda.set_device(0)
    if args.mode == "decode":
        return bench_decode(args, torch, pa)
    w = synth.WORKLOADS[args.workload]
    q, k, v = synth.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty((w.batch, w.seq_len, w.n_heads, w.head_dim), dtype=torch.float32, device="cuda")
    attn = pa.PrefillAttention(w.n_heads, w.n_kv_heads, w.head_dim, w.max_seq or w.seq_len, w.rope_theta)
    stream = torch.cuda.current_stream()

    if args.mode == "prefill":
        def step():
            attn(qd, kd, vd, score_scale=w.score_scale, out=out, stream=stream, quantize=w.dtype == "bf16q",
                 pwl_softmax=args.pwl_softmax)
    else:
        # Ring cache of seq_len slots starting at slot 1000 (wraps), one map row per sequence.
        S, B = w.seq_len, w.batch
        kc = torch.empty((B * S, w.n_kv_heads, w.head_dim), dtype=kd.dtype, device="cuda")
        vc = torch.empty((B * S, w.n_kv_heads, w.head_dim), dtype=vd.dtype, device="cuda")
        ring = [pa.prefill_attn_ring_map(S, 1000 % S, S).astype("int64") + b * S for b in range(B)]
        kv_map = torch.tensor(ring, dtype=torch.int32, device="cuda")
        chunks = [(p, min(args.chunk, S - p)) for p in range(0, S, args.chunk)]
        pieces = [(torch.full((B,), p, dtype=torch.int32, device="cuda"), qd[:, p:p + n].contiguous(),
                   kd[:, p:p + n].contiguous(), vd[:, p:p + n].contiguous()) for p, n in chunks]
        outs = [torch.empty(x[1].shape, dtype=torch.float32, device="cuda") for x in pieces]
        # Split-K over the cached keys (the library picks the split), workspace for up to 16 splits.
        ws = torch.empty(pa.prefill_attn_run_cached_workspace_size(attn.handle, B, args.chunk,
                                                                   max(16, args.n_split)),
                         dtype=torch.uint8, device="cuda")

        def step():
            for (off, qc, kn, vn), oc in zip(pieces, outs):
                if args.fuse:
                    attn.run_cached_update(qc, kn, vn, kc, vc, kv_map, pos_offsets=off, score_scale=w.score_scale,
                                           out=oc, stream=stream, n_split=args.n_split if args.split else 1,
                                           workspace=ws if args.split else None)
                    continue
                attn.kv_cache_update(kn, vn, kc, vc, kv_map, off, stream=stream)
                attn.run_cached(qc, kc, vc, kv_map, pos_offsets=off, score_scale=w.score_scale, out=oc,
                                stream=stream, n_split=args.n_split if args.split else 1,
                                workspace=ws if args.split else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if attn.status() != pa.PA_OK:
        raise RuntimeError("status word set during warm-up")

    if args.calib_copy:
        calib_copy(torch)

    # Measured roofline denominators (matrix-core peak, shader clock).
    peak_meas, clock_ghz = max(pa.prefill_attn_device_peak(stream) for _ in range(2))
    log(f"measured matrix-core peak {peak_meas:.0f} TFLOP/s at {clock_ghz:.3f} GHz "
        f"(vendor {PEAK_TFLOPS} at 2.4 GHz)")

    # The timed steps in equal samples, each bracketed by events on the launch
    # stream; the median sample is the figure (the clock and the temperature
    # move between samples).
    n_samples = max(1, min(args.samples, args.steps))
    per = args.steps // n_samples
    sizes = [per + (1 if i < args.steps % n_samples else 0) for i in range(n_samples)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_samples + 1)]
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    marks[0].record(stream)
    for i, n in enumerate(sizes):
        for _ in range(n):
            step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    if attn.status() != pa.PA_OK:
        raise RuntimeError("status word set during the timed steps")
    sample_ms = sorted(marks[i].elapsed_time(marks[i + 1]) / sizes[i] for i in range(n_samples))
    ms = sample_ms[len(sample_ms) // 2]
    log(f"{w.name} [{args.mode}]: median {ms * 1e3:.1f} us/step over {n_samples} samples "
        f"(min {sample_ms[0] * 1e3:.1f}, max {sample_ms[-1] * 1e3:.1f}; "
        f"host wall {t_host / args.steps * 1e6:.1f} us/step)")

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = w.tokens / (ms * 1e-3)
    log(f"{tflops:.1f} TFLOP/s = {100 * tflops / PEAK_TFLOPS:.1f}% of {PEAK_TFLOPS} ; {tokens_s:.4g} tokens/s")

    # The roofline's achieved rate is per launch: a second pass brackets every
    # launch with its own pair of events on the launch stream, so the gaps
    # between back-to-back launches that the step time includes are left out.
    # (One launch per step in prefill mode; a chunked step is all its launches.)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a0, a1 in pairs:
        a0.record(stream)
        step()
        a1.record(stream)
    torch.cuda.synchronize()
    launch_all = sorted(a0.elapsed_time(a1) for a0, a1 in pairs)
    launch_ms = launch_all[len(launch_all) // 2]
    launch_tflops = flops / (launch_ms * 1e-3) / 1e12
    log(f"per launch (median of {len(launch_all)}): {launch_ms * 1e3:.1f} us = {launch_tflops:.1f} TFLOP/s "
        f"({100 * launch_tflops / PEAK_TFLOPS:.1f}% of {PEAK_TFLOPS}, "
        f"{100 * launch_tflops / peak_meas:.1f}% of the measured {peak_meas:.0f})")
    algo = algorithmic_bytes(w)
    hbm_bound = args.mode == "prefill" and flops / algo < BALANCE
    if hbm_bound:
        gbs = algo / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}
        log(f"HBM-bound workload ({flops / algo:.0f} FLOP/B < {BALANCE:.0f}): {gbs:.0f} GB/s")
    else:
        roof = {"bound": "mfma", "achieved": launch_tflops, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": launch_tflops / PEAK_TFLOPS}

    cpu = None
    if not args.no_cpu_baseline and args.mode == "prefill":
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
        "dtype": "f16" if w.dtype == "bf16" else {"f32": "f32", "i16": "i8", "bf16q": "i8"}[w.dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name if args.mode == "prefill" else
            f"{w.name}, chunked prefill in chunks of {args.chunk}" + ("" if args.split else ", no split-K")
            + ("" if args.fuse else ", separate cache update"),
            "mode": args.mode,
            "softmax": "piecewise-linear" if args.pwl_softmax else "exp",
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
        "roofline": dict(roof, **{
            "launch_us": launch_ms * 1e3,
            "traffic": traffic_record(w) if args.mode == "prefill" else None,
            "algorithmic_bytes": algo,
            "flop": flops,
            "measured_mfma_peak_tflops": peak_meas,
            "shader_clock_ghz": clock_ghz,
            "frac_of_measured_peak": launch_tflops / peak_meas if peak_meas else None,
            "samples_us": [round(x * 1e3, 2) for x in sample_ms],
        }),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    attn.close()


if __name__ == "__main__":
    main()
