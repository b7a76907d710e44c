"""The bench's output contract and the inputs of its roofline.

CPU: a request for more than one GPU is refused before any GPU work; the
FLOP and algorithmic-byte figures of the long-prompt workload are the closed
forms; the HBM-traffic record is used only when it was taken on the current
kernel source.  GPU: one short bench run prints one JSON line with every
field of the contract.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _run_bench(*args, env=None, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run_bench(env=env, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_long_prompt_roofline_inputs():
    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    B, S, H, Hkv, D = w.batch, w.seq_len, w.n_heads, w.n_kv_heads, w.head_dim
    assert (B, S, H, Hkv, D, w.dtype) == (1, 4096, 32, 32, 96, "bf16")
    # Causal pairs S(S+1)/2 per head, 2 matmuls x 2 FLOP per multiply-add.
    assert w.flops() == 4 * B * H * D * (S * (S + 1) // 2) == 103_104_380_928
    # Q, K, V bf16 read once + O fp32 written once + one fp32 (cos, sin) table row per position.
    assert bench.algorithmic_bytes(w) == 3 * S * H * D * 2 + S * H * D * 4 + S * D * 4 == 127_401_984
    assert bench.PEAK_TFLOPS == 2516.6
    # matrix-bound: its FLOP per algorithmic byte is above the machine balance
    assert w.flops() / bench.algorithmic_bytes(w) > bench.BALANCE


def test_short_prompts_are_hbm_bound():
    """The 512-token prompts sit below the balance point: the bench reports them in GB/s."""
    for name in ("mha_bf16_h32_s512_d128", "gqa_bf16_b16_h16kv8_s512_d128"):
        w = synth.WORKLOADS[name]
        assert w.flops() / bench.algorithmic_bytes(w) < bench.BALANCE, name
    assert abs(bench.BALANCE - 2516.6e12 / 8000e9) < 1e-9


def test_traffic_record_only_for_the_current_kernel_source(monkeypatch):
    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(path) as f:
        rec = json.load(f)
    got = bench.traffic_record(w)
    assert got is None or (rec["kernel_sha"] == bench.kernel_sha() and got == rec["hbm_bytes_per_launch"])
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 64)
    assert bench.traffic_record(w) is None


@pytest.mark.gpu
def test_bench_prints_one_contract_line():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    print("[gpu-case] bench.py --steps 3 --warmup 1 --no-cpu-baseline", flush=True)
    r = _run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline", timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(d[key], typ), key
    assert d["metric"] == bench.METRIC and d["unit"] == "tokens/s"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["config"]["workload"] == bench.DEFAULT_WORKLOAD
    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert abs(d["value"] - w.tokens / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == bench.PEAK_TFLOPS
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # achieved is the rate of one launch, timed on its own (no inter-launch gaps)
    assert 0 < rf["launch_us"] <= 1.25e3 * d["ms_per_step"]  # a sanity bound: 3 launches, a cold box
    assert abs(rf["achieved"] - w.flops() / (rf["launch_us"] * 1e-6) / 1e12) <= 1e-6 * rf["achieved"]
    assert rf["traffic"] is None or rf["traffic"] > 0
    # measured denominators beside the vendor peak: the matrix-core rate the
    # chip holds and its shader clock
    assert 200 < rf["measured_mfma_peak_tflops"] < 1.2 * bench.PEAK_TFLOPS
    assert 0.3 < rf["shader_clock_ghz"] < 3.0
    assert len(rf["samples_us"]) == 3 and rf["samples_us"] == sorted(rf["samples_us"])
    assert d["cpu_baseline"] is None  # --no-cpu-baseline
