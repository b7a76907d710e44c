"""Seeded synthetic inputs for fused RoPE causal prefill attention.

This module only draws random tensors and names workloads.  It holds none of
the attention arithmetic, so both the CPU oracle's tests and the GPU path's
tests and bench can take their inputs from it without sharing any of the
method.

Recipe (every workload):

* ``torch.Generator('cpu').manual_seed(seed)``;
* draw order Q ``randn[B,S,Hq,D]``, K ``randn[B,S,Hkv,D]``, V
  ``randn[B,S,Hkv,D]``, all fp32;
* the long-prompt workload then draws ``rand(3, Hq)`` and multiplies Q, K and
  V of head h by 0.5 + 1.5*u[0,h], 0.5 + 1.5*u[1,h], 0.5 + 1.5*u[2,h]
  ("independent" reading; the "shared" reading uses row 0 for all three);
* one cast to the workload's dtype (bf16 rounds to nearest even; the tiny
  workload stays fp32);
* the int16 workload draws Q and K as ``randint(-2048, 2048)`` int16 and V as
  ``randn`` cast to bf16;
* dtype "bf16q" draws like "bf16"; it names bf16 inputs that the library
  quantises to int16 per (token, head) row inside the kernel.

The workloads stand in for the prompts the pages time (a 512-token prompt on
a 7B model, a pp512 prefill batch on a small GQA model, a long prompt on a
Phi-3-mini-sized model); no dataset or trained weight is involved.
"""

import math
from dataclasses import dataclass, field, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload", "to_f64"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    dtype: str              # "f32" | "bf16" | "i16" | "bf16q"
    rope_theta: float
    seed: int
    head_scale: str = ""    # "" | "independent" | "shared"
    score_scale: float = 0.0  # 0 -> 1/sqrt(D) (float); explicit for int16
    max_seq: int = 0        # 0 -> seq_len
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self):
        return self.batch * self.seq_len

    def flops(self):
        """Causal attention FLOP: 2 matmuls x 2 FLOP/MAC over visible pairs."""
        S = self.seq_len
        return 4 * self.batch * self.n_heads * self.head_dim * S * (S + 1) // 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_s32_d64", 1, 1, 1, 32, 64, "f32", 1e4, 1001),
        Workload("mha_bf16_h32_s512_d128", 1, 32, 32, 512, 128, "bf16", 1e4, 1002),
        Workload("mha_bf16_h32_s4096_d96", 1, 32, 32, 4096, 96, "bf16", 1e4, 1003,
                 head_scale="independent"),
        Workload("gqa_bf16_b16_h16kv8_s512_d128", 16, 16, 8, 512, 128, "bf16", 1e6, 1004),
        Workload("i16_h32_s2048_d128", 1, 32, 32, 2048, 128, "i16", 1e4, 1005,
                 score_scale=2.0 ** -22 / math.sqrt(128)),
        Workload("q16_bf16_h32_s2048_d128", 1, 32, 32, 2048, 128, "bf16q", 1e4, 1006),
    ]
}


def workload(name, **overrides):
    """A named workload, optionally with fields replaced (for small cases)."""
    return replace(WORKLOADS[name], **overrides)


def make_inputs(w):
    """Draw (q, k, v) on the CPU for workload ``w`` following the recipe."""
    g = torch.Generator("cpu").manual_seed(int(w.seed))
    B, S, Hq, Hkv, D = w.batch, w.seq_len, w.n_heads, w.n_kv_heads, w.head_dim
    if w.dtype == "i16":
        q = torch.randint(-2048, 2048, (B, S, Hq, D), generator=g, dtype=torch.int16)
        k = torch.randint(-2048, 2048, (B, S, Hkv, D), generator=g, dtype=torch.int16)
        v = torch.randn((B, S, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
        return q, k, v
    q = torch.randn((B, S, Hq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, S, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, S, Hkv, D), generator=g, dtype=torch.float32)
    if w.head_scale:
        u = torch.rand((3, Hq), generator=g, dtype=torch.float32)
        sc = 0.5 + 1.5 * u
        if w.head_scale == "shared":
            sc = sc[0:1].expand(3, Hq)
        q = q * sc[0].view(1, 1, Hq, 1)
        k = k * sc[1, :Hkv].view(1, 1, Hkv, 1)
        v = v * sc[2, :Hkv].view(1, 1, Hkv, 1)
    if w.dtype in ("bf16", "bf16q"):
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype}")
    return q.contiguous(), k.contiguous(), v.contiguous()


def to_f64(t):
    """Exact conversion of a CPU tensor (f32/bf16/int16) to a float64 array."""
    if t.dtype in (torch.int16, torch.int32, torch.int64):
        return t.to(torch.int64).numpy()
    return t.to(torch.float64).numpy()
