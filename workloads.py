"""Seeded synthetic workloads for the fused RMSNorm -> QKV projection -> RoPE path.

This module only draws random numbers and arranges them into the shapes of the
workloads; it holds none of the method's arithmetic (no norm, no projection, no
rotation).  Both sides of every parity check -- the HIP path and the CPU oracle --
take their inputs from here, so they see bit-identical tensors.

Shapes follow the models the pages measure on (Llama-7B, Llama-3-8B, Qwen-7B
prefill and a batched single-token decode step); the value distributions are
those of a freshly initialised transformer layer:

  x       ~ N(0, 1)              activations entering the layer
  W_qkv   ~ N(0, 0.02)           [H, N] row-major, columns [Q heads | K heads | V heads]
  w_norm  = 1 + N(0, 0.1)        learned RMSNorm weight
  bias    ~ N(0, 0.02)           QKV bias (Qwen-style configuration only)
  pos     = t mod seq_len        per-sequence position reset (prefill)
          ~ U[0, 32768)          independent decode positions

Each tensor is drawn in fp32 from its own torch CPU generator seeded with
``1000 * config_id + k`` (k = 1 x, 2 W, 3 w_norm, 4 bias, 5 pos), then rounded to
the configuration's dtype with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    batch: int
    seq: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    has_bias: bool
    rope_theta: float
    eps: float
    dtype: str            # "fp32" or "bf16"
    pos_kind: str         # "per_seq" or "uniform32768"

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def n_q(self) -> int:
        return self.num_q_heads * self.head_dim

    @property
    def n_kv(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def n_total(self) -> int:
        return self.n_q + 2 * self.n_kv

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def with_tokens(self, batch: int, seq: int, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, batch=batch, seq=seq, name=name or f"{self.name}@{batch}x{seq}")

    def flops(self, T: Optional[int] = None) -> int:
        """Dense contraction flops of one forward (2*T*H*N)."""
        T = self.tokens if T is None else T
        return 2 * T * self.hidden * self.n_total

    def algorithmic_bytes(self, T: Optional[int] = None) -> int:
        """One read of every input plus one write of Q, K and V."""
        T = self.tokens if T is None else T
        e = 4 if self.dtype == "fp32" else 2
        H, N = self.hidden, self.n_total
        b = T * H * e + H * e + H * N * e + T * 4 + T * N * e
        if self.has_bias:
            b += N * e
        return b


WORKLOADS = {
    1: Workload(1, "tiny_fp32", 1, 16, 64, 4, 4, 16, False, 1.0e4, 1e-6, "fp32", "per_seq"),
    2: Workload(2, "llama7b_prefill", 4, 2048, 4096, 32, 32, 128, False, 1.0e4, 1e-6, "bf16", "per_seq"),
    3: Workload(3, "llama3_8b_gqa_prefill", 1, 8192, 4096, 32, 8, 128, False, 5.0e5, 1e-5, "bf16", "per_seq"),
    4: Workload(4, "gqa_decode", 64, 1, 4096, 32, 8, 128, False, 5.0e5, 1e-6, "bf16", "uniform32768"),
    5: Workload(5, "qwen7b_prefill_bias", 2, 8192, 4096, 32, 32, 128, True, 1.0e4, 1e-6, "bf16", "per_seq"),
}
BY_NAME = {w.name: w for w in WORKLOADS.values()}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def positions(wl: Workload, seed: int) -> torch.Tensor:
    if wl.pos_kind == "uniform32768":
        return torch.randint(0, 32768, (wl.tokens,), generator=_gen(seed), dtype=torch.int64).to(torch.int32)
    return (torch.arange(wl.tokens, dtype=torch.int64) % wl.seq).to(torch.int32)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """Host (CPU) tensors for one forward of ``wl``; dtype is the workload's."""
    base = 1000 * wl.cid if seed is None else seed
    T, H, N = wl.tokens, wl.hidden, wl.n_total
    dt = wl.torch_dtype
    x = torch.randn(T, H, generator=_gen(base + 1), dtype=torch.float32).to(dt)
    w_qkv = (torch.randn(H, N, generator=_gen(base + 2), dtype=torch.float32) * 0.02).to(dt)
    w_norm = (1.0 + 0.1 * torch.randn(H, generator=_gen(base + 3), dtype=torch.float32)).to(dt)
    bias = None
    if wl.has_bias:
        bias = (torch.randn(N, generator=_gen(base + 4), dtype=torch.float32) * 0.02).to(dt)
    pos = positions(wl, base + 5)
    return {"x": x, "w_norm": w_norm, "w_qkv": w_qkv, "bias": bias, "pos": pos}


def digest(t: Optional[torch.Tensor]) -> str:
    if t is None:
        return "-"
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """Gated-MLP input of one Llama-style layer: RMSNorm, then [H, 2I] gate|up weights."""
    name: str
    batch: int
    seq: int
    hidden: int
    intermediate: int
    eps: float

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def flops(self, T: Optional[int] = None) -> int:
        """Dense contraction flops of one forward (2*T*H*2I)."""
        T = self.tokens if T is None else T
        return 2 * T * self.hidden * 2 * self.intermediate

    def algorithmic_bytes(self, T: Optional[int] = None) -> int:
        """One read of x, w_norm and the gate|up weights, one write of the output (bf16)."""
        T = self.tokens if T is None else T
        H, inter = self.hidden, self.intermediate
        return 2 * (T * H + H + H * 2 * inter + T * inter)


# Llama-7B MLP shape at the page's "seq_len 2k, hidden 4096" SwiGLU comparison, batch 4
MLP_WORKLOADS = {
    "llama7b_mlp": MlpWorkload("llama7b_mlp", 4, 2048, 4096, 11008, 1e-6),
}


def make_mlp_inputs(wl: MlpWorkload, seed: int = 6000) -> dict:
    """Host bf16 tensors: x ~ N(0,1), w_norm ~ 1 + N(0, 0.1), W_gate_up ~ N(0, 0.02)."""
    T, H, inter = wl.tokens, wl.hidden, wl.intermediate
    x = torch.randn(T, H, generator=_gen(seed + 1), dtype=torch.float32).to(torch.bfloat16)
    w_gate_up = (torch.randn(H, 2 * inter, generator=_gen(seed + 2), dtype=torch.float32) * 0.02).to(torch.bfloat16)
    w_norm = (1.0 + 0.1 * torch.randn(H, generator=_gen(seed + 3), dtype=torch.float32)).to(torch.bfloat16)
    return {"x": x, "w_norm": w_norm, "w_gate_up": w_gate_up}


def make_grads(wl: Workload, seed: Optional[int] = None) -> dict:
    """Host tensors of upstream gradients for Q, K, V (N(0,1), the workload's dtype)."""
    base = 1000 * wl.cid + 500 if seed is None else seed
    T, dt = wl.tokens, wl.torch_dtype
    return {
        "dq": torch.randn(T, wl.n_q, generator=_gen(base + 1), dtype=torch.float32).to(dt),
        "dk": torch.randn(T, wl.n_kv, generator=_gen(base + 2), dtype=torch.float32).to(dt),
        "dv": torch.randn(T, wl.n_kv, generator=_gen(base + 3), dtype=torch.float32).to(dt),
    }
