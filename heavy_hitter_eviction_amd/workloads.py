"""Workload shapes for the scored decode step (sizes only, no arithmetic).

Each workload is one decode configuration: batch, head layout, head dim,
scored layers, KV dtype, cache mode, context, decode steps and the selection
parameters. The shapes follow the model sizes named on the pages:

* the 35B shape of Context Optimization ("FP8 KV Cache / Memory Savings"):
  10 full-attention layers, 4 KV heads, head dim 128;
* the 397B shape of the same table: 15 layers, 8 KV heads, head dim 128;
* the 128K document-QA example of Per-Head Attention as a Scoring Signal
  ("Example: 128K Context Document QA"): anchor at positions 0-100, a key fact
  near 64K, recent tokens at the end.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

BLOCK_TOKENS = 16


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    kv_dtype: str          # "f32" | "bf16" | "fp8"
    q_dtype: str           # "f32" | "bf16"
    context: int           # positions written before the first decode step
    steps: int             # decode steps (one new position per sequence each)
    capacity: int          # slots per sequence
    window: int = 0        # 0 = unlimited; >0 masks by absolute position
    ring: bool = False     # slots reused as position mod capacity
    budget_blocks: int = 0
    recent_tokens: int = 1
    sink_tokens: int = 0
    alpha: float = 0.5
    traj_cap: int = 64
    select: bool = True
    planted: bool = False

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks_max(self) -> int:
        if self.ring:
            total = self.context + self.steps
            return (total + BLOCK_TOKENS - 1) // BLOCK_TOKENS
        return self.capacity // BLOCK_TOKENS

    def keys_at_step(self, t: int) -> int:
        """Keys read by every sequence at decode step ``t`` (0-based)."""
        i = self.context + t
        n = i + 1
        if self.window:
            n = min(n, self.window)
        return n

    def kv_bytes_per_key(self) -> int:
        """Algorithmic bytes read per (sequence, layer, key): K and V codes of
        every KV head, plus the two FP8 scales when the cache is FP8."""
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        b = 2 * self.n_kv_heads * self.head_dim * elem
        if self.kv_dtype == "fp8":
            b += 2 * 4
        return b

    def kv_bytes_at_step(self, t: int) -> int:
        return self.batch * self.n_layers * self.keys_at_step(t) * self.kv_bytes_per_key()

    def blocks_at_step(self, t: int) -> int:
        """(sequence, layer, block) units scored at step ``t``."""
        i = self.context + t
        lo = 0 if not self.window else max(0, i - self.window + 1)
        nb = i // BLOCK_TOKENS - lo // BLOCK_TOKENS + 1
        return self.batch * self.n_layers * nb

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


def _cap(n: int) -> int:
    return (n + BLOCK_TOKENS - 1) // BLOCK_TOKENS * BLOCK_TOKENS


TINY = Workload(
    name="tiny: 1 seq, 1 layer, 4q/2kv heads, d16, fp32, 64 cached tokens, 8 steps",
    batch=1, n_q_heads=4, n_kv_heads=2, head_dim=16, n_layers=1,
    kv_dtype="f32", q_dtype="f32", context=64, steps=8, capacity=_cap(64 + 8),
    budget_blocks=2, recent_tokens=16, alpha=0.5)

QWEN35B_BF16 = Workload(
    name="35B-like full-attn layers: batch 8, 16q/4kv, d128, 10 layers, bf16, 4096 context",
    batch=8, n_q_heads=16, n_kv_heads=4, head_dim=128, n_layers=10,
    kv_dtype="bf16", q_dtype="bf16", context=4096, steps=64, capacity=_cap(4096 + 64),
    budget_blocks=128, recent_tokens=256)

QWEN35B_FP8_RING = Workload(
    name="35B-like, FP8 KV, circular window 4096 over 32768 decode positions",
    batch=8, n_q_heads=16, n_kv_heads=4, head_dim=128, n_layers=10,
    kv_dtype="fp8", q_dtype="bf16", context=0, steps=32768, capacity=4096,
    window=4096, ring=True, select=False)

QWEN397B_FP8 = Workload(
    name="397B-like: batch 16, 32q/8kv, d128, 15 layers, FP8 KV, 32768 context",
    batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=15,
    kv_dtype="fp8", q_dtype="bf16", context=32768, steps=128, capacity=_cap(32768 + 128),
    budget_blocks=512, recent_tokens=1024)

DOCQA_128K = Workload(
    name="128K planted document-QA: 4 seqs, 32q/8kv, d128, 1 layer, bf16, 131072 context",
    batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=1,
    kv_dtype="bf16", q_dtype="bf16", context=131072, steps=64, capacity=_cap(131072 + 64),
    budget_blocks=1024, recent_tokens=1000, planted=True)

ALL = {
    "tiny": TINY,
    "35b_bf16": QWEN35B_BF16,
    "35b_fp8_ring": QWEN35B_FP8_RING,
    "397b_fp8": QWEN397B_FP8,
    "docqa_128k": DOCQA_128K,
}

# Planted structure of the 128K example (positions of the prefilled context).
PLANT_ANCHOR = range(0, 101)
PLANT_NEEDLE = range(65536, 65552)          # block 4096
PLANT_RECENT = range(131072 - 100, 131072)
