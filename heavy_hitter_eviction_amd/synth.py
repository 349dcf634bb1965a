"""Seeded synthetic inputs for the decode workloads.

This module only draws numbers: it holds none of the attention, scoring,
encoding or selection arithmetic, so both the GPU path and the float64
checker can take their inputs from it.

Every chunk of input is named by a key ``(seed, workload tag, tensor, layer,
sequence or step chunk)``. On the CPU the key seeds numpy's PCG64 through a
SeedSequence; on a GPU it seeds torch's device generator with a 63-bit value
derived from the same SeedSequence. The two streams differ, so a test draws a
chunk once and hands the same tensor to both sides; to see a chunk again the
caller re-draws it from its key on the same device kind.

Values are float32 N(0, 1); bf16 inputs are the round-to-nearest-even cast of
those draws. The 128K document-QA workload adds planted structure: per
(sequence, KV head) a random unit direction ``u``; queries are ``z + g*u`` and
the keys at the anchor, needle and recent positions are ``z + g*u`` with
``g = sqrt(3*sqrt(d))``, so those keys score about 3 logit units (about 3
sigma) above the rest, mirroring the anchor, retrieval and recency heads of
the 128K example in Per-Head Attention as a Scoring Signal.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from .workloads import PLANT_ANCHOR, PLANT_NEEDLE, PLANT_RECENT, Workload

T_Q, T_K, T_V, T_U = 0, 1, 2, 3
STEP_CHUNK = 256


def _tag(w: Workload) -> int:
    return sum((i + 1) * ord(c) for i, c in enumerate(w.name)) % 1_000_003


def seed64(key) -> int:
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def normal(shape, key, device="cpu") -> torch.Tensor:
    """float32 N(0, 1) draws for one named chunk."""
    device = torch.device(device)
    if device.type == "cpu":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    g = torch.Generator(device=device)
    g.manual_seed(seed64(key))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def plant_gain(d: int) -> float:
    return math.sqrt(3.0 * math.sqrt(d))


def _directions(w: Workload, seed: int, device) -> torch.Tensor:
    u = normal((w.batch, w.n_kv_heads, w.head_dim), (seed, _tag(w), T_U), device)
    return u / u.norm(dim=-1, keepdim=True)


def prefill_rows(w: Workload, seed: int, layer: int, seq: int, tensor: int, device="cpu",
                 lo: int = 0, hi: int | None = None) -> torch.Tensor:
    """K or V rows of the prefilled context of one (layer, sequence):
    ``[hi-lo, Hkv*d]`` float32 for positions ``lo..hi-1``."""
    hi = w.context if hi is None else hi
    rows = normal((w.context, w.n_kv_heads * w.head_dim), (seed, _tag(w), tensor, layer, seq, 0), device)
    rows = rows[lo:hi]
    if w.planted and tensor == T_K:
        u = _directions(w, seed, device)[seq].reshape(-1) * plant_gain(w.head_dim)
        planted = torch.zeros(w.context, dtype=torch.bool, device=rows.device)
        for r in (PLANT_ANCHOR, PLANT_NEEDLE, PLANT_RECENT):
            planted[r.start:r.stop] = True
        rows = rows + planted[lo:hi, None].to(rows.dtype) * u[None, :]
    return rows.contiguous()


def step_block(w: Workload, seed: int, layer: int, chunk: int, tensor: int, device="cpu") -> torch.Tensor:
    """Per-step rows for the decode steps ``chunk*256 .. chunk*256+255`` (fewer
    in the last chunk): ``[n, B, Hq*d]`` queries for ``T_Q``, or the new
    positions' K or V ``[n, B, Hkv*d]`` for ``T_K`` / ``T_V``."""
    width = (w.n_q_heads if tensor == T_Q else w.n_kv_heads) * w.head_dim
    n = min(STEP_CHUNK, w.steps - chunk * STEP_CHUNK)
    block = normal((n, w.batch, width), (seed, _tag(w), tensor, layer, 1 << 20 | chunk), device)
    if w.planted and tensor == T_Q:
        u = _directions(w, seed, device) * plant_gain(w.head_dim)
        block = block + u.repeat_interleave(w.group, dim=1).reshape(1, w.batch, -1)
    return block.contiguous()


def new_query(w: Workload, seed: int, layer: int, device="cpu") -> torch.Tensor:
    """A query ``[B, Hq*d]`` from a stream no decode step draws: the "new
    question" of a re-attend over stored spans."""
    q = normal((w.batch, w.n_q_heads * w.head_dim), (seed, _tag(w), T_Q, layer, 2 << 20), device)
    if w.planted:
        u = _directions(w, seed, device) * plant_gain(w.head_dim)
        q = q + u.repeat_interleave(w.group, dim=1).reshape(w.batch, -1)
    return q.contiguous()


def step_rows(w: Workload, seed: int, layer: int, step: int, tensor: int, device="cpu") -> torch.Tensor:
    """The rows of one decode step (see ``step_block``)."""
    chunk = step // STEP_CHUNK
    return step_block(w, seed, layer, chunk, tensor, device)[step - chunk * STEP_CHUNK].contiguous()


def as_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return {"f32": x.float(), "bf16": x.to(torch.bfloat16)}[dtype]
