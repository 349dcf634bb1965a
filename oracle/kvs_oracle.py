"""Float64 CPU oracle for scored decode attention, its block side-car and
heavy-hitter block selection.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The HIP library never calls it, and it imports
nothing from the HIP package (inputs are handed in as numpy arrays).

Everything is computed in float64 with plain numpy, one definition per step,
in the order the source pages state them:

* Context Optimization (Flash-MoE docs), "FP8 KV Cache / How It Works":
  E4M3 with 1 sign, 4 exponent and 3 mantissa bits, bias 7, range +-448; a
  per-position scale ``absmax / 240``; every value divided by it, clipped and
  rounded to an 8-bit code; the scale stored beside the codes.
* Context Optimization, "Sliding Window Attention / Design": the write slot of
  a circular cache is ``position mod capacity``.
* LLM mechanics III (four-slot cache), sections 1, 3 and 5: position ``i``
  reads ``i-w+1 .. i`` clipped at 0, the current token included; masking is by
  absolute position, never by slot; processed count, absolute positions and
  slots are three separate indices.
* Context views at marginal cost, section 2 (Tier 0 and Tier 1): the
  post-softmax weights are summed per span as the pass makes them, a single
  addition for each weight; the side-car keeps Attended (this turn), EMA,
  Cumulative and a 64-turn trajectory ring, a constant amount of work per span
  and turn.
* Per-Head Attention as a Scoring Signal, "Scoring granularity, not eviction
  granularity": the unit that is scored and kept is a (sequence, 16-token
  block); heads are only a scoring input. "Fix: score per head, place per
  block": a block is kept while at least one head gives it weight (the max
  over heads of the per-head masses).
* Context views at marginal cost, section 4: the observer's layer and head
  axes may be kept as a reduced per-span profile instead of being summed.
* Context views at marginal cost, "Tier 2 — RE-ATTEND" and "Fact 3": a new
  query is run against the cached keys of a chosen subset of spans, and the
  resulting distribution is read; cached keys and values are reused as they
  are.
* Context views at marginal cost, section 7, SOTA grounding, per-system
  reductions: SnapKV adds up, per head, the weights the last N prompt queries
  give each prompt token, then replaces each token's score by the maximum
  over its 7-token neighbourhood; Scissorhands counts the turns a token's
  attention passes a threshold; TOVA evicts the block the latest query
  weights least.
* Context Optimization, "H2O KV Cache Eviction": post-softmax scores are summed
  over all query heads (GQA-aware) and over steps; sinks and recent tokens are
  kept unconditionally and the top scorers among the rest survive.

Readings taken where the pages are silent (each is listed, with its reason, in
the design notes of the repository): softmax scale ``f32(1/sqrt(d))``; query
head ``h`` reads KV head ``h // (Hq/Hkv)``; masses are summed over heads and
over scored layers; a block is ``position // 16``; ``EMA <- a*A + (1-a)*EMA``
from zero; selection keys are (score descending, block index ascending); the
recent region is every block that meets the last ``R`` tokens; blocks not yet
written are never marked evicted.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against facts the pages or mathematics fix (format tables, closed forms,
brute force, an independent float64 attention, and the pages' printed sizes).
Nothing in this file is "parity unpinned".
"""

from __future__ import annotations

import itertools
import math

import numpy as np

# Per-Head Attention as a Scoring Signal: the placed unit is a 16-token block of one sequence.
BLOCK_TOKENS = 16
# Context views at marginal cost, section 2 Tier 1: the trajectory ring holds 64 turns.
TRAJ_CAP = 64
# Context Optimization, FP8 KV Cache: bias 7, range [-448, 448], scale absmax/240.
E4M3_BIAS = 7
E4M3_MAX = 448.0
FP8_SCALE_DIVISOR = 240.0


# ---------------------------------------------------------------------------
# FP8 E4M3 (Context Optimization, "FP8 KV Cache / How It Works")
# ---------------------------------------------------------------------------

def e4m3_to_float(code: int) -> float:
    """Value of one E4M3 byte from the format definition: the top bit is the
    sign, the next four the exponent (bias 7), the low three the mantissa. Exponent field 0 holds the
    subnormals ``(m/8) * 2**(1-7)``; otherwise ``(1 + m/8) * 2**(e-7)``. The
    pair exponent 15 / mantissa 7 is NaN (the range stops at 448, so there is no
    infinity)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


def e4m3_table() -> np.ndarray:
    """All 256 decoded values (float64), NaN at 0x7F and 0xFF."""
    return np.array([e4m3_to_float(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round values to the nearest E4M3 code, ties to even, after clipping to
    +-448 (the pages clip before quantising). The sign is kept, so -0 gives
    0x80. Inputs must be finite.

    Step by step: clip |y| to 448; the non-negative finite values of the
    format (codes 0x00 .. 0x7E, ascending) and the midpoints between
    neighbours are taken from the format definition (``e4m3_table``); the
    number of midpoints strictly below |y| is the code of the nearest value,
    unless |y| sits exactly on a midpoint, where the tie goes to the even one
    of the two codes; the sign bit is then set for negative inputs."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    sign = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    values = e4m3_table()[:0x7F]                              # 0, subnormals, normals .. 448
    mids = np.append((values[:-1] + values[1:]) / 2, np.inf)  # exact in float64
    code = np.searchsorted(mids, a, side="left")               # midpoints strictly below |y|
    code = code + ((a == mids[code]) & (code % 2 == 1))        # a tie goes to the even code
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def fp8_encode_rows(x: np.ndarray):
    """Encode each row (one position's ``Hkv*d`` values of K or of V) with its
    own scale: ``absmax = max|x|``, ``s = f32(absmax / 240)``,
    ``code = E4M3(f32(x / s))``. A row of zeros gets ``s = 0`` and codes 0x00.

    Division is done in float64 and rounded once to float32, which equals a
    correctly rounded float32 division (53 >= 2*24 + 2). Returns
    ``(codes uint8 [rows, n], scales float32 [rows])``."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("fp8_encode_rows takes float32 rows (bf16 sources are widened exactly first)")
    x2 = np.atleast_2d(x)
    if not np.all(np.isfinite(x2)):
        raise ValueError("FP8 encode: non-finite input is outside the contract")
    codes = np.zeros(x2.shape, dtype=np.uint8)
    scales = np.zeros(x2.shape[0], dtype=np.float32)
    for r0 in range(0, x2.shape[0], 64):       # every row on its own; 64 at a time
        xr = x2[r0:r0 + 64].astype(np.float64)
        absmax = np.max(np.abs(xr), axis=1)
        s = (absmax / FP8_SCALE_DIVISOR).astype(np.float32)
        scales[r0:r0 + 64] = s
        nz = s > 0
        if np.any(nz):
            y = (xr[nz] / s[nz, None].astype(np.float64)).astype(np.float32)
            codes[r0:r0 + 64][nz] = e4m3_encode(y.astype(np.float64))
    return codes.reshape(x.shape), scales


def fp8_decode_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """``value = E4M3(code) * scale`` in float64 (exact: a 4-bit significand
    times a float32)."""
    table = e4m3_table()
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return table[codes] * scales.reshape(scales.shape + (1,) * (codes.ndim - scales.ndim))


# ---------------------------------------------------------------------------
# Which keys a query reads (LLM mechanics III, sections 1, 3, 5)
# ---------------------------------------------------------------------------

def ring_slot(position: int, capacity: int) -> int:
    """Context Optimization, Sliding Window Attention: ``cache_pos = len % window_size``."""
    return position % capacity


def key_visible(p: int, i: int, window: int) -> bool:
    """Absolute position ``p`` is visible to the query at absolute position ``i``
    when ``p <= i`` and, for a window ``w >= 1``, ``p >= i - w + 1`` (clipped at
    0 by ``p >= 0``). ``w == 0`` means unlimited."""
    if window < 0:
        raise ValueError("invalid window")
    if p < 0 or p > i:
        return False
    return window == 0 or p >= i - window + 1


def visible_mask(positions, i: int, window: int, alive=None) -> np.ndarray:
    """``key_visible(p, i, window)`` and ``block_alive(alive, p // 16)`` for
    every entry of ``positions`` at once (boolean array of the same shape)."""
    if window < 0:
        raise ValueError("invalid window")
    p = np.asarray(positions, dtype=np.int64)
    vis = (p >= 0) & (p <= i)
    if window:
        vis &= p >= i - window + 1
    if alive is not None:
        alive = np.asarray(alive, dtype=bool)
        vis &= alive[np.clip(p // BLOCK_TOKENS, 0, len(alive) - 1)]
    return vis


def block_of(position: int) -> int:
    """Per-Head Attention as a Scoring Signal: the unit is a 16-token block."""
    return position // BLOCK_TOKENS


def block_alive(alive, b: int) -> bool:
    return True if alive is None else bool(alive[b])


# ---------------------------------------------------------------------------
# Attention with the post-softmax tap
# ---------------------------------------------------------------------------

def softmax_scale(d: int) -> float:
    """Reading: the pages do not state the logit scale; the usual ``1/sqrt(d)``
    is used, rounded once to float32 (the GPU receives the same float32)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Explicit softmax attention for one decode query of one sequence.

    ``q`` is ``[Hq, d]``; ``K`` and ``V`` are ``[Hkv, n, d]`` holding only the
    visible keys. Query head ``h`` reads KV head ``h // (Hq // Hkv)``.
    Returns ``(o [Hq, d], p [Hq, n])`` where ``p`` are the post-softmax weights
    that the tap reduces."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    Hkv, n, _ = K.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if n == 0:
        raise ValueError("all-masked row: the query sees no key")
    G = Hq // Hkv
    o = np.zeros((Hq, d))
    p = np.zeros((Hq, n))
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)        # the query heads that read KV head g
        s = (q[hs] @ K[g].T) * scale          # their logits, [G, n]
        e = np.exp(s - np.max(s, axis=1, keepdims=True))
        p[hs] = e / np.sum(e, axis=1, keepdims=True)
        o[hs] = p[hs] @ V[g]
    return o, p


def block_mass(p: np.ndarray, positions: np.ndarray, n_blocks: int) -> np.ndarray:
    """Tier 0 reduction: for every block ``b``, the sum over heads and over the
    block's visible keys of the post-softmax weight.
    ``positions`` are the absolute positions of the columns of ``p``."""
    p = np.asarray(p, dtype=np.float64)
    blocks = np.asarray(positions, dtype=np.int64) // BLOCK_TOKENS
    if blocks.size and (blocks.min() < 0 or blocks.max() >= n_blocks):
        raise ValueError("block index out of range")
    mass = np.zeros(n_blocks)
    for h in range(p.shape[0]):
        mass += np.bincount(blocks, weights=p[h], minlength=n_blocks)
    return mass


def block_mass_per_head(p: np.ndarray, positions: np.ndarray, n_blocks: int) -> np.ndarray:
    """The per-head profile (Context views at marginal cost, section 4, "within
    head H"): ``[Hq, n_blocks]``, row ``h`` is head h's post-softmax weight
    summed over each block's visible keys, before any sum over heads."""
    p = np.asarray(p, dtype=np.float64)
    blocks = np.asarray(positions, dtype=np.int64) // BLOCK_TOKENS
    if blocks.size and (blocks.min() < 0 or blocks.max() >= n_blocks):
        raise ValueError("block index out of range")
    return np.stack([np.bincount(blocks, weights=p[h], minlength=n_blocks) for h in range(p.shape[0])])


def max_over_heads(head_mass: np.ndarray) -> np.ndarray:
    """Per-Head Attention as a Scoring Signal, "Fix: score per head, place per
    block": a block is kept while at least one head gives it weight, so the
    block's score is the largest of its per-head masses."""
    return np.max(np.asarray(head_mass, dtype=np.float64), axis=0)


def attend_profiled(q, K_all, V_all, positions, i, window, alive, scale, n_blocks):
    """attend_scored plus the per-head profile and its max over heads:
    ``(o, mass, head_mass [Hq, n_blocks], mass_max [n_blocks])``."""
    positions = np.asarray(positions, dtype=np.int64)
    sel = visible_mask(positions, i, window, alive)
    o, p = attend(q, np.asarray(K_all)[:, sel], np.asarray(V_all)[:, sel], scale)
    hm = block_mass_per_head(p, positions[sel], n_blocks)
    return o, block_mass(p, positions[sel], n_blocks), hm, max_over_heads(hm)


def attend_scored(q, K_all, V_all, positions, i, window, alive, scale, n_blocks):
    """One (sequence, layer) of the scored decode step.

    ``K_all`` / ``V_all`` are ``[Hkv, n, d]`` for candidate keys at absolute
    ``positions`` (any order: a linear cache or the slots of a ring). A key is
    read when it is visible (window rule) and its block is alive. Returns
    ``(o [Hq, d], mass [n_blocks])`` with the mass summed over query heads."""
    positions = np.asarray(positions, dtype=np.int64)
    sel = visible_mask(positions, i, window, alive)
    o, p = attend(q, np.asarray(K_all)[:, sel], np.asarray(V_all)[:, sel], scale)
    return o, block_mass(p, positions[sel], n_blocks)


def reattend_blocks(q, K_all, V_all, positions, i, block_ids, scale, n_blocks):
    """Tier 2 re-attend (Context views at marginal cost, "Tier 2 — RE-ATTEND",
    "Fact 3"): attention of the query ``q`` over only the cached keys whose
    block is among ``block_ids`` (a set: order and repeats do not matter) and
    whose position is at most ``i``. Returns ``(o, mass)`` as attend_scored;
    the mass is the new query's distribution over the chosen spans, summed
    over query heads. With no such key the output and the mass are zero."""
    chosen = {int(b) for b in np.asarray(block_ids).ravel()}
    positions = np.asarray(positions, dtype=np.int64)
    sel = np.array([int(p) <= i and block_of(int(p)) in chosen for p in positions], dtype=bool)
    if not sel.any():
        return np.zeros(np.asarray(q).shape), np.zeros(n_blocks)
    o, p = attend(q, np.asarray(K_all)[:, sel], np.asarray(V_all)[:, sel], scale)
    return o, block_mass(p, positions[sel], n_blocks)


# ---------------------------------------------------------------------------
# Incremental ring cache versus the full masked reference (LLM mechanics III)
# ---------------------------------------------------------------------------

class RingCache:
    """A bounded per-sequence cache with three separate indices: the processed
    count ``next_position``, the absolute position held by each slot, and the
    slot itself. Writes go to ``position mod capacity``; masking uses the held
    absolute positions only."""

    def __init__(self, n_kv_heads: int, d: int, capacity: int):
        if capacity < 1:
            raise ValueError("capacity must be positive")
        self.capacity = capacity
        self.K = np.zeros((n_kv_heads, capacity, d))
        self.V = np.zeros((n_kv_heads, capacity, d))
        self.pos_of_slot = np.full(capacity, -1, dtype=np.int64)
        self.next_position = 0

    def append(self, k: np.ndarray, v: np.ndarray):
        """Append a chunk ``k, v [Hkv, n, d]`` at the next absolute positions."""
        n = k.shape[1]
        positions = np.arange(self.next_position, self.next_position + n)
        for j, pos in enumerate(positions):
            s = ring_slot(int(pos), self.capacity)
            self.K[:, s] = k[:, j]
            self.V[:, s] = v[:, j]
            self.pos_of_slot[s] = pos
        self.next_position += n          # eviction never resets the position
        return positions

    def attend(self, q, i, window, scale, n_blocks, alive=None, mask_by_slot=False):
        """Attend the query at absolute position ``i`` over the held slots.
        ``mask_by_slot=True`` is the deliberately wrong negative control that
        treats slot indices as positions."""
        held = self.pos_of_slot >= 0
        pos = np.where(held, self.pos_of_slot, -1)
        if mask_by_slot:
            pos = np.where(held, np.arange(self.capacity), -1)
        return attend_scored(q, self.K, self.V, pos, i, window, alive, scale, n_blocks)


def full_masked_reference(q, K_hist, V_hist, i, window, scale, n_blocks, alive=None):
    """The full reference: every position ``0..i`` of the history, with the
    window applied as a mask by absolute position."""
    n = i + 1
    return attend_scored(q, K_hist[:, :n], V_hist[:, :n], np.arange(n), i, window, alive,
                         scale, n_blocks)


# ---------------------------------------------------------------------------
# Side-car (Context views at marginal cost, section 2 Tier 1 and section 3)
# ---------------------------------------------------------------------------

class SideCar:
    """Per-block state ``{Attended, EMA, Cumulative, traj[64]}``, all zero at
    the start, updated once per turn (one decode step)."""

    def __init__(self, n_blocks: int, traj_cap: int = TRAJ_CAP):
        self.attended = np.zeros(n_blocks)
        self.ema = np.zeros(n_blocks)
        self.cum = np.zeros(n_blocks)
        self.traj = np.zeros((traj_cap, n_blocks))
        self.step = 0

    def update(self, A: np.ndarray, alpha: float):
        """Close the turn with this turn's mass ``A``: Attended = A;
        EMA = alpha*A + (1-alpha)*EMA; Cumulative += A; the trajectory ring
        slot ``step mod trajCap`` receives A; the turn counter advances."""
        A = np.asarray(A, dtype=np.float64)
        self.attended = A.copy()
        self.ema = alpha * A + (1.0 - alpha) * self.ema
        self.cum = self.cum + A
        self.traj[self.step % self.traj.shape[0]] = A
        self.step += 1


# ---------------------------------------------------------------------------
# Threshold views and counters (Context views at marginal cost, section 3)
# ---------------------------------------------------------------------------

def hot_count_update(count: np.ndarray, attended: np.ndarray, theta: float) -> np.ndarray:
    """Scissorhands (section 7, SOTA grounding, per-system reductions): per
    span, the number of turns whose attention exceeded the threshold; one
    increment per turn above it."""
    return np.asarray(count) + (np.asarray(attended) > theta).astype(np.asarray(count).dtype)


def cold_gc_update(cold_turns: np.ndarray, ema: np.ndarray, traj: np.ndarray, theta: float, limit: int):
    """The threshold as a storage GC policy (section 3, "Pure side-car vs.
    materialized"): count the consecutive turns a span's EMA has stayed below
    theta; once that reaches ``limit`` (> 0) the span drops its fine-grained
    trajectory (its ring column is cleared) and keeps only the cumulative
    scalar. Returns the new counts and trajectory."""
    ema = np.asarray(ema)
    cold = np.where(ema < theta, np.asarray(cold_turns) + 1, 0)
    traj = np.array(traj, copy=True)
    if limit > 0:
        traj[:, cold >= limit] = 0.0
    return cold, traj


def filter_blocks(score: np.ndarray, alive, i: int, theta: float) -> np.ndarray:
    """A threshold view (section 3: filter(a_s > theta), computed at query
    time): the ascending ids of the blocks that exist at position ``i``, are
    alive, and score strictly above theta."""
    n_exist = i // BLOCK_TOKENS + 1
    return np.array([b for b in range(min(n_exist, len(score)))
                     if block_alive(alive, b) and score[b] > theta], dtype=np.int64)


# ---------------------------------------------------------------------------
# Heavy-hitter block selection (Context Optimization, "H2O KV Cache Eviction")
# ---------------------------------------------------------------------------

def protected_blocks(i: int, recent_tokens: int, sink_tokens: int):
    """Blocks kept unconditionally: every block meeting the last
    ``recent_tokens`` positions ``[max(0, i-R+1), i]``, and every block meeting
    the first ``sink_tokens`` positions."""
    if recent_tokens < 1:
        raise ValueError("recent_tokens must be at least 1 (the current token)")
    if sink_tokens < 0:
        raise ValueError("sink_tokens must be non-negative")
    lo = max(0, i - recent_tokens + 1) // BLOCK_TOKENS
    prot = set(range(lo, i // BLOCK_TOKENS + 1))
    if sink_tokens > 0:
        prot |= set(range(0, (min(sink_tokens, i + 1) - 1) // BLOCK_TOKENS + 1))
    return prot


def select_blocks(score, alive, i, budget_blocks, recent_tokens, sink_tokens=0):
    """Keep = protected blocks, plus the ``budget_blocks`` highest-scoring
    alive candidates among the other existing blocks ``b <= i // 16``, ordered
    by score descending and then by block index ascending (lowest index wins a
    tie). Returns the kept block ids in ascending order."""
    if budget_blocks < 0:
        raise ValueError("budget must be non-negative")
    score = np.asarray(score)
    n_exist = i // BLOCK_TOKENS + 1
    prot = protected_blocks(i, recent_tokens, sink_tokens)
    cand = [b for b in range(n_exist) if block_alive(alive, b) and b not in prot]
    cand.sort(key=lambda b: (-float(score[b]), b))
    keep = prot | set(cand[:budget_blocks])
    return np.array(sorted(keep), dtype=np.int64)


def select_blocks_bruteforce(score, alive, i, budget_blocks, recent_tokens, sink_tokens=0):
    """Small-case check of ``select_blocks``: among all candidate subsets of the
    allowed size, take the one whose scores, sorted descending, are largest
    lexicographically, breaking equal score lists by the smallest sorted index
    list. Exponential; tiny inputs only."""
    score = np.asarray(score)
    n_exist = i // BLOCK_TOKENS + 1
    prot = protected_blocks(i, recent_tokens, sink_tokens)
    cand = [b for b in range(n_exist) if block_alive(alive, b) and b not in prot]
    k = min(budget_blocks, len(cand))
    best = None
    for sub in itertools.combinations(cand, k):
        key = (tuple(sorted((-float(score[b]) for b in sub))), tuple(sorted(sub)))
        if best is None or key < best[0]:
            best = (key, sub)
    return np.array(sorted(prot | set(best[1] if best else ())), dtype=np.int64)


def keep_mask_after(keep_ids, i, n_blocks):
    """Alive set for the next step in evict mode: the kept blocks, plus every
    block not yet written (``b > i // 16``), which cannot have been evicted."""
    alive = np.zeros(n_blocks, dtype=bool)
    alive[np.asarray(keep_ids, dtype=np.int64)] = True
    alive[i // BLOCK_TOKENS + 1:] = True
    return alive


# ---------------------------------------------------------------------------
# KV memory sizes (Context Optimization, "Memory Budget Calculator")
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# SnapKV-style prefill scoring (Context views at marginal cost, section 7,
# SOTA grounding, per-system reductions)
# ---------------------------------------------------------------------------

def snapkv_token_scores(q_window: np.ndarray, K: np.ndarray, n_prompt: int, scale: float) -> np.ndarray:
    """Once, when the prompt is done: each prompt token's score for head h is
    the sum of the weights the last W prompt queries (the observation window)
    give it, ``score[h][j] = sum_w p_{w,h,j}``. ``q_window`` is
    ``[W, Hq, d]``, query w at position ``n_prompt - W + w`` reading keys at or
    before it; ``K`` is ``[Hkv, >= n_prompt, d]``. Returns ``[Hq, n_prompt]``."""
    q_window = np.asarray(q_window, dtype=np.float64)
    W, Hq, _ = q_window.shape
    score = np.zeros((Hq, n_prompt))
    for w in range(W):
        pos = n_prompt - W + w
        if pos < 0:
            continue
        Kw = np.asarray(K)[:, :pos + 1]
        _, p = attend(q_window[w], Kw, Kw, scale)
        score[:, :pos + 1] += p
    return score


def max_pool_tokens(score: np.ndarray, kernel: int) -> np.ndarray:
    """SnapKV's max-pooling along tokens (kernel 7 on the page) so that a kept
    key drags its neighbours: ``out[h][j] = max score[h][j-R .. j+R]`` inside
    the prompt, R = (kernel - 1) / 2."""
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("the pooling kernel must be odd")
    score = np.asarray(score, dtype=np.float64)
    R = kernel // 2
    n = score.shape[1]
    return np.stack([[score[h, max(0, j - R):min(n, j + R + 1)].max() for j in range(n)]
                     for h in range(score.shape[0])]) if n else score.copy()


def snapkv_block_scores(pooled: np.ndarray, n_blocks: int) -> np.ndarray:
    """Placed per block (Per-Head Attention as a Scoring Signal): the pooled
    per-head token scores summed over heads and over each block's tokens."""
    pooled = np.asarray(pooled, dtype=np.float64)
    blocks = np.arange(pooled.shape[1]) // BLOCK_TOKENS
    return np.bincount(blocks, weights=pooled.sum(axis=0), minlength=n_blocks)


# ---------------------------------------------------------------------------
# Block compaction (Context Optimization, "H2O KV Cache Eviction / How It
# Works in Flash-MoE", step 4)
# ---------------------------------------------------------------------------

def compact_rows(rows: np.ndarray, keep_ids, n_slots_after: int) -> np.ndarray:
    """Survivors moved to contiguous positions: the per-position rows
    ``[positions, ...]`` of one sequence, with kept block ``keep_ids[k]``
    becoming block ``k`` (16 rows each), in order. Returns the first
    ``n_slots_after`` rows of the compacted sequence."""
    rows = np.asarray(rows)
    out = np.zeros((n_slots_after,) + rows.shape[1:], dtype=rows.dtype)
    for k, b in enumerate(keep_ids):
        lo = k * BLOCK_TOKENS
        if lo >= n_slots_after:
            break
        n = min(BLOCK_TOKENS, n_slots_after - lo, rows.shape[0] - b * BLOCK_TOKENS)
        out[lo:lo + n] = rows[b * BLOCK_TOKENS: b * BLOCK_TOKENS + n]
    return out


def compact_table(table: np.ndarray, keep_ids) -> np.ndarray:
    """A per-block table ``[rows, n_blocks]`` compacted alike: column
    ``keep_ids[k]`` becomes column ``k``; the columns after the kept ones are
    zero (their blocks are free)."""
    table = np.asarray(table)
    out = np.zeros_like(table)
    ids = list(keep_ids)
    if ids:
        out[:, :len(ids)] = table[:, ids]
    return out


def compacted_position(i: int, n_keep: int) -> int:
    """The current position after compaction when the current block (that of
    position i) is the last one kept: the same offset inside the block."""
    return (n_keep - 1) * BLOCK_TOKENS + i % BLOCK_TOKENS


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, bytes_per_elem, positions,
                   scale_bytes_per_position_per_cache=0):
    """Elements ``n_layers * 2 * n_kv_heads * head_dim * positions`` (K and V)
    times their size in bytes, plus the
    FP8 scale overhead of one scale per position per cache (K and V of each
    layer)."""
    elems = n_layers * 2 * n_kv_heads * head_dim * positions
    return elems * bytes_per_elem + n_layers * 2 * positions * scale_bytes_per_position_per_cache
