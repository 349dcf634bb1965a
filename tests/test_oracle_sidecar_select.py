"""Pins for the oracle's side-car update, heavy-hitter selection and the KV
size formula.

Checked against: closed forms of the side-car recurrences under constant input,
the trajectory ring's wrap, brute-force subset search for the selection (with
planted exact ties), the protected-region definitions, the planted 128K-style
structure, and the sizes the pages print (golden file).
"""

import os

import numpy as np
import pytest

from oracle import kvs_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.txt")


@pytest.mark.parametrize("alpha", [0.5, 0.25, 0.9])
def test_sidecar_closed_forms_under_constant_input(alpha):
    a = np.array([0.0, 0.5, 1.25, 3.0])
    sc = orc.SideCar(4)
    for s in range(100):
        sc.update(a, alpha)
        assert np.allclose(sc.cum, (s + 1) * a, rtol=1e-14, atol=0)
        assert np.allclose(sc.ema, a * (1 - (1 - alpha) ** (s + 1)), rtol=1e-12, atol=1e-15)
        assert np.array_equal(sc.attended, a)
    assert sc.step == 100


def test_trajectory_ring_wraps_at_64():
    sc = orc.SideCar(3)
    for s in range(64 + 10):
        sc.update(np.full(3, float(s)), 0.5)
    for k in range(64):
        want = 64 + k if k < 10 else k
        assert np.all(sc.traj[k] == want)


def test_ema_first_step_and_linearity():
    sc = orc.SideCar(2)
    sc.update(np.array([2.0, 4.0]), 0.5)
    assert list(sc.ema) == [1.0, 2.0]
    sc.update(np.array([0.0, 0.0]), 0.5)
    assert list(sc.ema) == [0.5, 1.0] and list(sc.cum) == [2.0, 4.0]


def test_protected_regions():
    # recent window of 16 tokens at i = 70 covers positions 55..70: blocks 3 and 4
    assert orc.protected_blocks(70, 16, 0) == {3, 4}
    assert orc.protected_blocks(79, 16, 0) == {4}
    assert orc.protected_blocks(5, 1000, 0) == {0}
    # sinks: first 4 tokens are block 0; first 17 tokens are blocks 0 and 1
    assert orc.protected_blocks(100, 1, 4) == {0, 6}
    assert orc.protected_blocks(100, 1, 17) == {0, 1, 6}
    with pytest.raises(ValueError):
        orc.protected_blocks(10, 0, 0)


@pytest.mark.parametrize("seed", range(12))
def test_selection_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    i = int(rng.integers(16, 200))
    nb = i // 16 + 1
    score = np.round(rng.random(nb + 3) * 4) / 4          # coarse grid -> many exact ties
    alive = rng.random(nb + 3) < 0.8 if seed % 2 else None
    budget = int(rng.integers(0, 6))
    R = int(rng.integers(1, 40))
    S = int(rng.integers(0, 20)) if seed % 3 == 0 else 0
    got = orc.select_blocks(score, alive, i, budget, R, S)
    ref = orc.select_blocks_bruteforce(score, alive, i, budget, R, S)
    assert np.array_equal(got, ref)


def test_exact_ties_go_to_lowest_index():
    score = np.array([1.0, 5.0, 5.0, 5.0, 2.0, 5.0, 0.0, 0.0])
    # i = 127 -> blocks 0..7 exist; recent 1 token protects block 7 only
    got = orc.select_blocks(score, None, 127, 2, 1, 0)
    assert list(got) == [1, 2, 7]
    got = orc.select_blocks(score, None, 127, 4, 1, 0)
    assert list(got) == [1, 2, 3, 5, 7]


def test_dead_blocks_are_never_selected_and_keep_mask_marks_future_blocks():
    score = np.arange(10, dtype=float)
    alive = np.ones(10, dtype=bool)
    alive[8] = False
    got = orc.select_blocks(score, alive, 9 * 16 + 3, 2, 1, 0)
    assert list(got) == [6, 7, 9]
    mask = orc.keep_mask_after(got, 9 * 16 + 3, 12)
    assert list(np.flatnonzero(mask)) == [6, 7, 9, 10, 11]


def test_budget_larger_than_candidates_keeps_everything_alive():
    score = np.zeros(5)
    got = orc.select_blocks(score, None, 79, 100, 1, 0)
    assert list(got) == [0, 1, 2, 3, 4]


def test_planted_anchor_needle_recent_are_selected():
    """Per-Head Attention as a Scoring Signal, 128K example, scaled down: keys
    aligned with the queries at the anchor (0-100), a needle block and the most
    recent 100 tokens pull the most mass, so the heavy set with budget 8 is the
    anchor blocks plus the needle block (the recent ones are protected)."""
    rng = np.random.default_rng(0)
    d, Hq, Hkv, n = 128, 8, 2, 4096
    g = np.sqrt(3 * np.sqrt(d))
    u = rng.standard_normal((Hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    K = rng.standard_normal((Hkv, n, d))
    V = rng.standard_normal((Hkv, n, d))
    needle = 2048
    for r in (range(0, 101), range(needle, needle + 16), range(n - 100, n)):
        K[:, r.start:r.stop] += g * u[:, None, :]
    q = rng.standard_normal((Hq, d)) + g * np.repeat(u, Hq // Hkv, axis=0)
    nb = n // 16
    _, mass = orc.attend_scored(q, K, V, np.arange(n), n - 1, 0, None, orc.softmax_scale(d), nb)
    keep = orc.select_blocks(mass, None, n - 1, 8, 100, 0)
    recent = orc.protected_blocks(n - 1, 100, 0)
    heavy = set(keep.tolist()) - recent
    assert heavy == set(range(0, 7)) | {needle // 16}


def _sizes():
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if line:
            f = [s.strip() for s in line.split("|")]
            yield f[0], [int(x) for x in f[1:7]]


def test_kv_sizes_printed_by_pages():
    n = 0
    for name, (L, H, d, b, pos, want) in _sizes():
        assert orc.kv_cache_bytes(L, H, d, b, pos) == want, name
        n += 1
    assert n >= 10


def test_fp8_scale_overhead_reading():
    # one float32 scale per position per cache: 10 layers x 2 caches x 4 B = 80 B
    per_pos = orc.kv_cache_bytes(10, 4, 128, 1, 1, scale_bytes_per_position_per_cache=4)
    assert per_pos == 10320
    assert 10 * 1024 < per_pos < 11 * 1024      # the page's "~10.5 KB/position"


# ---------------------------------------------------------------- threshold views and counters

def test_hot_count_is_the_number_of_turns_above_threshold():
    """Scissorhands (Context views at marginal cost, section 7, SOTA grounding): the
    count of turns whose attention exceeded the threshold; strict inequality."""
    rng = np.random.default_rng(2)
    nb, turns, theta = 9, 40, 0.35
    A = rng.random((turns, nb))
    A[5, 3] = theta                       # exactly at the threshold: not above it
    count = np.zeros(nb, dtype=np.int32)
    for t in range(turns):
        count = orc.hot_count_update(count, A[t], theta)
    assert np.array_equal(count, np.array([sum(1 for t in range(turns) if A[t, b] > theta) for b in range(nb)]))
    const = np.zeros(nb, dtype=np.int32)
    for _ in range(17):
        const = orc.hot_count_update(const, np.full(nb, 0.5), 0.4)
    assert (const == 17).all()


@pytest.mark.parametrize("alpha", [0.5, 0.25])
def test_cold_gc_turn_has_a_closed_form(alpha):
    """The threshold as a storage GC policy (section 3): after one burst of
    attention a at turn 0 the EMA is alpha*a*(1-alpha)^t, so it first drops
    below theta at t* = floor(log(theta/(alpha*a)) / log(1-alpha)) + 1, and
    the trajectory column is cleared exactly limit-1 turns later."""
    a, theta, limit, nb = 3.0, 0.01, 5, 4
    t_star = int(np.floor(np.log(theta / (alpha * a)) / np.log(1 - alpha))) + 1
    sc = orc.SideCar(nb)
    cold = np.zeros(nb, dtype=np.int64)
    traj = sc.traj
    cleared_at = None
    for t in range(t_star + limit + 3):
        A = np.zeros(nb)
        if t == 0:
            A[1] = a
        sc.update(A, alpha)
        cold, traj = orc.cold_gc_update(cold, sc.ema, sc.traj, theta, limit)
        sc.traj = traj
        if t == 0:
            assert traj[0, 1] == a           # the burst is in the ring until GC
        if cleared_at is None and cold[1] >= limit:
            cleared_at = t
    assert cleared_at == t_star + limit - 1
    assert not traj[:, 1].any() and sc.cum[1] == a   # the cumulative scalar is kept
    assert (cold[[0, 2, 3]] == t_star + limit + 3).all()  # never-attended blocks are cold from turn 0


def test_filter_blocks_brute_force_and_boundaries():
    """A threshold view (section 3, filter(a_s > theta)): existing, alive
    blocks strictly above theta, ascending."""
    rng = np.random.default_rng(8)
    nb, i, theta = 50, 16 * 37 + 3, 0.6
    score = rng.random(nb)
    score[4] = theta                      # not strictly above
    score[45] = 0.99                      # does not exist yet at position i
    alive = rng.random(nb) < 0.8
    ids = orc.filter_blocks(score, alive, i, theta)
    want = [b for b in range(nb) if b <= i // 16 and alive[b] and score[b] > theta]
    assert ids.tolist() == want and 4 not in ids and 45 not in ids
    assert orc.filter_blocks(score, None, i, 2.0).size == 0


def test_selection_on_attended_is_tova():
    """TOVA (Context views at marginal cost, section 7, SOTA grounding): the latest query's head-summed weight, evict
    the minimum. Selecting on Attended with one block less than the candidates
    drops exactly the least-attended candidate."""
    rng = np.random.default_rng(12)
    nb, i, R = 40, 16 * 39 + 5, 16
    att = rng.random(nb)
    prot = set(orc.protected_blocks(i, R, 0))
    cand = [b for b in range(nb) if b not in prot]
    keep = orc.select_blocks(att, None, i, len(cand) - 1, R, 0)
    dropped = set(range(nb)) - set(keep.tolist())
    assert dropped == {min(cand, key=lambda b: att[b])}


# ---------------------------------------------------------------- block compaction

def test_compaction_preserves_attention_over_the_kept_blocks():
    """Context Optimization, H2O step 4: after moving the survivors to
    contiguous positions the kernels see a shorter sequence with the same
    keys, so attention at the compacted position equals attention over the
    original with the evicted blocks masked, and each kept block's mass moves
    with it."""
    rng = np.random.default_rng(14)
    Hq, Hkv, d, i, nb = 8, 2, 16, 16 * 20 + 6, 24
    K = rng.standard_normal((Hkv, i + 1, d))
    V = rng.standard_normal((Hkv, i + 1, d))
    q = rng.standard_normal((Hq, d))
    score = rng.random(nb)
    keep = orc.select_blocks(score, None, i, 6, 20, 4)
    assert keep[-1] == i // 16
    alive = np.zeros(nb, dtype=bool)
    alive[keep] = True
    o_mask, m_mask = orc.attend_scored(q, K, V, np.arange(i + 1), i, 0, alive, 0.25, nb)
    i2 = orc.compacted_position(i, len(keep))
    Kc = orc.compact_rows(K.transpose(1, 0, 2), keep, i2 + 1).transpose(1, 0, 2)
    Vc = orc.compact_rows(V.transpose(1, 0, 2), keep, i2 + 1).transpose(1, 0, 2)
    o_c, m_c = orc.attend_scored(q, Kc, Vc, np.arange(i2 + 1), i2, 0, None, 0.25, nb)
    assert np.abs(o_c - o_mask).max() <= 1e-12
    assert np.abs(m_c[:len(keep)] - m_mask[keep]).max() <= 1e-12 and not m_c[len(keep):].any()


def test_compaction_gather_brute_force():
    rng = np.random.default_rng(15)
    rows = rng.standard_normal((16 * 9 + 5, 3))
    keep = [0, 2, 3, 7, 9]
    n_after = 16 * 4 + 5
    out = orc.compact_rows(rows, keep, n_after)
    for s_new in range(n_after):
        k, t = divmod(s_new, 16)
        assert np.array_equal(out[s_new], rows[16 * keep[k] + t])
    table = rng.random((3, 12))
    ct = orc.compact_table(table, keep)
    for k in range(12):
        assert np.array_equal(ct[:, k], table[:, keep[k]] if k < len(keep) else np.zeros(3))
    assert orc.compacted_position(16 * 9 + 4, 5) == 16 * 4 + 4
