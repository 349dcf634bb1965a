"""Pins for the oracle's attention, block mass and window handling.

Checked against: torch's float64 scaled_dot_product_attention (an independent
implementation, GQA by repeating KV heads), special cases with closed forms
(one key, identical keys, window 1, zero queries), the sum-to-one invariant of
post-softmax weights, the window rule the four-slot-cache page prints, and that
page's own method: an incremental slot cache checked against the full masked
reference at 1e-12, with a slot-as-position negative control that must fail.
"""

import os

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden", "window_rule.txt")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_attend_matches_torch_sdpa_float64_gqa():
    rng = np.random.default_rng(41)
    for Hq, Hkv, d, n in [(4, 2, 16, 65), (16, 4, 128, 300), (8, 8, 32, 1), (32, 8, 64, 97)]:
        q, K, V = _rand(rng, Hq, d), _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d)
        scale = orc.softmax_scale(d)
        o, p = orc.attend(q, K, V, scale)
        G = Hq // Hkv
        Kt = torch.from_numpy(K).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], Kt, Vt, scale=scale)[0, :, 0].numpy()
        assert np.abs(o - ref).max() <= 1e-12
        assert np.abs(p.sum(axis=1) - 1).max() <= 1e-12


def test_single_key_returns_its_value_and_identical_keys_are_uniform():
    rng = np.random.default_rng(7)
    q, K, V = _rand(rng, 4, 16), _rand(rng, 2, 1, 16), _rand(rng, 2, 1, 16)
    o, p = orc.attend(q, K, V, 0.25)
    assert np.array_equal(p, np.ones((4, 1)))
    assert np.allclose(o, np.repeat(V[:, 0], 2, axis=0), atol=0, rtol=0)
    K = np.repeat(_rand(rng, 2, 1, 16), 10, axis=1)
    V = _rand(rng, 2, 10, 16)
    o, p = orc.attend(q, K, V, 0.25)
    assert np.abs(p - 0.1).max() <= 1e-15
    assert np.abs(o - np.repeat(V.mean(axis=1), 2, axis=0)).max() <= 1e-14


def test_window_rule_golden():
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        kind, i, w, rest = [s.strip() for s in line.split("|")]
        i, w, want = int(i), int(w), [int(x) for x in rest.split()]
        if kind == "visible":
            got = [p for p in range(i + 1) if orc.key_visible(p, i, w)]
            assert got == want, line
        else:
            assert orc.ring_slot(i, w) == want[0]
    with pytest.raises(ValueError):
        orc.key_visible(0, 0, -1)


def test_visible_mask_follows_the_window_rule():
    """The vectorised mask gives the page's window examples (golden file) and
    agrees with the scalar rule, alive blocks included, on random cases."""
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line or not line.startswith("visible"):
            continue
        _, i, w, rest = [s.strip() for s in line.split("|")]
        i, w = int(i), int(w)
        got = np.flatnonzero(orc.visible_mask(np.arange(i + 1), i, w)).tolist()
        assert got == [int(x) for x in rest.split()], line
    rng = np.random.default_rng(5)
    for _ in range(200):
        i = int(rng.integers(0, 300))
        w = int(rng.choice([0, 1, 4, int(rng.integers(1, 300))]))
        pos = rng.integers(-3, 320, 64)
        alive = rng.random(21) < 0.6 if rng.random() < 0.5 else None
        want = [orc.key_visible(int(p), i, w) and (int(p) < 0 or orc.block_alive(alive, orc.block_of(int(p))))
                for p in pos]
        assert orc.visible_mask(pos, i, w, alive).tolist() == want
    with pytest.raises(ValueError):
        orc.visible_mask(np.arange(3), 2, -1)


def test_window_one_returns_current_value():
    rng = np.random.default_rng(19)
    n, i = 40, 33
    K, V, q = _rand(rng, 2, n, 16), _rand(rng, 2, n, 16), _rand(rng, 4, 16)
    o, mass = orc.full_masked_reference(q, K, V, i, 1, 0.25, n_blocks=3)
    assert np.allclose(o, np.repeat(V[:, i], 2, axis=0), rtol=0, atol=1e-15)
    assert mass[i // 16] == pytest.approx(4.0, abs=1e-12) and mass.sum() == pytest.approx(4.0, abs=1e-12)


def test_block_mass_sums_to_heads_and_is_proportional_under_uniform_logits():
    rng = np.random.default_rng(3)
    Hq, Hkv, d, n = 16, 4, 64, 100
    K, V = _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d)
    positions = np.arange(n)
    _, p = orc.attend(_rand(rng, Hq, d), K, V, orc.softmax_scale(d))
    mass = orc.block_mass(p, positions, 7)
    assert abs(mass.sum() - Hq) <= 1e-12
    _, p = orc.attend(np.zeros((Hq, d)), K, V, orc.softmax_scale(d))
    mass = orc.block_mass(p, positions, 7)
    counts = np.bincount(positions // 16, minlength=7)
    assert np.abs(mass - Hq * counts / n).max() <= 1e-12


def test_mass_brute_force_loop():
    """The vectorised reduction equals a plain double loop over heads and keys."""
    rng = np.random.default_rng(11)
    p = rng.random((3, 50))
    pos = rng.permutation(80)[:50]
    m = orc.block_mass(p, pos, 5)
    ref = np.zeros(5)
    for h in range(3):
        for j in range(50):
            ref[pos[j] // 16] += p[h, j]
    assert np.abs(m - ref).max() <= 1e-14


@pytest.mark.parametrize("seed", [7, 19, 41])
@pytest.mark.parametrize("window", [1, 4, 0])
@pytest.mark.parametrize("length", [1, 2, 8, 17])
def test_ring_cache_equals_full_masked_reference(seed, window, length):
    """LLM mechanics III, sections 2 and 5: windows {1, 4, none} x lengths
    {1, 2, 8, 17} x seeds {7, 19, 41}, single-token and chunked appends, checked
    at 1e-12 against the full masked reference."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, d = 4, 2, 16
    K = _rand(rng, Hkv, length, d)
    V = _rand(rng, Hkv, length, d)
    Q = _rand(rng, length, Hq, d)
    nb = (length + 15) // 16
    caps = [length] if window == 0 else sorted({window, window + 16, 2 * window})
    for cap in caps:
        for chunk in (1, 3):
            cache = orc.RingCache(Hkv, d, cap)
            t = 0
            while t < length:
                n = min(chunk, length - t)
                cache.append(K[:, t:t + n], V[:, t:t + n])
                for i in range(t, t + n):
                    if chunk > 1 and i < t + n - 1 and window > 0 and t + n - 1 - i >= cap - window + 1:
                        continue  # that query's window was overwritten by the chunk: not a decode read
                    ref_o, ref_m = orc.full_masked_reference(Q[i], K, V, i, window, 0.25, nb)
                    o, m = cache.attend(Q[i], i, window, 0.25, nb)
                    assert np.abs(o - ref_o).max() <= 1e-12
                    assert np.abs(m - ref_m).max() <= 1e-12
                t += n
            assert cache.next_position == length


def test_slot_as_position_negative_control_fails_after_wrap():
    """LLM mechanics III, section 3 (slots are not positions): reading slot
    indices as positions must give wrong block masses once the ring wraps, and
    a wrong key set when a window is applied."""
    rng = np.random.default_rng(7)
    Hq, Hkv, d, cap, length = 4, 2, 16, 16, 40
    K, V, Q = _rand(rng, Hkv, length, d), _rand(rng, Hkv, length, d), _rand(rng, length, Hq, d)
    nb = 3
    cache = orc.RingCache(Hkv, d, cap)
    worst_mass = 0.0
    for i in range(length):
        cache.append(K[:, i:i + 1], V[:, i:i + 1])
        lo = max(0, i - cap + 1)
        ref_o, ref_m = orc.attend_scored(Q[i], K[:, lo:i + 1], V[:, lo:i + 1], np.arange(lo, i + 1),
                                         i, 0, None, 0.25, nb)
        o, m = cache.attend(Q[i], i, 0, 0.25, nb)
        assert np.abs(o - ref_o).max() <= 1e-12 and np.abs(m - ref_m).max() <= 1e-12
        _, m_bad = cache.attend(Q[i], i, 0, 0.25, nb, mask_by_slot=True)
        if i < cap:
            assert np.abs(m_bad - ref_m).max() <= 1e-12
        else:
            worst_mass = max(worst_mass, np.abs(m_bad - ref_m).max())
    assert worst_mass > 0.5
    # with a window the slot reading also picks the wrong keys
    w = 8
    cache = orc.RingCache(Hkv, d, cap)
    worst_o = 0.0
    for i in range(cap + w - 1):
        cache.append(K[:, i:i + 1], V[:, i:i + 1])
        ref_o, _ = orc.full_masked_reference(Q[i], K, V, i, w, 0.25, nb)
        o, _ = cache.attend(Q[i], i, w, 0.25, nb)
        assert np.abs(o - ref_o).max() <= 1e-12
        if i >= cap:
            o_bad, _ = cache.attend(Q[i], i, w, 0.25, nb, mask_by_slot=True)
            worst_o = max(worst_o, np.abs(o_bad - ref_o).max())
    assert worst_o > 1e-3


def test_all_masked_row_is_rejected():
    with pytest.raises(ValueError):
        orc.attend(np.zeros((2, 4)), np.zeros((1, 0, 4)), np.zeros((1, 0, 4)), 0.5)
    with pytest.raises(ValueError):
        orc.attend(np.zeros((3, 4)), np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), 0.5)


def test_alive_mask_equals_attending_kept_blocks_only():
    """Masking dropped blocks gives the same result as compacting the kept keys
    into a shorter sequence (attention is invariant to key order)."""
    rng = np.random.default_rng(5)
    Hq, Hkv, d, n = 8, 2, 32, 90
    K, V, q = _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d), _rand(rng, Hq, d)
    alive = np.array([True, False, True, False, True, True])
    o, m = orc.attend_scored(q, K, V, np.arange(n), n - 1, 0, alive, 0.2, 6)
    keep = np.array([alive[j // 16] for j in range(n)])
    perm = rng.permutation(np.flatnonzero(keep))
    o2, p2 = orc.attend(q, K[:, perm], V[:, perm], 0.2)
    assert np.abs(o - o2).max() <= 1e-12
    assert np.abs(m - orc.block_mass(p2, perm, 6)).max() <= 1e-12
    assert m[1] == 0 and m[3] == 0


# ---------------------------------------------------------------- Tier 2 re-attend

def _sdpa_over(q, K, V, cols, scale):
    """torch float64 attention over the key columns ``cols`` (GQA by repeat)."""
    G = q.shape[0] // K.shape[0]
    Kt = torch.from_numpy(K[:, cols]).repeat_interleave(G, 0)[None]
    Vt = torch.from_numpy(V[:, cols]).repeat_interleave(G, 0)[None]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], Kt, Vt, scale=scale)[0, :, 0].numpy()


def test_reattend_matches_sdpa_over_gathered_blocks():
    """Context views at marginal cost, Tier 2: the new query attends over the
    cached keys of the chosen spans only. Pinned against torch attention over the
    gathered columns and an explicit per-block loop for the distribution."""
    rng = np.random.default_rng(23)
    Hq, Hkv, d, n, nb = 8, 2, 32, 150, 12
    K, V, q = _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d), _rand(rng, Hq, d)
    i = 140                      # keys after i exist in the cache but are not read
    ids = [9, 2, 2, 7, 0, 11]    # any order, repeats; block 9 holds keys 144..149 > i only partly
    o, m = orc.reattend_blocks(q, K, V, np.arange(n), i, ids, 0.17, nb)
    cols = [j for j in range(n) if j <= i and j // 16 in set(ids)]
    assert np.abs(o - _sdpa_over(q, K, V, cols, 0.17)).max() <= 1e-12
    G = Hq // Hkv
    want = np.zeros(nb)
    for h in range(Hq):
        s = np.array([K[h // G, j] @ q[h] * 0.17 for j in cols])
        w = np.exp(s - s.max())
        w /= w.sum()
        for j, wj in zip(cols, w):
            want[j // 16] += wj
    assert np.abs(m - want).max() <= 1e-12
    assert abs(m.sum() - Hq) <= 1e-12
    assert all(m[b] == 0 for b in range(nb) if b not in set(ids))


def test_reattend_over_every_block_is_full_attention_and_empty_set_is_zero():
    rng = np.random.default_rng(29)
    Hq, Hkv, d, n = 4, 4, 16, 40
    K, V, q = _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d), _rand(rng, Hq, d)
    o, m = orc.reattend_blocks(q, K, V, np.arange(n), n - 1, [2, 1, 0], 0.25, 3)
    assert np.abs(o - _sdpa_over(q, K, V, list(range(n)), 0.25)).max() <= 1e-12
    o0, m0 = orc.reattend_blocks(q, K, V, np.arange(n), n - 1, [], 0.25, 3)
    assert not o0.any() and not m0.any()
    # a block past the query position contributes nothing
    o1, m1 = orc.reattend_blocks(q, K, V, np.arange(n), 15, [1, 2], 0.25, 3)
    assert not o1.any() and not m1.any()


# ---------------------------------------------------------------- per-head profile, max over heads

def test_per_head_profile_brute_force_and_invariants():
    """Context views at marginal cost, section 4 (per-head profile) and
    Per-Head Attention as a Scoring Signal (max over heads): per-head block
    masses from an explicit loop over keys, each head's row sums to one, the
    rows sum to the head-summed mass, and the max lies between mean and sum."""
    rng = np.random.default_rng(31)
    Hq, Hkv, d, n, nb = 8, 2, 16, 77, 6
    K, V, q = _rand(rng, Hkv, n, d), _rand(rng, Hkv, n, d), _rand(rng, Hq, d)
    alive = np.array([True, True, False, True, True, True])
    o, mass, hm, mx = orc.attend_profiled(q, K, V, np.arange(n), n - 1, 0, alive, 0.3, nb)
    G = Hq // Hkv
    cols = [j for j in range(n) if alive[j // 16]]
    want = np.zeros((Hq, nb))
    for h in range(Hq):
        s = np.array([K[h // G, j] @ q[h] * 0.3 for j in cols])
        w = np.exp(s - s.max())
        w /= w.sum()
        for j, wj in zip(cols, w):
            want[h, j // 16] += wj
    assert np.abs(hm - want).max() <= 1e-12
    assert np.abs(hm.sum(axis=1) - 1).max() <= 1e-12
    assert np.abs(hm.sum(axis=0) - mass).max() <= 1e-12
    assert np.abs(mx - want.max(axis=0)).max() <= 1e-12
    assert (mx <= mass + 1e-15).all() and (mx >= mass / Hq - 1e-15).all()
    assert mx[2] == 0


def test_max_over_heads_keeps_a_block_one_head_weights():
    """Per-Head Attention as a Scoring Signal: an anchor head that looks only at
    block 0 keeps it on top of the max-over-heads score even when every other
    head has moved on to the recent blocks, while the head sum ranks it last."""
    d, n = 16, 64
    Hq, Hkv = 8, 8
    K = np.zeros((Hkv, n, d))
    V = np.ones((Hkv, n, d))
    q = np.zeros((Hq, d))
    K[0, :16, 0] = 400.0         # head 0 (its own KV head) locks onto block 0
    for h in range(1, Hq):
        K[h, 48:, 1] = 400.0      # the others onto block 3
        q[h, 1] = 1.0
    q[0, 0] = 1.0
    _, mass, hm, mx = orc.attend_profiled(q, K, V, np.arange(n), n - 1, 0, None, 0.25, 4)
    assert abs(mx[0] - 1.0) <= 1e-9 and abs(mx[3] - 1.0) <= 1e-9
    assert mass[0] < mass[3] / 5


# ---------------------------------------------------------------- SnapKV prefill scoring

def test_snapkv_token_scores_independent_softmax_and_invariants():
    """Context views at marginal cost, section 3 (SnapKV): window queries'
    weights summed per (token, head). Pinned by explicit torch softmaxes per
    query, the per-head total equal to the number of window queries, and the
    one-query window equal to that query's attention weights."""
    rng = np.random.default_rng(33)
    Hq, Hkv, d, n, W = 8, 2, 16, 70, 5
    K = rng.standard_normal((Hkv, n + 4, d))      # slots past the prompt are never read
    qw = rng.standard_normal((W, Hq, d))
    s = orc.snapkv_token_scores(qw, K, n, 0.3)
    G = Hq // Hkv
    want = np.zeros((Hq, n))
    for w in range(W):
        pos = n - W + w
        for h in range(Hq):
            logits = torch.from_numpy(K[h // G, :pos + 1] @ qw[w, h] * 0.3)
            want[h, :pos + 1] += torch.softmax(logits, 0).numpy()
    assert np.abs(s - want).max() <= 1e-12
    assert np.abs(s.sum(axis=1) - W).max() <= 1e-12
    one = orc.snapkv_token_scores(qw[-1:], K, n, 0.3)
    _, p = orc.attend(qw[-1], K[:, :n], K[:, :n], 0.3)
    assert np.abs(one - p).max() <= 1e-12
    short = orc.snapkv_token_scores(qw, K, 3, 0.3)   # queries at negative positions read nothing
    assert abs(short.sum(axis=1)[0] - 3) <= 1e-12


def test_max_pool_matches_torch_and_drags_neighbours():
    """SnapKV's max-pool (kernel 7): against torch's max_pool1d with -inf
    padding; kernel 1 is the identity; one spike spreads to +-3 tokens."""
    rng = np.random.default_rng(34)
    sc = rng.random((3, 45))
    for k in (1, 3, 7):
        ref = torch.nn.functional.max_pool1d(torch.from_numpy(sc)[None], k, stride=1, padding=k // 2)[0].numpy()
        assert np.array_equal(orc.max_pool_tokens(sc, k), ref)
    spike = np.zeros((1, 20))
    spike[0, 10] = 1.0
    assert orc.max_pool_tokens(spike, 7)[0].tolist() == [0.0] * 7 + [1.0] * 7 + [0.0] * 6
    b = orc.snapkv_block_scores(np.ones((2, 40)), 4)
    assert b.tolist() == [32.0, 32.0, 16.0, 0.0]
