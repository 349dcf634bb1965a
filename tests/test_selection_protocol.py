"""The selection comparison used by the GPU tests (near-tie protocol plus the
observed-error band) accepts a swap of two near-tied blocks and rejects a
wrong block, on the CPU."""

import numpy as np
import pytest

from oracle import kvs_oracle as orc
from tests import gpu_support as gs


def _case():
    rng = np.random.default_rng(4)
    score = rng.random(400)
    i, budget, recent = 400 * 16 - 1, 40, 64
    ref = orc.select_blocks(score, None, i, budget, recent)
    return score, i, budget, recent, ref


def test_identical_sets_pass_and_report_the_bands():
    score, i, budget, recent, ref = _case()
    n = gs.compare_selection(ref, ref, score, i, budget, recent, 0, None, 1e-4, score_gpu=score.astype(np.float32))
    assert n >= 1          # v itself is always within the band


def test_swap_of_a_near_tie_passes_when_the_scores_allow_it():
    score, i, budget, recent, ref = _case()
    prot = orc.protected_blocks(i, recent, 0)
    cand = sorted((b for b in range(len(score)) if b not in prot), key=lambda b: (-score[b], b))
    last_in, first_out = cand[budget - 1], cand[budget]
    score = score.copy()
    score[first_out] = score[last_in] - 1e-9          # a near tie at the boundary
    ref = orc.select_blocks(score, None, i, budget, recent)
    gpu_score = score.copy()
    gpu_score[first_out] += 2e-9                       # the GPU's rounding flips the pair
    gpu = orc.select_blocks(gpu_score, None, i, budget, recent)
    assert set(gpu) != set(ref)
    gs.compare_selection(gpu, ref, score, i, budget, recent, 0, None, 1e-4, score_gpu=gpu_score)


def test_a_wrong_block_fails():
    score, i, budget, recent, ref = _case()
    prot = orc.protected_blocks(i, recent, 0)
    cand = sorted((b for b in range(len(score)) if b not in prot), key=lambda b: (-score[b], b))
    gpu = sorted((set(ref) - {cand[0]}) | {cand[-1]})     # best block dropped, worst kept
    with pytest.raises(AssertionError):
        gs.compare_selection(gpu, ref, score, i, budget, recent, 0, None, 1e-4, score_gpu=score)
    # a swap just outside the observed-error band fails the sharper check
    last_in, first_out = cand[budget - 1], cand[budget]
    gap = score[last_in] - score[first_out]
    gpu = sorted((set(ref) - {last_in}) | {first_out})
    noisy = score + np.where(np.arange(len(score)) % 2 == 0, 1, -1) * gap / 5
    # (rel_tol 1 puts every candidate inside the protocol's Amb: only the band check can fail)
    with pytest.raises(AssertionError, match="observed-error band"):
        gs.compare_selection(gpu, ref, score, i, budget, recent, 0, None, 1.0, score_gpu=noisy)
