"""The bf16/FP8 output check can fail: CPU controls at the 397B-like shape
(32769 cached keys, head dim 128, 4 query heads per KV head, FP8 E4M3 values
with per-position scales).

* The arithmetic the decode kernel does to the weights (each p_j times the
  V scale rounded to bf16 before the PV product, the output rounded to bf16),
  simulated in float64 on the oracle's own weights, passes ``close_o``.
* The same output with one 16-key V tile read as zeros (a tile skipped or
  never loaded) fails it, whichever tile is dropped. Block masses do not
  depend on V, so only the output check can see such a bug.
"""

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as orc
from tests import gpu_support as gs

N_KEYS, D, HKV, G = 32769, 128, 8, 4


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(2024)
    # one KV head's share of FP8 rows that cover all 8 KV heads (scales are
    # per position over the whole row)
    k_rows = rng.standard_normal((N_KEYS, HKV * D)).astype(np.float32)
    v_rows = rng.standard_normal((N_KEYS, HKV * D)).astype(np.float32)
    kc, ks = orc.fp8_encode_rows(k_rows)
    vc, vs = orc.fp8_encode_rows(v_rows)
    K = orc.fp8_decode_rows(kc[:, :D], ks)[None]          # KV head 0: [1, n, d]
    Vcode = orc.e4m3_table()[vc[:, :D]]                    # exact bf16 values
    V = Vcode * vs.astype(np.float64)[:, None]
    q = _bf16(rng.standard_normal((G, D)))
    scale = orc.softmax_scale(D)
    o, p = orc.attend(q, K, V[None], scale)
    spread = gs.out_spread(p, V[None])
    return dict(o=o, p=p, V=V, Vcode=Vcode, vs=vs.astype(np.float64), spread=spread, rng=rng)


def _kernel_like(c, p, V_code, vs, rng):
    """Output as the kernel forms it: pw_j = bf16(p_j * r * vs_j) with r a
    power-of-two-free rescale (the running max the weights are taken relative
    to), products with the exact code values, the scale r divided out, then
    rounded to bf16."""
    r = rng.uniform(1.0, 2.0)
    pw = _bf16(p * r * vs[None, :]) / r
    return _bf16(pw @ V_code)


def test_kernel_rounding_passes(case):
    c = case
    for trial in range(5):
        got = _kernel_like(c, c["p"], c["Vcode"], c["vs"], c["rng"])
        gs.close_o(got, c["o"], "fp8", c["spread"])


def test_one_zeroed_v_tile_fails(case):
    c = case
    n_tiles = (N_KEYS + 15) // 16
    tiles = c["rng"].choice(n_tiles, 20, replace=False)
    for t in tiles:
        Vcode = c["Vcode"].copy()
        Vcode[16 * t:16 * t + 16] = 0.0
        got = _kernel_like(c, c["p"], Vcode, c["vs"], c["rng"])
        with pytest.raises(AssertionError):
            gs.close_o(got, c["o"], "fp8", c["spread"])


def test_bound_is_far_below_the_output_scale(case):
    """At 32K keys the rounding term is a small fraction of a typical output
    (the earlier 2^-8 sum_j p_j |v_j| floor was about half of it)."""
    c = case
    term = gs.OUT_SIGMAS * 2.0 ** -9 * c["spread"][1] + gs.OUT_F32_FLOOR * c["spread"][0]
    assert np.median(term) < 0.05 * np.median(np.abs(c["o"]))
