"""The once-per-step block masses (kvs_append_decode_attn_tap /
kvs_decode_attn_tap per layer, then kvs_tap_masses) against one scored call
per layer, in deterministic mode: outputs, masses, per-head masses, their max
and every cache buffer must agree bit for bit, over several layers and steps,
on linear, windowed, keep-masked and ring caches, and with more layers than
the combine's LDS holds at once. The per-layer path is checked against the
float64 oracle by the other parity tests; the workload tests run the session,
which uses the tap path, against the oracle too."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import gpu_support as gs
from tests.test_gpu_fused_append import FUSED_CASES, _prefill, _rows, _setup

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from heavy_hitter_eviction_amd import api as _api
    return _api


# kv, d, Hq, Hkv, C, B, window, ring, src, keep  (+ layers)
TAP_CASES = [c + (3,) for c in FUSED_CASES] + [
    ("bf16", 64, 16, 1, 16384, 1, 0, False, "bf16", False, 3),   # 256 partitions: two layers' tables per LDS chunk
    ("fp8", 128, 32, 8, 2064, 2, 0, False, "f32", True, 5),
    # one and two layers: the layer combine's waves split the tiles (8 and 4 groups)
    ("fp8", 128, 32, 8, 8208, 2, 0, False, "f32", False, 1),
    ("bf16", 128, 16, 4, 4112, 3, 0, False, "bf16", True, 2),
    ("fp8", 128, 16, 4, 1024, 2, 1000, True, "f32", False, 1),
    ("bf16", 64, 8, 2, 2064, 2, 700, False, "bf16", False, 2),
    # group sizes that are not powers of two (G = 3 and 6)
    ("fp8", 128, 12, 4, 1040, 2, 0, False, "f32", True, 3),
    ("bf16", 128, 24, 4, 528, 2, 500, True, "bf16", False, 2),
]
STEPS = 6


@pytest.mark.parametrize("case", TAP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_tap_masses_equal_per_layer_scored_calls(api, case):
    kv, d, Hq, Hkv, C, B, window, ring, src, use_keep, L = case
    geom, K, V, src_dt, start, keep, _ = _setup(api, case[:10], deterministic=True)
    ref = [_prefill(api, geom, K, V, src_dt, start) for _ in range(L)]
    tap = [_prefill(api, geom, K, V, src_dt, start) for _ in range(L)]
    qdt = torch.float32 if kv == "f32" else torch.bfloat16
    ws_ref = api.decode_workspace(geom)
    ws_tap = [api.decode_workspace(geom) for _ in range(L)]
    f32 = dict(dtype=torch.float32, device="cuda")
    mass_r, mass_t = torch.zeros((B, geom.nb), **f32), torch.zeros((B, geom.nb), **f32)
    hm_r, hm_t = torch.zeros((B, Hq, geom.nb), **f32), torch.zeros((B, Hq, geom.nb), **f32)
    mx_r, mx_t = torch.zeros((B, geom.nb), **f32), torch.zeros((B, geom.nb), **f32)
    seqs = torch.arange(B, dtype=torch.int32, device="cuda")
    for t in range(STEPS):
        pos = np.array([s + t for s in start], dtype=np.int32)
        cur = gs.to_dev(pos)
        krow = torch.from_numpy(np.stack([K[b, pos[b]] for b in range(B)])).to(src_dt).cuda()
        vrow = torch.from_numpy(np.stack([V[b, pos[b]] for b in range(B)])).to(src_dt).cuda()
        profiled = t % 2 == 1            # per-head masses and their max on odd steps
        outs_r, outs_t = [], []
        for l in range(L):
            q = torch.from_numpy(_rows((B, Hq, d), (29, 3, t, l))).to(qdt).cuda()
            o_r, o_t = torch.empty_like(q), torch.empty_like(q)
            if profiled:
                ref[l].append(krow, vrow, seqs, cur)
                api.decode_attn_profiled(ref[l], q, cur, o_r, ws_ref, mass_accum=mass_r, head_mass=hm_r,
                                         mass_max=mx_r, keep_mask=keep)
                tap[l].append(krow, vrow, seqs, cur)
                api.decode_attn_tap(tap[l], q, cur, o_t, ws_tap[l], keep_mask=keep)
            else:
                api.append_decode_attn(ref[l], krow, vrow, q, cur, o_r, ws_ref, mass_accum=mass_r, keep_mask=keep)
                api.decode_attn_tap(tap[l], q, cur, o_t, ws_tap[l], keep_mask=keep, k_new=krow, v_new=vrow)
            outs_r.append(o_r)
            outs_t.append(o_t)
        if profiled:
            api.tap_masses(geom, ws_tap, cur, mass_accum=mass_t, head_mass=hm_t, mass_max=mx_t)
        else:
            api.tap_masses(geom, ws_tap, cur, mass_accum=mass_t)
        torch.cuda.synchronize()
        iv = torch.int16 if kv != "f32" else torch.int32
        for l in range(L):
            assert torch.equal(outs_r[l].view(iv), outs_t[l].view(iv)), f"step {t} layer {l}: out"
        assert torch.equal(mass_r, mass_t), f"step {t}: mass"
        assert torch.equal(hm_r, hm_t) and torch.equal(mx_r, mx_t), f"step {t}: per-head masses"
        for l in range(L):
            for x, y in zip((ref[l].k, ref[l].v, ref[l].k_scale, ref[l].v_scale, ref[l].pos_of_slot),
                            (tap[l].k, tap[l].v, tap[l].k_scale, tap[l].v_scale, tap[l].pos_of_slot)):
                if x is not None:
                    assert torch.equal(x, y), f"step {t} layer {l}: cache"
