"""The whole-step call (kvs_decode_step) against the calls it stands for, in
deterministic mode: per layer kvs_append_decode_attn_tap (or
kvs_decode_attn_tap when nothing is appended), then kvs_tap_masses, then
kvs_update_sidecar_select (or kvs_update_sidecar). Outputs, masses, every
side-car array, the keep words, the selected ids and every cache buffer must
agree bit for bit after each step, on linear, windowed, keep-masked
(evict-mode feedback: the keep words the selection writes are read by the
next step) and ring caches, with and without the selection, and in the
layers-only form (masses left in the workspaces for a separate
kvs_tap_masses, or closed by kvs_close_step, whose side-car update without
selection runs in the mass combine's launch). The per-layer calls are checked against the float64 oracle
by the other parity tests, and the workload tests run the session, which
takes this call, against the oracle too."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import gpu_support as gs
from tests.test_gpu_fused_append import FUSED_CASES, _cache_buffers, _prefill, _rows, _setup

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from heavy_hitter_eviction_amd import api as _api
    return _api


# a FUSED_CASES entry, the layer count, the turn ("select", "sidecar",
# "layers": masses added by a separate tap_masses, no turn; "close-...": a
# layers-only step closed by kvs_close_step), appended rows
STEP_CASES = [
    (FUSED_CASES[0], 3, "select", True),
    (FUSED_CASES[1], 2, "sidecar", True),
    (FUSED_CASES[2], 3, "select", True),     # keep words fed back every step
    (FUSED_CASES[3], 4, "layers", True),
    (FUSED_CASES[4], 2, "select", False),    # nothing appended: kvs_decode_attn_tap per layer
    (FUSED_CASES[5], 2, "select", True),
    (FUSED_CASES[6], 3, "sidecar", True),    # FP8 ring
    (FUSED_CASES[7], 2, "select", True),     # bf16 ring with a window
    (FUSED_CASES[8], 2, "layers", True),
    # layers-only step, then kvs_close_step (the side-car in the combine's
    # launch without selection)
    (FUSED_CASES[1], 2, "close-sidecar", True),
    (FUSED_CASES[6], 3, "close-sidecar", True),  # FP8 ring
    (FUSED_CASES[7], 2, "close-sidecar", True),  # bf16 ring with a window
    (FUSED_CASES[2], 2, "close-select", True),   # keep words fed back every step
]
STEPS = 5


class _State:
    def __init__(self, geom, B, traj_cap=8):
        f32 = dict(dtype=torch.float32, device="cuda")
        nb = geom.nb
        self.mass = torch.zeros((B, nb), **f32)
        self.att = torch.zeros((B, nb), **f32)
        self.ema = torch.zeros((B, nb), **f32)
        self.cum = torch.zeros((B, nb), **f32)
        self.traj = torch.zeros((B, traj_cap, nb), **f32)
        self.keep = torch.full((B, geom.words), -1, dtype=torch.int32, device="cuda")
        self.sel = torch.zeros((B, nb), dtype=torch.int32, device="cuda")
        self.n_sel = torch.zeros((B,), dtype=torch.int32, device="cuda")

    def tensors(self):
        return [self.mass, self.att, self.ema, self.cum, self.traj, self.keep, self.sel, self.n_sel]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "-".join(map(str, c[0])) + f"-L{c[1]}-{c[2]}-{c[3]}")
def test_decode_step_equals_the_calls_it_stands_for(api, case):
    fcase, L, mode, append = case
    kv, d, Hq, Hkv, C, B, window, ring, src, use_keep = fcase
    geom, K, V, src_dt, start, _, _ = _setup(api, fcase, deterministic=True)
    ref = [_prefill(api, geom, K, V, src_dt, start) for _ in range(L)]
    stp = [_prefill(api, geom, K, V, src_dt, start) for _ in range(L)]
    qdt = torch.float32 if kv == "f32" else torch.bfloat16
    ws_r = [api.decode_workspace(geom) for _ in range(L)]
    ws_s = [api.decode_workspace(geom) for _ in range(L)]
    sr, ss = _State(geom, B), _State(geom, B)
    budget, recent, sinks = 3, 16, 4
    # keep-masked cases run in evict mode: the selection's keep words are the
    # next step's mask (no keep mask with a window)
    evict = use_keep and not window
    seqs = torch.arange(B, dtype=torch.int32, device="cuda")
    for t in range(STEPS):
        pos = np.array([s + t for s in start], dtype=np.int32)
        cur = gs.to_dev(pos)
        krow = torch.from_numpy(np.stack([K[b, pos[b]] for b in range(B)])).to(src_dt).cuda()
        vrow = torch.from_numpy(np.stack([V[b, pos[b]] for b in range(B)])).to(src_dt).cuda()
        qs = [torch.from_numpy(_rows((B, Hq, d), (31, 5, t, l))).to(qdt).cuda() for l in range(L)]
        o_r = [torch.empty_like(q) for q in qs]
        o_s = [torch.empty_like(q) for q in qs]
        # the calls
        for l in range(L):
            if append:
                api.decode_attn_tap(ref[l], qs[l], cur, o_r[l], ws_r[l], keep_mask=sr.keep if evict else None,
                                    k_new=krow, v_new=vrow)
            else:
                api.decode_attn_tap(ref[l], qs[l], cur, o_r[l], ws_r[l], keep_mask=sr.keep if evict else None)
        api.tap_masses(geom, ws_r, cur, mass_accum=sr.mass)
        if mode in ("select", "close-select"):
            api.update_sidecar_select(sr.mass, sr.att, sr.ema, sr.cum, sr.traj, t, 0.5, cur, budget, recent, sinks,
                                      alive=sr.keep if evict else None, keep_mask=sr.keep, sel_ids=sr.sel,
                                      n_sel=sr.n_sel)
        elif mode in ("sidecar", "close-sidecar"):
            api.update_sidecar(sr.mass, sr.att, sr.ema, sr.cum, sr.traj, t, 0.5)
        # the one call (two in the layers-only form)
        turn = None
        if mode != "layers":
            turn = api.Turn(ss.att, ss.ema, ss.cum, ss.traj, step=t, alpha=0.5,
                            select=mode in ("select", "close-select"), budget_blocks=budget,
                            recent_tokens=recent, sink_tokens=sinks, alive=ss.keep if evict else None,
                            keep_out=ss.keep, sel_ids=ss.sel, n_sel=ss.n_sel)
        layers_only = mode == "layers" or mode.startswith("close")
        api.decode_step(stp, qs, cur, o_s, ws_s, k_new=[krow] * L if append else None,
                        v_new=[vrow] * L if append else None, keep_mask=ss.keep if evict else None,
                        mass_accum=None if layers_only else ss.mass, turn=None if layers_only else turn)
        if mode == "layers":
            api.tap_masses(geom, ws_s, cur, mass_accum=ss.mass)
        elif mode.startswith("close"):
            api.close_step(geom, ws_s, cur, ss.mass, turn)
        torch.cuda.synchronize()
        iv = torch.int16 if kv != "f32" else torch.int32
        for l in range(L):
            assert torch.equal(o_r[l].view(iv), o_s[l].view(iv)), f"step {t} layer {l}: out"
            for x, y in zip(_cache_buffers(ref[l]), _cache_buffers(stp[l])):
                assert torch.equal(x, y), f"step {t} layer {l}: cache"
        for name, x, y in zip(("mass", "attended", "ema", "cum", "traj", "keep", "sel_ids", "n_sel"),
                              sr.tensors(), ss.tensors()):
            assert torch.equal(x, y), f"step {t}: {name}"
