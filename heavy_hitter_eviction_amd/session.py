"""A whole scored decode step over L layers, driven through the C ABI.

For every layer: append the new position's K/V (FP8-encoding when the cache
is FP8), then the scored attention. By default the append runs inside the
attention's partial kernel and each layer leaves its per-block sums in its own
workspace (kvs_append_decode_attn_tap); after the last layer one call adds all
layers' block masses into ``mass`` (kvs_tap_masses). ``tap=False`` adds them
layer by layer instead (kvs_append_decode_attn / kvs_decode_attn_scored), and
``fused=False`` makes the append a launch of its own. After the last layer the side-car closes the turn,
and the heavy-hitter selection produces the keep mask. In evict mode that
mask feeds the next step's attention, so dropped blocks are never read again
(Context Optimization, "H2O KV Cache Eviction"); in score-only mode the full
context is read and the mask is only reported. Compact mode (linear caches) is
evict mode plus, every ``compact_every`` steps, moving the kept blocks to the
front of every layer's cache with the side-car arrays (H2O step 4); the
sequence then continues at its compacted position.

Host code here only sequences library calls and owns torch buffers.
"""

from __future__ import annotations

import torch

from . import api
from .workloads import Workload


def geom_of(w: Workload, deterministic: bool = False) -> api.CacheGeom:
    return api.CacheGeom(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         head_dim=w.head_dim, capacity=w.capacity, window=w.window, ring=w.ring,
                         n_blocks_max=w.n_blocks_max, kv_dtype=w.kv_dtype, q_dtype=w.q_dtype,
                         deterministic=deterministic)


class ScoredDecoder:
    def __init__(self, w: Workload, evict: bool = False, device="cuda", layers: int | None = None,
                 compact: bool = False, compact_every: int = 1, fused: bool = True, tap: bool = True,
                 deterministic: bool = False):
        if compact and (w.ring or w.window or not w.select):
            raise ValueError("compaction needs a linear cache with selection and no window")
        if compact_every < 1:
            raise ValueError("compact_every must be at least 1")
        self.w = w
        self.evict = evict
        self.compact = compact
        self.compact_every = compact_every
        self.fused = fused
        self.tap = tap
        self.device = torch.device(device)
        self.geom = geom_of(w, deterministic)
        self.n_layers = w.n_layers if layers is None else layers
        self.caches = [api.KVCache(self.geom, device) for _ in range(self.n_layers)]
        self.workspace = api.decode_workspace(self.geom, device)
        # tap mode: one workspace per layer, read once per step by tap_masses
        self.workspaces = ([api.decode_workspace(self.geom, device) for _ in range(self.n_layers)]
                           if tap else [])
        B, nb = w.batch, self.geom.nb
        f32 = dict(dtype=torch.float32, device=device)
        self.mass = torch.zeros((B, nb), **f32)
        self.attended = torch.zeros((B, nb), **f32)
        self.ema = torch.zeros((B, nb), **f32)
        self.cum = torch.zeros((B, nb), **f32)
        self.traj = torch.zeros((B, w.traj_cap, nb), **f32)
        self.keep = torch.full((B, self.geom.words), -1, dtype=torch.int32, device=device)
        self.sel_ids = torch.zeros((B, nb), dtype=torch.int32, device=device)
        self.n_sel = torch.zeros((B,), dtype=torch.int32, device=device)
        qdt = api.TORCH_DTYPES[w.q_dtype]
        self.out = [torch.empty((B, w.n_q_heads, w.head_dim), dtype=qdt, device=device)
                    for _ in range(self.n_layers)]
        self.row_seq = torch.arange(B, dtype=torch.int32, device=device)
        self.step_index = 0
        # compact mode: each sequence's next position in its compacted cache
        self.pos = torch.full((B,), w.context, dtype=torch.int32, device=device)

    def prefill(self, layer: int, seq: int, k_rows: torch.Tensor, v_rows: torch.Tensor, pos0: int = 0):
        n = k_rows.shape[0]
        seqs = torch.full((n,), seq, dtype=torch.int32, device=self.device)
        pos = torch.arange(pos0, pos0 + n, dtype=torch.int32, device=self.device)
        self.caches[layer].append(k_rows, v_rows, seqs, pos)

    def attend_layer(self, layer: int, q: torch.Tensor, cur_pos: torch.Tensor, scored: bool = True):
        keep = self.keep if (self.evict and not self.w.window) else None
        api.decode_attn_scored(self.caches[layer], q, cur_pos, self.out[layer], self.workspace,
                               mass_accum=self.mass if scored else None, keep_mask=keep)

    def step(self, q_layers, k_layers, v_layers, cur_pos: torch.Tensor):
        """One decode step. ``q_layers[l]`` is [B, Hq, d]; ``k_layers[l]`` and
        ``v_layers[l]`` are the new position's rows [B, Hkv*d]; ``cur_pos`` is
        the int32 [B] absolute position being written and read. Fused tap
        mode makes it one library call (kvs_decode_step)."""
        if self.fused and self.tap:
            api.decode_step(self.caches, q_layers, cur_pos, self.out, self.workspaces, k_new=k_layers,
                            v_new=v_layers, keep_mask=self._attn_keep(), mass_accum=self.mass,
                            turn=self.turn_args())
            self.step_index += 1
            return
        for l in range(self.n_layers):
            self.append_attend_layer(l, q_layers[l], k_layers[l], v_layers[l], cur_pos)
        self._finish(cur_pos)

    def attend_layers(self, q_layers, k_layers, v_layers, cur_pos: torch.Tensor):
        """Fused tap mode: every layer's append and scored attention in one
        library call, the block sums left in the layers' workspaces; the step
        goes on with ``finish_step``."""
        if not (self.fused and self.tap):
            raise RuntimeError("attend_layers needs fused tap mode")
        api.decode_step(self.caches, q_layers, cur_pos, self.out, self.workspaces, k_new=k_layers,
                        v_new=v_layers, keep_mask=self._attn_keep())

    def _attn_keep(self):
        return self.keep if (self.evict and not self.w.window) else None

    def turn_args(self) -> api.Turn:
        """The side-car (and selection) arguments closing the current turn."""
        w = self.w
        return api.Turn(self.attended, self.ema, self.cum, self.traj, step=self.step_index, alpha=w.alpha,
                        select=bool(w.select), budget_blocks=w.budget_blocks, recent_tokens=w.recent_tokens,
                        sink_tokens=w.sink_tokens, alive=self.keep if self.evict else None,
                        keep_out=self.keep, sel_ids=self.sel_ids, n_sel=self.n_sel)

    def capture_step(self, q_layers, k_layers, v_layers, cur_pos: torch.Tensor, step_index: int | None = None,
                     split: bool = False):
        """Record one whole decode step as HIP graphs, without running it:
        every layer's append and scored attention, the mass combine, the
        side-car update and the selection, exactly the launches ``step``
        makes, with the trajectory slot of turn ``step_index`` (default: the
        next turn). Returns a ``CapturedStep``; its ``replay()`` performs the
        step on the tensors given here (their contents may change, their
        addresses may not). With ``split`` the layers' launches and the rest
        of the step are two graphs (``replay_layers``, ``replay_rest``), so a
        caller can time the layers alone. The step makes no allocation,
        memset or synchronisation, so the graphs hold kernel nodes only."""
        idx = self.step_index if step_index is None else step_index
        keep_idx = self.step_index
        graphs = []
        try:
            self.step_index = idx
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if self.fused and self.tap:
                    self.attend_layers(q_layers, k_layers, v_layers, cur_pos)
                else:
                    for l in range(self.n_layers):
                        self.append_attend_layer(l, q_layers[l], k_layers[l], v_layers[l], cur_pos)
                if not split:
                    self._finish(cur_pos)
            graphs.append(g)
            if split:
                self.step_index = idx
                g2 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g2):
                    self._finish(cur_pos)
                graphs.append(g2)
        finally:
            self.step_index = keep_idx
        return CapturedStep(self, graphs, idx)

    def finish_masses(self, cur_pos: torch.Tensor):
        """Tap mode: add every layer's block masses into ``mass`` (one call)."""
        if self.tap:
            api.tap_masses(self.geom, self.workspaces, cur_pos, mass_accum=self.mass)

    def finish_step(self, cur_pos: torch.Tensor):
        """Tap mode: ``finish_masses`` then ``close_turn`` as one library call
        (kvs_close_step: without selection the side-car update runs in the
        mass combine's launch)."""
        if not self.tap:
            raise RuntimeError("finish_step needs tap mode")
        api.close_step(self.geom, self.workspaces, cur_pos, self.mass, self.turn_args())
        self.step_index += 1

    def append_attend_layer(self, layer: int, q, k_rows, v_rows, cur_pos: torch.Tensor,
                            keep: torch.Tensor | None = None, use_own_keep: bool = True):
        """Append row b of ``k_rows`` / ``v_rows`` at ``cur_pos[b]``, then the
        scored attention of ``layer`` (one launch pair when fused)."""
        if use_own_keep:
            keep = self.keep if (self.evict and not self.w.window) else None
        if self.tap:
            if self.fused:
                api.decode_attn_tap(self.caches[layer], q, cur_pos, self.out[layer], self.workspaces[layer],
                                    keep_mask=keep, k_new=k_rows, v_new=v_rows)
            else:
                self.caches[layer].append(k_rows, v_rows, self.row_seq, cur_pos)
                api.decode_attn_tap(self.caches[layer], q, cur_pos, self.out[layer], self.workspaces[layer],
                                    keep_mask=keep)
            return
        if self.fused:
            api.append_decode_attn(self.caches[layer], k_rows, v_rows, q, cur_pos, self.out[layer],
                                   self.workspace, mass_accum=self.mass, keep_mask=keep)
        else:
            self.caches[layer].append(k_rows, v_rows, self.row_seq, cur_pos)
            api.decode_attn_scored(self.caches[layer], q, cur_pos, self.out[layer], self.workspace,
                                   mass_accum=self.mass, keep_mask=keep)

    def step_compact(self, q_layers, k_layers, v_layers, compact_now: bool | None = None):
        """One decode step in compact mode: evict mode at each sequence's
        compacted position (dropped blocks are masked out of the reads), and
        every ``compact_every`` steps the kept blocks and their side-car
        entries move to the front of every layer's cache, which frees the
        dropped blocks' slots (H2O step 4)."""
        cur = self.pos
        for l in range(self.n_layers):
            self.append_attend_layer(l, q_layers[l], k_layers[l], v_layers[l], cur, keep=self.keep,
                                     use_own_keep=False)
        self.finish_masses(cur)
        api.update_sidecar_select(self.mass, self.attended, self.ema, self.cum, self.traj, self.step_index,
                                  self.w.alpha, cur, self.w.budget_blocks, self.w.recent_tokens,
                                  self.w.sink_tokens, alive=self.keep, keep_mask=self.keep,
                                  sel_ids=self.sel_ids, n_sel=self.n_sel)
        self.step_index += 1
        if compact_now is None:
            compact_now = self.step_index % self.compact_every == 0
        if not compact_now:
            self.pos = cur + 1
            return
        side = (self.attended, self.ema, self.cum, self.traj)
        for l in range(self.n_layers):
            # the side-car arrays move once, with the last layer's cache
            api.compact_blocks(self.caches[l], self.sel_ids, self.n_sel,
                               tables=side if l == self.n_layers - 1 else ())
        self.keep.fill_(-1)                      # every block of the compacted cache is alive
        # the current block is always kept last: same offset inside it
        self.pos = ((self.n_sel - 1) * 16 + cur % 16 + 1).to(torch.int32)

    def _finish(self, cur_pos: torch.Tensor):
        if self.tap:
            self.finish_step(cur_pos)
        else:
            self.finish_masses(cur_pos)
            self.close_turn(cur_pos)

    def close_turn(self, cur_pos: torch.Tensor):
        if self.w.select:
            # side-car update and selection on the updated Cumulative, one launch
            alive = self.keep if self.evict else None
            api.update_sidecar_select(self.mass, self.attended, self.ema, self.cum, self.traj,
                                      self.step_index, self.w.alpha, cur_pos, self.w.budget_blocks,
                                      self.w.recent_tokens, self.w.sink_tokens, alive=alive,
                                      keep_mask=self.keep, sel_ids=self.sel_ids, n_sel=self.n_sel)
        else:
            api.update_sidecar(self.mass, self.attended, self.ema, self.cum, self.traj,
                               self.step_index, self.w.alpha)
        self.step_index += 1


class CapturedStep:
    """One decode step recorded by ``ScoredDecoder.capture_step``. Replay it
    once, when the decoder is at the turn it was recorded for; the decoder's
    turn count then advances as after ``step``."""

    def __init__(self, dec: ScoredDecoder, graphs, step_index: int):
        self.dec, self.graphs, self.step_index = dec, graphs, step_index

    def _check(self):
        if self.dec.step_index != self.step_index:
            raise RuntimeError(f"step recorded for turn {self.step_index}, decoder is at turn {self.dec.step_index}")

    def replay(self):
        self._check()
        for g in self.graphs:
            g.replay()
        self.dec.step_index += 1

    def replay_layers(self):
        """Split recordings: the layers' launches only (follow with replay_rest)."""
        self._check()
        self.graphs[0].replay()

    def replay_rest(self):
        self._check()
        self.graphs[1].replay()
        self.dec.step_index += 1
