"""Thin ctypes binding of libkvs (include/kvs.h).

Argument marshalling only: every computation runs in the library's HIP
kernels. Tensors are torch device tensors; each call passes their
``data_ptr()`` and ``torch.cuda.current_stream()`` to the C ABI and raises
``KvsError`` on a non-zero status. Importing this module loads
``libkvs.so`` and fails loudly if it has not been built
(``python -m heavy_hitter_eviction_amd.build``).
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvs.so")

KVS_OK, KVS_EINVAL, KVS_EDTYPE, KVS_EALIGN, KVS_EWS, KVS_EHIP, KVS_ENOTIMPL, KVS_ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 16 << 20
KVS_F32, KVS_BF16, KVS_FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"f32": KVS_F32, "bf16": KVS_BF16, "fp8": KVS_FP8_E4M3}
TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}

EXPORTED = (
    "kvs_cache_bytes", "kvs_encode_fp8", "kvs_append_kv", "kvs_decode_workspace_bytes",
    "kvs_decode_workspace_init",
    "kvs_decode_attn_scored", "kvs_decode_attn_scored_noalloc", "kvs_decode_partial", "kvs_decode_combine", "kvs_append_decode_attn",
    "kvs_append_decode_partial", "kvs_decode_attn_tap", "kvs_append_decode_attn_tap", "kvs_tap_masses",
    "kvs_decode_attn_profiled",
    "kvs_reattend_blocks",
    "kvs_update_sidecar", "kvs_update_counters", "kvs_filter_blocks", "kvs_select_blocks",
    "kvs_update_sidecar_select", "kvs_decode_step", "kvs_close_step", "kvs_compact_blocks", "kvs_stream_read", "kvs_snapkv_workspace_bytes", "kvs_snapkv_scores", "kvs_status_str",
    "kvs_version",
)


class KvsError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call} failed: {status} ({status_str(status)})")
        self.status = status


class BlockTable(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int32)]


class Geom(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32), ("window", ctypes.c_int32),
        ("ring", ctypes.c_int32), ("n_blocks_max", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("deterministic", ctypes.c_int32),
    ]


class LayerBufs(ctypes.Structure):
    """``kvs_layer_bufs``: one layer's device buffers for kvs_decode_step."""
    _fields_ = [("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("pos_of_slot", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p)]


class TurnArgs(ctypes.Structure):
    """``kvs_turn_args``: the side-car update (and selection) closing a step."""
    _fields_ = [("attended", ctypes.c_void_p), ("ema", ctypes.c_void_p), ("cum", ctypes.c_void_p),
                ("traj", ctypes.c_void_p), ("traj_cap", ctypes.c_int32), ("select", ctypes.c_int32),
                ("step", ctypes.c_int64), ("alpha", ctypes.c_float), ("score_source", ctypes.c_int32),
                ("alive", ctypes.c_void_p), ("budget_blocks", ctypes.c_int32), ("recent_tokens", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("keep_out", ctypes.c_void_p), ("sel_ids", ctypes.c_void_p),
                ("n_sel", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkvs.so not built at {LIB_PATH}; run python -m heavy_hitter_eviction_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    G = ctypes.POINTER(Geom)
    SZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "kvs_cache_bytes": [G, SZP, SZP, SZP],
        "kvs_encode_fp8": [P, I32, I64, I32, P, P, P],
        "kvs_append_kv": [G, P, P, I32, I32, P, P, P, P, P, P, P, P],
        "kvs_decode_workspace_bytes": [G, SZP],
        "kvs_decode_workspace_init": [G, P, SZ, P],
        "kvs_decode_attn_scored": [G, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_decode_attn_scored_noalloc": [G, P, P, P, P, P, P, P, P, P, P, P],
        "kvs_decode_partial": [G, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_decode_combine": [G, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_append_decode_attn": [G, P, P, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_append_decode_partial": [G, P, P, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_decode_attn_tap": [G, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_append_decode_attn_tap": [G, P, P, I32, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_tap_masses": [G, P, I32, SZ, P, P, P, P, P],
        "kvs_reattend_blocks": [G, P, P, P, P, P, P, P, P, I32, P, P, P, SZ, P],
        "kvs_decode_attn_profiled": [G, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "kvs_update_sidecar": [P, P, P, P, P, I32, I32, I32, I64, F, P],
        "kvs_update_counters": [P, P, P, P, P, I32, I32, I32, F, F, I32, P],
        "kvs_filter_blocks": [P, P, P, I32, I32, F, P, P, I32, P],
        "kvs_compact_blocks": [G, P, P, P, P, P, P, I32, P, I32, P],
        "kvs_snapkv_workspace_bytes": [G, I32, SZP],
        "kvs_snapkv_scores": [G, P, I32, P, P, P, P, P, I32, P, SZ, P],
        "kvs_select_blocks": [P, P, P, I32, I32, I32, I32, I32, P, P, P, P],
        "kvs_stream_read": [P, SZ, P, I32, P],
        "kvs_update_sidecar_select": [P, P, P, P, P, I32, I32, I32, I64, F, I32, P, P, I32, I32, I32, P, P, P, P],
        "kvs_decode_step": [G, I32, ctypes.POINTER(LayerBufs), I32, P, P, SZ, P, ctypes.POINTER(TurnArgs), P],
        "kvs_close_step": [G, P, I32, SZ, P, P, ctypes.POINTER(TurnArgs), P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.kvs_status_str.argtypes = [ctypes.c_int]
    lib.kvs_status_str.restype = ctypes.c_char_p
    lib.kvs_version.argtypes = []
    lib.kvs_version.restype = ctypes.c_char_p
    return lib


LIB = _load()


def status_str(status: int) -> str:
    return LIB.kvs_status_str(int(status)).decode()


def version() -> str:
    return LIB.kvs_version().decode()


def _check(status: int, call: str):
    if status != KVS_OK:
        raise KvsError(status, call)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor or None")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def _device_check(*tensors):
    for t in tensors:
        if t is not None and t.device.type != "cuda":
            raise ValueError("libkvs works on device tensors only")


@dataclass(frozen=True)
class CacheGeom:
    """Python mirror of ``kvs_geom``."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    window: int = 0
    ring: bool = False
    n_blocks_max: int = 0
    kv_dtype: str = "bf16"
    q_dtype: str = "bf16"
    softmax_scale: float = 0.0
    deterministic: bool = False

    def c(self) -> Geom:
        """The ``kvs_geom`` struct (built once; the library only reads it)."""
        g = self.__dict__.get("_c")
        if g is None:
            nb = self.n_blocks_max or self.capacity // 16
            scale = self.softmax_scale or float(torch.tensor(self.head_dim, dtype=torch.float64).rsqrt())
            g = Geom(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.capacity,
                     self.window, int(self.ring), nb, DTYPE_CODES[self.kv_dtype],
                     DTYPE_CODES[self.q_dtype], scale, int(self.deterministic))
            object.__setattr__(self, "_c", g)  # frozen dataclass: a cache, not a field
        return g

    @property
    def nb(self) -> int:
        return self.n_blocks_max or self.capacity // 16

    @property
    def words(self) -> int:
        return (self.nb + 31) // 32


def cache_bytes(geom: CacheGeom):
    kv, sc, pos = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(LIB.kvs_cache_bytes(ctypes.byref(geom.c()), ctypes.byref(kv), ctypes.byref(sc),
                               ctypes.byref(pos)), "kvs_cache_bytes")
    return kv.value, sc.value, pos.value


def decode_workspace_bytes(geom: CacheGeom) -> int:
    n = ctypes.c_size_t()
    _check(LIB.kvs_decode_workspace_bytes(ctypes.byref(geom.c()), ctypes.byref(n)),
           "kvs_decode_workspace_bytes")
    return n.value


def decode_workspace_init(geom: CacheGeom, workspace: torch.Tensor, stream=None):
    """kvs_decode_workspace_init: ready ``workspace`` for calls with ``geom``
    (needed once after allocation and again after use with another geometry)."""
    _device_check(workspace)
    _check(LIB.kvs_decode_workspace_init(ctypes.byref(geom.c()), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "kvs_decode_workspace_init")
    return workspace


def decode_workspace(geom: CacheGeom, device="cuda", stream=None) -> torch.Tensor:
    """A new decode workspace for ``geom``, initialised on the stream."""
    ws = torch.empty(decode_workspace_bytes(geom), dtype=torch.uint8, device=device)
    return decode_workspace_init(geom, ws, stream)


def encode_fp8(src: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
               stream=None):
    """Per-row E4M3 encoding of ``src [rows, n]`` (float32 or bfloat16)."""
    _device_check(src)
    if src.dim() != 2:
        raise ValueError("src must be [rows, row_len]")
    rows, n = src.shape
    dt = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16}.get(src.dtype)
    if dt is None:
        raise TypeError("src must be float32 or bfloat16")
    if codes is None:
        codes = torch.empty((rows, n), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=src.device)
    _check(LIB.kvs_encode_fp8(_ptr(src), dt, rows, n, _ptr(codes), _ptr(scales), _stream(stream)),
           "kvs_encode_fp8")
    return codes, scales


class KVCache:
    """One layer's KV cache allocated with the sizes libkvs reports."""

    def __init__(self, geom: CacheGeom, device="cuda"):
        self.geom = geom
        kv, sc, pos = cache_bytes(geom)
        elt = TORCH_DTYPES[geom.kv_dtype]
        n = kv // torch.empty((), dtype=elt).element_size()
        self.k = torch.empty(n, dtype=elt, device=device)
        self.v = torch.empty(n, dtype=elt, device=device)
        self.k_scale = torch.zeros(sc // 4, dtype=torch.float32, device=device) if sc else None
        self.v_scale = torch.zeros(sc // 4, dtype=torch.float32, device=device) if sc else None
        self.pos_of_slot = torch.full((pos // 4,), -1, dtype=torch.int32, device=device) if pos else None

    def append(self, k_rows, v_rows, row_seq, row_pos, stream=None):
        """Write rows ``[n, Hkv*d]`` at (sequence, absolute position) pairs."""
        _device_check(k_rows, v_rows, row_seq, row_pos)
        dt = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16}.get(k_rows.dtype)
        if dt is None or v_rows.dtype != k_rows.dtype:
            raise TypeError("rows must be float32 or bfloat16, K and V alike")
        if row_seq.dtype != torch.int32 or row_pos.dtype != torch.int32:
            raise TypeError("row_seq and row_pos must be int32")
        n = k_rows.shape[0]
        w = self.geom.n_kv_heads * self.geom.head_dim
        if k_rows.shape != (n, w) or v_rows.shape != (n, w) or row_seq.numel() != n or row_pos.numel() != n:
            raise ValueError("row shapes do not match the geometry")
        g = self.geom.c()
        _check(LIB.kvs_append_kv(ctypes.byref(g), _ptr(k_rows), _ptr(v_rows), dt, n, _ptr(row_seq),
                                 _ptr(row_pos), _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                                 _ptr(self.v_scale), _ptr(self.pos_of_slot), _stream(stream)),
               "kvs_append_kv")


def decode_attn_scored(cache: KVCache, q: torch.Tensor, cur_pos: torch.Tensor, out: torch.Tensor,
                       workspace: torch.Tensor, mass_accum: torch.Tensor | None = None,
                       keep_mask: torch.Tensor | None = None, stream=None, phase: str = "both"):
    """One layer of the scored decode step (kvs_decode_attn_scored). ``phase``
    "partial" or "combine" runs one of its two phases (kvs_decode_partial,
    kvs_decode_combine)."""
    g = cache.geom
    _device_check(q, cur_pos, out, workspace, mass_accum, keep_mask)
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if mass_accum is not None and (mass_accum.dtype != torch.float32 or mass_accum.numel() != g.batch * g.nb):
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    if keep_mask is not None and (keep_mask.dtype != torch.int32 or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    ws_bytes = workspace.numel() * workspace.element_size()
    gc = g.c()
    fn = {"both": LIB.kvs_decode_attn_scored, "partial": LIB.kvs_decode_partial,
          "combine": LIB.kvs_decode_combine}[phase]
    _check(fn(ctypes.byref(gc), _ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale),
              _ptr(cache.v_scale), _ptr(cache.pos_of_slot), _ptr(cur_pos), _ptr(keep_mask), _ptr(out),
              _ptr(mass_accum), _ptr(workspace), ws_bytes, _stream(stream)),
           f"kvs_decode ({phase})")
    return out


def decode_attn_scored_noalloc(cache: KVCache, q: torch.Tensor, cur_pos: torch.Tensor, out: torch.Tensor,
                               mass_accum: torch.Tensor | None = None, keep_mask: torch.Tensor | None = None,
                               stream=None):
    """kvs_decode_attn_scored_noalloc: decode_attn_scored with the library's
    static per-GPU scratch as workspace (no allocation; overlapping calls on
    one GPU race)."""
    g = cache.geom
    _device_check(q, cur_pos, out, mass_accum, keep_mask)
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if mass_accum is not None and (mass_accum.dtype != torch.float32 or mass_accum.numel() != g.batch * g.nb):
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    if keep_mask is not None and (keep_mask.dtype != torch.int32 or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    gc = g.c()
    _check(LIB.kvs_decode_attn_scored_noalloc(ctypes.byref(gc), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                              _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(cache.pos_of_slot),
                                              _ptr(cur_pos), _ptr(keep_mask), _ptr(out), _ptr(mass_accum),
                                              _stream(stream)),
           "kvs_decode_attn_scored_noalloc")
    return out


def append_decode_attn(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                       cur_pos: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                       mass_accum: torch.Tensor | None = None, keep_mask: torch.Tensor | None = None,
                       stream=None, phase: str = "both"):
    """kvs_append_decode_attn: write row b of ``k_new`` / ``v_new`` ([B, Hkv*d],
    float32 or bfloat16) at position ``cur_pos[b]`` and run the scored decode
    step over the cache that now holds it, in one pass. ``phase`` "partial"
    runs kvs_append_decode_partial only (append + partial phase); follow it
    with ``decode_attn_scored(..., phase="combine")``."""
    g = cache.geom
    _device_check(k_new, v_new, q, cur_pos, out, workspace, mass_accum, keep_mask)
    dt = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16}.get(k_new.dtype)
    if dt is None or v_new.dtype != k_new.dtype:
        raise TypeError("new rows must be float32 or bfloat16, K and V alike")
    w = g.n_kv_heads * g.head_dim
    if k_new.shape != (g.batch, w) or v_new.shape != (g.batch, w):
        raise ValueError("new rows must be [B, Hkv*d]")
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if mass_accum is not None and (mass_accum.dtype != torch.float32 or mass_accum.numel() != g.batch * g.nb):
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    if keep_mask is not None and (keep_mask.dtype != torch.int32 or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    fn = {"both": LIB.kvs_append_decode_attn, "partial": LIB.kvs_append_decode_partial}[phase]
    ws_bytes = workspace.numel() * workspace.element_size()
    gc = g.c()
    _check(fn(ctypes.byref(gc), _ptr(k_new), _ptr(v_new), dt, _ptr(q), _ptr(cache.k), _ptr(cache.v),
              _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(cache.pos_of_slot), _ptr(cur_pos),
              _ptr(keep_mask), _ptr(out), _ptr(mass_accum), _ptr(workspace), ws_bytes, _stream(stream)),
           f"kvs_append_decode ({phase})")
    return out


def decode_attn_tap(cache: KVCache, q: torch.Tensor, cur_pos: torch.Tensor, out: torch.Tensor,
                    workspace: torch.Tensor, keep_mask: torch.Tensor | None = None, stream=None,
                    k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None):
    """kvs_decode_attn_tap (or, with ``k_new`` / ``v_new``, kvs_append_decode_attn_tap):
    the layer's output, and its per-block sums left in ``workspace`` for
    :func:`tap_masses`. ``workspace`` is this layer's own."""
    g = cache.geom
    _device_check(q, cur_pos, out, workspace, keep_mask, k_new, v_new)
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if keep_mask is not None and (keep_mask.dtype != torch.int32 or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    ws_bytes = workspace.numel() * workspace.element_size()
    gc = g.c()
    if k_new is None:
        _check(LIB.kvs_decode_attn_tap(ctypes.byref(gc), _ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale),
                                       _ptr(cache.v_scale), _ptr(cache.pos_of_slot), _ptr(cur_pos),
                                       _ptr(keep_mask), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
               "kvs_decode_attn_tap")
        return out
    dt = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16}.get(k_new.dtype)
    if dt is None or v_new is None or v_new.dtype != k_new.dtype:
        raise TypeError("new rows must be float32 or bfloat16, K and V alike")
    w = g.n_kv_heads * g.head_dim
    if k_new.shape != (g.batch, w) or v_new.shape != (g.batch, w):
        raise ValueError("new rows must be [B, Hkv*d]")
    _check(LIB.kvs_append_decode_attn_tap(ctypes.byref(gc), _ptr(k_new), _ptr(v_new), dt, _ptr(q), _ptr(cache.k),
                                          _ptr(cache.v), _ptr(cache.k_scale), _ptr(cache.v_scale),
                                          _ptr(cache.pos_of_slot), _ptr(cur_pos), _ptr(keep_mask), _ptr(out),
                                          _ptr(workspace), ws_bytes, _stream(stream)),
           "kvs_append_decode_attn_tap")
    return out


def tap_masses(geom: CacheGeom, workspaces, cur_pos: torch.Tensor, mass_accum: torch.Tensor | None = None,
               head_mass: torch.Tensor | None = None, mass_max: torch.Tensor | None = None, stream=None):
    """kvs_tap_masses: add the block masses the per-layer tap calls left in
    ``workspaces`` (one per layer, in call order)."""
    _device_check(cur_pos, mass_accum, head_mass, mass_max, *workspaces)
    if not workspaces:
        raise ValueError("need at least one layer workspace")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != geom.batch:
        raise ValueError("cur_pos must be int32 [B]")
    for t, shape in ((mass_accum, (geom.batch, geom.nb)), (mass_max, (geom.batch, geom.nb)),
                     (head_mass, (geom.batch, geom.n_q_heads, geom.nb))):
        if t is not None and (t.dtype != torch.float32 or t.numel() != math.prod(shape)):
            raise ValueError(f"mass outputs must be float32 {shape}")
    ws_bytes = min(w.numel() * w.element_size() for w in workspaces)
    arr = (ctypes.c_void_p * len(workspaces))(*[w.data_ptr() for w in workspaces])
    gc = geom.c()
    _check(LIB.kvs_tap_masses(ctypes.byref(gc), arr, len(workspaces), ws_bytes, _ptr(cur_pos), _ptr(mass_accum),
                              _ptr(head_mass), _ptr(mass_max), _stream(stream)), "kvs_tap_masses")


@dataclass
class Turn:
    """The side-car arrays and selection arguments that close a decode step
    (``kvs_turn_args``); ``select=False`` updates the side-car only."""
    attended: torch.Tensor
    ema: torch.Tensor
    cum: torch.Tensor
    traj: torch.Tensor | None
    step: int
    alpha: float
    select: bool = True
    budget_blocks: int = 0
    recent_tokens: int = 1
    sink_tokens: int = 0
    score: str = "cumulative"
    alive: torch.Tensor | None = None
    keep_out: torch.Tensor | None = None
    sel_ids: torch.Tensor | None = None
    n_sel: torch.Tensor | None = None


def _turn_args(turn: Turn, B: int, nb: int) -> TurnArgs:
    words = (nb + 31) // 32
    for t in (turn.attended, turn.ema, turn.cum):
        if t.device.type != "cuda" or t.dtype != torch.float32 or t.numel() != B * nb:
            raise ValueError("side-car arrays must be float32 [B, NBmax] device tensors")
    traj_cap = 1
    if turn.traj is not None:
        if turn.traj.device.type != "cuda" or turn.traj.dtype != torch.float32 or turn.traj.dim() != 3 \
                or turn.traj.shape[0] != B or turn.traj.shape[2] != nb:
            raise ValueError("traj must be float32 [B, traj_cap, NBmax]")
        traj_cap = turn.traj.shape[1]
    a = TurnArgs()
    a.attended, a.ema, a.cum = turn.attended.data_ptr(), turn.ema.data_ptr(), turn.cum.data_ptr()
    a.traj = turn.traj.data_ptr() if turn.traj is not None else None
    a.traj_cap, a.step, a.alpha, a.select = traj_cap, int(turn.step), float(turn.alpha), int(bool(turn.select))
    if turn.select:
        if turn.score not in SCORE_SOURCES:
            raise ValueError(f"score must be one of {sorted(SCORE_SOURCES)}")
        for t, n in ((turn.keep_out, B * words), (turn.sel_ids, B * nb), (turn.n_sel, B)):
            if t is None or t.device.type != "cuda" or t.dtype != torch.int32 or t.numel() != n:
                raise ValueError("keep_out [B, W], sel_ids [B, NBmax] and n_sel [B] must be int32 device tensors")
        if turn.alive is not None and (turn.alive.device.type != "cuda" or turn.alive.dtype != torch.int32
                                       or turn.alive.numel() != B * words):
            raise ValueError("alive must be int32 bit words [B, W]")
        a.score_source = SCORE_SOURCES[turn.score]
        a.alive = turn.alive.data_ptr() if turn.alive is not None else None
        a.budget_blocks, a.recent_tokens, a.sink_tokens = int(turn.budget_blocks), int(turn.recent_tokens), \
            int(turn.sink_tokens)
        a.keep_out, a.sel_ids, a.n_sel = turn.keep_out.data_ptr(), turn.sel_ids.data_ptr(), turn.n_sel.data_ptr()
    return a


def decode_step(caches, q_layers, cur_pos: torch.Tensor, outs, workspaces, k_new=None, v_new=None,
                keep_mask: torch.Tensor | None = None, mass_accum: torch.Tensor | None = None,
                turn: Turn | None = None, stream=None):
    """kvs_decode_step: for every layer ``l`` the append of ``k_new[l]`` /
    ``v_new[l]`` (lists, or None: nothing appended) and the scored attention
    of ``q_layers[l]`` into ``outs[l]``, leaving its block sums in
    ``workspaces[l]``; then, with ``mass_accum``, the masses of all layers
    added once; then, with ``turn``, the side-car update and selection. One
    library call: the same launches and results as the per-layer calls,
    tap_masses and update_sidecar(_select)."""
    L = len(caches)
    if L < 1 or not (len(q_layers) == len(outs) == len(workspaces) == L):
        raise ValueError("one query, output and workspace per layer")
    if (k_new is None) != (v_new is None) or (k_new is not None and (len(k_new) != L or len(v_new) != L)):
        raise ValueError("k_new and v_new: both None or one row tensor per layer each")
    g = caches[0].geom
    qdt = TORCH_DTYPES[g.q_dtype]
    qshape = (g.batch, g.n_q_heads, g.head_dim)
    rshape = (g.batch, g.n_kv_heads * g.head_dim)
    if cur_pos.device.type != "cuda" or cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be an int32 [B] device tensor")
    if keep_mask is not None and (keep_mask.device.type != "cuda" or keep_mask.dtype != torch.int32
                                  or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    if mass_accum is not None and (mass_accum.device.type != "cuda" or mass_accum.dtype != torch.float32
                                   or mass_accum.numel() != g.batch * g.nb):
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    src = KVS_F32
    if k_new is not None:
        src = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16}.get(k_new[0].dtype)
        if src is None:
            raise TypeError("new rows must be float32 or bfloat16")
    arr = (LayerBufs * L)()
    ws_bytes = None
    for l in range(L):
        c, q, o, w = caches[l], q_layers[l], outs[l], workspaces[l]
        if c.geom != g:
            raise ValueError("every layer's cache must have the same geometry")
        for t in (q, o, w):
            if t.device.type != "cuda" or not t.is_contiguous():
                raise ValueError("q, out and workspace must be contiguous device tensors")
        if q.dtype != qdt or o.dtype != qdt or q.shape != qshape or o.shape != qshape:
            raise ValueError("q and out must be [B, Hq, d] of the geometry's q dtype")
        b = arr[l]
        b.q, b.out, b.workspace = q.data_ptr(), o.data_ptr(), w.data_ptr()
        nbytes = w.numel() * w.element_size()
        ws_bytes = nbytes if ws_bytes is None else min(ws_bytes, nbytes)
        b.k_cache, b.v_cache = c.k.data_ptr(), c.v.data_ptr()
        b.k_scale = c.k_scale.data_ptr() if c.k_scale is not None else None
        b.v_scale = c.v_scale.data_ptr() if c.v_scale is not None else None
        b.pos_of_slot = c.pos_of_slot.data_ptr() if c.pos_of_slot is not None else None
        if k_new is not None:
            kn, vn = k_new[l], v_new[l]
            for t in (kn, vn):
                if t.device.type != "cuda" or not t.is_contiguous() or t.shape != rshape \
                        or t.dtype != k_new[0].dtype:
                    raise ValueError("new rows must be contiguous [B, Hkv*d] device tensors of one dtype")
            b.k_new, b.v_new = kn.data_ptr(), vn.data_ptr()
    targs = None
    if turn is not None:
        if mass_accum is None:
            raise ValueError("closing the turn needs mass_accum")
        targs = ctypes.byref(_turn_args(turn, g.batch, g.nb))
    _check(LIB.kvs_decode_step(ctypes.byref(g.c()), L, arr, src, _ptr(cur_pos), _ptr(keep_mask), ws_bytes,
                               _ptr(mass_accum), targs, _stream(stream)), "kvs_decode_step")


def close_step(geom: CacheGeom, workspaces, cur_pos: torch.Tensor, mass_accum: torch.Tensor, turn: Turn,
               stream=None):
    """kvs_close_step: the layers' block masses (left in ``workspaces`` by a
    layers-only decode_step or the per-layer tap calls) added into
    ``mass_accum``, then the turn closed: the results of tap_masses followed
    by update_sidecar(_select), the side-car update in the combine's launch
    where it can."""
    _device_check(cur_pos, mass_accum, *workspaces)
    if not workspaces:
        raise ValueError("need at least one layer workspace")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != geom.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if mass_accum.dtype != torch.float32 or mass_accum.numel() != geom.batch * geom.nb:
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    ws_bytes = min(w.numel() * w.element_size() for w in workspaces)
    arr = (ctypes.c_void_p * len(workspaces))(*[w.data_ptr() for w in workspaces])
    targs = _turn_args(turn, geom.batch, geom.nb)
    _check(LIB.kvs_close_step(ctypes.byref(geom.c()), arr, len(workspaces), ws_bytes, _ptr(cur_pos),
                              _ptr(mass_accum), ctypes.byref(targs), _stream(stream)), "kvs_close_step")


def decode_attn_profiled(cache: KVCache, q: torch.Tensor, cur_pos: torch.Tensor, out: torch.Tensor,
                         workspace: torch.Tensor, mass_accum: torch.Tensor | None = None,
                         head_mass: torch.Tensor | None = None, mass_max: torch.Tensor | None = None,
                         keep_mask: torch.Tensor | None = None, stream=None):
    """kvs_decode_attn_profiled: the scored decode step with per-head block
    masses (``head_mass`` [B, Hq, NBmax], +=) and their running max over heads
    (``mass_max`` [B, NBmax])."""
    g = cache.geom
    _device_check(q, cur_pos, out, workspace, mass_accum, head_mass, mass_max, keep_mask)
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    for name, t, n in (("mass_accum", mass_accum, g.batch * g.nb), ("mass_max", mass_max, g.batch * g.nb),
                       ("head_mass", head_mass, g.batch * g.n_q_heads * g.nb)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 with {n} elements")
    if keep_mask is not None and (keep_mask.dtype != torch.int32 or keep_mask.numel() != g.batch * g.words):
        raise ValueError("keep_mask must be int32 (bit words) [B, W]")
    ws_bytes = workspace.numel() * workspace.element_size()
    gc = g.c()
    _check(LIB.kvs_decode_attn_profiled(ctypes.byref(gc), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                        _ptr(cache.k_scale), _ptr(cache.v_scale), _ptr(cache.pos_of_slot),
                                        _ptr(cur_pos), _ptr(keep_mask), _ptr(out), _ptr(mass_accum),
                                        _ptr(head_mass), _ptr(mass_max), _ptr(workspace), ws_bytes,
                                        _stream(stream)),
           "kvs_decode_attn_profiled")
    return out


def reattend_blocks(cache: KVCache, q: torch.Tensor, cur_pos: torch.Tensor, block_ids: torch.Tensor,
                    n_ids: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                    mass_accum: torch.Tensor | None = None, stream=None):
    """Attention of a new query over the listed blocks only (kvs_reattend_blocks):
    ``block_ids`` int32 [B, S] (any order, repeats allowed), ``n_ids`` int32 [B]."""
    g = cache.geom
    _device_check(q, cur_pos, block_ids, n_ids, out, workspace, mass_accum)
    qdt = TORCH_DTYPES[g.q_dtype]
    if q.dtype != qdt or out.dtype != qdt:
        raise TypeError("q and out must have the geometry's q dtype")
    if q.shape != (g.batch, g.n_q_heads, g.head_dim) or out.shape != q.shape:
        raise ValueError("q/out must be [B, Hq, d]")
    if cur_pos.dtype != torch.int32 or cur_pos.numel() != g.batch:
        raise ValueError("cur_pos must be int32 [B]")
    if block_ids.dtype != torch.int32 or block_ids.dim() != 2 or block_ids.shape[0] != g.batch \
            or not block_ids.is_contiguous():
        raise ValueError("block_ids must be contiguous int32 [B, S]")
    if n_ids.dtype != torch.int32 or n_ids.numel() != g.batch:
        raise ValueError("n_ids must be int32 [B]")
    if mass_accum is not None and (mass_accum.dtype != torch.float32 or mass_accum.numel() != g.batch * g.nb):
        raise ValueError("mass_accum must be float32 [B, NBmax]")
    ws_bytes = workspace.numel() * workspace.element_size()
    gc = g.c()
    _check(LIB.kvs_reattend_blocks(ctypes.byref(gc), _ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale),
                                   _ptr(cache.v_scale), _ptr(cur_pos), _ptr(block_ids), _ptr(n_ids),
                                   block_ids.shape[1], _ptr(out), _ptr(mass_accum), _ptr(workspace), ws_bytes,
                                   _stream(stream)),
           "kvs_reattend_blocks")
    return out


def update_counters(attended, ema, hot_count=None, cold_turns=None, traj=None, hot_theta: float = 0.0,
                    cold_theta: float = 0.0, cold_limit: int = 0, stream=None):
    """kvs_update_counters: Scissorhands hot counts and cold-turn trajectory GC."""
    _device_check(attended, ema, hot_count, cold_turns, traj)
    B, nb = attended.shape
    for name, t in (("hot_count", hot_count), ("cold_turns", cold_turns)):
        if t is not None and (t.dtype != torch.int32 or t.shape != (B, nb) or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous int32 [B, NBmax]")
    cap = traj.shape[1] if traj is not None else 0
    _check(LIB.kvs_update_counters(_ptr(attended), _ptr(ema), _ptr(hot_count), _ptr(cold_turns), _ptr(traj), B, nb,
                                   cap, hot_theta, cold_theta, cold_limit, _stream(stream)),
           "kvs_update_counters")


def filter_blocks(score, cur_pos, theta: float, ids, n_ids, alive=None, stream=None):
    """kvs_filter_blocks: ascending ids of existing, alive blocks with score > theta."""
    _device_check(score, cur_pos, ids, n_ids, alive)
    B, nb = score.shape
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[0] != B or not ids.is_contiguous():
        raise ValueError("ids must be contiguous int32 [B, S]")
    _check(LIB.kvs_filter_blocks(_ptr(score), _ptr(alive), _ptr(cur_pos), B, nb, theta, _ptr(ids), _ptr(n_ids),
                                 ids.shape[1], _stream(stream)),
           "kvs_filter_blocks")


def compact_blocks(cache: KVCache, keep_ids: torch.Tensor, n_keep: torch.Tensor, tables=(), stream=None):
    """kvs_compact_blocks: kept blocks (ascending ids [B, S], counts [B]) move
    to the front of the cache; ``tables`` are per-block arrays of 4-byte
    entries shaped [B, NBmax] or [B, rows, NBmax], compacted alike."""
    g = cache.geom
    if g.ring:
        raise ValueError("compaction applies to linear caches")
    _device_check(keep_ids, n_keep, *tables)
    if keep_ids.dtype != torch.int32 or keep_ids.dim() != 2 or keep_ids.shape[0] != g.batch \
            or not keep_ids.is_contiguous():
        raise ValueError("keep_ids must be contiguous int32 [B, S]")
    arr = (BlockTable * max(1, len(tables)))()
    for j, t in enumerate(tables):
        if t.element_size() != 4 or not t.is_contiguous() or t.shape[0] != g.batch or t.shape[-1] != g.nb:
            raise ValueError("tables must be contiguous 4-byte [B, (rows,) NBmax]")
        arr[j] = BlockTable(t.data_ptr(), 1 if t.dim() == 2 else int(t.shape[1]))
    _check(LIB.kvs_compact_blocks(ctypes.byref(g.c()), _ptr(cache.k), _ptr(cache.v), _ptr(cache.k_scale),
                                  _ptr(cache.v_scale), _ptr(keep_ids), _ptr(n_keep), keep_ids.shape[1],
                                  arr if tables else None, len(tables), _stream(stream)),
           "kvs_compact_blocks")


def snapkv_workspace_bytes(geom: CacheGeom, window: int) -> int:
    n = ctypes.c_size_t()
    _check(LIB.kvs_snapkv_workspace_bytes(ctypes.byref(geom.c()), window, ctypes.byref(n)),
           "kvs_snapkv_workspace_bytes")
    return n.value


def snapkv_scores(cache: KVCache, q_window: torch.Tensor, n_prompt: torch.Tensor, token_score: torch.Tensor,
                  workspace: torch.Tensor, block_score: torch.Tensor | None = None, pool_kernel: int = 7,
                  stream=None):
    """kvs_snapkv_scores: observation-window scores per (token, head) and
    max-pooled block scores (+=). ``q_window`` bf16 [B, W, Hq, d]."""
    g = cache.geom
    _device_check(q_window, n_prompt, token_score, workspace, block_score)
    if q_window.dtype != torch.bfloat16 or q_window.dim() != 4 or q_window.shape[0] != g.batch \
            or q_window.shape[2:] != (g.n_q_heads, g.head_dim) or not q_window.is_contiguous():
        raise ValueError("q_window must be contiguous bf16 [B, W, Hq, d]")
    if token_score.dtype != torch.float32 or token_score.numel() != g.batch * g.n_q_heads * g.capacity:
        raise ValueError("token_score must be float32 [B, Hq, C]")
    if block_score is not None and (block_score.dtype != torch.float32 or block_score.numel() != g.batch * g.nb):
        raise ValueError("block_score must be float32 [B, NBmax]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(LIB.kvs_snapkv_scores(ctypes.byref(g.c()), _ptr(q_window), q_window.shape[1], _ptr(cache.k),
                                 _ptr(cache.k_scale), _ptr(n_prompt), _ptr(token_score), _ptr(block_score),
                                 pool_kernel, _ptr(workspace), ws_bytes, _stream(stream)),
           "kvs_snapkv_scores")


def update_sidecar(mass_accum, attended, ema, cum, traj, step: int, alpha: float, stream=None):
    """Close one turn: Attended, EMA, Cumulative, trajectory ring; zero the accumulator."""
    _device_check(mass_accum, attended, ema, cum, traj)
    B, nb = attended.shape
    traj_cap = traj.shape[1] if traj is not None else 1
    for t in (mass_accum, ema, cum):
        if t.numel() != B * nb or t.dtype != torch.float32:
            raise ValueError("side-car arrays must be float32 [B, NBmax]")
    _check(LIB.kvs_update_sidecar(_ptr(mass_accum), _ptr(attended), _ptr(ema), _ptr(cum), _ptr(traj),
                                  B, nb, traj_cap, int(step), float(alpha), _stream(stream)),
           "kvs_update_sidecar")


def select_blocks(score, cur_pos, budget_blocks: int, recent_tokens: int, sink_tokens: int = 0,
                  alive=None, keep_mask=None, sel_ids=None, n_sel=None, stream=None):
    """Heavy-hitter block selection; returns (keep_mask, sel_ids, n_sel)."""
    _device_check(score, cur_pos, alive)
    B, nb = score.shape
    words = (nb + 31) // 32
    dev = score.device
    if keep_mask is None:
        keep_mask = torch.empty((B, words), dtype=torch.int32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, nb), dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=dev)
    if score.dtype != torch.float32 or cur_pos.dtype != torch.int32:
        raise TypeError("score float32, cur_pos int32")
    if alive is not None and (alive.dtype != torch.int32 or alive.numel() != B * words):
        raise ValueError("alive must be int32 bit words [B, W]")
    _check(LIB.kvs_select_blocks(_ptr(score), _ptr(alive), _ptr(cur_pos), B, nb, int(budget_blocks),
                                 int(recent_tokens), int(sink_tokens), _ptr(keep_mask), _ptr(sel_ids),
                                 _ptr(n_sel), _stream(stream)),
           "kvs_select_blocks")
    return keep_mask, sel_ids, n_sel


SCORE_SOURCES = {"cumulative": 0, "ema": 1, "attended": 2}


def update_sidecar_select(mass_accum, attended, ema, cum, traj, step: int, alpha: float, cur_pos,
                          budget_blocks: int, recent_tokens: int, sink_tokens: int = 0,
                          score: str = "cumulative", alive=None, keep_mask=None, sel_ids=None, n_sel=None,
                          stream=None):
    """update_sidecar then select_blocks on the updated ``score`` array
    ("cumulative", "ema" or "attended"), in one launch; returns (keep_mask,
    sel_ids, n_sel)."""
    _device_check(mass_accum, attended, ema, cum, traj, cur_pos, alive)
    B, nb = attended.shape
    traj_cap = traj.shape[1] if traj is not None else 1
    for t in (mass_accum, ema, cum):
        if t.numel() != B * nb or t.dtype != torch.float32:
            raise ValueError("side-car arrays must be float32 [B, NBmax]")
    if score not in SCORE_SOURCES:
        raise ValueError(f"score must be one of {sorted(SCORE_SOURCES)}")
    words = (nb + 31) // 32
    dev = attended.device
    if keep_mask is None:
        keep_mask = torch.empty((B, words), dtype=torch.int32, device=dev)
    if sel_ids is None:
        sel_ids = torch.empty((B, nb), dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty((B,), dtype=torch.int32, device=dev)
    if cur_pos.dtype != torch.int32:
        raise TypeError("cur_pos int32")
    if alive is not None and (alive.dtype != torch.int32 or alive.numel() != B * words):
        raise ValueError("alive must be int32 bit words [B, W]")
    _check(LIB.kvs_update_sidecar_select(_ptr(mass_accum), _ptr(attended), _ptr(ema), _ptr(cum), _ptr(traj),
                                         B, nb, traj_cap, int(step), float(alpha), SCORE_SOURCES[score],
                                         _ptr(alive), _ptr(cur_pos), int(budget_blocks), int(recent_tokens),
                                         int(sink_tokens), _ptr(keep_mask), _ptr(sel_ids), _ptr(n_sel),
                                         _stream(stream)),
           "kvs_update_sidecar_select")
    return keep_mask, sel_ids, n_sel


def stream_read(buf: torch.Tensor, sums: torch.Tensor, workgroups: int, stream=None):
    """kvs_stream_read: read every byte of ``buf`` once (the streaming-read
    probe); ``sums`` is uint32/int32 [workgroups]."""
    _device_check(buf, sums)
    if sums.numel() < workgroups or sums.element_size() != 4:
        raise ValueError("sums must hold one 32-bit word per workgroup")
    _check(LIB.kvs_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sums), workgroups,
                               _stream(stream)), "kvs_stream_read")
