"""The C ABI: the library loads, exports every entry point the header declares,
and its host-side checks reject bad arguments before anything is launched
(these calls never reach the GPU, so they run on any machine)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")


def _lib():
    from heavy_hitter_eviction_amd import build as B
    if not os.path.exists(B.OUT):
        B.build()
    from heavy_hitter_eviction_amd import api
    return api


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"KVS_API\s+[\w\s\*]+?\b(kvs_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    for n in ("kvs_encode_fp8", "kvs_decode_attn_scored", "kvs_update_sidecar", "kvs_select_blocks",
              "kvs_append_kv", "kvs_decode_workspace_bytes", "kvs_cache_bytes", "kvs_status_str",
              "kvs_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    api = _lib()
    for name in declared_functions():
        assert hasattr(api.LIB, name), name
    assert set(api.EXPORTED) == set(declared_functions())
    assert api.version().startswith("libkvs")
    assert api.status_str(api.KVS_EWS) == "workspace too small"


def _geom(api, **kw):
    base = dict(batch=2, n_q_heads=16, n_kv_heads=4, head_dim=128, capacity=256, window=0, ring=0,
                n_blocks_max=16, kv_dtype=api.KVS_BF16, q_dtype=api.KVS_BF16, softmax_scale=0.088388,
                deterministic=0)
    base.update(kw)
    return api.Geom(*[base[f] for f, _ in api.Geom._fields_])


def _decode(api, g, ws_bytes=1 << 20, **ptrs):
    P = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    d = dict(q=0x1000, k=0x2000, v=0x3000, ks=None, vs=None, pos=None, cur=0x4000, keep=None,
             out=0x5000, mass=0x6000, ws=0x7000)
    d.update(ptrs)
    return api.LIB.kvs_decode_attn_scored(ctypes.byref(g), P(d["q"]), P(d["k"]), P(d["v"]), P(d["ks"]),
                                          P(d["vs"]), P(d["pos"]), P(d["cur"]), P(d["keep"]),
                                          P(d["out"]), P(d["mass"]), P(d["ws"]), ws_bytes, None)


@pytest.mark.parametrize("field,value,code", [
    ("n_q_heads", 15, "KVS_EINVAL"),
    ("n_q_heads", 80, "KVS_ENOTIMPL"),      # group of 20 query heads per KV head
    ("capacity", 100, "KVS_EINVAL"),
    ("capacity", 0, "KVS_EINVAL"),
    ("window", -1, "KVS_EINVAL"),
    ("ring", 2, "KVS_EINVAL"),
    ("n_blocks_max", 8, "KVS_EINVAL"),      # linear cache needs NBmax >= C/16
    ("head_dim", 96, "KVS_EDTYPE"),
    ("q_dtype", 0, "KVS_EDTYPE"),           # bf16 cache with an f32 query
    ("kv_dtype", 7, "KVS_EDTYPE"),
    ("softmax_scale", 0.0, "KVS_EINVAL"),
    ("softmax_scale", float("inf"), "KVS_EINVAL"),
    ("deterministic", 2, "KVS_EINVAL"),
])
def test_bad_geometry_is_rejected(field, value, code):
    api = _lib()
    g = _geom(api, **{field: value})
    assert _decode(api, g) == getattr(api, code)
    n = ctypes.c_size_t()
    assert api.LIB.kvs_decode_workspace_bytes(ctypes.byref(g), ctypes.byref(n)) == getattr(api, code)


def test_dtype_flag_must_match_the_buffers():
    """Context Optimization, Flag Ordering: an FP8 cache without scale buffers,
    or a float cache handed scale buffers, is refused."""
    api = _lib()
    g = _geom(api, kv_dtype=api.KVS_FP8_E4M3)
    assert _decode(api, g) == api.KVS_EINVAL
    g = _geom(api)
    assert _decode(api, g, ks=0x8000, vs=0x9000) == api.KVS_EINVAL


def test_window_with_keep_mask_is_rejected_and_ring_needs_positions():
    api = _lib()
    assert _decode(api, _geom(api, window=64), keep=0xA000) == api.KVS_EINVAL
    assert _decode(api, _geom(api, ring=1)) == api.KVS_EINVAL
    assert _decode(api, _geom(api), pos=0xB000) == api.KVS_EINVAL


def test_alignment_and_workspace_checks():
    api = _lib()
    g = _geom(api)
    assert _decode(api, g, q=0x1004) == api.KVS_EALIGN
    assert _decode(api, g, mass=0x6008) == api.KVS_EALIGN
    need = ctypes.c_size_t()
    assert api.LIB.kvs_decode_workspace_bytes(ctypes.byref(g), ctypes.byref(need)) == 0
    assert need.value > 0
    assert _decode(api, g, ws_bytes=need.value - 1) == api.KVS_EWS
    assert _decode(api, g, cur=None) == api.KVS_EINVAL


def test_cache_bytes_closed_form():
    api = _lib()
    g = _geom(api, kv_dtype=api.KVS_FP8_E4M3, ring=1, n_blocks_max=64)
    kv, sc, pos = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert api.LIB.kvs_cache_bytes(ctypes.byref(g), ctypes.byref(kv), ctypes.byref(sc), ctypes.byref(pos)) == 0
    assert kv.value == 2 * 4 * 256 * 128 and sc.value == 2 * 256 * 4 and pos.value == 2 * 256 * 4


def test_other_entry_points_reject_bad_arguments():
    api = _lib()
    L = api.LIB
    vp = ctypes.c_void_p
    assert L.kvs_encode_fp8(vp(0x1000), 5, 4, 16, vp(0x2000), vp(0x3000), None) == api.KVS_EDTYPE
    assert L.kvs_encode_fp8(vp(0x1000), 0, -1, 16, vp(0x2000), vp(0x3000), None) == api.KVS_EINVAL
    assert L.kvs_encode_fp8(vp(0x1000), 0, 0, 16, vp(0x2000), vp(0x3000), None) == api.KVS_OK
    assert L.kvs_encode_fp8(vp(0x1001), 0, 4, 16, vp(0x2000), vp(0x3000), None) == api.KVS_EALIGN
    ok = [vp(0x1000)] * 5
    assert L.kvs_update_sidecar(*ok, 2, 16, 64, 0, 1.5, None) == api.KVS_EINVAL
    assert L.kvs_update_sidecar(*ok, 2, 16, 0, 0, 0.5, None) == api.KVS_EINVAL
    assert L.kvs_update_sidecar(*ok, 2, 16, 64, -1, 0.5, None) == api.KVS_EINVAL
    cnt = lambda *a: L.kvs_update_counters(*a)  # noqa: E731
    f, i1 = vp(0x1000), vp(0x2000)
    assert cnt(f, f, i1, i1, None, 2, 16, 64, 0.5, 0.1, -1, None) == api.KVS_EINVAL      # cold_limit < 0
    assert cnt(None, f, i1, None, None, 2, 16, 64, 0.5, 0.1, 3, None) == api.KVS_EINVAL  # hot without input
    assert cnt(f, f, None, None, f, 2, 16, 64, 0.5, 0.1, 3, None) == api.KVS_EINVAL      # traj without cold
    assert cnt(f, f, i1, i1, None, 2, 16, 64, float("nan"), 0.1, 3, None) == api.KVS_EINVAL
    assert cnt(f, f, vp(0x2004), None, None, 2, 16, 64, 0.5, 0.1, 3, None) == api.KVS_EALIGN
    flt = lambda *a: L.kvs_filter_blocks(*a)  # noqa: E731
    assert flt(f, None, i1, 2, 16, float("nan"), i1, i1, 8, None) == api.KVS_EINVAL
    assert flt(f, None, i1, 2, 16, 0.5, i1, i1, 0, None) == api.KVS_EINVAL
    assert flt(f, None, None, 2, 16, 0.5, i1, i1, 8, None) == api.KVS_EINVAL
    assert flt(f, None, i1, 2, 16, 0.5, vp(0x3008), i1, 8, None) == api.KVS_EALIGN


def test_reattend_and_profiled_reject_bad_arguments():
    api = _lib()
    L = api.LIB
    vp = ctypes.c_void_p
    re = lambda g, ids=0x8000, n=0x9000, stride=8: L.kvs_reattend_blocks(  # noqa: E731
        ctypes.byref(g), vp(0x1000), vp(0x2000), vp(0x3000), None, None, vp(0x4000),
        vp(ids) if ids else None, vp(n) if n else None, stride, vp(0x5000), vp(0x6000), vp(0x7000), 1 << 20, None)
    g = _geom(api)
    assert re(_geom(api, ring=1)) == api.KVS_EINVAL          # the list replaces ring masking
    assert re(_geom(api, window=8)) == api.KVS_EINVAL        # and windows
    assert re(g, ids=0) == api.KVS_EINVAL
    assert re(g, stride=0) == api.KVS_EINVAL
    assert re(g, ids=0x8004) == api.KVS_EALIGN
    pr = lambda hm: L.kvs_decode_attn_profiled(  # noqa: E731
        ctypes.byref(g), vp(0x1000), vp(0x2000), vp(0x3000), None, None, None, vp(0x4000), None, vp(0x5000),
        vp(0x6000), vp(hm), None, vp(0x7000), 1 << 20, None)
    assert pr(0x8008) == api.KVS_EALIGN
    sel = lambda **kw: L.kvs_select_blocks(vp(0x1000), None, vp(0x2000), kw.get("B", 2), 16,  # noqa: E731
                                           kw.get("budget", 4), kw.get("recent", 16), kw.get("sinks", 0),
                                           vp(0x3000), vp(0x4000), vp(0x5000), None)
    assert sel(recent=0) == api.KVS_EINVAL
    assert sel(budget=-1) == api.KVS_EINVAL
    assert sel(sinks=-4) == api.KVS_EINVAL
    assert sel(B=0) == api.KVS_EINVAL
    g = _geom(api, kv_dtype=api.KVS_FP8_E4M3)
    app = lambda g, **kw: L.kvs_append_kv(ctypes.byref(g), vp(0x1000), vp(0x2000), kw.get("src", 0), 4,  # noqa: E731
                                          vp(0x3000), vp(0x4000), vp(0x5000), vp(0x6000),
                                          kw.get("ks"), kw.get("vs"), kw.get("pos"), None)
    assert app(g) == api.KVS_EINVAL                     # FP8 cache without scale buffers
    assert app(_geom(api), src=0) == api.KVS_EDTYPE     # f32 rows into a bf16 cache
    assert app(g, src=3, ks=vp(0x7000), vs=vp(0x8000)) == api.KVS_EDTYPE


def test_fused_append_decode_rejects_bad_arguments():
    """kvs_append_decode_attn / _partial: the decode checks, then the new
    rows' pointers, alignment and dtype; every call below fails a check."""
    api = _lib()
    L = api.LIB
    vp = ctypes.c_void_p

    def fz(g, kn=0x8000, vn=0x9000, src=None, ws=1 << 20, fn=L.kvs_append_decode_attn):
        return fn(ctypes.byref(g), vp(kn) if kn else None, vp(vn) if vn else None,
                  api.KVS_BF16 if src is None else src, vp(0x1000), vp(0x2000), vp(0x3000), None, None, None,
                  vp(0x4000), None, vp(0x5000), vp(0x6000), vp(0x7000), ws, None)

    g = _geom(api)                                        # bf16 cache
    assert fz(_geom(api, n_q_heads=15)) == api.KVS_EINVAL  # geometry first
    assert fz(g, ws=16) == api.KVS_EWS
    assert fz(g, kn=0) == api.KVS_EINVAL
    assert fz(g, vn=0) == api.KVS_EINVAL
    assert fz(g, vn=0x9004) == api.KVS_EALIGN
    assert fz(g, src=3) == api.KVS_EDTYPE
    assert fz(g, src=api.KVS_F32) == api.KVS_EDTYPE        # f32 rows into a bf16 cache
    assert fz(g, kn=0, fn=L.kvs_append_decode_partial) == api.KVS_EINVAL
    assert fz(_geom(api, kv_dtype=api.KVS_FP8_E4M3)) == api.KVS_EINVAL  # FP8 cache without scales


def test_sidecar_select_rejects_bad_arguments():
    """kvs_update_sidecar_select: the checks of both calls it stands for,
    plus the score source; every call below fails one."""
    api = _lib()
    L = api.LIB
    vp = ctypes.c_void_p
    f = vp(0x1000)

    def ss(alpha=0.5, src=0, budget=8, recent=16, sinks=0, cap=64, step=0, alive=None, mass=f, traj=f,
           keep=vp(0x2000), B=2, nb=16):
        return L.kvs_update_sidecar_select(mass, f, f, f, traj, B, nb, cap, step, alpha, src, alive,
                                           vp(0x3000), budget, recent, sinks, keep, vp(0x4000),
                                           vp(0x5000), None)

    assert ss(alpha=1.5) == api.KVS_EINVAL
    assert ss(alpha=float("nan")) == api.KVS_EINVAL
    assert ss(src=3) == api.KVS_EINVAL
    assert ss(src=-1) == api.KVS_EINVAL
    assert ss(budget=-1) == api.KVS_EINVAL
    assert ss(recent=0) == api.KVS_EINVAL
    assert ss(sinks=-1) == api.KVS_EINVAL
    assert ss(cap=0) == api.KVS_EINVAL
    assert ss(step=-1) == api.KVS_EINVAL
    assert ss(B=0) == api.KVS_EINVAL
    assert ss(mass=None) == api.KVS_EINVAL
    assert ss(keep=None) == api.KVS_EINVAL
    assert ss(alive=vp(0x6004)) == api.KVS_EALIGN
    assert ss(traj=vp(0x6008)) == api.KVS_EALIGN


def test_snapkv_rejects_bad_arguments():
    """kvs_snapkv_scores: every call below fails one check, so no kernel runs."""
    api = _lib()
    vp = ctypes.c_void_p
    f = vp(0x1000)

    def sk(g, window=8, ks=None, pool=7, ws_bytes=1 << 20, ts=vp(0x2000), q=f):
        return api.LIB.kvs_snapkv_scores(ctypes.byref(g), q, window, f, ks, f, ts, None, pool, vp(0x3000),
                                         ws_bytes, None)

    g = _geom(api)                                           # bf16, G = 4
    assert sk(g, window=0) == api.KVS_EINVAL
    assert sk(g, pool=0) == api.KVS_EINVAL
    assert sk(g, pool=8) == api.KVS_EINVAL                   # even kernel
    assert sk(g, pool=35) == api.KVS_EINVAL
    assert sk(g, window=33) == api.KVS_ENOTIMPL              # 132 window columns
    assert sk(_geom(api, n_q_heads=12)) == api.KVS_ENOTIMPL  # G = 3 does not divide 16
    assert sk(_geom(api, ring=1)) == api.KVS_EINVAL
    assert sk(_geom(api, kv_dtype=api.KVS_F32, q_dtype=api.KVS_F32)) == api.KVS_ENOTIMPL
    assert sk(_geom(api, kv_dtype=api.KVS_FP8_E4M3)) == api.KVS_EINVAL  # FP8 cache without scales
    assert sk(g, ks=f) == api.KVS_EINVAL                     # scales with a bf16 cache
    assert sk(g, q=None) == api.KVS_EINVAL
    assert sk(g, ts=vp(0x2004)) == api.KVS_EALIGN
    assert sk(g, ws_bytes=0) == api.KVS_EWS


def test_workspace_init_rejects_bad_arguments():
    api = _lib()
    g = _geom(api)
    need = ctypes.c_size_t()
    assert api.LIB.kvs_decode_workspace_bytes(ctypes.byref(g), ctypes.byref(need)) == 0
    init = api.LIB.kvs_decode_workspace_init
    assert init(ctypes.byref(g), None, need.value, None) == api.KVS_EINVAL
    assert init(ctypes.byref(g), ctypes.c_void_p(0x7008), need.value, None) == api.KVS_EALIGN
    assert init(ctypes.byref(g), ctypes.c_void_p(0x7000), need.value - 16, None) == api.KVS_EWS
    bad = _geom(api, capacity=250)
    assert init(ctypes.byref(bad), ctypes.c_void_p(0x7000), need.value, None) == api.KVS_EINVAL


def test_noalloc_rejects_geometries_beyond_its_scratch_before_any_launch():
    """kvs_decode_attn_scored_noalloc checks every argument, and that the
    geometry's workspace fits its static scratch, before touching the GPU."""
    api = _lib()
    P = ctypes.c_void_p
    big = _geom(api, batch=64, n_q_heads=32, n_kv_heads=8, capacity=131072, n_blocks_max=8192,
                kv_dtype=api.KVS_FP8_E4M3)
    need = ctypes.c_size_t()
    assert api.LIB.kvs_decode_workspace_bytes(ctypes.byref(big), ctypes.byref(need)) == 0
    assert need.value > api.NOALLOC_SCRATCH_BYTES
    fn = api.LIB.kvs_decode_attn_scored_noalloc
    args = [P(0x1000), P(0x2000), P(0x3000), P(0x8000), P(0x9000), None, P(0x4000), None, P(0x5000), P(0x6000), None]
    assert fn(ctypes.byref(big), *args) == api.KVS_ESCRATCH
    assert api.status_str(api.KVS_ESCRATCH).startswith("geometry needs more than the static scratch")
    small = _geom(api, kv_dtype=api.KVS_FP8_E4M3)
    assert fn(ctypes.byref(small), *args[:2], None, *args[3:]) == api.KVS_EINVAL     # no V cache
    assert fn(ctypes.byref(small), P(0x1008), *args[1:]) == api.KVS_EALIGN


def test_stream_read_rejects_bad_arguments():
    api = _lib()
    f = api.LIB.kvs_stream_read
    P = ctypes.c_void_p
    assert f(None, 1024, P(0x2000), 1, None) == api.KVS_EINVAL
    assert f(P(0x1000), 1000, P(0x2000), 1, None) == api.KVS_EINVAL          # not whole KiB
    assert f(P(0x1000), 2048, P(0x2000), 3, None) == api.KVS_EINVAL          # fewer runs than workgroups
    assert f(P(0x1000), 2048, P(0x2000), 0, None) == api.KVS_EINVAL
    assert f(P(0x1008), 2048, P(0x2000), 1, None) == api.KVS_EALIGN


def test_decode_step_structs_match_the_header(tmp_path):
    """kvs_layer_bufs and kvs_turn_args as the C compiler lays them out
    (sizes and field offsets) equal the binding's ctypes mirrors."""
    import shutil
    import subprocess
    api = _lib()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = {"kvs_layer_bufs": api.LayerBufs, "kvs_turn_args": api.TurnArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kvs.h"', "int main(void) {"]
    for cname, cls in fields.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    for cname, cls in fields.items():
        assert int(out[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(out[f"{cname}.{f}"]) == getattr(cls, f).offset, f"{cname}.{f}"


def test_decode_step_rejects_bad_arguments():
    """kvs_decode_step: every layer's checks, the mass and turn checks, all
    before the first launch (a bad last layer is reported, not launched
    around); every call below fails one check."""
    api = _lib()
    L = api.LIB
    vp = ctypes.c_void_p
    g = _geom(api)                                         # bf16 linear cache, 16 blocks

    def layer(**kw):
        d = dict(q=0x1000, k_new=0x8000, v_new=0x9000, k_cache=0x2000, v_cache=0x3000, k_scale=None,
                 v_scale=None, pos_of_slot=None, out=0x5000, workspace=0x7000)
        d.update(kw)
        b = api.LayerBufs()
        for f, v in d.items():
            setattr(b, f, v)
        return b

    def turn(**kw):
        t = api.TurnArgs()
        d = dict(attended=0xa000, ema=0xb000, cum=0xc000, traj=0xd000, traj_cap=64, select=1, step=0, alpha=0.5,
                 score_source=0, alive=None, budget_blocks=4, recent_tokens=16, sink_tokens=0, keep_out=0xe000,
                 sel_ids=0xf000, n_sel=0x10000)
        d.update(kw)
        for f, v in d.items():
            setattr(t, f, v)
        return t

    def step(layers, geom=g, src=api.KVS_BF16, ws=1 << 20, mass=0x6000, trn=None, n=None, cur=0x4000):
        arr = (api.LayerBufs * len(layers))(*layers)
        return L.kvs_decode_step(ctypes.byref(geom), len(layers) if n is None else n, arr, src,
                                 vp(cur) if cur else None, None, ws, vp(mass) if mass else None,
                                 ctypes.byref(trn) if trn is not None else None, None)

    ok = [layer(), layer(), layer()]
    assert step(ok, n=0) == api.KVS_EINVAL
    assert step(ok, n=129) == api.KVS_EINVAL
    assert step(ok, geom=_geom(api, n_q_heads=15)) == api.KVS_EINVAL
    assert step(ok, ws=16) == api.KVS_EWS
    assert step(ok, cur=0) == api.KVS_EINVAL
    assert step(ok, mass=0x6004) == api.KVS_EALIGN
    assert step(ok, src=api.KVS_F32) == api.KVS_EDTYPE              # f32 rows into a bf16 cache
    assert step(ok[:2] + [layer(q=0x1004)]) == api.KVS_EALIGN        # the last layer's error, nothing launched
    assert step(ok[:2] + [layer(v_new=None)]) == api.KVS_EINVAL      # K without V
    assert step(ok[:2] + [layer(out=None)]) == api.KVS_EINVAL
    assert step(ok[:2] + [layer(k_scale=0x11000)]) == api.KVS_EINVAL  # scales on a bf16 cache
    assert step(ok, mass=0, trn=turn()) == api.KVS_EINVAL             # a turn needs the masses
    assert step(ok, trn=turn(alpha=1.5)) == api.KVS_EINVAL
    assert step(ok, trn=turn(select=2)) == api.KVS_EINVAL
    assert step(ok, trn=turn(score_source=3)) == api.KVS_EINVAL
    assert step(ok, trn=turn(recent_tokens=0)) == api.KVS_EINVAL
    assert step(ok, trn=turn(keep_out=None)) == api.KVS_EINVAL
    assert step(ok, trn=turn(traj=0xd008)) == api.KVS_EALIGN
    assert step(ok, trn=turn(select=0, keep_out=None, traj_cap=0)) == api.KVS_EINVAL
    fp8 = _geom(api, kv_dtype=api.KVS_FP8_E4M3)
    assert step(ok, geom=fp8) == api.KVS_EINVAL                       # FP8 cache without scales
