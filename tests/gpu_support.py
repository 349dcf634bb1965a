"""Helpers shared by the GPU parity tests: build caches through the C ABI from
seeded rows, compute the same quantities with the float64 oracle, compare."""

from __future__ import annotations

import numpy as np
import torch

from oracle import kvs_oracle as orc


def dequant_rows(rows_f32: np.ndarray, kv_dtype: str) -> np.ndarray:
    """The values a cache of ``kv_dtype`` holds for float32 source rows, in
    float64: FP8 rows are encoded and decoded by the oracle itself; bf16 rows
    are the round-to-nearest-even cast done when the inputs were made."""
    if kv_dtype == "fp8":
        codes, scales = orc.fp8_encode_rows(rows_f32.astype(np.float32))
        return orc.fp8_decode_rows(codes, scales)
    if kv_dtype == "bf16":
        return torch.from_numpy(rows_f32).to(torch.bfloat16).double().numpy()
    return rows_f32.astype(np.float64)


def heads(rows: np.ndarray, n_heads: int, d: int) -> np.ndarray:
    """[n, H*d] -> [H, n, d]"""
    return rows.reshape(rows.shape[0], n_heads, d).transpose(1, 0, 2)


def out_spread(p: np.ndarray, Vsel: np.ndarray, absV=None, sqV=None) -> np.ndarray:
    """``[2, Hq, d]`` spread of the PV sum for weights ``p [Hq, n]`` over the
    read values ``Vsel [Hkv, n, d]`` (query head h reads KV head h // G): row 0
    is ``sum_j p_j |v_j|``, row 1 ``sqrt(sum_j p_j^2 v_j^2)``. Computed in
    float32 (it only sizes the tolerance); ``absV`` / ``sqV`` may hold
    ``|Vsel|`` and ``Vsel**2`` as float32, precomputed."""
    Hq, Hkv = p.shape[0], Vsel.shape[0]
    G = Hq // Hkv
    p32 = p.astype(np.float32)
    out = np.zeros((2, Hq, Vsel.shape[2]), dtype=np.float64)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        a = absV[g] if absV is not None else np.abs(Vsel[g]).astype(np.float32)
        q2 = sqV[g] if sqV is not None else np.square(Vsel[g]).astype(np.float32)
        out[0, hs] = p32[hs] @ a
        out[1, hs] = np.sqrt(np.square(p32[hs]) @ q2)
    return out


def oracle_layer(q, Kd, Vd, positions, i, window, alive, scale, n_blocks, absV=None, sqV=None):
    """Oracle output, block mass and the output's spread (``out_spread``) for
    one (sequence, layer): ``Kd``, ``Vd`` are [Hkv, n, d] float64 values held
    at absolute ``positions`` (``absV``, ``sqV``: optional float32 |Vd|, Vd**2)."""
    positions = np.asarray(positions)
    sel = orc.visible_mask(positions, i, window, alive)
    idx = np.flatnonzero(sel)
    if len(idx) and idx[-1] - idx[0] + 1 == len(idx):
        cut = slice(int(idx[0]), int(idx[-1]) + 1)   # a run of columns: views, no copies
    else:
        cut = idx
    Ks, Vs = Kd[:, cut], Vd[:, cut]
    a = absV[:, cut] if absV is not None else None
    s2 = sqV[:, cut] if sqV is not None else None
    o, p = orc.attend(q, Ks, Vs, scale)
    mass = orc.block_mass(p, positions[sel], n_blocks)
    return o, mass, out_spread(p, Vs, a, s2)


# Output tolerance for bf16 and FP8 caches (float32 caches: rtol 1e-5, atol
# 1e-6). The kernel takes the post-softmax weights into the PV product as
# bf16 (for FP8 the V scale folded in first): each term p_j v_j gets an
# independent relative rounding error of at most 2^-8 (round to nearest even
# with 8 significant bits), zero-mean and of standard deviation below 2^-9,
# so the output moves by about 2^-9 sqrt(sum_j p_j^2 v_j^2) and, with the
# largest of ~10^5 elements checked per call, stays far below 8 of those.
# The output itself is rounded to bf16 (relative 2^-8) and lies inside the
# spec relative tolerance 2e-2. Float32 logits, exponentials and
# accumulation add far less than 2^-20 sum_j p_j |v_j|.
OUT_REL = 2e-2
OUT_SIGMAS = 8.0
OUT_F32_FLOOR = 2.0 ** -20


def out_bound(ref: np.ndarray, spread: np.ndarray, runs: int = 1) -> np.ndarray:
    """Largest allowed |got - ref| per element for a bf16/FP8-cache output;
    ``runs = 2`` bounds the difference of two independently rounded GPU runs."""
    return (OUT_REL * np.abs(ref) + runs * OUT_SIGMAS * 2.0 ** -9 * spread[1]
            + runs * OUT_F32_FLOOR * spread[0])


# worst |got - ref| / bound per test, reported at the end of a GPU session
WORST_RATIO: dict = {}


def _note_ratio(ratio: float):
    import os
    key = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    WORST_RATIO[key] = max(WORST_RATIO.get(key, 0.0), ratio)


def close_o(got: np.ndarray, ref: np.ndarray, kv_dtype: str, spread: np.ndarray | None = None):
    """Output check: float32 caches within rtol 1e-5, atol 1e-6; bf16 and FP8
    caches within ``out_bound`` (see above)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    if kv_dtype == "f32":
        bound = 1e-5 * np.abs(ref) + 1e-6
    else:
        assert spread is not None
        bound = out_bound(ref, spread)
    _note_ratio(float((err / bound).max()) if err.size else 0.0)
    bad = err > bound
    assert not bad.any(), (f"O mismatch at {np.argwhere(bad)[:5].tolist()}: max err {err.max()}, "
                           f"worst err/bound {(err / bound).max():.3g}")


def close_mass(got: np.ndarray, ref: np.ndarray, kv_dtype: str, what="mass"):
    got = np.asarray(got, dtype=np.float64)
    if kv_dtype == "f32":
        bad = np.abs(got - ref) > 1e-5 * np.abs(ref) + 1e-6
    else:
        bad = np.abs(got - ref) > 1e-4 * np.maximum(1.0, np.abs(ref))
    assert not bad.any(), f"{what} mismatch at {np.argwhere(bad)[:5].tolist()}: max err {np.abs(got - ref).max()}"


def keep_ids_from_mask(mask_words: np.ndarray, n_exist: int) -> np.ndarray:
    w = mask_words.astype(np.int64) & 0xFFFFFFFF
    bits = [(int(w[b >> 5]) >> (b & 31)) & 1 for b in range(n_exist)]
    return np.flatnonzero(np.array(bits, dtype=bool))


# |Amb| per checked (test, step, sequence), reported at the end of a GPU session
AMB_LOG: dict = {}


def compare_selection(gpu_ids, ref_ids, score_ref, i, budget, recent, sinks, alive, rel_tol, where=None,
                      score_gpu=None):
    """Near-tie protocol: with v the oracle's budget-th candidate score, blocks
    whose oracle score is within tol = rel_tol * max(1, |v|) of v are
    ambiguous (Amb); outside them the sets must be equal, and both must take
    the same number of ambiguous blocks. Returns |Amb| (recorded under
    ``where``, e.g. (step, sequence), when given).

    With the GPU's own scores ``score_gpu`` a sharper check runs as well: if
    every candidate's GPU score is within e of the oracle's, a block whose
    oracle score is more than 2e above v is kept by both, one more than 2e
    below v by neither (at most budget - 1 candidates score above v, so a
    block the GPU ranks wrongly past one of them would make budget + 1), so
    the sets must agree outside the band |score - v| <= 2e; its size is
    recorded too."""
    gpu, ref = set(int(x) for x in gpu_ids), set(int(x) for x in ref_ids)
    prot = orc.protected_blocks(i, recent, sinks)
    cand = [b for b in range(i // 16 + 1) if (alive is None or alive[b]) and b not in prot]
    amb, band = set(), set()
    if budget > 0 and cand:
        cand.sort(key=lambda b: (-float(score_ref[b]), b))
        v = float(score_ref[cand[min(budget, len(cand)) - 1]])
        tol = rel_tol * max(1.0, abs(v))
        amb = {b for b in cand if abs(float(score_ref[b]) - v) <= tol}
        if score_gpu is not None:
            idx = np.array(cand)
            e = float(np.abs(np.asarray(score_gpu, dtype=np.float64)[idx] - np.asarray(score_ref)[idx]).max())
            band = {b for b in cand if abs(float(score_ref[b]) - v) <= 2.0 * e}
    if where is not None:
        import os
        key = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        AMB_LOG.setdefault(key, []).append((*where, len(amb), len(band) if score_gpu is not None else -1, gpu == ref))
    if gpu != ref:
        assert amb, f"selection differs: gpu-only {sorted(gpu - ref)}, oracle-only {sorted(ref - gpu)}"
        assert (gpu - amb) == (ref - amb), f"selection differs outside near-ties: {sorted(gpu ^ ref)}"
        assert len(gpu & amb) == len(ref & amb)
        if score_gpu is not None:
            assert (gpu - band) == (ref - band), f"selection differs outside the observed-error band: {sorted(gpu ^ ref)}"
    return len(amb)


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if dtype is None else t.to(dtype)


def k_tile_offset(t, x, eb):
    """Byte offset of K element (slot t in its 16-slot tile, dim x): the layout
    documented in include/kvs.h."""
    xb = x * eb
    return ((xb // 64 * 4 + (xb % 64) // 16) * 16 + t) * 16 + xb % 16


def v_tile_offset(t, x, D, eb):
    kg, e, j, n = t // 4, t % 4, x // (D // 16), x % (D // 16)
    ub = (4 * n + e) * eb
    return ((ub // 16 * 4 + kg) * 16 + j) * 16 + ub % 16


def logical_rows(buf: np.ndarray, B, Hkv, C, D, eb, seq, slots, which="k") -> np.ndarray:
    """Read cache bytes back as [len(slots), Hkv*D] element rows (raw bytes of
    width eb per element) for one sequence."""
    raw = buf.view(np.uint8).reshape(B, Hkv, C // 16, 16 * D * eb)
    slots = np.asarray(slots)
    t = (slots % 16)[:, None]
    x = np.arange(D)[None, :]
    off = k_tile_offset(t, x, eb) if which == "k" else v_tile_offset(t, x, D, eb)
    out = np.zeros((len(slots), Hkv, D, eb), dtype=np.uint8)
    for g in range(Hkv):
        tiles = raw[seq, g, slots // 16]                       # [n, tile bytes]
        for k in range(eb):
            out[:, g, :, k] = np.take_along_axis(tiles, off + k, axis=1)
    return out.reshape(len(slots), Hkv * D * eb)
