"""Acceptance rules for comparing the HIP path with the CPU oracle.

Index sets (retrieval, prune): the GPU list must hold k distinct in-range
indices in ascending order.  It passes if it equals the oracle's set, or if
every swapped pair straddles the oracle's k-th value by less than
``band`` relative: max over missed oracle picks minus min over extra GPU picks
< band * |sigma_k|, where sigma_k is the oracle's k-th largest score (the
RMS of the scores when sigma_k is ~0).

Attention: per (b, h), max_d |o_gpu - o_ref| / max_d |o_ref| <= 2e-3.
Salience: per element |s_gpu - s_ref| / s_ref <= 1e-4 and each frame's GPU
salience sums to 1 within 1e-5.
"""
from __future__ import annotations

import numpy as np

INDEX_BAND = 1e-5
ATTN_TOL = 2e-3
SAL_REL = 1e-4
SAL_SUM = 1e-5


def check_index_row(gpu_idx, s_ref, k, band=INDEX_BAND):
    """Return (ok, n_swaps, message) for one row."""
    g = np.asarray(gpu_idx, dtype=np.int64)
    s = np.asarray(s_ref, dtype=np.float64)
    N = s.shape[0]
    if g.shape != (k,):
        return False, -1, f"shape {g.shape} != ({k},)"
    if k == 0:
        return True, 0, ""
    if g.min() < 0 or g.max() >= N:
        return False, -1, "index out of range"
    if np.any(np.diff(g) <= 0):
        return False, -1, "not strictly ascending (duplicate or unsorted)"
    order = np.lexsort((np.arange(N), -s))
    ref = set(order[:k].tolist())
    got = set(g.tolist())
    if got == ref:
        return True, 0, ""
    sigma_k = s[order[k - 1]]
    scale = abs(sigma_k)
    if scale < 1e-12 * np.abs(s).max():
        scale = float(np.sqrt(np.mean(s * s)))
    missed = np.array(sorted(ref - got))
    extra = np.array(sorted(got - ref))
    gap = s[missed].max() - s[extra].min()
    ok = gap < band * scale
    return bool(ok), len(missed), f"{len(missed)} swaps, worst gap {gap:.3e} vs band {band * scale:.3e}"


def check_index_sets(gpu_idx, s_ref, k, band=INDEX_BAND):
    """All rows; returns (ok, total_swaps, messages)."""
    gpu_idx = np.asarray(gpu_idx)
    s_ref = np.asarray(s_ref)
    total, msgs, ok = 0, [], True
    for r in range(s_ref.shape[0]):
        o, n, m = check_index_row(gpu_idx[r], s_ref[r], k, band)
        ok &= o
        total += max(n, 0)
        if not o:
            msgs.append(f"row {r}: {m}")
    return ok, total, msgs


def attn_errors(out_gpu, out_ref):
    """Per-(b, h) max-abs error relative to max |ref|, shape [B][Hq]."""
    o = np.asarray(out_gpu, dtype=np.float64)
    r = np.asarray(out_ref, dtype=np.float64)
    num = np.abs(o - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def check_attention(out_gpu, out_ref, tol=ATTN_TOL):
    e = attn_errors(out_gpu, out_ref)
    return bool(np.all(e <= tol)), float(e.max())


def check_salience(s_gpu, s_ref, rel=SAL_REL, sum_tol=SAL_SUM):
    g = np.asarray(s_gpu, dtype=np.float64)
    r = np.asarray(s_ref, dtype=np.float64)
    rel_err = np.abs(g - r) / np.abs(r)
    sums = np.abs(g.sum(axis=-1) - 1.0)
    return bool(rel_err.max() <= rel and sums.max() <= sum_tol), float(rel_err.max()), float(sums.max())
