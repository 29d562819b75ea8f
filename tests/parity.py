"""Comparison rules between the HIP path and the fp64 oracle (shared by the GPU tests).

Tolerances (written here, used by every parity test):
  * page meta: exact (value equality; min / max of stored values is representable, and
    the fp8 outward rounding is a deterministic function of exact fp32 products);
  * top-K page scores: |gpu - oracle| <= 1e-4 * max_g sum_c |q_gc| max(|kmax_c|, |kmin_c|)
    (fp32 accumulation of a 128-term sum whose magnitude is that scale);
  * coverage shares: |gpu - oracle| <= 1e-4 * pi + 1e-9;
  * top-K lists: the GPU list has the oracle list's size, holds every forced page, every
    page scoring above s_K + eps and none below s_K - eps, where s_K is the oracle's
    K'-th best free score and eps = 1e-5 * max(|s_K|, scale) -- ties within eps may go
    either way;
  * coverage lists: a threshold set up to a 1e-5 relative band whose mass reaches
    t - 1e-5 and stops being minimal only within 1e-5;
  * attention: max |O - O_ref| <= 2e-3 (f32 / f16 pools) or 2e-2 (fp8 pools), same bound
    on lse.
"""
from __future__ import annotations

import numpy as np

from oracle import spd_oracle as O

SCORE_RTOL = 1e-4
TIE_RTOL = 1e-5
ATTN_TOL = {"f32": 2e-3, "f16": 2e-3, "fp8": 2e-2}


def pool_meta(meta, block_table, seq_lens, num_pool_pages, fill=0):
    """The library's key statistics in the oracle's layout.

    The library keeps them per request in logical page order ([B, Hkv, max_pages * g, 2, d], g
    logical pages per physical page); the oracle keeps them with the physical page that holds each
    logical page ([num_pool_pages, Hkv, 2, d], or [num_pool_pages, Hkv, g, 2, d] when g > 1).  The
    result holds the entries of each request's first ceil(L / 16) logical pages at their physical
    page; pool pages that hold none of them keep ``fill``."""
    meta = np.asarray(meta)
    bt = np.asarray(block_table)
    B, H, LP = meta.shape[:3]
    g = LP // bt.shape[1]
    out = np.full((num_pool_pages, H, g) + meta.shape[3:], fill, dtype=meta.dtype)
    for b in range(B):
        n = min(O.n_pages(int(seq_lens[b])), LP)
        lp = np.arange(n)
        phys = bt[b, lp // g].astype(np.int64)
        ok = (phys >= 0) & (phys < num_pool_pages)
        out[phys[ok], :, (lp % g)[ok]] = meta[b][:, lp[ok]].swapaxes(0, 1)
    return out[:, :, 0] if g == 1 else out


def meta_past_rows(meta, seq_lens):
    """The library's key-statistics entries past each request's logical pages (never written by a
    build over the request's pages), flattened."""
    meta = np.asarray(meta)
    LP = meta.shape[2]
    return np.concatenate([meta[b, :, min(O.n_pages(int(L)), LP):].ravel() for b, L in enumerate(seq_lens)])


def bound_scale(inp, meta, b, h):
    """Per page: max over the group's heads of sum_c |q_c| max(|kmax_c|, |kmin_c|)."""
    w = inp.workload
    G = w.group
    n = O.n_pages(inp.seq_lens[b])
    phys = inp.block_table[b, :n].astype(np.int64)
    m = np.abs(meta[phys, h].astype(np.float64)).max(axis=1)  # [n, d]
    q = np.abs(inp.q[b, h * G:(h + 1) * G].astype(np.float64))  # [G, d]
    return (q @ m.T).max(axis=0)


def check_topk_scores(gpu, ref, scale):
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = err > SCORE_RTOL * np.maximum(scale, 1e-30)
    assert not bad.any(), f"score mismatch at pages {np.nonzero(bad)[0][:10]}: err {err[bad][:5]}"


def check_coverage_shares(gpu, ref):
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = err > SCORE_RTOL * ref + 1e-9
    assert not bad.any(), f"share mismatch at pages {np.nonzero(bad)[0][:10]}: {gpu[bad][:5]} vs {ref[bad][:5]}"


def check_topk_list(lst, ref_scores, n, budget, forced, scale):
    lst = list(lst)
    assert lst == sorted(set(lst)), "list not strictly ascending"
    assert all(0 <= p < n for p in lst)
    want = O.select_topk(ref_scores, n, budget, forced)
    assert len(lst) == len(want), (len(lst), len(want))
    fset = set(forced)
    assert fset <= set(lst)
    free = [p for p in range(n) if p not in fset]
    k_rest = budget - len(forced)
    if k_rest <= 0 or len(free) <= k_rest:
        assert lst == want
        return
    order = sorted(free, key=lambda p: (-float(ref_scores[p]), p))
    sK = float(ref_scores[order[k_rest - 1]])
    chosen = set(lst) - fset
    for p in free:
        eps = TIE_RTOL * max(abs(sK), float(scale[p]))
        if ref_scores[p] > sK + eps:
            assert p in chosen, f"page {p} (score {ref_scores[p]}) above the cut {sK} missing"
        if ref_scores[p] < sK - eps:
            assert p not in chosen, f"page {p} (score {ref_scores[p]}) below the cut {sK} selected"


def check_coverage_list(lst, pi, n, gamma, forced):
    lst = list(lst)
    assert lst == sorted(set(lst)) and all(0 <= p < n for p in lst)
    fset = set(forced)
    assert fset <= set(lst)
    t = gamma - sum(float(pi[p]) for p in forced)
    chosen = [p for p in lst if p not in fset]
    free = [p for p in range(n) if p not in fset]
    if not free:  # nothing to choose from: an empty row, or every page forced
        assert not chosen
        return
    if t <= TIE_RTOL:
        assert len(chosen) == 0 or t > -TIE_RTOL
        return
    if not chosen:
        raise AssertionError("coverage list holds no free page although t > 0")
    mass = sum(float(pi[p]) for p in chosen)
    total_free = sum(float(pi[p]) for p in free)
    if len(chosen) == len(free):
        assert mass >= min(t, total_free) - TIE_RTOL
    else:
        assert mass >= t - TIE_RTOL, (mass, t)
        assert mass - min(float(pi[p]) for p in chosen) < t + TIE_RTOL, "not minimal"
    # threshold set up to the band
    lo = min(float(pi[p]) for p in chosen)
    chosen_set = set(chosen)
    unchosen = [p for p in free if p not in chosen_set]
    if unchosen:
        hi = max(float(pi[p]) for p in unchosen)
        assert hi <= lo * (1 + TIE_RTOL) + 1e-12, (hi, lo)


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, kv_dtype, where=""):
    tol = ATTN_TOL[kv_dtype]
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert np.isfinite(o_gpu).all(), f"{where}: non-finite output"
    assert err.max() <= tol, f"{where}: max |dO| = {err.max()}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{where}: lse finiteness differs"
    if fin.any():
        e2 = np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin]).max()
        assert e2 <= tol, f"{where}: max |dlse| = {e2}"
