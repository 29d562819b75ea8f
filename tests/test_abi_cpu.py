"""The C ABI without a GPU: exports, host-side validation and the planning helpers.

Every call here returns before anything is launched, so no device is needed (the stream
argument is passed as 0 so that torch never initialises HIP).
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from sparse_paged_decode_quest_amd import _abi as A
from sparse_paged_decode_quest_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return A.lib()


def declared_functions():
    with open(os.path.join(ROOT, "include", "spd.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(A.EXPORTS)
    assert A.abi_version() == 18


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert A.error_string(code) not in ("", "unknown status")
    assert A.error_string(-99) == "unknown status"


def desc_for(w, **over):
    d = dict(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
             page_size=16, max_pages_per_seq=w.pages_per_seq, num_pool_pages=1000, max_list=w.list_capacity,
             q_dtype=A.DTYPE[w.q_dtype], kv_dtype=A.DTYPE[w.kv_dtype])
    d.update(over)
    return A.Desc(**d)


def sel_for(w, **over):
    s = dict(mode=A.SELECT_COVERAGE if w.mode == "coverage" else A.SELECT_TOPK, budget_pages=w.budget_pages or 1,
             gamma=w.gamma or 1.0, sm_scale=w.sm_scale, n_sink=w.n_sink, n_local=w.n_local,
             n_sink_stream=w.n_sink_stream, n_local_stream=w.n_local_stream)
    s.update(over)
    return A.SelectParams(**s)


FAKE = 0x1000  # never dereferenced: every case below fails validation first


def score_rc(desc, sel, heads=None, ws=FAKE, ws_bytes=1 << 30, lse=FAKE, tail=0, k_pool=FAKE, k_scale=FAKE):
    heads = heads if heads is not None else [0] * max(1, desc.num_kv_heads)
    arr = (ctypes.c_uint8 * len(heads))(*heads)
    return A.lib().spd_page_score(ctypes.byref(desc), ctypes.byref(sel), FAKE, FAKE, k_pool, k_scale, tail, FAKE,
                                  FAKE, arr, FAKE, lse, ws, ws_bytes, 0)


def select_rc(desc, sel, heads=None, bt=FAKE, phys=None, k_pool=FAKE, k_scale=FAKE, meta=None):
    heads = heads if heads is not None else [0] * max(1, desc.num_kv_heads)
    arr = (ctypes.c_uint8 * len(heads))(*heads)
    return A.lib().spd_page_select(ctypes.byref(desc), ctypes.byref(sel), FAKE, FAKE, arr, bt, k_pool, k_scale, meta,
                                   FAKE, phys, FAKE, None, 0)


def fused_rc(desc, sel, heads=None, ws=FAKE, ws_bytes=1 << 30, tail=0, k_pool=FAKE, k_scale=FAKE, bt=FAKE):
    heads = heads if heads is not None else [0] * max(1, desc.num_kv_heads)
    arr = (ctypes.c_uint8 * len(heads))(*heads)
    return A.lib().spd_page_score_select(ctypes.byref(desc), ctypes.byref(sel), FAKE, FAKE, k_pool, k_scale, tail,
                                         bt, FAKE, arr, FAKE, None, FAKE, None, None, None, ws, ws_bytes, 0)


def decode_rc(desc, plan, sm_scale=0.1, **null):
    ptrs = {k: FAKE for k in ("q", "k", "v", "ks", "vs", "bt", "sl", "pl", "pp", "ll", "o", "lse", "po", "pls")}
    ptrs.update(null)
    return A.lib().spd_sparse_paged_decode(
        ctypes.byref(desc), ctypes.byref(plan), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["ks"], ptrs["vs"], ptrs["bt"],
        ptrs["sl"], ptrs["pl"], ptrs["pp"], ptrs["ll"], ctypes.c_float(sm_scale), ptrs["o"], ptrs["lse"], ptrs["po"],
        ptrs["pls"], 0)


@pytest.mark.parametrize("over,code", [
    (dict(num_q_heads=9), A.SPD_ERR_INVALID_ARG),          # Hq % Hkv != 0
    (dict(num_kv_heads=0), A.SPD_ERR_INVALID_ARG),
    (dict(num_kv_heads=65, num_q_heads=260), A.SPD_ERR_INVALID_ARG),
    (dict(batch=-1), A.SPD_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=0), A.SPD_ERR_INVALID_ARG),
    (dict(q_dtype=7), A.SPD_ERR_INVALID_ARG),
    (dict(q_dtype=2), A.SPD_ERR_INVALID_ARG),               # fp8 queries are not an input format
    (dict(head_dim=96), A.SPD_ERR_UNSUPPORTED),
    (dict(page_size=32), A.SPD_ERR_UNSUPPORTED),
    (dict(num_q_heads=16), A.SPD_ERR_UNSUPPORTED),          # G = 8
    (dict(q_dtype=0, kv_dtype=1), A.SPD_ERR_UNSUPPORTED),   # f32 q with f16 pool
    (dict(head_dim=64, kv_dtype=2), A.SPD_ERR_UNSUPPORTED),  # fp8 compiled for d = 128 only
])
def test_descriptor_validation(lib, over, code):
    w = W.small()
    assert score_rc(desc_for(w, **over), sel_for(w)) == code
    assert decode_rc(desc_for(w, **over), A.PlanParams(4, 16, 512)) == code


def test_select_param_validation(lib):
    w = W.small()
    d = desc_for(w)
    assert score_rc(d, sel_for(w, budget_pages=0)) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, sel_for(w, mode=5)) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, sel_for(w, n_sink=-1)) == A.SPD_ERR_INVALID_ARG
    for g in (0.0, -0.5, 1.5, float("nan")):
        assert score_rc(d, sel_for(w, mode=A.SELECT_COVERAGE, gamma=g)) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, sel_for(w, mode=A.SELECT_COVERAGE, sm_scale=0.0)) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, sel_for(w), heads=[0, 2]) == A.SPD_ERR_INVALID_ARG      # unknown head kind


def test_list_capacity_and_workspace_checks(lib):
    w = W.small(budget=24)
    assert select_rc(desc_for(w, max_list=23), sel_for(w)) == A.SPD_ERR_INVALID_ARG
    assert select_rc(desc_for(w, max_list=4), sel_for(w, n_sink_stream=3, n_local_stream=3), heads=[1, 1]) \
        == A.SPD_ERR_INVALID_ARG
    wc = W.small(mode="coverage")
    assert select_rc(desc_for(wc, max_list=wc.pages_per_seq - 1), sel_for(wc)) == A.SPD_ERR_INVALID_ARG
    need = A.spd_workspace_bytes(desc_for(wc), sel_for(wc), A.OP_PAGE_SCORE)
    assert need > 0
    assert score_rc(desc_for(wc), sel_for(wc), ws=FAKE, ws_bytes=need - 1) == A.SPD_ERR_WORKSPACE
    assert score_rc(desc_for(wc), sel_for(wc), ws=None, ws_bytes=need) == A.SPD_ERR_WORKSPACE
    assert score_rc(desc_for(wc), sel_for(wc), lse=None) == A.SPD_ERR_INVALID_ARG
    assert A.spd_workspace_bytes(desc_for(w), sel_for(w), A.OP_PAGE_SCORE) == 0
    assert A.spd_workspace_bytes(desc_for(w), sel_for(w), A.OP_PAGE_SELECT) == 0
    assert A.spd_workspace_bytes(desc_for(w), sel_for(w), A.OP_PAGE_SCORE_SELECT) >= 4 * w.batch * 2 * w.pages_per_seq
    # coverage keeps G log-masses per page in the fused workspace
    assert A.spd_workspace_bytes(desc_for(wc), sel_for(wc), A.OP_PAGE_SCORE_SELECT) >= \
        16 * wc.batch * 2 * wc.pages_per_seq
    with pytest.raises(A.SpdError):
        A.spd_workspace_bytes(desc_for(w), sel_for(w), 9)
    fneed = A.spd_workspace_bytes(desc_for(wc), sel_for(wc), A.OP_PAGE_SCORE_SELECT)
    assert fused_rc(desc_for(wc), sel_for(wc), ws_bytes=fneed - 1) == A.SPD_ERR_WORKSPACE
    assert fused_rc(desc_for(wc), sel_for(wc), ws=None, ws_bytes=fneed) == A.SPD_ERR_WORKSPACE


def test_decode_argument_checks(lib):
    w = W.small()
    d = desc_for(w)
    plan = A.PlanParams(4, 16, 512)
    assert decode_rc(d, A.PlanParams(0, 16, 512)) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, A.PlanParams(4, 0, 512)) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, plan, sm_scale=0.0) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, plan, sm_scale=float("inf")) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, plan, q=None) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, plan, pls=None) == A.SPD_ERR_INVALID_ARG
    wf = W.small(kv="fp8")
    assert decode_rc(desc_for(wf), plan, ks=None) == A.SPD_ERR_INVALID_ARG


def test_list_refresh_argument_checks(lib):
    w = W.small()
    d = desc_for(w)
    heads = (ctypes.c_uint8 * d.num_kv_heads)(*([0] * d.num_kv_heads))

    def rc(sl=FAKE, bt=FAKE, k_pool=FAKE, meta=None, pl=FAKE, ll=FAKE, desc=d):
        return A.lib().spd_page_list_refresh(ctypes.byref(desc), ctypes.byref(sel_for(w)), sl, heads, bt, k_pool, FAKE,
                                             meta, pl, None, ll, 0)

    for kw in (dict(sl=None), dict(bt=None), dict(pl=None), dict(ll=None)):
        assert rc(**kw) == A.SPD_ERR_INVALID_ARG, kw
    assert rc(k_pool=None, meta=FAKE) == A.SPD_ERR_INVALID_ARG  # the newest-page rebuild reads K
    assert rc(desc=desc_for(w, max_list=2)) == A.SPD_ERR_INVALID_ARG  # lists must hold a selection
    assert rc(desc=desc_for(w, batch=0)) == A.SPD_OK  # nothing to do, nothing launched


def test_select_and_fused_argument_checks(lib):
    w = W.small()
    d = desc_for(w)
    assert select_rc(d, sel_for(w), bt=None, phys=FAKE) == A.SPD_ERR_INVALID_ARG   # physical pages need the table
    assert select_rc(d, sel_for(w), bt=None, meta=FAKE) == A.SPD_ERR_INVALID_ARG   # so does the tail rebuild
    assert select_rc(d, sel_for(w), k_pool=None, meta=FAKE) == A.SPD_ERR_INVALID_ARG  # which reads K
    assert select_rc(desc_for(W.small(kv="fp8")), sel_for(w), k_scale=None, meta=FAKE) == A.SPD_ERR_INVALID_ARG
    assert fused_rc(d, sel_for(w), bt=None) == A.SPD_ERR_INVALID_ARG
    assert fused_rc(d, sel_for(w), tail=A.TAIL_REBUILD, k_pool=None) == A.SPD_ERR_INVALID_ARG  # a rebuild reads K
    assert score_rc(d, sel_for(w), tail=A.TAIL_REBUILD, k_pool=None) == A.SPD_ERR_INVALID_ARG
    wf = W.small(kv="fp8")
    assert fused_rc(desc_for(wf), sel_for(wf), tail=A.TAIL_REBUILD, k_scale=None) == A.SPD_ERR_INVALID_ARG
    for bad in (-1, 3):
        assert score_rc(d, sel_for(w), tail=bad) == A.SPD_ERR_INVALID_ARG
        assert fused_rc(d, sel_for(w), tail=bad) == A.SPD_ERR_INVALID_ARG
    # skipping the last page needs top-K with a local window (which keeps that page)
    assert fused_rc(d, sel_for(w), tail=A.TAIL_SKIP, k_pool=None, ws=None) == A.SPD_ERR_WORKSPACE  # passes the tail check
    no_local = sel_for(w)
    no_local.n_local = 0
    assert score_rc(d, no_local, tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    assert fused_rc(d, no_local, tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    wc = W.small(mode="coverage", gamma=0.9)
    assert score_rc(desc_for(wc), sel_for(wc), tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    assert fused_rc(desc_for(wc), sel_for(wc), tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    # rows longer than the longest compiled selection workgroup (65536 pages) are routed elsewhere
    long = desc_for(w, max_pages_per_seq=65537, max_list=65537)
    assert select_rc(long, sel_for(w)) == A.SPD_ERR_UNSUPPORTED
    assert fused_rc(long, sel_for(w)) == A.SPD_ERR_UNSUPPORTED
    with pytest.raises(A.SpdError):
        A.spd_workspace_bytes(long, sel_for(w), A.OP_PAGE_SCORE_SELECT)


def test_mvar_estimator_argument_checks(lib):
    wc = W.small(mode="coverage", gamma=0.9, estimator="mvar")
    d = desc_for(wc)
    mv = sel_for(wc, estimator=A.ESTIMATOR_MVAR)
    assert score_rc(d, sel_for(wc, estimator=2)) == A.SPD_ERR_INVALID_ARG           # unknown estimator
    w = W.small()
    assert score_rc(desc_for(w), sel_for(w, estimator=A.ESTIMATOR_MVAR)) == A.SPD_ERR_INVALID_ARG  # top-K
    assert score_rc(d, mv, k_pool=None) == A.SPD_ERR_INVALID_ARG   # the first and last pages read K
    wf = W.small(mode="coverage", gamma=0.9, kv="fp8", estimator="mvar")
    assert score_rc(desc_for(wf), sel_for(wf, estimator=A.ESTIMATOR_MVAR), k_scale=None) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, mv, tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    need = A.spd_workspace_bytes(d, mv, A.OP_PAGE_SCORE)
    assert need == A.spd_workspace_bytes(d, sel_for(wc), A.OP_PAGE_SCORE) > 0
    assert score_rc(d, mv, ws_bytes=need - 1) == A.SPD_ERR_WORKSPACE
    # the fused launch has no mvar estimator
    assert fused_rc(d, mv) == A.SPD_ERR_UNSUPPORTED
    with pytest.raises(A.SpdError):
        A.spd_workspace_bytes(d, mv, A.OP_PAGE_SCORE_SELECT)
    # summary builds: same checks as the key-box build
    stats = A.lib().spd_page_stats_build
    assert stats(ctypes.byref(d), None, None, FAKE, FAKE, None, 0, FAKE, 0) == A.SPD_ERR_INVALID_ARG
    assert stats(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, 0) == A.SPD_ERR_INVALID_ARG  # span >= 1
    assert stats(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, -1, FAKE, 0) == A.SPD_ERR_INVALID_ARG
    assert stats(ctypes.byref(desc_for(wf)), FAKE, None, FAKE, FAKE, None, 0, FAKE, 0) == A.SPD_ERR_INVALID_ARG
    assert stats(ctypes.byref(desc_for(wc, batch=0)), None, None, None, None, None, 0, None, 0) == A.SPD_OK


def test_empty_batch_launches_nothing(lib):
    w = W.small()
    d = desc_for(w, batch=0)
    assert score_rc(d, sel_for(w)) == A.SPD_OK
    assert select_rc(d, sel_for(w)) == A.SPD_OK
    assert fused_rc(d, sel_for(w)) == A.SPD_OK
    assert decode_rc(d, A.PlanParams(4, 16, 512)) == A.SPD_OK


def test_self_planning_worked_example(lib, golden_dir):
    with open(os.path.join(golden_dir, "self_planning_example.json")) as f:
        g = json.load(f)
    used = 0
    for n, c_want, m_want in zip(g["rows"], g["chunk_pages"], g["blocks_used"]):
        c, m = A.spd_plan_chunks(n, g["J"], g["C"])
        assert (c, m) == (c_want, m_want)
        used += m
    assert g["J"] * len(g["rows"]) - used == g["blocks_idle"]
    assert A.spd_plan_chunks(0, 4, 2) == (0, 0)


def test_plan_grid_formula(lib):
    w = W.small()
    for B, Hkv, C, NJ, NT in [(1, 8, 4, 32, 4096), (4, 8, 24, 32, 4096), (8, 8, 4, 16, 512), (1, 2, 1, 1, 0)]:
        d = desc_for(w, batch=B, num_kv_heads=Hkv, num_q_heads=4 * Hkv)
        J = A.spd_plan_grid(d, A.PlanParams(C, NJ, NT))
        assert J == max(NJ, -(-NT // (B * Hkv)))
        po, pl = A.spd_partials_size(d, A.PlanParams(C, NJ, NT))
        assert pl == B * Hkv * J * 4 and po == pl * w.head_dim
    # balanced plan: the grid is N_T + rows and holds one chunk state per block
    for B, Hkv, NT in [(1, 8, 512), (4, 8, 1024), (2, 2, 1)]:
        d = desc_for(w, batch=B, num_kv_heads=Hkv, num_q_heads=4 * Hkv)
        assert A.spd_plan_grid(d, A.PlanParams(4, 16, NT, 1)) == NT + B * Hkv
        po, pl = A.spd_partials_size(d, A.PlanParams(4, 16, NT, 1))
        assert pl == (NT + B * Hkv) * 4 and po == pl * w.head_dim
    d = desc_for(w)
    for bad in (A.PlanParams(4, 16, 0, 1), A.PlanParams(4, 16, 512, 2), A.PlanParams(0, 16, 512, 1)):
        with pytest.raises(A.SpdError):
            A.spd_plan_grid(d, bad)
    # ... and the chunk count it documents never exceeds that grid, nor 1024 chunks in a row
    rng = np.random.default_rng(1)
    for _ in range(300):
        rows, NT, C = int(rng.integers(1, 200)), int(rng.integers(1, 5000)), int(rng.integers(1, 40))
        n = rng.integers(0, 70000, size=rows) * (rng.random(rows) < 0.8)
        T, nmax, z = int(n.sum()), int(n.max()), int((n > 0).sum())
        slots = NT - z if NT > z else NT
        c = max(C, -(-T // slots), -(-nmax // 1024))
        m = -(-n // c)
        assert int(m.sum()) <= NT + rows and int(m.max()) <= 1024
        if NT > z:
            assert int(m.sum()) < NT  # one round of the N_T blocks
    # chunk sizes: every chunk holds at least C pages, at most J chunks, all pages covered once
    rng = np.random.default_rng(0)
    for _ in range(500):
        n, J, C = int(rng.integers(0, 5000)), int(rng.integers(1, 100)), int(rng.integers(1, 40))
        c, m = A.spd_plan_chunks(n, J, C)
        if n == 0:
            assert (c, m) == (0, 0)
            continue
        assert c >= C and m <= J and (m - 1) * c < n <= m * c


def test_hierarchical_paging_argument_checks(lib):
    """64-token physical pages (LServe, "Hierarchical Paging"): both rules, both estimators, the
    unfused entry points and tail modes NONE / SKIP; everything else is reported unsupported."""
    w = W.small(page_size=64, budget=6, n_local=1)
    d = desc_for(w, page_size=64)
    cov = sel_for(w, mode=A.SELECT_COVERAGE, gamma=0.9)
    mv = sel_for(w, mode=A.SELECT_COVERAGE, gamma=0.9, estimator=A.ESTIMATOR_MVAR)
    assert score_rc(d, mv, tail=A.TAIL_REBUILD) == A.SPD_ERR_UNSUPPORTED  # the in-scorer rebuild: 16-token pages
    assert score_rc(d, mv, k_pool=None) == A.SPD_ERR_INVALID_ARG          # exact first / current pages need keys
    assert select_rc(desc_for(w, page_size=64, max_list=w.pages_per_seq - 1), cov) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, cov, ws_bytes=A.spd_workspace_bytes(d, cov, A.OP_PAGE_SCORE) - 1) == A.SPD_ERR_WORKSPACE
    # the coverage log-masses are kept per logical page: four times the 16-token layout's workspace
    flat = desc_for(w, page_size=16, max_pages_per_seq=w.pages_per_seq * 4)
    assert A.spd_workspace_bytes(d, cov, A.OP_PAGE_SCORE) == A.spd_workspace_bytes(flat, cov, A.OP_PAGE_SCORE)
    assert score_rc(d, sel_for(w), tail=A.TAIL_REBUILD) == A.SPD_ERR_UNSUPPORTED
    assert fused_rc(d, sel_for(w)) == A.SPD_ERR_UNSUPPORTED
    assert A.lib().spd_workspace_bytes(ctypes.byref(d), ctypes.byref(sel_for(w)), A.OP_PAGE_SCORE_SELECT) == \
        ctypes.c_size_t(-1).value
    rc = A.lib().spd_page_stats_build(ctypes.byref(d), None, FAKE, FAKE, FAKE, None, 0, FAKE, 0)
    assert rc == A.SPD_ERR_INVALID_ARG
    # f32 pools at d = 128: a logical page's key box spans 32 lanes, more than hierarchical scoring folds
    w32 = W.small(page_size=64, kv="f32", q="f32", d=128, budget=6, n_local=1)
    assert score_rc(desc_for(w32, page_size=64), sel_for(w32)) == A.SPD_ERR_UNSUPPORTED
    assert decode_rc(desc_for(w32, page_size=64), A.PlanParams(4, 16, 512)) == A.SPD_ERR_UNSUPPORTED
    # argument errors are still found first on the supported shapes
    assert score_rc(d, sel_for(w, budget_pages=0)) == A.SPD_ERR_INVALID_ARG
    assert decode_rc(d, A.PlanParams(4, 16, 512), q=None) == A.SPD_ERR_INVALID_ARG


def test_several_query_tokens_argument_checks(lib):
    w = W.small(num_queries=4, budget=6)
    d = desc_for(w, max_list=24)
    plan = A.PlanParams(4, 16, 512)
    L = A.lib()

    def union_rc(desc, T=4, tml=6, **null):
        p = {k: FAKE for k in ("tl", "tn", "bt", "sl", "pl", "pp", "pm", "ll")}
        p.update(null)
        return L.spd_page_list_union(ctypes.byref(desc), T, tml, p["tl"], p["tn"], p["bt"], p["sl"], p["pl"], p["pp"],
                                     p["pm"], p["ll"], None, 0)

    def dec_rc(desc, T=4, pl=plan, **null):
        p = {k: FAKE for k in ("q", "k", "v", "ks", "vs", "bt", "sl", "pl", "pp", "pm", "ll", "o", "lse", "po", "pls")}
        p.update(null)
        return L.spd_sparse_paged_decode_mq(ctypes.byref(desc), T, ctypes.byref(pl), p["q"], p["k"], p["v"], p["ks"],
                                            p["vs"], p["bt"],
                                            p["sl"], p["pl"], p["pp"], p["pm"], p["ll"], ctypes.c_float(0.1), p["o"],
                                            p["lse"], p["po"], p["pls"], 0)

    for T in (0, 5):
        assert union_rc(d, T=T) == A.SPD_ERR_INVALID_ARG
        assert dec_rc(d, T=T) == A.SPD_ERR_INVALID_ARG
    assert union_rc(desc_for(w, max_list=23)) == A.SPD_ERR_INVALID_ARG      # cannot hold 4 lists of 6
    assert union_rc(d, tml=0) == A.SPD_ERR_INVALID_ARG
    assert union_rc(d, pm=None) == A.SPD_ERR_INVALID_ARG
    assert union_rc(d, bt=None) == A.SPD_ERR_INVALID_ARG                    # physical pages wanted
    assert union_rc(desc_for(w, max_list=24, page_size=64)) == A.SPD_ERR_UNSUPPORTED
    assert union_rc(desc_for(w, max_list=24, max_pages_per_seq=40000)) == A.SPD_ERR_UNSUPPORTED
    assert dec_rc(d, pl=A.PlanParams(4, 16, 512, 1)) == A.SPD_ERR_UNSUPPORTED  # per-row plan only
    assert dec_rc(desc_for(W.small(num_queries=4, d=64), max_list=24)) == A.SPD_ERR_UNSUPPORTED
    assert dec_rc(desc_for(W.small(num_queries=4, kv="f32", q="f32"), max_list=24)) == A.SPD_ERR_UNSUPPORTED
    assert dec_rc(desc_for(W.small(num_queries=4, kv="fp8"), max_list=24), ks=None) == A.SPD_ERR_INVALID_ARG
    assert dec_rc(d, pm=None) == A.SPD_ERR_INVALID_ARG
    rc = L.spd_lse_merge_mq(ctypes.byref(d), 4, ctypes.byref(plan), FAKE, None, FAKE, FAKE, FAKE, 0)
    assert rc == A.SPD_ERR_INVALID_ARG

    def score_rc(desc, T=4, sel=None, tail=A.TAIL_NONE, **null):
        p = {k: FAKE for k in ("q", "meta", "bt", "sl", "sc")}
        p.update(null)
        heads = (ctypes.c_uint8 * desc.num_kv_heads)(*([0] * desc.num_kv_heads))
        s = sel if sel is not None else sel_for(w)
        return L.spd_page_score_mq(ctypes.byref(desc), T, ctypes.byref(s), p["q"], p["meta"], tail, p["bt"], p["sl"],
                                   heads, p["sc"], 0)

    for T in (0, 5):
        assert score_rc(d, T=T) == A.SPD_ERR_INVALID_ARG
    for k in ("q", "meta", "bt", "sl", "sc"):
        assert score_rc(d, **{k: None}) == A.SPD_ERR_INVALID_ARG, k
    assert score_rc(d, sel=sel_for(w, mode=A.SELECT_COVERAGE)) == A.SPD_ERR_UNSUPPORTED
    assert score_rc(d, sel=sel_for(w, mode=A.SELECT_COVERAGE, estimator=A.ESTIMATOR_MVAR)) == A.SPD_ERR_UNSUPPORTED
    assert score_rc(desc_for(w, max_list=24, page_size=64)) == A.SPD_ERR_UNSUPPORTED
    assert score_rc(desc_for(w, max_list=24, batch=0)) == A.SPD_OK
    # skipping the last two pages needs them in every token's local window (n_local >= 2)
    assert score_rc(d, sel=sel_for(w, n_local=1), tail=A.TAIL_SKIP) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, tail=A.TAIL_REBUILD) == A.SPD_ERR_INVALID_ARG
    assert score_rc(d, tail=7) == A.SPD_ERR_INVALID_ARG


def test_several_query_token_selection_argument_checks(lib):
    """spd_page_select_mq: token counts, the token lists' capacity, the rule, null pointers."""
    w = W.small(num_queries=4, budget=6, n_sink_stream=2, n_local_stream=3)
    d = desc_for(w, max_list=24)
    L = A.lib()

    def sel_rc(desc, T=4, tml=6, sel=None, **null):
        p = {k: FAKE for k in ("sc", "sl", "bt", "tl", "tp", "tn")}
        p.update({"kp": None, "ks": None, "pm": None})
        p.update(null)
        heads = (ctypes.c_uint8 * desc.num_kv_heads)(*([0] * desc.num_kv_heads))
        s = sel if sel is not None else sel_for(w)
        return L.spd_page_select_mq(ctypes.byref(desc), T, tml, ctypes.byref(s), p["sc"], p["sl"], heads, p["bt"],
                                    p["kp"], p["ks"], p["pm"], p["tl"], p["tp"], p["tn"], 0)

    for T in (0, 5):
        assert sel_rc(d, T=T) == A.SPD_ERR_INVALID_ARG
    assert sel_rc(d, tml=0) == A.SPD_ERR_INVALID_ARG
    assert sel_rc(d, tml=5) == A.SPD_ERR_INVALID_ARG             # cannot hold a budget of 6 pages
    for k in ("sc", "sl", "tl", "tn"):
        assert sel_rc(d, **{k: None}) == A.SPD_ERR_INVALID_ARG, k
    assert sel_rc(d, bt=None) == A.SPD_ERR_INVALID_ARG           # physical pages wanted
    assert sel_rc(d, sel=sel_for(w, mode=A.SELECT_COVERAGE)) == A.SPD_ERR_UNSUPPORTED
    assert sel_rc(desc_for(w, max_list=24, page_size=64)) == A.SPD_ERR_UNSUPPORTED
    assert sel_rc(desc_for(w, max_list=24, max_pages_per_seq=40000)) == A.SPD_ERR_UNSUPPORTED
    assert sel_rc(desc_for(w, max_list=24, batch=0)) == A.SPD_OK
    # the rebuild of the last two pages needs the K pool and the block table
    assert sel_rc(d, pm=FAKE) == A.SPD_ERR_INVALID_ARG
    assert sel_rc(d, pm=FAKE, kp=FAKE, bt=None, tp=None) == A.SPD_ERR_INVALID_ARG
    dq = desc_for(W.small(num_queries=4, budget=6, n_sink_stream=2, n_local_stream=3, kv="fp8"), max_list=24)
    assert sel_rc(dq, pm=FAKE, kp=FAKE) == A.SPD_ERR_INVALID_ARG  # fp8 pools need k_scale


def test_noalloc_decode_rejects_partials_beyond_its_array(lib):
    """spd_sparse_paged_decode_noalloc refuses a descriptor and plan whose chunk partials exceed its
    array, before touching the device; invalid descriptors and plans are refused as elsewhere."""
    w = W.small("noalloc_huge", seq_lens=(100,) * 64, Hkv=64, Hq=256)
    L = A.lib()

    def rc(desc, plan):
        return L.spd_sparse_paged_decode_noalloc(ctypes.byref(desc), ctypes.byref(plan), FAKE, FAKE, FAKE, None, None,
                                                 FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, 0)

    d = desc_for(w)
    assert rc(d, A.PlanParams(4, 1024, 0, 0)) == A.SPD_ERR_WORKSPACE     # 4096 rows x 1024 chunks
    assert rc(d, A.PlanParams(0, 16, 512, 0)) == A.SPD_ERR_INVALID_ARG   # min_chunk < 1
    assert rc(desc_for(w, head_dim=96), A.PlanParams(4, 16, 512, 0)) == A.SPD_ERR_UNSUPPORTED
    assert rc(desc_for(w, batch=0), A.PlanParams(4, 16, 512, 0)) == A.SPD_OK
