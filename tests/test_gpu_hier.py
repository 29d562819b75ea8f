"""Hierarchical paging on the GPU against the fp64 oracle (needs a gfx950 GPU).

LServe, "Hierarchical Paging": 64-token physical pages holding four 16-token logical pages;
key statistics per logical page, a physical page scored by the largest bound of its logical
pages, top-K over physical pages, attention over whole physical pages.  Every comparison
calls the library through the C ABI; the rules and tolerances are those of tests/parity.py,
applied to physical pages.
"""
import copy

import numpy as np
import pytest
import torch

from oracle import spd_oracle as O
from sparse_paged_decode_quest_amd import _abi as A
from sparse_paged_decode_quest_amd import step as S
from sparse_paged_decode_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu
NP = 64


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    A.lib()
    yield


def say(*a):
    print(*a, flush=True)


HSMALL = {
    "h_f16_d128": W.small("h_f16_d128", page_size=NP, seq_lens=(700, 37, 2050, 1, 33, 4000, 65), budget=6, n_local=1,
                          Hkv=3, Hq=12, streaming=(1,), n_sink_stream=1, n_local_stream=2),
    "h_f16_d64": W.small("h_f16_d64", page_size=NP, d=64, seq_lens=(513, 300, 2, 129), budget=4, n_local=2),
    "h_fp8_d128": W.small("h_fp8_d128", page_size=NP, kv="fp8", seq_lens=(1500, 250, 31), budget=5, n_local=1),
    "h_f32_d64": W.small("h_f32_d64", page_size=NP, kv="f32", q="f32", d=64, seq_lens=(700, 37, 2050, 16, 17),
                         budget=5, n_local=1),
    # the coverage rule over physical pages: shares of logical pages summed per page
    "h_cov_f16": W.small("h_cov_f16", page_size=NP, mode="coverage", gamma=0.9, n_local=1, seq_lens=(1200, 333, 64, 1),
                         planted=("fixed", 6), delta=("nats", 6.0)),
    "h_cov_f32_d64": W.small("h_cov_f32_d64", page_size=NP, kv="f32", q="f32", d=64, mode="coverage", gamma=0.95,
                             n_local=1, seq_lens=(900, 77), streaming=(0,), n_sink_stream=1, n_local_stream=1),
    # more than 1024 logical pages: the share passes take several workgroups per row
    "h_cov_long": W.small("h_cov_long", page_size=NP, mode="coverage", gamma=0.99, n_local=1, seq_lens=(20000, 5000),
                          Hq=4, Hkv=1, planted=("fixed", 40), delta=("nats", 9.0)),
}
TOPK_SMALL = [k for k in HSMALL if HSMALL[k].mode == "topk"]
COV_SMALL = [k for k in HSMALL if HSMALL[k].mode == "coverage"]


def run_case(w, plan=None, tail="auto"):
    say(f"[case] {w.name} seq={w.seq_lens[:8]} kv={w.kv_dtype} page={w.page_size} seed={w.seed} tail={tail}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, plan=plan, fused=False, tail=tail)
    st.run()
    torch.cuda.synchronize()
    return inp, d, st


def phys_scale(inp, meta, b, h):
    """Per physical page: the largest sum_c |q_gc| max(|kmax_c|, |kmin_c|) over its logical pages and heads."""
    w = inp.workload
    G, g = w.group, NP // 16
    L = int(inp.seq_lens[b])
    n_log = O.n_pages(L)
    lps = np.arange(n_log)
    m = np.abs(meta[inp.block_table[b, lps // g].astype(np.int64), h, lps % g].astype(np.float64)).max(axis=1)
    per_log = (np.abs(inp.q[b, h * G:(h + 1) * G].astype(np.float64)) @ m.T).max(axis=0)
    return np.array([per_log[j * g:(j + 1) * g].max() for j in range(O.hier_n_physical(L, NP))])


def set_lists(st, lists):
    pl = torch.zeros_like(st.page_list)
    pp = torch.zeros_like(st.page_list)
    ll = torch.zeros_like(st.list_len)
    bt = st.d.block_table.cpu()
    for (b, h), lst in lists.items():
        if lst:
            pl[b, h, :len(lst)] = torch.tensor(lst, dtype=torch.int32)
            pp[b, h, :len(lst)] = bt[b, lst]
        ll[b, h] = len(lst)
    st.page_list.copy_(pl)
    st.list_len.copy_(ll)
    st.page_phys.copy_(pp)


def check_rows(inp, st, meta_ref, rows):
    """Scores, lists and physical pages of the given rows; returns the oracle's lists of those rows."""
    w = inp.workload
    scores = st.scores.cpu().numpy()
    lists = st.lists()
    pp = st.page_phys.cpu().numpy()
    oracle_lists = {}
    for b, h in rows:
        n = O.hier_n_physical(inp.seq_lens[b], NP)
        lst = lists[(b, h)]
        assert pp[b, h, :len(lst)].tolist() == inp.block_table[b, lst].tolist(), (b, h)
        if inp.head_kind[h]:
            oracle_lists[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
            assert lst == oracle_lists[(b, h)], (b, h)
            continue
        forced = O.forced_pages(n, w.n_sink, w.n_local)
        if w.mode == "coverage":
            if n == 0:
                oracle_lists[(b, h)] = []
                assert lst == []
                continue
            pi, lse = O.hier_row_shares(inp, meta_ref, b, h)
            P.check_coverage_shares(scores[b, h, :n], pi)
            G = w.group
            head_lse = st.head_lse.cpu().numpy()[b, h * G:(h + 1) * G]
            assert np.allclose(head_lse, lse, rtol=0, atol=1e-4 * np.abs(lse).max()), (b, h)
            P.check_coverage_list(lst, pi, n, w.gamma, forced)
            oracle_lists[(b, h)] = O.select_coverage(pi, n, w.gamma, forced)
            continue
        ref, _ = O.hier_row_scores(inp, meta_ref, b, h)
        scale = phys_scale(inp, meta_ref, b, h)
        if st.tail == "select" and n > 0:  # the scorer skips the last physical page (the local window keeps it)
            assert scores[b, h, n - 1] == -np.inf
            P.check_topk_scores(scores[b, h, :n - 1], ref[:n - 1], scale[:n - 1])
        else:
            P.check_topk_scores(scores[b, h, :n], ref, scale)
        P.check_topk_list(lst, ref, n, w.budget_pages, forced, scale)
        oracle_lists[(b, h)] = O.select_topk(ref, n, w.budget_pages, forced)
    return oracle_lists


@pytest.mark.parametrize("tail", ["none", "select"])
@pytest.mark.parametrize("name", TOPK_SMALL + COV_SMALL)
def test_hier_small_meta_scores_lists_attention(name, tail):
    w = HSMALL[name]
    if w.mode == "coverage" and tail == "select":
        tail = "serial"  # coverage counts the forced pages' shares: their statistics are rebuilt first
    inp, d, st = run_case(w, tail=tail)
    meta_ref = O.hier_meta_build(inp)
    got = P.pool_meta(d.page_meta.cpu().numpy(), inp.block_table, inp.seq_lens, d.num_pool_pages)
    assert np.array_equal(got, meta_ref), "logical page meta differs"
    rows = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    oracle_lists = check_rows(inp, st, meta_ref, rows)
    lists = st.lists()
    o_ref, lse_ref = O.hier_sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    G = w.group
    for (b, h), lst in oracle_lists.items():
        if lists[(b, h)] == lst:
            sl = slice(h * G, (h + 1) * G)
            P.check_attention(out[b, sl], out_lse[b, sl], o_ref[b, sl], lse_ref[b, sl], w.kv_dtype, f"row {b},{h}")
    set_lists(st, oracle_lists)  # decode alone, fed the oracle's lists
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, "oracle lists")


@pytest.mark.parametrize("plan", [S.Plan(1, 1, 0), S.Plan(3, 5, 0), S.Plan(4, 16, 512), S.Plan(1000, 1, 0),
                                  S.Plan(1, 1, 1, True), S.Plan(3, 1, 7, True), S.Plan(4, 16, 1024, True)])
def test_hier_plan_invariance(plan):
    w = HSMALL["h_f16_d128"].replace(budget_pages=20)
    inp, d, st = run_case(w, plan=plan)
    lists = O.hier_page_select(inp, O.hier_meta_build(inp))["lists"]
    o_ref, lse_ref = O.hier_sparse_paged_decode(inp, lists, w.sm_scale)
    set_lists(st, lists)
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, str(plan))


@pytest.mark.parametrize("plan", [None, S.Plan(1, 1, 2, True)], ids=["per_row", "balanced_tiny_grid"])
def test_hier_edge_lengths(plan):
    # empty, single-token, one-logical-page, page-boundary and partial-sub-page requests
    w = W.small("h_edges", page_size=NP, seq_lens=(0, 1, 15, 16, 17, 63, 64, 65, 128, 129, 200, 1000), budget=2,
                n_sink=1, n_local=1, streaming=(1,), n_sink_stream=1, n_local_stream=1, Hkv=2, Hq=8, hole=0.5)
    inp, d, st = run_case(w, plan=plan)
    ref = O.decode_step(inp)
    assert st.lists() == ref["lists"]
    out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))  # empty request
    P.check_attention(out, lse, ref["O"], ref["out_lse"], w.kv_dtype, "edges")


def test_hier_reuse_chunk_of_growing_steps():
    """Reusable page selection over physical pages: each later step keeps the chunk's lists plus the
    current sink and local physical pages, and rebuilds the newest logical page's statistics."""
    reuse = 20
    full = (64 * 20 + 7, 64 * 3 + 60, 64 + 1 + reuse, 700)  # the pools hold keys up to these lengths
    w = W.small("h_reuse", page_size=NP, seq_lens=full, budget=6, n_sink=1, n_local=1, streaming=(1,),
                n_sink_stream=1, n_local_stream=2, Hkv=2, Hq=8)
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    L = np.array(full, dtype=np.int64) - (reuse - 1)
    d.seq_lens.copy_(torch.from_numpy(L.astype(np.int32)))
    st = S.DecodeStep(w, d, fused=False, reuse=reuse)
    st.run()
    torch.cuda.synchronize()
    expect = st.lists()
    for i in range(1, reuse):
        L = L + 1
        d.seq_lens.add_(1)
        st.out.fill_(float("nan"))
        st.reuse_step()
        torch.cuda.synchronize()
        for (b, h), lst in expect.items():
            n = O.hier_n_physical(int(L[b]), NP)
            if inp.head_kind[h]:
                expect[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
            else:
                last = lst[-1] if lst else -1
                expect[(b, h)] = lst + [p for p in O.forced_pages(n, w.n_sink, w.n_local) if p > last]
        got = st.lists()
        assert got == expect, i
        at = copy.copy(inp)
        at.seq_lens = L.astype(inp.seq_lens.dtype)
        o_ref, lse_ref = O.hier_sparse_paged_decode(at, expect, w.sm_scale)
        P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, f"step {i}")
    at = copy.copy(inp)
    at.seq_lens = L.astype(inp.seq_lens.dtype)
    ref = O.hier_meta_build(at)
    got = d.page_meta.cpu().numpy()
    for b, x in enumerate(L):  # the newest logical page holds the statistics of its tokens at the final length
        lp = O.n_pages(int(x)) - 1
        phys = int(inp.block_table[b, lp // 4])
        assert np.array_equal(got[b, :, lp], ref[phys, :, lp % 4]), b


def test_hier_named_workload_in_the_bench_configuration():
    w = W.named("llama3_8b_b1_128k_f16_hier64")
    say(f"[workload] {w.name} seq={w.seq_lens} page={w.page_size} budget={w.budget_pages}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d)  # the benchmark's configuration
    st.run()
    torch.cuda.synchronize()
    assert st.tail == "select"
    meta_ref = O.hier_meta_build(inp)
    got = P.pool_meta(d.page_meta.cpu().numpy(), inp.block_table, inp.seq_lens, d.num_pool_pages)
    rng = np.random.default_rng(7)
    n = O.hier_n_physical(w.seq_lens[0], NP)
    for j in sorted(set(rng.choice(n, size=32, replace=False).tolist()) | {n - 1}):
        phys = int(inp.block_table[0, j])
        assert np.array_equal(got[phys], meta_ref[phys]), j
    dyn = [h for h in range(w.num_kv_heads) if not inp.head_kind[h]]
    strm = [h for h in range(w.num_kv_heads) if inp.head_kind[h]]
    rows = [(0, h) for h in dyn] + [(0, strm[0])]
    oracle_lists = check_rows(inp, st, meta_ref, rows)
    lists = st.lists()
    for (b, h), lst in oracle_lists.items():
        say(f"  row {b},{h}: gpu {len(lists[(b, h)])} pages, same as oracle: {lists[(b, h)] == lst}")
    o_ref, lse_ref = O.hier_sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    G = w.group
    for (b, h), lst in oracle_lists.items():
        sl = slice(h * G, (h + 1) * G)
        if lists[(b, h)] == lst:
            P.check_attention(out[b, sl], out_lse[b, sl], o_ref[b, sl], lse_ref[b, sl], w.kv_dtype, f"step {b},{h}")
    set_lists(st, {**lists, **oracle_lists})
    st.out.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    for (b, h) in oracle_lists:
        sl = slice(h * G, (h + 1) * G)
        P.check_attention(out[b, sl], out_lse[b, sl], o_ref[b, sl], lse_ref[b, sl], w.kv_dtype, f"lists {b},{h}")


@pytest.mark.parametrize("seq", [(1200, 333, 64, 1), (20000, 5000)], ids=["ragged", "long"])
def test_hier_mvar_summaries_shares_lists_attention(seq):
    """Moira's mvar estimate over 64-token pages: bf16 summaries per 16-token logical page, Eq. 2 per
    logical page (the first and current logical pages exact), page share = the sum of its logical
    pages' shares."""
    w = W.small("h_mvar", page_size=NP, mode="coverage", estimator="mvar", gamma=0.95, n_local=1, seq_lens=seq,
                planted=("fixed", 12), delta=("nats", 6.0))
    inp, d, st = run_case(w)
    assert st.tail == "serial"
    stats_ref = O.hier_stats_build(inp)
    got = P.pool_meta(d.page_meta.float().cpu().numpy(), inp.block_table, inp.seq_lens, d.num_pool_pages,
                      fill=np.nan)
    built = np.isfinite(stats_ref)
    assert np.array_equal(got[built], stats_ref[built]), "page summaries differ"
    scores = st.scores.cpu().numpy()
    lists = st.lists()
    oracle_lists = {}
    for b, L in enumerate(w.seq_lens):
        n = O.hier_n_physical(L, NP)
        for h in range(w.num_kv_heads):
            forced = O.forced_pages(n, w.n_sink, w.n_local)
            if n == 0:
                oracle_lists[(b, h)] = []
                continue
            pi, _ = O.hier_row_shares_mvar(inp, stats_ref, b, h)
            P.check_coverage_shares(scores[b, h, :n], pi)
            P.check_coverage_list(lists[(b, h)], pi, n, w.gamma, forced)
            oracle_lists[(b, h)] = O.select_coverage(pi, n, w.gamma, forced)
    o_ref, lse_ref = O.hier_sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    set_lists(st, oracle_lists)
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, "mvar lists")
