"""HIP path vs the fp64 oracle on the same seeded inputs (needs a gfx950 GPU).

Small ragged workloads are compared element by element; the full-size workloads are
compared on sampled pages and rows in the launch configuration the benchmark uses.  The
comparison rules and tolerances are in tests/parity.py.
"""
import numpy as np
import pytest
import torch

from oracle import spd_oracle as O
from sparse_paged_decode_quest_amd import _abi as A
from sparse_paged_decode_quest_amd import step as S
from sparse_paged_decode_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    A.lib()  # raises when libspd.so is not built: there is no fallback
    yield


def say(*a):
    print(*a, flush=True)


def run_case(w, plan=None, fused=True, tail="none"):
    """Generate, upload, bulk-meta, one step.  Returns (inputs, device inputs, step)."""
    say(f"[case] {w.name} seq={w.seq_lens[:8]} kv={w.kv_dtype} mode={w.mode} seed={w.seed} fused={fused} "
        f"tail={tail}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, plan=plan, fused=fused, tail=tail)
    st.run()
    torch.cuda.synchronize()
    return inp, d, st


SMALL = {
    "f32_d64": W.small("f32_d64", kv="f32", q="f32", d=64, seq_lens=(700, 37, 2050, 16, 17), budget=20),
    "f16_d128": W.small("f16_d128", seq_lens=(700, 37, 2050, 1, 33, 4000), budget=24, Hkv=3, Hq=12,
                        streaming=(1,)),
    "f16_d64": W.small("f16_d64", d=64, seq_lens=(513, 300, 2), budget=9, n_local=3),
    "fp8_d128": W.small("fp8_d128", kv="fp8", seq_lens=(1500, 250, 31), budget=16),
    "cov_f16": W.small("cov_f16", mode="coverage", gamma=0.9, n_local=1, seq_lens=(1200, 333, 64),
                       planted=("fixed", 6), delta=("nats", 6.0)),
    "cov_f32": W.small("cov_f32", kv="f32", q="f32", d=64, mode="coverage", gamma=0.95, n_local=1,
                       seq_lens=(900, 77), streaming=(0,)),
    # more than 64 requests (the scorer numbers its work 64 requests at a time), empty ones among them
    "f16_b70": W.small("f16_b70", seq_lens=tuple((i * 977) % 3100 for i in range(70)), budget=12),
    "cov_b66": W.small("cov_b66", mode="coverage", gamma=0.9, n_local=1,
                       seq_lens=tuple((i * 613) % 2900 for i in range(66)), planted=("fixed", 3),
                       delta=("nats", 6.0)),
}


def oracle_row(inp, meta, b, h):
    """Oracle scores, list and score scale of dynamic row (b, h)."""
    w = inp.workload
    n = O.n_pages(inp.seq_lens[b])
    S_ = O.row_bounds(inp, meta, b, h)
    forced = O.forced_pages(n, w.n_sink, w.n_local)
    if w.mode == "topk":
        sc = O.topk_scores(S_)
        return sc, O.select_topk(sc, n, w.budget_pages, forced), forced, None
    pi, lse = O.coverage_shares(S_, int(inp.seq_lens[b]), w.sm_scale) if n else (np.zeros(0), None)
    return pi, (O.select_coverage(pi, n, w.gamma, forced) if n else []), forced, lse


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_meta_scores_lists_attention(name, fused):
    w = SMALL[name]
    inp, d, st = run_case(w, fused=fused)
    meta_ref = O.page_meta_build(inp)
    meta_gpu = P.pool_meta(d.page_meta.cpu().numpy(), inp.block_table, inp.seq_lens, d.num_pool_pages)
    used = np.unique(np.concatenate([inp.block_table[b, :O.n_pages(L)] for b, L in enumerate(w.seq_lens)]))
    assert np.array_equal(meta_gpu[used], meta_ref[used]), "page meta differs"

    scores = st.scores.cpu().numpy()
    lists = st.lists()
    head_lse = st.head_lse.cpu().numpy()
    oracle_lists = {}
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        for h in range(w.num_kv_heads):
            if inp.head_kind[h]:
                oracle_lists[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
                assert lists[(b, h)] == oracle_lists[(b, h)], (b, h)
                continue
            ref, lst, forced, lse = oracle_row(inp, meta_ref, b, h)
            oracle_lists[(b, h)] = lst
            if w.mode == "topk":
                scale = P.bound_scale(inp, meta_ref, b, h)
                P.check_topk_scores(scores[b, h, :n], ref, scale)
                P.check_topk_list(lists[(b, h)], ref, n, w.budget_pages, forced, scale)
            else:
                P.check_coverage_shares(scores[b, h, :n], ref)
                if n:
                    G = w.group
                    assert np.allclose(head_lse[b, h * G:(h + 1) * G], lse, rtol=0, atol=1e-4 * np.abs(lse).max())
                P.check_coverage_list(lists[(b, h)], ref, n, w.gamma, forced)

    # the physical pages written beside the lists are the block-table entries of the listed pages
    pp = st.page_phys.cpu().numpy()
    for (b, h), lst in lists.items():
        assert pp[b, h, :len(lst)].tolist() == inp.block_table[b, lst].tolist(), (b, h)

    # attention over the GPU's own lists where they equal the oracle's
    o_ref, lse_ref = O.sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    G = w.group
    for (b, h), lst in oracle_lists.items():
        if lists[(b, h)] == lst:
            sl = slice(h * G, (h + 1) * G)
            P.check_attention(out[b, sl], out_lse[b, sl], o_ref[b, sl], lse_ref[b, sl], w.kv_dtype, f"row {b},{h}")

    # decode alone, fed the oracle's lists
    set_lists(st, oracle_lists)
    poison_outputs(st)
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, "oracle lists")


def poison_outputs(st):
    """NaN in every output, so a row the decode or merge fails to write cannot pass."""
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))


@pytest.mark.parametrize("plan", [S.Plan(1, 1, 0), S.Plan(2, 3, 0), S.Plan(4, 16, 512), S.Plan(24, 32, 4096),
                                  S.Plan(1000, 1, 0), S.Plan(1, 1, 1, True), S.Plan(2, 1, 3, True),
                                  S.Plan(4, 16, 16, True), S.Plan(4, 16, 1024, True)])
def test_plan_invariance(plan):
    w = SMALL["f16_d128"].replace(budget_pages=60)
    inp, d, st = run_case(w, plan=plan)
    lists = st.lists()
    o_ref, lse_ref = O.sparse_paged_decode(inp, lists_from_oracle(inp), w.sm_scale)
    # decode over oracle lists under this plan
    set_lists(st, lists_from_oracle(inp))
    poison_outputs(st)
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, str(plan))


def lists_from_oracle(inp):
    return O.page_select(inp, O.page_meta_build(inp))["lists"]


def set_lists(st, lists):
    """Page lists (and, when the step keeps them, their physical pages) written by the host."""
    pl = torch.zeros_like(st.page_list)
    ll = torch.zeros_like(st.list_len)
    bt = st.d.block_table.cpu()
    pp = torch.zeros_like(pl)
    for (b, h), lst in lists.items():
        pl[b, h, :len(lst)] = torch.tensor(lst, dtype=torch.int32)
        pp[b, h, :len(lst)] = bt[b, lst] if lst else pp[b, h, :0]
        ll[b, h] = len(lst)
    st.page_list.copy_(pl)
    st.list_len.copy_(ll)
    if st.page_phys is not None:
        st.page_phys.copy_(pp)


@pytest.mark.parametrize("plan", [None, S.Plan(1, 1, 2, True), S.Plan(4, 16, 512, True)],
                         ids=["per_row", "balanced_tiny_grid", "balanced"])
def test_edge_cases_empty_tiny_and_degenerate_rows(plan):
    # lengths 0, 1, 15, 16, 17; budget larger than rows; forced pages overlapping
    w = W.small("edges", seq_lens=(0, 1, 15, 16, 17, 48, 49, 160), budget=3, n_sink=2, n_local=2,
                streaming=(1,), n_sink_stream=3, n_local_stream=3, Hkv=2, Hq=8, hole=0.5)
    inp, d, st = run_case(w, plan=plan)
    ref = O.decode_step(inp)
    assert st.lists() == ref["lists"]
    poison_outputs(st)
    st.attend()
    torch.cuda.synchronize()
    out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))  # empty request
    P.check_attention(out, lse, ref["O"], ref["out_lse"], w.kv_dtype, "edges")


def test_all_heads_tail_rebuild_updates_only_last_pages():
    w = W.small("tail", seq_lens=(333, 48, 1), budget=10)
    inp = W.generate(w)
    d = S.upload(inp)
    st = S.DecodeStep(w, d, fused=False, tail="serial")
    sentinel = 3.0
    d.page_meta.fill_(sentinel)
    st.refresh_tail()
    torch.cuda.synchronize()
    raw = d.page_meta.cpu().numpy()
    got = P.pool_meta(raw, inp.block_table, inp.seq_lens, d.num_pool_pages, fill=sentinel)
    first = [max(O.n_pages(L) - 1, 0) for L in w.seq_lens]
    ref = O.page_meta_build(inp, meta=np.full(got.shape, sentinel, dtype=got.dtype), first_page=first)
    assert np.array_equal(got, ref)
    assert np.all(P.meta_past_rows(raw, w.seq_lens) == sentinel)  # entries past each request untouched


LONG_ROWS = {  # rows long enough for every selector geometry (2, 8, 32 and 64 key slots per lane)
    "f16_8192_pages": dict(seq_lens=(8192 * 16, 3000), budget=256),
    "f16_8193_pages": dict(seq_lens=(8193 * 16 - 7, 2049 * 16), budget=256),
    "fp8_32768_pages": dict(kv="fp8", seq_lens=(32768 * 16,), budget=256, planted=("fixed", 64)),
    "f16_40000_pages": dict(seq_lens=(40000 * 16 - 3, 5), budget=300),
    "cov_8193_pages": dict(mode="coverage", gamma=0.99, n_local=1, seq_lens=(8193 * 16 - 1, 700),
                           planted=("fixed", 40), delta=("nats", 10.0)),
}


@pytest.mark.parametrize("name", list(LONG_ROWS))
def test_fused_score_select_on_long_rows(name):
    """The fused score + select launch on rows of 8,192 to 40,000 pages (the workgroup geometries that
    long contexts take), against the oracle: every dynamic row's scores, its list by the tie rule, and
    attention over the GPU's lists; the unfused step must give the same lists."""
    kw = dict(LONG_ROWS[name])
    w = W.small("long_" + name, Hkv=2, Hq=8, streaming=(1,), n_sink_stream=2, n_local_stream=4, **kw)
    inp, d, st = run_case(w, fused=True, tail="auto")
    meta_ref = O.page_meta_build(inp)
    scores = st.scores.cpu().numpy()
    lists = st.lists()
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        h = 0  # the dynamic head
        ref, lst, forced, _ = oracle_row(inp, meta_ref, b, h)
        say(f"  row b={b} n={n} gpu_len={len(lists[(b, h)])} oracle_len={len(lst)} same={lists[(b, h)] == lst}")
        if w.mode == "topk":
            scale = P.bound_scale(inp, meta_ref, b, h)
            P.check_topk_scores(scores[b, h, :n], ref, scale)
            P.check_topk_list(lists[(b, h)], ref, n, w.budget_pages, forced, scale)
        else:
            P.check_coverage_shares(scores[b, h, :n], ref)
            P.check_coverage_list(lists[(b, h)], ref, n, w.gamma, forced)
        assert lists[(b, 1)] == O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
    o_ref, lse_ref = O.sparse_paged_decode(inp, lists, w.sm_scale)
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, name)
    unfused = S.DecodeStep(w, d, fused=False, tail="none")
    unfused.run()
    torch.cuda.synchronize()
    assert unfused.lists() == lists


@pytest.mark.parametrize("mode", ["topk", "coverage"])
def test_fused_select_equals_unfused(mode):
    kw = dict(budget=40) if mode == "topk" else dict(mode="coverage", gamma=0.9, n_local=1, planted=("fixed", 6),
                                                     delta=("nats", 6.0))
    w = W.small("fused_" + mode, seq_lens=(3000, 700, 37, 0), streaming=(1,), Hkv=2, Hq=8, **kw)
    inp, d, _ = run_case(w, fused=False)
    st = S.DecodeStep(w, d, fused=False, tail="none", keep_sel_scores=True)
    st.run()
    torch.cuda.synchronize()
    lists_unfused = st.lists()
    # the score written beside each listed page of a dynamic row is that page's score
    sc, ss = st.scores.cpu().numpy(), st.sel_scores.cpu().numpy()
    for (b, h), lst in lists_unfused.items():
        if not inp.head_kind[h]:
            assert np.array_equal(ss[b, h, :len(lst)], sc[b, h, lst]), (b, h)
    st2 = S.DecodeStep(w, d, fused=True, tail="none", keep_sel_scores=True)
    for rep in range(3):  # counters must return to zero between calls
        st2.run()
        torch.cuda.synchronize()
        assert st2.lists() == lists_unfused, rep
        assert torch.equal(st2.out, st.out) and torch.equal(st2.out_lse, st.out_lse)
        assert torch.equal(st2.page_phys, st.page_phys) and torch.equal(st2.sel_scores, st.sel_scores)
        for b in range(w.batch):
            n = O.n_pages(w.seq_lens[b])
            assert torch.equal(st2.scores[b, 0, :n], st.scores[b, 0, :n]), (rep, b)  # dynamic head 0
        if mode == "coverage":
            assert torch.equal(st2.head_lse[:, :4], st.head_lse[:, :4])
    rows = w.batch * w.num_kv_heads
    counters = st2.workspace[st2.ws_bytes - (-(-rows * 4 // 256) * 256):].view(torch.int32)
    assert int(counters.abs().sum()) == 0  # tickets back at zero


@pytest.mark.parametrize("fused,tail", [(True, "rebuild"), (True, "side"), (True, "serial"), (False, "rebuild"),
                                        (False, "side"), (False, "serial"), (False, "select")])
def test_step_tail_modes_rebuild_the_last_page(fused, tail):
    """A step rebuilds the statistics of each request's last page, for every KV head, and of no
    other page: in the scorer ("rebuild"), by the meta-build kernel ("side", "serial") or by the
    selector's spare workgroups ("select")."""
    for kv in ("f16", "fp8", "f32"):
        w = W.small("tail_" + kv, kv=kv, q="f32" if kv == "f32" else "f16", d=64 if kv == "f32" else 128,
                    seq_lens=(333, 48, 1, 0), budget=10, streaming=(1,), Hkv=2, Hq=8)
        say(f"[case] tail={tail} fused={fused} kv={kv}")
        inp = W.generate(w)
        d = S.upload(inp)
        S.build_meta(w, d)
        ref_full = d.page_meta.clone()
        d.page_meta.fill_(3.0)  # sentinel everywhere
        st = S.DecodeStep(w, d, fused=fused, tail=tail)
        st.run()
        torch.cuda.synchronize()
        got = d.page_meta.cpu().numpy()
        full = ref_full.cpu().numpy()
        for b, L in enumerate(w.seq_lens):
            n = O.n_pages(L)
            for p in range(n):
                for h in range(w.num_kv_heads):
                    if p == n - 1:
                        assert np.array_equal(got[b, h, p], full[b, h, p]), (kv, b, p, h)
                    else:
                        assert np.all(got[b, h, p] == 3.0), (kv, b, p, h)
        assert np.all(P.meta_past_rows(got, w.seq_lens) == 3.0), kv


@pytest.mark.parametrize("mode", ["topk", "coverage"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_tail_modes_agree_on_current_statistics(mode, fused):
    """With statistics already current, every tail mode gives the lists, physical pages and
    outputs of the plain step bit for bit; the scores too, except that a skipping scorer
    writes -inf for each dynamic row's last page."""
    kw = dict(budget=40) if mode == "topk" else dict(mode="coverage", gamma=0.9, n_local=1, planted=("fixed", 6),
                                                     delta=("nats", 6.0))
    w = W.small("tails_" + mode, seq_lens=(3000, 700, 37, 1, 0, 16, 17), streaming=(1,), Hkv=2, Hq=8, **kw)
    inp, d, ref = run_case(w, fused=fused, tail="none")
    tails = ["rebuild", "serial"] + (["side"] if mode == "topk" else []) + \
        (["select"] if mode == "topk" and not fused else [])
    for tail in tails:
        say(f"  tail={tail}")
        st = S.DecodeStep(w, d, fused=fused, tail=tail)
        for rep in range(2):
            st.run()
            torch.cuda.synchronize()
            assert st.lists() == ref.lists(), (tail, rep)
            for name in ("page_phys", "out", "out_lse"):
                assert torch.equal(getattr(st, name), getattr(ref, name)), (tail, rep, name)
            for b in range(w.batch):
                n = O.n_pages(w.seq_lens[b])
                got, want = st.scores[b, 0, :n].clone(), ref.scores[b, 0, :n]  # dynamic head 0
                if tail in ("side", "select") and n:
                    assert got[n - 1].item() == -np.inf, (tail, b)
                    got[n - 1] = want[n - 1]
                assert torch.equal(got, want), (tail, rep, b)
            if mode == "coverage":
                assert torch.equal(st.head_lse[:, :4], ref.head_lse[:, :4]), tail


def test_balanced_plan_on_skewed_coverage_lists():
    """Coverage lists from the forced pages up to whole rows, decoded under the step-wide split
    and under the per-row split: both match the oracle over the GPU's lists."""
    w = W.small("skew", mode="coverage", gamma=0.97, n_local=1, seq_lens=(16000, 40, 0, 5000, 17, 9000),
                planted=("fixed", 6), delta=("nats", 6.0), Hkv=2, Hq=8)
    inp, d, st = run_case(w, plan=S.Plan(4, 16, 64, True))
    lists = st.lists()
    o_ref, lse_ref = O.sparse_paged_decode(inp, lists, w.sm_scale)
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, "balanced")
    for plan in (S.Plan(), S.Plan(1, 1, 1, True), S.Plan(4, 16, 4096, True)):
        st2 = S.DecodeStep(w, d, plan=plan)
        set_lists(st2, lists)
        poison_outputs(st2)
        st2.attend()
        torch.cuda.synchronize()
        P.check_attention(st2.out.cpu().numpy(), st2.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, str(plan))


@pytest.mark.parametrize("seq", [40000, 131072 + 5], ids=["2500_pages", "8193_pages"])
def test_equal_scores_are_taken_in_page_order(seq):
    """All free pages score the same (every page's key box is the same), so the cut key is shared by
    thousands of pages spread over every wave of the selecting workgroup: the list must be the forced
    pages plus the lowest-numbered free pages."""
    w = W.small("ties", seq_lens=(seq, 3000), budget=300, n_sink=2, n_local=3, Hkv=2, Hq=8)
    inp = W.generate(w)
    d = S.upload(inp)
    d.page_meta.fill_(0.25)  # identical statistics everywhere
    st = S.DecodeStep(w, d, fused=False, tail="none")
    st.run()
    torch.cuda.synchronize()
    lists = st.lists()
    pp = st.page_phys.cpu().numpy()
    for b, L in enumerate(w.seq_lens):
        n = O.n_pages(L)
        forced = O.forced_pages(n, w.n_sink, w.n_local)
        free = [p for p in range(n) if p not in set(forced)]
        want = sorted(set(forced) | set(free[:w.budget_pages - len(forced)]))
        for h in range(w.num_kv_heads):
            assert lists[(b, h)] == want, (b, h)
            assert pp[b, h, :len(want)].tolist() == inp.block_table[b, want].tolist(), (b, h)  # physical pages


@pytest.mark.parametrize("reuse", [4, 20])
def test_reusable_selection_serves_a_chunk_of_growing_steps(reuse):
    """LServe's reusable page selection: the first step of a chunk selects; each later step, one
    token longer, keeps those lists plus the current sink and local pages (a page opened during the
    chunk is appended) and rebuilds the newest page's statistics.  Lists, physical pages and
    attention are checked against the oracle at every length."""
    import copy

    full = (16 * 40 + 2, 16 * 12 + 9, 16 * 3 + 1 + reuse, 700)  # the pools hold keys up to these lengths
    w = W.small("reuse", seq_lens=full, budget=12, n_sink=1, n_local=2, streaming=(1,), n_sink_stream=2,
                n_local_stream=2, Hkv=2, Hq=8)
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
        poison_outputs(st)
        st.reuse_step()
        torch.cuda.synchronize()
        at = copy.copy(inp)
        at.seq_lens = L.astype(inp.seq_lens.dtype)
        expect = O.reuse_lists(at, expect)
        got = st.lists()
        assert got == expect, i
        pp = st.page_phys.cpu().numpy()
        for (b, h), lst in got.items():
            assert pp[b, h, :len(lst)].tolist() == inp.block_table[b, lst].tolist(), (i, b, h)
        at = copy.copy(inp)
        at.seq_lens = L.astype(inp.seq_lens.dtype)
        o_ref, lse_ref = O.sparse_paged_decode(at, expect, w.sm_scale)
        P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, f"step {i}")
    # the newest page of every request holds the statistics of its tokens at the final length
    at = copy.copy(inp)
    at.seq_lens = L.astype(inp.seq_lens.dtype)
    last = [max(O.n_pages(int(x)) - 1, 0) for x in L]
    ref = O.page_meta_build(at, first_page=last)
    got = d.page_meta.cpu().numpy()
    for b, x in enumerate(L):
        phys = int(inp.block_table[b, last[b]])
        assert np.array_equal(got[b, :, last[b]], ref[phys]), b


def test_deterministic_bitwise():
    w = SMALL["cov_f16"]
    inp, d, st = run_case(w)
    a = [t.clone() for t in (st.scores, st.page_list, st.list_len, st.out, st.out_lse)]
    st.run()
    torch.cuda.synchronize()
    b = [st.scores, st.page_list, st.list_len, st.out, st.out_lse]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_graph_replay_equals_eager_and_follows_new_inputs():
    w = W.small("graph", seq_lens=(2500, 900, 60), budget=32, streaming=(0,), Hkv=2, Hq=8)
    inp, d, st = run_case(w, fused=False, tail="side")  # the step's second stream is captured too
    eager = [t.clone() for t in (st.page_list, st.list_len, st.out, st.out_lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(eager, (st.page_list, st.list_len, st.out, st.out_lse)):
            assert torch.equal(x, y), rep
    # new queries in the same buffer: the graph must select and attend for them
    rng = np.random.default_rng(99)
    q2 = rng.standard_normal(inp.q.shape).astype(np.float16)
    d.q.copy_(torch.from_numpy(q2))
    g.replay()
    torch.cuda.synchronize()
    graph_out = [t.clone() for t in (st.page_list, st.list_len, st.out, st.out_lse)]
    st.run()
    torch.cuda.synchronize()
    for x, y in zip(graph_out, (st.page_list, st.list_len, st.out, st.out_lse)):
        assert torch.equal(x, y)
    inp.q = q2
    ref = O.decode_step(inp)
    lists = st.lists()
    for key, lst in ref["lists"].items():
        if lists[key] == lst:
            b, h = key
            sl = slice(h * 4, (h + 1) * 4)
            P.check_attention(st.out.cpu().numpy()[b, sl], st.out_lse.cpu().numpy()[b, sl], ref["O"][b, sl],
                              ref["out_lse"][b, sl], w.kv_dtype, str(key))
