"""Several query tokens per request on the GPU against the fp64 oracle (needs a gfx950 GPU).

LiteTopK, section 3.4 (LiteDSA): each draft token selects its own pages; the tokens' lists are
scanned as one union with a membership mask per entry, and each token attends to exactly its own
list over its causal prefix.  Every call goes through the C ABI; rules and tolerances are those of
tests/parity.py.
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


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    A.lib()
    yield


def say(*a):
    print(*a, flush=True)


MQ_SMALL = {
    "t4": W.small("mq_t4", num_queries=4, seq_lens=(700, 37, 2050, 3, 17, 4000), budget=12, Hkv=3, Hq=12,
                  streaming=(1,), n_sink_stream=1, n_local_stream=2),
    "t2": W.small("mq_t2", num_queries=2, seq_lens=(513, 300, 2, 129), budget=9, n_local=3),
    "t3_planted": W.small("mq_t3", num_queries=3, seq_lens=(1500, 250, 31), budget=16, planted=("fixed", 8),
                          delta=3.0),
    "t4_fp8": W.small("mq_fp8", num_queries=4, kv="fp8", seq_lens=(1500, 250, 31, 3), budget=16,
                      streaming=(0,), n_sink_stream=1, n_local_stream=2),
    # four token lists of 256 entries: the union's capacity is exactly 1024 entries (the rank merge's limit)
    "t4_cap1024": W.small("mq_cap", num_queries=4, seq_lens=(9000, 4100, 700), budget=256, Hkv=2, Hq=8),
    # more than 64 requests: the scan's work is numbered 64 requests at a time
    "t2_b66": W.small("mq_b66", num_queries=2, seq_lens=tuple((i * 733) % 2600 + 4 for i in range(66)), budget=9),
}


def run_case(w, plan=None):
    say(f"[case] {w.name} T={w.num_queries} seq={w.seq_lens[:8]} seed={w.seed} plan={plan}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.MQDecodeStep(w, d, plan=plan)
    st.run()
    torch.cuda.synchronize()
    return inp, d, st


def check_token_lists(inp, st, meta_ref):
    """Each token's page scores (tolerance of parity.py) and lists (tie rule) against the oracle's, on
    every token row; returns the GPU's and the oracle's lists.  A step whose scan skips each request's
    last two pages (the "select" tail) holds -inf there, and the lists take those pages as forced."""
    w = inp.workload
    T = w.num_queries
    gpu = st.token_lists()
    scores = st.scores.cpu().numpy()
    want = []
    for t in range(T):
        one = O.mq_token_inputs(inp, t)
        ref = {}
        for b in range(w.batch):
            n = O.n_pages(one.seq_lens[b])
            for h in range(w.num_kv_heads):
                if inp.head_kind[h]:
                    ref[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
                    assert gpu[t][(b, h)] == ref[(b, h)], (t, b, h)
                    continue
                S_ = O.row_bounds(one, meta_ref, b, h)
                sc = O.topk_scores(S_)
                scale = P.bound_scale(one, meta_ref, b, h)
                k = max(O.n_pages(inp.seq_lens[b]) - 2, 0) if st.tail == "select" else n
                P.check_topk_scores(scores[b * T + t, h, :min(k, n)], sc[:min(k, n)], scale[:min(k, n)])
                assert np.all(scores[b * T + t, h, k:n] == -np.inf), (t, b, h)
                forced = O.forced_pages(n, w.n_sink, w.n_local)
                P.check_topk_list(gpu[t][(b, h)], sc, n, w.budget_pages, forced, scale)
                ref[(b, h)] = O.select_topk(sc, n, w.budget_pages, forced)
        want.append(ref)
    return gpu, want


def set_union(st, union):
    pl = torch.zeros_like(st.page_list)
    pp = torch.zeros_like(st.page_phys)
    pm = torch.zeros_like(st.page_mask)
    ll = torch.zeros_like(st.list_len)
    bt = st.d.block_table.cpu()
    for (b, h), (pages, masks) in union.items():
        if pages:
            pl[b, h, :len(pages)] = torch.tensor(pages, dtype=torch.int32)
            pp[b, h, :len(pages)] = bt[b, pages]
            pm[b, h, :len(pages)] = torch.tensor(masks, dtype=torch.int32)
        ll[b, h] = len(pages)
    for dst, src in ((st.page_list, pl), (st.page_phys, pp), (st.page_mask, pm), (st.list_len, ll)):
        dst.copy_(src)


@pytest.mark.parametrize("wide", [False, True], ids=["bytemap_union", "rank_union"])
@pytest.mark.parametrize("name", list(MQ_SMALL))
def test_mq_lists_union_attention(name, wide):
    # block tables of 16384 pages take the union kernel's rank merge of the sorted token lists
    w = MQ_SMALL[name].replace(max_pages_per_seq=16384) if wide else MQ_SMALL[name]
    inp, d, st = run_case(w)
    meta_ref = O.page_meta_build(inp)
    assert np.array_equal(P.pool_meta(d.page_meta.cpu().numpy(), inp.block_table, inp.seq_lens, d.num_pool_pages),
                          meta_ref)
    gpu_lists, ref_lists = check_token_lists(inp, st, meta_ref)
    # the union is exact integer work: it must be the union of the GPU's own token lists
    union = st.union_lists()
    assert union == O.union_lists(gpu_lists)
    # and it was built the intended way: ascending token lists of at most 1,024 entries on a 16,384-page
    # table are merged by rank, every other row in the byte map
    path = torch.full((w.batch, w.num_kv_heads), -1, dtype=torch.int32, device="cuda")
    st.union(path=path)
    torch.cuda.synchronize()
    assert st.token_cap * w.num_queries <= 1024
    assert (path.cpu().numpy() == (1 if wide else 0)).all(), path.cpu().numpy()
    assert st.union_lists() == union
    pp = st.page_phys.cpu().numpy()
    for (b, h), (pages, _) in union.items():
        assert pp[b, h, :len(pages)].tolist() == inp.block_table[b, pages].tolist()
    # attention of every token over its own list, where the GPU's lists equal the oracle's
    res = O.mq_decode_step(inp, meta_ref)
    out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    G = w.group
    same = 0
    for t in range(w.num_queries):
        for (b, h), lst in ref_lists[t].items():
            if gpu_lists[t][(b, h)] == lst:
                sl = slice(h * G, (h + 1) * G)
                P.check_attention(out[b, t, sl], lse[b, t, sl], res["O"][b, t, sl], res["out_lse"][b, t, sl],
                                  w.kv_dtype, f"token {t} row {b},{h}")
                same += 1
    assert same >= w.num_queries * w.batch * w.num_kv_heads - 2
    # decode fed the oracle's union
    set_union(st, res["union"])
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), res["O"], res["out_lse"], w.kv_dtype,
                      "oracle union")


SCORE_ONLY = {
    "d64_f16": W.small("mq_s64", num_queries=3, d=64, seq_lens=(513, 300, 2, 129, 4000), budget=9, Hkv=3, Hq=12,
                       streaming=(2,)),
    "d128_f32": W.small("mq_s32", num_queries=4, kv="f32", q="f32", seq_lens=(1500, 250, 31, 3), budget=16),
    "dense_short": W.small("mq_dense", num_queries=4, seq_lens=(333, 48, 17, 5, 2), budget=1000, Hkv=2, Hq=8),
}


def per_token_scores(w, d, st):
    """The token rows' scores from the single-query scorer: a descriptor of B * T rows whose block-table
    rows and key statistics repeat each request's and whose lengths are the tokens' causal lengths (built
    here, in the test, only to compare the two scorers)."""
    T = w.num_queries
    seq_x = torch.tensor([max(L - T + 1 + t, 0) for L in d.seq_lens.cpu().tolist() for t in range(T)],
                         dtype=torch.int32, device=d.q.device)
    bt_x = d.block_table.repeat_interleave(T, dim=0).contiguous()
    meta_x = d.page_meta.repeat_interleave(T, dim=0).contiguous()
    desc_x = S.make_desc(w.replace(seq_lens=tuple(w.seq_lens) * T), d.num_pool_pages, st.token_cap)
    q_x = d.q.view(w.batch * T, w.num_q_heads, w.head_dim)
    out = torch.full_like(st.scores, float("nan"))
    head_lse = torch.zeros((w.batch * T, w.num_q_heads), dtype=torch.float32, device=d.q.device)
    A.spd_page_score(desc_x, st.sel, q_x, meta_x, d.k_pool, d.k_scale, A.TAIL_NONE, bt_x, seq_x, d.head_kind,
                     out, head_lse, None, 0)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(MQ_SMALL) + list(SCORE_ONLY))
def test_mq_one_scan_scores_match_the_oracle(name):
    """The one-scan scorer of the T token rows against the oracle's bound on every token's pages (the
    tolerance of parity.py), and bit for bit against the single-query scorer run on each token row;
    streaming heads are left untouched."""
    w = MQ_SMALL.get(name) or SCORE_ONLY[name]
    say(f"[case] {name} T={w.num_queries} d={w.head_dim} kv={w.kv_dtype} seq={w.seq_lens[:8]}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.MQDecodeStep(w, d)
    st.refresh_tail()
    st.scores.fill_(float("nan"))
    st.score(tail_mode=A.TAIL_NONE)
    torch.cuda.synchronize()
    one = st.scores.clone()
    # skipping the last two pages: the same scores elsewhere, -inf on those pages where a token sees them
    st.scores.fill_(float("nan"))
    st.score(tail_mode=A.TAIL_SKIP)
    torch.cuda.synchronize()
    skip = st.scores.clone()
    per = per_token_scores(w, d, st)
    meta_ref = O.page_meta_build(inp)
    got = one.cpu().numpy()
    T = w.num_queries
    for t in range(T):
        tok = O.mq_token_inputs(inp, t)
        for b in range(w.batch):
            n_t = O.n_pages(tok.seq_lens[b])
            r = b * T + t
            for h in range(w.num_kv_heads):
                if inp.head_kind[h]:
                    assert torch.isnan(one[r, h]).all()
                    continue
                ref = O.topk_scores(O.row_bounds(tok, meta_ref, b, h))
                P.check_topk_scores(got[r, h, :n_t], ref, P.bound_scale(tok, meta_ref, b, h))
                assert torch.equal(one[r, h, :n_t], per[r, h, :n_t]), (b, t, h)
                k = max(O.n_pages(inp.seq_lens[b]) - 2, 0)
                assert torch.equal(skip[r, h, :min(k, n_t)], one[r, h, :min(k, n_t)]), (b, t, h)
                assert torch.all(skip[r, h, k:n_t] == float("-inf")), (b, t, h)
                assert torch.isnan(skip[r, h, n_t:]).all(), (b, t, h)


@pytest.mark.parametrize("name", ["t4", "t4_fp8", "t2"])
def test_mq_last_pages_rebuilt_beside_the_selection(name):
    """The default step skips each request's last two pages in the scan and rebuilds their statistics in
    the selector's spare workgroups: exactly those pages' statistics are written (all KV heads, equal to
    the oracle's), the other entries are left alone, and the lists, unions and outputs are those of the
    step that rebuilds the pages before a scan over every page."""
    w = MQ_SMALL[name]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    serial = S.MQDecodeStep(w, d, tail="serial")
    sel = S.MQDecodeStep(w, d, gated=False)
    assert sel.tail == "select"
    serial.run()
    torch.cuda.synchronize()
    sentinel = 3.0
    full = d.page_meta.clone()
    d.page_meta.fill_(sentinel)
    sel.select()
    torch.cuda.synchronize()
    got = d.page_meta.cpu().numpy()
    ref = full.cpu().numpy()
    for b, L in enumerate(w.seq_lens):
        n = O.n_pages(L)
        for p in range(got.shape[2]):
            want = ref[b, :, p] if n - 2 <= p < n else np.full_like(got[b, :, p], sentinel)
            assert np.array_equal(got[b, :, p], want), (name, b, p)
    d.page_meta.copy_(full)
    sel.run()
    torch.cuda.synchronize()
    assert sel.token_lists() == serial.token_lists()
    assert sel.union_lists() == serial.union_lists()
    assert torch.equal(sel.out, serial.out) and torch.equal(sel.out_lse, serial.out_lse)
    assert torch.equal(d.page_meta, full)


@pytest.mark.parametrize("plan", [S.Plan(1, 1, 0), S.Plan(2, 3, 0), S.Plan(4, 16, 512), S.Plan(1000, 1, 0)])
def test_mq_plan_invariance(plan):
    w = MQ_SMALL["t4"].replace(budget_pages=40)
    inp, d, st = run_case(w, plan=plan)
    res = O.mq_decode_step(inp)
    set_union(st, res["union"])
    st.out.fill_(float("nan"))
    st.out_lse.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), res["O"], res["out_lse"], w.kv_dtype, str(plan))


def test_mq_every_page_listed_is_dense_causal_attention():
    # budget above every row: each token attends to its whole causal prefix
    w = W.small("mq_dense", num_queries=4, seq_lens=(333, 48, 17, 5, 2), budget=1000, Hkv=2, Hq=8)
    inp, d, st = run_case(w)
    res = O.mq_decode_step(inp)
    assert st.union_lists() == res["union"]
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), res["O"], res["out_lse"], w.kv_dtype, "dense")
    out = st.out.cpu().numpy()
    assert np.all(out[4, :2] == 0)  # two keys, four draft tokens: the first two tokens see no key


@pytest.mark.parametrize("name", [n for n in W.NAMED if W.named(n).num_queries > 1])
def test_mq_named_workload_in_the_bench_configuration(name):
    w = W.named(name)
    inp, d, st = run_case(w)
    meta_ref = O.page_meta_build(inp)
    gpu_lists, ref_lists = check_token_lists(inp, st, meta_ref)
    union = st.union_lists()
    assert union == O.union_lists(gpu_lists)
    for h in range(w.num_kv_heads):
        say(f"  head {h}: union {len(union[(0, h)][0])} pages, token lists "
            f"{[len(gpu_lists[t][(0, h)]) for t in range(w.num_queries)]}")
    res = O.mq_decode_step(inp, meta_ref)
    set_union(st, res["union"])
    st.out.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), res["O"], res["out_lse"], w.kv_dtype,
                      "oracle union")


def test_mq_graph_replay_equals_eager():
    """The whole several-query step captured once replays bit for bit, with eager work between replays,
    and follows new queries written into the same buffer."""
    w = MQ_SMALL["t4"]
    inp, d, st = run_case(w)
    eager = [t.clone() for t in (st.out, st.out_lse, st.page_list, st.page_mask, st.list_len)]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        st.run(stream.cuda_stream)
    stream.synchronize()
    with torch.cuda.graph(g, stream=stream):
        st.run(stream.cuda_stream)
    for _ in range(3):
        st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (st.out, st.out_lse, st.page_list, st.page_mask, st.list_len)):
            assert torch.equal(a, b)
    # new queries in the same buffer: the replay follows them
    inp.q[:] = inp.q[:, ::-1]
    d.q.copy_(torch.from_numpy(np.ascontiguousarray(inp.q)))
    g.replay()
    torch.cuda.synchronize()
    res = O.mq_decode_step(inp)
    gpu_lists = st.token_lists()
    G = w.group
    out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    for t in range(w.num_queries):
        for (b, h), lst in res["lists_by_token"][t].items():
            if gpu_lists[t][(b, h)] == lst:
                sl = slice(h * G, (h + 1) * G)
                P.check_attention(out[b, t, sl], lse[b, t, sl], res["O"][b, t, sl], res["out_lse"][b, t, sl],
                                  w.kv_dtype, f"replay token {t} row {b},{h}")


@pytest.mark.parametrize("factor", [1e5, 1e-3], ids=["large_v", "small_v"])
def test_mq_fp8_value_scales_at_both_ends(factor):
    """fp8 V scales far above and below the usual (V amax about 3e5 and 3e-3): the decode's fp16
    probability operand carries each scale relative to its page's largest, so neither overflows to inf
    nor loses precision in fp16 subnormals.  Attention is linear in V, so outputs are compared after
    dividing by the factor."""
    w = MQ_SMALL["t4_fp8"]
    inp = W.generate(w)
    vs = inp.v_scale.astype(np.float64) * factor
    assert np.isfinite(vs[np.isfinite(inp.v_scale)]).all() and vs[np.isfinite(vs)].max() < 65504
    inp.v_scale = vs.astype(np.float16)
    say(f"[case] v_scale x {factor}: stored scales {np.nanmin(inp.v_scale):.3g} .. {np.nanmax(inp.v_scale):.3g}")
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.MQDecodeStep(w, d)
    st.run()
    torch.cuda.synchronize()
    res = O.mq_decode_step(inp)
    gpu_lists = st.token_lists()
    out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    assert np.isfinite(out).all()
    G = w.group
    for t in range(w.num_queries):
        for (b, h), lst in res["lists_by_token"][t].items():
            if gpu_lists[t][(b, h)] == lst:
                sl = slice(h * G, (h + 1) * G)
                P.check_attention(out[b, t, sl] / factor, lse[b, t, sl], res["O"][b, t, sl] / factor,
                                  res["out_lse"][b, t, sl], w.kv_dtype, f"x{factor} token {t} row {b},{h}")
