"""A decode step captured once as a graph, replayed while the requests grow (needs a gfx950 GPU).

At replay only device memory changes (Moira, section 3.3 "The constraint"): the lengths advance by
one token per step, as a serving loop appends each decoded token.  The step must read the lengths
on the device, rebuild the statistics of the page the newest token lands in, select and attend over
the grown requests.  Replays run one token at a time, so every page is finalized while it is the
newest; after 1, 15 and 17 more tokens (crossing page boundaries) the page statistics, scores, lists
and attention are checked against the oracle at the current lengths.  Rules and tolerances are those
of tests/parity.py.
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

ADVANCES = (1, 15, 17)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    A.lib()
    yield


def say(*a):
    print(*a, flush=True)


def at_lengths(inp, L):
    """The oracle's view of the inputs at lengths L (the pools hold keys up to the full lengths)."""
    at = copy.copy(inp)
    at.seq_lens = np.asarray(L, dtype=inp.seq_lens.dtype)
    return at


def capture(fn):
    """Warm fn on a side stream, then capture it once."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn(stream.cuda_stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn(stream.cuda_stream)
    return g


def check_meta(at, d, heads=None):
    """Every page of every request holds the statistics of its keys at the current lengths (for the
    given KV heads; all by default)."""
    ref = O.page_meta_build(at)
    got = P.pool_meta(d.page_meta.cpu().numpy(), at.block_table, at.seq_lens, d.num_pool_pages)
    hs = list(range(got.shape[1])) if heads is None else list(heads)
    for b, L in enumerate(at.seq_lens):
        phys = at.block_table[b, :O.n_pages(L)].astype(np.int64)
        assert np.array_equal(got[phys][:, hs], ref[phys][:, hs]), \
            f"request {b}: page statistics differ at length {L}"
    return ref


def check_single_query_step(at, st, meta_ref, where):
    w = at.workload
    scores = st.scores.cpu().numpy()
    lists = st.lists()
    oracle_lists = {}
    for b, L in enumerate(at.seq_lens):
        n = O.n_pages(L)
        for h in range(w.num_kv_heads):
            if at.head_kind[h]:
                oracle_lists[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
                assert lists[(b, h)] == oracle_lists[(b, h)], (where, b, h)
                continue
            S_ = O.row_bounds(at, meta_ref, b, h)
            forced = O.forced_pages(n, w.n_sink, w.n_local)
            if w.mode == "topk":
                ref = O.topk_scores(S_)
                scale = P.bound_scale(at, meta_ref, b, h)
                m = n - 1 if st.tail in ("select", "side") else n  # a skipping scorer writes -inf for the last page
                P.check_topk_scores(scores[b, h, :m], ref[:m], scale[:m])
                P.check_topk_list(lists[(b, h)], ref, n, w.budget_pages, forced, scale)
                oracle_lists[(b, h)] = O.select_topk(ref, n, w.budget_pages, forced)
            else:
                pi, _ = O.coverage_shares(S_, int(L), w.sm_scale) if n else (np.zeros(0), None)
                P.check_coverage_shares(scores[b, h, :n], pi)
                P.check_coverage_list(lists[(b, h)], pi, n, w.gamma, forced)
                oracle_lists[(b, h)] = O.select_coverage(pi, n, w.gamma, forced) if n else []
    # attention over the GPU's own lists (each valid by the rules above), for every row
    o_ref, lse_ref = O.sparse_paged_decode(at, lists, w.sm_scale)
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, where)
    same = sum(lists[k] == v for k, v in oracle_lists.items())
    assert same >= len(oracle_lists) - 1, f"{where}: only {same} of {len(oracle_lists)} lists equal the oracle's"


CASES = {
    "topk_select": (dict(budget=24, streaming=(1,), n_sink_stream=2, n_local_stream=3), dict(fused=False)),
    "topk_fused_rebuild": (dict(budget=24, streaming=(1,), n_sink_stream=2, n_local_stream=3), dict(fused=True)),
    "topk_fp8": (dict(kv="fp8", budget=20), dict(fused=False)),
    "coverage": (dict(mode="coverage", gamma=0.9, n_local=1, planted=("fixed", 6), delta=("nats", 6.0)),
                 dict(fused=False)),
    "topk_merged": (dict(budget=24), dict(fused=False, merged=True)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_single_query_step_replay_follows_growing_lengths(name):
    wkw, skw = CASES[name]
    full = (2050, 100, 40, 700)  # keys exist up to these lengths
    w = W.small("grow_" + name, seq_lens=full, Hkv=3, Hq=12, **wkw)
    inp = W.generate(w)
    d = S.upload(inp)
    L = np.array(full, dtype=np.int64) - sum(ADVANCES)
    d.seq_lens.copy_(torch.from_numpy(L.astype(np.int32)))
    S.build_meta(w, d)  # prefill statistics at the starting lengths
    st = S.DecodeStep(w, d, **skw)
    say(f"[case] {name} tail={st.tail} start={L.tolist()} full={list(full)}")
    # the in-scorer rebuild covers dynamic heads only: streaming heads are never scored
    heads = [h for h in range(w.num_kv_heads) if not inp.head_kind[h]] if st.tail == "rebuild" else None
    g = capture(st.run)
    g.replay()
    torch.cuda.synchronize()
    at = at_lengths(inp, L)
    check_single_query_step(at, st, check_meta(at, d, heads), f"{name} start")
    for adv in ADVANCES:
        for _ in range(adv):
            d.seq_lens.add_(1)  # the serving loop appends a token (outside the graph)
            L = L + 1
            st.out.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        at = at_lengths(inp, L)
        say(f"  lengths {L.tolist()}")
        check_single_query_step(at, st, check_meta(at, d, heads), f"{name} +{adv} -> {L.tolist()}")


def test_mq_step_replay_follows_growing_lengths():
    """The several-query step: each token's causal length is derived from the live lengths, so after
    growth every token selects over its own longer prefix and attends to its newest keys."""
    from test_gpu_mq import check_token_lists

    full = (2050, 100, 40, 700)
    w = W.small("grow_mq", num_queries=4, seq_lens=full, budget=12, Hkv=3, Hq=12, streaming=(1,),
                n_sink_stream=1, n_local_stream=2)
    inp = W.generate(w)
    d = S.upload(inp)
    L = np.array(full, dtype=np.int64) - sum(ADVANCES)
    d.seq_lens.copy_(torch.from_numpy(L.astype(np.int32)))
    S.build_meta(w, d)
    st = S.MQDecodeStep(w, d)
    say(f"[case] mq start={L.tolist()}")
    g = capture(st.run)
    g.replay()
    torch.cuda.synchronize()
    for adv in (0,) + ADVANCES:
        for _ in range(adv):
            d.seq_lens.add_(1)
            L = L + 1
            st.out.fill_(float("nan"))
            g.replay()
        torch.cuda.synchronize()
        at = at_lengths(inp, L)
        meta_ref = check_meta(at, d)
        say(f"  lengths {L.tolist()}")
        gpu_lists, ref_lists = check_token_lists(at, st, meta_ref)
        assert st.union_lists() == O.union_lists(gpu_lists)
        res = O.mq_decode_step(at, meta_ref)
        out, lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
        G, T = w.group, w.num_queries
        same = 0
        for t in range(T):
            # attention of each token over the GPU's own list (valid by the tie rule)
            one = O.mq_token_inputs(at, t)
            o_t, lse_t = O.sparse_paged_decode(one, gpu_lists[t], w.sm_scale)
            P.check_attention(out[:, t], lse[:, t], o_t, lse_t, w.kv_dtype, f"+{adv} token {t}")
            same += sum(gpu_lists[t][k] == v for k, v in ref_lists[t].items())
        assert same >= T * w.batch * w.num_kv_heads - 2
        if same == T * w.batch * w.num_kv_heads:
            P.check_attention(out, lse, res["O"], res["out_lse"], w.kv_dtype, f"+{adv} oracle")
