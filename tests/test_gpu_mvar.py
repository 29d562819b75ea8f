"""Moira's mvar page estimate on the GPU against the fp64 oracle (needs a gfx950 GPU).

The page summaries (key mean / variance rounded to bf16) are compared for equality; the shares,
per-head log-sum-exps, lists and attention of whole steps with the coverage tolerances of
tests/parity.py.
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
    A.lib()
    yield


def say(*a):
    print(*a, flush=True)


MVAR = {
    "f16_d128": W.small("mvar_f16_d128", mode="coverage", estimator="mvar", gamma=0.9, n_local=1, Hkv=3, Hq=12,
                        seq_lens=(1200, 333, 40, 16, 17, 1), streaming=(1,), planted=("fixed", 6),
                        delta=("nats", 6.0), seed=W.BASE_SEED + 60),
    "f32_d64": W.small("mvar_f32_d64", kv="f32", q="f32", d=64, mode="coverage", estimator="mvar", gamma=0.95,
                       n_local=1, seq_lens=(900, 77, 31), seed=W.BASE_SEED + 61),
    "fp8_d128": W.small("mvar_fp8_d128", kv="fp8", mode="coverage", estimator="mvar", gamma=0.9, n_local=2,
                        seq_lens=(1500, 250, 2), planted=("fixed", 4), delta=("nats", 5.0), seed=W.BASE_SEED + 62),
    "f16_d64": W.small("mvar_f16_d64", d=64, mode="coverage", estimator="mvar", gamma=0.8, n_sink=2, n_local=0,
                       seq_lens=(513, 300, 32), seed=W.BASE_SEED + 63),
    # more than 64 requests: the scan's work is numbered 64 requests at a time
    "f16_b67": W.small("mvar_f16_b67", mode="coverage", estimator="mvar", gamma=0.9, n_local=1,
                       seq_lens=tuple((i * 541) % 2300 + 1 for i in range(67)), planted=("fixed", 3),
                       delta=("nats", 6.0), seed=W.BASE_SEED + 64),
}


def used_pages(inp):
    return np.unique(np.concatenate([inp.block_table[b, :O.n_pages(L)] for b, L in enumerate(inp.seq_lens)]))


def stats_host(d, inp):
    """The device's page summaries in the oracle's layout (with their physical pages; others 0)."""
    return P.pool_meta(d.page_meta.float().cpu().numpy().astype(np.float64), inp.block_table, inp.seq_lens,
                       d.num_pool_pages)


def last_pages(w):
    """(request, logical page) of each non-empty request's newest page."""
    return [(b, O.n_pages(L) - 1) for b, L in enumerate(w.seq_lens) if L > 0]


def set_pages(d, pages, value):
    """Overwrite the device's summaries of the given (request, logical page) pairs, every KV head."""
    for b, p in pages:
        d.page_meta[b, :, p] = value


@pytest.mark.parametrize("name", list(MVAR))
def test_page_summaries_equal_the_rounded_statistics(name):
    w = MVAR[name]
    say(f"[stats] {name} seq={w.seq_lens} kv={w.kv_dtype} d={w.head_dim}")
    inp = W.generate(w)
    d = S.upload(inp)
    assert d.page_meta.dtype == torch.bfloat16
    S.build_meta(w, d)
    torch.cuda.synchronize()
    ref = O.page_stats_build(inp)
    got = stats_host(d, inp)
    u = used_pages(inp)
    assert np.array_equal(got[u], ref[u]), f"{np.sum(got[u] != ref[u])} summary values differ"
    # the last page of each request only (span 1 from the end), over a zeroed buffer
    d.page_meta.zero_()
    S.build_summaries(w, d, None, 1)
    torch.cuda.synchronize()
    got = stats_host(d, inp)
    last = [O.n_pages(L) - 1 for L in w.seq_lens]
    ref_last = O.page_stats_build(inp, first_page=last)
    for b, p in enumerate(last):
        phys = int(inp.block_table[b, p])
        assert np.array_equal(got[phys], ref_last[phys]), (b, p)
    others = np.setdiff1d(u, [int(inp.block_table[b, p]) for b, p in enumerate(last)])
    assert np.all(got[others] == 0)


def run_mvar(w, tail="auto", plan=None):
    say(f"[case] {w.name} seq={w.seq_lens} kv={w.kv_dtype} tail={tail} seed={w.seed}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, plan=plan, tail=tail)
    return inp, d, st


def check_rows(inp, st, stats_ref):
    """Shares, head lse and lists of every row against the oracle; returns the oracle's lists."""
    w = inp.workload
    ref = O.page_select(inp, None, stats_ref)
    scores = st.scores.cpu().numpy()
    head_lse = st.head_lse.cpu().numpy()
    lists = st.lists()
    G = w.group
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        for h in range(w.num_kv_heads):
            if inp.head_kind[h]:
                assert lists[(b, h)] == ref["lists"][(b, h)], (b, h)
                continue
            pi = ref["scores"][(b, h)]
            P.check_coverage_shares(scores[b, h, :n], pi)
            lse = ref["lse"][(b, h)]
            assert np.allclose(head_lse[b, h * G:(h + 1) * G], lse, rtol=0, atol=1e-4 * max(1.0, np.abs(lse).max()))
            P.check_coverage_list(lists[(b, h)], pi, n, w.gamma, O.forced_pages(n, w.n_sink, w.n_local))
    return ref["lists"]


@pytest.mark.parametrize("name", list(MVAR))
def test_mvar_step_scores_lists_attention(name):
    w = MVAR[name]
    inp, d, st = run_mvar(w)
    assert st.tail == "rebuild"
    # the scorer must rebuild the current pages' summaries: clear them first
    last_phys = [int(inp.block_table[b, O.n_pages(L) - 1]) for b, L in enumerate(w.seq_lens) if L > 0]
    set_pages(d, last_pages(w), 0)
    st.run()
    torch.cuda.synchronize()
    stats_ref = O.page_stats_build(inp)
    got = stats_host(d, inp)
    dyn = [h for h in range(w.num_kv_heads) if not inp.head_kind[h]]  # streaming heads keep no summaries
    assert np.array_equal(got[last_phys][:, dyn], stats_ref[last_phys][:, dyn]), "current-page summaries not rebuilt"
    oracle_lists = check_rows(inp, st, stats_ref)
    lists = st.lists()
    pp = st.page_phys.cpu().numpy()
    for (b, h), lst in lists.items():
        assert pp[b, h, :len(lst)].tolist() == inp.block_table[b, lst].tolist(), (b, h)
    o_ref, lse_ref = O.sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    G = w.group
    same = 0
    for (b, h), lst in oracle_lists.items():
        if lists[(b, h)] == lst:
            same += 1
            sl = slice(h * G, (h + 1) * G)
            P.check_attention(out[b, sl], out_lse[b, sl], o_ref[b, sl], lse_ref[b, sl], w.kv_dtype, f"row {b},{h}")
    say(f"  rows with the oracle's list: {same} of {len(oracle_lists)}")


def test_tail_none_scores_the_current_page_exactly_too():
    """Without the rebuild the current page's summary is neither read nor written: a stale
    summary there changes nothing."""
    w = MVAR["f16_d128"]
    inp, d, st = run_mvar(w, tail="none")
    set_pages(d, last_pages(w), 7.0)  # stale
    st.run()
    torch.cuda.synchronize()
    assert all(torch.all(d.page_meta[b, :, p] == 7.0) for b, p in last_pages(w))
    check_rows(inp, st, O.page_stats_build(inp))


def test_first_and_current_pages_are_exact():
    """Summaries of the first pages poisoned to huge values: the shares do not move, since those
    pages are computed from the keys."""
    w = MVAR["f32_d64"]
    inp, d, st = run_mvar(w, tail="none")
    st.run()
    torch.cuda.synchronize()
    before = st.scores.clone()
    set_pages(d, [(b, 0) for b in range(w.batch)], 1e30)
    st.run()
    torch.cuda.synchronize()
    assert torch.equal(st.scores, before)


def test_mvar_reuse_chunk_rebuilds_the_newest_summaries():
    """A reuse step (list refresh) after the requests grew writes the newest page's summary, so the
    next selection sees the summaries the oracle builds from the keys."""
    w = MVAR["f16_d128"]
    inp = W.generate(w)
    grown = [max(0, L - 20) for L in w.seq_lens]  # the chunk's first step saw shorter requests
    d = S.upload(inp)
    st = S.DecodeStep(w, d, reuse=32)
    d.seq_lens.copy_(torch.tensor(grown, dtype=torch.int32))
    torch.cuda.synchronize()
    S.build_meta(w, d)
    st.run()
    d.seq_lens.copy_(torch.tensor(w.seq_lens, dtype=torch.int32))
    torch.cuda.synchronize()
    st.reuse_step()
    torch.cuda.synchronize()
    got = stats_host(d, inp)
    ref = O.page_stats_build(inp)
    last_phys = [int(inp.block_table[b, O.n_pages(L) - 1]) for b, L in enumerate(w.seq_lens) if L > 0]
    assert np.array_equal(got[last_phys], ref[last_phys])
