"""LiteTopK's gated top-K selection against the ungated one and the oracle (needs a gfx950 GPU).

LiteTopK (section 3.2 "Sampling", "Top-k Selection"; section 3.3 "Predictive Gating"): each row's gate is
predicted from its previous selection, and the selector ranks only the free pages at or above it when
they hold the top K' pages -- else it cuts the whole row.  Either way the lists must be exactly those of
the ungated selection (the same exact top-K with ties in page order), call after call: with no history,
with a history from the same query, from an unrelated query and from the negated query (a gate far off),
and with more candidates than the selector ranks.
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


CASES = {
    "f16_d128": W.small("g_f16", seq_lens=(9000, 700, 37, 2050, 1, 4000), budget=40, Hkv=3, Hq=12, streaming=(1,)),
    "f32_d64": W.small("g_f32", kv="f32", q="f32", d=64, seq_lens=(5000, 37, 2050, 16, 17), budget=30),
    "fp8_d128": W.small("g_fp8", kv="fp8", seq_lens=(6000, 250, 31), budget=64, planted=("fixed", 20)),
    "long_8193": W.small("g_long", seq_lens=(8193 * 16 - 5, 3000), budget=256, Hkv=2, Hq=8, planted=("fixed", 64)),
}


def paths(st, rows):
    return S.gate_paths(st.topk_state, rows)


def run_both(w, d, gated, ungated, where):
    gated.run()
    ungated.run()
    torch.cuda.synchronize()
    assert gated.lists() == ungated.lists(), where
    assert torch.equal(gated.page_phys, ungated.page_phys), where
    assert torch.equal(gated.out, ungated.out) and torch.equal(gated.out_lse, ungated.out_lse), where


def free_rows(w, inp):
    """Dynamic rows whose free pages outnumber the free budget (the rows the gate can serve)."""
    out = []
    for b, L in enumerate(inp.seq_lens):
        n = O.n_pages(L)
        n_forced = len(O.forced_pages(n, w.n_sink, w.n_local))
        for h in range(w.num_kv_heads):
            if not inp.head_kind[h] and n - n_forced > w.budget_pages - n_forced > 0:
                out.append(b * w.num_kv_heads + h)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_gated_selection_equals_ungated_call_after_call(name):
    w = CASES[name]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    gated = S.DecodeStep(w, d)
    assert gated.gated
    ungated = S.DecodeStep(w, d, gated=False)
    rows = w.batch * w.num_kv_heads
    served = free_rows(w, inp)
    say(f"[case] {name}: {len(served)} rows the gate can serve")
    run_both(w, d, gated, ungated, "first call (no history)")
    assert (paths(gated, rows)[:, 0] == 0).all()
    for call in range(2):
        run_both(w, d, gated, ungated, f"same query, call {call + 2}")
        p = paths(gated, rows)
        say(f"  call {call + 2}: rows from candidates {int(p[served, 0].sum())}/{len(served)}, "
            f"candidates seen {p[served, 1].tolist()[:8]}")
        assert p[served, 0].sum() >= len(served) - 1, "the gate from the same query should hold the top K'"
    # the lists are the oracle's (tie rule) on every dynamic row
    meta_ref = O.page_meta_build(inp)
    lists = gated.lists()
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        for h in range(w.num_kv_heads):
            if inp.head_kind[h]:
                continue
            ref = O.topk_scores(O.row_bounds(inp, meta_ref, b, h))
            P.check_topk_list(lists[(b, h)], ref, n, w.budget_pages, O.forced_pages(n, w.n_sink, w.n_local),
                              P.bound_scale(inp, meta_ref, b, h))
    o_ref, lse_ref = O.sparse_paged_decode(inp, lists, w.sm_scale)
    P.check_attention(gated.out.cpu().numpy(), gated.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, name)


@pytest.mark.parametrize("name", ["f16_d128", "fp8_d128"])
def test_gate_from_another_query_stays_exact(name):
    """A gate predicted from unrelated queries, then from the negated queries (scores far from the gate):
    the selector takes the candidates when they still hold the top K' and the whole row otherwise; the
    lists never differ from the ungated selection's."""
    w = CASES[name]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    gated = S.DecodeStep(w, d)
    ungated = S.DecodeStep(w, d, gated=False)
    rows = w.batch * w.num_kv_heads
    run_both(w, d, gated, ungated, "prime")
    q0 = d.q.clone()
    rng = np.random.default_rng(123)
    for label, q in (("unrelated", torch.from_numpy(rng.standard_normal(inp.q.shape).astype(inp.q.dtype))),
                     ("negated", -q0.cpu()), ("scaled x4", q0.cpu() * 4), ("back", q0.cpu())):
        d.q.copy_(q.to(d.q.device))
        run_both(w, d, gated, ungated, label)
        p = paths(gated, rows)
        say(f"  {label}: rows from candidates {int(p[:, 0].sum())}, candidates seen {p[:, 1].tolist()[:8]}")


def test_overflowing_candidates_fall_back():
    """A gate that admits every free page (more candidates than the selector ranks): the whole row is cut,
    exactly, and the next gate is tight again."""
    w = CASES["long_8193"]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    gated = S.DecodeStep(w, d)
    ungated = S.DecodeStep(w, d, gated=False)
    rows = w.batch * w.num_kv_heads
    run_both(w, d, gated, ungated, "prime")
    run_both(w, d, gated, ungated, "gated")
    assert paths(gated, rows)[0, 0] == 1
    # every row's gate set to -inf, still valid: row 0 (8,193 pages) has more free pages than 2,048
    hdr = gated.topk_state[:rows * A.GATE_ROW_BYTES].view(torch.float32).view(rows, 8)
    hdr[:, 0] = float("-inf")
    run_both(w, d, gated, ungated, "overflow")
    p = paths(gated, rows)
    assert p[0, 0] == 0 and p[0, 1] > 2048, p[0]
    run_both(w, d, gated, ungated, "after overflow")
    assert paths(gated, rows)[0, 0] == 1


@pytest.mark.parametrize("name", ["t4", "t3_planted", "t4_fp8", "t4_cap1024"])
def test_mq_gated_token_selection_equals_ungated(name):
    """The several-query step: each token row's gate comes from its previous selection; the token lists,
    unions and outputs equal the ungated step's, call after call."""
    from test_gpu_mq import MQ_SMALL

    w = MQ_SMALL[name]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    gated = S.MQDecodeStep(w, d)
    ungated = S.MQDecodeStep(w, d, gated=False)
    rows = w.batch * w.num_queries * w.num_kv_heads
    for call in range(3):
        gated.run()
        ungated.run()
        torch.cuda.synchronize()
        assert gated.token_lists() == ungated.token_lists(), call
        assert gated.union_lists() == ungated.union_lists(), call
        assert torch.equal(gated.out, ungated.out), call
        p = S.gate_paths(gated.topk_state, rows)
        say(f"  call {call + 1}: token rows from candidates {int(p[:, 0].sum())}/{rows}")
