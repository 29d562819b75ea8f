"""Pins of the oracle's multi-query step (CPU only).

LiteTopK, section 3.4 (LiteDSA): each query token keeps its own top-k list; the lists of a group
are scanned as one union, with a per-query membership mask so that each query still attends to
exactly its own candidates.  Here the query tokens are T draft tokens of one decode step, each
attending causally.  The tests tie the oracle to dense causal attention read token by token, to
the single-query step, and to brute-force set membership.
"""
import numpy as np
import pytest
import torch

from oracle import spd_oracle as O
from sparse_paged_decode_quest_amd import workloads as W


def _mq(**kw):
    base = dict(seq_lens=(333, 48, 1000, 17), Hq=8, Hkv=2, num_queries=4, budget=6, n_sink=1, n_local=2,
                planted=("fixed", 3), streaming=(1,), n_sink_stream=1, n_local_stream=2, seed=91)
    base.update(kw)
    return W.small("mq", **base)


def _sdpa(q, K, V, scale):
    qt = torch.from_numpy(q)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, torch.from_numpy(K)[None, None],
                                                         torch.from_numpy(V)[None, None], scale=scale)
    return o[0, 0, 0].numpy(), float(torch.logsumexp(torch.from_numpy(K @ q) * scale, dim=0))


def test_one_query_token_is_the_single_query_step():
    w = _mq(num_queries=1)
    inp = W.generate(w)
    inp.q = inp.q[:, None]  # [B, 1, Hq, d]
    res = O.mq_decode_step(inp)
    inp.q = inp.q[:, 0]
    ref = O.decode_step(inp)
    assert res["lists_by_token"][0] == ref["lists"]
    assert np.array_equal(res["O"][:, 0], ref["O"]) and np.array_equal(res["out_lse"][:, 0], ref["out_lse"])


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_every_page_listed_is_dense_causal_attention(kv):
    w = _mq(kv=kv, q="f32" if kv == "f32" else "f16", d=64, budget=1000, streaming=())
    inp = W.generate(w)
    res = O.mq_decode_step(inp)
    T, G = w.num_queries, w.group
    for b, L in enumerate(w.seq_lens):
        for h in range(w.num_kv_heads):
            for t in range(T):
                Lt = L - T + 1 + t  # query t sits at position L - T + t
                ks = [inp.k_pool[inp.block_table[b, x // 16], h, x % 16].astype(np.float64) for x in range(Lt)]
                vs = [inp.v_pool[inp.block_table[b, x // 16], h, x % 16].astype(np.float64) for x in range(Lt)]
                for g in range(G):
                    o_ref, lse_ref = _sdpa(inp.q[b, t, h * G + g].astype(np.float64), np.array(ks), np.array(vs),
                                           w.sm_scale)
                    assert np.allclose(res["O"][b, t, h * G + g], o_ref, rtol=0, atol=1e-12)
                    assert abs(res["out_lse"][b, t, h * G + g] - lse_ref) < 1e-12


def test_union_holds_every_listed_page_once_with_its_tokens_bits():
    w = _mq()
    inp = W.generate(w)
    res = O.mq_decode_step(inp)
    for (b, h), (pages, masks) in res["union"].items():
        assert pages == sorted(set(pages))
        n = -(-int(w.seq_lens[b]) // 16)
        for p in range(n):
            bits = sum(1 << t for t in range(w.num_queries) if p in res["lists_by_token"][t][(b, h)])
            if bits:
                assert masks[pages.index(p)] == bits, (b, h, p)
            else:
                assert p not in pages


def test_last_query_token_selects_as_the_single_query_step_at_full_length():
    w = _mq()
    inp = W.generate(w)
    res = O.mq_decode_step(inp)
    one = O.mq_token_inputs(inp, w.num_queries - 1)
    assert np.array_equal(one.seq_lens, inp.seq_lens)
    assert res["lists_by_token"][-1] == O.decode_step(one)["lists"]


def test_causal_lengths():
    assert O.mq_lengths(100, 4) == [97, 98, 99, 100]
    assert O.mq_lengths(1, 1) == [1]
