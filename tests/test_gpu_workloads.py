"""The named full-size workloads on the GPU, in the launch configuration the benchmark
uses, checked against the fp64 oracle: page statistics on sampled pages, and every row's scores,
list and attention (needs a gfx950 GPU)."""
import numpy as np
import pytest
import torch

from oracle import spd_oracle as O
from sparse_paged_decode_quest_amd import _abi as A
from sparse_paged_decode_quest_amd import step as S
from sparse_paged_decode_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


# 64-token pages: test_gpu_hier.py; several query tokens per request: test_gpu_mq.py
@pytest.mark.parametrize("name", [n for n in W.NAMED if W.named(n).page_size == 16 and W.named(n).num_queries == 1])
def test_named_workload(name):
    check_named(name, fused=False)


def test_fp8_512k_fused_score_select():
    """The 512k-context fp8 layer with scoring and selection fused into one launch (the fused top-K
    over 32,768 pages per row)."""
    check_named("fp8_b1_512k", fused=True)


def check_named(name, fused):
    assert torch.cuda.is_available()
    A.lib()
    w = W.named(name)
    say(f"[workload] {name} B={w.batch} seq={w.seq_lens} kv={w.kv_dtype} mode={w.mode} fused={fused}")
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, fused=fused)  # the benchmark's configuration: default plan, tail mode and selector
    st.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)

    # 1. page meta (or mvar summaries) on sampled pages (all heads), exact
    mvar = w.estimator == "mvar"
    meta_gpu = (d.page_meta.float() if mvar else d.page_meta).cpu().numpy()
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        pages = sorted(set(rng.choice(n, size=min(n, 24), replace=False).tolist()) | {n - 1})
        for p in pages:
            phys = int(inp.block_table[b, p])
            valid = O.valid_tokens(inp.seq_lens[b], p)
            for h in range(w.num_kv_heads):
                sc = None if inp.k_scale is None else inp.k_scale[phys, h]
                keys = O.stored_values(inp.k_pool[phys, h], sc, w.kv_dtype)
                if mvar:
                    mu, var = O.page_mean_var(keys, valid)
                    lo, hi = O.round_bf16(mu), O.round_bf16(var)
                else:
                    lo, hi = O.to_stored_meta(*O.page_key_minmax(keys, valid), w.kv_dtype)
                assert np.array_equal(meta_gpu[b, h, p, 0], lo) and np.array_equal(meta_gpu[b, h, p, 1], hi), \
                    (b, p, h)

    # 2. every row: scores, lists (tie rule), attention over the GPU's own lists
    gpu_lists = st.lists()
    gpu_scores = st.scores.cpu().numpy()
    gpu_phys = st.page_phys.cpu().numpy()
    for (b, h), lst in gpu_lists.items():  # the physical page written beside every list entry
        assert gpu_phys[b, h, :len(lst)].tolist() == inp.block_table[b, lst].tolist(), (b, h)
    meta_ref = None if mvar else O.page_meta_build(inp)
    stats_ref = O.page_stats_build(inp) if mvar else None
    oracle_lists = {}
    for b in range(w.batch):
        n = O.n_pages(inp.seq_lens[b])
        for h in range(w.num_kv_heads):
            if inp.head_kind[h]:
                oracle_lists[(b, h)] = O.forced_pages(n, w.n_sink_stream, w.n_local_stream)
                assert gpu_lists[(b, h)] == oracle_lists[(b, h)], (b, h)
                continue
            forced = O.forced_pages(n, w.n_sink, w.n_local)
            if w.mode == "topk":
                ref = O.topk_scores(O.row_bounds(inp, meta_ref, b, h))
                scale = P.bound_scale(inp, meta_ref, b, h)
                if st.tail in ("side", "select"):  # the scorer skips the last page (kept by the local window)
                    assert gpu_scores[b, h, n - 1] == -np.inf
                    P.check_topk_scores(gpu_scores[b, h, :n - 1], ref[:n - 1], scale[:n - 1])
                else:
                    P.check_topk_scores(gpu_scores[b, h, :n], ref, scale)
                P.check_topk_list(gpu_lists[(b, h)], ref, n, w.budget_pages, forced, scale)
                oracle_lists[(b, h)] = O.select_topk(ref, n, w.budget_pages, forced)
            else:
                if mvar:
                    pi, _ = O.shares_from_logmass(O.row_logmass_mvar(inp, stats_ref, b, h))
                else:
                    pi, _ = O.coverage_shares(O.row_bounds(inp, meta_ref, b, h), int(inp.seq_lens[b]), w.sm_scale)
                P.check_coverage_shares(gpu_scores[b, h, :n], pi)
                P.check_coverage_list(gpu_lists[(b, h)], pi, n, w.gamma, forced)
                oracle_lists[(b, h)] = O.select_coverage(pi, n, w.gamma, forced)
    same = sum(gpu_lists[k] == v for k, v in oracle_lists.items())
    say(f"  {same} of {len(oracle_lists)} rows list exactly the oracle's pages (the rest within the tie band)")
    assert same >= 0.9 * len(oracle_lists)
    G = w.group
    out, out_lse = st.out.cpu().numpy(), st.out_lse.cpu().numpy()
    o_gpu_ref, lse_gpu_ref = O.sparse_paged_decode(inp, gpu_lists, w.sm_scale)
    P.check_attention(out, out_lse, o_gpu_ref, lse_gpu_ref, w.kv_dtype, "step over its own lists")

    # 3. decode fed the oracle's lists on every row
    o_ref, lse_ref = O.sparse_paged_decode(inp, oracle_lists, w.sm_scale)
    pl = torch.zeros_like(st.page_list)
    pp = torch.zeros_like(st.page_phys)
    ll = torch.zeros_like(st.list_len)
    for (b, h), lst in oracle_lists.items():
        pl[b, h, :len(lst)] = torch.tensor(lst, dtype=torch.int32)
        pp[b, h, :len(lst)] = torch.from_numpy(inp.block_table[b, lst].astype(np.int32))
        ll[b, h] = len(lst)
    st.page_list.copy_(pl)
    st.list_len.copy_(ll)
    st.page_phys.copy_(pp)
    st.out.fill_(float("nan"))
    st.attend()
    torch.cuda.synchronize()
    P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, "oracle lists")

    if w.mode == "coverage":
        lens = st.list_len.cpu().numpy().ravel()
        say(f"  coverage list lengths: min {lens.min()} median {int(np.median(lens))} max {lens.max()} "
            f"hist {np.histogram(lens, bins=[0, 20, 50, 100, 200, 500, 1000, 2000, 4000, 8193])[0].tolist()}")
