"""The decode entry point that allocates nothing (needs a gfx950 GPU).

spd_sparse_paged_decode_noalloc keeps its chunk partials in the library's own device array; it
must give what spd_sparse_paged_decode followed by spd_lse_merge gives with caller-allocated
partials, call after call -- the second call here has fewer requests and shorter lists than the
first, so it runs over what the first left in the array -- and both must match the oracle.
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


def say(*a):
    print(*a, flush=True)


def run_both(w, plan):
    """One step's lists, then attention through both entry points on the same lists."""
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, plan=plan)
    st.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = st.out.clone(), st.out_lse.clone()
    out = torch.full_like(st.out, float("nan"))
    lse = torch.full_like(st.out_lse, float("nan"))
    A.spd_sparse_paged_decode_noalloc(st.desc, st.pp, d.q, d.k_pool, d.v_pool, d.k_scale, d.v_scale, d.block_table,
                                      d.seq_lens, st.page_list, st.page_phys, st.list_len, w.sm_scale, out, lse)
    torch.cuda.synchronize()
    return inp, st, ref_out, ref_lse, out, lse


@pytest.mark.parametrize("plan", [S.Plan(), S.Plan(4, 16, 1024, True), S.Plan(1, 1, 0)],
                         ids=["per_row", "balanced", "one_chunk"])
def test_noalloc_decode_matches_the_allocating_entry_points(plan):
    assert torch.cuda.is_available()
    A.lib()
    first = W.small("noalloc_big", seq_lens=(9000, 700, 37, 2050, 4000, 16, 3000, 5000), budget=200, Hkv=4, Hq=16,
                    streaming=(1,), n_sink_stream=2, n_local_stream=5)
    second = W.small("noalloc_small", seq_lens=(300, 41), budget=9, Hkv=2, Hq=8, seed=W.BASE_SEED + 77)
    for w in (first, second):
        say(f"[case] {w.name} plan={plan} B={w.batch} Hkv={w.num_kv_heads}")
        inp, st, ref_out, ref_lse, out, lse = run_both(w, plan)
        assert torch.equal(out, ref_out), w.name
        assert torch.equal(lse, ref_lse), w.name
        o_ref, lse_ref = O.sparse_paged_decode(inp, st.lists(), w.sm_scale)
        P.check_attention(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, w.name)
