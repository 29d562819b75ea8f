"""Decode with the merge in the same launch (the last block of each split row merges it) against the
fp64 oracle (needs a gfx950 GPU).  PersistentKV, section 3.3: the merge of chunk states is exact, so
the fused launch must give the oracle's attention under every plan; its row tickets must be left at
zero for the next call.  Calls go through the C ABI; tolerances are those of tests/parity.py.
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


CASES = {
    "f16_d128": W.small("m_f16", seq_lens=(700, 37, 2050, 1, 33, 4000), budget=60, Hkv=3, Hq=12, streaming=(1,)),
    "fp8_d128": W.small("m_fp8", kv="fp8", seq_lens=(1500, 250, 31), budget=40),
    "f32_d64": W.small("m_f32", kv="f32", q="f32", d=64, seq_lens=(700, 37, 2050, 16, 17), budget=50),
    "coverage": W.small("m_cov", mode="coverage", gamma=0.95, n_local=1, seq_lens=(1200, 333, 64),
                        planted=("fixed", 6), delta=("nats", 5.0)),
}
PLANS = [S.Plan(1, 1, 0), S.Plan(4, 16, 512), S.Plan(2, 3, 0), S.Plan(1, 1, 2, True), S.Plan(4, 16, 1024, True)]


@pytest.mark.parametrize("plan", PLANS, ids=[str(p) for p in PLANS])
@pytest.mark.parametrize("name", list(CASES))
def test_merged_decode_matches_the_oracle_and_leaves_tickets_at_zero(name, plan):
    w = CASES[name]
    print(f"[case] {name} plan={plan}", flush=True)
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, plan=plan, merged=True)
    st.run()
    torch.cuda.synchronize()
    ref = O.decode_step(inp)
    lists = st.lists()
    o_ref, lse_ref = O.sparse_paged_decode(inp, lists, w.sm_scale)  # attention over the GPU's own lists
    for _ in range(2):  # a second call starts from the tickets the first left
        P.check_attention(st.out.cpu().numpy(), st.out_lse.cpu().numpy(), o_ref, lse_ref, w.kv_dtype, name)
        assert int(st.counters.abs().sum()) == 0
        st.out.fill_(float("nan"))
        st.out_lse.fill_(float("nan"))
        st.attend()
        torch.cuda.synchronize()
    assert sum(lists[k] == v for k, v in ref["lists"].items()) >= len(ref["lists"]) - 1


def test_merged_graph_replay_equals_eager():
    w = CASES["f16_d128"]
    inp = W.generate(w)
    d = S.upload(inp)
    S.build_meta(w, d)
    st = S.DecodeStep(w, d, merged=True)
    st.run()
    torch.cuda.synchronize()
    eager = (st.out.clone(), st.out_lse.clone())
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
        assert torch.equal(st.out, eager[0]) and torch.equal(st.out_lse, eager[1])
        assert int(st.counters.abs().sum()) == 0
