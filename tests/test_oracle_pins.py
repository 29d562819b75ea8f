"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties one oracle function to a closed form, a worked example printed on
the pages (fixtures under tests/golden/ carry the citation), a library routine,
an invariant, or brute force on tiny inputs, chosen so that a dropped term, a
wrong sign or index, or a transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import spd_oracle as O
from sparse_paged_decode_quest_amd import workloads as W


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ fp8 decoding

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3fn_spec_values(golden_dir):
    g = _load(golden_dir, "e4m3fn_known_values.json")
    for item in g["values"]:
        v = float(O.decode_e4m3fn(np.array([int(item["code"], 16)], dtype=np.uint8))[0])
        if item["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == item["value"] and math.copysign(1, v) == math.copysign(1, item["value"])


# ------------------------------------------------------------------ key min / max

def _torch_fp8_values(codes, scale):
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return t.numpy() * scale.astype(np.float64)[..., None]


@pytest.mark.parametrize("kv", ["f32", "f16", "fp8"])
def test_meta_matches_elementwise_loops(kv):
    w = W.small(kv=kv, q="f32" if kv == "f32" else "f16", d=64, seq_lens=(70, 16, 5, 33), Hq=4, Hkv=2,
                seed=11)
    inp = W.generate(w)
    meta = O.page_meta_build(inp)
    for b, L in enumerate(w.seq_lens):
        for p in range((L + 15) // 16):
            phys = inp.block_table[b, p]
            valid = min(16, L - 16 * p)
            for h in range(w.num_kv_heads):
                if kv == "fp8":
                    vals = _torch_fp8_values(inp.k_pool[phys, h], inp.k_scale[phys, h])
                else:
                    vals = inp.k_pool[phys, h].astype(np.float64)
                for c in range(w.head_dim):
                    col = [vals[t, c] for t in range(valid)]
                    lo, hi = min(col), max(col)
                    slo, shi = float(meta[phys, h, 0, c]), float(meta[phys, h, 1, c])
                    if kv == "fp8":
                        # smallest fp16 >= max and largest fp16 <= min
                        assert shi >= hi and float(np.nextafter(np.float16(shi), np.float16(-np.inf))) < hi
                        assert slo <= lo and float(np.nextafter(np.float16(slo), np.float16(np.inf))) > lo
                    else:
                        assert slo == lo and shi == hi


def test_meta_first_page_only_touches_tail():
    w = W.small(seq_lens=(100, 40), d=64, seed=3)
    inp = W.generate(w)
    full = O.page_meta_build(inp)
    sentinel = np.full_like(full, 7.0)
    first = np.array([(100 + 15) // 16 - 1, (40 + 15) // 16 - 1])
    tail = O.page_meta_build(inp, meta=sentinel, first_page=first)
    for b, L in enumerate(w.seq_lens):
        n = (L + 15) // 16
        for p in range(n):
            phys = inp.block_table[b, p]
            if p >= first[b]:
                assert np.array_equal(tail[phys], full[phys])
            else:
                assert np.all(tail[phys] == 7.0)


# ------------------------------------------------------------------ the page bound

def test_bound_is_max_over_box_corners():
    rng = np.random.default_rng(5)
    for _ in range(20):
        d, G = 5, 3
        q = rng.standard_normal((G, d))
        a = rng.standard_normal((1, d))
        b = rng.standard_normal((1, d))
        kmin, kmax = np.minimum(a, b), np.maximum(a, b)
        S = O.quest_bound(q, kmin, kmax)
        for g in range(G):
            best = max(sum(q[g, c] * (kmax[0, c] if bit else kmin[0, c]) for c, bit in enumerate(bits))
                       for bits in itertools.product([0, 1], repeat=d))
            assert abs(S[g, 0] - best) < 1e-12


def test_bound_identical_keys_is_exact_dot():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 64))
    k = rng.standard_normal((1, 64))
    S = O.quest_bound(q, k, k)
    assert np.allclose(S[:, 0], q @ k[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", ["f32", "f16", "fp8"])
def test_bound_upper_bounds_every_key(kv):
    w = W.small(kv=kv, q="f32" if kv == "f32" else "f16", seq_lens=(300, 23, 129), Hq=8, Hkv=2,
                planted=("fixed", 3), seed=21)
    inp = W.generate(w)
    meta = O.page_meta_build(inp)
    G = w.group
    for b, L in enumerate(w.seq_lens):
        n = (L + 15) // 16
        for h in range(w.num_kv_heads):
            S = O.row_bounds(inp, meta, b, h)
            assert S.shape == (G, n)
            for p in range(n):
                K, _ = O.gather_tokens(inp, b, h, [p])
                for g in range(G):
                    qg = inp.q[b, h * G + g].astype(np.float64)
                    tol = 1e-12 * float(np.abs(qg) @ np.abs(K).max(axis=0))
                    assert S[g, p] >= (K @ qg).max() - tol


# ------------------------------------------------------------------ top-K selection

def test_topk_matches_rank_counting():
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(0, 40))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        budget = int(rng.integers(1, 20))
        ns, nl = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        forced = O.forced_pages(n, ns, nl)
        got = O.select_topk(scores, n, budget, forced)
        fset = set(forced)
        others = [p for p in range(n) if p not in fset]
        k_rest = max(0, budget - len(forced))
        want = set(forced)
        for p in others:
            rank = sum(1 for r in others if scores[r] > scores[p] or (scores[r] == scores[p] and r < p))
            if rank < k_rest:
                want.add(p)
        assert got == sorted(want), (trial, n, budget)
        assert got == sorted(got) and len(set(got)) == len(got)


def test_topk_budget_covering_row_keeps_all():
    s = np.arange(10, dtype=np.float64)[::-1]
    assert O.select_topk(s, 10, 10, O.forced_pages(10, 1, 2)) == list(range(10))
    assert O.select_topk(s, 10, 50, O.forced_pages(10, 1, 2)) == list(range(10))


def test_topk_forced_exceeding_budget_is_forced_set():
    s = np.zeros(30)
    assert O.select_topk(s, 30, 2, O.forced_pages(30, 1, 2)) == [0, 28, 29]


def test_streaming_table(golden_dir):
    g = _load(golden_dir, "streaming_index_table.json")
    for c in g["cases"]:
        assert O.forced_pages(c["n_pages"], c["n_sink"], c["n_local"]) == c["table"]


def test_streaming_rows_get_the_static_table():
    w = W.small(seq_lens=(1000, 20), streaming=(1,), n_sink_stream=2, n_local_stream=5, seed=8)
    inp = W.generate(w)
    sel = O.page_select(inp, O.page_meta_build(inp))
    assert sel["lists"][(0, 1)] == [0, 1] + list(range(63 - 5, 63))
    assert sel["lists"][(1, 1)] == [0, 1]  # 20 tokens are 2 pages
    assert sel["scores"][(0, 1)] is None


# ------------------------------------------------------------------ coverage selection

def test_coverage_worked_example(golden_dir):
    g = _load(golden_dir, "coverage_worked_example.json")
    pi = np.array(g["shares"])
    for c in g["cases"]:
        got = O.select_coverage(pi, len(pi), c["gamma"], forced=[])
        assert len(got) == c["kept"] and got == c["pages"]


def test_coverage_minimal_by_enumeration():
    rng = np.random.default_rng(9)
    for trial in range(200):
        n = int(rng.integers(2, 13))
        pi = rng.dirichlet(np.full(n, 0.3))
        gamma = float(rng.uniform(0.3, 0.999))
        forced = O.forced_pages(n, 1, 1)
        got = O.select_coverage(pi, n, gamma, forced)
        others = [p for p in range(n) if p not in forced]
        t = gamma - sum(pi[p] for p in forced)
        assert set(forced) <= set(got)
        if t <= 0:
            assert got == forced
            continue
        best = None
        for r in range(len(others) + 1):
            if any(sum(pi[p] for p in sub) >= t for sub in itertools.combinations(others, r)):
                best = r
                break
        chosen = [p for p in got if p not in forced]
        assert len(chosen) == best, trial
        assert sum(pi[p] for p in chosen) >= t - 1e-12
        # threshold set: every unchosen page has a smaller share than every chosen one
        unchosen = [p for p in others if p not in chosen]
        if chosen and unchosen:
            assert max(pi[p] for p in unchosen) < min(pi[p] for p in chosen)


def test_coverage_ties_at_threshold_are_all_kept():
    pi = np.array([0.0, 0.4, 0.2, 0.2, 0.2, 0.0])
    got = O.select_coverage(pi, 6, 0.55, forced=[0, 5])
    assert got == [0, 1, 2, 3, 4, 5]  # tau = 0.2 and every page with share >= tau is kept


def test_coverage_gamma_one_keeps_all_and_forced_mass_short_circuits():
    rng = np.random.default_rng(10)
    pi = rng.dirichlet(np.ones(50))
    assert O.select_coverage(pi, 50, 1.0, O.forced_pages(50, 1, 1)) == list(range(50))
    pi2 = np.zeros(20)
    pi2[0], pi2[19] = 0.6, 0.4
    assert O.select_coverage(pi2, 20, 0.99, O.forced_pages(20, 1, 1)) == [0, 19]


def test_coverage_shares_normalise_and_lse_matches_library():
    from scipy.special import logsumexp
    rng = np.random.default_rng(12)
    S = rng.standard_normal((4, 37)) * 30
    pi, lse = O.coverage_shares(S, 37 * 16 - 5, 0.125)
    assert abs(pi.sum() - 1.0) < 1e-12
    valid = np.array([16] * 36 + [11], dtype=np.float64)
    ell = 0.125 * S + np.log(valid)
    assert np.allclose(lse, logsumexp(ell, axis=1), rtol=0, atol=1e-12)
    # the share of a page grows with its bound (monotone in every head)
    S2 = S.copy()
    S2[:, 3] += 1.0
    pi2, _ = O.coverage_shares(S2, 37 * 16 - 5, 0.125)
    assert pi2[3] > pi[3]


# ------------------------------------------------------------------ mvar (Moira Eq. 2)

def test_mean_var_hand_example():
    keys = np.array([[1.0, 2.0], [3.0, 6.0], [9.0, 9.0]])
    mu, var = O.page_mean_var(keys, 2)  # the third row is not a valid token
    assert mu.tolist() == [2.0, 4.0]
    assert var.tolist() == [1.0, 4.0]  # population variance: ((1-2)^2 + (3-2)^2) / 2


def test_bf16_rounding_matches_library():
    import torch
    rng = np.random.default_rng(26)
    x32 = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000)),
                          # exact halfway cases between neighbouring bf16 values, both parities
                          (np.arange(1, 2000) * 2 + 1) * 2.0 ** -8, -(np.arange(1, 2000) * 2 + 1) * 2.0 ** -8,
                          [0.0, -0.0, 2.0 ** -133, 3 * 2.0 ** -134, 3.3e38]]).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_stored_stats_are_the_rounded_mean_and_variance():
    w = W.small(mode="coverage", estimator="mvar", gamma=0.9, seq_lens=(40,), Hq=4, Hkv=1, seed=27)
    inp = W.generate(w)
    st = O.page_stats_build(inp)
    for p, valid in ((0, 16), (2, 8)):
        phys = int(inp.block_table[0, p])
        keys = inp.k_pool[phys, 0, :valid].astype(np.float64)
        assert np.array_equal(st[phys, 0, 0], O.round_bf16(keys.mean(axis=0)))
        assert np.array_equal(st[phys, 0, 1], O.round_bf16(keys.var(axis=0)))  # numpy's var: population


def test_mvar_identical_keys_is_the_exact_page_mass():
    rng = np.random.default_rng(21)
    k = rng.standard_normal(64)
    q = rng.standard_normal((4, 64))
    keys = np.repeat(k[None, :], 11, axis=0)
    mu, var = O.page_mean_var(keys, 11)
    ell = O.mvar_logmass(q, mu[None], var[None], np.array([11.0]), 0.125)[:, 0]
    assert np.allclose(ell, O.exact_logmass(q, keys, 0.125), rtol=0, atol=1e-12)
    assert np.allclose(ell, 0.125 * q @ k + np.log(11.0), rtol=0, atol=1e-12)  # closed form


def test_mvar_is_the_gaussian_expectation():
    """Eq. 2 is log(S * E[exp(s q.k)]) for keys independent Gaussian per channel: check it against a
    Monte Carlo average over many drawn keys (seeded)."""
    rng = np.random.default_rng(22)
    d, S, s = 16, 16.0, 0.25
    mu = rng.standard_normal(d) * 0.5
    var = rng.uniform(0.1, 0.6, d)
    q = rng.standard_normal((3, d))
    keys = mu[None, :] + rng.standard_normal((400_000, d)) * np.sqrt(var)[None, :]
    mc = np.log(S * np.exp(s * keys @ q.T).mean(axis=0))
    ell = O.mvar_logmass(q, mu[None], var[None], np.array([S]), s)[:, 0]
    assert np.allclose(ell, mc, rtol=0, atol=0.01), (ell, mc)
    # dropping the variance term is off by far more than the sampling error
    assert np.abs(ell - (s * q @ mu + np.log(S))).max() > 0.05


def test_exact_logmass_matches_library():
    from scipy.special import logsumexp
    rng = np.random.default_rng(23)
    q, keys = rng.standard_normal((4, 32)), rng.standard_normal((13, 32)) * 3
    assert np.allclose(O.exact_logmass(q, keys, 0.2), logsumexp(0.2 * keys @ q.T, axis=0), rtol=0, atol=1e-12)


def test_mvar_two_page_rows_give_the_exact_page_shares():
    """With one or two pages, the first and current pages are exact, so the shares equal the
    dense softmax mass of each page's tokens, averaged over the group."""
    w = W.small(mode="coverage", estimator="mvar", gamma=0.9, seq_lens=(31, 9, 16), Hq=8, Hkv=2, seed=24)
    inp = W.generate(w)
    stats = O.page_stats_build(inp)
    G = w.group
    for b, L in enumerate(w.seq_lens):
        n = O.n_pages(L)
        for h in range(w.num_kv_heads):
            pi, lse = O.shares_from_logmass(O.row_logmass_mvar(inp, stats, b, h))
            K, _ = _dense_unpaged(inp, b, h)
            q = inp.q[b, h * G:(h + 1) * G].astype(np.float64)
            x = w.sm_scale * q @ K.T  # [G, L]
            prob = np.exp(x - x.max(axis=1, keepdims=True))
            prob /= prob.sum(axis=1, keepdims=True)
            want = np.array([prob[:, 16 * p:16 * (p + 1)].sum(axis=1).mean() for p in range(n)])
            assert np.allclose(pi, want, rtol=0, atol=1e-12), (b, h)


def test_mvar_selection_runs_the_coverage_rule():
    w = W.small(mode="coverage", estimator="mvar", gamma=0.9, n_local=1, seq_lens=(1200, 333, 40), Hq=8, Hkv=2,
                planted=("fixed", 6), delta=("nats", 6.0), seed=25)
    inp = W.generate(w)
    stats = O.page_stats_build(inp)
    sel = O.page_select(inp, O.page_meta_build(inp), stats)
    for (b, h), lst in sel["lists"].items():
        n = O.n_pages(w.seq_lens[b])
        pi, _ = O.shares_from_logmass(O.row_logmass_mvar(inp, stats, b, h))
        assert lst == O.select_coverage(pi, n, w.gamma, O.forced_pages(n, w.n_sink, w.n_local))
        assert abs(pi.sum() - 1) < 1e-12


# ------------------------------------------------------------------ attention

def _dense_unpaged(inp, b, h):
    """Contiguous keys / values of request b, KV head h, read token by token."""
    L = int(inp.seq_lens[b])
    w = inp.workload
    ks, vs = [], []
    for t in range(L):
        phys = inp.block_table[b, t // 16]
        if w.kv_dtype == "fp8":
            ks.append(_torch_fp8_values(inp.k_pool[phys, h, t % 16][None], inp.k_scale[phys, h, t % 16][None])[0])
            vs.append(_torch_fp8_values(inp.v_pool[phys, h, t % 16][None], inp.v_scale[phys, h, t % 16][None])[0])
        else:
            ks.append(inp.k_pool[phys, h, t % 16].astype(np.float64))
            vs.append(inp.v_pool[phys, h, t % 16].astype(np.float64))
    return np.array(ks), np.array(vs)


def _sdpa(q, K, V, scale):
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    lse = torch.logsumexp(torch.from_numpy(K @ q) * scale, dim=0)
    return o[0, 0, 0].numpy(), float(lse)


@pytest.mark.parametrize("kv,mode", [("f32", "topk"), ("f16", "topk"), ("fp8", "topk"), ("f16", "coverage")])
def test_all_pages_equals_dense_attention(kv, mode):
    seq = (333, 48, 17)
    w = W.small(kv=kv, q="f32" if kv == "f32" else "f16", seq_lens=seq, Hq=8, Hkv=2,
                mode=mode, budget=1000, gamma=1.0, seed=13)
    inp = W.generate(w)
    res = O.decode_step(inp)
    G = w.group
    for b in range(len(seq)):
        for h in range(w.num_kv_heads):
            assert res["lists"][(b, h)] == list(range((seq[b] + 15) // 16))
            K, V = _dense_unpaged(inp, b, h)
            for g in range(G):
                qh = inp.q[b, h * G + g].astype(np.float64)
                o_ref, lse_ref = _sdpa(qh, K, V, w.sm_scale)
                assert np.allclose(res["O"][b, h * G + g], o_ref, rtol=0, atol=1e-12)
                assert abs(res["out_lse"][b, h * G + g] - lse_ref) < 1e-12


def test_streaming_attention_is_dense_over_sink_and_local_tokens():
    w = W.small(seq_lens=(500,), streaming=(0,), n_sink_stream=2, n_local_stream=3, Hq=4, Hkv=2, seed=14)
    inp = W.generate(w)
    res = O.decode_step(inp)
    K, V = _dense_unpaged(inp, 0, 0)
    keep = list(range(32)) + list(range(29 * 16, 500))  # pages 0,1 and 29,30,31 (last partial)
    for g in range(2):
        qh = inp.q[0, g].astype(np.float64)
        o_ref, lse_ref = _sdpa(qh, K[keep], V[keep], w.sm_scale)
        assert np.allclose(res["O"][0, g], o_ref, rtol=0, atol=1e-12)
        assert abs(res["out_lse"][0, g] - lse_ref) < 1e-12


def test_split_merge_is_exact():
    rng = np.random.default_rng(15)
    q = rng.standard_normal(64)
    K = rng.standard_normal((200, 64)) * 3
    V = rng.standard_normal((200, 64))
    o_ref, lse_ref = O.attention(q, K, V, 0.125)
    for _ in range(20):
        cuts = sorted(rng.choice(np.arange(1, 200), size=int(rng.integers(1, 8)), replace=False))
        bounds = [0, *cuts, 200]
        states = [O.split_state(q, K[a:b], V[a:b], 0.125) for a, b in zip(bounds[:-1], bounds[1:])]
        states.append(O.split_state(q, K[:0], V[:0], 0.125))  # an empty split is neutral
        o, lse = O.merge_states(states)
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12) and abs(lse - lse_ref) < 1e-12


def test_empty_row_convention():
    o, lse = O.attention(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 0.5)
    assert np.all(o == 0) and lse == -np.inf


# ------------------------------------------------------------------ the generator

def test_generator_is_deterministic():
    w = W.small(kv="fp8", seq_lens=(90, 31), seed=16)
    a, b = W.generate(w), W.generate(w)
    for name in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "block_table", "seq_lens", "head_kind"):
        x, y = getattr(a, name), getattr(b, name)
        assert x.tobytes() == y.tobytes(), name
    c = W.generate(w, seed=17)
    assert c.q.tobytes() != a.q.tobytes()


def test_partial_pages_and_holes_hold_nan_yet_results_are_finite():
    w = W.small(seq_lens=(37, 5), hole=0.5, seed=18)
    inp = W.generate(w)
    assert np.isnan(inp.k_pool[inp.block_table[0, 2], :, 5:]).all()
    res = O.decode_step(inp)
    assert np.isfinite(res["O"]).all() and np.isfinite(res["out_lse"]).all()


def test_tiny_workload_selects_its_planted_pages():
    w = W.named("tiny_b1_hq8_d64_4k_f32")
    inp = W.generate(w)
    res = O.decode_step(inp)
    for h in range(2):
        lst = res["lists"][(0, h)]
        assert len(lst) == 32
        # a +2 sigma shift along the query direction lifts the bound by about two standard
        # deviations of its spread over N(0, 1) pages, so most (not all) planted pages rank high
        hit = len(set(inp.planted[(0, h)].tolist()) & set(lst))
        assert hit >= 5, hit


# ---------------------------------------------------------------------------------- reuse rule

def _reuse_inputs(seq_lens, streaming=(1,)):
    w = W.small("reuse_pin", seq_lens=seq_lens, budget=6, n_sink=1, n_local=2, streaming=streaming,
                n_sink_stream=2, n_local_stream=2, Hkv=2, Hq=8)
    return W.generate(w)


def test_reuse_rule_worked_example():
    """Hand-worked: a top-K list selected at 12 pages, reused one token later (13 pages): the newly
    opened page 12 is appended; page 10, local when selected, stays; the streaming row follows the length."""
    import copy

    inp = _reuse_inputs((16 * 12,))
    sel = {(0, 0): [0, 5, 9, 10, 11], (0, 1): [0, 1, 10, 11]}
    later = copy.copy(inp)
    later.seq_lens = np.array([16 * 12 + 1], dtype=inp.seq_lens.dtype)
    got = O.reuse_lists(later, sel)
    assert got[(0, 0)] == [0, 5, 9, 10, 11, 12]
    assert got[(0, 1)] == [0, 1, 11, 12]


def test_reuse_rule_is_the_selection_when_lengths_do_not_change():
    """At the chunk's first step's own lengths the reused lists are the selected lists: every forced page
    is already listed (a selection always holds the sink and the local window)."""
    inp = _reuse_inputs((700, 37, 2050, 16, 17))
    sel = O.page_select(inp, O.page_meta_build(inp))["lists"]
    assert O.reuse_lists(inp, sel) == sel


@pytest.mark.parametrize("grow", [1, 15, 16, 17, 40])
def test_reuse_rule_keeps_the_chunk_and_the_current_forced_pages(grow):
    """After growth every reused dynamic list is ascending without repeats, holds the chunk's selection
    and the current sink and local pages, adds only pages that did not exist or were past the old last
    entry, and is at most the chunk's list plus the pages opened since."""
    import copy

    full = np.array([700, 37, 2050, 16, 17]) + 40
    inp = _reuse_inputs(tuple(int(x) for x in full))
    first = copy.copy(inp)
    first.seq_lens = (full - 40).astype(inp.seq_lens.dtype)
    sel = O.page_select(first, O.page_meta_build(first))["lists"]
    later = copy.copy(inp)
    later.seq_lens = (full - 40 + grow).astype(inp.seq_lens.dtype)
    got = O.reuse_lists(later, sel)
    w = inp.workload
    for (b, h), lst in got.items():
        n_old, n_new = O.n_pages(first.seq_lens[b]), O.n_pages(later.seq_lens[b])
        if inp.head_kind[h]:
            assert lst == list(range(min(2, n_new))) + [p for p in range(max(2, n_new - 2), n_new)]
            continue
        assert lst == sorted(set(lst))
        assert set(sel[(b, h)]) <= set(lst)
        assert set(O.forced_pages(n_new, w.n_sink, w.n_local)) <= set(lst)
        added = [p for p in lst if p not in set(sel[(b, h)])]
        assert all(p > max(sel[(b, h)]) for p in added)
        assert len(lst) <= len(sel[(b, h)]) + (n_new - n_old)
