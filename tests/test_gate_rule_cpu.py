"""The rule behind LiteTopK's gated selection, checked on the CPU against the oracle's top-K (no GPU).

LiteTopK (section 3.2 "Top-k Selection", section 3.3 "Predictive Gating") ranks only the candidates that
pass a gate, and falls back when fewer than k pass.  The selector's gate is predicted from the previous
selection; whatever its value, the claim it relies on is: when at least K' free pages score at or above the
gate, the top K' free pages by (score desc, page asc) -- ties at the K'-th included -- are all candidates,
so selecting among the candidates gives the whole row's list.  The cases draw scores with many ties
(small integer grids) and gates at, between and around the scores, including gates that admit exactly K'
pages, and check the oracle's selection over the candidates against its selection over the row whenever
the candidates number at least K'.  A gate that admits fewer must not be trusted: such cases are counted
and some of them must differ from the whole-row list, so the test would notice a fallback that is missing.
"""
import numpy as np

from oracle import spd_oracle as O


def candidates_select(scores, n, budget, forced, gate):
    """The oracle's top-K with the free pages restricted to those scoring at or above `gate`."""
    fset = set(forced)
    k_rest = budget - len(forced)
    cand = [p for p in range(n) if p not in fset and scores[p] >= gate]
    order = sorted(cand, key=lambda p: (-float(scores[p]), p))
    return sorted(fset | set(order[:k_rest])), len(cand)


def test_candidates_hold_the_top_k_whenever_enough_pass():
    rng = np.random.default_rng(20261203)
    checked = short = short_differs = 0
    for case in range(600):
        n = int(rng.integers(5, 120))
        levels = int(rng.integers(2, 12))
        scores = rng.integers(0, levels, size=n).astype(np.float64) * float(rng.choice([1.0, 0.25, -0.5]))
        if case % 3 == 0:
            scores = scores + rng.standard_normal(n) * 1e-3  # mostly distinct, near-ties
        forced = O.forced_pages(n, int(rng.integers(0, 3)), int(rng.integers(0, 4)))
        budget = len(forced) + int(rng.integers(1, max(2, n - len(forced))))
        if budget - len(forced) >= n - len(forced):
            continue  # every free page is kept: nothing to rank
        full = O.select_topk(scores, n, budget, forced)
        free = np.array([scores[p] for p in range(n) if p not in set(forced)])
        gates = set(np.quantile(free, rng.random(6)).tolist()) | set(np.unique(free)[:4].tolist())
        kth = np.sort(free)[::-1][budget - len(forced) - 1]
        gates |= {kth, np.nextafter(kth, np.inf), np.nextafter(kth, -np.inf), -np.inf, np.inf}
        for g in gates:
            got, count = candidates_select(scores, n, budget, forced, g)
            if count >= budget - len(forced):
                assert got == full, (case, g, count)
                checked += 1
            else:
                short += 1
                short_differs += got != full
    assert checked > 2000 and short > 500
    assert short_differs > 0.9 * short  # too few candidates: the lists differ, so the fallback is needed


def test_gate_at_the_kth_score_admits_every_tie():
    # ties at the K'-th score straddle the cut: a gate at that score admits all of them, and the cut among
    # the candidates still takes them in page order
    scores = np.array([5, 3, 3, 3, 1, 3, 0, 3], dtype=np.float64)
    n, budget, forced = 8, 3, []
    full = O.select_topk(scores, n, budget, forced)
    assert full == [0, 1, 2]
    got, count = candidates_select(scores, n, budget, forced, 3.0)
    assert count == 6 and got == full
    got, count = candidates_select(scores, n, budget, forced, np.nextafter(3.0, np.inf))
    assert count == 1 and got != full  # a gate above the K'-th score must fall back
