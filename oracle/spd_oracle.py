"""fp64 CPU oracle for one sparse paged decode step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The HIP library never routes through it, and it shares
no code, tables or constants with the HIP path: every function here is written
from the definitions on the source pages, in plain numpy float64 with no
blocking, fusion or reordering beyond what those definitions state.

Inputs are the *stored* tensors (numpy arrays in their storage dtypes); fp16 and
fp8 values are decoded exactly to float64 first.

Pages and their definitions:
  * LServe ("Hierarchical Paging" and "Key statistics storage and updating"):
    per logical page channel-wise key min / max; page importance
    S_j = sum_i max(q_i * kmax_i, q_i * kmin_i); top-K page selection under a
    token budget; streaming heads read a static sink + local index table
    ("Decoding Stage: Kernel Implementation with Two-Level Indexing").
  * Moira (section 3.2 "The coverage rule", Eq. 3): group-mean softmax share
    pi_bar of each page, forced {P0, Pcur}, tau_b = max tau such that the share
    above tau reaches gamma minus the forced shares.
  * PersistentKV (section 3.1, Eq. 1): exact decode attention over the kept
    tokens; section 3.3: split states and their exact merge.
  * LServe ("Hierarchical Paging", "Token budget and physical page selection"):
    physical pages of N_P = g * N_L tokens hold g logical pages of N_L = 16
    tokens; each logical page keeps its own key min / max, and a physical page's
    importance is the largest importance of its logical pages; the top-K runs
    over physical pages and attention reads whole physical pages.
  * LiteTopK (section 3.4, LiteDSA): several query tokens take their own top-k
    lists, whose union is scanned once; a per-query membership mask keeps each
    query's attention on exactly its own list.  Here the query tokens are the T
    draft tokens of one decode step, each attending causally.
  * Moira (section 3.1 "Page summaries and the mvar estimate", Eq. 2): per page
    and KV head the channel-wise mean and variance of the keys; the page's
    estimated attention mass for query head g is
    log m_{g,P} = s q_g . mu_P + (1/2) (s q_g)^2 . sigma^2_P + log(tokens); the
    first page and the current page are computed exactly.

Readings where the pages leave a step open:
  * GQA combine for top-K: score_p = max over the group's query heads of S_{g,p}.
  * Coverage log-mass from the bound: l_{g,p} = s * S_{g,p} + ln(valid_p), s = 1/sqrt(d);
    every page, sink and current included, is estimated the same way.
  * The budget counts the forced pages; if the forced set alone reaches it the
    list is the forced set.
  * Top-K order (score desc, logical page asc); lists are ascending logical pages.
  * Coverage threshold test in fp64 uses 1e-12 slack (the printed worked example
    sums to 0.8999999999999999 in binary floating point).
  * fp8 pools are OCP E4M3FN with a per-(page, head, token) fp16 scale; their key
    min / max is stored as fp16 rounded outward (max up, min down).
  * An empty row (no kept tokens) gives O = 0 and lse = -inf.
  * Several query tokens per request (T draft tokens at positions L-T .. L-1 of a
    request whose cache holds L keys): query t attends to positions < L - T + 1 + t
    and selects its pages as a single query with that length would, from key
    statistics that cover every cached key (the draft tokens' included).
  * Hierarchical paging: the GQA group is combined as above (max over query heads)
    after the max over logical pages; logical pages with no valid token do not
    enter the max; the budget, the sink and the local window count physical pages.
    Under the coverage rule the shares are taken over logical pages (each logical
    page's log-mass from its own box and valid tokens) and a physical page's share
    is the sum of its logical pages' shares: mass is additive, where the top-K
    importance bound takes the max.
  * mvar: the variance is the population variance over the page's valid tokens
    (divided by their count), and the token count in Eq. 2 is the page's valid
    token count; mean and variance are stored rounded to bf16 (nearest, ties to even)
    and Eq. 2 is evaluated on the stored values.
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 16
COVERAGE_SLACK = 1e-12


# --------------------------------------------------------------------------------------
# Storage decoding
# --------------------------------------------------------------------------------------

def decode_e4m3fn(codes) -> np.ndarray:
    """OCP 8-bit floating point E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no
    infinity, so S.1111.000 .. S.1111.110 are ordinary normals (up to 448).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def stored_values(pool: np.ndarray, scale: np.ndarray | None, kv_dtype: str) -> np.ndarray:
    """Exact float64 value of stored K or V entries (fp8: code value times its token scale)."""
    if kv_dtype == "fp8":
        return decode_e4m3fn(pool) * np.asarray(scale, dtype=np.float64)[..., None]
    return np.asarray(pool, dtype=np.float64)


def n_pages(seq_len: int) -> int:
    return (int(seq_len) + PAGE - 1) // PAGE


def valid_tokens(seq_len: int, p: int) -> int:
    """Row-local token count of logical page p (PersistentKV section 3.3, N*_i = seq_lens[i])."""
    return max(0, min(PAGE, int(seq_len) - PAGE * p))


# --------------------------------------------------------------------------------------
# a0: per-page key statistics
# --------------------------------------------------------------------------------------

def meta_dtype(kv_dtype: str):
    return np.float32 if kv_dtype == "f32" else np.float16


def _round_outward_f16(x: np.ndarray, up: bool) -> np.ndarray:
    """Nearest fp16, then one fp16 step outward if rounding moved the value inward."""
    r = x.astype(np.float16)
    rf = r.astype(np.float64)
    if up:
        moved_in = rf < x
        r = np.where(moved_in, np.nextafter(r, np.float16(np.inf)), r)
    else:
        moved_in = rf > x
        r = np.where(moved_in, np.nextafter(r, np.float16(-np.inf)), r)
    return r.astype(np.float16)


def page_key_minmax(k_page: np.ndarray, valid: int):
    """Channel-wise min and max of the valid keys of one page (LServe, k_min / k_max).

    k_page: float64 [P, d]. Returns (kmin, kmax) float64 [d].
    """
    keys = k_page[:valid]
    return keys.min(axis=0), keys.max(axis=0)


def page_meta_build(inp, meta: np.ndarray | None = None, first_page=None, heads=None,
                    requests=None) -> np.ndarray:
    """Key min / max for every page p >= first_page[b] of every request, all KV heads.

    Layout [num_pool_pages, Hkv, 2, d]: index 0 = kmin, 1 = kmax, in the meta dtype
    (f32 pools: f32; f16 pools: f16; fp8 pools: f16 rounded outward).  Pages not
    visited keep the values of ``meta`` (zeros when it is None).  ``heads`` and
    ``requests`` restrict the work to some KV heads / requests (others are left as they are).
    """
    w = inp.workload
    Hkv, d = inp.k_pool.shape[1], inp.k_pool.shape[3]
    mdt = meta_dtype(w.kv_dtype)
    out = np.zeros((inp.k_pool.shape[0], Hkv, 2, d), dtype=mdt) if meta is None else meta.copy()
    hs = list(range(Hkv)) if heads is None else [int(h) for h in heads]
    reqs = range(len(inp.seq_lens)) if requests is None else [int(b) for b in requests]
    for b in reqs:
        L = int(inp.seq_lens[b])
        start = 0 if first_page is None else max(0, int(first_page[b]))
        pages = list(range(start, n_pages(L)))
        full = [p for p in pages if valid_tokens(L, p) == PAGE]
        part = [p for p in pages if valid_tokens(L, p) < PAGE]
        # full pages, vectorised over chunks of pages (min / max over the token axis)
        for c in range(0, len(full), 512):
            phys = inp.block_table[b, full[c:c + 512]].astype(np.int64)
            for h in hs:
                scale = None if inp.k_scale is None else inp.k_scale[phys, h]
                kv = stored_values(inp.k_pool[phys, h], scale, w.kv_dtype)  # [n, P, d]
                lo, hi = to_stored_meta(kv.min(axis=1), kv.max(axis=1), w.kv_dtype)
                out[phys, h, 0] = lo
                out[phys, h, 1] = hi
        for p in part:
            phys = int(inp.block_table[b, p])
            valid = valid_tokens(L, p)
            for h in hs:
                scale = None if inp.k_scale is None else inp.k_scale[phys, h]
                kv = stored_values(inp.k_pool[phys, h], scale, w.kv_dtype)  # [P, d]
                lo, hi = to_stored_meta(*page_key_minmax(kv, valid), w.kv_dtype)
                out[phys, h, 0] = lo
                out[phys, h, 1] = hi
    return out


def to_stored_meta(kmin: np.ndarray, kmax: np.ndarray, kv_dtype: str):
    """Stored form of float64 min / max: exact in the pool dtype, or fp16 outward for fp8."""
    if kv_dtype == "fp8":
        return _round_outward_f16(kmin, up=False), _round_outward_f16(kmax, up=True)
    mdt = meta_dtype(kv_dtype)
    return kmin.astype(mdt), kmax.astype(mdt)  # exact: min / max of representable values


# --------------------------------------------------------------------------------------
# a1: page scores
# --------------------------------------------------------------------------------------

def quest_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """LServe page importance S = sum_i max(q_i * kmax_i, q_i * kmin_i).

    q: [G, d]; kmin, kmax: [n, d] -> S: [G, n] (float64).
    """
    a = q[:, None, :] * kmax[None, :, :]
    b = q[:, None, :] * kmin[None, :, :]
    return np.maximum(a, b).sum(axis=-1)


def row_bounds(inp, meta: np.ndarray, b: int, h: int) -> np.ndarray:
    """S_{g,p} for the G query heads of KV head h of request b over its pages, from stored meta."""
    w = inp.workload
    G = w.group
    n = n_pages(inp.seq_lens[b])
    phys = inp.block_table[b, :n].astype(np.int64)
    m = meta[phys, h].astype(np.float64)          # [n, 2, d]
    q = inp.q[b, h * G:(h + 1) * G].astype(np.float64)
    return quest_bound(q, m[:, 0], m[:, 1])


def topk_scores(S: np.ndarray) -> np.ndarray:
    """Per-KV-head score of each page: the largest bound over the group's query heads."""
    return S.max(axis=0)


def coverage_shares(S: np.ndarray, seq_len: int, sm_scale: float):
    """Moira's group-mean share pi_bar of each page, from the bound as the page log-mass.

    l_{g,p} = s * S_{g,p} + ln(valid_p);  pi_bar_p = (1/G) sum_g softmax_p(l_{g,.}).
    Returns (pi_bar [n], lse_g [G]).
    """
    n = S.shape[1]
    valid = np.array([valid_tokens(seq_len, p) for p in range(n)], dtype=np.float64)
    return shares_from_logmass(sm_scale * S + np.log(valid)[None, :])


def shares_from_logmass(ell: np.ndarray):
    """Group-mean share of each page from page log-masses ell [G, n] (Moira section 3.2, Eq. 3):
    pi_bar_p = (1/G) sum_g exp(ell_{g,p} - lse_g), lse_g = log sum_p exp(ell_{g,p})."""
    mx = ell.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(ell - mx).sum(axis=1))
    share = np.exp(ell - lse[:, None])
    return share.mean(axis=0), lse


# --------------------------------------------------------------------------------------
# a0 / a1, second estimator: Moira's page summaries and the mvar estimate
# --------------------------------------------------------------------------------------

def page_mean_var(k_page: np.ndarray, valid: int):
    """Channel-wise mean and population variance of the valid keys of one page ([P, d] float64)."""
    keys = k_page[:valid]
    mu = keys.sum(axis=0) / valid
    var = ((keys - mu[None, :]) ** 2).sum(axis=0) / valid
    return mu, var


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits, ties to even), returned as float64.

    bfloat16 keeps float32's exponent range: normal exponents down to -126, subnormal steps of
    2^-133, largest finite (2 - 2^-7) * 2^127; values rounding past it become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                                # x = m 2^e, 0.5 <= |m| < 1
    step = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    r = np.round(x / step) * step                     # numpy rounds halves to even
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    return np.where(np.abs(r) > big, np.copysign(np.inf, x), np.where(x == 0, x, r))


def page_stats_build(inp, first_page=None, heads=None, requests=None, stats=None) -> np.ndarray:
    """Stored page summaries: mean and variance of the keys of every page p >= first_page[b]
    of every request, rounded to bfloat16 (Moira, "Memory for page summaries": the summaries
    are kept in bf16).

    Layout [num_pool_pages, Hkv, 2, d] float64 holding bf16 values: index 0 = mean,
    1 = variance; pages not visited are NaN, or keep their values in ``stats`` when given.
    """
    w = inp.workload
    Hkv, d = inp.k_pool.shape[1], inp.k_pool.shape[3]
    out = np.full((inp.k_pool.shape[0], Hkv, 2, d), np.nan) if stats is None else np.array(stats, dtype=np.float64)
    hs = list(range(Hkv)) if heads is None else [int(h) for h in heads]
    reqs = range(len(inp.seq_lens)) if requests is None else [int(b) for b in requests]
    for b in reqs:
        L = int(inp.seq_lens[b])
        start = 0 if first_page is None else max(0, int(first_page[b]))
        for p in range(start, n_pages(L)):
            phys = int(inp.block_table[b, p])
            for h in hs:
                scale = None if inp.k_scale is None else inp.k_scale[phys, h]
                kv = stored_values(inp.k_pool[phys, h], scale, w.kv_dtype)
                mu, var = page_mean_var(kv, valid_tokens(L, p))
                out[phys, h, 0], out[phys, h, 1] = round_bf16(mu), round_bf16(var)
    return out


def mvar_logmass(q: np.ndarray, mu: np.ndarray, var: np.ndarray, valid: np.ndarray, sm_scale: float) -> np.ndarray:
    """Moira Eq. 2: log m_{g,P} = s q_g . mu_P + 0.5 (s q_g)^2 . sigma^2_P + log(tokens).

    q: [G, d]; mu, var: [n, d]; valid: [n] -> [G, n].
    """
    sq = sm_scale * q
    return sq @ mu.T + 0.5 * ((sq * sq) @ var.T) + np.log(valid)[None, :]


def exact_logmass(q: np.ndarray, keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """log sum_{k in page} exp(s q_g . k) for each query head: q [G, d], keys [valid, d] -> [G]."""
    x = sm_scale * (q @ keys.T)
    mx = x.max(axis=1)
    return mx + np.log(np.exp(x - mx[:, None]).sum(axis=1))


def row_logmass_mvar(inp, stats: np.ndarray, b: int, h: int) -> np.ndarray:
    """Page log-masses of dynamic row (b, h) under the mvar estimator, [G, n]: Eq. 2 from the
    page summaries, except the first page and the current (last) page, computed exactly."""
    w = inp.workload
    G = w.group
    L = int(inp.seq_lens[b])
    n = n_pages(L)
    q = inp.q[b, h * G:(h + 1) * G].astype(np.float64)
    phys = inp.block_table[b, :n].astype(np.int64)
    st = stats[phys, h]
    valid = np.array([valid_tokens(L, p) for p in range(n)], dtype=np.float64)
    ell = mvar_logmass(q, st[:, 0], st[:, 1], valid, w.sm_scale)
    for p in sorted({0, n - 1}):
        ph = int(phys[p])
        scale = None if inp.k_scale is None else inp.k_scale[ph, h]
        keys = stored_values(inp.k_pool[ph, h], scale, w.kv_dtype)[:valid_tokens(L, p)]
        ell[:, p] = exact_logmass(q, keys, w.sm_scale)
    return ell


# --------------------------------------------------------------------------------------
# a2: page selection
# --------------------------------------------------------------------------------------

def forced_pages(n: int, n_sink: int, n_local: int) -> list:
    """Sink pages 0..n_sink-1 and local pages n-n_local..n-1 (LServe static index table)."""
    s = set(range(min(max(n_sink, 0), n))) | set(range(max(0, n - max(n_local, 0)), n))
    return sorted(s)


def select_topk(scores: np.ndarray, n: int, budget: int, forced: list) -> list:
    """Forced pages plus the (budget - |forced|) best others by (score desc, page asc)."""
    fset = set(forced)
    k_rest = budget - len(forced)
    others = [p for p in range(n) if p not in fset]
    if k_rest <= 0:
        return sorted(fset)
    order = sorted(others, key=lambda p: (-float(scores[p]), p))
    return sorted(fset | set(order[:k_rest]))


def select_coverage(pi: np.ndarray, n: int, gamma: float, forced: list) -> list:
    """Moira Eq. 3: forced pages plus every other page with share >= tau_b."""
    fset = set(forced)
    t = gamma - sum(float(pi[p]) for p in forced)
    if t - COVERAGE_SLACK <= 0:
        return sorted(fset)
    others = [p for p in range(n) if p not in fset]
    order = sorted(others, key=lambda p: (-float(pi[p]), p))
    cum = 0.0
    for p in order:
        cum += float(pi[p])
        if cum >= t - COVERAGE_SLACK:
            tau = float(pi[p])
            return sorted(fset | {r for r in others if float(pi[r]) >= tau})
    return list(range(n))


def reuse_lists(inp, lists: dict) -> dict:
    """Lists for a later step of a reuse chunk (LServe, "Reusable Page Selection": the pages selected
    on the chunk's first step serve its remaining steps), at the current lengths inp.seq_lens.

    Reading of the pages: a dynamic row keeps its selected pages and gains the pages of the current
    forced set (sink and local window) that lie past its last entry, appended in ascending order --
    a query must attend to its own newest page, and every rule here keeps the sink and local pages;
    pages that were local when the chunk selected stay listed.  A streaming row takes its static sink
    + local table for the current length."""
    w = inp.workload
    out = {}
    for (b, h), lst in lists.items():
        n = n_pages(inp.seq_lens[b])
        if inp.head_kind[h]:
            out[(b, h)] = forced_pages(n, w.n_sink_stream, w.n_local_stream)
            continue
        last = lst[-1] if lst else -1
        out[(b, h)] = list(lst) + [p for p in forced_pages(n, w.n_sink, w.n_local) if p > last]
    return out


def page_select(inp, meta: np.ndarray, stats: np.ndarray | None = None):
    """Scores and lists for every (request, KV head) row.

    Returns dict with 'lists' {(b,h): [pages]}, 'scores' {(b,h): per-page key or None
    for streaming rows}, 'S' {(b,h): [G, n] bounds}, 'lse' {(b,h): [G]} (coverage only).
    With the mvar estimator the page log-masses come from ``stats`` (page_stats_build).
    """
    w = inp.workload
    if w.estimator == "mvar":
        return _page_select_mvar(inp, page_stats_build(inp) if stats is None else stats)
    out = {"lists": {}, "scores": {}, "S": {}, "lse": {}}
    for b in range(len(inp.seq_lens)):
        L = int(inp.seq_lens[b])
        n = n_pages(L)
        for h in range(inp.k_pool.shape[1]):
            if inp.head_kind[h]:
                out["lists"][(b, h)] = forced_pages(n, w.n_sink_stream, w.n_local_stream)
                out["scores"][(b, h)] = None
                continue
            S = row_bounds(inp, meta, b, h)
            out["S"][(b, h)] = S
            forced = forced_pages(n, w.n_sink, w.n_local)
            if w.mode == "topk":
                sc = topk_scores(S)
                out["scores"][(b, h)] = sc
                out["lists"][(b, h)] = select_topk(sc, n, w.budget_pages, forced)
            else:
                pi, lse = coverage_shares(S, L, w.sm_scale) if n else (np.zeros(0), np.full(w.group, -np.inf))
                out["scores"][(b, h)] = pi
                out["lse"][(b, h)] = lse
                out["lists"][(b, h)] = select_coverage(pi, n, w.gamma, forced) if n else []
    return out


def _page_select_mvar(inp, stats: np.ndarray):
    """page_select for coverage rows whose page log-masses come from the mvar estimate."""
    w = inp.workload
    out = {"lists": {}, "scores": {}, "S": {}, "lse": {}}
    for b in range(len(inp.seq_lens)):
        L = int(inp.seq_lens[b])
        n = n_pages(L)
        for h in range(inp.k_pool.shape[1]):
            if inp.head_kind[h]:
                out["lists"][(b, h)] = forced_pages(n, w.n_sink_stream, w.n_local_stream)
                out["scores"][(b, h)] = None
                continue
            if n == 0:
                out["scores"][(b, h)], out["lse"][(b, h)], out["lists"][(b, h)] = np.zeros(0), np.full(w.group, -np.inf), []
                continue
            pi, lse = shares_from_logmass(row_logmass_mvar(inp, stats, b, h))
            out["scores"][(b, h)] = pi
            out["lse"][(b, h)] = lse
            out["lists"][(b, h)] = select_coverage(pi, n, w.gamma, forced_pages(n, w.n_sink, w.n_local))
    return out


# --------------------------------------------------------------------------------------
# a3 + a4: attention over the kept pages
# --------------------------------------------------------------------------------------

def gather_tokens(inp, b: int, h: int, pages) -> tuple:
    """Valid keys and values (float64) of the listed logical pages of row (b, h), in list order."""
    w = inp.workload
    L = int(inp.seq_lens[b])
    ks, vs = [], []
    for p in pages:
        phys = int(inp.block_table[b, int(p)])
        valid = valid_tokens(L, int(p))
        ksc = None if inp.k_scale is None else inp.k_scale[phys, h]
        vsc = None if inp.v_scale is None else inp.v_scale[phys, h]
        ks.append(stored_values(inp.k_pool[phys, h], ksc, w.kv_dtype)[:valid])
        vs.append(stored_values(inp.v_pool[phys, h], vsc, w.kv_dtype)[:valid])
    d = inp.k_pool.shape[3]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """PersistentKV Eq. 1 for one query: O = sum_j softmax_j(s q.k_j) v_j, lse = log sum_j e^{s q.k_j}.

    q [d], K/V [N, d] float64.  N = 0 gives (zeros, -inf).
    """
    if K.shape[0] == 0:
        return np.zeros(K.shape[1]), -np.inf
    x = sm_scale * (K @ q)
    m = x.max()
    e = np.exp(x - m)
    lsum = e.sum()
    return (e @ V) / lsum, m + math.log(lsum)


def sparse_paged_decode(inp, lists: dict, sm_scale: float):
    """O [B, Hq, d] and lse [B, Hq] of attention restricted to each row's listed pages."""
    w = inp.workload
    B, Hq, d = inp.q.shape
    G = w.group
    O = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for (b, h), pages in lists.items():
        K, V = gather_tokens(inp, b, h, pages)
        for g in range(G):
            qh = inp.q[b, h * G + g].astype(np.float64)
            O[b, h * G + g], lse[b, h * G + g] = attention(qh, K, V, sm_scale)
    return O, lse


def merge_states(states):
    """PersistentKV section 3.3 exact merge of split states (m_s, l_s, a_s) -> (O, lse)."""
    ms = np.array([s[0] for s in states], dtype=np.float64)
    m = ms.max()
    if not np.isfinite(m):
        return np.zeros_like(states[0][2]), -np.inf
    ell = sum(math.exp(s[0] - m) * s[1] for s in states if np.isfinite(s[0]))
    acc = sum(math.exp(s[0] - m) * s[2] for s in states if np.isfinite(s[0]))
    return acc / ell, m + math.log(ell)


def split_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """One split's partial state (m_s, l_s, a_s); the empty split is (-inf, 0, 0)."""
    if K.shape[0] == 0:
        return (-np.inf, 0.0, np.zeros(K.shape[1]))
    x = sm_scale * (K @ q)
    m = x.max()
    e = np.exp(x - m)
    return (m, e.sum(), e @ V)


# --------------------------------------------------------------------------------------
# Hierarchical paging: N_P-token physical pages over N_L = 16-token logical pages
# --------------------------------------------------------------------------------------

def physical_page_tokens(inp) -> int:
    """N_P, the tokens of one physical page: the pool's third axis."""
    return int(inp.k_pool.shape[2])


def hier_n_physical(seq_len: int, page_tokens: int) -> int:
    return (int(seq_len) + page_tokens - 1) // page_tokens


def hier_logical_keys(inp, b: int, h: int, lp: int) -> np.ndarray:
    """Valid keys (float64 [valid, d]) of logical page lp of request b, KV head h.

    Logical page lp covers tokens [16 lp, 16 lp + 16) of the request; they sit in physical page
    block_table[b, lp // g] at token slots 16 (lp % g) ... 16 (lp % g) + 15.
    """
    w = inp.workload
    g = physical_page_tokens(inp) // PAGE
    phys = int(inp.block_table[b, lp // g])
    sl = slice(PAGE * (lp % g), PAGE * (lp % g) + PAGE)
    scale = None if inp.k_scale is None else inp.k_scale[phys, h, sl]
    return stored_values(inp.k_pool[phys, h, sl], scale, w.kv_dtype)[:valid_tokens(inp.seq_lens[b], lp)]


def hier_meta_build(inp, meta: np.ndarray | None = None, first_page=None) -> np.ndarray:
    """Key min / max of every logical page lp >= first_page[b] of every request, all KV heads
    (LServe: statistics on N_L-token logical pages, stored with the physical page that holds them).

    Layout [num_pool_pages, Hkv, g, 2, d]: entry [P, h, i] is logical sub-page i of physical page
    P; 0 = kmin, 1 = kmax, in the meta dtype (fp8 pools: fp16 rounded outward).  Entries not
    visited keep the values of ``meta`` (zeros when it is None).
    """
    w = inp.workload
    Npool, Hkv, NP, d = inp.k_pool.shape
    g = NP // PAGE
    out = np.zeros((Npool, Hkv, g, 2, d), dtype=meta_dtype(w.kv_dtype)) if meta is None else meta.copy()
    for b in range(len(inp.seq_lens)):
        start = 0 if first_page is None else max(0, int(first_page[b]))
        for lp in range(start, n_pages(inp.seq_lens[b])):
            phys = int(inp.block_table[b, lp // g])
            for h in range(Hkv):
                keys = hier_logical_keys(inp, b, h, lp)
                lo, hi = to_stored_meta(keys.min(axis=0), keys.max(axis=0), w.kv_dtype)
                out[phys, h, lp % g, 0] = lo
                out[phys, h, lp % g, 1] = hi
    return out


def hier_row_scores(inp, meta: np.ndarray, b: int, h: int):
    """Physical page scores of dynamic row (b, h) (LServe, "Physical page importance
    aggregation"): each logical page's bound S_{g,lp} from its stored key box, then the largest
    over the logical pages of each physical page and over the group's query heads.

    Returns (scores [n_physical], S [G, n_logical]).
    """
    w = inp.workload
    G = w.group
    NP = physical_page_tokens(inp)
    g = NP // PAGE
    L = int(inp.seq_lens[b])
    n_log = n_pages(L)
    lps = np.arange(n_log)
    phys = inp.block_table[b, lps // g].astype(np.int64)
    m = meta[phys, h, lps % g].astype(np.float64)            # [n_log, 2, d]
    q = inp.q[b, h * G:(h + 1) * G].astype(np.float64)
    S = quest_bound(q, m[:, 0], m[:, 1])                      # [G, n_log]
    per_logical = S.max(axis=0) if n_log else np.zeros(0)
    scores = np.array([per_logical[j * g:(j + 1) * g].max() for j in range(hier_n_physical(L, NP))])
    return scores, S


def hier_row_shares(inp, meta: np.ndarray, b: int, h: int):
    """Coverage shares of the physical pages of dynamic row (b, h): Moira's group-mean share of
    every logical page (log-mass s * S_{g,lp} + ln(valid_lp) from its own key box, softmax over
    the row's logical pages per query head, mean over the group; section 3.2, Eq. 3), summed over
    the logical pages of each physical page.

    Returns (shares [n_physical], lse_g [G]).
    """
    w = inp.workload
    NP = physical_page_tokens(inp)
    g = NP // PAGE
    L = int(inp.seq_lens[b])
    _, S = hier_row_scores(inp, meta, b, h)
    pi_log, lse = coverage_shares(S, L, w.sm_scale)
    return np.array([pi_log[j * g:(j + 1) * g].sum() for j in range(hier_n_physical(L, NP))]), lse


def hier_stats_build(inp, stats: np.ndarray | None = None, first_page=None) -> np.ndarray:
    """Moira's page summaries per 16-token logical page (mean and variance of its valid keys, stored in
    bf16), kept with the physical page that holds it: layout [num_pool_pages, Hkv, g, 2, d] float64
    holding bf16 values; entries not visited are NaN, or keep their values in ``stats``."""
    Npool, Hkv, NP, d = inp.k_pool.shape
    g = NP // PAGE
    out = np.full((Npool, Hkv, g, 2, d), np.nan) if stats is None else np.array(stats, dtype=np.float64)
    for b in range(len(inp.seq_lens)):
        start = 0 if first_page is None else max(0, int(first_page[b]))
        for lp in range(start, n_pages(inp.seq_lens[b])):
            phys = int(inp.block_table[b, lp // g])
            for h in range(Hkv):
                keys = hier_logical_keys(inp, b, h, lp)
                mu, var = page_mean_var(keys, len(keys))
                out[phys, h, lp % g, 0], out[phys, h, lp % g, 1] = round_bf16(mu), round_bf16(var)
    return out


def hier_row_shares_mvar(inp, stats: np.ndarray, b: int, h: int):
    """Coverage shares of the physical pages of dynamic row (b, h) under the mvar estimate: Eq. 2 for every
    logical page from its summary, the row's first and current logical pages computed exactly, the group-
    mean share of each logical page, summed over the logical pages of each physical page."""
    w = inp.workload
    G = w.group
    NP = physical_page_tokens(inp)
    g = NP // PAGE
    L = int(inp.seq_lens[b])
    n_log = n_pages(L)
    lps = np.arange(n_log)
    st = stats[inp.block_table[b, lps // g].astype(np.int64), h, lps % g]
    q = inp.q[b, h * G:(h + 1) * G].astype(np.float64)
    valid = np.array([valid_tokens(L, p) for p in lps], dtype=np.float64)
    ell = mvar_logmass(q, st[:, 0], st[:, 1], valid, w.sm_scale)
    for p in sorted({0, n_log - 1}):
        ell[:, p] = exact_logmass(q, hier_logical_keys(inp, b, h, p), w.sm_scale)
    pi_log, lse = shares_from_logmass(ell)
    return np.array([pi_log[j * g:(j + 1) * g].sum() for j in range(hier_n_physical(L, NP))]), lse


def hier_page_select(inp, meta: np.ndarray):
    """Lists of physical pages for every row: streaming rows keep their sink + local physical
    pages; dynamic rows the forced physical pages plus the best others under the physical page
    budget (top-K by (score desc, page asc)), or the coverage rule over physical shares.  Same
    dict as page_select."""
    w = inp.workload
    NP = physical_page_tokens(inp)
    out = {"lists": {}, "scores": {}, "S": {}, "lse": {}}
    for b in range(len(inp.seq_lens)):
        n = hier_n_physical(inp.seq_lens[b], NP)
        for h in range(inp.k_pool.shape[1]):
            if inp.head_kind[h]:
                out["lists"][(b, h)] = forced_pages(n, w.n_sink_stream, w.n_local_stream)
                out["scores"][(b, h)] = None
                continue
            forced = forced_pages(n, w.n_sink, w.n_local)
            if w.mode == "topk":
                sc, S = hier_row_scores(inp, meta, b, h)
                out["scores"][(b, h)], out["S"][(b, h)] = sc, S
                out["lists"][(b, h)] = select_topk(sc, n, w.budget_pages, forced)
            elif n == 0:
                out["scores"][(b, h)], out["lse"][(b, h)], out["lists"][(b, h)] = np.zeros(0), np.full(w.group, -np.inf), []
            else:
                pi, lse = (hier_row_shares_mvar if w.estimator == "mvar" else hier_row_shares)(inp, meta, b, h)
                out["scores"][(b, h)], out["lse"][(b, h)] = pi, lse
                out["lists"][(b, h)] = select_coverage(pi, n, w.gamma, forced)
    return out


def hier_gather_tokens(inp, b: int, h: int, pages) -> tuple:
    """Valid keys and values (float64) of the listed physical pages of row (b, h), in list order."""
    w = inp.workload
    NP = physical_page_tokens(inp)
    L = int(inp.seq_lens[b])
    ks, vs = [], []
    for j in pages:
        phys = int(inp.block_table[b, int(j)])
        valid = max(0, min(NP, L - NP * int(j)))
        ksc = None if inp.k_scale is None else inp.k_scale[phys, h]
        vsc = None if inp.v_scale is None else inp.v_scale[phys, h]
        ks.append(stored_values(inp.k_pool[phys, h], ksc, w.kv_dtype)[:valid])
        vs.append(stored_values(inp.v_pool[phys, h], vsc, w.kv_dtype)[:valid])
    d = inp.k_pool.shape[3]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


def hier_sparse_paged_decode(inp, lists: dict, sm_scale: float):
    """O [B, Hq, d] and lse [B, Hq] of attention over every valid token of the listed physical pages."""
    w = inp.workload
    B, Hq, d = inp.q.shape
    G = w.group
    O = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for (b, h), pages in lists.items():
        K, V = hier_gather_tokens(inp, b, h, pages)
        for g in range(G):
            O[b, h * G + g], lse[b, h * G + g] = attention(inp.q[b, h * G + g].astype(np.float64), K, V, sm_scale)
    return O, lse


# --------------------------------------------------------------------------------------
# Whole step
# --------------------------------------------------------------------------------------

def decode_step(inp, meta: np.ndarray | None = None):
    """Metadata (if not given) -> scores -> lists -> attention, as the method orders them."""
    if physical_page_tokens(inp) != PAGE:  # hierarchical paging
        if meta is None:
            meta = hier_stats_build(inp) if inp.workload.estimator == "mvar" else hier_meta_build(inp)
        sel = hier_page_select(inp, meta)
        O, lse = hier_sparse_paged_decode(inp, sel["lists"], inp.workload.sm_scale)
        return {"meta": meta, **sel, "O": O, "out_lse": lse}
    if meta is None:
        meta = page_meta_build(inp)
    sel = page_select(inp, meta)
    O, lse = sparse_paged_decode(inp, sel["lists"], inp.workload.sm_scale)
    return {"meta": meta, **sel, "O": O, "out_lse": lse}


# --------------------------------------------------------------------------------------
# Several query tokens per request (LiteDSA union with per-query membership masks)
# --------------------------------------------------------------------------------------

def mq_lengths(seq_len: int, T: int) -> list:
    """Causal length of each of the T query tokens of a request whose cache holds seq_len keys."""
    return [int(seq_len) - T + 1 + t for t in range(T)]


def mq_token_inputs(inp, t: int):
    """The single-query view of query token t: its queries and its causal lengths."""
    import copy
    T = inp.q.shape[1]
    one = copy.copy(inp)
    one.workload = inp.workload.replace(num_queries=1)
    one.q = np.ascontiguousarray(inp.q[:, t])
    one.seq_lens = np.array([mq_lengths(L, T)[t] for L in inp.seq_lens], dtype=inp.seq_lens.dtype)
    return one


def union_lists(lists_by_token: list) -> dict:
    """LiteDSA candidate union: {(b, h): (ascending union of the T lists, mask per entry with bit t
    set when the page is in token t's list)}."""
    out = {}
    for key in lists_by_token[0]:
        pages = sorted(set().union(*[set(lt[key]) for lt in lists_by_token]))
        masks = [sum(1 << t for t, lt in enumerate(lists_by_token) if p in set(lt[key])) for p in pages]
        out[key] = (pages, masks)
    return out


def mq_decode_step(inp, meta: np.ndarray | None = None):
    """Several query tokens per request: key statistics over every cached key, each token's own
    selection over its causal prefix, the union of the lists, and each token's attention over its
    own list (the union and masks change which pages are read, not what a query attends to).

    Returns dict with 'lists_by_token' [T] of {(b,h): pages}, 'union' {(b,h): (pages, masks)},
    'O' [B, T, Hq, d] and 'out_lse' [B, T, Hq]."""
    if meta is None:
        meta = page_meta_build(inp)
    B, T, Hq, d = inp.q.shape
    lists_by_token, O, lse = [], np.zeros((B, T, Hq, d)), np.full((B, T, Hq), -np.inf)
    for t in range(T):
        one = mq_token_inputs(inp, t)
        sel = page_select(one, meta)
        lists_by_token.append(sel["lists"])
        O[:, t], lse[:, t] = sparse_paged_decode(one, sel["lists"], inp.workload.sm_scale)
    return {"meta": meta, "lists_by_token": lists_by_token, "union": union_lists(lists_by_token), "O": O,
            "out_lse": lse}
