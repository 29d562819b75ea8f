"""Seeded synthetic inputs for one sparse paged decode step.

This module only *draws* inputs: queries, paged K/V pools (with per-token fp8
scales where the pool is quantised), block tables, sequence lengths and the
streaming/dynamic kind of every KV head.  It holds none of the method's
arithmetic -- no key bounds, page scores, selection or attention -- so the HIP
library and the fp64 oracle can both consume what it produces without sharing
any of the computation they are compared on.

Layouts follow the native paged-attention layout of the PersistentKV page
(section 3.2, "Native Block-Table Execution"): ``K,V[physical_page, Hkv,
page_size, d]`` plus a per-request block table of physical page ids.  Block
tables are built the way that page's section 3.7 ("Page-Table Generation")
describes: every request owns ceil(len / P) logical pages, the physical page
universe is ceil(sum / (1 - rho)) ids, and a seeded permutation of it hands each
request a consecutive slice.

"Planted" pages give the selectors something real to find: for KV head h of
request b, every key of a planted page is ``z + delta * u`` where ``z`` is the
N(0, 1) draw and ``u`` is the unit vector along the sum of the group's queries.

Physical pages hold ``page_size`` tokens: 16 (one logical page each), or 64 for
the hierarchical layout of the LServe page ("Hierarchical Paging", N_P = 64
physical tokens over N_L = 16-token logical pages).  Planted pages are always
16-token logical pages, so a physical page of 64 tokens may hold one planted
logical page among three ordinary ones.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16      # logical page (N_L), and the default physical page
LOGICAL_PAGE = 16
BASE_SEED = 20261202

KV_DTYPES = ("f32", "f16", "fp8")
Q_DTYPES = ("f32", "f16")
FP8_MAX = 448.0  # largest finite OCP E4M3FN value


@dataclass(frozen=True)
class Workload:
    """Shape and structure of one decode step's inputs.

    ``planted`` is one of ("fixed", n) -- n planted pages per (request, KV
    head); ("per_pages", k) -- max(1, n_pages // k); ("loguniform", lo, hi) --
    round(exp(U[ln lo, ln hi])) per (request, KV head).
    ``delta`` is either a float (shift in key units) or ("nats", x): the shift is
    chosen per (request, KV head) so that scale * delta * mean_g(q_g . u) = x.
    """

    name: str
    seq_lens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    q_dtype: str
    mode: str  # "topk" | "coverage"
    estimator: str = "bound"  # coverage page mass: "bound" (Quest key box) | "mvar" (Moira mean / variance)
    budget_pages: int = 0
    gamma: float = 0.0
    n_sink: int = 1
    n_local: int = 2
    n_sink_stream: int = 0
    n_local_stream: int = 0
    streaming_heads: tuple = ()
    planted: tuple = ("fixed", 0)
    delta: object = 2.0
    hole_fraction: float = 0.0
    seed: int = BASE_SEED
    max_pages_per_seq: int | None = None
    max_list: int | None = None
    shuffle_lengths: bool = False
    page_size: int = PAGE_SIZE  # physical page tokens (N_P): 16, or 64 over 16-token logical pages
    num_queries: int = 1        # query tokens per request (T > 1: draft tokens verified in one step)

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def n_pages(self) -> np.ndarray:
        """Physical pages of each request (ceil(len / page_size))."""
        P = self.page_size
        return np.array([(int(L) + P - 1) // P for L in self.seq_lens], dtype=np.int64)

    @property
    def n_logical(self) -> np.ndarray:
        """16-token logical pages of each request."""
        return np.array([(int(L) + LOGICAL_PAGE - 1) // LOGICAL_PAGE for L in self.seq_lens], dtype=np.int64)

    @property
    def pages_per_seq(self) -> int:
        mp = int(self.n_pages.max()) if self.batch else 0
        if self.max_pages_per_seq is not None:
            assert self.max_pages_per_seq >= mp
            return int(self.max_pages_per_seq)
        return max(mp, 1)

    @property
    def list_capacity(self) -> int:
        if self.max_list is not None:
            return int(self.max_list)
        if self.mode == "coverage":
            return self.pages_per_seq
        return max(self.budget_pages, self.n_sink_stream + self.n_local_stream,
                   self.n_sink + self.n_local, 1)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


@dataclass
class Inputs:
    """One step's inputs, as stored (numpy arrays in their storage dtypes)."""

    workload: Workload
    q: np.ndarray            # [B, Hq, d] float32 | float16
    k_pool: np.ndarray       # [Npool, Hkv, P, d] float32 | float16 | uint8 (E4M3FN codes)
    v_pool: np.ndarray
    k_scale: np.ndarray | None  # [Npool, Hkv, P] float16 (fp8 pools only)
    v_scale: np.ndarray | None
    block_table: np.ndarray  # [B, max_pages_per_seq] int32
    seq_lens: np.ndarray     # [B] int32
    head_kind: np.ndarray    # [Hkv] uint8, 1 = streaming head
    planted: dict = field(default_factory=dict)  # (b, h) -> sorted logical pages
    deltas: dict = field(default_factory=dict)   # (b, h) -> shift used

    @property
    def num_pool_pages(self) -> int:
        return int(self.k_pool.shape[0])


# --------------------------------------------------------------------------------------
# Named workloads.  The Llama-3-8B-class attention geometry (Hq 32 / Hkv 8 / d 128,
# 16-token pages) is the shape the PersistentKV and Moira pages evaluate on.
# --------------------------------------------------------------------------------------

def _powerlaw_lengths(rng: np.random.Generator, n: int, lo: int, hi: int, a: float) -> list:
    """Lengths from p(L) ~ L^-a truncated to [lo, hi] (inverse-CDF draw)."""
    u = rng.random(n)
    e = 1.0 - a
    x = (lo ** e + u * (hi ** e - lo ** e)) ** (1.0 / e)
    return [int(min(hi, max(lo, math.floor(v)))) for v in x]


def named(name: str, seed_offset: int = 0) -> Workload:
    """The decode-step workloads the library is measured and checked on."""
    if name == "tiny_b1_hq8_d64_4k_f32":
        return Workload(name=name, seq_lens=(4096,), num_q_heads=8, num_kv_heads=2, head_dim=64,
                        kv_dtype="f32", q_dtype="f32", mode="topk", budget_pages=32,
                        n_sink=1, n_local=2, planted=("fixed", 8), delta=2.0,
                        seed=BASE_SEED + 0 + seed_offset)
    if name == "llama3_8b_b1_128k_f16":
        return Workload(name=name, seq_lens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="f16", q_dtype="f16", mode="topk", budget_pages=256,
                        n_sink=1, n_local=2, n_sink_stream=4, n_local_stream=16,
                        streaming_heads=(0, 1, 2, 3), planted=("fixed", 64), delta=2.0,
                        seed=BASE_SEED + 1 + seed_offset)
    if name == "mixed_b8_bimodal_f16":
        rng = np.random.default_rng(BASE_SEED + 2 + seed_offset)
        lens = [4096] * 4 + [65536] * 4
        rng.shuffle(lens)
        return Workload(name=name, seq_lens=tuple(int(x) for x in lens), num_q_heads=32,
                        num_kv_heads=8, head_dim=128, kv_dtype="f16", q_dtype="f16", mode="topk",
                        budget_pages=128, n_sink=1, n_local=2, planted=("per_pages", 128),
                        delta=2.0, seed=BASE_SEED + 2 + seed_offset)
    if name == "mixed_b8_powerlaw_f16":
        rng = np.random.default_rng(BASE_SEED + 12 + seed_offset)
        lens = _powerlaw_lengths(rng, 8, 1024, 131072, 1.1)
        return Workload(name=name, seq_lens=tuple(lens), num_q_heads=32, num_kv_heads=8,
                        head_dim=128, kv_dtype="f16", q_dtype="f16", mode="topk", budget_pages=128,
                        n_sink=1, n_local=2, planted=("per_pages", 128), delta=2.0,
                        seed=BASE_SEED + 12 + seed_offset)
    if name == "coverage_b4_128k_f16":
        return Workload(name=name, seq_lens=(131072,) * 4, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, kv_dtype="f16", q_dtype="f16", mode="coverage", gamma=0.99,
                        n_sink=1, n_local=1, planted=("loguniform", 20, 2000), delta=("nats", 12.0),
                        seed=BASE_SEED + 3 + seed_offset)
    if name == "fp8_b1_512k":
        return Workload(name=name, seq_lens=(524288,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="fp8", q_dtype="f16", mode="topk", budget_pages=256,
                        n_sink=1, n_local=2, planted=("fixed", 512), delta=2.0,
                        seed=BASE_SEED + 4 + seed_offset)
    if name == "llama3_8b_b1_128k_f16_dense":
        # the 128k layer with every page of every KV head listed: a streaming check of decode
        # (512 MiB of K/V per step) next to the sparse step
        return Workload(name=name, seq_lens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="f16", q_dtype="f16", mode="topk", budget_pages=8192,
                        n_sink=1, n_local=2, planted=("fixed", 64), delta=2.0,
                        seed=BASE_SEED + 5 + seed_offset)
    if name == "coverage_mvar_b4_128k_f16":
        # the coverage step with Moira's mvar page estimate (section 3.1) in place of the key box
        return Workload(name=name, seq_lens=(131072,) * 4, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, kv_dtype="f16", q_dtype="f16", mode="coverage", estimator="mvar",
                        gamma=0.99, n_sink=1, n_local=1, planted=("loguniform", 20, 2000),
                        delta=("nats", 12.0), seed=BASE_SEED + 6 + seed_offset)
    if name == "mtp4_b1_128k_f16":
        # the 128k layer verifying 4 draft tokens in one step (speculative decoding): each query token
        # selects its own 256 pages over its causal prefix, and the four lists share one scan (LiteDSA
        # union with per-query membership masks)
        return Workload(name=name, seq_lens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="f16", q_dtype="f16", mode="topk", budget_pages=256, num_queries=4,
                        n_sink=1, n_local=2, n_sink_stream=4, n_local_stream=16,
                        streaming_heads=(0, 1, 2, 3), planted=("fixed", 64), delta=2.0,
                        seed=BASE_SEED + 8 + seed_offset)
    if name == "mtp4_b1_512k_fp8":
        # the 512k fp8 layer verifying 4 draft tokens: each token's 256 pages over 32768
        return Workload(name=name, seq_lens=(524288,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="fp8", q_dtype="f16", mode="topk", budget_pages=256, num_queries=4,
                        n_sink=1, n_local=2, planted=("fixed", 512), delta=2.0, seed=BASE_SEED + 9 + seed_offset)
    if name == "llama3_8b_b1_128k_f16_hier64":
        # the 128k layer with 64-token physical pages scored through 16-token logical pages (LServe,
        # "Hierarchical Paging", N_P = 64, N_L = 16): token budget 4096 = 64 physical pages
        # ("Token budget and physical page selection", K = ceil(B / N_P)); one sink and one local
        # physical page per dynamic head; streaming heads keep the same 64 + 256 tokens (1 + 4 pages)
        return Workload(name=name, seq_lens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype="f16", q_dtype="f16", mode="topk", page_size=64,
                        budget_pages=-(-4096 // 64), n_sink=1, n_local=1, n_sink_stream=1, n_local_stream=4,
                        streaming_heads=(0, 1, 2, 3), planted=("fixed", 64), delta=2.0,
                        seed=BASE_SEED + 7 + seed_offset)
    raise KeyError(name)


NAMED = ("tiny_b1_hq8_d64_4k_f32", "llama3_8b_b1_128k_f16", "mixed_b8_bimodal_f16",
         "mixed_b8_powerlaw_f16", "coverage_b4_128k_f16", "fp8_b1_512k", "llama3_8b_b1_128k_f16_dense",
         "coverage_mvar_b4_128k_f16", "llama3_8b_b1_128k_f16_hier64", "mtp4_b1_128k_f16", "mtp4_b1_512k_fp8")


# --------------------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------------------

def _np_dtype(tag: str):
    return {"f32": np.float32, "f16": np.float16}[tag]


def _quantize_e4m3fn(x):
    """Per-token symmetric fp8 quantisation of an input pool (input preparation only).

    x: float32 torch tensor [..., d].  Scale per (page, head, token) = amax / 448
    stored as fp16 (1.0 when amax is 0); codes are the OCP E4M3FN
    round-to-nearest-even encodings of x / scale, clamped to +-448, produced by
    torch's float8_e4m3fn conversion.
    """
    import torch

    scale = (x.abs().amax(dim=-1) / FP8_MAX).to(torch.float16)
    scale[scale == 0] = 1.0
    codes = torch.empty(x.shape, dtype=torch.uint8)
    step = max(1, (1 << 24) // max(1, x[0].numel()))
    for s in range(0, x.shape[0], step):
        xs = (x[s:s + step] / scale[s:s + step].float()[..., None]).clamp_(-FP8_MAX, FP8_MAX)
        codes[s:s + step] = xs.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), scale.numpy()


def generate(w: Workload, seed: int | None = None) -> Inputs:
    """Draw every input of one decode step for workload ``w`` (deterministic in the seed)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    assert Hq % Hkv == 0 and w.kv_dtype in KV_DTYPES and w.q_dtype in Q_DTYPES
    G = Hq // Hkv
    P = w.page_size
    assert P % LOGICAL_PAGE == 0
    g = P // LOGICAL_PAGE  # logical pages per physical page
    n_pages = w.n_pages
    maxp = w.pages_per_seq

    # queries: float64 draw, stored in the query dtype; T > 1 query tokens per request: [B, T, Hq, d]
    T = w.num_queries
    q = rng.standard_normal((B, Hq, d) if T == 1 else (B, T, Hq, d)).astype(_np_dtype(w.q_dtype))

    # block table: seeded permutation of the physical universe, consecutive slices
    total = int(n_pages.sum())
    universe = max(1, int(math.ceil(total / (1.0 - w.hole_fraction)))) if total else 1
    perm = rng.permutation(universe).astype(np.int32)
    block_table = np.zeros((B, maxp), dtype=np.int32)
    off = 0
    for b in range(B):
        nb = int(n_pages[b])
        block_table[b, :nb] = perm[off:off + nb]
        off += nb
    used = perm[:total]

    # pools: N(0, 1) in float32 from torch's CPU generator, seeded from this stream
    # (the pools are large; torch's sampler is the faster of the two)
    import torch

    tg = torch.Generator().manual_seed(int(rng.integers(0, 2**62)))
    kz = torch.randn((universe, Hkv, P, d), generator=tg, dtype=torch.float32)
    vz = torch.randn((universe, Hkv, P, d), generator=tg, dtype=torch.float32)

    # planted high-affinity pages
    qf = q.astype(np.float64)
    planted, deltas = {}, {}
    for b in range(B):
        nb = int(n_pages[b])
        forced = set(range(min(w.n_sink, nb))) | set(range(max(0, nb - w.n_local), nb))
        # logical pages outside the forced physical pages (g = 1: the non-forced pages)
        candidates = np.array([p for p in range(int(w.n_logical[b])) if p // g not in forced], dtype=np.int64)
        for h in range(Hkv):
            kind, *args = w.planted
            if kind == "fixed":
                n_plant = args[0]
            elif kind == "per_pages":
                n_plant = max(1, nb // args[0])
            elif kind == "loguniform":
                n_plant = int(round(math.exp(rng.uniform(math.log(args[0]), math.log(args[1])))))
            else:
                raise ValueError(kind)
            n_plant = min(n_plant, len(candidates))
            if n_plant <= 0:
                planted[(b, h)] = np.zeros(0, dtype=np.int64)
                continue
            pages = np.sort(rng.choice(candidates, size=n_plant, replace=False))
            qs = qf[b, h * G:(h + 1) * G] if T == 1 else qf[b, :, h * G:(h + 1) * G].reshape(T * G, d)
            u = qs.sum(axis=0)
            u = u / np.linalg.norm(u)
            if isinstance(w.delta, tuple):
                _, nats = w.delta
                proj = float((qs @ u).mean())
                delta = nats / (w.sm_scale * proj) if proj > 0 else 0.0
            else:
                delta = float(w.delta)
            shift = torch.from_numpy((delta * u).astype(np.float32))
            if g == 1:
                phys = torch.from_numpy(block_table[b, pages].astype(np.int64))
                kz[phys, h] += shift[None, None, :]
            else:  # the 16 token slots of each planted logical page inside its physical page
                phys = np.repeat(block_table[b, pages // g].astype(np.int64), LOGICAL_PAGE)
                slot = ((pages % g) * LOGICAL_PAGE)[:, None] + np.arange(LOGICAL_PAGE)[None, :]
                kz[torch.from_numpy(phys), h, torch.from_numpy(slot.reshape(-1))] += shift[None, :]
            planted[(b, h)] = pages
            deltas[(b, h)] = delta

    # invalid slots: tail of each partial last page and unused (hole) pages hold NaN
    valid_tail = {}
    for b in range(B):
        nb = int(n_pages[b])
        if nb and w.seq_lens[b] % P:
            valid_tail[int(block_table[b, nb - 1])] = int(w.seq_lens[b]) - P * (nb - 1)
    holes = np.setdiff1d(np.arange(universe), used)

    if w.kv_dtype == "fp8":
        k_pool, k_scale = _quantize_e4m3fn(kz)
        v_pool, v_scale = _quantize_e4m3fn(vz)
        for pg, valid in valid_tail.items():
            for arr in (k_pool, v_pool):
                arr[pg, :, valid:, :] = 0x7F
            for arr in (k_scale, v_scale):
                arr[pg, :, valid:] = np.float16(np.nan)
        for arr in (k_pool, v_pool):
            arr[holes] = 0x7F
        for arr in (k_scale, v_scale):
            arr[holes] = np.float16(np.nan)
    else:
        tdt = {"f32": torch.float32, "f16": torch.float16}[w.kv_dtype]
        k_pool = kz.to(tdt).numpy()
        v_pool = vz.to(tdt).numpy()
        k_scale = v_scale = None
        for pg, valid in valid_tail.items():
            k_pool[pg, :, valid:, :] = np.nan
            v_pool[pg, :, valid:, :] = np.nan
        k_pool[holes] = np.nan
        v_pool[holes] = np.nan
    del kz, vz

    head_kind = np.zeros(Hkv, dtype=np.uint8)
    for h in w.streaming_heads:
        head_kind[h] = 1

    return Inputs(workload=w, q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
                  block_table=block_table, seq_lens=np.array(w.seq_lens, dtype=np.int32),
                  head_kind=head_kind, planted=planted, deltas=deltas)


def small(name: str = "small", *, seq_lens=(700, 37, 2050), Hq=8, Hkv=2, d=128, kv="f16", q="f16",
          mode="topk", budget=24, gamma=0.95, n_sink=1, n_local=2, n_sink_stream=2,
          n_local_stream=3, streaming=(), planted=("fixed", 4), delta=2.0, hole=0.25,
          seed=BASE_SEED + 50, **kw) -> Workload:
    """A small ragged workload for parity tests (several tiles plus a partial tail)."""
    return Workload(name=name, seq_lens=tuple(seq_lens), num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=d, kv_dtype=kv, q_dtype=q, mode=mode, budget_pages=budget, gamma=gamma,
                    n_sink=n_sink, n_local=n_local, n_sink_stream=n_sink_stream,
                    n_local_stream=n_local_stream, streaming_heads=tuple(streaming),
                    planted=planted, delta=delta, hole_fraction=hole, seed=seed, **kw)
