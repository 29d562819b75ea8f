"""Device buffers and the call sequence of one decode step (marshalling only).

Every arithmetic step runs in the HIP library: this module allocates torch tensors for
inputs, intermediates and outputs, fills the C descriptors, and calls the entry points of
``include/spd.h`` in the method's order --

    page_meta_build (tail page) -> page_score -> page_select -> sparse_paged_decode -> lse_merge

(or page_score_select in place of the middle two), so the whole step can be captured into
one hipGraph and replayed.  In top-K mode the last page of a row is always kept by the local
window, so its score is not needed in the step that appends to it: by default the scorer
skips it and the selector's spare workgroups rebuild its statistics beside the selection.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import _abi as A
from .workloads import Inputs, Workload

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "fp8": torch.uint8}


@dataclasses.dataclass
class Plan:
    """Self-planned split constants (Moira, section 3.3, Eq. 4), re-chosen for 16-token pages
    and 256 compute units: a chunk of at least 4 pages (one per wave of a block), at least 8
    blocks per row and at least 512 blocks over the grid -- the blocks that two waves per SIMD
    keep resident at once, so rows of a batch of 8 requests are not split into a second round of
    blocks.  ``balanced`` splits the step's total listed pages evenly instead of each row into J
    chunks (for skewed list lengths; see spd_plan_params)."""
    min_chunk: int = 4
    min_blocks_per_row: int = 8
    min_grid_blocks: int = 512
    balanced: bool = False

    def params(self) -> A.PlanParams:
        return A.PlanParams(self.min_chunk, self.min_blocks_per_row, self.min_grid_blocks, int(self.balanced))


@dataclasses.dataclass
class DeviceInputs:
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scale: torch.Tensor | None
    v_scale: torch.Tensor | None
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    head_kind: np.ndarray      # host
    page_meta: torch.Tensor    # [B, Hkv, pages * g, 2, d]: key min / max, or (mvar) key mean / variance in bf16

    @property
    def num_pool_pages(self) -> int:
        return int(self.k_pool.shape[0])


def upload(inp: Inputs, device="cuda") -> DeviceInputs:
    """Copy one step's stored inputs to the device and allocate the page-summary buffer."""
    w = inp.workload

    def t(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)

    k_scale = None if inp.k_scale is None else t(inp.k_scale.view(np.int16))
    v_scale = None if inp.v_scale is None else t(inp.v_scale.view(np.int16))
    mdt = torch.bfloat16 if w.estimator == "mvar" else torch.float32 if w.kv_dtype == "f32" else torch.float16
    g = w.page_size // 16  # logical pages per physical page (hierarchical paging)
    # per request in logical page order, head-major: a row's scan reads one contiguous run
    meta = torch.zeros((w.batch, w.num_kv_heads, w.pages_per_seq * g, 2, w.head_dim), dtype=mdt, device=device)
    return DeviceInputs(q=t(inp.q), k_pool=t(inp.k_pool), v_pool=t(inp.v_pool), k_scale=k_scale, v_scale=v_scale,
                        block_table=t(inp.block_table), seq_lens=t(inp.seq_lens), head_kind=inp.head_kind.copy(),
                        page_meta=meta)


def make_desc(w: Workload, num_pool_pages: int, max_list: int | None = None) -> A.Desc:
    return A.Desc(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  page_size=w.page_size, max_pages_per_seq=w.pages_per_seq, num_pool_pages=num_pool_pages,
                  max_list=max_list or w.list_capacity, q_dtype=A.DTYPE[w.q_dtype], kv_dtype=A.DTYPE[w.kv_dtype])


def reuse_slack(reuse: int, page_size: int = 16) -> int:
    """List entries a chunk of `reuse` steps can append to a selection: one page per page_size
    tokens appended, plus the page a step may open."""
    return 0 if reuse <= 1 else (reuse - 1) // page_size + 2


def make_select(w: Workload) -> A.SelectParams:
    return A.SelectParams(mode=A.SELECT_COVERAGE if w.mode == "coverage" else A.SELECT_TOPK,
                          budget_pages=max(1, w.budget_pages), gamma=float(w.gamma) if w.gamma else 1.0,
                          sm_scale=w.sm_scale, n_sink=w.n_sink, n_local=w.n_local,
                          n_sink_stream=w.n_sink_stream, n_local_stream=w.n_local_stream,
                          estimator=A.ESTIMATOR_MVAR if w.estimator == "mvar" else A.ESTIMATOR_BOUND)


def build_summaries(w: Workload, d: DeviceInputs, first_page, span: int, stream=None) -> None:
    """Page summaries of the workload's estimator: key min / max, or key mean / variance (mvar)."""
    fn = A.spd_page_stats_build if w.estimator == "mvar" else A.spd_page_meta_build
    fn(make_desc(w, d.num_pool_pages), d.k_pool, d.k_scale, d.block_table, d.seq_lens, first_page, span, d.page_meta,
       stream)


def build_meta(w: Workload, d: DeviceInputs, stream=None) -> None:
    """Bulk page statistics of every page in the block tables (done once, at prefill)."""
    build_summaries(w, d, None, 0, stream)


TAILS = ("auto", "none", "select", "side", "serial", "rebuild")


def gate_state(rows: int, device) -> torch.Tensor:
    """A zeroed LiteTopK gate state for `rows` (token) rows (spd_select_params.topk_state)."""
    return torch.zeros(A.spd_topk_state_bytes(rows), dtype=torch.uint8, device=device)


def gate_paths(state: torch.Tensor, rows: int) -> np.ndarray:
    """How each row's last selection ran (1: from the gated candidates, 0: whole row) and the candidates it saw."""
    hdr = state[:rows * A.GATE_ROW_BYTES].view(torch.int32).view(rows, 8).cpu().numpy()
    return hdr[:, 3:5]


class DecodeStep:
    """Buffers for one decode step of workload ``w`` over device inputs ``d``.

    ``fused`` scores and selects in one launch; otherwise (default: faster on MI355X, where one
    workgroup per row selects either way) scoring and selection are two calls.  ``tail`` says
    how the key statistics of the page each request's newest token is in are rebuilt:

    * ``"none"``: not at all (the statistics are current);
    * ``"select"``: by the selector's spare workgroups (all heads), after a scorer that skips
      that page (top-K with a local window, unfused);
    * ``"side"``: the all-heads rebuild (``refresh_tail``) on a second stream, concurrent with a
      scorer that skips that page (top-K with a local window);
    * ``"serial"``: the all-heads rebuild, then a scorer that reads the rebuilt statistics;
    * ``"rebuild"``: inside the scorer, by workgroups at the front of its grid (one per request
      and KV head: the bound estimator), which run beside the scan;
    * ``"auto"`` (default): ``"select"`` where it applies, else ``"rebuild"`` on 16-token pages
      (a fused top-K step, coverage, top-K without a local window, and the mvar estimator, whose
      scorer reads that page's keys anyway), else ``"serial"``.

    With the mvar estimator (Moira, section 3.1) ``d.page_meta`` holds the bf16 page summaries
    and the scorer computes each row's first and current pages exactly; scoring and selection are
    then two calls.

    ``phys_lists`` (default) has the selector write the physical page of every list entry so
    the decode kernel does not read the block table.  ``keep_sel_scores`` has it also write the
    score of every listed page (``sel_scores``); the step itself does not need them.

    ``reuse`` = C > 1 sizes the lists for reusable page selection (LServe, "Reusable Page
    Selection"): ``run`` selects on the first step of a chunk of C steps and ``reuse_step`` serves
    the other C - 1, after the requests have grown, with the chunk's lists plus the current sink and
    local pages.
    """

    def __init__(self, w: Workload, d: DeviceInputs, plan: Plan | None = None, fused: bool = False,
                 tail: str = "auto", phys_lists: bool = True, keep_sel_scores: bool = False, reuse: int = 1,
                 merged: bool = False, gated: bool | None = None):
        if tail not in TAILS:
            raise ValueError(f"tail must be one of {TAILS}")
        skippable = w.mode == "topk" and w.n_local >= 1
        if fused and w.estimator == "mvar":
            raise ValueError("the fused score + select launch has no mvar estimator")
        if tail == "auto":
            tail = (("rebuild" if fused else "select") if skippable else
                    "rebuild" if w.page_size == 16 else "serial")
        if tail in ("select", "side") and not skippable:
            raise ValueError(f"tail={tail!r} skips the last page: top-K with a local window only")
        if tail == "select" and fused:
            raise ValueError("tail='select' needs the separate selector (fused=False)")
        self.w, self.d = w, d
        # coverage lists range from the forced pages to the whole row: split the step evenly
        self.plan = plan or (Plan(balanced=True) if w.mode == "coverage" else Plan())
        self.fused = fused
        self.tail = tail
        self.tail_mode = {"none": A.TAIL_NONE, "select": A.TAIL_SKIP, "side": A.TAIL_SKIP, "serial": A.TAIL_NONE,
                          "rebuild": A.TAIL_REBUILD}[tail]
        self.side = torch.cuda.Stream(device=d.q.device) if tail == "side" else None
        self.phys_lists = phys_lists
        dev = d.q.device
        self.reuse = reuse
        self.max_list = w.list_capacity + reuse_slack(reuse, w.page_size)
        self.desc = make_desc(w, d.num_pool_pages, self.max_list)
        self.sel = make_select(w)
        self.pp = self.plan.params()
        B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        # LiteTopK gate (top-K, bound estimator, 16-token pages, separate scorer and selector)
        gate_ok = w.mode == "topk" and w.estimator == "bound" and w.page_size == 16 and not fused
        self.gated = gate_ok if gated is None else bool(gated)
        if self.gated and not gate_ok:
            raise ValueError("the LiteTopK gate needs top-K, the bound estimator, 16-token pages and fused=False")
        self.topk_state = gate_state(B * Hkv, d.q.device) if self.gated else None
        if self.gated:
            self.sel.topk_state = self.topk_state.data_ptr()
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.zeros((B, Hkv, w.pages_per_seq), **f32)
        self.head_lse = torch.zeros((B, Hq), **f32)
        self.page_list = torch.zeros((B, Hkv, self.max_list), **i32)
        self.page_phys = torch.zeros((B, Hkv, self.max_list), **i32) if phys_lists else None
        self.list_len = torch.zeros((B, Hkv), **i32)
        self.sel_scores = torch.zeros((B, Hkv, self.max_list), **f32) if keep_sel_scores else None
        self.out = torch.zeros((B, Hq, D), **f32)
        self.out_lse = torch.zeros((B, Hq), **f32)
        self.J = A.spd_plan_grid(self.desc, self.pp)
        n_po, n_pl = A.spd_partials_size(self.desc, self.pp)
        self.part_o = torch.zeros(max(1, n_po), **f32)
        self.part_lse = torch.zeros(max(1, n_pl), **f32)
        op = A.OP_PAGE_SCORE_SELECT if self.fused else A.OP_PAGE_SCORE
        self.ws_bytes = A.spd_workspace_bytes(self.desc, self.sel, op)
        self.workspace = torch.zeros(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        # merged: decode and merge in one launch (row tickets, zero between calls)
        self.merged = merged
        self.counters = torch.zeros((B, Hkv), **i32) if merged else None

    def refresh_tail(self, stream=None):
        """Summary of the page the newest token is in (one page per request, all heads)."""
        build_summaries(self.w, self.d, None, 1, stream)

    def score(self, stream=None, tail_mode=None):
        """Page scores, treating each dynamic row's last page by the step's tail mode."""
        d = self.d
        tm = self.tail_mode if tail_mode is None else tail_mode
        A.spd_page_score(self.desc, self.sel, d.q, d.page_meta, d.k_pool, d.k_scale, tm, d.block_table,
                         d.seq_lens, d.head_kind, self.scores, self.head_lse, self.workspace, self.ws_bytes, stream)

    def select_only(self, stream=None):
        """Page lists from the scores (and, with tail="select", the last pages' statistics)."""
        d = self.d
        rebuild = self.tail == "select"
        A.spd_page_select(self.desc, self.sel, self.scores, d.seq_lens, d.head_kind, d.block_table,
                          d.k_pool if rebuild else None, d.k_scale if rebuild else None,
                          d.page_meta if rebuild else None, self.page_list, self.page_phys, self.list_len,
                          self.sel_scores, stream)

    def score_select(self, stream=None):
        d = self.d
        A.spd_page_score_select(self.desc, self.sel, d.q, d.page_meta, d.k_pool, d.k_scale, self.tail_mode,
                                d.block_table, d.seq_lens, d.head_kind, self.page_list, self.page_phys,
                                self.list_len, self.sel_scores, self.scores, self.head_lse, self.workspace,
                                self.ws_bytes, stream)

    def select(self, stream=None):
        """Scores and page lists (the fused launch, or the scorer then the selector)."""
        if self.fused:
            self.score_select(stream)
        else:
            self.score(stream)
            self.select_only(stream)

    def decode(self, stream=None):
        d = self.d
        A.spd_sparse_paged_decode(self.desc, self.pp, d.q, d.k_pool, d.v_pool, d.k_scale, d.v_scale, d.block_table,
                                  d.seq_lens, self.page_list, self.page_phys, self.list_len, self.w.sm_scale,
                                  self.out, self.out_lse, self.part_o, self.part_lse, stream)

    def merge(self, stream=None):
        A.spd_lse_merge(self.desc, self.pp, self.part_o, self.part_lse, self.list_len, self.out, self.out_lse,
                        stream)

    def attend(self, stream=None):
        if self.merged:
            d = self.d
            A.spd_sparse_paged_decode_merged(self.desc, self.pp, d.q, d.k_pool, d.v_pool, d.k_scale, d.v_scale,
                                             d.block_table, d.seq_lens, self.page_list, self.page_phys, self.list_len,
                                             self.w.sm_scale, self.out, self.out_lse, self.part_o, self.part_lse,
                                             self.counters, stream)
            return
        self.decode(stream)
        self.merge(stream)

    def reuse_step(self, stream=None):
        """A later step of a reuse chunk: the chunk's lists plus the current forced pages (and the
        newest pages' statistics rebuilt beside them), then attention."""
        d = self.d
        rebuild = self.tail != "none"
        A.spd_page_list_refresh(self.desc, self.sel, d.seq_lens, d.head_kind, d.block_table,
                                d.k_pool if rebuild else None, d.k_scale if rebuild else None,
                                d.page_meta if rebuild else None, self.page_list, self.page_phys, self.list_len,
                                stream)
        self.attend(stream)

    def run(self, stream=None):
        """One whole step on `stream` (a torch stream or a raw HIP stream handle; None: torch's
        current stream)."""
        if self.tail == "serial":
            self.refresh_tail(stream)
        if self.tail != "side":
            self.select(stream)
            self.attend(stream)
            return
        if stream is None:
            main = torch.cuda.current_stream()
        elif isinstance(stream, int):
            main = torch.cuda.ExternalStream(stream, device=self.d.q.device)
        else:
            main = stream
        self.side.wait_stream(main)  # fork: the rebuild starts after what `stream` already holds
        self.refresh_tail(self.side.cuda_stream)
        self.select(stream)
        self.attend(stream)
        main.wait_stream(self.side)  # join

    def lists(self) -> dict:
        """Host copy of the page lists: {(b, h): [pages]}."""
        pl = self.page_list.cpu().numpy()
        ll = self.list_len.cpu().numpy()
        return {(b, h): pl[b, h, :ll[b, h]].tolist() for b in range(self.w.batch)
                for h in range(self.w.num_kv_heads)}


class MQDecodeStep:
    """One decode step for T > 1 query tokens per request (the draft tokens speculative decoding
    verifies at once), with the tokens' page lists scanned as one union (LiteTopK, section 3.4).

    Request b's cache holds ``seq_lens[b]`` = L keys, the draft tokens' included; token t attends to
    positions < L - T + 1 + t.  Each token selects its pages as a single query of that length: the
    scorer and the selector run over B * T rows that share their request's block-table row.  The
    rows' lists are merged per (request, KV head) with a membership mask per entry, and the
    several-query decode reads each union page once for all T x G query rows.  ``d.q`` is
    [B, T, Hq, d]; ``out`` is [B, T, Hq, d] and ``out_lse`` [B, T, Hq].
    """

    def __init__(self, w: Workload, d: DeviceInputs, plan: Plan | None = None, gated: bool = True,
                 tail: str = "auto"):
        T = w.num_queries
        if T < 2 or w.mode != "topk" or w.page_size != 16:
            raise ValueError("several query tokens: top-K over 16-token pages, T >= 2")
        # "select": the scorer skips each request's last two pages (in every token's local window of
        # at least two pages) and the selector's spare workgroups rebuild their statistics; "serial":
        # a rebuild launch before a scorer that reads them; "auto" picks "select" where it applies
        skippable = w.n_local >= 2
        if tail == "auto":
            tail = "select" if skippable else "serial"
        if tail not in ("select", "serial"):
            raise ValueError("tail must be 'auto', 'select' or 'serial'")
        if tail == "select" and not skippable:
            raise ValueError("tail='select' needs a local window of at least two pages")
        self.tail = tail
        self.w, self.d, self.T = w, d, T
        self.plan = plan or Plan()
        self.pp = self.plan.params()
        dev = d.q.device
        B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.token_cap = w.list_capacity
        self.union_cap = min(T * self.token_cap, w.pages_per_seq)
        self.desc = make_desc(w, d.num_pool_pages, self.union_cap)                 # the B requests
        self.sel = make_select(w)
        # LiteTopK gate of the B * T token rows, each predicted from that row's previous selection
        self.gated = gated
        self.topk_state = gate_state(B * T * Hkv, dev) if gated else None
        if gated:
            self.sel.topk_state = self.topk_state.data_ptr()
        # the B * T token rows (row b T + t) share their request's block-table row and length; the
        # library derives each token's causal length from d.seq_lens on every call
        self.scores = torch.zeros((B * T, Hkv, w.pages_per_seq), **f32)
        self.token_list = torch.zeros((B * T, Hkv, self.token_cap), **i32)
        self.token_len = torch.zeros((B * T, Hkv), **i32)
        self.page_list = torch.zeros((B, Hkv, self.union_cap), **i32)
        self.page_phys = torch.zeros((B, Hkv, self.union_cap), **i32)
        self.page_mask = torch.zeros((B, Hkv, self.union_cap), **i32)  # uint32 bits
        self.list_len = torch.zeros((B, Hkv), **i32)
        self.out = torch.zeros((B, T, Hq, D), **f32)
        self.out_lse = torch.zeros((B, T, Hq), **f32)
        self.J = A.spd_plan_grid(self.desc, self.pp)
        self.part_o = torch.zeros(B * Hkv * self.J * A.MQ_ROWS * D, **f32)
        self.part_lse = torch.zeros(B * Hkv * self.J * A.MQ_ROWS, **f32)

    def refresh_tail(self, stream=None):
        """Key statistics of the pages the draft tokens are in (the last two pages of each request)."""
        A.spd_page_meta_build(self.desc, self.d.k_pool, self.d.k_scale, self.d.block_table, self.d.seq_lens, None, 2,
                              self.d.page_meta, stream)

    def score(self, stream=None, tail_mode=None):
        """Page scores of every token row: one scan that reads each key box once for the T tokens (with
        the "select" tail, the request's last two pages are not scored)."""
        d = self.d
        tm = (A.TAIL_SKIP if self.tail == "select" else A.TAIL_NONE) if tail_mode is None else tail_mode
        A.spd_page_score_mq(self.desc, self.T, self.sel, d.q, d.page_meta, tm, d.block_table, d.seq_lens,
                            d.head_kind, self.scores, stream)

    def select_only(self, stream=None):
        """Each token row's page list from its scores (lengths read on the device); with the "select"
        tail, spare workgroups rebuild the statistics of each request's last two pages."""
        d = self.d
        meta = d.page_meta if self.tail == "select" else None
        A.spd_page_select_mq(self.desc, self.T, self.token_cap, self.sel, self.scores, d.seq_lens, d.head_kind,
                             d.block_table, d.k_pool, d.k_scale, meta, self.token_list, None, self.token_len,
                             stream)

    def select(self, stream=None):
        self.score(stream)
        self.select_only(stream)

    def union(self, stream=None, path=None):
        """The union of the token lists; `path` ([B, Hkv] int32, optional) receives 1 for rows merged by rank
        and 0 for rows built in the byte map."""
        d = self.d
        A.spd_page_list_union(self.desc, self.T, self.token_cap, self.token_list, self.token_len, d.block_table,
                              d.seq_lens, self.page_list, self.page_phys, self.page_mask, self.list_len, stream,
                              union_path=path)

    def attend(self, stream=None):
        d = self.d
        A.spd_sparse_paged_decode_mq(self.desc, self.T, self.pp, d.q, d.k_pool, d.v_pool, d.k_scale, d.v_scale,
                                     d.block_table, d.seq_lens,
                                     self.page_list, self.page_phys, self.page_mask, self.list_len, self.w.sm_scale,
                                     self.out, self.out_lse, self.part_o, self.part_lse, stream)
        A.spd_lse_merge_mq(self.desc, self.T, self.pp, self.part_o, self.part_lse, self.list_len, self.out,
                           self.out_lse, stream)

    def run(self, stream=None):
        if self.tail == "serial":
            self.refresh_tail(stream)
        self.select(stream)
        self.union(stream)
        self.attend(stream)

    def token_lists(self) -> list:
        """Host copy of each token's lists: [T] of {(b, h): [pages]}."""
        pl = self.token_list.cpu().numpy()
        ll = self.token_len.cpu().numpy()
        B, T = self.w.batch, self.T
        return [{(b, h): pl[b * T + t, h, :ll[b * T + t, h]].tolist() for b in range(B)
                 for h in range(self.w.num_kv_heads)} for t in range(T)]

    def union_lists(self) -> dict:
        """Host copy of the union lists: {(b, h): (pages, masks)}."""
        pl = self.page_list.cpu().numpy()
        pm = self.page_mask.cpu().numpy().astype(np.int64) & 0xffffffff
        ll = self.list_len.cpu().numpy()
        return {(b, h): (pl[b, h, :ll[b, h]].tolist(), pm[b, h, :ll[b, h]].tolist()) for b in range(self.w.batch)
                for h in range(self.w.num_kv_heads)}
