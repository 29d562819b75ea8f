"""ctypes binding of ``libspd.so`` -- argument marshalling only.

Each ``spd_*`` function here has the name and argument order of the C entry point in
``include/spd.h``; torch tensors are passed as their ``data_ptr()`` (``None`` -> NULL) and
the stream defaults to torch's current stream.  A non-zero status raises ``SpdError``.
There is no fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_uint8, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspd.so")

SPD_OK = 0
SPD_ERR_INVALID_ARG = -1
SPD_ERR_UNSUPPORTED = -2
SPD_ERR_LAUNCH = -3
SPD_ERR_WORKSPACE = -4

DTYPE = {"f32": 0, "f16": 1, "fp8": 2}
SELECT_TOPK, SELECT_COVERAGE = 0, 1
HEAD_DYNAMIC, HEAD_STREAMING = 0, 1
OP_PAGE_SCORE, OP_PAGE_SELECT, OP_PAGE_SCORE_SELECT = 0, 1, 2
TAIL_NONE, TAIL_REBUILD, TAIL_SKIP = 0, 1, 2
ESTIMATOR_BOUND, ESTIMATOR_MVAR = 0, 1

EXPORTS = ("spd_page_meta_build", "spd_page_stats_build", "spd_page_score", "spd_page_select", "spd_page_score_select",
           "spd_sparse_paged_decode", "spd_lse_merge", "spd_plan_grid", "spd_plan_chunks", "spd_page_list_refresh",
           "spd_partials_size", "spd_workspace_bytes", "spd_error_string", "spd_abi_version",
           "spd_page_list_union", "spd_sparse_paged_decode_mq", "spd_lse_merge_mq", "spd_sparse_paged_decode_merged",
           "spd_page_score_mq", "spd_page_select_mq", "spd_sparse_paged_decode_noalloc", "spd_topk_state_bytes")
MQ_ROWS = 16  # chunk-state rows per (request, KV head) of the several-query decode


class SpdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {error_string(status)} ({status})")


class Desc(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("num_q_heads", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("page_size", c_int32), ("max_pages_per_seq", c_int32),
                ("num_pool_pages", c_int32), ("max_list", c_int32), ("q_dtype", c_int32),
                ("kv_dtype", c_int32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("budget_pages", c_int32), ("gamma", c_float), ("sm_scale", c_float),
                ("n_sink", c_int32), ("n_local", c_int32), ("n_sink_stream", c_int32),
                ("n_local_stream", c_int32), ("estimator", c_int32), ("topk_state", c_void_p)]


class PlanParams(ctypes.Structure):
    _fields_ = [("min_chunk", c_int32), ("min_blocks_per_row", c_int32), ("min_grid_blocks", c_int32),
                ("balanced", c_int32)]


_lib = None


def lib():
    """Load the built library (raises when it is missing: there is no other path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_paged_decode_quest_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D, S, P = POINTER(Desc), POINTER(SelectParams), POINTER(PlanParams)
        v = c_void_p
        L.spd_page_meta_build.argtypes = [D, v, v, v, v, v, c_int32, v, v]
        L.spd_page_stats_build.argtypes = [D, v, v, v, v, v, c_int32, v, v]
        L.spd_page_score.argtypes = [D, S, v, v, v, v, c_int32, v, v, POINTER(c_uint8), v, v, v, c_size_t, v]
        L.spd_page_select.argtypes = [D, S, v, v, POINTER(c_uint8), v, v, v, v, v, v, v, v, v]
        L.spd_page_list_refresh.argtypes = [D, S, v, POINTER(c_uint8), v, v, v, v, v, v, v, v]
        L.spd_page_score_select.argtypes = [D, S, v, v, v, v, c_int32, v, v, POINTER(c_uint8), v, v, v, v, v, v, v,
                                            c_size_t, v]
        L.spd_sparse_paged_decode.argtypes = [D, P, v, v, v, v, v, v, v, v, v, v, c_float, v, v, v, v, v]
        L.spd_lse_merge.argtypes = [D, P, v, v, v, v, v, v]
        L.spd_sparse_paged_decode_noalloc.argtypes = [D, P, v, v, v, v, v, v, v, v, v, v, c_float, v, v, v]
        L.spd_sparse_paged_decode_merged.argtypes = [D, P, v, v, v, v, v, v, v, v, v, v, c_float, v, v, v, v, v, v]
        L.spd_page_list_union.argtypes = [D, c_int32, c_int32, v, v, v, v, v, v, v, v, v, v]
        L.spd_page_score_mq.argtypes = [D, c_int32, S, v, v, c_int32, v, v, POINTER(c_uint8), v, v]
        L.spd_page_select_mq.argtypes = [D, c_int32, c_int32, S, v, v, POINTER(c_uint8), v, v, v, v, v, v, v, v]
        L.spd_sparse_paged_decode_mq.argtypes = [D, c_int32, P, v, v, v, v, v, v, v, v, v, v, v, c_float, v, v, v, v,
                                                 v]
        L.spd_lse_merge_mq.argtypes = [D, c_int32, P, v, v, v, v, v, v]
        L.spd_plan_grid.argtypes = [D, P, POINTER(c_int32)]
        L.spd_plan_chunks.argtypes = [c_int32, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32)]
        L.spd_partials_size.argtypes = [D, P, POINTER(c_size_t), POINTER(c_size_t)]
        L.spd_workspace_bytes.argtypes = [D, S, c_int32]
        L.spd_workspace_bytes.restype = c_size_t
        L.spd_topk_state_bytes.argtypes = [c_int32]
        L.spd_topk_state_bytes.restype = c_size_t
        L.spd_error_string.argtypes = [c_int32]
        L.spd_error_string.restype = ctypes.c_char_p
        L.spd_abi_version.argtypes = []
        for name in EXPORTS:
            if name not in ("spd_workspace_bytes", "spd_error_string", "spd_topk_state_bytes"):
                getattr(L, name).restype = c_int32
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _heads(head_kind):
    arr = (c_uint8 * len(head_kind))(*[int(x) for x in head_kind])
    return arr


def _check(rc: int, where: str):
    if rc != SPD_OK:
        raise SpdError(rc, where)


def error_string(status: int) -> str:
    return lib().spd_error_string(status).decode()


def abi_version() -> int:
    return lib().spd_abi_version()


def spd_page_meta_build(desc, k_pool, k_scale, block_table, seq_lens, first_page, span_pages, page_meta,
                        stream=None):
    _check(lib().spd_page_meta_build(ctypes.byref(desc), _ptr(k_pool), _ptr(k_scale), _ptr(block_table),
                                     _ptr(seq_lens), _ptr(first_page), int(span_pages), _ptr(page_meta),
                                     _stream(stream)), "spd_page_meta_build")


def spd_page_stats_build(desc, k_pool, k_scale, block_table, seq_lens, first_page, span_pages, page_stats,
                         stream=None):
    _check(lib().spd_page_stats_build(ctypes.byref(desc), _ptr(k_pool), _ptr(k_scale), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(first_page), int(span_pages), _ptr(page_stats),
                                      _stream(stream)), "spd_page_stats_build")


def spd_page_score(desc, sel, q, page_meta, k_pool, k_scale, tail_mode, block_table, seq_lens, head_kind, scores,
                   head_lse, workspace, workspace_bytes, stream=None):
    _check(lib().spd_page_score(ctypes.byref(desc), ctypes.byref(sel), _ptr(q), _ptr(page_meta), _ptr(k_pool),
                                _ptr(k_scale), int(tail_mode), _ptr(block_table), _ptr(seq_lens), _heads(head_kind),
                                _ptr(scores), _ptr(head_lse), _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "spd_page_score")


def spd_page_select(desc, sel, scores, seq_lens, head_kind, block_table, k_pool, k_scale, page_meta, page_list,
                    page_phys, list_len, sel_scores, stream=None):
    _check(lib().spd_page_select(ctypes.byref(desc), ctypes.byref(sel), _ptr(scores), _ptr(seq_lens),
                                 _heads(head_kind), _ptr(block_table), _ptr(k_pool), _ptr(k_scale), _ptr(page_meta),
                                 _ptr(page_list), _ptr(page_phys), _ptr(list_len), _ptr(sel_scores),
                                 _stream(stream)), "spd_page_select")


def spd_page_list_refresh(desc, sel, seq_lens, head_kind, block_table, k_pool, k_scale, page_meta, page_list,
                          page_phys, list_len, stream=None):
    _check(lib().spd_page_list_refresh(ctypes.byref(desc), ctypes.byref(sel), _ptr(seq_lens), _heads(head_kind),
                                       _ptr(block_table), _ptr(k_pool), _ptr(k_scale), _ptr(page_meta),
                                       _ptr(page_list), _ptr(page_phys), _ptr(list_len), _stream(stream)),
           "spd_page_list_refresh")


def spd_page_score_select(desc, sel, q, page_meta, k_pool, k_scale, tail_mode, block_table, seq_lens, head_kind,
                          page_list, page_phys, list_len, sel_scores, scores, head_lse, workspace, workspace_bytes,
                          stream=None):
    _check(lib().spd_page_score_select(ctypes.byref(desc), ctypes.byref(sel), _ptr(q), _ptr(page_meta), _ptr(k_pool),
                                       _ptr(k_scale), int(tail_mode), _ptr(block_table), _ptr(seq_lens),
                                       _heads(head_kind), _ptr(page_list), _ptr(page_phys), _ptr(list_len),
                                       _ptr(sel_scores), _ptr(scores), _ptr(head_lse), _ptr(workspace),
                                       int(workspace_bytes), _stream(stream)), "spd_page_score_select")


def spd_sparse_paged_decode(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, page_list,
                            page_phys, list_len, sm_scale, out, out_lse, part_o, part_lse, stream=None):
    _check(lib().spd_sparse_paged_decode(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k_pool),
                                         _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                         _ptr(seq_lens), _ptr(page_list), _ptr(page_phys), _ptr(list_len),
                                         float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(part_o), _ptr(part_lse),
                                         _stream(stream)), "spd_sparse_paged_decode")


def spd_sparse_paged_decode_merged(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, page_list,
                                   page_phys, list_len, sm_scale, out, out_lse, part_o, part_lse, counters,
                                   stream=None):
    _check(lib().spd_sparse_paged_decode_merged(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k_pool),
                                                _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                                _ptr(seq_lens), _ptr(page_list), _ptr(page_phys), _ptr(list_len),
                                                float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(part_o),
                                                _ptr(part_lse), _ptr(counters), _stream(stream)),
           "spd_sparse_paged_decode_merged")


def spd_sparse_paged_decode_noalloc(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                                    page_list, page_phys, list_len, sm_scale, out, out_lse, stream=None):
    _check(lib().spd_sparse_paged_decode_noalloc(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k_pool),
                                                 _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                                 _ptr(seq_lens), _ptr(page_list), _ptr(page_phys), _ptr(list_len),
                                                 float(sm_scale), _ptr(out), _ptr(out_lse), _stream(stream)),
           "spd_sparse_paged_decode_noalloc")


def spd_lse_merge(desc, plan, part_o, part_lse, list_len, out, out_lse, stream=None):
    _check(lib().spd_lse_merge(ctypes.byref(desc), ctypes.byref(plan), _ptr(part_o), _ptr(part_lse),
                               _ptr(list_len), _ptr(out), _ptr(out_lse), _stream(stream)), "spd_lse_merge")


def spd_page_score_mq(desc, num_tokens, sel, q, page_meta, tail_mode, block_table, seq_lens, head_kind, scores,
                      stream=None):
    _check(lib().spd_page_score_mq(ctypes.byref(desc), int(num_tokens), ctypes.byref(sel), _ptr(q), _ptr(page_meta),
                                   int(tail_mode), _ptr(block_table), _ptr(seq_lens), _heads(head_kind),
                                   _ptr(scores), _stream(stream)),
           "spd_page_score_mq")


def spd_page_select_mq(desc, num_tokens, token_max_list, sel, scores, seq_lens, head_kind, block_table, k_pool,
                       k_scale, page_meta, token_list, token_phys, token_len, stream=None):
    _check(lib().spd_page_select_mq(ctypes.byref(desc), int(num_tokens), int(token_max_list), ctypes.byref(sel),
                                    _ptr(scores), _ptr(seq_lens), _heads(head_kind), _ptr(block_table),
                                    _ptr(k_pool), _ptr(k_scale), _ptr(page_meta), _ptr(token_list),
                                    _ptr(token_phys), _ptr(token_len), _stream(stream)),
           "spd_page_select_mq")


def spd_page_list_union(desc, num_tokens, token_max_list, token_list, token_len, block_table, seq_lens, page_list,
                        page_phys, page_mask, list_len, stream=None, union_path=None):
    _check(lib().spd_page_list_union(ctypes.byref(desc), int(num_tokens), int(token_max_list), _ptr(token_list),
                                     _ptr(token_len), _ptr(block_table), _ptr(seq_lens), _ptr(page_list),
                                     _ptr(page_phys), _ptr(page_mask), _ptr(list_len), _ptr(union_path),
                                     _stream(stream)),
           "spd_page_list_union")


def spd_sparse_paged_decode_mq(desc, num_tokens, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                               page_list, page_phys, page_mask, list_len, sm_scale, out, out_lse, part_o, part_lse,
                               stream=None):
    _check(lib().spd_sparse_paged_decode_mq(ctypes.byref(desc), int(num_tokens), ctypes.byref(plan), _ptr(q),
                                            _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                            _ptr(block_table), _ptr(seq_lens),
                                            _ptr(page_list), _ptr(page_phys), _ptr(page_mask), _ptr(list_len),
                                            float(sm_scale), _ptr(out), _ptr(out_lse), _ptr(part_o), _ptr(part_lse),
                                            _stream(stream)), "spd_sparse_paged_decode_mq")


def spd_lse_merge_mq(desc, num_tokens, plan, part_o, part_lse, list_len, out, out_lse, stream=None):
    _check(lib().spd_lse_merge_mq(ctypes.byref(desc), int(num_tokens), ctypes.byref(plan), _ptr(part_o),
                                  _ptr(part_lse), _ptr(list_len), _ptr(out), _ptr(out_lse), _stream(stream)),
           "spd_lse_merge_mq")


def spd_plan_grid(desc, plan) -> int:
    j = c_int32(0)
    _check(lib().spd_plan_grid(ctypes.byref(desc), ctypes.byref(plan), ctypes.byref(j)), "spd_plan_grid")
    return j.value


def spd_plan_chunks(n_pages: int, blocks_per_row: int, min_chunk: int):
    c, m = c_int32(0), c_int32(0)
    _check(lib().spd_plan_chunks(n_pages, blocks_per_row, min_chunk, ctypes.byref(c), ctypes.byref(m)),
           "spd_plan_chunks")
    return c.value, m.value


def spd_partials_size(desc, plan):
    a, b = c_size_t(0), c_size_t(0)
    _check(lib().spd_partials_size(ctypes.byref(desc), ctypes.byref(plan), ctypes.byref(a), ctypes.byref(b)),
           "spd_partials_size")
    return a.value, b.value


def spd_workspace_bytes(desc, sel, op) -> int:
    n = lib().spd_workspace_bytes(ctypes.byref(desc), ctypes.byref(sel), int(op))
    if n == ctypes.c_size_t(-1).value:
        raise SpdError(SPD_ERR_INVALID_ARG, "spd_workspace_bytes")
    return n


def spd_topk_state_bytes(rows: int) -> int:
    n = lib().spd_topk_state_bytes(int(rows))
    if n == ctypes.c_size_t(-1).value:
        raise SpdError(SPD_ERR_INVALID_ARG, "spd_topk_state_bytes")
    return n


# gate state of one row (spd_topk_state_bytes): float gate, float top, uint32 valid, path, seen, 3 x reserved
GATE_ROW_BYTES = 32
