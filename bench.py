"""Benchmark of one sparse paged decode step on one MI355X.

Workload: the Llama-3-8B-shaped attention layer at 128k context (batch 1, Hq 32 / Hkv 8,
d 128, 16-token fp16 pages, KV heads 0-3 streaming with 4 sink + 16 local pages, heads 4-7
top-K 256 pages with 1 sink + 2 local pages forced, 64 planted pages per head).

A step is the whole hot path: tail-page key statistics refresh -> page scores -> page
selection -> split-K decode attention -> log-sum-exp merge, captured in a hipGraph.  To
measure HBM rather than the 256 MB Infinity Cache, the bench keeps R independent copies
("layers") of every input and output and rotates through them, so a timed run touches
R x ~26 MB; every step reads its inputs from HBM-resident buffers.

Prints one JSON line (see the "metric" / "value" fields): value = achieved HBM TB/s on the
algorithmic bytes of a step (page meta scanned + the selected K/V pages + Q + O + the block
table + tail page), ms_per_step = step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse paged decode step us + achieved HBM TB/s (128k ctx, Hq32/Hkv8/d128)"
WORKLOAD = "llama3_8b_b1_128k_f16"
PEAK_HBM_TBS = 8.0
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = ["page_score.hip", "score_common.h", "page_select.hip", "select_row.h", "sparse_paged_decode.hip",
                  "page_meta_build.hip", "page_score_select.hip"]


def kernel_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_paged_decode_quest_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, list_len: np.ndarray, head_kind: np.ndarray) -> dict:
    """Minimal bytes one step must move (meta scanned, selected K/V pages, Q, O, tables)."""
    d = w.head_dim
    kv_bytes = {"f32": 4, "f16": 2, "fp8": 1}[w.kv_dtype]
    meta_bytes = 4 if w.kv_dtype == "f32" else 2
    n_pages = w.n_pages
    dyn_rows = int((head_kind == 0).sum())
    meta = sum(int(n_pages[b]) for b in range(w.batch)) * dyn_rows * 2 * d * meta_bytes
    page_kv = 16 * d * kv_bytes * 2 + (16 * 2 * 2 if w.kv_dtype == "fp8" else 0)
    kv = int(list_len.sum()) * page_kv
    q = w.batch * w.num_q_heads * d * (4 if w.q_dtype == "f32" else 2)
    o = w.batch * w.num_q_heads * (d + 1) * 4
    tables = int(n_pages.sum()) * 4 + w.batch * 4
    tail = w.batch * w.num_kv_heads * (16 * d * kv_bytes + 2 * d * meta_bytes)
    total = meta + kv + q + o + tables + tail
    return {"meta": meta, "kv": kv, "q": q, "o": o, "tables": tables, "tail": tail, "total": total}


def cpu_baseline(w, inp, seconds: float) -> dict:
    """The fp64 oracle (untuned) on the host: whole decode steps of this workload."""
    from threadpoolctl import threadpool_limits

    from oracle import spd_oracle as O

    with threadpool_limits(limits=1):
        meta = O.page_meta_build(inp)  # setup (the GPU builds it once before timing too)
        first = [max(O.n_pages(L) - 1, 0) for L in inp.seq_lens]
        steps, t0 = 0, time.perf_counter()
        while True:
            m2 = O.page_meta_build(inp, meta=meta, first_page=first)
            sel = O.page_select(inp, m2)
            O.sparse_paged_decode(inp, sel["lists"], w.sm_scale)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"steps": steps, "seconds": el, "step_s": el / steps,
            "lens": np.array([len(v) for v in sel["lists"].values()])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=40, help="independent input copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--phase-only", default=None,
                    help="launch only one phase per step (tail|score|select|decode|merge) -- for profiling")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the decode step is a single-GPU "
                                   "kernel pipeline with no collectives; more GPUs would each run it on their own requests or KV heads"}))
        sys.exit(2)

    import torch

    assert torch.cuda.is_available()
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}))
        return

    from sparse_paged_decode_quest_amd import _abi as A
    from sparse_paged_decode_quest_amd import step as S
    from sparse_paged_decode_quest_amd import workloads as W

    w = W.named(WORKLOAD)
    t_gen = time.perf_counter()
    inp = W.generate(w)
    base = S.upload(inp)
    S.build_meta(w, base)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    R = max(1, args.layers)
    layers = [base] + [S.DeviceInputs(q=base.q.clone(), k_pool=base.k_pool.clone(), v_pool=base.v_pool.clone(),
                                      k_scale=None, v_scale=None, block_table=base.block_table.clone(),
                                      seq_lens=base.seq_lens.clone(), head_kind=base.head_kind.copy(),
                                      page_meta=base.page_meta.clone()) for _ in range(R - 1)]
    steps = [S.DecodeStep(w, d) for d in layers]
    for st in steps:
        st.run()
    torch.cuda.synchronize()
    ref_lists = steps[0].lists()
    for st in (steps[1], steps[-1]):
        assert st.lists() == ref_lists and torch.equal(st.out, steps[0].out), "layer copies disagree"

    phases = {"tail": lambda st, s: st.refresh_tail(s), "select": lambda st, s: st.select(s),
              "decode": lambda st, s: A.spd_sparse_paged_decode(
                  st.desc, st.pp, st.d.q, st.d.k_pool, st.d.v_pool, st.d.k_scale, st.d.v_scale, st.d.block_table,
                  st.d.seq_lens, st.page_list, st.list_len, w.sm_scale, st.out, st.out_lse, st.part_o, st.part_lse,
                  s),
              "merge": lambda st, s: A.spd_lse_merge(st.desc, st.pp, st.part_o, st.part_lse, st.list_len,
                                                          st.out, st.out_lse, s)}
    if not steps[0].fused:
        phases["score"] = lambda st, s: A.spd_page_score(st.desc, st.sel, st.d.q, st.d.page_meta,
                                                               st.d.block_table, st.d.seq_lens, st.d.head_kind,
                                                               st.scores, st.head_lse, st.workspace, st.ws_bytes, s)
        phases["select"] = lambda st, s: A.spd_page_select(st.desc, st.sel, st.scores, st.d.seq_lens,
                                                                 st.d.head_kind, st.page_list, st.list_len,
                                                                 st.sel_scores, None, 0, s)

    stream = torch.cuda.Stream()

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(count):
                fn(steps[i % R], stream.cuda_stream)  # warm the exact launch sequence
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                fn(steps[i % R], stream.cuda_stream)
        return g

    def timed(fn, total, reps_per_graph):
        """Run `total` calls of fn (rotating layers) as graphs; returns seconds (device events)."""
        full = capture(fn, reps_per_graph)
        rem = total % reps_per_graph
        part = capture(fn, rem) if rem else None
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):  # replay() launches on the current stream: the events' stream
            ev0.record(stream)
            for _ in range(total // reps_per_graph):
                full.replay()
            if part is not None:
                part.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3

    whole = (lambda st, s: st.run(s))
    if args.phase_only:
        fn = phases[args.phase_only]
        timed(fn, args.warmup, R)
        sec = timed(fn, args.steps, R)
        print(json.dumps({"phase": args.phase_only, "us_per_launch": sec / args.steps * 1e6}))
        return

    timed(whole, args.warmup, R)                      # warm-up: W untimed steps
    torch.cuda.synchronize()
    step_s = timed(whole, args.steps, R) / args.steps  # exactly K timed steps
    # per-phase time (each phase alone, rotated over the same layers)
    phase_us = {}
    for name, fn in phases.items():
        timed(fn, R, R)
        phase_us[name] = timed(fn, max(R, args.steps // 4), R) / max(R, args.steps // 4) * 1e6

    list_len = steps[0].list_len.cpu().numpy()
    ab = algorithmic_bytes(w, list_len, inp.head_kind)
    tbs = ab["total"] / step_s / 1e12

    # dominant kernel: the page scorer (reads the page meta of every dynamic row once; also the
    # block-table row, the group queries of the dynamic heads, and writes one fp32 score per page)
    dyn_rows = int((inp.head_kind == 0).sum())
    score_bytes = ab["meta"] + int(w.n_pages.sum()) * 4 + w.batch * dyn_rows * 4 * w.head_dim * 2 + \
        int(w.n_pages.sum()) * dyn_rows * 4
    dom_us = phase_us.get("score", phase_us["select"])
    achieved = score_bytes / (dom_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as f:
            pmc = json.load(f)
        if pmc.get("kernel_hash") == kernel_hash() and pmc.get("workload") == WORKLOAD:
            traffic = pmc.get("page_score_bytes_per_launch")
    roofline = {"bound": "hbm", "kernel": "page_score_topk_kernel", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_TBS * 1000, "unit": "GB/s", "frac": round(achieved / (PEAK_HBM_TBS * 1000), 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": score_bytes,
                "avg_launch_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu:
        cb = cpu_baseline(w, inp, args.cpu_seconds)
        cpu = {"value": round(ab["total"] / cb["step_s"] / 1e12, 8), "unit": "TB/s", "cores": 1, "kind": "oracle",
               "sample": f"{cb['steps']} whole decode steps of {WORKLOAD} (tail meta refresh, scores, selection, "
                         f"attention; fp64 numpy, 1 thread) in {cb['seconds']:.1f} s",
               "step_ms": round(cb["step_s"] * 1e3, 2)}

    sel_us = phase_us["select"]
    score_us = phase_us.get("score", 0.0)
    line = {
        "metric": METRIC, "value": round(tbs, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": w.batch, "context": int(w.seq_lens[0]),
                   "heads": f"Hq{w.num_q_heads}/Hkv{w.num_kv_heads}", "head_dim": w.head_dim, "page": 16,
                   "kv_dtype": w.kv_dtype, "budget_pages": w.budget_pages, "streaming_kv_heads": 4,
                   "layers_rotated": R, "graph": True},
        "step_us": round(step_s * 1e6, 3), "tokens_per_s": round(w.batch / step_s, 1),
        "bytes_per_step": ab, "frac_of_peak": round(tbs / PEAK_HBM_TBS, 4),
        "phase_us": {k: round(v, 3) for k, v in phase_us.items()},
        "selection_overhead": {"literal_score_plus_select": round((score_us + sel_us) / (step_s * 1e6), 4),
                               "operative_select_only": round(sel_us / (step_s * 1e6), 4)},
        "roofline": roofline, "cpu_baseline": cpu,
        "setup_s": round(gen_s, 1), "kernel_hash": kernel_hash(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
