"""Benchmark of one sparse paged decode step on one MI355X.

Default workload: the Llama-3-8B-shaped attention layer at 128k context (batch 1, Hq 32 /
Hkv 8, d 128, 16-token fp16 pages; KV heads 0-3 streaming with 4 sink + 16 local pages, heads
4-7 top-K 256 pages with 1 sink + 2 local pages forced; 64 planted pages per head).

A step is the whole hot path, captured in a hipGraph: page scores -> page selection (or both in
one launch with --fused), with the key statistics of the page each request's newest token is in
rebuilt on the way (top-K: by the selector beside the selection; coverage: before scoring) ->
split-K decode attention -> log-sum-exp merge.
To measure HBM rather than the 256 MB Infinity Cache, the bench keeps R independent copies
("layers") of every input and output and rotates through them, so one rotation touches
well over 1 GB.

Prints one JSON line: value = achieved HBM TB/s on the algorithmic bytes of a step (page meta
scanned + the selected K/V pages + Q + O + block table + the tail page), ms_per_step = step
time.  The roofline object is for the kernel that moves the most bytes (the page scorer),
timed alone with HIP events on the stream its graph replays on.  step_us_spread gives the
per-step time of single replays of the rotation graph, and beta_copy_TBs a plain device copy's
bandwidth on the same GPU (read + write bytes), the practical streaming ceiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse paged decode step us + achieved HBM TB/s (128k ctx, Hq32/Hkv8/d128)"
DEFAULT_WORKLOAD = "llama3_8b_b1_128k_f16"
PEAK_HBM_TBS = 8.0
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = ["score_common.h", "page_score.hip", "spd_device.h", "spd_launch.h"]  # what page_score_kernel is built from
MVAR_SOURCES = KERNEL_SOURCES + ["page_score_mvar.hip", "meta_build.h"]  # page_score_mvar_kernel
DECODE_SOURCES = ["sparse_paged_decode.hip", "spd_device.h", "spd_launch.h"]  # sparse_paged_decode_kernel
HELD_OUT = (100, 101, 102, 103, 104)  # timing seeds beside the calibration seed (offsets from each workload's seed)


def kernel_hash(files=KERNEL_SOURCES) -> str:
    """Hash of the scorer sources (stored counter figures are void once they change)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_paged_decode_quest_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, list_len: np.ndarray, head_kind: np.ndarray) -> dict:
    """Minimal bytes one step must move (meta scanned, selected K/V pages, Q, O, tables, tail page)."""
    d = w.head_dim
    kv_bytes = {"f32": 4, "f16": 2, "fp8": 1}[w.kv_dtype]
    meta_bytes = 4 if w.kv_dtype == "f32" else 2
    n_pages = w.n_pages  # physical pages (block-table slots)
    dyn_heads = int((head_kind == 0).sum())
    # one key box per 16-token logical page, except the newest one of each request: its statistics are
    # rebuilt from its keys (the tail term), so its stored box need not be read
    rebuilt_rows = int((w.n_logical > 0).sum()) * dyn_heads
    meta = (int(w.n_logical.sum()) * dyn_heads - rebuilt_rows) * 2 * d * meta_bytes
    key_page = 16 * d * kv_bytes + (32 if w.kv_dtype == "fp8" else 0)
    tail = rebuilt_rows * (key_page + 2 * d * meta_bytes)
    if w.estimator == "mvar":  # bf16 summaries; the first and current pages read as keys, one summary written
        meta = int(np.maximum(n_pages - 2, 0).sum()) * dyn_heads * 2 * d * 2
        tail = dyn_heads * int(np.minimum(n_pages, 2).sum()) * key_page + w.batch * dyn_heads * 2 * d * 2
    P = w.page_size  # a listed page is read whole: K and V (+ their fp16 scales) of P tokens
    page_kv = P * d * kv_bytes * 2 + (P * 2 * 2 if w.kv_dtype == "fp8" else 0)
    kv = int(list_len.sum()) * page_kv
    q = w.batch * w.num_q_heads * d * (4 if w.q_dtype == "f32" else 2)
    o = w.batch * w.num_q_heads * (d + 1) * 4
    tables = int(n_pages.sum()) * 4 + w.batch * 4
    total = meta + kv + q + o + tables + tail
    return {"meta": meta, "kv": kv, "q": q, "o": o, "tables": tables, "tail": tail, "total": total}


def scorer_bytes(w, head_kind: np.ndarray, tail: str) -> int:
    """Algorithmic bytes of one scorer launch (or fused score + select launch): the meta rows
    and block-table entries of the dynamic rows' scanned pages, the group queries, the scores
    written, and -- when the scorer rebuilds the last page -- that page's keys (the list
    write-back of a fused launch is small).  A skipping scorer ("side") leaves out the last
    page; a rebuilding one ("rebuild") reads its keys instead of its meta."""
    d = w.head_dim
    meta_bytes = 4 if w.kv_dtype == "f32" else 2
    kv_bytes = {"f32": 4, "f16": 2, "fp8": 1}[w.kv_dtype]
    dyn_heads = int((head_kind == 0).sum())
    q = w.batch * dyn_heads * w.group * d * (4 if w.q_dtype == "f32" else 2)
    if w.estimator == "mvar":
        # summaries + block-table entries + G log-masses of the estimated pages; keys of the first and
        # current pages and their log-masses; the rebuilt summary of the current page
        est = int(np.maximum(w.n_pages - 2, 0).sum()) * dyn_heads
        exact = int(np.minimum(w.n_pages, 2).sum()) * dyn_heads
        key_page = 16 * d * kv_bytes + (32 if w.kv_dtype == "fp8" else 0)
        rebuilt = int((w.n_pages > 0).sum()) * dyn_heads * 2 * d * 2 if tail == "rebuild" else 0
        return est * (2 * d * 2 + 4 + 4 * w.group) + exact * (key_page + 4 * w.group) + q + rebuilt
    if w.page_size != 16:
        # hierarchical paging: the key boxes of the scanned logical pages (the skipping scorer leaves out
        # the last physical page), one block-table entry and one score per physical page
        g = w.page_size // 16
        skip = 1 if tail in ("side", "select") else 0
        logical = sum(min(int(nl), g * max(int(npg) - skip, 0)) for nl, npg in zip(w.n_logical, w.n_pages))
        return dyn_heads * (logical * 2 * d * meta_bytes + int(w.n_pages.sum()) * 8) + q
    # every scanned (page, dynamic head) pair reads its block-table entry and writes its score; the meta
    # row of each row's last page is not read when the scorer skips that page or rebuilds it from its keys
    rows = int((w.n_pages > 0).sum()) * dyn_heads
    pairs = int(w.n_pages.sum()) * dyn_heads
    meta_rows = pairs - (rows if tail in ("side", "select", "rebuild") else 0)
    rebuilt = rows * (16 * d * kv_bytes + (32 if w.kv_dtype == "fp8" else 0) + 2 * d * meta_bytes) \
        if tail == "rebuild" else 0
    return pairs * (4 + 4) + meta_rows * 2 * d * meta_bytes + q + rebuilt


def copy_bandwidth(stream, mib: int = 1024, reps: int = 10) -> float:
    """Measured streaming bandwidth of this GPU (TB/s, read + write bytes): a plain device copy."""
    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return 2 * (mib << 20) / sec / 1e12


def _oracle_steps(w, inp, seconds: float) -> dict:
    """Whole decode steps of the fp64 oracle (untuned), one thread, for about `seconds`."""
    from threadpoolctl import threadpool_limits

    from oracle import spd_oracle as O

    mvar = w.estimator == "mvar"
    hier = w.page_size != 16
    with threadpool_limits(limits=1):
        # setup (the GPU builds the page summaries once before timing too)
        meta = O.page_stats_build(inp) if mvar else O.hier_meta_build(inp) if hier else O.page_meta_build(inp)
        first = [max(O.n_pages(L) - 1, 0) for L in inp.seq_lens]  # the newest token's (logical) page
        steps, t0 = 0, time.perf_counter()
        while True:
            if mvar:
                sel = O.page_select(inp, None, O.page_stats_build(inp, first_page=first, stats=meta))
            elif hier:
                sel = O.hier_page_select(inp, O.hier_meta_build(inp, meta=meta, first_page=first))
            else:
                sel = O.page_select(inp, O.page_meta_build(inp, meta=meta, first_page=first))
            if hier:
                O.hier_sparse_paged_decode(inp, sel["lists"], w.sm_scale)
            else:
                O.sparse_paged_decode(inp, sel["lists"], w.sm_scale)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"steps": steps, "seconds": el, "step_s": el / steps}


def cpu_baseline(w, inp, seconds: float) -> dict:
    """The fp64 oracle on the host: whole decode steps of this workload on one thread."""
    return _oracle_steps(w, inp, seconds)


_ARRAYS = ("q", "k_pool", "v_pool", "k_scale", "v_scale", "block_table", "seq_lens", "head_kind")


def _oracle_worker(job):
    """A host process running whole oracle steps over inputs held in shared memory (it imports no GPU code)."""
    from multiprocessing import shared_memory

    from sparse_paged_decode_quest_amd import workloads as W

    w, specs, seconds = job
    shms, arrs = [], {}
    for name, spec in specs.items():
        if spec is None:
            arrs[name] = None
            continue
        shm_name, shape, dtype = spec
        shm = shared_memory.SharedMemory(name=shm_name)
        shms.append(shm)
        arrs[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)
    try:
        inp = W.Inputs(workload=w, **arrs)
        return _oracle_steps(w, inp, seconds)
    finally:
        for shm in shms:
            shm.close()


def host_cpu() -> dict:
    """The host's CPU model and the cores this process may use (read at run time)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return {"model": model, "cores_available": cores}


def cpu_baseline_parallel(w, inp, seconds: float, procs: int) -> dict:
    """The same oracle steps in `procs` host processes at once (one thread each), over shared copies of the
    inputs: the host's whole-step throughput with that many cores."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    shms, specs = [], {}
    try:
        for name in _ARRAYS:
            a = getattr(inp, name)
            if a is None:
                specs[name] = None
                continue
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            shms.append(shm)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            specs[name] = (shm.name, a.shape, a.dtype.str)
        from concurrent.futures import ProcessPoolExecutor

        # a worker that cannot start raises here (BrokenProcessPool) instead of being respawned, and the
        # wait is bounded
        with ProcessPoolExecutor(max_workers=procs, mp_context=mp.get_context("spawn")) as ex:
            futs = [ex.submit(_oracle_worker, (w, specs, seconds)) for _ in range(procs)]
            res = [f.result(timeout=4 * seconds + 300) for f in futs]
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    steps = sum(r["steps"] for r in res)
    el = max(r["seconds"] for r in res)
    return {"steps": steps, "seconds": el, "step_s": el / steps, "procs": procs}


def traffic_record(w_name: str, kernel: str, sources) -> dict | None:
    """The committed counter record of `kernel` on workload `w_name`, if its sources still hash to the value
    the counters were taken at."""
    if not os.path.exists(PMC_FILE):
        return None
    with open(PMC_FILE) as f:
        pmc = json.load(f)
    h = kernel_hash(sources)
    for rec in pmc.get("records", []):
        if rec["workload"] == w_name and rec["kernel"] == kernel and rec["kernel_hash"] == h:
            return rec
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=0, help="independent input copies rotated per step (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="host processes of the all-cores CPU baseline (capped at the cores this process may use)")
    ap.add_argument("--held-out-steps", type=int, default=420,
                    help="timed steps on each held-out seed (0: skip)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--fused", action="store_true", help="scorer and selector in one launch")
    ap.add_argument("--merged", action="store_true", help="decode and merge in one launch (last-block merge)")
    ap.add_argument("--no-gate", action="store_true", help="top-K selection without the LiteTopK gate")
    ap.add_argument("--tail", default="auto", choices=("auto", "none", "select", "side", "serial", "rebuild"),
                    help="how the newest page's key statistics are rebuilt (DecodeStep's tail)")
    ap.add_argument("--plan", default=None,
                    help="self-planning constants C,N_J,N_T[,balanced] (default: the step's for the workload)")
    ap.add_argument("--phase-only", default=None,
                    help="time only one phase per step (select|decode|merge|score|select_only)")
    ap.add_argument("--reuse", type=int, default=4,
                    help="also time chunks of this many steps that reuse one page selection (1: off)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--gate-drift", default=None,
                    help="only measure LiteTopK's gate under drifting queries, for these comma-separated noise "
                         "levels (one JSON line each)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the decode step is a single-GPU "
                                   "kernel pipeline with no collectives; more GPUs would each run it on their own "
                                   "requests or KV heads"}))
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

    from sparse_paged_decode_quest_amd import step as S
    from sparse_paged_decode_quest_amd import workloads as W

    w = W.named(args.workload)
    t_gen = time.perf_counter()
    inp = W.generate(w)
    base = S.upload(inp)
    S.build_meta(w, base)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    if args.gate_drift:
        return gate_drift(args, w, inp, base)
    plan = None
    if args.plan:
        v = [int(x) for x in args.plan.split(",")]
        plan = S.Plan(*v[:3], balanced=bool(v[3]) if len(v) > 3 else False)
    if w.num_queries > 1:
        return bench_mq(args, w, inp, base, plan, gen_s)
    gated = False if args.no_gate else None
    probe = S.DecodeStep(w, base, plan=plan, fused=args.fused, merged=args.merged, gated=gated,
                             tail=args.tail)
    probe.run()
    torch.cuda.synchronize()
    ab0 = algorithmic_bytes(w, probe.list_len.cpu().numpy(), inp.head_kind)
    layer_bytes = sum(t.numel() * t.element_size() for t in (base.k_pool, base.v_pool, base.page_meta))
    R = args.layers or int(min(64, max(4, math.ceil((1 << 30) / ab0["total"]))))
    R = max(1, min(R, int(100e9 // max(layer_bytes, 1))))

    def clone(t):
        return None if t is None else t.clone()

    layers = [base] + [S.DeviceInputs(q=clone(base.q), k_pool=clone(base.k_pool), v_pool=clone(base.v_pool),
                                      k_scale=clone(base.k_scale), v_scale=clone(base.v_scale),
                                      block_table=clone(base.block_table), seq_lens=clone(base.seq_lens),
                                      head_kind=base.head_kind.copy(), page_meta=clone(base.page_meta))
                       for _ in range(R - 1)]
    steps = [probe] + [S.DecodeStep(w, d, plan=plan, fused=args.fused, merged=args.merged, gated=gated,
                             tail=args.tail)
                       for d in layers[1:]]
    for st in steps:
        st.run()
    torch.cuda.synchronize()
    ref_lists = steps[0].lists()
    for st in (steps[1 % R], steps[-1]):
        assert st.lists() == ref_lists and torch.equal(st.out, steps[0].out), "layer copies disagree"

    phases = ({"decode_merged": lambda st, s: st.attend(s)} if args.merged else
              {"decode": lambda st, s: st.decode(s), "merge": lambda st, s: st.merge(s)})
    if probe.tail in ("side", "serial"):
        phases["tail"] = lambda st, s: st.refresh_tail(s)
    if not args.fused:
        phases.update({"score": lambda st, s: st.score(s),
                       "select_only": lambda st, s: st.select_only(s)})
    else:
        phases["select"] = lambda st, s: st.score_select(s)
        # reference for the selection overhead: the standalone scorer over the same meta
        ref_steps = [S.DecodeStep(w, d, fused=False) for d in layers]
        phases["score"] = lambda st, s, _r={id(a): b for a, b in zip(steps, ref_steps)}: _r[id(st)].score(s)

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
        """Run `total` calls of fn (rotating layers) as graphs; returns seconds (HIP events on `stream`)."""
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
        print(json.dumps({"phase": args.phase_only, "workload": w.name, "us_per_launch": sec / args.steps * 1e6}))
        return

    timed(whole, max(args.warmup, 1), R)              # warm-up: W untimed steps
    torch.cuda.synchronize()
    step_s = timed(whole, args.steps, R) / args.steps  # exactly K timed steps

    # spread: the R-step graph replayed on its own, one pair of events per replay
    g_all = capture(whole, R)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(20, args.steps // R))]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for e0, e1 in evs:
            e0.record(stream)
            g_all.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    per_step = np.array([e0.elapsed_time(e1) * 1e3 / R for e0, e1 in evs])
    spread = {"p10": round(float(np.percentile(per_step, 10)), 3), "p50": round(float(np.median(per_step)), 3),
              "p90": round(float(np.percentile(per_step, 90)), 3), "replays": len(evs), "steps_per_replay": R}
    beta = copy_bandwidth(stream)

    # Reusable page selection (LServe, "Reusable Page Selection"), top-K only: chunks of C steps, the
    # first selecting, the others one token longer each and reusing its lists.  The lengths are
    # rewound by C - 1 tokens first (the pools hold those keys), advanced inside the chunk and
    # restored at its end, so every replay is the same chunk.
    reuse = None
    if w.mode == "topk" and not args.fused and args.reuse > 1:
        C = args.reuse
        rsteps = [S.DecodeStep(w, d, plan=plan, reuse=C, merged=args.merged) for d in layers]
        for d in layers:
            d.seq_lens.sub_(C - 1)
        torch.cuda.synchronize()

        def chunk(st, s_, _r={id(a): b for a, b in zip(steps, rsteps)}):
            r = _r[id(st)]
            r.run(s_)
            for _ in range(C - 1):
                r.d.seq_lens.add_(1)
                r.reuse_step(s_)
            r.d.seq_lens.sub_(C - 1)

        timed(chunk, R, R)
        reps = max(R, args.steps // C)
        chunk_s = timed(chunk, reps, R) / reps
        for d in layers:
            d.seq_lens.add_(C - 1)
        torch.cuda.synchronize()
        reuse = {"C": C, "us_per_token": round(chunk_s / C * 1e6, 3), "chunk_us": round(chunk_s * 1e6, 3)}
    phase_us = {}
    for name, fn in phases.items():                   # each phase alone, rotated over the same layers
        reps = max(R, args.steps // 4)
        timed(fn, R, R)
        phase_us[name] = timed(fn, reps, R) / reps * 1e6

    # LiteTopK's predicted gate (top-K with the bound estimator): how the last timed selection ran, and the
    # same step and selection with the gate off.  Each layer repeats its own query, so every gate is the
    # one its previous call predicted for the same scores: the served share is the best case, and a step
    # whose gates all miss costs about the ungated step plus one count over the loaded keys.
    gate = None
    if probe.gated:
        rows = w.batch * w.num_kv_heads
        gp = S.gate_paths(probe.topk_state, rows)
        dyn = [b * w.num_kv_heads + h for b in range(w.batch) for h in range(w.num_kv_heads) if not inp.head_kind[h]]
        ung = {id(a): S.DecodeStep(w, d, plan=plan, merged=args.merged, gated=False) for a, d in zip(steps, layers)}
        for st in ung.values():
            st.run()
        reps = max(R, args.steps // 4)
        ug = {}
        for name, fn in (("step_us", lambda st, s: ung[id(st)].run(s)),
                         ("select_only_us", lambda st, s: ung[id(st)].select_only(s))):
            timed(fn, R, R)
            ug[name] = round(timed(fn, reps, R) / reps * 1e6, 3)
        served = gp[dyn, 0]
        gate = {"rows_from_candidates": int(served.sum()), "dynamic_rows": len(dyn),
                "candidates_median": int(np.median(gp[dyn, 1][served == 1])) if served.any() else None,
                "ungated": ug, "query": "repeated per layer (the gate predicted from the same scores)"}
        del ung
        torch.cuda.synchronize()

    list_len = steps[0].list_len.cpu().numpy()
    ab = algorithmic_bytes(w, list_len, inp.head_kind)
    tbs = ab["total"] / step_s / 1e12

    # Held-out seeds: the same workload drawn from the timing seeds (the calibration seed above chose the
    # plan constants), each with its own rotated layer copies; step time and achieved bandwidth per seed.
    held = None
    if args.held_out_steps > 0:
        per_seed = {}
        for off in HELD_OUT:
            ws = W.named(w.name, seed_offset=off)
            inp_s = W.generate(ws)
            d0 = S.upload(inp_s)
            S.build_meta(ws, d0)
            ds = [d0] + [S.DeviceInputs(q=clone(d0.q), k_pool=clone(d0.k_pool), v_pool=clone(d0.v_pool),
                                        k_scale=clone(d0.k_scale), v_scale=clone(d0.v_scale),
                                        block_table=clone(d0.block_table), seq_lens=clone(d0.seq_lens),
                                        head_kind=d0.head_kind.copy(), page_meta=clone(d0.page_meta))
                         for _ in range(R - 1)]
            st_s = [S.DecodeStep(ws, d, plan=plan, fused=args.fused, merged=args.merged, gated=gated,
                             tail=args.tail) for d in ds]
            saved = steps[:]
            steps[:] = st_s  # `timed` replays the layers in `steps`
            timed(whole, R, R)
            sec = timed(whole, args.held_out_steps, R) / args.held_out_steps
            ab_s = algorithmic_bytes(ws, st_s[0].list_len.cpu().numpy(), inp_s.head_kind)
            steps[:] = saved
            per_seed[str(ws.seed)] = {"step_us": round(sec * 1e6, 3), "TBs": round(ab_s["total"] / sec / 1e12, 4)}
            del ds, st_s, d0, inp_s
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        us = [v["step_us"] for v in per_seed.values()]
        held = {"seeds": per_seed, "median_step_us": round(float(np.median(us)), 3),
                "steps_each": args.held_out_steps, "calibration_seed": w.seed}

    dom_name = "select" if args.fused else "score"
    mvar = w.estimator == "mvar"
    dom_kernel = "page_score_select_kernel" if args.fused else "page_score_mvar_kernel" if mvar else "page_score_kernel"
    dom_hash = kernel_hash(MVAR_SOURCES if mvar else KERNEL_SOURCES)
    dom_bytes = scorer_bytes(w, inp.head_kind, probe.tail)
    dom_us = phase_us[dom_name]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    rec = traffic_record(w.name, dom_kernel, MVAR_SOURCES if mvar else KERNEL_SOURCES)
    traffic = rec["hbm_bytes_per_launch"] if rec else None
    dec_rec = traffic_record(w.name, "sparse_paged_decode_kernel", DECODE_SOURCES)
    roofline = {"bound": "hbm", "kernel": dom_kernel, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_TBS * 1000, "unit": "GB/s", "frac": round(achieved / (PEAK_HBM_TBS * 1000), 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3),
                "frac_of_beta_copy": round(achieved / (beta * 1000), 4)}

    cpu = cpu_all = None
    if not args.no_cpu:
        host = host_cpu()
        cb = cpu_baseline(w, inp, args.cpu_seconds)
        cpu = {"value": round(ab["total"] / cb["step_s"] / 1e12, 8), "unit": "TB/s", "cores": 1, "kind": "oracle",
               "sample": f"{cb['steps']} whole decode steps of {w.name} (tail meta refresh, scores, selection, "
                         f"attention; fp64 numpy, 1 thread) in {cb['seconds']:.1f} s",
               "step_ms": round(cb["step_s"] * 1e3, 2), "cpu_model": host["model"]}
        procs = max(1, min(args.cpu_procs, host["cores_available"]))
        if procs > 1:
            cp = cpu_baseline_parallel(w, inp, args.cpu_seconds, procs)
            cpu_all = {"value": round(ab["total"] / cp["step_s"] / 1e12, 8), "unit": "TB/s", "cores": procs,
                       "kind": "oracle",
                       "sample": f"{cp['steps']} whole decode steps of {w.name} in {procs} host processes at once "
                                 f"(one thread each, inputs shared) in {cp['seconds']:.1f} s",
                       "step_ms": round(cp["step_s"] * 1e3, 3), "cpu_model": host["model"],
                       "cores_available": host["cores_available"]}

    step_us = step_s * 1e6
    if not args.fused:
        sel_over = {"literal_score_plus_select": round((phase_us["score"] + phase_us["select_only"]) / step_us, 4),
                    "operative_select_only": round(phase_us["select_only"] / step_us, 4)}
    else:
        sel_over = {"literal_score_plus_select": round(phase_us["select"] / step_us, 4),
                    "operative_beyond_pure_scan": round(max(0.0, phase_us["select"] - phase_us["score"]) / step_us, 4)}
    heads = f"Hq{w.num_q_heads}/Hkv{w.num_kv_heads}"
    line = {
        "metric": METRIC, "value": round(tbs, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": int(max(w.seq_lens)), "heads": heads,
                   "head_dim": w.head_dim, "page": w.page_size, "logical_page": 16, "kv_dtype": w.kv_dtype, "mode": w.mode,
                   "estimator": w.estimator,
                   "budget_pages": w.budget_pages, "gamma": w.gamma, "streaming_kv_heads": len(w.streaming_heads),
                   "layers_rotated": R, "graph": True, "fused_select": args.fused, "merged_decode": args.merged,
                   "plan": [probe.plan.min_chunk, probe.plan.min_blocks_per_row, probe.plan.min_grid_blocks,
                            int(probe.plan.balanced)]},
        "step_us": round(step_us, 3), "step_us_spread": spread, "tokens_per_s": round(w.batch / step_s, 1),
        "bytes_per_step": ab, "frac_of_peak": round(tbs / PEAK_HBM_TBS, 4),
        "beta_copy_TBs": round(beta, 3), "frac_of_beta": round(tbs / beta, 4),
        "phase_us": {k: round(v, 3) for k, v in phase_us.items()},
        "selection_overhead": sel_over, "gate": gate, "reuse": reuse,
        "list_len": {"min": int(list_len.min()), "median": int(np.median(list_len)), "max": int(list_len.max())},
        "roofline": roofline, "cpu_baseline": cpu, "cpu_baseline_all_cores": cpu_all,
        "decode_traffic": None if dec_rec is None else {
            "hbm_bytes_per_launch": dec_rec["hbm_bytes_per_launch"], "listed_kv_bytes": dec_rec["reference_bytes"],
            "ratio": round(dec_rec["hbm_bytes_per_launch"] / dec_rec["reference_bytes"], 4)},
        "held_out_seeds": held,
        "setup_s": round(gen_s, 1), "kernel_hash": dom_hash,
    }
    print(json.dumps(line))


def gate_drift(args, w, inp, base):
    """LiteTopK's gate when consecutive queries differ.  Per layer copy, two steps read the same KV and page
    statistics with queries q_a and q_b = (q_a + eps n) / sqrt(1 + eps^2) (n fresh Gaussian noise, eps relative to
    q_a's standard deviation) and share one gate state; the calls alternate, so every gate was predicted from
    the other query's scores.  Reports the rows served from candidates after each query's call, the share of a
    row's list the two queries have in common, and the alternating step and selection times with the gate on
    and off (graph replays over the rotated layers, HIP events on the replay stream)."""
    import dataclasses

    import torch

    from sparse_paged_decode_quest_amd import step as S

    if w.num_queries > 1 or not S.DecodeStep(w, base).gated:
        print(json.dumps({"error": f"{w.name} has no LiteTopK gate (single-query top-K with the bound estimator "
                                   "on 16-token pages only)"}))
        sys.exit(2)
    R = args.layers or (12 if max(w.seq_lens) > 262144 else 24)

    def clone(t):
        return None if t is None else t.clone()

    layers = [base] + [S.DeviceInputs(q=clone(base.q), k_pool=clone(base.k_pool), v_pool=clone(base.v_pool),
                                      k_scale=clone(base.k_scale), v_scale=clone(base.v_scale),
                                      block_table=clone(base.block_table), seq_lens=clone(base.seq_lens),
                                      head_kind=base.head_kind.copy(), page_meta=clone(base.page_meta))
                       for _ in range(R - 1)]
    rows = w.batch * w.num_kv_heads
    dyn = [b * w.num_kv_heads + h for b in range(w.batch) for h in range(w.num_kv_heads) if not inp.head_kind[h]]
    stream = torch.cuda.Stream()

    def timed(fn, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(2 * R):
                fn(i, stream.cuda_stream)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(2 * R):
                fn(i, stream.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, steps // (2 * R))
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * 2 * R)

    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    for eps in [float(x) for x in args.gate_drift.split(",")]:
        pairs, upairs = [], []
        for d in layers:
            n = torch.randn(d.q.shape, generator=gen, device="cuda", dtype=torch.float32)
            qa = d.q.float()
            db = dataclasses.replace(d, q=((qa + eps * qa.std() * n) / (1 + eps * eps) ** 0.5).to(d.q.dtype))
            sa, sb = S.DecodeStep(w, d), S.DecodeStep(w, db)
            sb.topk_state = sa.topk_state  # one gate state for both queries
            sb.sel.topk_state = sa.topk_state.data_ptr()
            pairs.append((sa, sb))
            upairs.append((S.DecodeStep(w, d, gated=False), S.DecodeStep(w, db, gated=False)))
        sa, sb = pairs[0]
        served = []
        for _ in range(2):
            for st in (sa, sb):
                st.run()
                torch.cuda.synchronize()
                served.append(int(S.gate_paths(sa.topk_state, rows)[dyn, 0].sum()))
        la, lb = sa.lists(), sb.lists()
        ua, ub = upairs[0]
        ua.run()
        ub.run()
        torch.cuda.synchronize()
        assert ua.lists() == la and ub.lists() == lb, "gated lists differ from the ungated selection's"
        overlap = [len(set(la[k]) & set(lb[k])) / max(1, len(la[k])) for k in la if not inp.head_kind[k[1]]]
        pick = lambda ps, i: ps[i % R][i // R % 2]  # R calls with q_a, then R with q_b
        res = {"step_us_gated": timed(lambda i, s: pick(pairs, i).run(s), args.steps),
               "step_us_ungated": timed(lambda i, s: pick(upairs, i).run(s), args.steps),
               "select_us_gated": timed(lambda i, s: pick(pairs, i).select_only(s), args.steps),
               "select_us_ungated": timed(lambda i, s: pick(upairs, i).select_only(s), args.steps)}
        print(json.dumps({"gate_drift": w.name, "eps": eps, "dynamic_rows": len(dyn), "rows_from_candidates": served[2:],
                          "list_overlap_mean": round(float(np.mean(overlap)), 4),
                          "list_overlap_min": round(float(np.min(overlap)), 4), "layers_rotated": R,
                          **{k: round(v, 3) for k, v in res.items()}}), flush=True)
        del pairs, upairs
        torch.cuda.synchronize()


def bench_mq(args, w, inp, base, plan, gen_s):
    """Several query tokens per request (LiteDSA union): same timing protocol as the single-query
    step -- rotated layer copies, graph replays, HIP events on the replay stream."""
    import torch

    from sparse_paged_decode_quest_amd import step as S

    T = w.num_queries
    if args.tail not in ("auto", "select", "serial"):
        raise SystemExit("several query tokens: --tail must be auto, select or serial")
    probe = S.MQDecodeStep(w, base, plan=plan, gated=not args.no_gate, tail=args.tail)
    probe.run()
    torch.cuda.synchronize()
    d = w.head_dim
    dyn = int((inp.head_kind == 0).sum())
    union_len = probe.list_len.cpu().numpy()
    token_len = probe.token_len.cpu().numpy()
    # algorithmic bytes: the dynamic rows' key boxes, read once for the T tokens (one scan scores every
    # token row); the union pages' K / V, read once for the T tokens; queries, outputs, block-table rows;
    # the rebuilt last two pages (not scanned when the scorer skips them: the "select" tail)
    kvb = {"f16": 2, "fp8": 1}[w.kv_dtype]
    page_kv = 16 * d * kvb * 2 + (16 * 2 * 2 if w.kv_dtype == "fp8" else 0)  # K and V (+ fp16 scales)
    skipped = int(np.minimum(w.n_pages, 2).sum()) if probe.tail == "select" else 0
    meta = (int(w.n_pages.sum()) - skipped) * dyn * 2 * d * 2
    kv = int(union_len.sum()) * page_kv
    per_token_kv = int(token_len.sum()) * page_kv  # what T independent decodes would read
    q = w.batch * T * w.num_q_heads * d * 2
    o = w.batch * T * w.num_q_heads * (d + 1) * 4
    tables = int(w.n_pages.sum()) * 4
    tail = w.batch * w.num_kv_heads * 2 * (16 * d * kvb + (32 if w.kv_dtype == "fp8" else 0) + 2 * d * 2)
    ab = {"meta": meta, "kv": kv, "q": q, "o": o, "tables": tables, "tail": tail,
          "total": meta + kv + q + o + tables + tail}
    layer_bytes = sum(t.numel() * t.element_size() for t in (base.k_pool, base.v_pool, base.page_meta))
    R = args.layers or int(min(64, max(4, math.ceil((1 << 30) / ab["total"]))))
    R = max(1, min(R, int(100e9 // max(layer_bytes, 1))))
    def clone(t):
        return None if t is None else t.clone()

    layers = [base] + [S.DeviceInputs(q=base.q.clone(), k_pool=base.k_pool.clone(), v_pool=base.v_pool.clone(),
                                      k_scale=clone(base.k_scale), v_scale=clone(base.v_scale),
                                      block_table=base.block_table.clone(),
                                      seq_lens=base.seq_lens.clone(), head_kind=base.head_kind.copy(),
                                      page_meta=base.page_meta.clone()) for _ in range(R - 1)]
    steps = [probe] + [S.MQDecodeStep(w, x, plan=plan, gated=not args.no_gate, tail=args.tail) for x in layers[1:]]
    for st in steps:
        st.run()
    torch.cuda.synchronize()
    assert steps[-1].union_lists() == probe.union_lists() and torch.equal(steps[-1].out, probe.out)
    stream = torch.cuda.Stream()

    def timed(fn, total):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(R):
                fn(steps[i], stream.cuda_stream)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(R):
                fn(steps[i], stream.cuda_stream)
        reps = max(1, total // R)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (reps * R)

    whole = (lambda st, s: st.run(s))
    timed(whole, max(args.warmup, R))
    step_s = timed(whole, args.steps)
    phases = {"score": lambda st, s: st.score(s), "select_only": lambda st, s: st.select_only(s),
              "union": lambda st, s: st.union(s), "attend": lambda st, s: st.attend(s)}
    if probe.tail == "serial":
        phases = {"tail": lambda st, s: st.refresh_tail(s), **phases}
    phase_us = {}
    for name, fn in phases.items():
        timed(fn, R)
        phase_us[name] = timed(fn, max(R, args.steps // 4)) * 1e6
    gate = None
    if probe.gated:  # the same step with the token rows' gates off (each layer repeats its queries)
        rows = w.batch * T * w.num_kv_heads
        gp = S.gate_paths(probe.topk_state, rows)
        ung = {id(a): S.MQDecodeStep(w, x, plan=plan, gated=False, tail=args.tail) for a, x in zip(steps, layers)}
        for st in ung.values():
            st.run()
        ug = {}
        for name, fn in (("step_us", lambda st, s: ung[id(st)].run(s)),
                         ("select_only_us", lambda st, s: ung[id(st)].select_only(s))):
            timed(fn, R)
            ug[name] = round(timed(fn, max(R, args.steps // 4)) * 1e6, 3)
        gate = {"token_rows_from_candidates": int(gp[:, 0].sum()), "token_rows": rows, "ungated": ug,
                "query": "repeated per layer (the gate predicted from the same scores)"}
        del ung
        torch.cuda.synchronize()
    beta = copy_bandwidth(stream)
    cpu = None
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import spd_oracle as O

        with threadpool_limits(limits=1):
            m0 = O.page_meta_build(inp)
            last = [max(O.n_pages(L) - 2, 0) for L in inp.seq_lens]
            n, t0 = 0, time.perf_counter()
            while True:
                O.mq_decode_step(inp, O.page_meta_build(inp, meta=m0, first_page=last))
                n += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        cpu = {"value": round(ab["total"] / (el / n) / 1e12, 8), "unit": "TB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} whole steps of {w.name} ({T} query tokens: last-page statistics, each token's "
                         f"scores and selection, attention; fp64 numpy, 1 thread) in {el:.1f} s",
               "step_ms": round(el / n * 1e3, 2)}
    # the scan of the T token rows is the kernel that moves the most bytes: key boxes and block-table
    # entries of every (page, dynamic head), the queries, T scores per (page, dynamic head)
    sc_bytes = meta + int(w.n_pages.sum()) * dyn * (4 + 4 * T) + w.batch * T * dyn * w.group * d * 2
    line = {
        "metric": METRIC, "value": round(ab["total"] / step_s / 1e12, 4), "unit": "TB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "query_tokens": T, "context": int(max(w.seq_lens)),
                   "heads": f"Hq{w.num_q_heads}/Hkv{w.num_kv_heads}", "head_dim": d, "page": w.page_size,
                   "kv_dtype": w.kv_dtype, "mode": w.mode, "budget_pages": w.budget_pages,
                   "streaming_kv_heads": len(w.streaming_heads), "layers_rotated": R, "graph": True,
                   "plan": [probe.plan.min_chunk, probe.plan.min_blocks_per_row, probe.plan.min_grid_blocks, 0],
                   "tail": probe.tail},
        "step_us": round(step_s * 1e6, 3), "tokens_per_s": round(w.batch * T / step_s, 1),
        "bytes_per_step": ab, "kv_bytes_without_union": per_token_kv, "frac_of_peak": round(ab["total"] / step_s / 1e12 / PEAK_HBM_TBS, 4),
        "beta_copy_TBs": round(beta, 3), "phase_us": {k: round(v, 3) for k, v in phase_us.items()},
        "union_len": {"min": int(union_len.min()), "median": int(np.median(union_len)), "max": int(union_len.max())},
        "gate": gate,
        "roofline": {"bound": "hbm", "kernel": "mq_page_score_kernel (T token rows per scan)",
                     "achieved": round(sc_bytes / (phase_us["score"] * 1e-6) / 1e9, 1), "peak": PEAK_HBM_TBS * 1000,
                     "unit": "GB/s", "frac": round(sc_bytes / (phase_us["score"] * 1e-6) / 1e9 / (PEAK_HBM_TBS * 1000), 4),
                     "traffic": None, "algorithmic_bytes_per_launch": sc_bytes, "avg_launch_us": round(phase_us["score"], 3)},
        "cpu_baseline": cpu, "setup_s": round(gen_s, 1),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
