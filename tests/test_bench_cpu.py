"""Host-side checks of bench.py (CPU only): its refusal of more than one GPU and its byte accounting.

The accounting gives the algorithmic bytes behind the bench line's achieved bandwidth and roofline;
here it is compared with a page-by-page enumeration of what each access of the step moves.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_paged_decode_quest_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _enumerated_scorer_bytes(w, head_kind, skip_last_meta):
    d = w.head_dim
    meta_row = 2 * d * (4 if w.kv_dtype == "f32" else 2)
    total = 0
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            if head_kind[h]:
                continue  # streaming heads are not scored
            total += w.group * d * (4 if w.q_dtype == "f32" else 2)  # the group's queries
            n = int(w.n_pages[b])
            for p in range(n):
                total += 4 + 4  # block-table entry read, score written
                if not (skip_last_meta and p == n - 1):
                    total += meta_row
    return total


@pytest.mark.parametrize("kv", ["f16", "f32", "fp8"])
@pytest.mark.parametrize("tail,skip", [("select", True), ("side", True), ("none", False), ("serial", False)])
def test_scorer_bytes_by_enumeration(kv, tail, skip):
    w = W.small("acct", kv=kv, q="f32" if kv == "f32" else "f16", d=64 if kv == "f32" else 128,
                seq_lens=(700, 37, 2050, 1, 16, 17), Hkv=4, Hq=16, streaming=(1, 2))
    head_kind = np.array([0, 1, 1, 0])
    assert bench.scorer_bytes(w, head_kind, tail) == _enumerated_scorer_bytes(w, head_kind, skip)


def test_headline_scorer_bytes():
    # 131072 tokens in 8192 pages, KV heads 4-7 dynamic: 4 x 8192 (entry + score), 4 x 8191 fp16 meta rows
    # of 2 x 128 channels, and 4 groups of 4 fp16 queries
    w = W.named("llama3_8b_b1_128k_f16")
    head_kind = np.array([1, 1, 1, 1, 0, 0, 0, 0])
    assert bench.scorer_bytes(w, head_kind, "select") == 4 * 8192 * 8 + 4 * 8191 * 512 + 4 * 4 * 128 * 2
    assert bench.scorer_bytes(w, head_kind, "select") == _enumerated_scorer_bytes(w, head_kind, True)


def test_step_bytes_by_enumeration():
    w = W.small("acct", seq_lens=(700, 37, 2050, 1, 16, 17), Hkv=4, Hq=16, streaming=(1, 2))
    head_kind = np.array([0, 1, 1, 0])
    rng = np.random.default_rng(5)
    list_len = np.array([[int(rng.integers(0, int(n) + 1)) for _ in range(4)] for n in w.n_pages])
    d = w.head_dim
    page_kv = 2 * 16 * d * 2
    meta = tail = 0
    for b in range(w.batch):
        n = int(w.n_pages[b])
        for h in range(4):
            if head_kind[h] or n == 0:
                continue
            meta += (n - 1) * 2 * d * 2  # every stored box but the newest page's
            tail += 16 * d * 2 + 2 * d * 2  # the newest page's keys read, its box written
    kv = sum(int(list_len[b, h]) * page_kv for b in range(w.batch) for h in range(4))
    q = w.batch * w.num_q_heads * d * 2
    o = w.batch * w.num_q_heads * (d + 1) * 4
    tables = int(w.n_pages.sum()) * 4 + w.batch * 4
    got = bench.algorithmic_bytes(w, list_len, head_kind)
    assert (got["meta"], got["tail"], got["kv"], got["q"], got["o"], got["tables"]) == (meta, tail, kv, q, o, tables)
    assert got["total"] == meta + tail + kv + q + o + tables
