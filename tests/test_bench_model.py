"""CPU checks of the benchmark's byte and flop models.

The roofline fraction that bench.py reports is only as good as the
algorithmic byte count (decode) and flop count (prefill) it divides by.
These tests count the same quantities a different way — row by row from the
element sizes and head dimensions, or by enumerating the attention masks of
a small prefill — and tie the headline workload's byte count to the figure
the committed traffic profile was computed against.
"""

from __future__ import annotations

import json
import os
import re

import numpy as np
import pytest

import bench
from head_wise_sparse_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tiny(**kw):
    wl = W.make_workload(1, n=40, batch=2)
    wl.seq_lens = [40, 17]
    wl.Hq, wl.Hkv = 4, 2
    wl.head_kinds = ["retrieval", "local"]
    for k, v in kw.items():
        setattr(wl, k, v)
    return wl


def _count_rows(wl, sel_counts):
    """Row-by-row count: each stored element is 2 bytes (bf16) or 1 (e4m3),
    index entries 4 (f32) or 2 (bf16); fp8 gathers read one 4+4 byte K/V
    scale pair per 16 rows; queries are bf16 and outputs fp32."""
    kv_elt = 1 if wl.kv_dtype == "fp8" else 2
    idx_elt = 2 if wl.index_dtype == "bf16" else 4
    score = attend = 0
    for b, n in enumerate(wl.seq_lens):
        for h, kind in enumerate(wl.head_kinds):
            cnt = int(sel_counts[b, h])
            if kind == "retrieval":
                for _tok in range(n):
                    score += wl.d * kv_elt if wl.score_mode == "full" else wl.r * idx_elt
                for _row in range(cnt):
                    attend += wl.d * kv_elt                      # V
                    if wl.score_mode != "full":
                        attend += wl.d * kv_elt                  # K as well
                attend += 8 * -(-cnt // 16) if wl.kv_dtype == "fp8" else 0
            else:
                ring = wl.local_ring
                elt = 2 if ring else kv_elt
                for _row in range(cnt):
                    attend += 2 * wl.d * elt
                if wl.kv_dtype == "fp8" and not ring:
                    attend += 8 * -(-cnt // 16)
    io = wl.B * wl.Hq * wl.d * 2 + wl.B * wl.Hq * wl.d * 4
    return score, attend, io


@pytest.mark.parametrize("score_mode", ["index", "full"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("index_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ring", [False, True])
def test_algorithmic_bytes_row_count(score_mode, kv_dtype, index_dtype, ring):
    wl = _tiny(score_mode=score_mode, kv_dtype=kv_dtype, index_dtype=index_dtype, local_ring=ring)
    sel = np.array([[7, 33], [17, 9]], dtype=np.int64)
    by = bench.algorithmic_bytes(wl, sel)
    score, attend, io = _count_rows(wl, sel)
    assert (by["score"], by["attend"], by["io"]) == (score, attend, io)
    assert by["total"] == score + attend + io


def test_algorithmic_bytes_ring_reads_bf16_rows():
    """With a local ring the local heads' rows are bf16 even over an fp8 cache;
    retrieval heads still read e4m3 rows."""
    sel = np.array([[0, 20], [0, 20]], dtype=np.int64)
    ring = bench.algorithmic_bytes(_tiny(kv_dtype="fp8", local_ring=True), sel)
    paged = bench.algorithmic_bytes(_tiny(kv_dtype="fp8", local_ring=False), sel)
    assert ring["attend"] == 2 * 20 * 2 * 128 * 2                 # 2 seqs x 20 rows x (K,V) x 128 x 2 B
    assert paged["attend"] == 2 * (20 * 2 * 128 + 8 * 2)          # e4m3 rows + two pages of scales


def test_headline_bytes_match_traffic_profile():
    """128K oracle top-k: all K rows of every head once, V of the k kept rows,
    q and out.  The committed counter summary divides by the same figure."""
    wl = W.make_workload(3)
    k = int(wl.top_k[0])
    assert k == 2621
    sel = np.full((wl.B, wl.Hkv), k, dtype=np.int64)
    by = bench.algorithmic_bytes(wl, sel)
    assert by["score"] == 4 * 8 * 131072 * 256
    assert by["attend"] == 4 * 8 * k * 256
    assert by["io"] == 4 * 32 * 128 * 6
    assert bench.stage_bytes("fused", by) == by["total"] == 1095311360
    path = os.path.join(ROOT, "profiles", "fused_g4_kernel_oracle_topk_128k_traffic.md")
    rec = json.loads(re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), re.S).group(1))
    assert rec["algorithmic_bytes_per_launch"] == by["total"]


def _mask_count(n_tok, n_sink, window, causal_only):
    """Attended (query, key) pairs of a prefill of positions 0..n_tok-1, by
    enumerating each query's keys."""
    total = 0
    for i in range(n_tok):
        j = np.arange(i + 1)
        keep = np.ones_like(j, bool) if causal_only else (j < n_sink) | (j > i - window)
        total += int(keep.sum())
    return total


@pytest.mark.parametrize("n_tok", [1, 5, 63, 300, 1500])
@pytest.mark.parametrize("dense", [False, True])
def test_prefill_flops_mask_count(n_tok, dense):
    wl = W.make_workload(2, n=64, batch=1)
    wl.window = 256
    n_ret = wl.head_kinds.count("retrieval")
    n_loc = wl.head_kinds.count("local")
    causal = _mask_count(n_tok, wl.n_sink, wl.window, True)
    local = causal if dense else _mask_count(n_tok, wl.n_sink, wl.window, False)
    want = 4 * wl.d * wl.G * (n_ret * causal + n_loc * local)
    assert bench.prefill_flops(wl, n_tok, dense) == want


def test_prefill_flops_closed_form_32k():
    """Llama-3-8B layer shape, 32768 positions: causal pairs n(n+1)/2 for the
    retrieval heads; for the local heads L(L+1)/2 + (n-L)L with L = sinks + window."""
    wl = W.make_workload(2)
    n, L = 32768, wl.n_sink + wl.window
    causal = n * (n + 1) // 2
    local = L * (L + 1) // 2 + (n - L) * L
    G, d = wl.G, wl.d
    assert bench.prefill_flops(wl, n, dense=True) == 4 * d * G * 8 * causal
    assert bench.prefill_flops(wl, n, dense=False) == 4 * d * G * (2 * causal + 6 * local)


def test_stage_kernel_names():
    assert bench.stage_kernel("score", W.make_workload(3)) == "score_full_g4_kernel"
    assert bench.stage_kernel("score", W.make_workload(2, n=64, batch=1)) == "score_index_kernel"
    assert bench.stage_kernel("score", W.make_workload(3, rope_theta=5e5)) == "score_full_kernel"
    assert bench.stage_kernel("fused", None) == "fused_g4_kernel"
    assert bench.stage_kernel("tail", None) == "tail_kernel"
    by = {"score": 5, "attend": 7, "io": 11, "total": 23}
    assert bench.stage_bytes("tail", by) == 18
    assert bench.stage_bytes("score", by) == 5


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_record_needs_matching_source_hash(tmp_path, monkeypatch):
    """bench.py reports HBM traffic only from a counter summary taken on the
    current kernel sources."""
    rec = {"kernel": "k", "workload": "w", "traffic_bytes_per_launch": 123,
           "source_sha256": bench.kernel_source_sha("fused")}
    path = tmp_path / "k_w_traffic.md"
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    path.write_text("# summary\n\n```json\n" + json.dumps(rec) + "\n```\n")
    assert bench._read_traffic("fused", "k", "w") == 123
    rec["source_sha256"] = "0" * 64
    path.write_text("```json\n" + json.dumps(rec) + "\n```\n")
    assert bench._read_traffic("fused", "k", "w") is None
    assert bench._read_traffic("fused", "k", "missing") is None
    # the fused and tail stages hash the same kernel file, the score stage another
    assert bench.kernel_source_sha("fused") == bench.kernel_source_sha("tail")
    assert bench.kernel_source_sha("score") != bench.kernel_source_sha("fused")
