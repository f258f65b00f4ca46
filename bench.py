#!/usr/bin/env python3
"""Benchmark one head-wise sparse decode step on one MI355X.

Default workload: oracle top-k decode at 50x sparsity, B=4, 32 query / 8 KV
heads, head_dim 128, 131072-token context, bf16 paged KV, every head scoring
all tokens with full-dim q.k and keeping the exact top 2 % (k = 2621).  A
"step" is one ``hws_decode`` call: score, select, gather-attend, merge for
the whole batch.  Inputs (K/V pages, queries, block tables) are resident in
HBM before the timed region starts.

Prints one JSON line.  ``value`` is decode tokens/s for one attention layer
(B tokens per step).  ``roofline`` describes the kernel that moves the most
algorithmic bytes, timed with HIP events on the decode stream over the timed
region.  ``cpu_baseline`` is the float64 CPU oracle timed on this host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_GBS = 8000.0          # MI355X HBM3E peak
PROFILE_DIR = os.path.join(ROOT, "profiles")
STAGE_SOURCE = {"score": "k_score.hip", "attend": "k_attend.hip", "tail": "k_tail.hip", "fused": "k_tail.hip",
                "fused_index": "k_tail.hip", "select": "k_tail.hip", "attend_balanced": "k_attend.hip",
                "merge": "k_attend.hip"}


def stage_kernel(stage: str, wl) -> str:
    """Name of the kernel that a profiled stage times (as rocprofv3 lists it)."""
    if stage == "score":
        if wl.score_mode == "index":
            return "score_index_kernel"
        return "score_full_g4_kernel" if (wl.G == 4 and not wl.rope_theta) else "score_full_kernel"
    return {"attend": "attend_kernel", "tail": "tail_kernel", "fused": "fused_g4_kernel",
            "fused_index": "fused_index_kernel", "select": "select_single_kernel",
            "attend_balanced": "attend_balanced_kernel", "merge": "merge_kernel"}.get(stage, stage)


def stage_bytes(stage: str, by: dict) -> int:
    """Algorithmic bytes a stage moves: the fused launch moves all of them, the
    tail launch the attention's and the step's inputs/outputs."""
    if stage in ("fused", "fused_index"):
        return by["total"]
    if stage == "tail":
        return by["attend"] + by["io"]
    if stage == "attend_balanced":
        return by["attend"]
    return by.get(stage, 0)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = 128K headline)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--context", type=int, default=None,
                    help="context length of every sequence (workload 5: the longest drawn length), "
                         "keeping the workload's recipe")
    ap.add_argument("--batch", type=int, default=None, help="batch size, keeping the workload's recipe")
    ap.add_argument("--top-k", type=float, default=None,
                    help="retrieval heads keep a fixed top-k: a count, or a fraction of the context if < 1")
    ap.add_argument("--top-p", type=float, default=None,
                    help="retrieval heads keep the top-p set of this mass (every sequence)")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default=None,
                    help="KV cache storage, overriding the workload's (fp8: e4m3 with per-page scales)")
    ap.add_argument("--rope-theta", type=float, default=None,
                    help="rotate-half RoPE with this base (K stored rotated, queries rotated at N-1)")
    ap.add_argument("--cold-iters", type=int, default=100,
                    help="graph replays each preceded by an untimed 1 GiB cache flush (0 = skip)")
    ap.add_argument("--launch", choices=["auto", "single", "multi", "cooperative", "scan-select", "scan-single"],
                    default="auto",
                    help="auto: the library's default; single: one launch with (or after) the scoring "
                         "scan, grid sized to the device; cooperative: the same as a cooperative launch; "
                         "multi: a kernel per stage; scan-single: the scan, then the single launch; "
                         "scan-select: the scan, the selection as one launch, then attention and merge")
    ap.add_argument("--index", choices=["f32", "bf16"], default="f32",
                    help="storage of the r=16 index (64 or 32 bytes per token and retrieval head)")
    ap.add_argument("--scope", choices=["kv", "query"], default="kv",
                    help="one token set per KV head (kv) or per query head (query)")
    ap.add_argument("--ring", action="store_true",
                    help="local heads keep only sinks + window in a per-sequence ring (bf16 caches)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the head-wise chunked prefill (Llama-3-8B layer shape) instead of decode")
    ap.add_argument("--prefill-len", type=int, default=32768,
                    help="with --prefill: positions prefilled in one chunk from position 0")
    ap.add_argument("--prefill-fp8", action="store_true",
                    help="with --prefill: the cache in fp8 (e4m3 with per-page scales)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the decode step captured once as a HIP graph and replayed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB read + 1 GiB write elementwise kernel (counter calibration)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# byte model: only the bytes the method has to move
# ---------------------------------------------------------------------------

def algorithmic_bytes(wl, sel_counts) -> dict:
    """Required HBM bytes of one decode step, by stage.

    score : every token of every retrieval head once: the 16-dim index
            (64 B fp32 / 32 B bf16) or, with full-dim scores, the K row
            (256 B bf16 / 128 B fp8);
    attend: K and V rows of every selected token (V only with full-dim
            scores, whose logits are already known) and of the local heads'
            sinks + window (bf16 rows when a local ring holds them); fp8
            adds one 8 B K/V scale pair per 16 rows gathered (a page's
            worth: the fewest pages the rows can come from);
    io    : queries (bf16) and outputs (fp32).
    Scratch (scores, aggregates, histograms, partials) and block-table reads
    are not counted.
    """
    row = 128 if wl.kv_dtype == "fp8" else 256
    score = attend = 0
    for b, n in enumerate(wl.seq_lens):
        for h, kind in enumerate(wl.head_kinds):
            cnt = int(sel_counts[b, h])
            if kind == "retrieval":
                score += n * (row if wl.score_mode == "full" else (32 if wl.index_dtype == "bf16" else 64))
                attend += cnt * (row if wl.score_mode == "full" else 2 * row)
            elif wl.local_ring:
                attend += cnt * 2 * 256              # the ring keeps bf16 rows
                continue
            else:
                attend += cnt * 2 * row
            if wl.kv_dtype == "fp8":
                attend += 8 * ((cnt + 15) // 16)
    io = wl.B * wl.Hq * wl.d * (2 + 4)
    return {"score": score, "attend": attend, "io": io, "total": score + attend + io}


def _read_traffic(stage: str, kernel: str, workload: str):
    """HBM traffic per launch from the committed counter summary, or None if it
    is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != kernel_source_sha(stage):
        return None
    return rec.get("traffic_bytes_per_launch")


def kernel_source_sha(stage: str) -> str:
    """sha256 over the stage's kernel source and the device headers it includes."""
    csrc = os.path.join(ROOT, "head_wise_sparse_02_amd", "csrc")
    h = hashlib.sha256()
    for f in (STAGE_SOURCE[stage], "attend_rows.h", "hws_device.h", "hws_internal.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


# ---------------------------------------------------------------------------

def calibrate_copy():
    import torch
    n = 1 << 28                                  # 2^28 fp32 = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy", "read_bytes": 4 * n, "write_bytes": 4 * n,
                      "dispatches": 3}), flush=True)


def cpu_baseline(wl, setup, reps: int) -> dict:
    """Time the float64 oracle on the host for the whole decode step."""
    import numpy as np
    import oracle as O
    from head_wise_sparse_02_amd.runner import append_segments
    from threadpoolctl import threadpool_limits
    cores = host_threads()
    times = []
    with threadpool_limits(limits=cores):
        times = _time_oracle(wl, setup, reps, O, append_segments)
    t = statistics.median(times)
    return {"value": wl.B / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"whole decode step (all {wl.B} sequences x {wl.Hkv} KV heads), "
                      f"median of {len(times)} runs, {t:.2f} s per step, BLAS/OpenMP pools at {cores} threads"}


def host_threads() -> int:
    """Threads the CPU baseline uses: the cores this process may run on,
    capped by OMP_NUM_THREADS when that is set."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(aff, int(env))) if env.isdigit() else aff


def _time_oracle(wl, setup, reps, O, append_segments) -> list:
    times = []
    for _ in range(max(1, reps)):
        t0 = time.perf_counter()
        for b in range(wl.B):
            seq = setup.host[b]
            n = wl.seq_lens[b]
            O.decode_sequence_ref(
                seq.q, seq.k, seq.v, head_kinds=wl.head_kinds, proj=setup.proj_host,
                score_mode=wl.score_mode, select_mode=wl.select_mode, top_p=float(wl.top_p[b]),
                top_k=int(wl.top_k[b]), n_sink=wl.n_sink, window=wl.window,
                attn_scale=wl.attn_scale, index_scale=wl.index_scale, rope_theta=wl.rope_theta,
                kv_fp8=wl.kv_dtype == "fp8", segments=append_segments(n))
        times.append(time.perf_counter() - t0)
    return times


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA peak


def prefill_flops(wl, n_tok: int, dense: bool) -> int:
    """Algorithmic flops of one prefill of positions 0..n_tok-1: 4 * d per
    (query row, attended key) (q.k and p v), over each head's key sets."""
    n = np.arange(1, n_tok + 1, dtype=np.int64)              # keys of position i: i + 1
    loc = np.minimum(n, wl.n_sink + wl.window)               # |sinks U window| of a context of n
    per_head = {"retrieval": int(n.sum()), "local": int(loc.sum())}
    total = 0
    for kind in wl.head_kinds:
        total += wl.G * per_head["retrieval" if dense else kind]
    return 4 * wl.d * total


def prefill_main(args) -> int:
    import torch
    from head_wise_sparse_02_amd import workloads as W
    from head_wise_sparse_02_amd.runner import DecodeSetup, append_segments

    N = args.prefill_len
    wl = W.make_workload(2, n=N, batch=1, seed=args.seed)
    if args.prefill_fp8:
        wl.kv_dtype = "fp8"
    print(f"[bench] prefill: building a {N}-token cache (Llama-3-8B layer shape)", file=sys.stderr, flush=True)
    st = DecodeSetup(wl, keep_host=not args.no_cpu_baseline)
    qh = wl.prefill_queries(0, N)
    q = torch.from_numpy(qh[None]).to(torch.bfloat16).cuda()
    sp = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((1, N, wl.Hq, wl.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, N, wl.Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for dense in (False, True):
        for _ in range(args.warmup):
            st.ctx.prefill(q=q, block_tables=st.block_tables, start_pos=sp, out=out, lse=lse, dense=dense)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            st.ctx.prefill(q=q, block_tables=st.block_tables, start_pos=sp, out=out, lse=lse, dense=dense)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        st.ctx.profile_enable(True)
        st.ctx.profile_read()
        for _ in range(args.steps):
            st.ctx.prefill(q=q, block_tables=st.block_tables, start_pos=sp, out=out, lse=lse, dense=dense)
        torch.cuda.synchronize()
        kms, calls = st.ctx.profile_read()["prefill"]
        st.ctx.profile_enable(False)
        fl = prefill_flops(wl, N, dense)
        res[dense] = {"ms": ms, "kernel_us": 1000.0 * kms / calls, "flops": fl}
    hw = res[False]
    achieved = hw["flops"] / (hw["kernel_us"] * 1e-6) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        rows = np.linspace(0, N - 1, 32).astype(np.int64)          # a bounded sample of positions
        seq = st.host[0]
        t0 = time.perf_counter()
        O.prefill_sequence_ref(qh, seq.k, seq.v, head_kinds=wl.head_kinds, start=0, n_sink=wl.n_sink,
                               window=wl.window, attn_scale=wl.attn_scale, rows=rows,
                               kv_fp8=args.prefill_fp8, segments=append_segments(N))
        t = time.perf_counter() - t0
        cpu = {"value": round(rows.size / t, 2), "unit": "tokens/s", "cores": host_threads(),
               "kind": "oracle", "sample": f"{rows.size} evenly spaced positions of the {N}-token chunk, "
                                           f"all heads, {t:.2f} s"}
    line = {
        "metric": "head-wise chunked prefill tokens/s and achieved bf16 TFLOP/s, 1 GPU",
        "value": round(N / (hw["ms"] / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(hw["ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes and structure of the workload, no dataset or weights)",
        "config": {"workload": "llama3_8b_layer_prefill" + ("_fp8" if args.prefill_fp8 else ""),
                   "kv_dtype": wl.kv_dtype, "batch": 1, "q_heads": wl.Hq,
                   "kv_heads": wl.Hkv, "head_dim": wl.d, "prefill_len": N, "n_sink": wl.n_sink,
                   "window": wl.window, "head_kinds": wl.head_kinds},
        "dense_ms_per_step": round(res[True]["ms"], 4),
        "speedup_vs_dense": round(res[True]["ms"] / hw["ms"], 3),
        "dense_tflops": round(res[True]["flops"] / (res[True]["kernel_us"] * 1e-6) / 1e12, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "flops_per_launch": hw["flops"],
                     "avg_launch_us": round(hw["kernel_us"], 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def build_workload(args, W):
    """The workload ``--config`` names, with the context, batch and selection
    overrides applied; an overridden workload's name carries them."""
    if args.top_k is not None and args.top_p is not None:
        raise SystemExit("--top-k and --top-p exclude each other")
    wl = W.make_workload(args.config, seed=args.seed, n=args.context, batch=args.batch,
                         select_scope=args.scope, index_dtype=args.index, local_ring=args.ring)
    tags = []
    if args.context is not None:
        tags.append(f"n{args.context}")
    if args.batch is not None:
        tags.append(f"b{args.batch}")
    if args.top_k is not None:
        frac = args.top_k < 1.0
        wl.select_mode = "top_k"
        wl.top_k = np.array([int(args.top_k * n) if frac else int(args.top_k) for n in wl.seq_lens], np.int32)
        wl.top_p = np.ones(wl.B, np.float32)
        tags.append(f"topk{args.top_k * 100:g}pct" if frac else f"topk{int(args.top_k)}")
    if args.top_p is not None:
        wl.select_mode = "top_p"
        wl.top_p = np.full(wl.B, args.top_p, np.float32)
        wl.top_k = np.zeros(wl.B, np.int32)
        tags.append(f"topp{args.top_p:g}")
    if args.kv is not None and args.kv != wl.kv_dtype:
        wl.kv_dtype = args.kv
        tags.append(args.kv)
    if args.rope_theta:
        wl.rope_theta = float(args.rope_theta)
        tags.append(f"rope{args.rope_theta:g}")
    if tags:
        wl.name = wl.name + "_" + "_".join(tags)
    return wl


def dense_decode_bytes(wl) -> int:
    """Bytes a dense decode step reads and writes: every cached K and V row of
    every KV head (fp8: with one K/V scale pair per page), queries and outputs."""
    row = 128 if wl.kv_dtype == "fp8" else 256
    total = 0
    for n in wl.seq_lens:
        per_head = 2 * row * n + (8 * ((n + 15) // 16) if wl.kv_dtype == "fp8" else 0)
        total += wl.Hkv * per_head
    return total + wl.B * wl.Hq * wl.d * (2 + 4)


def retained_mass(wl, setup) -> dict | None:
    """Per retrieval head: the share of the aggregate index (or full-dim)
    softmax mass the kept set holds, as the selection computed it, and the
    full-dim softmax mass of every query head over its kept set,
    exp(lse - lse_full), with lse_full from the dense log-sum-exp call.
    Also the kept fraction of the context.  Untimed."""
    import torch
    if not wl.retrieval_heads:
        return None
    setup.decode(mass=True)
    torch.cuda.synchronize()
    sm = setup.sel_mass.cpu().numpy()
    lse = setup.lse.cpu().numpy()
    cnt = setup.sel_counts.cpu().numpy()
    G = wl.G
    ret = wl.retrieval_heads
    qheads = [h * G + g for h in ret for g in range(G)]
    if wl.select_scope == "query":
        kept_mass = sm[:, qheads]
        kept = cnt[:, qheads].astype(np.float64)
    else:
        kept_mass = sm[:, ret]
        kept = cnt[:, ret].astype(np.float64)
    n = np.asarray(wl.seq_lens, np.float64)[:, None]
    out = {"selection_mass_mean": round(float(kept_mass.mean()), 5),
           "selection_mass_min": round(float(kept_mass.min()), 5),
           "selection_mass_of": "index" if wl.score_mode == "index" else "full-dim",
           "kept_fraction_mean": round(float((kept / n).mean()), 5),
           "sparsity_mean": round(float(1.0 - (kept / n).mean()), 5)}
    if wl.local_ring and len(ret) < wl.Hkv:
        out["full_dim_mass"] = None          # the dense pass cannot read the ring's local heads
        return out
    full = setup.dense_lse()
    fm = np.exp(lse[:, qheads].astype(np.float64) - full[:, qheads].astype(np.float64))
    out.update({"full_dim_mass_mean": round(float(fm.mean()), 5),
                "full_dim_mass_min": round(float(fm.min()), 5)})
    return out


def cold_graph_steps(setup, stream, iters: int, warmup: int, use_graph: bool) -> dict:
    """Step latencies with cold caches: the step captured once as a HIP graph,
    each replay preceded by an untimed write of a 1 GiB buffer (larger than L2
    and the Infinity Cache) and bracketed by HIP events on the stream."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    g = None
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            setup.decode()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            setup.decode()
    run = g.replay if g is not None else setup.decode
    for i in range(warmup):
        flush.fill_(float(i))
        run()
    torch.cuda.synchronize()
    times = []
    for i in range(iters):
        flush.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del g, flush
    times.sort()
    return {"graph": use_graph, "iters": iters, "p10_ms": round(times[len(times) // 10], 4),
            "p50_ms": round(statistics.median(times), 4), "p90_ms": round(times[(9 * len(times)) // 10], 4)}


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the decode path "
              "has no multi-GPU mode.", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy()
        return 0
    if args.prefill:
        return prefill_main(args)

    import numpy as np
    import torch
    from head_wise_sparse_02_amd import hws
    from head_wise_sparse_02_amd import workloads as W
    from head_wise_sparse_02_amd.runner import DecodeSetup

    wl = build_workload(args, W)
    want_cpu = not args.no_cpu_baseline
    print(f"[bench] building workload {args.config}: {W.CONFIG_NAMES[args.config]}",
          file=sys.stderr, flush=True)
    setup = DecodeSetup(wl, keep_host=want_cpu)
    setup.ctx.set_launch_mode({"auto": hws.HWS_LAUNCH_AUTO, "multi": hws.HWS_LAUNCH_MULTI,
                               "single": hws.HWS_LAUNCH_SINGLE,
                               "cooperative": hws.HWS_LAUNCH_COOPERATIVE,
                               "scan-select": hws.HWS_LAUNCH_SCAN_SELECT,
                               "scan-single": hws.HWS_LAUNCH_SCAN_SINGLE}[args.launch])
    print("[bench] cache filled; warming up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        setup.decode()
    torch.cuda.synchronize()

    # timed region: exactly `steps` decode calls, nothing else in the stream
    ctx = setup.ctx
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        setup.decode()
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps

    # optionally: one decode step captured as a HIP graph (its kernels only),
    # replayed `steps` times
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            setup.decode()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            setup.decode()
        g.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        del g

    # per-kernel durations: the same `steps` decode calls again, each stage's
    # first/last dispatch carrying HIP timing events on the decode stream (the
    # events add bubbles between dispatches, so this loop is not the one timed
    # for `value`)
    ctx.profile_enable(True)
    ctx.profile_read()
    for _ in range(args.steps):
        setup.decode()
    torch.cuda.synchronize()
    prof = ctx.profile_read()
    ctx.profile_enable(False)

    sel_counts = setup.sel_counts.cpu().numpy()
    if wl.select_scope == "query":
        # bytes follow the union of a group's per-query-head sets (one untimed debug call)
        dbg = setup.decode(debug=True)
        kv_counts = np.zeros((wl.B, wl.Hkv), np.int64)
        for b in range(wl.B):
            for h in range(wl.Hkv):
                if h in wl.retrieval_heads:
                    hr = wl.retrieval_heads.index(h)
                    sets = [dbg["sel_idx"][b, hr, g][:dbg["sel_counts"][b, h * wl.G + g]] for g in range(wl.G)]
                    kv_counts[b, h] = np.unique(np.concatenate(sets)).size
                else:
                    kv_counts[b, h] = sel_counts[b, h * wl.G]
        sel_counts = kv_counts
    by = algorithmic_bytes(wl, sel_counts)
    stages = {}
    for name, (ms, calls) in prof.items():
        if calls:
            us = 1000.0 * ms / calls
            b = stage_bytes(name, by)
            stages[name] = {"us": round(us, 2), "bytes": b, "kernel": stage_kernel(name, wl),
                            "GBps": round(b / (us * 1e3), 1) if b else None}
    # the kernel that moves the most algorithmic bytes
    dom = max(stages, key=lambda n: stages[n]["bytes"])
    dom_us = stages[dom]["us"]
    dom_bytes = stages[dom]["bytes"]
    achieved = dom_bytes / (dom_us * 1e3)
    traffic = _read_traffic(dom, stage_kernel(dom, wl), wl.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                "kernel": stage_kernel(dom, wl), "bytes_per_launch": dom_bytes,
                "avg_launch_us": dom_us}

    cold = None
    if args.cold_iters > 0:
        cold = cold_graph_steps(setup, stream, args.cold_iters, min(args.warmup, 10),
                                use_graph=args.launch != "cooperative")
        cold_gbs = by["total"] / (cold["p50_ms"] * 1e6)
        cold.update({"tokens_per_s_p50": round(wl.B / (cold["p50_ms"] / 1000.0), 1),
                     "step_GBps_p50": round(cold_gbs, 1), "step_frac_of_peak_p50": round(cold_gbs / PEAK_GBS, 4)})
    mass = retained_mass(wl, setup)
    dense_bytes = dense_decode_bytes(wl)

    cpu = cpu_baseline(wl, setup, args.cpu_reps) if want_cpu else None

    step_gbs = by["total"] / (ms_per_step * 1e6)
    value = wl.B * args.steps / (total_ms / 1000.0)
    line = {
        "metric": "sparse decode-attn tokens/s & achieved HBM GB/s (% of peak) at 128K ctx, 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.kv_dtype == "bf16" else "fp8",
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "data": "synthetic (seeded; shapes and structure of the workload, no dataset or weights)",
        "config": {"workload": wl.name, "description": W.CONFIG_NAMES[wl.cfg], "batch": wl.B,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d,
                   "context": int(max(wl.seq_lens)), "score_mode": wl.score_mode,
                   "select_mode": wl.select_mode, "kv_dtype": wl.kv_dtype, "launch": args.launch,
                   "select_scope": wl.select_scope, "index_dtype": wl.index_dtype,
                   "local_ring": wl.local_ring, "rope_theta": wl.rope_theta,
                   "top_k": sorted({int(x) for x in wl.top_k}) if wl.select_mode == "top_k" else None,
                   "top_p": sorted({round(float(x), 4) for x in wl.top_p}) if wl.select_mode == "top_p" else None},
        "kv_cache_bytes": int(sum(t.numel() * t.element_size() for t in (
            setup.k_pool, setup.v_pool, setup.kv_scales, setup.index_pool, setup.local_k_pool,
            setup.local_v_pool) if t is not None)),
        "step_bytes": by["total"], "step_GBps": round(step_gbs, 1),
        "step_frac_of_peak": round(step_gbs / PEAK_GBS, 4),
        "dense_decode_bytes": dense_bytes, "dense_to_sparse_bytes": round(dense_bytes / by["total"], 2),
        "retained_mass": mass,
        "value_protocol": "warm: steps back to back on one stream, HIP events around the whole loop; "
                          "cold_graph_step is the flushed, graph-replayed per-step distribution",
        "selected_per_head_mean": round(float(sel_counts[:, [h for h in wl.retrieval_heads]].mean()), 1)
        if wl.retrieval_heads else None,
        "stages": stages, "cold_graph_step": cold,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
