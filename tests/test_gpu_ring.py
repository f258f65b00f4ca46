"""GPU parity of the local-head ring: local heads keep only their sinks and
window in a per-sequence ring, the pages hold only the retrieval heads.

A local head reads nothing but its sinks and window ([RTPurbo] Methodology
§1), so the decode result is the oracle's, with every append schedule; and
since the rows, their order and the arithmetic are those of the paged cache,
the outputs equal the paged cache's bit for bit.
"""

import numpy as np
import pytest
import torch

from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup, ring_mod, ring_rows, ring_sink
from gpu_check import check_decode

pytestmark = pytest.mark.gpu

AUTO, MULTI, SINGLE = hws.HWS_LAUNCH_AUTO, hws.HWS_LAUNCH_MULTI, hws.HWS_LAUNCH_SINGLE


def _pair(wl, launch=AUTO, segments=None, check=True):
    """Decode wl with the ring and with the paged cache; check the ring against
    the oracle and return both results."""
    print(f"\n[case] ring {wl.name} B={wl.B} N={wl.seq_lens[:4]} G={wl.G} {wl.score_mode}/"
          f"{wl.select_mode} window={wl.window} rope={wl.rope_theta} launch={launch}", flush=True)
    wl.local_ring = True
    ring = DecodeSetup(wl, keep_host=True, segments=segments)
    ring.ctx.set_launch_mode(launch)
    r = ring.decode(debug=True)
    if check:
        check_decode(ring, r, verbose=True)
    wl.local_ring = False
    paged = DecodeSetup(wl, segments=segments)
    paged.ctx.set_launch_mode(launch)
    p = paged.decode(debug=True)
    wl.local_ring = True
    return ring, r, p


def _same(r, p):
    for key in ("out", "lse", "sel_counts"):
        np.testing.assert_array_equal(r[key], p[key])
    if "sel_idx" in p:
        np.testing.assert_array_equal(r["sel_idx"], p["sel_idx"])


@pytest.mark.parametrize("launch", [MULTI, SINGLE], ids=["multi", "single"])
@pytest.mark.parametrize("n", [1, 17, 63, 64, 65, 200, 320, 321, 1000, 5000])
def test_ring_tiny_matches_oracle_and_pages(n, launch):
    """Sinks 4, window 256: the ring keeps positions 0..63 in their own rows
    and cycles later ones through 256 rows; lengths inside the first rows, at
    and past their end, inside the first cycle, at its end, one past it, and
    far beyond it."""
    wl = W.make_workload(1, n=n, extra={"needle_range": (0, None)})
    _, r, p = _pair(wl, launch=launch)
    _same(r, p)


def _schedule(seed):
    """Append calls of random lengths: some longer than the window, some a
    few tokens, some single tokens, so the ring wraps inside and across calls."""
    def seg(n):
        rng = np.random.default_rng(seed + n)
        out, pos = [], 0
        while pos < n:
            c = int(rng.choice([1, 1, 3, 16, 77, 300, 1100, 2500]))
            c = min(c, n - pos)
            out.append((pos, c))
            pos += c
        return out
    return seg


@pytest.mark.parametrize("cfg,kw", [(1, dict(n=3001)), (2, dict(n=4100, batch=3)),
                                    (4, dict(n=9000, batch=2))])
def test_ring_append_schedules(cfg, kw):
    wl = W.make_workload(cfg, **kw)
    _, r, p = _pair(wl, segments=_schedule(11))
    _same(r, p)


def test_ring_ragged_batch_rope_and_query_scope():
    wl = W.make_workload(2, n=3000, batch=4, rope_theta=10000.0)
    wl.seq_lens = [3000, 1, 1030, 257]
    _, r, p = _pair(wl, segments=_schedule(5))
    _same(r, p)
    wl = W.make_workload(2, n=2500, batch=2, select_scope="query")
    _, r, p = _pair(wl)
    _same(r, p)


def test_ring_single_launch_with_scan_inside():
    """Full-dim scores with G = 4 and a local head run as one launch; its local
    chunks read the ring."""
    wl = W.make_workload(1, n=20000, score_mode="full", select_mode="top_k",
                         top_k=np.full(1, 400, np.int32), extra={"needle_range": (0, None)})
    wl.local_ring = True
    st = DecodeSetup(wl, keep_host=True)
    st.ctx.profile_enable(True)
    r = st.decode(debug=True)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["fused"][1] == 1, prof
    check_decode(st, r, verbose=True)


@pytest.mark.parametrize("n_sink,window", [(70, 100), (0, 300), (5, 0), (200, 64)])
def test_ring_geometry_edges(n_sink, window):
    """Sinks over one 64-key tile, no sinks, sinks only, sinks longer than the
    window: decode from the ring against the oracle and the paged cache."""
    wl = W.make_workload(1, n=3001, n_sink=n_sink, window=window, extra={"needle_range": (0, None)})
    _, r, p = _pair(wl, launch=MULTI, segments=_schedule(9))
    _same(r, p)


@pytest.mark.parametrize("launch", [AUTO, SINGLE, MULTI], ids=["auto", "single", "multi"])
def test_ring_with_fp8_pages(launch):
    """fp8 pages for the retrieval heads, bf16 ring rows for the local heads,
    in a ragged batch appended in calls of random lengths (page scales set by
    several calls), against the oracle."""
    wl = W.make_workload(5, n=12000, batch=6)
    wl.local_ring = True
    print(f"\n[case] ring fp8 {wl.name} B={wl.B} N={wl.seq_lens} launch={launch}", flush=True)
    st = DecodeSetup(wl, keep_host=True, segments=_schedule(7))
    st.ctx.set_launch_mode(launch)
    r = st.decode(debug=True)
    check_decode(st, r, verbose=False)
    assert st.k_pool.dtype == torch.uint8 and st.local_k_pool.dtype == torch.bfloat16


@pytest.mark.parametrize("cfg", [2, 5], ids=["bf16", "fp8_pages"])
def test_ring_rows_hold_sinks_and_window(cfg):
    """After appends the ring holds exactly the bf16 rows of the sinks and the
    window, at the documented ring rows; rows of evicted tokens are gone."""
    wl = W.make_workload(cfg, n=2100, batch=2)
    wl.local_ring = True
    st = DecodeSetup(wl, keep_host=True, segments=_schedule(3))
    torch.cuda.synchronize()
    lk = st.local_k_pool.cpu().float().numpy()     # [slots][nL][W/16][4][16][32]
    lv = st.local_v_pool.cpu().float().numpy()     # [slots][nL][W][128]
    W_ = ring_rows(wl.n_sink, wl.window)
    assert lv.shape[2] == W_
    local = [h for h, k in enumerate(wl.head_kinds) if k == "local"]
    for b in range(wl.B):
        n = wl.seq_lens[b]
        slot = int(st.seq_slots_host[b])
        toks = sorted(set(range(min(wl.n_sink, n))) | set(range(max(0, n - wl.window), n)))
        for l, h in enumerate(local):
            kpage = lk[slot, l].transpose(0, 2, 1, 3).reshape(W_, 128)   # page-blocked -> rows
            for t in toks:
                S, M = ring_sink(wl.n_sink), ring_mod(wl.window)
                rr = t if t < S else S + t % M
                np.testing.assert_array_equal(kpage[rr], st.host[b].k[t, h])
                np.testing.assert_array_equal(lv[slot, l, rr], st.host[b].v[t, h])
    # the pages hold the retrieval heads only
    assert st.k_pool.shape[1] == len(wl.retrieval_heads)


def test_ring_slot_out_of_range_reads_nothing():
    """A sequence whose slot is out of range: its local heads see an empty set
    (output 0, lse -inf); its retrieval heads and the other sequences are as
    before."""
    wl = W.make_workload(2, n=1500, batch=3)
    wl.local_ring = True
    st = DecodeSetup(wl)
    good = st.decode(debug=True)
    st.seq_slots[1] = st.max_seqs + 7
    bad = st.decode(debug=True)
    G = wl.G
    for h, kind in enumerate(wl.head_kinds):
        qs = slice(h * G, (h + 1) * G)
        for b in range(wl.B):
            if b == 1 and kind == "local":
                assert (bad["out"][b, qs] == 0).all()
                assert np.isneginf(bad["lse"][b, qs]).all()
            else:
                np.testing.assert_array_equal(bad["out"][b, qs], good["out"][b, qs])
