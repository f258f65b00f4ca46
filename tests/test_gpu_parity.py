"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every test runs the whole decode path (append, score, select, attend, merge)
on seeded inputs and checks each stage with the tolerances in gpu_check.
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup, append_segments
from gpu_check import check_decode

pytestmark = pytest.mark.gpu

AUTO, MULTI, COOP, SINGLE = (hws.HWS_LAUNCH_AUTO, hws.HWS_LAUNCH_MULTI, hws.HWS_LAUNCH_COOPERATIVE,
                              hws.HWS_LAUNCH_SINGLE)
BOTH = pytest.mark.parametrize("launch", [SINGLE, MULTI], ids=["single", "multi"])


def _run(wl, pairs=None, sequences=None, verbose=True, launch=AUTO, **kw):
    print(f"\n[case] {wl.name} cfg={wl.cfg} B={wl.B} N={wl.seq_lens[:4]} G={wl.G} "
          f"{wl.score_mode}/{wl.select_mode} kv={wl.kv_dtype} rope={wl.rope_theta} launch={launch}", flush=True)
    st = DecodeSetup(wl, keep_host=True, sequences=sequences)
    st.ctx.set_launch_mode(launch)
    res = st.decode(debug=True)
    reps = check_decode(st, res, pairs=pairs, verbose=verbose, **kw)
    return st, res, reps


@BOTH
def test_tiny_workload_full_parity(launch):
    st, res, reps = _run(W.make_workload(1), launch=launch)
    r0 = [r for r in reps if r["kind"] == "retrieval"][0]
    seq = st.host[0]
    sel = res["sel_idx"][0, 0][:res["sel_counts"][0, 0]]
    assert set(seq.needles[0].tolist()) <= set(sel.tolist())      # all 8 needles kept
    assert r0["n_diff"] == 0


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (16, 2)])
def test_group_sizes(hq, hkv):
    _run(W.make_workload(1, n=3000, Hq=hq, Hkv=hkv))


@BOTH
@pytest.mark.parametrize("n", [1, 2, 15, 17, 255, 1023, 1025, 16385, 20001, 32769])
def test_ragged_lengths(n, launch):
    _run(W.make_workload(1, n=n, extra={"needle_range": (0, None)}), launch=launch)


@BOTH
def test_full_scores_top_k(launch):
    wl = W.make_workload(3, n=5000, batch=2)
    _, res, reps = _run(wl, launch=launch)
    assert all(r["n_gpu"] == int(0.02 * 5000) for r in reps)


@BOTH
def test_full_scores_top_p_and_index_top_k(launch):
    _run(W.make_workload(1, n=4100, score_mode="full"), launch=launch)
    _run(W.make_workload(2, n=3000, batch=2, select_mode="top_k",
                         top_k=np.array([37, 1], np.int32)), launch=launch)


def test_auto_top_k_counts():
    """The default launch shape with top-k on the per-stage path (index scores,
    and full-dim scores at G = 2): |S| = min(k, N) for every head."""
    wl = W.make_workload(2, n=3000, batch=3, select_mode="top_k", top_k=np.array([37, 1, 5000], np.int32))
    _, res, reps = _run(wl, launch=AUTO)
    for r in reps:
        if r["kind"] == "retrieval":
            assert r["n_gpu"] == min(int(wl.top_k[r["b"]]), wl.seq_lens[r["b"]])
    wl = W.make_workload(1, n=4000, Hq=4, Hkv=2, score_mode="full", select_mode="top_k",
                         top_k=np.array([100], np.int32))
    _, res, reps = _run(wl, launch=AUTO)
    assert [r["n_gpu"] for r in reps if r["kind"] == "retrieval"] == [100]


@pytest.mark.parametrize("launch", [AUTO, SINGLE, MULTI], ids=["auto", "single", "multi"])
def test_full_scores_fp8_cache(launch):
    """Full-dim scores over e4m3 pages (products on the codes, scaled by each
    page's K scale): top-k with local heads in a ragged batch, top-p at G = 4,
    and G = 2 with RoPE (split query)."""
    _run(W.make_workload(5, n=20000, batch=4, score_mode="full", select_mode="top_k",
                         top_k=np.array([300, 1, 5000, 20000], np.int32)), launch=launch)
    _run(W.make_workload(1, n=6000, kv_dtype="fp8", score_mode="full"), launch=launch)
    _run(W.make_workload(1, n=5000, Hq=4, Hkv=2, kv_dtype="fp8", score_mode="full", rope_theta=10000.0),
         launch=launch)


@pytest.mark.parametrize("launch", [AUTO, MULTI], ids=["auto", "multi"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_full_scores_g4_rope(kv, launch):
    """G = 4 full-dim scores with rotated queries (each split into a bf16 part
    and the bf16 rounding of the rest), bf16 and e4m3 pages: AUTO runs them
    in the fused launch, MULTI in the per-stage scan.  A ragged batch with a
    local head (ragged tiles, local chunks in the same launch), then top-k
    over one sequence of 40000 positions (three tiles)."""
    _run(W.make_workload(1, n=9000, batch=3, kv_dtype=kv, score_mode="full", rope_theta=10000.0,
                         seq_lens=[9000, 17, 4100]), launch=launch)
    _run(W.make_workload(3, n=40000, batch=1, kv_dtype=kv, rope_theta=500000.0), launch=launch)


@BOTH
@pytest.mark.parametrize("mode", ["top_p_one", "top_k_all", "window_all", "tiny_p"])
def test_reductions_to_dense_and_degenerate(mode, launch):
    n = 777
    if mode == "top_p_one":
        wl = W.make_workload(1, n=n, top_p=np.array([1.0], np.float32))
    elif mode == "top_k_all":
        wl = W.make_workload(1, n=n, select_mode="top_k", top_k=np.array([5000], np.int32))
    elif mode == "window_all":
        wl = W.make_workload(1, n=n, window=4096, n_sink=8)
    else:
        wl = W.make_workload(1, n=n, top_p=np.array([1e-7], np.float32))
    st, res, _ = _run(wl, launch=launch)
    if mode in ("top_p_one", "top_k_all"):
        assert res["sel_counts"][0, 0] == n
    if mode == "window_all":
        assert res["sel_counts"][0, 1] == n
    if mode == "tiny_p":
        assert res["sel_counts"][0, 0] == 1


@BOTH
def test_exact_ties_top_k_lowest_positions(launch):
    """All keys of the retrieval head equal: every a_i ties, so top-k keeps
    positions 0..k-1; top-p keeps every token (ties at the threshold)."""
    n = 40000
    seq = W.make_workload(1, n=n).sequence(0)
    seq.k[:, 0, :] = seq.k[0, 0, :]
    for k in (1234, 20000, 39000):     # inside the first chunk / tile, across them
        wl = W.make_workload(1, n=n, select_mode="top_k", top_k=np.array([k], np.int32))
        _, res, _ = _run(wl, sequences=[seq], launch=launch)
        assert res["sel_counts"][0, 0] == k
        np.testing.assert_array_equal(res["sel_idx"][0, 0, :k], np.arange(k))
    wl2 = W.make_workload(1, n=n)
    _, res2, _ = _run(wl2, sequences=[seq], launch=launch)
    assert res2["sel_counts"][0, 0] == n


def test_llama8b_layer_full_size():
    _run(W.make_workload(2), verbose=False)


def _sample_pairs(wl, n_pairs: int, must=()):
    """A seeded sample of n_pairs distinct (sequence, KV head) pairs that
    includes ``must``; it covers every sequence before repeating one."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.cfg, wl.seed, 5000]))
    pairs = list(dict.fromkeys(tuple(x) for x in must))
    order = rng.permutation(wl.B * wl.Hkv)
    for b_first in (True, False):
        for i in order:
            b, h = int(i) // wl.Hkv, int(i) % wl.Hkv
            if len(pairs) >= n_pairs:
                break
            if (b, h) in pairs or (b_first and any(pb == b for pb, _ in pairs)):
                continue
            pairs.append((b, h))
    return pairs[:n_pairs]


def test_oracle_topk_128k_sampled_and_timed_path():
    """The headline workload at its full size (B = 4, N = 131072, the fused
    launch over 256 tiles): 8 sampled (sequence, KV head) pairs against the
    oracle, then the timed call (no debug outputs, only kept scores written)
    bitwise equal to the debug call."""
    wl = W.make_workload(3)
    pairs = _sample_pairs(wl, 8)
    st = DecodeSetup(wl, keep_host=sorted({b for b, _ in pairs}))
    st.ctx.profile_enable(True)
    res = st.decode(debug=True)
    assert st.ctx.profile_read()["fused"][1] == 1
    check_decode(st, res, pairs=pairs, verbose=True)
    st.decode()
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["fused"][1] == 1, prof
    torch.cuda.synchronize()
    for key, t in (("out", st.out), ("lse", st.lse), ("sel_counts", st.sel_counts)):
        np.testing.assert_array_equal(t.cpu().numpy(), res[key], err_msg=key)


def test_layer_recipe_128k_top_k_sampled():
    """The r = 16 index path at a 128K context: the Llama-3-8B layer recipe
    (B = 8, 2 retrieval + 6 local KV heads) at N = 131072 with a fixed top-k of
    2 % (k = 2621) in place of top-p.  8 sampled pairs, among them both
    retrieval heads of sequence 0, then the timed call bitwise equal to the
    debug call."""
    wl = W.make_workload(2, n=131072, select_mode="top_k", top_k=np.full(8, 2621, np.int32),
                         top_p=np.ones(8, np.float32))
    pairs = _sample_pairs(wl, 8, must=[(0, h) for h in wl.retrieval_heads])
    print(f"\n[case] layer recipe 128K top-k 2%: pairs {pairs}", flush=True)
    st = DecodeSetup(wl, keep_host=sorted({b for b, _ in pairs}))
    res = st.decode(debug=True)
    check_decode(st, res, pairs=pairs, verbose=True)
    assert (res["sel_counts"][:, wl.retrieval_heads] == 2621).all()
    st.decode()
    torch.cuda.synchronize()
    for key, t in (("out", st.out), ("lse", st.lse), ("sel_counts", st.sel_counts)):
        np.testing.assert_array_equal(t.cpu().numpy(), res[key], err_msg=key)


def test_long_256k_all_heads():
    wl = W.make_workload(4)
    _, res, reps = _run(wl, pairs=[(0, h) for h in range(wl.Hkv)])
    print("config 4 retrieval |S| =", res["sel_counts"][0, 0], flush=True)


@pytest.mark.parametrize("n,launch,scope", [(40, MULTI, "kv"), (1000, MULTI, "kv"), (5000, MULTI, "kv"),
                                           (5000, AUTO, "kv"), (40, AUTO, "query"), (5000, AUTO, "query")],
                         ids=["40-multi", "1000-multi", "5000-multi", "5000-auto", "40-query", "5000-query"])
def test_g8_rows_on_matrix_cores(n, launch, scope):
    """G = 8 rows with K (bf16 pages, queries not rotated) take the
    matrix-core attention: two ragged sequences, so chunks leave waves with
    no 32-row batch, a partial one or several; with one set per query head
    each row's head bits mask its logits.  Every head of both sequences
    against the oracle, and the rows each read."""
    wl = W.make_workload(4, n=n, batch=2, select_scope=scope)
    wl.seq_lens = [n, n // 3 + 1]
    _run(wl, launch=launch, pairs=[(b, h) for b in range(2) for h in range(wl.Hkv)])


def test_ragged_fp8_mix_full_size_sampled():
    """The ragged fp8 workload at its full size (B = 32, contexts drawn from
    8K..128K, the default launch shape): 8 sampled (sequence, KV head) pairs,
    among them both retrieval heads of the longest sequence."""
    wl = W.make_workload(5)
    longest = int(np.argmax(wl.seq_lens))
    pairs = _sample_pairs(wl, 8, must=[(longest, h) for h in wl.retrieval_heads])
    print(f"\n[case] ragged fp8 full size: longest N={wl.seq_lens[longest]}, pairs {pairs}", flush=True)
    st = DecodeSetup(wl, keep_host=sorted({b for b, _ in pairs}))
    res = st.decode(debug=True)
    check_decode(st, res, pairs=pairs, verbose=True)


@BOTH
def test_ragged_fp8_mix_reduced(launch):
    wl = W.make_workload(5, n=40000, batch=12)
    _run(wl, verbose=False, launch=launch)


@BOTH
@pytest.mark.parametrize("score_mode", ["index", "full"])
def test_rope_on(score_mode, launch):
    _run(W.make_workload(1, n=3000, rope_theta=10000.0, score_mode=score_mode), launch=launch)


@pytest.mark.parametrize("cfg,kw", [(3, dict(n=40000, batch=4)), (2, dict(n=33000, batch=3)),
                                    (5, dict(n=30000, batch=8)), (3, dict(n=40000, batch=2, kv_dtype="fp8")),
                                    (3, dict(n=40000, batch=2, rope_theta=10000.0)),
                                    (3, dict(n=33000, batch=2, kv_dtype="fp8", rope_theta=10000.0))],
                         ids=["oracle-topk", "layer", "ragged-fp8", "oracle-topk-fp8", "oracle-topk-rope",
                              "oracle-topk-fp8-rope"])
def test_single_launch_matches_multi(cfg, kw):
    """Same token sets from every launch shape; outputs equal up to the fp32
    rounding order of the attention splits.  AUTO and SINGLE run the single
    launch with the scan inside (full-dim G = 4: fused; index scores:
    fused_index), which the recorded profile stages confirm; COOPERATIVE is
    the same kernel and grid, bit for bit; SCAN_SINGLE and SCAN_SELECT run
    the scan as its own kernel first."""
    wl = W.make_workload(cfg, **kw)
    st = DecodeSetup(wl)
    single = "fused" if wl.score_mode == "full" else "fused_index"
    st.ctx.profile_enable(True)

    def run(mode, stage, absent=()):
        st.ctx.set_launch_mode(mode)
        res = st.decode(debug=True)
        prof = st.ctx.profile_read()
        assert prof[stage][1] == 1, (mode, prof)
        for other in absent:
            assert prof[other][1] == 0, (mode, prof)
        assert res["status"] == 0
        return res

    auto = run(AUTO, single, ("select", "tail"))
    a = run(SINGLE, single, ("select", "tail"))
    m = run(MULTI, "select", ("tail", "fused", "fused_index"))
    c = run(COOP, single, ("select", "tail"))
    # (the single launch after a full-dim scan reads bf16 V rows only: with
    # e4m3 pages SCAN_SINGLE runs the per-stage kernels)
    if wl.score_mode == "full" and wl.kv_dtype == "fp8":
        ss = run(hws.HWS_LAUNCH_SCAN_SINGLE, "select", ("tail", "fused", "fused_index"))
    else:
        ss = run(hws.HWS_LAUNCH_SCAN_SINGLE, "tail", ("select", "fused", "fused_index"))
    sel = run(hws.HWS_LAUNCH_SCAN_SELECT, "select", ("tail", "fused", "fused_index"))
    st.ctx.profile_enable(False)
    for key in ("out", "lse", "sel_counts", "sel_idx", "scores", "rows_read", "sel_mass"):
        np.testing.assert_array_equal(auto[key], a[key], err_msg=key)
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)    # same kernel, same grid
    for other in (m, ss, sel):
        for key in ("sel_counts", "sel_idx", "scores", "rows_read"):
            np.testing.assert_array_equal(a[key], other[key], err_msg=key)
        for key in ("out", "lse"):
            np.testing.assert_allclose(a[key], other[key], rtol=0, atol=2e-5, err_msg=key)
        np.testing.assert_allclose(a["sel_mass"], other["sel_mass"], rtol=0, atol=1e-6)
    # the one-launch selection and the three selection kernels give the same
    # sets (after it, index scores take the attention balanced by kept rows,
    # full-dim scores the per-stage attention of MULTI: then bit for bit)
    for key in ("sel_counts", "sel_idx", "scores", "rows_read"):
        np.testing.assert_array_equal(sel[key], m[key], err_msg=key)
    for key in ("out", "lse"):
        if wl.score_mode == "full":
            np.testing.assert_array_equal(sel[key], m[key], err_msg=key)
        else:
            np.testing.assert_allclose(sel[key], m[key], rtol=0, atol=2e-5, err_msg=key)


SCAN_SELECT = hws.HWS_LAUNCH_SCAN_SELECT


@pytest.mark.parametrize("cfg,kw", [
    (1, dict(n=5000)),
    (1, dict(n=3000, Hq=2, Hkv=2)),
    (1, dict(n=3000, Hq=4, Hkv=2, batch=3)),
    (2, dict(n=9000, batch=3)),
    (2, dict(n=9000, batch=3, kv_dtype="fp8", local_ring=True)),
    (2, dict(n=3000, batch=3, select_mode="top_k", top_k=np.array([1, 37, 5000], np.int32))),
    (4, dict(n=60000)),
    (5, dict(n=30000, batch=8)),
    (2, dict(n=300, batch=16, select_mode="top_k", top_k=np.full(16, 1, np.int32), window=40)),
    (2, dict(n=5000, batch=3, rope_theta=10000.0)),
    (5, dict(n=20000, batch=4, rope_theta=10000.0)),
], ids=["tiny", "g1", "g2-batch", "layer", "layer-fp8-ring", "topk-edges", "long-g8", "ragged-fp8",
        "many-small-pairs", "layer-rope", "ragged-fp8-rope"])
def test_balanced_attention_against_oracle(cfg, kw):
    """The attention balanced by kept rows (equal row segments over all
    heads, the next batch of loads in flight) against the oracle: group sizes
    1 to 8, bf16 and fp8 pools, a bf16 local ring beside an fp8 cache, top-k
    sets of one row and of the whole context, a single retrieval head spread
    over most workgroups (G = 8), ragged fp8 sequences, 128 pairs of one or a
    few dozen rows (segments that end inside a pair's fixed cost), and RoPE
    (the rotated queries against the rotated K rows)."""
    wl = W.make_workload(cfg, **kw)
    _, res, _ = _run(wl, launch=SCAN_SELECT, verbose=False)
    assert res["status"] == 0


@pytest.mark.parametrize("n,expect", [(4096, "tail"), (4097, "select")])
def test_auto_short_contexts_take_single_launch(n, expect):
    """Full-dim scores at G = 2 (no scan inside a launch for them): AUTO runs
    short contexts (max_seq_len <= 4096) as the single launch after the scan,
    longer ones as the one-launch selection and the per-stage attention; index
    scores run the launch with the scan inside at either length.  All against
    the oracle."""
    wl = W.make_workload(1, n=n, Hq=4, Hkv=2, score_mode="full", batch=2)
    st = DecodeSetup(wl, keep_host=True)
    st.ctx.profile_enable(True)
    res = st.decode(debug=True)
    prof = st.ctx.profile_read()
    assert prof[expect][1] == 1 and prof["fused_index"][1] == 0, prof
    check_decode(st, res, verbose=False)
    wl = W.make_workload(2, n=n, batch=2)
    st = DecodeSetup(wl, keep_host=True)
    st.ctx.profile_enable(True)
    res = st.decode(debug=True)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["fused_index"][1] == 1 and prof["score"][1] == 0, prof
    check_decode(st, res, verbose=False)


def test_fp8_codes_and_scales_bit_exact():
    wl = W.make_workload(5, n=600, batch=3)
    st = DecodeSetup(wl, keep_host=True)
    torch.cuda.synchronize()
    kp = st.k_pool.cpu().numpy()
    vp = st.v_pool.cpu().numpy()
    sc = st.kv_scales.cpu().numpy()
    for b in range(wl.B):
        n = wl.seq_lens[b]
        seq = st.host[b]
        for h in range(wl.Hkv):
            for arr, pool, j in ((seq.k, kp, 0), (seq.v, vp, 1)):
                codes, scales, _ = O.fp8_store_rows(arr[:n, h].astype(np.float64), append_segments(n))
                for blk_l, s in scales.items():
                    phys = st.block_tables_host[b, blk_l]
                    lo, hi = blk_l * 16, min(n, blk_l * 16 + 16)
                    assert sc[phys, h, j] == s
                    page = pool[phys, h].reshape(-1)
                    if j == 0:   # K pages are stored in four 32-dim blocks
                        page = page.reshape(4, 16, 32).transpose(1, 0, 2)
                    page = page.reshape(16, 128)
                    np.testing.assert_array_equal(page[:hi - lo], codes[lo:hi])


def test_index_pool_matches_projection():
    wl = W.make_workload(2, n=2000, batch=2)
    st = DecodeSetup(wl, keep_host=True)
    ip = st.index_pool.cpu().numpy()
    for b in range(wl.B):
        for hr, h in enumerate(wl.retrieval_heads):
            n = wl.seq_lens[b]
            ref = st.host[b].k[:n, h].astype(np.float64) @ st.proj_host[h].astype(np.float64).T
            got = np.stack([ip[st.block_tables_host[b, i // 16], hr, i % 16] for i in range(n)])
            bound = 1e-5 * np.linalg.norm(st.host[b].k[:n, h], axis=1)[:, None] * \
                np.linalg.norm(st.proj_host[h], axis=1)[None, :]
            assert (np.abs(got - ref) <= bound).all()


def test_repeat_is_bitwise_deterministic():
    wl = W.make_workload(2, n=9000, batch=3)
    st = DecodeSetup(wl)
    first = st.decode(debug=True)
    for _ in range(5):
        again = st.decode(debug=True)
        for key in ("out", "lse", "sel_counts", "sel_idx", "scores"):
            np.testing.assert_array_equal(first[key], again[key])
    # without the debug outputs the timed path gives the same bits
    st.decode(debug=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.out.cpu().numpy(), first["out"])


# -- single launch with the scoring scan inside (full-dim scores, G = 4) ------

@pytest.mark.parametrize("n", [1, 17, 1000, 4097, 16384, 16385, 40000])
def test_fused_ragged_lengths(n):
    """Tiles past the end, partial pages and partial tiles; with a local head
    (config 1 shape) the local chunks run in the same launch."""
    _run(W.make_workload(1, n=n, score_mode="full", extra={"needle_range": (0, None)}))


def test_fused_top_k_batch_and_ties():
    _run(W.make_workload(3, n=33000, batch=3))
    n = 40000
    seq = W.make_workload(1, n=n).sequence(0)
    seq.k[:, 0, :] = seq.k[0, 0, :]                  # every logit of head 0 equal
    for k in (1234, 20000, 39000):
        wl = W.make_workload(1, n=n, score_mode="full", select_mode="top_k", top_k=np.array([k], np.int32))
        _, res, _ = _run(wl, sequences=[seq])
        assert res["sel_counts"][0, 0] == k
        np.testing.assert_array_equal(res["sel_idx"][0, 0, :k], np.arange(k))


@pytest.mark.parametrize("mode", ["top_p_one", "top_k_all", "tiny_p"])
def test_fused_degenerate(mode):
    n = 5000
    if mode == "top_p_one":
        wl = W.make_workload(1, n=n, score_mode="full", top_p=np.array([1.0], np.float32))
    elif mode == "top_k_all":
        wl = W.make_workload(1, n=n, score_mode="full", select_mode="top_k", top_k=np.array([9000], np.int32))
    else:
        wl = W.make_workload(1, n=n, score_mode="full", top_p=np.array([1e-7], np.float32))
    _, res, _ = _run(wl)
    assert res["sel_counts"][0, 0] == (1 if mode == "tiny_p" else n)


def test_fused_timed_path_matches_debug_path():
    """Without debug outputs the fused launch writes only the kept tokens'
    scores; the results are bitwise those of the debug run."""
    wl = W.make_workload(3, n=50000, batch=2)
    st = DecodeSetup(wl)
    st.ctx.profile_enable(True)
    full = st.decode(debug=True)
    st.decode(debug=False)
    torch.cuda.synchronize()
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["fused"][1] == 2, prof
    np.testing.assert_array_equal(st.out.cpu().numpy(), full["out"])
    np.testing.assert_array_equal(st.lse.cpu().numpy(), full["lse"])
    np.testing.assert_array_equal(st.sel_counts.cpu().numpy(), full["sel_counts"])


# -- one token set per query head (select_scope = query) ------------------------

@pytest.mark.parametrize("select_mode", ["top_p", "top_k"])
def test_query_scope_tiny_and_layer(select_mode):
    kw = {} if select_mode == "top_p" else dict(select_mode="top_k", top_k=np.array([61], np.int32))
    _run(W.make_workload(1, select_scope="query", **kw))
    kw2 = {} if select_mode == "top_p" else dict(select_mode="top_k", top_k=np.array([100, 7], np.int32))
    _run(W.make_workload(2, n=9000, batch=2, select_scope="query", **kw2), verbose=False)


def test_query_scope_peaky_and_diffuse_heads():
    """The 70B-shaped group (G = 8): peaky query heads keep a few tokens,
    diffuse ones thousands; each head attends over its own set."""
    wl = W.make_workload(4, n=20000, select_scope="query")
    st, res, reps = _run(wl, pairs=[(0, 0), (0, 3)])
    G = wl.G
    counts = res["sel_counts"][0, :G]
    print("per-query-head |S|:", counts.tolist(), flush=True)
    assert counts.max() > 20 * counts.min()


def test_query_scope_full_scores_and_degenerate():
    _run(W.make_workload(3, n=6000, batch=2, select_scope="query"))
    n = 777
    wl = W.make_workload(1, n=n, select_scope="query", top_p=np.array([1.0], np.float32))
    _, res, _ = _run(wl)
    assert (res["sel_counts"][0, :4] == n).all()
    wl = W.make_workload(1, n=n, select_scope="query", top_p=np.array([1e-7], np.float32))
    _, res, _ = _run(wl)
    assert (res["sel_counts"][0, :4] == 1).all()


def test_query_scope_ties_and_single_launch_falls_back():
    n = 30000
    seq = W.make_workload(1, n=n).sequence(0)
    seq.k[:, 0, :] = seq.k[0, 0, :]                  # every logit of head 0 equal
    wl = W.make_workload(1, n=n, select_scope="query", select_mode="top_k", top_k=np.array([1234], np.int32))
    st = DecodeSetup(wl, keep_host=True, sequences=[seq])
    st.ctx.set_launch_mode(SINGLE)                   # one set per query head runs per stage
    st.ctx.profile_enable(True)
    res = st.decode(debug=True)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["select"][1] == 1 and prof["tail"][1] == 0, prof
    check_decode(st, res)
    for g in range(wl.G):
        assert res["sel_counts"][0, g] == 1234
        np.testing.assert_array_equal(res["sel_idx"][0, 0, g, :1234], np.arange(1234))


# -- bf16 index (32 B per token and retrieval head) ------------------------------

@pytest.mark.parametrize("n", [1, 17, 1025, 20001])
def test_bf16_index_ragged(n):
    _run(W.make_workload(1, n=n, index_dtype="bf16", extra={"needle_range": (0, None)}))


@pytest.mark.parametrize("hq,hkv", [(2, 2), (16, 2), (8, 8)])
def test_bf16_index_group_sizes(hq, hkv):
    _run(W.make_workload(1, n=5000, Hq=hq, Hkv=hkv, head_kinds=["retrieval"] + ["local"] * (hkv - 1),
                         index_dtype="bf16"))


def test_bf16_index_layer_fp8_rope_and_query_scope():
    _run(W.make_workload(2, n=9000, batch=2, index_dtype="bf16"), verbose=False)
    _run(W.make_workload(5, n=30000, batch=6, index_dtype="bf16"), verbose=False)
    _run(W.make_workload(1, n=3000, rope_theta=10000.0, index_dtype="bf16"))
    _run(W.make_workload(1, n=6000, select_scope="query", index_dtype="bf16"))


def test_bf16_index_pool_values():
    """The stored index is bf16(P k) with P k in fp64: equal to the oracle's
    except where the fp64 value sits within 1e-12 of a bf16 rounding boundary
    (the two fp64 sums may round differently there)."""
    wl = W.make_workload(2, n=3000, batch=2, index_dtype="bf16")
    st = DecodeSetup(wl, keep_host=True)
    ip = st.index_pool.float().cpu().numpy()
    for b in range(wl.B):
        n = wl.seq_lens[b]
        for hr, h in enumerate(wl.retrieval_heads):
            ref = O.index_keys(st.host[b].k[:n, h], st.proj_host[h], index_bf16=True)
            raw = st.host[b].k[:n, h].astype(np.float64) @ st.proj_host[h].astype(np.float64).T
            got = np.stack([ip[st.block_tables_host[b, i // 16], hr, i % 16] for i in range(n)])
            diff = got != ref
            if diff.any():
                # a differing element must be a near-tie of the rounding
                ulp = 2.0 ** (np.floor(np.log2(np.abs(raw[diff]))) - 7)       # bf16 spacing at |raw|
                mid = np.abs(np.abs(raw[diff] - ref[diff]) - ulp / 2)
                assert (mid <= 1e-12 * np.abs(raw[diff]) + 1e-30).all()
            assert diff.mean() < 1e-6


# -- retained full-dim mass: the dense log-sum-exp diagnostic -----------------------

@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(n=6000, batch=2)), (5, dict(n=20000, batch=3)),
                                    (1, dict(n=3000, rope_theta=10000.0)), (4, dict(n=9000))])
def test_dense_lse_and_full_dim_mass(cfg, kw):
    """hws_dense_lse against the oracle's log-sum-exp of every full-dim logit
    (fp8 rows as stored, RoPE rotated), and the full-dim mass the GPU's sets
    keep, mean_g exp(lse_S - lse_full), against the oracle's full_mass on the
    same sets ([RTPurbo] Main results: attention mass retained)."""
    import scipy.special
    wl = W.make_workload(cfg, **kw)
    print(f"\n[case] dense lse {wl.name} B={wl.B} N={wl.seq_lens[:3]} kv={wl.kv_dtype} rope={wl.rope_theta}",
          flush=True)
    st = DecodeSetup(wl, keep_host=True)
    res = st.decode(debug=True)
    lf = st.dense_lse()
    G = wl.G
    worst_lse = worst_mass = 0.0
    for b in range(wl.B):
        seq = st.host[b]
        n = wl.seq_lens[b]
        for h in range(wl.Hkv):
            q_rot = O.rope(seq.q[h * G:(h + 1) * G].astype(np.float64), np.full(G, n - 1), wl.rope_theta)
            ks = O.stored_rows(seq.k[:n, h], np.arange(n), rope_theta=wl.rope_theta, kv_fp8=st.fp8,
                               segments=st.segments(n), rotate=True)
            _, z = O.full_logits(q_rot, ks, wl.attn_scale)
            lse_ref = scipy.special.logsumexp(z, axis=1)
            e = float(np.abs(lf[b, h * G:(h + 1) * G] - lse_ref).max())
            worst_lse = max(worst_lse, e)
            assert e <= 1e-4, f"dense lse off at (b={b}, h={h}): {e}"
            if wl.head_kinds[h] == "retrieval":
                hr = wl.retrieval_heads.index(h)
                S = res["sel_idx"][b, hr][:res["sel_counts"][b, h]].astype(np.int64)
            else:
                S = O.local_token_set(n, wl.n_sink, wl.window)
            ref = O.decode_sequence_ref(
                seq.q, seq.k, seq.v, head_kinds=wl.head_kinds, proj=st.proj_host, score_mode=wl.score_mode,
                select_mode=wl.select_mode, top_p=float(wl.top_p[b]), top_k=int(wl.top_k[b]), n_sink=wl.n_sink,
                window=wl.window, attn_scale=wl.attn_scale, index_scale=wl.index_scale, rope_theta=wl.rope_theta,
                kv_fp8=st.fp8, segments=st.segments(n), heads=[h], fixed_sets={h: S}, with_full_mass=True)[h]
            m_gpu = float(np.mean(np.exp(res["lse"][b, h * G:(h + 1) * G].astype(np.float64)
                                         - lf[b, h * G:(h + 1) * G].astype(np.float64))))
            em = abs(m_gpu - ref["full_mass"])
            worst_mass = max(worst_mass, em)
            assert em <= 1e-4, f"full-dim mass off at (b={b}, h={h}): {m_gpu} vs {ref['full_mass']}"
    print(f"[ok] dense lse err {worst_lse:.2e}, full-dim mass err {worst_mass:.2e}", flush=True)
