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


def test_oracle_topk_128k_sampled():
    wl = W.make_workload(3)
    _run(wl, pairs=[(0, 0), (1, 3), (2, 5), (3, 7)])


def test_long_256k_sampled():
    wl = W.make_workload(4)
    _, res, reps = _run(wl, pairs=[(0, 0), (0, 1), (0, 7)])
    print("config 4 retrieval |S| =", res["sel_counts"][0, 0], flush=True)


@BOTH
def test_ragged_fp8_mix_reduced(launch):
    wl = W.make_workload(5, n=40000, batch=12)
    _run(wl, verbose=False, launch=launch)


@BOTH
@pytest.mark.parametrize("score_mode", ["index", "full"])
def test_rope_on(score_mode, launch):
    _run(W.make_workload(1, n=3000, rope_theta=10000.0, score_mode=score_mode), launch=launch)


@pytest.mark.parametrize("cfg,kw", [(3, dict(n=40000, batch=4)), (2, dict(n=33000, batch=3)),
                                    (5, dict(n=30000, batch=8))])
def test_single_launch_matches_multi(cfg, kw):
    """Same token sets from both launch shapes; outputs equal up to the fp32
    rounding order of the attention splits.  The single launch is the one
    that ran (its profile stage is recorded)."""
    wl = W.make_workload(cfg, **kw)
    st = DecodeSetup(wl)
    fused = wl.score_mode == "full" and wl.G == 4 and not wl.rope_theta
    single = "fused" if fused else "tail"
    st.ctx.profile_enable(True)
    st.ctx.set_launch_mode(AUTO)                      # fused launch where it applies, else per stage
    auto = st.decode(debug=True)
    prof = st.ctx.profile_read()
    assert prof["fused" if fused else "select"][1] == 1, prof
    st.ctx.set_launch_mode(SINGLE)
    a = st.decode(debug=True)
    prof = st.ctx.profile_read()
    assert prof[single][1] == 1 and prof["select"][1] == 0, prof
    for key in ("out", "lse", "sel_counts", "sel_idx", "scores"):
        np.testing.assert_array_equal(auto[key], (a if fused else auto)[key])
    st.ctx.set_launch_mode(MULTI)
    m = st.decode(debug=True)
    prof = st.ctx.profile_read()
    assert prof["tail"][1] == 0 and prof["select"][1] == 1, prof
    st.ctx.set_launch_mode(COOP)
    c = st.decode(debug=True)
    prof = st.ctx.profile_read()
    assert prof[single][1] == 1 and prof["select"][1] == 0, prof
    st.ctx.profile_enable(False)
    for key in ("out", "lse", "sel_counts", "sel_idx", "scores"):   # same kernel, same grid
        np.testing.assert_array_equal(a[key], c[key])
    np.testing.assert_array_equal(a["sel_counts"], m["sel_counts"])
    np.testing.assert_array_equal(a["sel_idx"], m["sel_idx"])
    np.testing.assert_array_equal(a["scores"], m["scores"])
    np.testing.assert_allclose(a["out"], m["out"], rtol=0, atol=2e-5)
    np.testing.assert_allclose(a["lse"], m["lse"], rtol=0, atol=2e-5)
    if not fused:
        # AUTO: the selection in one launch, then the per-stage attention and
        # merge: the sets of the three-launch selection, and the same kernels
        # after it
        for key in ("sel_counts", "sel_idx", "scores", "out", "lse"):
            np.testing.assert_array_equal(auto[key], m[key])


@pytest.mark.parametrize("n,tail", [(4096, True), (4097, False)])
def test_auto_short_contexts_take_single_launch(n, tail):
    """AUTO runs short contexts (max_seq_len <= 4096) as the single launch
    after the scan, longer ones per stage; both against the oracle."""
    wl = W.make_workload(2, n=n, batch=2)
    st = DecodeSetup(wl, keep_host=True)
    st.ctx.profile_enable(True)
    res = st.decode(debug=True)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert (prof["tail"][1], prof["select"][1]) == ((1, 0) if tail else (0, 1)), prof
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
