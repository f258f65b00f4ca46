"""Pins for the CPU oracle: closed forms, brute force, invariants, library routines.

Each test checks the oracle against something other than itself, chosen so that
a plausible slip (a dropped term, a wrong sign or index, a transposed operand,
a lost tie rule) fails at least one of them.  No GPU is used.
"""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from head_wise_sparse_02_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- encodings

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)
    # the generator's float32 rounding agrees with torch as well
    x32 = x.astype(np.float32)
    ref32 = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(W.bf16_rne(x32), ref32)


def test_e4m3_table_exhaustive_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = O.e4m3_table()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(tab))
    np.testing.assert_array_equal(tab[~nan], ref[~nan])
    assert np.nanmax(tab) == 448.0 and tab[0x08] == 2.0 ** -6 and tab[0x01] == 2.0 ** -9


def test_e4m3_encode_roundtrip_and_torch_rne():
    tab = O.e4m3_table()
    finite = np.nonzero(~np.isnan(tab))[0]
    # every finite code value encodes to itself (0x80 is -0.0)
    np.testing.assert_array_equal(O.e4m3_encode(tab[finite]), finite.astype(np.uint8))
    # random values, clamped to the finite range: same code as torch's RNE cast
    rng = np.random.default_rng(2)
    y = rng.standard_normal(50000) * 10.0 ** rng.integers(-4, 3, 50000)
    y32 = np.clip(y.astype(np.float32), -448, 448)
    ref = torch.from_numpy(y32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(y32.astype(np.float64)), ref)
    # midpoints go to the even code; beyond 448 saturates
    assert O.e4m3_encode(np.array([1.0 + 1 / 16]))[0] == 0x38           # 1.0 (even) not 1.125
    assert O.e4m3_encode(np.array([1.0 + 3 / 16]))[0] == 0x3A           # 1.25 (even)
    assert O.e4m3_encode(np.array([1e6, -1e6])).tolist() == [0x7E, 0xFE]
    assert O.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00             # half of min subnormal -> 0
    assert O.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02         # 1.5 ulp -> 2 (even)


def test_fp8_store_rows_scale_rules():
    rng = np.random.default_rng(3)
    x = W.bf16_rne(rng.standard_normal((40, 8)).astype(np.float32)).astype(np.float64)
    # bulk append of 20 rows, then single-token appends 20..39
    segs = [(0, 20)] + [(i, 1) for i in range(20, 40)]
    codes, scales, deq = O.fp8_store_rows(x, segs)
    s0 = np.float32(np.abs(x[:16]).max()) / np.float32(448)
    s1 = np.float32(np.abs(x[16:20]).max()) / np.float32(448)
    assert scales[0] == s0 and scales[1] == s1
    # block 2 opened by the single-token append of position 32: scale from row 32 only
    assert scales[2] == np.float32(np.abs(x[32]).max()) / np.float32(448)
    # the row that set a block scale holds a +-448 code at its max element
    assert np.abs(O.e4m3_decode(codes[32])).max() == 448.0
    # later rows of block 1 reuse s1 and saturate if larger than the block max
    big = np.abs(x[20:32]).max() > np.abs(x[16:20]).max()
    assert (np.abs(O.e4m3_decode(codes[20:32])).max() == 448.0) == big
    # dequantised error within half an e4m3 step (relative 2**-4) or saturation
    rel = np.abs(deq[:16] - x[:16]) / np.maximum(np.abs(x[:16]), 2 ** -6 * s0)
    assert rel.max() <= 2 ** -4 + 1e-12


# ---------------------------------------------------------------- RoPE

def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(4)
    d, theta = 128, 10000.0
    x = rng.standard_normal((7, d))
    pos = np.array([0, 1, 5, 100, 4095, 131071, 262143])
    half = d // 2
    z = x[:, :half] + 1j * x[:, half:]
    freq = np.exp(-np.log(theta) * (2.0 * np.arange(half) / d))
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    np.testing.assert_allclose(O.rope(x, pos, theta), ref, rtol=0, atol=1e-9)
    # position 0 is the identity; theta <= 0 switches RoPE off
    np.testing.assert_array_equal(O.rope(x[:1], [0], theta), x[:1])
    np.testing.assert_array_equal(O.rope(x, pos, 0.0), x)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    a = O.rope(q[None], [1000], 10000.0)[0] @ O.rope(k[None], [990], 10000.0)[0]
    b = O.rope(q[None], [10], 10000.0)[0] @ O.rope(k[None], [0], 10000.0)[0]
    assert abs(a - b) < 1e-9


# ---------------------------------------------------------------- scores

def test_index_scores_identity_projection_is_full_dot():
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((4, 128)), rng.standard_normal((50, 128))
    s, l = O.index_logits(q, k, np.eye(128), 0.5)
    np.testing.assert_allclose(s, q @ k.T, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(l, 0.5 * (q @ k.T), rtol=1e-13, atol=1e-12)


def test_index_scores_brute_force_and_orientation():
    rng = np.random.default_rng(7)
    q, k, P = rng.standard_normal((3, 128)), rng.standard_normal((9, 128)), rng.standard_normal((16, 128))
    s, _ = O.index_logits(q, k, P, 1.0)
    for g in range(3):
        for i in range(9):
            qt = [sum(P[j, t] * q[g, t] for t in range(128)) for j in range(16)]
            kt = [sum(P[j, t] * k[i, t] for t in range(128)) for j in range(16)]
            assert abs(s[g, i] - sum(a * b for a, b in zip(qt, kt))) < 1e-9 * (1 + abs(s[g, i]))


def test_bf16_index_selecting_projection_is_exact():
    """P selecting 16 coordinates of bf16 keys: k~ is already bf16, so the
    bf16 index equals the fp32 one exactly (closed form)."""
    rng = np.random.default_rng(71)
    q = O.bf16_round(rng.standard_normal((4, 128)))
    k = O.bf16_round(rng.standard_normal((40, 128)))
    P = np.zeros((16, 128))
    P[np.arange(16), rng.choice(128, 16, replace=False)] = 1.0
    s32, _ = O.index_logits(q, k, P, 1.0)
    s16, _ = O.index_logits(q, k, P, 1.0, index_bf16=True)
    np.testing.assert_array_equal(s16, s32)
    np.testing.assert_array_equal(O.index_keys(k, P, True), k @ P.T)


def test_bf16_index_brute_force():
    """Scalar loop: k~_j = bf16(sum_t P[j,t] k[t]) (fp64 sum, one rounding)
    and s = q~ . k~ with q~ unrounded; torch's cast does the rounding."""
    rng = np.random.default_rng(72)
    q, k, P = rng.standard_normal((2, 128)), rng.standard_normal((5, 128)), rng.standard_normal((16, 128)) / 11
    s, _ = O.index_logits(q, k, P, 1.0, index_bf16=True)
    for i in range(5):
        kt = [float(torch.tensor(sum(P[j, t] * k[i, t] for t in range(128)), dtype=torch.float64)
                    .to(torch.bfloat16).to(torch.float64)) for j in range(16)]
        for g in range(2):
            qt = [sum(P[j, t] * q[g, t] for t in range(128)) for j in range(16)]
            assert abs(s[g, i] - sum(a * b for a, b in zip(qt, kt))) < 1e-9 * (1 + abs(s[g, i]))
    s32, _ = O.index_logits(q, k, P, 1.0)
    assert not np.array_equal(s, s32)              # the rounding is really applied


def test_full_scores_brute_force():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((2, 128)), rng.standard_normal((5, 128))
    s, l = O.full_logits(q, k, 0.125)
    for g in range(2):
        for i in range(5):
            ref = sum(q[g, t] * k[i, t] for t in range(128))
            assert abs(s[g, i] - ref) < 1e-10 and abs(l[g, i] - 0.125 * ref) < 1e-10


# ---------------------------------------------------------------- aggregate

def test_group_aggregate_invariants():
    rng = np.random.default_rng(9)
    l = rng.standard_normal((4, 300)) * 3
    a = O.group_aggregate(l)
    assert abs(a.sum() - 1.0) < 1e-12 and (a > 0).all()
    # shift of one head's logits leaves it unchanged
    l2 = l.copy()
    l2[2] += 17.0
    np.testing.assert_allclose(O.group_aggregate(l2), a, rtol=1e-12)
    # G = 1 is the plain softmax (library routine)
    np.testing.assert_allclose(O.group_aggregate(l[:1]), scipy.special.softmax(l[0]), rtol=1e-12)
    # mean of the per-head softmaxes, not softmax of the mean logits
    ref = np.mean([scipy.special.softmax(l[g]) for g in range(4)], axis=0)
    np.testing.assert_allclose(a, ref, rtol=1e-12)


# ---------------------------------------------------------------- top-p

def _brute_top_p(a, p):
    """Smallest subset with mass >= p; among those, the one with the most mass."""
    n = a.size
    for size in range(1, n + 1):
        best, best_mass = None, -1.0
        for sub in itertools.combinations(range(n), size):
            m = a[list(sub)].sum()
            if m >= p and m > best_mass:
                best, best_mass = sub, m
        if best is not None:
            return np.array(best)
    return np.arange(n)


@pytest.mark.parametrize("seed", range(12))
def test_top_p_brute_force_small(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 11))
    a = scipy.special.softmax(rng.standard_normal(n) * 2)
    for p in (0.05, 0.3, 0.5, 0.77, 0.9, 0.99):
        S, t = O.select_top_p(a, p)
        np.testing.assert_array_equal(S, _brute_top_p(a, p))
        assert a[S].sum() >= p and t == a[S].min()


def test_top_p_two_level_closed_form():
    # m tokens at logit A, the rest at 0: S is exactly the m tokens iff
    # m e^A / (m e^A + n - m) >= p (else the tie rule keeps everything).
    with open(os.path.join(GOLDEN, "top_p_two_level.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        n, m, A, p = c["n"], c["m"], c["A"], c["p"]
        logits = np.zeros((1, n))
        hot = np.array(c["hot"])
        logits[0, hot] = A
        S, _ = O.select_top_p(O.group_aggregate(logits), p)
        want = hot if c["expect"] == "hot" else np.arange(n)
        np.testing.assert_array_equal(S, np.sort(want))
        closed = m * np.exp(A) / (m * np.exp(A) + n - m) >= p
        assert closed == (c["expect"] == "hot")


def test_top_p_special_cases_and_nesting():
    a = np.full(10, 0.1)
    assert O.select_top_p(a, 0.35)[0].size == 10            # all-equal: tie rule keeps all
    rng = np.random.default_rng(11)
    a = scipy.special.softmax(rng.standard_normal(500) * 2)
    assert O.select_top_p(a, 1.0)[0].size == 500
    assert O.select_top_p(a, 1e-9)[0].tolist() == [int(np.argmax(a))]
    prev = set()
    for p in np.linspace(0.05, 0.999, 30):
        S, _ = O.select_top_p(a, p)
        assert prev <= set(S.tolist()) and a[S].sum() >= p
        # minimality: dropping the smallest kept value falls below p
        assert a[S].sum() - a[S].min() < p
        prev = set(S.tolist())


# ---------------------------------------------------------------- top-k

def test_top_k_matches_argpartition():
    rng = np.random.default_rng(12)
    a = rng.random(1000)
    for k in (1, 7, 100, 999):
        S, t = O.select_top_k(a, k)
        ref = np.sort(np.argpartition(-a, k - 1)[:k])
        np.testing.assert_array_equal(S, ref)
        assert t == np.sort(a)[::-1][k - 1]
    assert O.select_top_k(a, 1000)[0].size == 1000
    assert O.select_top_k(a, 5000)[0].size == 1000


def test_top_k_ties_lowest_position_and_nesting():
    a = np.array([0.1, 0.3, 0.3, 0.05, 0.3, 0.3, 0.2])
    np.testing.assert_array_equal(O.select_top_k(a, 2)[0], [1, 2])
    np.testing.assert_array_equal(O.select_top_k(a, 5)[0], [1, 2, 4, 5, 6])
    np.testing.assert_array_equal(O.select_top_k(np.full(6, 0.5), 3)[0], [0, 1, 2])
    rng = np.random.default_rng(13)
    a = rng.random(300)
    prev = set()
    for k in range(1, 300, 17):
        S = set(O.select_top_k(a, k)[0].tolist())
        assert prev <= S and len(S) == k
        prev = S


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1),
        torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1), scale=scale)
    return out[0, :, 0, :].numpy()


def test_attend_all_rows_is_dense_sdpa():
    rng = np.random.default_rng(14)
    q, k, v = rng.standard_normal((4, 128)), rng.standard_normal((333, 128)), rng.standard_normal((333, 128))
    o, lse = O.sparse_attend(q, k, v, 1 / np.sqrt(128))
    np.testing.assert_allclose(o, _sdpa(q, k, v, 1 / np.sqrt(128)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(q @ k.T / np.sqrt(128), axis=1), rtol=1e-13)


def test_attend_single_row_and_convex_hull():
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal((2, 128)), rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    o, _ = O.sparse_attend(q, k, v, 0.1)
    np.testing.assert_array_equal(o, np.repeat(v, 2, axis=0))
    k, v = rng.standard_normal((20, 128)), rng.standard_normal((20, 128))
    o, _ = O.sparse_attend(q, k, v, 0.1)
    assert (o <= v.max(axis=0) + 1e-12).all() and (o >= v.min(axis=0) - 1e-12).all()
    # permuting the rows changes nothing
    perm = rng.permutation(20)
    np.testing.assert_allclose(O.sparse_attend(q, k[perm], v[perm], 0.1)[0], o, rtol=1e-12, atol=1e-13)


def test_local_token_set_cases():
    np.testing.assert_array_equal(O.local_token_set(10, 4, 100), np.arange(10))      # w >= N
    np.testing.assert_array_equal(O.local_token_set(10, 0, 1), [9])
    np.testing.assert_array_equal(O.local_token_set(10, 4, 3), [0, 1, 2, 3, 7, 8, 9])
    np.testing.assert_array_equal(O.local_token_set(10, 4, 7), np.arange(10))        # overlap counted once
    np.testing.assert_array_equal(O.local_token_set(3, 4, 1), [0, 1, 2])


# ---------------------------------------------------------------- whole head

def _small_seq(n=600, G=4, seed=16):
    rng = np.random.default_rng(seed)
    q = W.bf16_rne(rng.standard_normal((2 * G, 128)).astype(np.float32))
    k = W.bf16_rne(rng.standard_normal((n, 2, 128)).astype(np.float32))
    v = W.bf16_rne(rng.standard_normal((n, 2, 128)).astype(np.float32))
    P = (rng.standard_normal((2, 16, 128)) / np.sqrt(128)).astype(np.float32)
    return q, k, v, P


@pytest.mark.parametrize("rope_theta", [0.0, 10000.0])
def test_decode_reductions_to_dense(rope_theta):
    """top-p = 1, top-k = N and window >= N all reduce to dense attention
    ([NHA] §2 item 3: a window covering the whole sequence is full attention)."""
    q, k, v, P = _small_seq()
    n = k.shape[0]
    sc = 1 / np.sqrt(128)
    for kw in (dict(kind="retrieval", select_mode="top_p", top_p=1.0),
               dict(kind="retrieval", select_mode="top_k", top_k=n),
               dict(kind="retrieval", select_mode="top_k", top_k=n, score_mode="full"),
               dict(kind="local", n_sink=4, window=n)):
        res = O.decode_sequence_ref(q, k, v, head_kinds=[kw["kind"]] * 2, proj=P,
                                    score_mode=kw.get("score_mode", "index"),
                                    select_mode=kw.get("select_mode", "top_p"),
                                    top_p=kw.get("top_p", 0.9), top_k=kw.get("top_k", 0),
                                    n_sink=kw.get("n_sink", 0), window=kw.get("window", 0),
                                    attn_scale=sc, index_scale=0.7, rope_theta=rope_theta)
        for h in range(2):
            qr = O.rope(q[4 * h:4 * h + 4].astype(np.float64), np.full(4, n - 1), rope_theta)
            kr = k[:, h].astype(np.float64)
            if rope_theta > 0:
                kr = O.bf16_round(O.rope(kr, np.arange(n), rope_theta))
            ref = _sdpa(qr, kr, v[:, h].astype(np.float64), sc)
            np.testing.assert_allclose(res[h]["o64"], ref, rtol=0, atol=1e-12)
            assert res[h]["S"].size == n


def test_local_sink_window_closed_form():
    q, k, v, P = _small_seq()
    n = k.shape[0]
    res = O.decode_sequence_ref(q, k, v, head_kinds=["local"] * 2, n_sink=0, window=1,
                                attn_scale=0.088)
    np.testing.assert_array_equal(res[1]["o64"], np.repeat(v[n - 1:n, 1].astype(np.float64), 4, 0))
    res = O.decode_sequence_ref(q, k, v, head_kinds=["local"] * 2, n_sink=3, window=5,
                                attn_scale=0.088)
    rows = [0, 1, 2] + list(range(n - 5, n))
    ref = _sdpa(q[:4].astype(np.float64), k[rows, 0].astype(np.float64), v[rows, 0].astype(np.float64), 0.088)
    np.testing.assert_allclose(res[0]["o64"], ref, atol=1e-12)


def test_needles_selected_full_dim_config1():
    wl = W.make_workload(1)
    s = wl.sequence(0)
    res = O.decode_sequence_ref(s.q, s.k, s.v, head_kinds=wl.head_kinds, proj=wl.projections(),
                                score_mode="full", select_mode="top_p", top_p=0.9,
                                attn_scale=wl.attn_scale, heads=[0])
    assert set(s.needles[0].tolist()) <= set(res[0]["S"].tolist())


def test_needle_recall_index_r16():
    """[RTPurbo] Methodology §2 claims >90 % recall with a 16-dim index: all 8
    needles on the tiny workload at seed 0, and >= 90 % over 20 seeds."""
    hits = total = 0
    for seed in range(20):
        wl = W.make_workload(1, seed=seed)
        s = wl.sequence(0)
        res = O.decode_sequence_ref(s.q, s.k, s.v, head_kinds=wl.head_kinds, proj=wl.projections(),
                                    top_p=0.9, attn_scale=wl.attn_scale,
                                    index_scale=wl.index_scale, heads=[0])
        got = np.isin(s.needles[0], res[0]["S"]).sum()
        if seed == 0:
            assert got == 8
        hits += got
        total += 8
    assert hits / total >= 0.9


def test_fp8_path_uses_dequantised_rows():
    q, k, v, P = _small_seq(n=40)
    res = O.decode_sequence_ref(q, k, v, head_kinds=["local"] * 2, n_sink=0, window=40,
                                attn_scale=0.088, kv_fp8=True)
    kd = O.fp8_store_rows(k[:, 0].astype(np.float64), [(0, 40)])[2]
    vd = O.fp8_store_rows(v[:, 0].astype(np.float64), [(0, 40)])[2]
    np.testing.assert_allclose(res[0]["o64"], _sdpa(q[:4].astype(np.float64), kd, vd, 0.088), atol=1e-12)


# -- per-query-head selection (scope "query") ----------------------------------

ATTN = 1.0 / np.sqrt(128)


def _qhead_case(G=4, n=300, seed=41, same_q=False):
    rng = np.random.default_rng(seed)
    q = O.bf16_round(rng.standard_normal((1 if same_q else G, 128)) * 1.5)
    q = np.repeat(q, G, axis=0) if same_q else q
    k = O.bf16_round(rng.standard_normal((n, 128)))
    v = O.bf16_round(rng.standard_normal((n, 128)))
    return q, k, v


@pytest.mark.parametrize("select_mode", ["top_p", "top_k"])
def test_query_scope_with_one_head_is_the_group_set(select_mode):
    """G = 1: the head's own distribution is the group aggregate."""
    q, k, v = _qhead_case(G=1)
    kw = dict(kind="retrieval", score_mode="full", select_mode=select_mode, top_p=0.8, top_k=37,
              attn_scale=ATTN)
    a = O.decode_head_ref(q, k, k, v, scope="kv", **kw)
    b = O.decode_head_ref(q, k, k, v, scope="query", **kw)
    np.testing.assert_array_equal(a["S"], b["S_heads"][0])
    np.testing.assert_array_equal(a["o64"], b["o64"])


def test_query_scope_identical_heads_share_the_group_set():
    """All G queries equal: every per-head distribution equals their mean."""
    q, k, v = _qhead_case(same_q=True)
    kw = dict(kind="retrieval", score_mode="full", select_mode="top_p", top_p=0.9, attn_scale=ATTN)
    a = O.decode_head_ref(q, k, k, v, scope="kv", **kw)
    b = O.decode_head_ref(q, k, k, v, scope="query", **kw)
    for g in range(4):
        np.testing.assert_array_equal(b["S_heads"][g], a["S"])
    np.testing.assert_allclose(b["o64"], a["o64"], rtol=0, atol=1e-12)


def test_query_scope_heads_are_independent():
    """Changing one query head changes no other head's set or output (a group
    aggregate anywhere would couple them)."""
    q, k, v = _qhead_case()
    kw = dict(kind="retrieval", score_mode="full", select_mode="top_p", top_p=0.9, attn_scale=ATTN,
              scope="query")
    a = O.decode_head_ref(q, k, k, v, **kw)
    q2 = q.copy()
    q2[2] = O.bf16_round(np.random.default_rng(5).standard_normal(128) * 3)
    b = O.decode_head_ref(q2, k, k, v, **kw)
    for g in (0, 1, 3):
        np.testing.assert_array_equal(a["S_heads"][g], b["S_heads"][g])
        np.testing.assert_array_equal(a["o64"][g], b["o64"][g])
    assert not np.array_equal(a["S_heads"][2], b["S_heads"][2])
    np.testing.assert_array_equal(a["S"], np.unique(np.concatenate(a["S_heads"])))


def test_query_scope_brute_force_and_dense():
    """Each head's set is the brute-force minimal top-p subset of its own
    softmax (tiny N); p = 1 gives dense attention per head (torch SDPA)."""
    rng = np.random.default_rng(77)
    n = 9
    q = O.bf16_round(rng.standard_normal((4, 128)) * 2)
    k = O.bf16_round(rng.standard_normal((n, 128)))
    v = O.bf16_round(rng.standard_normal((n, 128)))
    r = O.decode_head_ref(q, k, k, v, kind="retrieval", score_mode="full", select_mode="top_p",
                          top_p=0.7, attn_scale=ATTN, scope="query")
    z = ATTN * (q.astype(np.float64) @ k.astype(np.float64).T)
    for g in range(4):
        pi = scipy.special.softmax(z[g])
        np.testing.assert_array_equal(r["S_heads"][g], np.sort(_brute_top_p(pi, 0.7)))
    d = O.decode_head_ref(q, k, k, v, kind="retrieval", score_mode="full", select_mode="top_p",
                          top_p=1.0, attn_scale=ATTN, scope="query")
    np.testing.assert_allclose(d["o64"], _sdpa(q, k, v, ATTN), rtol=0, atol=1e-6)


# -- retained-mass diagnostics ([RTPurbo] Main results: attention mass kept) ----

def _two_level_mass_case(n=200, m=8):
    """Keys that give two-level logits, different in the index and in full dim.

    P selects dims 0..15 (index_scale 1) and attention uses attn_scale 1.
    Query head g = c_g e0 + f_g e20 with c = (1, 2), f = (1, 0); the m needle
    keys (positions 10, 20, ...) are 3 e0, the other keys 2 e20.  Index logits:
    3 c_g for needles, 0 otherwise; full-dim logits: 3 c_g for needles, 2 f_g
    otherwise (e20 lies outside the index's span)."""
    q = np.zeros((2, 128))
    q[0, 0], q[0, 20] = 1.0, 1.0
    q[1, 0] = 2.0
    k = np.zeros((n, 128))
    k[:, 20] = 2.0
    needles = np.arange(1, m + 1) * 10
    k[needles] = 0.0
    k[needles, 0] = 3.0
    P = np.zeros((16, 128))
    P[np.arange(16), np.arange(16)] = 1.0
    v = O.bf16_round(np.random.default_rng(9).standard_normal((n, 128)))
    return q, k, v, P, needles


def test_retained_mass_two_level_closed_form():
    """S = the needles.  Index mass = mean_g m e^{3c_g} / (m e^{3c_g} + n - m);
    full-dim mass = mean_g m e^{3c_g} / (m e^{3c_g} + (n - m) e^{2 f_g}).  A mass
    taken from the wrong logits, a softmax of the mean logits, or a mean over
    the wrong axis each gives another number."""
    n, m = 200, 8
    q, k, v, P, needles = _two_level_mass_case(n, m)
    r = O.decode_head_ref(q, k, k, v, kind="retrieval", proj=P, score_mode="index", select_mode="top_p",
                          top_p=0.6, attn_scale=1.0, index_scale=1.0, with_full_mass=True)
    np.testing.assert_array_equal(r["S"], needles)
    c, f = np.array([1.0, 2.0]), np.array([1.0, 0.0])
    idx = np.mean(m * np.exp(3 * c) / (m * np.exp(3 * c) + n - m))
    full = np.mean(m * np.exp(3 * c) / (m * np.exp(3 * c) + (n - m) * np.exp(2 * f)))
    assert abs(idx - 0.69973) < 1e-5 and abs(full - 0.52279) < 1e-5   # evaluated by hand
    np.testing.assert_allclose(r["index_mass"], idx, rtol=1e-12)
    np.testing.assert_allclose(r["full_mass"], full, rtol=1e-12)
    # per query head (scope "query", p = 0.4): head 0 keeps the needles
    # (7 of them hold only 0.399), head 1 reaches p after 4 and keeps their ties
    rq = O.decode_head_ref(q, k, k, v, kind="retrieval", proj=P, score_mode="index", select_mode="top_p",
                           top_p=0.4, attn_scale=1.0, index_scale=1.0, scope="query")
    for g in range(2):
        np.testing.assert_array_equal(rq["S_heads"][g], needles)
        np.testing.assert_allclose(rq["index_mass_heads"][g],
                                   m * np.exp(3 * c[g]) / (m * np.exp(3 * c[g]) + n - m), rtol=1e-12)


def test_retained_mass_all_tokens_and_local_heads():
    """p = 1 keeps every token: both masses are 1.  A local head over keys whose
    logit is A on its sinks and window and 0 elsewhere keeps
    |S| e^A / (|S| e^A + n - |S|) of the full-dim mass."""
    n = 300
    q, k, v, P, _ = _two_level_mass_case(n)
    r = O.decode_head_ref(q, k, k, v, kind="retrieval", proj=P, score_mode="index", select_mode="top_p",
                          top_p=1.0, attn_scale=1.0, index_scale=1.0, with_full_mass=True)
    assert r["S"].size == n
    np.testing.assert_allclose([r["index_mass"], r["full_mass"]], [1.0, 1.0], rtol=1e-12)
    n_sink, window, A = 4, 50, 1.5
    S = O.local_token_set(n, n_sink, window)
    assert S.size == n_sink + window
    ql = np.zeros((2, 128))
    ql[:, 0] = 1.0
    kl = np.zeros((n, 128))
    kl[S, 0] = A
    rl = O.decode_head_ref(ql, kl, kl, v, kind="local", n_sink=n_sink, window=window, attn_scale=1.0,
                           with_full_mass=True)
    L = S.size
    np.testing.assert_allclose(rl["full_mass"], L * np.exp(A) / (L * np.exp(A) + n - L), rtol=1e-12)
    assert rl["index_mass"] is None


# -- data-free head classification (effective rank) ------------------------------

def _weights_with_spectrum(sv, d_model, rng):
    """W_Q = U diag(sv) V^T (d_head x d_model) with W_K = [I 0]: M = W_K^T W_Q has
    singular values sv exactly."""
    d = len(sv)
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d_model, d)))
    wq = U @ np.diag(sv) @ V.T
    wk = np.zeros((d, d_model))
    wk[np.arange(d), np.arange(d)] = 1.0
    return wq, wk


def test_effective_rank_closed_forms():
    rng = np.random.default_rng(90)
    d_model = 160
    cases = [(np.ones(128), 128.0),                                  # flat spectrum: full rank
             (np.r_[1.0, np.zeros(127)], 1.0),                       # rank one
             (np.r_[2.0, 1.0, 1.0, np.zeros(125)], 2.0 ** 1.5),      # entropy of (1/2, 1/4, 1/4)
             (np.r_[np.ones(5), np.zeros(123)] * 7.0, 5.0)]          # scale-free
    for sv, expect in cases:
        wq, wk = _weights_with_spectrum(sv, d_model, rng)
        er = O.effective_rank(wq[None], wk[None])
        assert abs(er[0] - expect) < 1e-9 * expect, (er, expect)


def test_effective_rank_invariances_and_gqa():
    """Orthogonal changes of the model basis and a scale leave it unchanged;
    the query heads of a group share W_K; the Sylvester route (eigenvalues of
    (W_Q W_Q^T)(W_K W_K^T)) gives the same singular values."""
    rng = np.random.default_rng(91)
    d_model = 200
    wq = rng.standard_normal((4, 128, d_model)) * np.linspace(0.2, 3, 128)[None, :, None]
    wk = rng.standard_normal((2, 128, d_model))
    er = O.effective_rank(wq, wk)
    Q, _ = np.linalg.qr(rng.standard_normal((d_model, d_model)))
    np.testing.assert_allclose(O.effective_rank(wq @ Q, wk @ Q), er, rtol=1e-10)
    np.testing.assert_allclose(O.effective_rank(3.0 * wq, wk), er, rtol=1e-10)
    np.testing.assert_allclose(O.effective_rank(wq[2:], wk[1:]), er[2:], rtol=1e-12)
    for g in range(4):
        C = (wq[g] @ wq[g].T) @ (wk[g // 2] @ wk[g // 2].T)
        lam = np.sort(np.clip(np.linalg.eigvals(C).real, 0, None))[::-1]
        sv = np.sqrt(lam)
        s = sv / sv.sum()
        s = s[s > 0]
        assert abs(np.exp(-(s * np.log(s)).sum()) - er[g]) < 1e-8 * er[g]


# ---------------------------------------------------------------- prefill

def _prefill_seq(n=300, t=300, hq=8, hkv=2, seed=31):
    rng = np.random.default_rng(seed)
    q = W.bf16_rne(rng.standard_normal((t, hq, 128)).astype(np.float32))
    k = W.bf16_rne(rng.standard_normal((n, hkv, 128)).astype(np.float32))
    v = W.bf16_rne(rng.standard_normal((n, hkv, 128)).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("rope_theta", [0.0, 10000.0])
def test_prefill_dense_is_torch_causal_sdpa(rope_theta):
    """Every head dense from position 0: torch's causal attention (fp64, CPU)
    on the rotated queries and the stored keys."""
    q, k, v = _prefill_seq()
    n, G = k.shape[0], 4
    sc = 1 / np.sqrt(128)
    res = O.prefill_sequence_ref(q, k, v, head_kinds=["local", "retrieval"], start=0, n_sink=4,
                                 window=16, attn_scale=sc, rope_theta=rope_theta, dense_all=True)
    pos = np.arange(n)
    for h in range(2):
        kr = k[:, h].astype(np.float64)
        if rope_theta > 0:
            kr = O.bf16_round(O.rope(kr, pos, rope_theta))
        for g in range(G):
            qr = O.rope(q[:, h * G + g].astype(np.float64), pos, rope_theta)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qr)[None, None], torch.from_numpy(kr)[None, None],
                torch.from_numpy(v[:, h].astype(np.float64))[None, None], is_causal=True, scale=sc)
            np.testing.assert_allclose(res[h][0][:, g], ref[0, 0].numpy(), rtol=0, atol=1e-12)
            z = sc * (qr @ kr.T)
            z[np.triu_indices(n, 1)] = -np.inf
            np.testing.assert_allclose(res[h][1][:, g], scipy.special.logsumexp(z, axis=1), rtol=1e-13)


def test_prefill_local_mask_brute_force():
    for n_sink, window in ((4, 16), (0, 1), (3, 1), (20, 5), (0, 1000), (7, 0)):
        pos = np.arange(40, 90)
        m = O.prefill_mask(pos, 100, kind="local", n_sink=n_sink, window=window)
        for r, i in enumerate(pos):
            want = {j for j in range(100) if j <= i and (j < n_sink or i - j < window)}
            assert set(np.flatnonzero(m[r]).tolist()) == want
            np.testing.assert_array_equal(np.flatnonzero(m[r]), O.local_token_set(i + 1, n_sink, window))
        full = O.prefill_mask(pos, 100, kind="retrieval", n_sink=n_sink, window=window)
        np.testing.assert_array_equal(full, np.arange(100)[None, :] <= pos[:, None])


@pytest.mark.parametrize("rope_theta,kv_fp8", [(0.0, False), (10000.0, False), (0.0, True)])
def test_prefill_rows_are_decode_steps(rope_theta, kv_fp8):
    """Row i of a chunk is the decode of the prefix 0..i: dense for a
    retrieval head (top-p = 1 keeps every token), sinks + window for a local
    head (both pinned separately above); with fp8 storage both read the rows
    the append calls stored (the decode's fp8 path is pinned above)."""
    q, k, v = _prefill_seq(n=500, t=120)
    start = 380
    rows = [0, 1, 57, 118, 119]
    sc = 1 / np.sqrt(128)
    segs = [(0, 380), (380, 120)]
    res = O.prefill_sequence_ref(q, k, v, head_kinds=["retrieval", "local"], start=start, n_sink=4,
                                 window=64, attn_scale=sc, rope_theta=rope_theta, rows=rows,
                                 kv_fp8=kv_fp8, segments=segs)
    n = k.shape[0]
    # the rows the cache holds after the appends (fp8: page scales set by the
    # call that writes slot 0 of the page, over every row it writes there)
    store = {h: (O.stored_rows(k[:, h], np.arange(n), rope_theta=rope_theta, kv_fp8=kv_fp8, segments=segs,
                               rotate=True),
                 O.stored_rows(v[:, h], np.arange(n), rope_theta=rope_theta, kv_fp8=kv_fp8, segments=segs,
                               rotate=False)) for h in range(2)}
    for r, t in enumerate(rows):
        i = start + t
        for h, kind in enumerate(["retrieval", "local"]):
            dec = O.decode_head_ref(q[t, 4 * h:4 * h + 4], k[:i + 1, h], store[h][0][:i + 1], store[h][1][:i + 1],
                                    kind=kind, score_mode="full", select_mode="top_p", top_p=1.0, n_sink=4,
                                    window=64, attn_scale=sc, rope_theta=rope_theta)
            np.testing.assert_allclose(res[h][0][r], dec["o64"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(res[h][1][r], dec["lse64"], rtol=1e-13)


def test_prefill_closed_forms():
    q, k, v = _prefill_seq(n=200, t=200)
    v_const = np.broadcast_to(np.linspace(-1, 1, 128), v.shape).copy()
    res = O.prefill_sequence_ref(q, k, v_const, head_kinds=["retrieval", "local"], start=0, n_sink=2,
                                 window=9, attn_scale=0.09)
    for h in range(2):
        np.testing.assert_allclose(res[h][0], np.broadcast_to(v_const[0, 0], res[h][0].shape), atol=1e-13)
    # position 0 sees only itself: o = v_0, lse = z_00
    res = O.prefill_sequence_ref(q, k, v, head_kinds=["local", "retrieval"], start=0, n_sink=0,
                                 window=3, attn_scale=0.09, rows=[0])
    for h in range(2):
        np.testing.assert_array_equal(res[h][0][0], np.repeat(v[0:1, h].astype(np.float64), 4, 0))
        np.testing.assert_allclose(res[h][1][0], 0.09 * q[0, 4 * h:4 * h + 4].astype(np.float64)
                                   @ k[0, h].astype(np.float64), rtol=0, atol=1e-13)
    # a window that covers everything makes a local head a retrieval head
    a = O.prefill_sequence_ref(q, k, v, head_kinds=["local", "local"], start=0, n_sink=0, window=200,
                               attn_scale=0.09)
    b = O.prefill_sequence_ref(q, k, v, head_kinds=["retrieval", "retrieval"], start=0, n_sink=0,
                               window=1, attn_scale=0.09)
    for h in range(2):
        np.testing.assert_array_equal(a[h][0], b[h][0])
