"""Float64 NumPy oracle: the plain definition of one head-wise sparse decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): no blocking, no
splits, no histograms.  Every step is the textbook definition written out,
with library primitives (matmul, sort, cumsum) as the only helpers.

Notation (per sequence b and KV head h with its G query heads):
  N        context length, including the token appended this step
  q_g      pre-RoPE query of query head g, k_i / v_i key / value of token i
  P_h      r x d index projection of a retrieval head (r = 16)
  l_{g,i}  selection logit, a_i the group aggregate, S the selected set

Readings of points the pages leave open are marked "reading:" and are listed
with their reasons in the design notes of the repository.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0          # largest finite OCP e4m3fn value
BLOCK = 16                # tokens per KV page


# ---------------------------------------------------------------------------
# Storage encodings (inputs are bf16; config 5 stores K/V as fp8 e4m3fn)
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bf16 keeps 8 significant bits: with x = m * 2**e, m in [0.5, 1), the
    spacing of bf16 numbers around x is 2**(e - 8), and ``np.rint`` rounds the
    exactly scaled quotient half-to-even.
    reading: rotated keys are stored as bf16, so the oracle rounds them once.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)               # bf16 subnormal spacing floor
    ulp = np.ldexp(1.0, e - 8)
    return np.rint(x / ulp) * ulp


def e4m3_table() -> np.ndarray:
    """Values of all 256 OCP e4m3fn codes (NaN for 0x7F / 0xFF).

    Layout: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    Exponent field 0 is subnormal: (m/8) * 2**-6.  There is no infinity;
    S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2**8 = 448.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        ex = (code >> 3) & 0xF
        man = code & 0x7
        if ex == 0xF and man == 0x7:
            vals[code] = np.nan
        elif ex == 0:
            vals[code] = sign * (man / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (ex - 7)
    return vals


_E4M3 = e4m3_table()
_E4M3_POS = _E4M3[:127]                   # codes 0..126: 0 .. 448, increasing


def e4m3_encode(y) -> np.ndarray:
    """Encode real values as e4m3fn codes: saturate to +-448, round to nearest,
    ties to the even code (mantissa LSB 0).  The sign bit is copied from ``y``
    (so -0.0 and negatives that round to zero give 0x80).

    reading: the KV fp8 format is OCP e4m3fn with saturating conversion.
    """
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")      # first value >= mag
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def fp8_store_rows(x, segments, block: int = BLOCK):
    """Quantise one head's rows the way a paged fp8 cache stores them.

    ``x``: [N, d] values (bf16-exact).  ``segments``: the append calls that
    wrote positions [start, start + n), in call order.

    reading: one fp32 scale per (block, head, K|V).  When an append call
    writes slot 0 of a block, that block's scale becomes amax/448 over the
    rows this call writes into it (1.0 if they are all zero); later appends
    into the open block keep the scale and saturate.  The encoded quantity is
    the fp32 quotient x / scale (both operands fp32, correctly rounded).
    Returns (codes [N, d] uint8, scales {block: float32}, dequantised float64).
    """
    x = np.asarray(x, dtype=np.float64)
    n_tok, d = x.shape
    codes = np.zeros((n_tok, d), dtype=np.uint8)
    scales: dict[int, np.float32] = {}
    for start, n in segments:
        end = start + n
        for blk in range(start // block, (end - 1) // block + 1):
            lo = max(start, blk * block)
            hi = min(end, (blk + 1) * block)
            rows = x[lo:hi].astype(np.float32)
            if lo == blk * block:
                amax = np.float32(np.max(np.abs(rows)))
                scales[blk] = (np.float32(amax) / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
            scale = scales[blk]
            quot = (rows / np.float32(scale)).astype(np.float32)
            codes[lo:hi] = e4m3_encode(quot.astype(np.float64))
    deq = np.empty((n_tok, d), dtype=np.float64)
    for blk, scale in scales.items():
        lo, hi = blk * block, min(n_tok, (blk + 1) * block)
        deq[lo:hi] = e4m3_decode(codes[lo:hi]) * np.float64(scale)
    return codes, scales, deq


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing (j, j + d/2).

    reading: the pages only say the index is taken before RoPE ([RTPurbo]
    Methodology §2); the convention is the common one with angle
    pos * theta**(-2j/d) for pair j.  ``theta <= 0`` means RoPE off.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    inv = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def stored_rows(x_pre, positions, *, rope_theta: float, kv_fp8: bool, segments, rotate: bool):
    """What the cache holds for one head's K (rotate=True) or V rows, as float64.

    K: rotated (if RoPE is on) then rounded to bf16; V: the bf16 input.  With
    fp8 storage the bf16 rows are then quantised by ``fp8_store_rows``.
    """
    x = np.asarray(x_pre, dtype=np.float64)
    if rotate and rope_theta > 0:
        x = bf16_round(rope(x, positions, rope_theta))
    if kv_fp8:
        return fp8_store_rows(x, segments)[2]
    return x


# ---------------------------------------------------------------------------
# Selection scores  ([RTPurbo] Methodology §2; [ICS] §2 "Oracle top-k")
# ---------------------------------------------------------------------------

def index_keys(k_pre, proj, index_bf16: bool = False) -> np.ndarray:
    """The stored index k~ = P k of every token ([RTPurbo] Methodology §2).

    reading: fp32 storage keeps P k as computed; a bf16 index (32 B per
    token instead of 64) holds P k evaluated in fp64 and rounded once to bf16.
    """
    kt = np.asarray(k_pre, dtype=np.float64) @ np.asarray(proj, dtype=np.float64).T
    return bf16_round(kt) if index_bf16 else kt


def index_logits(q_pre, k_pre, proj, index_scale: float, index_bf16: bool = False):
    """Low-dim pre-RoPE index: q~ = P q, k~ = P k, s = q~ . k~.

    [RTPurbo] Methodology §2: a projection to r = 16 dims is applied to the
    query and key features before RoPE and relevance is estimated there.
    reading: one fp32 projection per retrieval KV head, shared by q and k and
    by the group's query heads; the logit is index_scale * s.  With a bf16
    index the stored k~ is rounded to bf16 (index_keys); q~ is not stored.
    Returns (s [G, N], logits [G, N]).
    """
    P = np.asarray(proj, dtype=np.float64)
    qt = np.asarray(q_pre, dtype=np.float64) @ P.T
    kt = index_keys(k_pre, proj, index_bf16)
    s = qt @ kt.T
    return s, index_scale * s


def full_logits(q_rot, k_rot, attn_scale: float):
    """Full-dim scores q . k used by oracle top-k ([ICS] §2, "Oracle Top-K")."""
    s = np.asarray(q_rot, dtype=np.float64) @ np.asarray(k_rot, dtype=np.float64).T
    return s, attn_scale * s


def head_probs(logits) -> np.ndarray:
    """pi_{g,i} = softmax_i(l_g) for each query head g (rows of the result)."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def group_aggregate(logits) -> np.ndarray:
    """a_i = mean over the group's query heads of softmax_i(l_g).

    reading: one token set per (sequence, KV head), shared by its G query
    heads; the per-head attention distributions are averaged (mean pooling to
    the GQA group, [AoH] Methodology §4), which keeps sum(a) = 1 so that a
    cumulative-mass threshold keeps its meaning.
    """
    return head_probs(logits).mean(axis=0)


def _desc_order(a) -> np.ndarray:
    """Token order by value descending, ties by position ascending."""
    a = np.asarray(a, dtype=np.float64)
    return np.lexsort((np.arange(a.size), -a))


def select_top_p(a, p: float):
    """Dynamic top-p set ([RTPurbo] Methodology §3).

    Attention mass is accumulated from the largest value down until the
    cumulative sum reaches p; the budget therefore adapts to the query.
    reading: the minimal descending prefix whose sum is >= p ends at value
    t*; every token with a_i >= t* is kept (ties at t* included).  p >= 1
    keeps every token.  If rounding leaves the total short of p, every
    token is kept.
    Returns (S ascending int64, t*).
    """
    a = np.asarray(a, dtype=np.float64)
    n = a.size
    if p >= 1.0:
        return np.arange(n), float(a.min())
    order = _desc_order(a)
    c = np.cumsum(a[order])
    hit = np.nonzero(c >= p)[0]
    j = int(hit[0]) if hit.size else n - 1
    t = float(a[order[j]])
    return np.nonzero(a >= t)[0], t


def select_top_k(a, k: int):
    """Fixed-budget top-k set ([RTPurbo] Methodology §3; [ICS] §2).

    reading: t* is the k-th largest value; S holds every a_i > t* plus the
    lowest-position tokens with a_i == t* up to k in total.  k >= N keeps all.
    Returns (S ascending int64, t*).
    """
    a = np.asarray(a, dtype=np.float64)
    n = a.size
    if k >= n:
        return np.arange(n), float(a.min())
    order = _desc_order(a)
    return np.sort(order[:k]), float(a[order[k - 1]])


def local_token_set(n: int, n_sink: int, window: int) -> np.ndarray:
    """Attention-sink tokens plus the sliding window of a local head.

    [RTPurbo] Methodology §1 (local heads use a sliding window with attention
    sinks); [AoH] Methodology §4 (streaming heads keep the first tokens and a
    recent window).  reading: sinks are positions 0..n_sink-1, the window is
    the last `window` positions including the current token, and a position
    in both is counted once.
    """
    sinks = np.arange(min(n_sink, n))
    win = np.arange(max(0, n - window), n)
    return np.union1d(sinks, win).astype(np.int64)


# ---------------------------------------------------------------------------
# Attention over a token set  ([ICS] §3c: only the selected rows are read)
# ---------------------------------------------------------------------------

def sparse_attend(q_rot, k_rows, v_rows, attn_scale: float):
    """Softmax attention of G queries over the given rows only.

    o_g = sum_i softmax(z_g)_i v_i with z_{g,i} = attn_scale * q_g . k_i and
    the softmax renormalised over the rows given.  Returns (o [G, d], lse [G]).
    """
    q = np.asarray(q_rot, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    z = attn_scale * (q @ k.T)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ v) / l
    return o, (m + np.log(l))[:, 0]


# ---------------------------------------------------------------------------
# One (sequence, KV head) and one sequence
# ---------------------------------------------------------------------------

def decode_head_ref(q_pre, k_pre, k_store, v_store, *, kind: str, proj=None,
                    score_mode: str = "index", select_mode: str = "top_p",
                    top_p: float = 0.9, top_k: int = 0, n_sink: int = 0,
                    window: int = 0, attn_scale: float, index_scale: float = 1.0,
                    rope_theta: float = 0.0, fixed_set=None, with_full_mass: bool = False,
                    scope: str = "kv", index_bf16: bool = False):
    """Decode one step for one (sequence, KV head).

    q_pre [G, d] pre-RoPE queries; k_pre [N, d] pre-RoPE keys (the index
    input); k_store / v_store [N, d] the rows as the cache holds them (rotated
    and/or dequantised).  ``kind`` is "retrieval" or "local" ([RTPurbo]
    Methodology §1).  ``fixed_set`` replaces selection (used to evaluate the
    attention on a set chosen elsewhere).

    Returns a dict: o [G, d] float32, lse [G] float32, o64 / lse64 float64,
    S (ascending), t (threshold or None), scores (raw s, retrieval only),
    a (aggregate), index_mass, full_mass.

    scope "query" (retrieval heads): every query head g keeps its own set by
    the same rule applied to its own distribution softmax(l_g) and attends over
    that set only ([ICS] §2: the sparsity pattern differs per token, per query
    and per head; [RTPurbo] Methodology §3: the budget adapts per query).  The
    result then also holds S_heads, t_heads, a_heads and index_mass_heads (one
    entry per query head); S is their union.  ``fixed_set`` is then a list of
    G sets.
    """
    q_pre = np.asarray(q_pre, dtype=np.float64)
    n = k_store.shape[0]
    pos_q = n - 1
    q_rot = rope(q_pre, np.full(q_pre.shape[0], pos_q), rope_theta)
    out = {"t": None, "scores": None, "a": None, "index_mass": None}
    if kind == "retrieval" and scope == "query":
        if score_mode == "index":
            s, l = index_logits(q_pre, k_pre, proj, index_scale, index_bf16)
        else:
            s, l = full_logits(q_rot, k_store, attn_scale)
        pi = head_probs(l)
        sets, ts, o, lse = [], [], [], []
        for g in range(q_pre.shape[0]):
            if fixed_set is not None:
                S_g, t_g = np.asarray(fixed_set[g], dtype=np.int64), None
            elif select_mode == "top_p":
                S_g, t_g = select_top_p(pi[g], top_p)
            else:
                S_g, t_g = select_top_k(pi[g], top_k)
            o_g, lse_g = sparse_attend(q_rot[g:g + 1], k_store[S_g], v_store[S_g], attn_scale)
            sets.append(S_g)
            ts.append(t_g)
            o.append(o_g[0])
            lse.append(lse_g[0])
        o, lse = np.stack(o), np.asarray(lse)
        out.update(scores=s, a=None, a_heads=pi, S_heads=sets, t_heads=ts,
                   index_mass_heads=[float(pi[g][sets[g]].sum()) for g in range(len(sets))],
                   S=np.unique(np.concatenate(sets)), full_mass=None,
                   o64=o, lse64=lse, o=o.astype(np.float32), lse=lse.astype(np.float32))
        return out
    if kind == "retrieval":
        if score_mode == "index":
            s, l = index_logits(q_pre, k_pre, proj, index_scale, index_bf16)
        else:
            s, l = full_logits(q_rot, k_store, attn_scale)
        a = group_aggregate(l)
        out["scores"], out["a"] = s, a
        if fixed_set is not None:
            S = np.asarray(fixed_set, dtype=np.int64)
        elif select_mode == "top_p":
            S, out["t"] = select_top_p(a, top_p)
        else:
            S, out["t"] = select_top_k(a, top_k)
        out["index_mass"] = float(a[S].sum())
    else:
        S = local_token_set(n, n_sink, window) if fixed_set is None else np.asarray(fixed_set)
    o, lse = sparse_attend(q_rot, k_store[S], v_store[S], attn_scale)
    out["full_mass"] = None
    if with_full_mass:
        # Full-dim attention mass of the kept set, averaged over the group
        # (the "retained attention mass" diagnostic, [RTPurbo] Main results).
        _, zf = full_logits(q_rot, k_store, attn_scale)
        pf = np.exp(zf - zf.max(axis=1, keepdims=True))
        pf /= pf.sum(axis=1, keepdims=True)
        out["full_mass"] = float(pf[:, S].sum(axis=1).mean())
    out.update(S=S, o64=o, lse64=lse, o=o.astype(np.float32), lse=lse.astype(np.float32))
    return out


def decode_sequence_ref(q_pre, k_pre, v_in, *, head_kinds, proj=None, score_mode="index",
                        select_mode="top_p", top_p=0.9, top_k=0, n_sink=0, window=0,
                        attn_scale, index_scale=1.0, rope_theta=0.0, kv_fp8=False,
                        segments=None, heads=None, fixed_sets=None, with_full_mass=False, scope="kv",
                        index_bf16=False):
    """Decode one step of one sequence for the KV heads in ``heads``.

    q_pre [Hq, d]; k_pre, v_in [N, Hkv, d] as appended (bf16-exact values);
    head_kinds [Hkv] of "retrieval" / "local"; proj [Hkv, r, d];
    segments: the append calls [(start, n)] (default: one call of N tokens).
    Query head g belongs to KV head g // G.  Returns {h: decode_head_ref(...)}.
    """
    q_pre = np.asarray(q_pre, dtype=np.float64)
    n, hkv, _ = k_pre.shape
    G = q_pre.shape[0] // hkv
    segments = segments if segments is not None else [(0, n)]
    positions = np.arange(n)
    res = {}
    for h in (range(hkv) if heads is None else heads):
        kp = np.asarray(k_pre[:, h, :], dtype=np.float64)
        ks = stored_rows(kp, positions, rope_theta=rope_theta, kv_fp8=kv_fp8,
                         segments=segments, rotate=True)
        vs = stored_rows(v_in[:, h, :], positions, rope_theta=rope_theta, kv_fp8=kv_fp8,
                         segments=segments, rotate=False)
        res[h] = decode_head_ref(
            q_pre[h * G:(h + 1) * G], kp, ks, vs, kind=head_kinds[h],
            proj=None if proj is None else proj[h], score_mode=score_mode,
            select_mode=select_mode, top_p=top_p, top_k=top_k, n_sink=n_sink,
            window=window, attn_scale=attn_scale, index_scale=index_scale,
            rope_theta=rope_theta,
            fixed_set=None if fixed_sets is None else fixed_sets.get(h),
            with_full_mass=with_full_mass, scope=scope, index_bf16=index_bf16)
    return res


# ---------------------------------------------------------------------------
# Head-wise prefill  ([RTPurbo] Methodology §1 and Results; [AoH] Methodology §4)
# ---------------------------------------------------------------------------

def prefill_mask(positions, n_keys: int, *, kind: str, n_sink: int, window: int) -> np.ndarray:
    """Which keys each query position attends to during prefill: [T, n_keys] bool.

    Causal: query position i sees keys j <= i.  A retrieval head keeps all of
    them in the prefill phase ([RTPurbo] Methodology §1: retrieval heads keep
    the full KV cache during prefill, the sparse selection starts at decode);
    a local head keeps its sinks and its window ([RTPurbo] Methodology §1;
    [AoH] Methodology §4: streaming heads in chunked prefill).
    reading: the local set of query position i is the decode-time local set of
    a context of length i + 1, i.e. positions 0..n_sink-1 and i-window+1..i.
    """
    i = np.asarray(positions, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    m = j <= i
    if kind == "local":
        m &= (j < n_sink) | (j > i - window)
    return m


def prefill_sequence_ref(q_pre, k_pre, v_in, *, head_kinds, start: int, n_sink: int, window: int,
                         attn_scale: float, rope_theta: float = 0.0, heads=None, rows=None,
                         dense_all: bool = False, with_abs_v: bool = False, kv_fp8: bool = False,
                         segments=None):
    """Prefill attention of the query positions start..start+T-1 of one sequence.

    q_pre [T, Hq, d] pre-RoPE queries; k_pre, v_in [N, Hkv, d] the appended
    rows (bf16-exact, N >= start + T).  For KV head h and its query heads g:
    z = attn_scale * rope(q_g, i) . k_j over the stored keys (rotated, bf16, or
    the fp8-decoded rows of the append calls ``segments`` with ``kv_fp8``),
    masked by ``prefill_mask``; o = softmax(z) V and lse = log sum exp z, all
    in float64 as masked matrix products.  ``dense_all`` treats every head as a
    retrieval head (plain causal attention).  ``rows``: indices into the T
    positions to evaluate (default all).  Returns {h: (o [T', G, d], lse [T', G])},
    with ``with_abs_v`` also the softmax-weighted mean of |v| per output
    element (sum_j p_j |v_jd|, the scale of a relative error in the weights).
    """
    q_pre = np.asarray(q_pre, dtype=np.float64)
    T, hq, d = q_pre.shape
    n, hkv, _ = k_pre.shape
    G = hq // hkv
    sel = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = start + sel
    keys = np.arange(n)
    res = {}
    for h in (range(hkv) if heads is None else heads):
        segs = segments if segments is not None else [(0, n)]
        ks = stored_rows(k_pre[:, h, :], keys, rope_theta=rope_theta, kv_fp8=kv_fp8, segments=segs,
                         rotate=True)
        vs = stored_rows(v_in[:, h, :], keys, rope_theta=rope_theta, kv_fp8=kv_fp8, segments=segs,
                         rotate=False)
        kind = "retrieval" if dense_all else head_kinds[h]
        mask = prefill_mask(pos, n, kind=kind, n_sink=n_sink, window=window)      # [T', n]
        qr = rope(q_pre[sel, h * G:(h + 1) * G, :], pos[:, None], rope_theta)    # [T', G, d]
        z = attn_scale * (qr @ ks.T)                                             # [T', G, n]
        z = np.where(mask[:, None, :], z, -np.inf)
        m = z.max(axis=2, keepdims=True)
        w = np.exp(z - m)
        l = w.sum(axis=2, keepdims=True)
        res[h] = ((w @ vs) / l, (m + np.log(l))[:, :, 0])
        if with_abs_v:
            res[h] = res[h] + ((w @ np.abs(vs)) / l,)
    return res


# ---------------------------------------------------------------------------
# Data-free head classification  ([AoH] Methodology §1-§4)
# ---------------------------------------------------------------------------

def effective_rank(w_q, w_k) -> np.ndarray:
    """Effective rank of every query head's query-key kernel.

    [AoH] Methodology §1: the kernel of query head g (KV head h = g // G) is
    M_g = W_K^h^T W_Q^g (d_model x d_model), with W_Q^g, W_K^h the d_head x
    d_model projections.  §2: eff_rank = exp(-sum_k s_k log s_k) over its
    singular values normalised to sum 1 (reading: zero singular values add
    nothing, 0 log 0 = 0).  Computed here from the SVD of M_g itself (the
    plain definition); low values mark concentrated spectra (retrieval heads).
    w_q [Hq, d_head, d_model], w_k [Hkv, d_head, d_model].  Returns [Hq].
    """
    wq = np.asarray(w_q, dtype=np.float64)
    wk = np.asarray(w_k, dtype=np.float64)
    G = wq.shape[0] // wk.shape[0]
    er = np.empty(wq.shape[0])
    for g in range(wq.shape[0]):
        M = wk[g // G].T @ wq[g]
        sv = np.linalg.svd(M, compute_uv=False)
        s = sv / sv.sum()
        s = s[s > 0]
        er[g] = np.exp(-(s * np.log(s)).sum())
    return er
