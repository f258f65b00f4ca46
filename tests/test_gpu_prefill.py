"""GPU parity of the head-wise chunked prefill against the CPU oracle.

Tolerance (from the arithmetic of the kernel), per query row:
* logits: bf16 inputs with fp32 accumulation, as the decode scores, so each
  logit is within delta = 1e-5 * attn_scale * |q| * max_j |k_j| (the decode
  score bound in natural-log units); with RoPE the rotated query is split
  into two bf16 parts, which adds 2^-15 * attn_scale * |q| * max_j |k_j|;
* the weighted sum of V runs in fp16 with fp32 accumulation: each weight p
  in (0, 1] is rounded once to fp16 (within 2^-11 of p, relative: REL), V
  values are exact in fp16 (bf16 values of magnitude 2^-14 .. 65504; the
  workloads' values are far inside; a smaller one is off by at most 2^-25,
  inside the 1e-5 term), a logit error delta moves a normalised weight by at
  most 2 delta (relative), and the fp32 sums over n keys (one rounding per
  32-key MFMA step, plus the online rescales) add at most (n / 16 + 4) 2^-24
  (relative).  Hence per element
    |o_gpu - o_ref| <= (REL + 2 delta + (n / 16 + 4) 2^-24) * sum_j p_j |v_jd| + 1e-5,
  with p the oracle's weights (``with_abs_v``);
* lse (summed from the unrounded weights): within 2e-5 + delta;
* and, whatever that bound allows, max |o_gpu - o_ref| <= 2e-3 (the decode
  attention tolerance) on every row checked.
FP8 cache: the K products run on the e4m3 codes, exact in bf16, and the page
K scales multiply the logits in fp32; each V code is multiplied by its page's
V scale in fp32 and rounded to fp16 (2^-11 relative, inside REL for the same
reason as the weights' rounding: the bound below counts REL once per element,
so it takes 2^-10 for fp8 V), so the same bound holds with the stored
(decoded) rows in place of k and v.
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup, append_segments

pytestmark = pytest.mark.gpu

REL = 2.0 ** -11
REL_FP8 = 2.0 ** -10      # fp8 V: the code times its scale is rounded to fp16 too
ABS_CAP = 2e-3
WORST_ABS = {"out": 0.0}


def chunk_segments(n_tok):
    """The cache filled by one append of everything before the chunk, then
    one append of the chunk itself."""
    return lambda n: [(0, n - n_tok), (n - n_tok, n_tok)] if n > n_tok else [(0, n)]


def _run(wl, n_tok, *, dense=False, rows=None, q_fn=None, stride=1, segments=None, ring_slack=None):
    """ring_slack: keep the local heads in a ring with this slack."""
    wl.local_ring = ring_slack is not None
    print(f"\n[case] prefill {wl.name} B={wl.B} N={wl.seq_lens[:4]} n_tok={n_tok} G={wl.G} "
          f"window={wl.window} sinks={wl.n_sink} rope={wl.rope_theta} kv={wl.kv_dtype} dense={dense} "
          f"ring_slack={ring_slack}", flush=True)
    segments = segments or append_segments
    st = DecodeSetup(wl, keep_host=True, segments=segments, ring_slack=ring_slack or 0)
    starts = [wl.seq_lens[b] - n_tok for b in range(wl.B)]
    qh = np.stack([wl.prefill_queries(b, n_tok) for b in range(wl.B)])
    if q_fn is not None:
        qh = q_fn(st, qh, starts)
    q = torch.from_numpy(qh).to(torch.bfloat16).cuda()
    sp = torch.tensor(starts, dtype=torch.int32, device="cuda")
    out, lse = st.prefill(q, sp, dense=dense)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    G = wl.G
    rows = np.arange(0, n_tok, stride) if rows is None else np.asarray(rows)
    worst = worst_abs = 0.0
    for b in range(wl.B):
        n = wl.seq_lens[b]
        seq = st.host[b]
        # rows as the cache holds them: fp8 pages, or bf16 for local heads in the ring
        ref = {}
        for heads, fp8 in (([h for h in range(wl.Hkv) if not (st.ring and wl.head_kinds[h] == "local")], st.fp8),
                           ([h for h in range(wl.Hkv) if st.ring and wl.head_kinds[h] == "local"], False)):
            if heads:
                ref.update(O.prefill_sequence_ref(
                    qh[b], seq.k[:n], seq.v[:n], head_kinds=wl.head_kinds, start=starts[b], n_sink=wl.n_sink,
                    window=wl.window, attn_scale=wl.attn_scale, rope_theta=wl.rope_theta, heads=heads, rows=rows,
                    dense_all=dense, with_abs_v=True, kv_fp8=fp8, segments=segments(n)))
        for h in range(wl.Hkv):
            o_ref, lse_ref, absv = ref[h]
            qn = np.linalg.norm(qh[b, rows, h * G:(h + 1) * G].astype(np.float64), axis=2)     # [T', G]
            kmax = float(np.linalg.norm(seq.k[:n, h].astype(np.float64), axis=1).max())
            if st.fp8:                                  # stored rows: within one e4m3 step (2^-3) of k
                kmax *= 1.125
            delta = (1e-5 + (2.0 ** -15 if wl.rope_theta > 0 else 0.0)) * wl.attn_scale * qn * kmax
            o_gpu = out[b, rows, h * G:(h + 1) * G].astype(np.float64)
            err = np.abs(o_gpu - o_ref)
            acc = (n / 16 + 4) * 2.0 ** -24
            fp8_rows = st.fp8 and not (st.ring and wl.head_kinds[h] == "local")
            bound = ((REL_FP8 if fp8_rows else REL) + acc + 2 * delta[:, :, None]) * absv + 1e-5
            ratio = float((err / bound).max())
            worst = max(worst, ratio)
            worst_abs = max(worst_abs, float(err.max()))
            assert ratio <= 1.0, f"output off at (b={b}, h={h}): {ratio:.3f} x tolerance"
            assert float(err.max()) <= ABS_CAP, f"output off at (b={b}, h={h}): {float(err.max())} > {ABS_CAP}"
            el = np.abs(lse[b, rows, h * G:(h + 1) * G] - lse_ref)
            assert (el <= 2e-5 + delta).all(), f"lse off at (b={b}, h={h}): {float(el.max())}"
    WORST_ABS["out"] = max(WORST_ABS["out"], worst_abs)
    print(f"[ok] worst error / tolerance = {worst:.3f}, max |o - o_ref| = {worst_abs:.3g} "
          f"(largest so far {WORST_ABS['out']:.3g})", flush=True)
    return st, out, lse


@pytest.mark.parametrize("n", [1, 17, 64, 65, 200, 259, 700, 1500])
def test_prefill_whole_sequence(n):
    """Chunks from position 0: partial query tiles, tiles across the window's
    lower edge (window 256), the sink tile, a single position."""
    _run(W.make_workload(1, n=n, extra={"needle_range": (0, None)}), n)


@pytest.mark.parametrize("n_tok", [1, 33, 300])
def test_prefill_chunk_at_offset(n_tok):
    _run(W.make_workload(1, n=3000), n_tok)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (16, 2)])
def test_prefill_group_sizes(hq, hkv):
    _run(W.make_workload(1, n=900, Hq=hq, Hkv=hkv), 900)


@pytest.mark.parametrize("n_tok", [700, 129])
def test_prefill_rope(n_tok):
    _run(W.make_workload(1, n=700, rope_theta=10000.0), n_tok)


def test_prefill_dense_every_head():
    _run(W.make_workload(1, n=1000), 1000, dense=True)


def test_prefill_layer_shape_sampled_rows():
    """32 query / 8 KV heads, 2 retrieval + 6 local heads, window 1024."""
    wl = W.make_workload(2, n=2600, batch=2)
    _run(wl, 2600, stride=13)


def test_prefill_layer_shape_benched_length_sampled_rows():
    """The benched prefill: one 32768-position chunk from position 0 of the 8B
    layer shape, on 48 sampled query positions (the first and last, the
    window's lower edge, and a seeded spread)."""
    n = 32768
    wl = W.make_workload(2, n=n, batch=1)
    rng = np.random.default_rng(np.random.SeedSequence([2, 0, 6000]))
    rows = np.unique(np.concatenate([[0, 1, 3, 4, 1023, 1024, 1025, n - 2, n - 1],
                                     rng.choice(n, size=39, replace=False)]))
    _run(wl, n, rows=rows)


def test_prefill_ragged_batch_offsets():
    wl = W.make_workload(2, n=2000, batch=3)
    wl.seq_lens = [900, 1300, 2000]
    _run(wl, 500)


def test_prefill_peaky_queries():
    """Queries aimed at one earlier key (4x its direction): one weight near 1,
    which rounds exactly, and many tiny ones."""
    def aim(st, qh, starts):
        rng = np.random.default_rng(5)
        wl = st.wl
        for b in range(wl.B):
            for t in range(qh.shape[1]):
                i = starts[b] + t
                for hq in range(wl.Hq):
                    h = hq // wl.G
                    lo = max(0, i - wl.window + 1) if wl.head_kinds[h] == "local" else 0
                    j = int(rng.integers(lo, i + 1))
                    qh[b, t, hq] = W.bf16_rne((4.0 * st.host[b].k[j, h]).astype(np.float32))
        return qh
    _run(W.make_workload(1, n=800), 400, q_fn=aim)


@pytest.mark.parametrize("n_tok", [500, 1])
def test_prefill_fp8_ragged_chunks(n_tok):
    """FP8 cache with per-page scales: the chunk appended on its own (its
    first page shared with the previous append), ragged offsets, 2 retrieval
    + 6 local heads."""
    wl = W.make_workload(5, n=2000, batch=3)
    wl.seq_lens = [700, 1301, 2000]
    _run(wl, n_tok, segments=chunk_segments(n_tok))


def test_prefill_fp8_whole_sequence_rope_and_dense():
    _run(W.make_workload(1, n=1100, kv_dtype="fp8", rope_theta=10000.0), 1100)
    _run(W.make_workload(1, n=900, kv_dtype="fp8"), 900, dense=True)


@pytest.mark.parametrize("n,n_tok,slack", [(700, 700, 699), (3000, 300, 299), (3000, 300, 1000),
                                           (3000, 1, 0), (70, 70, 69)])
def test_prefill_ring(n, n_tok, slack):
    """Local heads read their rows from the ring (sinks in their own rows, the
    rest cycling through window + slack rows), which still holds every row a
    chunk of up to slack + 1 positions needs, after wrapping many times."""
    _run(W.make_workload(1, n=n), n_tok, ring_slack=slack)


@pytest.mark.parametrize("n_sink,window,slack,n_tok", [(70, 100, 150, 151), (0, 300, 63, 64), (5, 0, 0, 1),
                                                        (200, 64, 20, 21)])
def test_prefill_ring_geometry_edges(n_sink, window, slack, n_tok):
    """Sinks over one 64-key tile (two sink tiles, 128 sink rows), no sinks,
    sinks only (no cycling rows), and sinks longer than the window."""
    wl = W.make_workload(1, n=1500, n_sink=n_sink, window=window, extra={"needle_range": (0, None)})
    _run(wl, n_tok, ring_slack=slack)


def test_prefill_ring_with_fp8_pages():
    """fp8 pages (retrieval heads) and the bf16 ring (local heads): two
    launches of the kernel, one per row type."""
    wl = W.make_workload(5, n=2000, batch=3)
    wl.seq_lens = [700, 1301, 2000]
    _run(wl, 400, segments=chunk_segments(400), ring_slack=399)


def test_prefill_ring_chunks_in_order():
    """Chunked prefill as a server runs it: append a chunk, prefill it, append
    the next.  The cache is rebuilt up to each chunk's end by appending the
    prefix again (every ring row is rewritten, so the ring is as a fresh
    append leaves it)."""
    wl = W.make_workload(2, n=2600, batch=2)
    n_tok, G = 500, wl.G
    wl.local_ring = True
    st = DecodeSetup(wl, keep_host=True, ring_slack=n_tok - 1, segments=chunk_segments(100))
    for e in (500, 1500, 2600):
        for b in range(wl.B):
            seq = st.host[b]
            k = torch.from_numpy(seq.k[:e]).to(torch.bfloat16).cuda()[None]
            v = torch.from_numpy(seq.v[:e]).to(torch.bfloat16).cuda()[None]
            for a in range(0, e, n_tok):
                c = min(n_tok, e - a)
                st.ctx.append(st.block_tables[b:b + 1], torch.tensor([a], dtype=torch.int32, device="cuda"),
                              k[:, a:a + c].contiguous(), v[:, a:a + c].contiguous(),
                              seq_slots=st.seq_slots[b:b + 1])
        t0 = e - min(n_tok, e)
        nt = e - t0
        print(f"[case] ring chunk [{t0}, {e})", flush=True)
        qh = np.stack([wl.prefill_queries(b, nt) for b in range(wl.B)])
        q = torch.from_numpy(qh).to(torch.bfloat16).cuda()
        out, lse = st.prefill(q, torch.full((wl.B,), t0, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        rows = np.arange(0, nt, 7)
        for b in range(wl.B):
            seq = st.host[b]
            ref = O.prefill_sequence_ref(qh[b], seq.k[:e], seq.v[:e], head_kinds=wl.head_kinds, start=t0,
                                         n_sink=wl.n_sink, window=wl.window, attn_scale=wl.attn_scale,
                                         rows=rows, with_abs_v=True)
            for h in range(wl.Hkv):
                o_ref, lse_ref, absv = ref[h]
                qn = np.linalg.norm(qh[b, rows, h * G:(h + 1) * G].astype(np.float64), axis=2)
                kmax = float(np.linalg.norm(seq.k[:e, h].astype(np.float64), axis=1).max())
                delta = 1e-5 * wl.attn_scale * qn * kmax
                err = np.abs(out[b, rows, h * G:(h + 1) * G].astype(np.float64) - o_ref)
                assert (err <= (REL + 2 * delta[:, :, None]) * absv + 1e-5).all(), (e, b, h)
                assert (np.abs(lse[b, rows, h * G:(h + 1) * G] - lse_ref) <= 2e-5 + delta).all(), (e, b, h)


def test_prefill_ring_slot_out_of_range_reads_nothing():
    wl = W.make_workload(2, n=600, batch=2)
    wl.local_ring = True
    st = DecodeSetup(wl, ring_slack=99)
    q = torch.from_numpy(np.stack([wl.prefill_queries(b, 100) for b in range(2)])).to(torch.bfloat16).cuda()
    sp = torch.tensor([500, 500], dtype=torch.int32, device="cuda")
    good, lgood = st.prefill(q, sp)
    st.seq_slots[1] = st.max_seqs + 5
    bad, lbad = st.prefill(q, sp)
    torch.cuda.synchronize()
    G = wl.G
    for h, kind in enumerate(wl.head_kinds):
        qs = slice(h * G, (h + 1) * G)
        if kind == "local":
            assert (bad[1, :, qs] == 0).all() and torch.isneginf(lbad[1, :, qs]).all()
        else:
            assert torch.equal(bad[1, :, qs], good[1, :, qs])
        assert torch.equal(bad[0, :, qs], good[0, :, qs])


def test_prefill_negative_start_skips_sequence():
    wl = W.make_workload(2, n=600, batch=2)
    st = DecodeSetup(wl, keep_host=False)
    q = torch.from_numpy(np.stack([wl.prefill_queries(b, 100) for b in range(2)])).to(torch.bfloat16).cuda()
    out = torch.full((2, 100, wl.Hq, 128), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((2, 100, wl.Hq), 7.0, dtype=torch.float32, device="cuda")
    sp = torch.tensor([500, -1], dtype=torch.int32, device="cuda")
    st.ctx.prefill(q=q, block_tables=st.block_tables, start_pos=sp, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out[1] == 7.0).all() and (lse[1] == 7.0).all()
    assert torch.isfinite(out[0]).all() and not (out[0] == 7.0).all()


def test_prefill_profile_stage_and_repeat():
    wl = W.make_workload(1, n=1200)
    st = DecodeSetup(wl)
    q = torch.from_numpy(wl.prefill_queries(0, 1200)[None]).to(torch.bfloat16).cuda()
    sp = torch.zeros(1, dtype=torch.int32, device="cuda")
    st.ctx.profile_enable(True)
    a, la = st.prefill(q, sp)
    b, lb = st.prefill(q, sp)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof["prefill"][1] == 2, prof
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
