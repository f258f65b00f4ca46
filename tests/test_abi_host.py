"""C-ABI host tests: library loads, exports every declared symbol, and every
validation error is reported before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

from head_wise_sparse_02_amd import hws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "hws.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(hws_\w+)\s*\(", text, re.M)))


def _cfg(**kw):
    base = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, index_dim=16, block_size=16,
                num_blocks=64, max_blocks_per_seq=32, kv_dtype=0, index_dtype=0, n_sink=4, window=256,
                local_ring=0, max_seqs=0, ring_slack=0, attn_scale=0.0883883, index_scale=0.7071,
                rope_theta=0.0)
    base.update(kw)
    return hws.Config(*[base[n] for n, _ in hws.Config._fields_])


def _create(**kw):
    L = hws.lib()
    h = ctypes.c_void_p()
    st = L.hws_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    return st, h


def test_library_exports_every_declared_symbol():
    L = hws.lib()
    decl = _declared()
    assert len(decl) >= 15
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(hws.EXPORTED) == decl
    assert L.hws_abi_version() == 5
    assert L.hws_status_string(hws.HWS_ERR_WORKSPACE) == b"workspace too small"


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), hws.HWS_ERR_UNSUPPORTED),
    (dict(index_dim=32), hws.HWS_ERR_UNSUPPORTED),
    (dict(block_size=32), hws.HWS_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=2), hws.HWS_ERR_UNSUPPORTED),     # G = 3
    (dict(num_q_heads=7, num_kv_heads=2), hws.HWS_ERR_INVALID_ARG),
    (dict(num_q_heads=128, num_kv_heads=128), hws.HWS_ERR_UNSUPPORTED),  # > 64 KV heads
    (dict(n_sink=0, window=0), hws.HWS_ERR_INVALID_ARG),
    (dict(window=-1), hws.HWS_ERR_INVALID_ARG),
    (dict(attn_scale=0.0), hws.HWS_ERR_INVALID_ARG),
    (dict(attn_scale=float("nan")), hws.HWS_ERR_INVALID_ARG),
    (dict(rope_theta=-1.0), hws.HWS_ERR_INVALID_ARG),
    (dict(kv_dtype=2), hws.HWS_ERR_INVALID_ARG),
    (dict(index_dtype=2), hws.HWS_ERR_INVALID_ARG),
    (dict(index_dtype=-1), hws.HWS_ERR_INVALID_ARG),
    (dict(num_blocks=0), hws.HWS_ERR_INVALID_ARG),
    (dict(local_ring=2, max_seqs=4), hws.HWS_ERR_INVALID_ARG),
    (dict(local_ring=1, max_seqs=0), hws.HWS_ERR_INVALID_ARG),
    (dict(local_ring=1, max_seqs=1 << 28), hws.HWS_ERR_INVALID_ARG),          # ring pages overflow int32
    (dict(local_ring=1, max_seqs=4, ring_slack=-1), hws.HWS_ERR_INVALID_ARG),
])
def test_create_rejects(kw, status):
    st, h = _create(**kw)
    assert st == status and not h.value


def test_ring_with_fp8_pages_is_accepted():
    """The ring keeps bf16 rows, so it combines with fp8 pages."""
    st, h = _create(local_ring=1, max_seqs=4, kv_dtype=1)
    assert st == hws.HWS_OK and h.value
    hws.lib().hws_destroy(h)


def test_create_null_arguments():
    L = hws.lib()
    h = ctypes.c_void_p()
    assert L.hws_create(None, ctypes.byref(h)) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_create(ctypes.byref(_cfg()), None) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_destroy(None) == hws.HWS_OK


def _ctx(**kw):
    return hws.Context(num_q_heads=kw.get("hq", 8), num_kv_heads=kw.get("hkv", 2), num_blocks=64,
                       max_blocks_per_seq=32, n_sink=4, window=256, attn_scale=0.088,
                       index_scale=0.707, kv_dtype=kw.get("kv", 0), local_ring=kw.get("ring", False),
                       max_seqs=kw.get("max_seqs", 0), ring_slack=kw.get("ring_slack", 0))


def test_head_kinds_and_classification():
    c = _ctx(hq=32, hkv=8)
    assert c.head_kinds() == [0] * 8
    with pytest.raises(hws.HwsError) as e:
        c.set_head_kinds([0, 1, 2, 0, 0, 0, 0, 0])
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    c.set_head_kinds([1, 0, 0, 1, 0, 0, 0, 0])
    assert c.head_kinds() == [1, 0, 0, 1, 0, 0, 0, 0]
    # mean pooling over each group of 4 query heads, then ranking
    s = [0.0] * 32
    for g in range(4):
        s[4 * 5 + g] = 1.0               # group 5 mean 1.0
        s[4 * 2 + g] = 3.0 if g == 0 else 0.0   # group 2 mean 0.75 (one large head)
    s[4 * 7] = 4.0                        # group 7 mean 1.0 as well: tie with 5 -> lower index wins
    c.classify_by_scores(s, 2, lower_is_retrieval=False)
    assert c.head_kinds() == [0, 0, 0, 0, 0, 1, 0, 1]
    c.classify_by_scores(s, 1, lower_is_retrieval=False)
    assert c.head_kinds() == [0, 0, 0, 0, 0, 1, 0, 0]
    # effective-rank rule: lowest scores become retrieval heads
    er = [float(10 - h) for h in range(8) for _ in range(4)]
    c.classify_by_scores(er, 3, lower_is_retrieval=True)
    assert c.head_kinds() == [0, 0, 0, 0, 0, 1, 1, 1]
    with pytest.raises(hws.HwsError):
        c.classify_by_scores(er, 9, lower_is_retrieval=True)
    with pytest.raises(hws.HwsError):
        c.classify_by_scores([float("inf")] * 32, 1, lower_is_retrieval=True)


def test_bind_and_state_errors():
    c = _ctx()
    with pytest.raises(hws.HwsError) as e:
        c.append(block_tables=8, start_pos=8, k=_FakeT(), v=_FakeT(), stream=0)
    assert e.value.status == hws.HWS_ERR_STATE
    with pytest.raises(hws.HwsError) as e:
        c.bind(0, 16)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    c8 = _ctx(kv=1)
    with pytest.raises(hws.HwsError) as e:
        c8.bind(16, 16)                  # fp8 without scales
    assert e.value.status == hws.HWS_ERR_INVALID_ARG


def test_local_ring_rules():
    # a ring context with max_seqs = 0 is rejected; with the ring off, max_seqs is ignored
    st, h = _create(local_ring=0, max_seqs=-5)
    assert st == hws.HWS_OK
    hws.lib().hws_destroy(h)
    c = _ctx(ring=True, max_seqs=4)
    c.set_head_kinds([1, 0])
    with pytest.raises(hws.HwsError) as e:
        c.bind(4096, 4096, None, 4096, 4096)                     # no ring pools
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    c.bind(4096, 4096, None, 4096, 4096, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:                        # local heads need seq_slots
        c.append(block_tables=_FakeT(), start_pos=_FakeT(), k=_FakeT(), v=_FakeT(), stream=0)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG and b"seq_slots" in hws.lib().hws_last_error(c.handle)
    with pytest.raises(hws.HwsError) as e:
        _decode(c)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG and b"seq_slots" in hws.lib().hws_last_error(c.handle)
    # every head a retrieval head: nothing goes to the ring, seq_slots may be NULL (the
    # decode then fails only on the workspace check, the last host check)
    c2 = _ctx(ring=True, max_seqs=4)
    c2.set_head_kinds([1, 1])
    c2.bind(4096, 4096, None, 4096, 4096, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:
        _decode(c2, workspace=_FakeT(nbytes=100))
    assert e.value.status == hws.HWS_ERR_WORKSPACE


def test_launch_mode_values():
    c = _ctx()
    c.set_launch_mode(hws.HWS_LAUNCH_MULTI)
    c.set_launch_mode(hws.HWS_LAUNCH_COOPERATIVE)
    c.set_launch_mode(hws.HWS_LAUNCH_SINGLE)
    c.set_launch_mode(hws.HWS_LAUNCH_SCAN_SELECT)
    c.set_launch_mode(hws.HWS_LAUNCH_SCAN_SINGLE)
    c.set_launch_mode(hws.HWS_LAUNCH_AUTO)
    for bad in (-1, 6, 99):
        with pytest.raises(hws.HwsError) as e:
            c.set_launch_mode(bad)
        assert e.value.status == hws.HWS_ERR_INVALID_ARG
    assert hws.lib().hws_profile_stage_name(4) == b"tail"
    assert hws.lib().hws_profile_stage_name(5) == b"fused"
    assert hws.lib().hws_profile_stage_name(6) == b"prefill"
    assert hws.lib().hws_profile_stage_name(7) == b"fused_index"
    assert hws.lib().hws_profile_stage_name(8) == b"attend_balanced"
    assert hws.lib().hws_profile_stage_name(9) == b""


def test_wait_limit_values():
    c = _ctx()
    for polls in (0, 1, 256, 1000, 1 << 24):
        c.set_wait_limit(polls)
    c.set_wait_limit(256, unreachable=True)
    c.set_wait_limit(0, unreachable=False)
    with pytest.raises(hws.HwsError) as e:
        c.set_wait_limit((1 << 24) + 1)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    assert hws.lib().hws_set_wait_limit(None, 0, 0) == hws.HWS_ERR_INVALID_ARG


class _FakeT:
    """Stand-in for a tensor: only shapes and addresses are read on the host."""
    def __init__(self, shape=(1, 1, 2, 128), nbytes=1 << 20):
        self.shape = shape
        self._n = nbytes

    def data_ptr(self):
        return 4096

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def _decode(c, **kw):
    args = dict(q=_FakeT((1, 8, 128)), block_tables=_FakeT(), seq_lens=_FakeT(), max_seq_len=100,
                select_mode=0, score_mode=0, out=_FakeT(), workspace=_FakeT(nbytes=1 << 30),
                top_p=_FakeT(), stream=0)
    args.update(kw)
    c.decode(**args)


def test_decode_validation_without_gpu():
    c = _ctx()
    with pytest.raises(hws.HwsError) as e:
        _decode(c)
    assert e.value.status == hws.HWS_ERR_STATE          # before bind
    c.set_head_kinds([1, 0])
    c.bind(4096, 4096, None, 4096, 4096)
    cases = [
        (dict(max_seq_len=32 * 16 + 1), hws.HWS_ERR_CAPACITY),
        (dict(max_seq_len=0), hws.HWS_ERR_INVALID_ARG),
        (dict(select_mode=2), hws.HWS_ERR_INVALID_ARG),
        (dict(score_mode=5), hws.HWS_ERR_INVALID_ARG),
        (dict(select_scope=2), hws.HWS_ERR_INVALID_ARG),
        (dict(select_scope=-1), hws.HWS_ERR_INVALID_ARG),
        (dict(q=None), hws.HWS_ERR_INVALID_ARG),
        (dict(top_p=None), hws.HWS_ERR_INVALID_ARG),
        (dict(select_mode=1), hws.HWS_ERR_INVALID_ARG),  # top-k without top_k
        (dict(sel_idx=_FakeT((1, 1, 0))), hws.HWS_ERR_INVALID_ARG),
        (dict(workspace=_FakeT(nbytes=100)), hws.HWS_ERR_WORKSPACE),
        (dict(workspace=None), hws.HWS_ERR_WORKSPACE),
    ]
    for kw, status in cases:
        with pytest.raises(hws.HwsError) as e:
            _decode(c, **kw)
        assert e.value.status == status, (kw, e.value)
        assert hws.lib().hws_last_error(c.handle)


def test_full_scores_with_fp8_cache_pass_validation():
    """Full-dim scores read fp8 pages too: the call is checked like any other
    (a missing workspace is the error it reports, not the cache type)."""
    c = _ctx(kv=1)
    c.set_head_kinds([1, 0])
    c.bind(4096, 4096, 4096, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:
        _decode(c, score_mode=1, workspace=None)
    assert e.value.status == hws.HWS_ERR_WORKSPACE


def test_workspace_size_rules():
    c = _ctx()
    c.set_head_kinds([1, 0])
    n1 = c.workspace_size(1, 500, 0)
    n2 = c.workspace_size(2, 500, 0)
    assert 0 < n1 < n2 and n1 % 256 == 0
    with pytest.raises(hws.HwsError) as e:
        c.workspace_size(1, 32 * 16 + 1, 0)
    assert e.value.status == hws.HWS_ERR_CAPACITY
    with pytest.raises(hws.HwsError):
        c.workspace_size(0, 10, 0)
    # scores region: 4 bytes x G per token per retrieval head at least
    assert n1 >= 500 * 4 * 4 + 500 * 4
    # one set per query head: G aggregates and G selection states per retrieval head
    nq = c.workspace_size(1, 500, 0, hws.HWS_SCOPE_QUERY_HEAD)
    assert nq >= 500 * 4 * 4 + 4 * 500 * 4
    with pytest.raises(hws.HwsError) as e:
        c.workspace_size(1, 500, 0, 7)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    # a workspace sized for one set per KV head is too small for one per query head
    c.bind(4096, 4096, None, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:
        _decode(c, max_seq_len=500, workspace=_FakeT(nbytes=n1), select_scope=hws.HWS_SCOPE_QUERY_HEAD)
    assert e.value.status == hws.HWS_ERR_WORKSPACE


def test_effective_rank_validation_without_gpu():
    assert hws.effective_rank_workspace(8, 2) == (3 * 8 + 2) * 128 * 128 * 8
    for hq, hkv in ((0, 1), (8, 3), (4, 0)):
        with pytest.raises(hws.HwsError) as e:
            hws.effective_rank_workspace(hq, hkv)
        assert e.value.status == hws.HWS_ERR_INVALID_ARG
    L = hws.lib()
    ws = 1 << 30
    assert L.hws_effective_rank(8, 2, 0, 4096, 4096, 4096, 4096, ws, None) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_effective_rank(8, 3, 64, 4096, 4096, 4096, 4096, ws, None) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_effective_rank(8, 2, 64, None, 4096, 4096, 4096, ws, None) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_effective_rank(8, 2, 64, 4096, 4096, 4096, 4096, 100, None) == hws.HWS_ERR_WORKSPACE
    assert L.hws_effective_rank(8, 2, 64, 4096, 4096, 4096, None, ws, None) == hws.HWS_ERR_WORKSPACE


def _prefill(c, **kw):
    args = dict(q=_FakeT((2, 300, 8, 128)), block_tables=_FakeT(), start_pos=_FakeT(), out=_FakeT(),
                stream=0)
    args.update(kw)
    c.prefill(**args)


def test_prefill_validation_without_gpu():
    c = _ctx()
    with pytest.raises(hws.HwsError) as e:
        _prefill(c)
    assert e.value.status == hws.HWS_ERR_STATE          # before bind
    c.set_head_kinds([1, 0])
    c.bind(4096, 4096, None, 4096, 4096)
    cases = [
        (dict(q=_FakeT((0, 5, 8, 128))), hws.HWS_ERR_INVALID_ARG),
        (dict(q=_FakeT((1, 0, 8, 128))), hws.HWS_ERR_INVALID_ARG),
        (dict(q=None), hws.HWS_ERR_INVALID_ARG),
        (dict(out=None), hws.HWS_ERR_INVALID_ARG),
        (dict(start_pos=None), hws.HWS_ERR_INVALID_ARG),
        (dict(block_tables=None), hws.HWS_ERR_INVALID_ARG),
        (dict(q=_FakeT((1, 32 * 16 + 1, 8, 128))), hws.HWS_ERR_CAPACITY),
    ]
    for kw, status in cases:
        with pytest.raises(hws.HwsError) as e:
            _prefill(c, **kw)
        assert e.value.status == status, (kw, e.value)
    L = hws.lib()
    a = hws.PrefillArgs(1, 4, 2, 4096, 4096, 4096, 4096, None)       # dense must be 0 or 1
    assert L.hws_prefill(c.handle, ctypes.byref(a), None) == hws.HWS_ERR_INVALID_ARG
    assert L.hws_prefill(c.handle, None, None) == hws.HWS_ERR_INVALID_ARG
    # an fp8 cache goes through the same checks; the local ring is not read by prefill
    c8 = _ctx(kv=1)
    c8.bind(4096, 4096, 4096, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:
        _prefill(c8, out=None)
    assert e.value.status == hws.HWS_ERR_INVALID_ARG
    # the local ring: seq_slots required, chunks of at most ring_slack + 1
    # positions, no dense prefill (the ring lacks the local heads' older rows)
    cr = _ctx(ring=True, max_seqs=2, ring_slack=299)
    cr.set_head_kinds([1, 0])
    cr.bind(4096, 4096, None, 4096, 4096, 4096, 4096)
    for kw, status in [(dict(), hws.HWS_ERR_INVALID_ARG),
                       (dict(seq_slots=_FakeT(), q=_FakeT((2, 301, 8, 128))), hws.HWS_ERR_CAPACITY),
                       (dict(seq_slots=_FakeT(), dense=True), hws.HWS_ERR_UNSUPPORTED)]:
        with pytest.raises(hws.HwsError) as e:
            _prefill(cr, **kw)
        assert e.value.status == status, (kw, e.value)


def test_decode_noalloc_validation_without_gpu():
    """hws_decode_noalloc checks a call like hws_decode (it needs no caller
    workspace) and refuses a step whose workspace exceeds its static scratch
    array, all before any HIP call."""
    c = _ctx()
    with pytest.raises(hws.HwsError) as e:
        _decode(c, workspace=None, noalloc=True)
    assert e.value.status == hws.HWS_ERR_STATE          # before bind
    c.set_head_kinds([1, 0])
    c.bind(4096, 4096, None, 4096, 4096)
    big = 600
    assert c.workspace_size(big, 512, 0) > hws.HWS_NOALLOC_SCRATCH_BYTES >= c.workspace_size(1, 512, 0)
    cases = [
        (dict(q=_FakeT((big, 8, 128)), max_seq_len=512), hws.HWS_ERR_CAPACITY),
        (dict(max_seq_len=32 * 16 + 1), hws.HWS_ERR_CAPACITY),
        (dict(q=None), hws.HWS_ERR_INVALID_ARG),
        (dict(select_mode=2), hws.HWS_ERR_INVALID_ARG),
        (dict(top_p=None), hws.HWS_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        with pytest.raises(hws.HwsError) as e:
            _decode(c, workspace=None, noalloc=True, **kw)
        assert e.value.status == status, (kw, e.value)
        assert b"hws_decode_noalloc" in str(e.value).encode() and hws.lib().hws_last_error(c.handle)


def test_dense_lse_validation_without_gpu():
    c = _ctx()
    ws = _FakeT(nbytes=1 << 30)
    call = dict(q=_FakeT((1, 8, 128)), block_tables=_FakeT(), seq_lens=_FakeT(), max_seq_len=100,
                lse_full=_FakeT(), workspace=ws, stream=0)
    with pytest.raises(hws.HwsError) as e:
        c.dense_lse(**call)
    assert e.value.status == hws.HWS_ERR_STATE          # before bind
    c.set_head_kinds([1, 0])
    c.bind(4096, 4096, None, 4096, 4096)
    assert 0 < c.dense_lse_workspace(1, 100) < c.dense_lse_workspace(8, 512)
    for kw, status in [(dict(max_seq_len=32 * 16 + 1), hws.HWS_ERR_CAPACITY), (dict(lse_full=None), hws.HWS_ERR_INVALID_ARG),
                       (dict(workspace=_FakeT(nbytes=8)), hws.HWS_ERR_WORKSPACE),
                       (dict(q=None), hws.HWS_ERR_INVALID_ARG)]:
        with pytest.raises(hws.HwsError) as e:
            c.dense_lse(**{**call, **kw})
        assert e.value.status == status, (kw, e.value)
    r = _ctx(ring=True, max_seqs=2)
    r.set_head_kinds([1, 0])
    r.bind(4096, 4096, None, 4096, 4096, 4096, 4096)
    with pytest.raises(hws.HwsError) as e:
        r.dense_lse(**call)
    assert e.value.status == hws.HWS_ERR_UNSUPPORTED
