"""ctypes binding of libhws (include/hws.h): same call names, marshalling only.

Tensors are torch tensors used as device memory: the binding passes
``data_ptr()`` and the current HIP stream handle and does no compute.  The
library is loaded on first use; if ``libhws.so`` is missing or cannot be
loaded, every call raises ``HwsError`` (there is no fallback path).
"""

from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhws.so")
_lib = None

# status codes and enums (include/hws.h)
HWS_OK = 0
HWS_ERR_INVALID_ARG = -1
HWS_ERR_STATE = -2
HWS_ERR_CAPACITY = -3
HWS_ERR_WORKSPACE = -4
HWS_ERR_UNSUPPORTED = -5
HWS_ERR_HIP = -6
HWS_KV_BF16, HWS_KV_FP8_E4M3 = 0, 1
HWS_HEAD_LOCAL, HWS_HEAD_RETRIEVAL = 0, 1
HWS_SELECT_TOP_P, HWS_SELECT_TOP_K = 0, 1
HWS_SCORE_INDEX, HWS_SCORE_FULL = 0, 1
HWS_SCOPE_KV_HEAD, HWS_SCOPE_QUERY_HEAD = 0, 1
HWS_INDEX_F32, HWS_INDEX_BF16 = 0, 1
HWS_LAUNCH_AUTO, HWS_LAUNCH_MULTI, HWS_LAUNCH_COOPERATIVE, HWS_LAUNCH_SINGLE = 0, 1, 2, 3
HWS_LAUNCH_SCAN_SELECT, HWS_LAUNCH_SCAN_SINGLE = 4, 5
HWS_STEP_OK, HWS_STEP_WAIT_TIMEOUT = 0, 1

EXPORTED = (
    "hws_abi_version", "hws_status_string", "hws_last_error", "hws_create", "hws_destroy",
    "hws_set_head_kinds", "hws_classify_by_scores", "hws_get_head_kinds", "hws_bind",
    "hws_workspace_size", "hws_append", "hws_decode", "hws_profile_enable",
    "hws_profile_read", "hws_profile_stage_name", "hws_set_launch_mode",
    "hws_effective_rank_workspace", "hws_effective_rank", "hws_prefill", "hws_set_wait_limit",
    "hws_decode_noalloc", "hws_profile_phases", "hws_dense_lse_workspace", "hws_dense_lse",
)
HWS_PHASES = 12
HWS_NOALLOC_SCRATCH_BYTES = 32 << 20


class HwsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_q_heads", "num_kv_heads", "head_dim", "index_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "kv_dtype", "index_dtype", "n_sink", "window", "local_ring",
        "max_seqs", "ring_slack")] + [
        ("attn_scale", ctypes.c_float), ("index_scale", ctypes.c_float),
        ("rope_theta", ctypes.c_float)]


class Buffers(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("kv_scales", ctypes.c_void_p), ("index_pool", ctypes.c_void_p),
                ("proj", ctypes.c_void_p), ("local_k_pool", ctypes.c_void_p),
                ("local_v_pool", ctypes.c_void_p)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("select_mode", ctypes.c_int32), ("score_mode", ctypes.c_int32),
                ("select_scope", ctypes.c_int32), ("q", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("seq_slots", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
                ("top_k", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("sel_counts", ctypes.c_void_p), ("sel_idx", ctypes.c_void_p),
                ("sel_cap", ctypes.c_int32), ("scores", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("rows_read", ctypes.c_void_p), ("sel_mass", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_tok", ctypes.c_int32), ("dense", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("start_pos", ctypes.c_void_p),
                ("seq_slots", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libhws.so (once).  Raises HwsError if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise HwsError(HWS_ERR_STATE, f"{_LIB_PATH} is not built; run "
                       "`python -m head_wise_sparse_02_amd.build` (no fallback exists)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
    sig = {
        "hws_abi_version": (i32, []),
        "hws_status_string": (ctypes.c_char_p, [i32]),
        "hws_last_error": (ctypes.c_char_p, [vp]),
        "hws_create": (i32, [P(Config), P(vp)]),
        "hws_destroy": (i32, [vp]),
        "hws_set_head_kinds": (i32, [vp, P(ctypes.c_uint8)]),
        "hws_classify_by_scores": (i32, [vp, P(ctypes.c_float), i32, i32]),
        "hws_get_head_kinds": (i32, [vp, P(ctypes.c_uint8)]),
        "hws_bind": (i32, [vp, P(Buffers)]),
        "hws_workspace_size": (i32, [vp, i32, i32, i32, i32, P(ctypes.c_size_t)]),
        "hws_append": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "hws_decode": (i32, [vp, P(DecodeArgs), vp]),
        "hws_decode_noalloc": (i32, [vp, P(DecodeArgs), vp]),
        "hws_prefill": (i32, [vp, P(PrefillArgs), vp]),
        "hws_profile_enable": (i32, [vp, i32]),
        "hws_set_launch_mode": (i32, [vp, i32]),
        "hws_set_wait_limit": (i32, [vp, ctypes.c_uint32, i32]),
        "hws_effective_rank_workspace": (i32, [i32, i32, P(ctypes.c_size_t)]),
        "hws_effective_rank": (i32, [i32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "hws_profile_read": (i32, [vp, P(ctypes.c_double), P(i32), i32]),
        "hws_profile_stage_name": (ctypes.c_char_p, [i32]),
        "hws_profile_phases": (i32, [vp, vp, i32]),
        "hws_dense_lse_workspace": (i32, [vp, i32, i32, P(ctypes.c_size_t)]),
        "hws_dense_lse": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(st: int) -> str:
    return lib().hws_status_string(st).decode()


class Context:
    """One attention layer: owns an hws_ctx (host object)."""

    def __init__(self, *, num_q_heads: int, num_kv_heads: int, num_blocks: int,
                 max_blocks_per_seq: int, n_sink: int, window: int, attn_scale: float,
                 index_scale: float = 1.0, rope_theta: float = 0.0, kv_dtype: int = HWS_KV_BF16,
                 index_dtype: int = HWS_INDEX_F32, local_ring: bool = False, max_seqs: int = 0,
                 ring_slack: int = 0, head_dim: int = 128, index_dim: int = 16, block_size: int = 16):
        self._L = lib()
        self.cfg = Config(num_q_heads, num_kv_heads, head_dim, index_dim, block_size, num_blocks,
                          max_blocks_per_seq, kv_dtype, index_dtype, n_sink, window, int(bool(local_ring)),
                          max_seqs, ring_slack, attn_scale, index_scale, rope_theta)
        h = ctypes.c_void_p()
        st = self._L.hws_create(ctypes.byref(self.cfg), ctypes.byref(h))
        if st != HWS_OK:
            raise HwsError(st, f"hws_create: {status_string(st)}")
        self.handle = h

    # -- lifecycle ---------------------------------------------------------
    def close(self):
        if getattr(self, "handle", None):
            self._L.hws_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int, what: str):
        if st != HWS_OK:
            msg = self._L.hws_last_error(self.handle).decode()
            raise HwsError(st, f"{what}: {status_string(st)}: {msg}")

    # -- head kinds ----------------------------------------------------------
    def set_head_kinds(self, kinds):
        arr = (ctypes.c_uint8 * len(kinds))(*[int(k) for k in kinds])
        self._check(self._L.hws_set_head_kinds(self.handle, arr), "hws_set_head_kinds")

    def classify_by_scores(self, q_head_scores, n_retrieval_kv: int, lower_is_retrieval: bool):
        arr = (ctypes.c_float * len(q_head_scores))(*[float(x) for x in q_head_scores])
        self._check(self._L.hws_classify_by_scores(self.handle, arr, int(n_retrieval_kv),
                                                   int(bool(lower_is_retrieval))),
                    "hws_classify_by_scores")

    def head_kinds(self) -> list:
        arr = (ctypes.c_uint8 * self.cfg.num_kv_heads)()
        self._check(self._L.hws_get_head_kinds(self.handle, arr), "hws_get_head_kinds")
        return list(arr)

    # -- memory --------------------------------------------------------------
    def bind(self, k_pool, v_pool, kv_scales=None, index_pool=None, proj=None, local_k_pool=None,
             local_v_pool=None):
        self._buf = Buffers(_ptr(k_pool), _ptr(v_pool), _ptr(kv_scales), _ptr(index_pool), _ptr(proj),
                            _ptr(local_k_pool), _ptr(local_v_pool))
        self._check(self._L.hws_bind(self.handle, ctypes.byref(self._buf)), "hws_bind")

    def workspace_size(self, batch: int, max_seq_len: int, score_mode: int, select_scope: int = 0) -> int:
        n = ctypes.c_size_t()
        self._check(self._L.hws_workspace_size(self.handle, batch, max_seq_len, score_mode, select_scope,
                                               ctypes.byref(n)), "hws_workspace_size")
        return n.value

    # -- device work -----------------------------------------------------------
    def append(self, block_tables, start_pos, k, v, stream=None, seq_slots=None):
        """k, v: [n_seq, n_tok, Hkv, 128] bf16 device tensors; seq_slots: [n_seq]
        int32 ring slots (local ring only)."""
        n_seq, n_tok = int(k.shape[0]), int(k.shape[1])
        self._check(self._L.hws_append(self.handle, n_seq, n_tok, _ptr(block_tables), _ptr(start_pos),
                                       _ptr(seq_slots), _ptr(k), _ptr(v), _stream(stream)), "hws_append")

    def decode(self, *, q, block_tables, seq_lens, max_seq_len: int, select_mode: int,
               score_mode: int, out, workspace, top_p=None, top_k=None, lse=None,
               sel_counts=None, sel_idx=None, scores=None, stream=None, select_scope: int = 0,
               seq_slots=None, rows_read=None, sel_mass=None, status=None, noalloc: bool = False):
        """hws_decode (or, with noalloc=True, hws_decode_noalloc, which ignores
        ``workspace`` and uses the library's static scratch array)."""
        a = DecodeArgs()
        a.select_scope = int(select_scope)
        a.batch = int(q.shape[0]) if q is not None else 0
        a.max_seq_len = int(max_seq_len)
        a.select_mode, a.score_mode = int(select_mode), int(score_mode)
        a.q, a.block_tables, a.seq_lens = _ptr(q), _ptr(block_tables), _ptr(seq_lens)
        a.seq_slots = _ptr(seq_slots)
        a.top_p, a.top_k = _ptr(top_p), _ptr(top_k)
        a.out, a.lse, a.sel_counts = _ptr(out), _ptr(lse), _ptr(sel_counts)
        a.sel_idx = _ptr(sel_idx)
        a.sel_cap = int(sel_idx.shape[-1]) if sel_idx is not None else 0
        a.scores = _ptr(scores)
        a.workspace = _ptr(workspace)
        a.workspace_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
        a.rows_read, a.sel_mass, a.status = _ptr(rows_read), _ptr(sel_mass), _ptr(status)
        if noalloc:
            self._check(self._L.hws_decode_noalloc(self.handle, ctypes.byref(a), _stream(stream)),
                        "hws_decode_noalloc")
        else:
            self._check(self._L.hws_decode(self.handle, ctypes.byref(a), _stream(stream)), "hws_decode")

    def decode_noalloc(self, **kw):
        """hws_decode_noalloc: the decode step with its workspace in the
        library's static device array (``workspace`` may be None)."""
        kw.setdefault("workspace", None)
        self.decode(noalloc=True, **kw)

    def dense_lse_workspace(self, batch: int, max_seq_len: int) -> int:
        n = ctypes.c_size_t()
        self._check(self._L.hws_dense_lse_workspace(self.handle, batch, max_seq_len, ctypes.byref(n)),
                    "hws_dense_lse_workspace")
        return n.value

    def dense_lse(self, *, q, block_tables, seq_lens, max_seq_len: int, lse_full, workspace, stream=None):
        """ln sum_i exp(attn_scale q.k_i) over every cached row, per query head:
        q [B, Hq, 128] bf16, lse_full [B, Hq] fp32 (device tensors)."""
        nbytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
        batch = int(q.shape[0]) if q is not None else 0
        self._check(self._L.hws_dense_lse(self.handle, batch, int(max_seq_len), _ptr(q),
                                          _ptr(block_tables), _ptr(seq_lens), _ptr(lse_full), _ptr(workspace),
                                          nbytes, _stream(stream)), "hws_dense_lse")

    def prefill(self, *, q, block_tables, start_pos, out, lse=None, dense: bool = False, stream=None,
                seq_slots=None):
        """Chunked prefill attention: q [n_seq, n_tok, Hq, 128] bf16 of the positions
        start_pos[s]..start_pos[s]+n_tok-1 (already appended); out [n_seq, n_tok, Hq, 128]
        fp32, lse [n_seq, n_tok, Hq] or None; dense: every head attends to every
        earlier position; seq_slots: [n_seq] int32 ring slots (local ring)."""
        a = PrefillArgs()
        a.n_seq = int(q.shape[0]) if q is not None else 0
        a.n_tok = int(q.shape[1]) if q is not None else 0
        a.dense = int(bool(dense))
        a.q, a.block_tables, a.start_pos = _ptr(q), _ptr(block_tables), _ptr(start_pos)
        a.seq_slots = _ptr(seq_slots)
        a.out, a.lse = _ptr(out), _ptr(lse)
        self._check(self._L.hws_prefill(self.handle, ctypes.byref(a), _stream(stream)), "hws_prefill")

    # -- timing ------------------------------------------------------------------
    def set_launch_mode(self, mode: int):
        """HWS_LAUNCH_AUTO (default), HWS_LAUNCH_SINGLE (one launch after or
        with the scoring scan, grid sized to the device), HWS_LAUNCH_COOPERATIVE
        (the same as a cooperative launch), HWS_LAUNCH_MULTI (one kernel per
        stage), HWS_LAUNCH_SCAN_SINGLE (the scan, then the single launch) or
        HWS_LAUNCH_SCAN_SELECT (the scan, the selection as one launch, then the
        per-stage attention and merge)."""
        self._check(self._L.hws_set_launch_mode(self.handle, int(mode)), "hws_set_launch_mode")

    def set_wait_limit(self, max_polls: int = 0, unreachable: bool = False):
        """Polls before a hand-off wait of the single launch gives up (0: the
        default 2^20); ``unreachable`` makes every wait give up (the step then
        ends normally with NaN outputs for the heads whose selection gave up)."""
        self._check(self._L.hws_set_wait_limit(self.handle, int(max_polls), int(bool(unreachable))),
                    "hws_set_wait_limit")

    def profile_enable(self, enable: bool = True):
        self._check(self._L.hws_profile_enable(self.handle, int(enable)), "hws_profile_enable")

    def profile_phases(self, buf=None, max_workgroups: int = 0):
        """Phase timestamps of later single-launch decodes into ``buf`` (a device
        int64 tensor of max_workgroups * HWS_PHASES entries), or off (None)."""
        self._check(self._L.hws_profile_phases(self.handle, _ptr(buf), int(max_workgroups)),
                    "hws_profile_phases")

    def profile_read(self) -> dict:
        n = 16
        ms = (ctypes.c_double * n)()
        calls = (ctypes.c_int32 * n)()
        self._check(self._L.hws_profile_read(self.handle, ms, calls, n), "hws_profile_read")
        out = {}
        for i in range(n):
            name = self._L.hws_profile_stage_name(i).decode()
            if name:
                out[name] = (ms[i], calls[i])
        return out


def effective_rank_workspace(num_q_heads: int, num_kv_heads: int) -> int:
    n = ctypes.c_size_t()
    st = lib().hws_effective_rank_workspace(num_q_heads, num_kv_heads, ctypes.byref(n))
    if st != HWS_OK:
        raise HwsError(st, f"hws_effective_rank_workspace: {status_string(st)}")
    return n.value


def effective_rank(w_q, w_k, eff_rank, workspace, stream=None):
    """Effective rank per query head ([AoH] Methodology §1-§3) of device fp32
    weights w_q [Hq, 128, d_model], w_k [Hkv, 128, d_model] into eff_rank [Hq]."""
    hq, hkv, d_model = int(w_q.shape[0]), int(w_k.shape[0]), int(w_q.shape[2])
    nbytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    st = lib().hws_effective_rank(hq, hkv, d_model, _ptr(w_q), _ptr(w_k), _ptr(eff_rank), _ptr(workspace),
                                  nbytes, _stream(stream))
    if st != HWS_OK:
        raise HwsError(st, f"hws_effective_rank: {status_string(st)}")
