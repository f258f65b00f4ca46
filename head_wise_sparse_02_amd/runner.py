"""Set up a paged cache for a workload and drive append + decode through libhws.

Torch supplies device memory and the stream; every step of the path runs in
the library's kernels.  Inputs come from ``workloads`` (seeded, bf16-exact).
The cache is filled the way a decode loop fills it: one bulk append of the
first N-1 tokens of each sequence, then a single-token append of the current
token, then the decode step.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import hws
from .workloads import Workload

KIND_CODE = {"local": hws.HWS_HEAD_LOCAL, "retrieval": hws.HWS_HEAD_RETRIEVAL}


def append_segments(n: int) -> list:
    """The append calls that fill a sequence of length n: [(start, count)]."""
    return [(0, n - 1), (n - 1, 1)] if n > 1 else [(0, 1)]


def ring_rows(n_sink: int, window: int, slack: int = 0) -> int:
    """Rows per (sequence slot, local head) of the local ring: the first
    positions (sinks rounded up to 64), then window + slack rounded up to 16."""
    return ring_sink(n_sink) + ring_mod(window, slack)


def ring_sink(n_sink: int) -> int:
    """Ring rows of the first positions (position t < this sits in row t)."""
    return (n_sink + 63) // 64 * 64


def ring_mod(window: int, slack: int = 0) -> int:
    """Ring rows that later positions cycle through (t sits in row ring_sink + t % this)."""
    return (window + slack + 15) // 16 * 16


class DecodeSetup:
    """``segments``: optional function n -> [(start, count)] giving the append
    calls of a sequence of length n (default ``append_segments``).  With
    ``wl.local_ring`` the pages hold only the retrieval heads and the local
    heads live in ring pools of ``max_seqs`` = B + 3 slots, assigned to the
    sequences by a seeded permutation, keeping ``ring_slack`` rows beyond the
    window (prefill chunks of up to ring_slack + 1 positions)."""

    def __init__(self, wl: Workload, device: str = "cuda", spare_pages: int = 2,
                 keep_host=False, sequences=None, segments=None, ring_slack: int = 0):
        self.wl = wl
        self.dev = torch.device(device)
        self.segments = segments or append_segments
        B, Hkv, Hq, d = wl.B, wl.Hkv, wl.Hq, wl.d
        self.Nmax = int(max(wl.seq_lens))
        self.max_blocks = (self.Nmax + 15) // 16 + spare_pages
        pages = [(n + 15) // 16 + spare_pages for n in wl.seq_lens]
        self.num_blocks = int(sum(pages))
        self.fp8 = wl.kv_dtype == "fp8"
        self.ring = bool(wl.local_ring)
        self.max_seqs = B + 3 if self.ring else 0
        n_sink_c = max(wl.n_sink, 0)
        window_c = max(wl.window, 1 if wl.n_sink == 0 else 0)
        self.ctx = hws.Context(
            num_q_heads=Hq, num_kv_heads=Hkv, num_blocks=self.num_blocks,
            max_blocks_per_seq=self.max_blocks, n_sink=n_sink_c, window=window_c,
            local_ring=self.ring, max_seqs=self.max_seqs, ring_slack=ring_slack,
            attn_scale=wl.attn_scale, index_scale=wl.index_scale, rope_theta=wl.rope_theta,
            kv_dtype=hws.HWS_KV_FP8_E4M3 if self.fp8 else hws.HWS_KV_BF16,
            index_dtype=hws.HWS_INDEX_BF16 if wl.index_dtype == "bf16" else hws.HWS_INDEX_F32)
        self.ctx.set_head_kinds([KIND_CODE[k] for k in wl.head_kinds])
        self.nR = len(wl.retrieval_heads)
        self.nL = Hkv - self.nR

        # pools and a seeded random page assignment (pages are not contiguous)
        kv_dt = torch.uint8 if self.fp8 else torch.bfloat16
        # K pages are dim-blocked [4][16][32]; V pages are row-major [16][128]
        Hp = max(self.nR, 1) if self.ring else Hkv          # heads per page
        self.k_pool = torch.zeros((self.num_blocks, Hp, 4, 16, 32), dtype=kv_dt, device=self.dev)
        self.v_pool = torch.zeros((self.num_blocks, Hp, 16, d), dtype=kv_dt, device=self.dev)
        self.kv_scales = (torch.ones((self.num_blocks, Hp, 2), dtype=torch.float32, device=self.dev)
                          if self.fp8 else None)
        self.local_k_pool = self.local_v_pool = self.seq_slots = None
        if self.ring:
            W = ring_rows(n_sink_c, window_c, ring_slack)
            nl = max(self.nL, 1)
            # the ring holds bf16 rows whatever the page type
            self.local_k_pool = torch.zeros((self.max_seqs, nl, W // 16, 4, 16, 32), dtype=torch.bfloat16,
                                            device=self.dev)
            self.local_v_pool = torch.zeros((self.max_seqs, nl, W, d), dtype=torch.bfloat16, device=self.dev)
            srng = np.random.default_rng(np.random.SeedSequence([wl.cfg, wl.seed, 3001]))
            self.seq_slots_host = srng.permutation(self.max_seqs)[:B].astype(np.int32)
            self.seq_slots = torch.from_numpy(self.seq_slots_host).to(self.dev)
        idx_dt = torch.bfloat16 if wl.index_dtype == "bf16" else torch.float32
        self.index_pool = (torch.zeros((self.num_blocks, max(self.nR, 1), 16, 16), dtype=idx_dt,
                                       device=self.dev) if self.nR else None)
        self.proj_host = wl.projections()
        self.proj = torch.from_numpy(self.proj_host).to(self.dev)
        rng = np.random.default_rng(np.random.SeedSequence([wl.cfg, wl.seed, 3000]))
        perm = rng.permutation(self.num_blocks).astype(np.int32)
        bt = np.full((B, self.max_blocks), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            bt[b, :pages[b]] = perm[off:off + pages[b]]
            off += pages[b]
        self.block_tables_host = bt
        self.block_tables = torch.from_numpy(bt).to(self.dev)
        self.seq_lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=self.dev)
        self.ctx.bind(self.k_pool, self.v_pool, self.kv_scales, self.index_pool,
                      self.proj if self.nR else None, self.local_k_pool, self.local_v_pool)

        # fill the cache, sequence by sequence (keep_host: True keeps every
        # sequence's host arrays, a collection of indices keeps only those)
        self.q_host = np.zeros((B, Hq, d), dtype=np.float32)
        if keep_host is True:
            keep = set(range(B))
        elif keep_host:
            keep = {int(x) for x in keep_host}
        else:
            keep = None
        self.host = [] if keep is not None else None
        # sequences are drawn on a few threads (numpy releases the GIL while it
        # fills arrays), at most `ahead` of them beyond the one being appended
        ahead = max(1, min(8, os.cpu_count() or 1, B))
        pool = ThreadPoolExecutor(ahead) if sequences is None and B > 1 else None
        pending = {}

        def fetch(b: int):
            if sequences is not None:
                return sequences[b]
            if pool is None:
                return wl.sequence(b)
            for nb in range(b, min(B, b + ahead + 1)):
                if nb not in pending:
                    pending[nb] = pool.submit(wl.sequence, nb)
            return pending.pop(b).result()

        for b in range(B):
            seq = fetch(b)
            self.q_host[b] = seq.q
            if keep is not None:
                self.host.append(seq if b in keep else None)
            k = torch.from_numpy(seq.k).to(torch.bfloat16).to(self.dev)[None]
            v = torch.from_numpy(seq.v).to(torch.bfloat16).to(self.dev)[None]
            for start, cnt in (segments or append_segments)(wl.seq_lens[b]):
                sp = torch.tensor([start], dtype=torch.int32, device=self.dev)
                self.ctx.append(self.block_tables[b:b + 1], sp, k[:, start:start + cnt].contiguous(),
                                v[:, start:start + cnt].contiguous(),
                                seq_slots=None if self.seq_slots is None else self.seq_slots[b:b + 1])
            del k, v, seq
        if pool is not None:
            pool.shutdown()
        torch.cuda.synchronize(self.dev)
        self.q = torch.from_numpy(self.q_host).to(torch.bfloat16).to(self.dev)
        self.top_p = torch.from_numpy(np.asarray(wl.top_p, np.float32)).to(self.dev)
        self.top_k = torch.from_numpy(np.asarray(wl.top_k, np.int32)).to(self.dev)
        self.select_mode = hws.HWS_SELECT_TOP_P if wl.select_mode == "top_p" else hws.HWS_SELECT_TOP_K
        self.score_mode = hws.HWS_SCORE_INDEX if wl.score_mode == "index" else hws.HWS_SCORE_FULL
        self.scope = hws.HWS_SCOPE_QUERY_HEAD if wl.select_scope == "query" else hws.HWS_SCOPE_KV_HEAD
        ws = self.ctx.workspace_size(B, self.Nmax, self.score_mode, self.scope)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=self.dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=self.dev)
        # |S| per KV head, or per query head with one set per query head
        self.sel_counts = torch.empty((B, Hq if self.scope else Hkv), dtype=torch.int32, device=self.dev)
        self.sel_mass = torch.empty((B, Hq if self.scope else Hkv), dtype=torch.float32, device=self.dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.dev)

    def dense_lse(self, stream=None) -> np.ndarray:
        """ln sum_i exp(attn_scale q.k_i) over every cached row, [B, Hq] (host)."""
        ws = torch.empty(self.ctx.dense_lse_workspace(self.wl.B, self.Nmax), dtype=torch.uint8, device=self.dev)
        out = torch.empty((self.wl.B, self.wl.Hq), dtype=torch.float32, device=self.dev)
        self.ctx.dense_lse(q=self.q, block_tables=self.block_tables, seq_lens=self.seq_lens, max_seq_len=self.Nmax,
                           lse_full=out, workspace=ws, stream=stream)
        torch.cuda.synchronize(self.dev)
        return out.cpu().numpy()

    def prefill(self, q, start_pos, *, dense: bool = False, stream=None):
        """Prefill attention of the chunk q [B, n_tok, Hq, d] (bf16 device tensor)
        at positions start_pos[b].. (int32 device tensor); the cache already holds
        them.  Returns (out, lse) device tensors."""
        B, n_tok = int(q.shape[0]), int(q.shape[1])
        out = torch.empty((B, n_tok, self.wl.Hq, self.wl.d), dtype=torch.float32, device=self.dev)
        lse = torch.empty((B, n_tok, self.wl.Hq), dtype=torch.float32, device=self.dev)
        self.ctx.prefill(q=q, block_tables=self.block_tables, start_pos=start_pos, out=out, lse=lse,
                         dense=dense, stream=stream, seq_slots=self.seq_slots)
        return out, lse

    def decode(self, *, debug: bool = False, sel_cap: int | None = None, stream=None,
               rows_read: bool | None = None, mass: bool | None = None, noalloc: bool = False):
        """Run one decode step.  With debug=True also return the raw scores,
        the ascending selected positions, the per-position row-read counts of
        the attention, the kept aggregate mass and the step status (host numpy
        arrays); ``rows_read`` / ``mass`` switch those two off or on alone.
        ``noalloc`` calls hws_decode_noalloc (the library's static scratch
        array instead of this setup's workspace)."""
        B, G = self.wl.B, self.wl.G
        scores = sel_idx = None
        rows_read = debug if rows_read is None else rows_read
        mass = debug if mass is None else mass
        if debug and self.nR:
            scores = torch.empty((B, self.nR, self.Nmax, G), dtype=torch.float32, device=self.dev)
            cap = sel_cap or self.Nmax
            shape = (B, self.nR, G, cap) if self.scope else (B, self.nR, cap)
            sel_idx = torch.full(shape, -1, dtype=torch.int32, device=self.dev)
        rr = (torch.full((B, self.wl.Hkv, self.Nmax), -7, dtype=torch.int32, device=self.dev)
              if rows_read else None)
        sm = self.sel_mass if mass else None
        status = self.status if debug else None
        if status is not None:
            status.fill_(-7)
        self.ctx.decode(q=self.q, block_tables=self.block_tables, seq_lens=self.seq_lens,
                        max_seq_len=self.Nmax, select_mode=self.select_mode,
                        score_mode=self.score_mode, out=self.out, workspace=self.workspace,
                        top_p=self.top_p, top_k=self.top_k, lse=self.lse,
                        sel_counts=self.sel_counts, sel_idx=sel_idx, scores=scores, stream=stream,
                        select_scope=self.scope, seq_slots=self.seq_slots, rows_read=rr,
                        sel_mass=sm, status=status, noalloc=noalloc)
        if not debug:
            return None
        torch.cuda.synchronize(self.dev)
        res = {"out": self.out.cpu().numpy(), "lse": self.lse.cpu().numpy(),
               "sel_counts": self.sel_counts.cpu().numpy(), "status": int(self.status.item())}
        if scores is not None:
            res["scores"] = scores.cpu().numpy()
            res["sel_idx"] = sel_idx.cpu().numpy()
        if rr is not None:
            res["rows_read"] = rr.cpu().numpy()
        if sm is not None:
            res["sel_mass"] = sm.cpu().numpy()
        return res
