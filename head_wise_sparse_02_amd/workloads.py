"""Seeded synthetic decode workloads (inputs only: none of the method's arithmetic).

Shared by the tests, the bench and the smoke check: it builds queries, keys,
values and index projections shaped like the workloads the pages discuss
(32K-256K contexts, GQA groups, planted "needle" tokens, ~2 % selections).
It computes no score, selection or attention.  All values are drawn as
float32 normals and rounded once to bfloat16 (ties to even), so the arrays
returned hold bf16-exact float32 values that both the HIP library (after an
exact cast) and the CPU oracle consume unchanged.

Random streams: ``SeedSequence([cfg, seed, b])`` per sequence (draw order:
q, K, V, needle positions, needle jitter, boost masks, orthogonal noise),
``SeedSequence([cfg, seed, 1000 + h])`` per index projection (a weight,
shared by all sequences) and ``SeedSequence([cfg, seed, 2000])`` for
batch-level draws (lengths, head kinds, per-sequence top-p).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128
R = 16
NEEDLE_NORM = 4.0          # needle key = 4 * sqrt(d) * u + jitter
NEEDLE_JITTER = 0.05


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 precision (ties to even), as float32.

    Adds 0x7FFF plus the lowest kept bit to the bit pattern and clears the
    16 dropped bits (in place on a copy, in slices, to keep temporaries small)."""
    out = np.array(x, dtype=np.float32, order="C", copy=True)
    flat = out.reshape(-1).view(np.uint32)
    tmp = np.empty(min(flat.size, 1 << 22), dtype=np.uint32)
    for lo in range(0, flat.size, tmp.size):
        u = flat[lo:lo + tmp.size]
        t = tmp[:u.size]
        np.right_shift(u, np.uint32(16), out=t)
        np.bitwise_and(t, np.uint32(1), out=t)
        np.add(t, np.uint32(0x7FFF), out=t)
        np.add(u, t, out=u)
        np.bitwise_and(u, np.uint32(0xFFFF0000), out=u)
    return out


def _unit(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / np.linalg.norm(v)


def _orth_units(rng, n: int, u: np.ndarray) -> np.ndarray:
    """n random unit vectors orthogonal to the unit vector u."""
    z = rng.standard_normal((n, u.size), dtype=np.float32).astype(np.float64)
    z -= np.outer(z @ u, u)
    return z / np.linalg.norm(z, axis=1, keepdims=True)


@dataclass
class Sequence:
    q: np.ndarray            # [Hq, d]  float32, bf16-exact, pre-RoPE
    k: np.ndarray            # [N, Hkv, d]
    v: np.ndarray            # [N, Hkv, d]
    needles: dict = field(default_factory=dict)   # KV head -> positions


@dataclass
class Workload:
    name: str
    cfg: int
    seed: int
    B: int
    Hq: int
    Hkv: int
    seq_lens: list
    head_kinds: list                 # per KV head: "retrieval" | "local"
    score_mode: str                  # "index" | "full"
    select_mode: str                 # "top_p" | "top_k"
    top_p: np.ndarray                # [B] float32
    top_k: np.ndarray                # [B] int32
    n_sink: int
    window: int
    kv_dtype: str                    # "bf16" | "fp8"
    rope_theta: float = 0.0
    select_scope: str = "kv"         # "kv": one set per KV head | "query": one per query head
    index_dtype: str = "f32"         # stored r=16 index: "f32" | "bf16"
    local_ring: bool = False         # local heads keep sinks + window in a per-sequence ring
    d: int = D
    r: int = R
    n_needles: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def attn_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def index_scale(self) -> float:
        # sqrt(d)/r makes index_scale * (Pq).(Pk) an unbiased estimate of
        # q.k/sqrt(d) for P with N(0, 1/d) entries.
        return float(np.sqrt(self.d)) / self.r

    @property
    def retrieval_heads(self) -> list:
        return [h for h, k in enumerate(self.head_kinds) if k == "retrieval"]

    def projections(self) -> np.ndarray:
        """[Hkv, r, d] float32; N(0,1)/sqrt(d) rows for retrieval heads, 0 else."""
        P = np.zeros((self.Hkv, self.r, self.d), dtype=np.float32)
        for h in self.retrieval_heads:
            rng = np.random.default_rng(np.random.SeedSequence([self.cfg, self.seed, 1000 + h]))
            P[h] = (rng.standard_normal((self.r, self.d), dtype=np.float32)
                    / np.float32(np.sqrt(self.d)))
        return P

    def sequence(self, b: int) -> Sequence:
        return _SEQ_BUILDERS[self.cfg](self, b)

    def prefill_queries(self, b: int, n_tok: int) -> np.ndarray:
        """Queries of a prefill chunk of sequence b: [n_tok, Hq, d] bf16-exact N(0, 1)."""
        rng = np.random.default_rng(np.random.SeedSequence([self.cfg, self.seed, 4000 + b]))
        return bf16_rne(rng.standard_normal((n_tok, self.Hq, self.d), dtype=np.float32))


# ---------------------------------------------------------------------------
# per-config sequence builders
# ---------------------------------------------------------------------------

def _base(wl: Workload, b: int):
    rng = np.random.default_rng(np.random.SeedSequence([wl.cfg, wl.seed, b]))
    n = wl.seq_lens[b]
    q = bf16_rne(rng.standard_normal((wl.Hq, wl.d), dtype=np.float32))
    k = rng.standard_normal((n, wl.Hkv, wl.d), dtype=np.float32)
    v = bf16_rne(rng.standard_normal((n, wl.Hkv, wl.d), dtype=np.float32))
    return rng, n, q, k, v


def _group_dir(wl: Workload, q: np.ndarray, h: int, lo: int = 0, hi: int | None = None) -> np.ndarray:
    G = wl.G
    hi = G if hi is None else hi
    return _unit(q[h * G + lo:h * G + hi].astype(np.float64).sum(axis=0))


def _plant_needles(wl, rng, q, k, n_needle, pos_lo, pos_hi, dirs=None):
    """Needle key = 4*sqrt(d)*u_h + 0.05*N(0, I) for each retrieval head."""
    heads = wl.retrieval_heads
    pos = {h: np.sort(rng.choice(np.arange(pos_lo, pos_hi), size=n_needle, replace=False))
           for h in heads}
    for h in heads:
        u = _group_dir(wl, q, h) if dirs is None else dirs[h]
        jit = rng.standard_normal((n_needle, wl.d), dtype=np.float32).astype(np.float64)
        k[pos[h], h, :] = (NEEDLE_NORM * np.sqrt(wl.d) * u[None, :]
                           + NEEDLE_JITTER * jit).astype(np.float32)
    return pos


def _seq_needles(wl: Workload, b: int) -> Sequence:
    """Configs 1, 2 and 5: N(0,1) keys plus planted needles in retrieval heads."""
    rng, n, q, k, v = _base(wl, b)
    lo, hi = wl.extra.get("needle_range", (0, None))
    hi = n if hi is None else (n + hi if hi < 0 else hi)
    pos = _plant_needles(wl, rng, q, k, min(wl.n_needles, max(0, hi - lo)), lo, hi)
    return Sequence(q=q, k=bf16_rne(k), v=v, needles=pos)


def _seq_boost(wl: Workload, b: int) -> Sequence:
    """Config 3: 5 % of tokens per head boosted to cos 0.5 with the query direction."""
    rng, n, q, k, v = _base(wl, b)
    frac = wl.extra.get("boost_frac", 0.05)
    cos = wl.extra.get("boost_cos", 0.5)
    n_boost = int(round(frac * n))
    masks = {h: rng.choice(n, size=n_boost, replace=False) for h in range(wl.Hkv)}
    for h in range(wl.Hkv):
        u = _group_dir(wl, q, h)
        nh = _orth_units(rng, n_boost, u)
        k[masks[h], h, :] = (np.sqrt(wl.d) * (cos * u[None, :] + np.sqrt(1 - cos * cos) * nh)
                             ).astype(np.float32)
    return Sequence(q=q, k=bf16_rne(k), v=v, needles={h: np.sort(m) for h, m in masks.items()})


def _seq_peaky_diffuse(wl: Workload, b: int) -> Sequence:
    """Config 4: in the retrieval group, query heads 0-3 are peaky (needles
    along their mean direction) and heads 4-7 diffuse (20 % of the other
    tokens share a 0.3-cos direction with their mean)."""
    rng, n, q, k, v = _base(wl, b)
    G = wl.G
    half = G // 2
    dirs = {h: _group_dir(wl, q, h, 0, half) for h in wl.retrieval_heads}
    pos = _plant_needles(wl, rng, q, k, wl.n_needles, 0, n, dirs=dirs)
    frac = wl.extra.get("diffuse_frac", 0.2)
    cos = wl.extra.get("diffuse_cos", 0.3)
    diffuse = {}
    for h in wl.retrieval_heads:
        others = np.setdiff1d(np.arange(n), pos[h])
        diffuse[h] = np.sort(rng.choice(others, size=int(round(frac * others.size)), replace=False))
    for h in wl.retrieval_heads:
        w = _group_dir(wl, q, h, half, G)
        nh = _orth_units(rng, diffuse[h].size, w)
        k[diffuse[h], h, :] = (np.sqrt(wl.d) * (cos * w[None, :] + np.sqrt(1 - cos * cos) * nh)
                               ).astype(np.float32)
    return Sequence(q=q, k=bf16_rne(k), v=v, needles=pos)


_SEQ_BUILDERS = {1: _seq_needles, 2: _seq_needles, 3: _seq_boost, 4: _seq_peaky_diffuse,
                 5: _seq_needles}


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny decode step: B=1, 8 Q / 2 KV heads, N=4096, 1 retrieval (top-p 0.9) + 1 local head",
    2: "Llama-3-8B-shaped layer: B=8, 32 Q / 8 KV heads, N=32768, 2 retrieval (top-p 0.9) + 6 local",
    3: "oracle top-k at 50x sparsity: B=4, 32 Q / 8 KV heads, N=131072, full-dim scores, k=2%",
    4: "70B-shaped long decode: B=1, 64 Q / 8 KV heads, N=262144, 1 retrieval (top-p 0.95) + 7 local",
    5: "ragged fp8 serving mix: B=32, N in [8K,128K], 32 Q / 8 KV heads, 2 retrieval + 6 local",
}


def make_workload(cfg: int, seed: int = 0, *, n: int | None = None, batch: int | None = None,
                  **overrides) -> Workload:
    """Build workload ``cfg`` (1..5).  ``n`` / ``batch`` shrink the context
    length / batch while keeping the recipe (for tests); ``overrides`` replace
    any other field."""
    if cfg == 1:
        N, B = n or 4096, batch or 1
        wl = Workload(name="tiny", cfg=1, seed=seed, B=B, Hq=8, Hkv=2, seq_lens=[N] * B,
                      head_kinds=["retrieval", "local"], score_mode="index",
                      select_mode="top_p", top_p=np.full(B, 0.9, np.float32),
                      top_k=np.zeros(B, np.int32), n_sink=4, window=256, kv_dtype="bf16",
                      n_needles=8, extra={"needle_range": (4, -256)})
    elif cfg == 2:
        N, B = n or 32768, batch or 8
        wl = Workload(name="llama3_8b_layer", cfg=2, seed=seed, B=B, Hq=32, Hkv=8,
                      seq_lens=[N] * B, head_kinds=["retrieval"] * 2 + ["local"] * 6,
                      score_mode="index", select_mode="top_p",
                      top_p=np.full(B, 0.9, np.float32), top_k=np.zeros(B, np.int32),
                      n_sink=4, window=1024, kv_dtype="bf16", n_needles=32)
    elif cfg == 3:
        N, B = n or 131072, batch or 4
        wl = Workload(name="oracle_topk_128k", cfg=3, seed=seed, B=B, Hq=32, Hkv=8,
                      seq_lens=[N] * B, head_kinds=["retrieval"] * 8, score_mode="full",
                      select_mode="top_k", top_p=np.ones(B, np.float32),
                      top_k=np.full(B, int(0.02 * N), np.int32), n_sink=0, window=0,
                      kv_dtype="bf16")
    elif cfg == 4:
        N, B = n or 262144, batch or 1
        wl = Workload(name="llama70b_long", cfg=4, seed=seed, B=B, Hq=64, Hkv=8,
                      seq_lens=[N] * B, head_kinds=["retrieval"] + ["local"] * 7,
                      score_mode="index", select_mode="top_p",
                      top_p=np.full(B, 0.95, np.float32), top_k=np.zeros(B, np.int32),
                      n_sink=4, window=2048, kv_dtype="bf16", n_needles=8)
    elif cfg == 5:
        B = batch or 32
        rng = np.random.default_rng(np.random.SeedSequence([5, seed, 2000]))
        lo, hi = (8192, 131072) if n is None else (max(1, n // 16), n)
        lens = [int(x) for x in rng.integers(lo, hi, size=B, endpoint=True)]
        ret = sorted(int(h) for h in rng.permutation(8)[:2])
        kinds = ["retrieval" if h in ret else "local" for h in range(8)]
        p = rng.choice(np.array([0.8, 0.9, 0.95], np.float32), size=B)
        wl = Workload(name="ragged_fp8_mix", cfg=5, seed=seed, B=B, Hq=32, Hkv=8,
                      seq_lens=lens, head_kinds=kinds, score_mode="index",
                      select_mode="top_p", top_p=p.astype(np.float32),
                      top_k=np.zeros(B, np.int32), n_sink=4, window=1024, kv_dtype="fp8",
                      n_needles=32)
    else:
        raise ValueError(f"unknown workload {cfg}")
    for key, val in overrides.items():
        if not hasattr(wl, key):
            raise AttributeError(key)
        setattr(wl, key, val)
    return wl
