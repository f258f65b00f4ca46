// Gathered decode attention of one 16-lane row processor, shared by the
// per-stage attention kernel and the single-launch tail.
//
// [ICS] "Inference-time context sparsity: illusion or opportunity?", §3c:
// sparse decode reads only the rows of the selected tokens.  A processor
// walks its rows RB at a time; lane `sub` holds dims 8*sub..8*sub+7.  All
// loads of a batch are issued before any is used: rows past the end (or on
// an out-of-range page) load row 0 of page 0 and are masked afterwards, so
// no load sits behind a per-lane branch (which would make the compiler wait
// for each one in turn).  The softmax runs online in log2 units.
#pragma once

#include <type_traits>

#include "hws_device.h"

namespace hws {

// Rows per processor per batch: all loads of a batch are in flight at once.
template <int G, int MODE>
struct AttRB {
  // MODE 1 reads V rows and stored scores; the others also read K rows.
  static constexpr int value = MODE == 1 ? 8 : (G <= 2 ? 8 : (G == 4 ? 4 : 2));
};

// Where local-head row `tok` of sequence b (local head number l) is stored:
// its 16-row page pg and its index ii (slot ii % 16 of the page).  Without a
// ring these are the sequence's cache page and the position; with a ring,
// the ring row of the token (ring_row: the first positions in their own
// rows, later ones modulo ring_mod) in the sequence's ring slot, or pg = -1
// for a slot out of range.
__device__ __forceinline__ void local_row_at(const DecodeParams& p, int b, int l, int tok, int& ii, int& pg) {
  if (p.ring_rows > 0) {
    const int slot = p.seq_slots[b];
    const int rr = ring_row(tok, p.ring_sink, p.ring_mod);
    ii = rr;
    pg = (unsigned)slot < (unsigned)p.max_seqs ? (int)((((long long)slot * p.nL + l) * p.ring_rows + rr) >> 4) : -1;
  } else {
    ii = tok;
    pg = p.block_tables[(size_t)b * p.max_blocks + (tok >> 4)];
  }
}

// Row r of the list: retrieval rows are offsets (from lo) in `rows`, whose
// page is pages[offset / 16]; local rows -- and retrieval rows when `rows` is
// null -- are at index ltok[r] of page lpg[r] (local_row_at), local ones in
// the ring pools when there is a ring.
// MODE 0: logits q.k from K rows; MODE 1: retrieval heads only, logits from
// the stored full-dim scores; MODE 2: both (scores for retrieval heads).
// RET: the rows are known to be a retrieval head's (no K path compiled in).
// lds_logits (full-dim scores only): the scores of row r at lds_logits[r*G];
// null reads them from the scores buffer at the row's position.
// row_mask (retrieval rows, one set per query head): bit g of row_mask[r] says
// whether query head g keeps row r; null means every head keeps every row.
// init = false continues the (m, l, o) of an earlier call on the same head.
template <int G, bool FP8, int MODE, int RB, bool RET = false, bool ROW_ORDER = FP8>
__device__ __forceinline__ void accumulate_rows(const DecodeParams& p, int b, int h, int hr, int lo, int nrows,
                                                int r_begin, int r_step, int sub, const unsigned short* rows,
                                                const int* pages, const int* ltok, const int* lpg,
                                                const float* lds_logits, float (&m)[G], float (&l)[G],
                                                float (&o)[G][8], const unsigned char* row_mask = nullptr,
                                                bool init = true) {
  static_assert(!RET || MODE != 0, "retrieval rows read K only in index mode");
  constexpr bool NEED_K = MODE != 1 && !RET;
  const bool is_ret = RET || hr >= 0;
  const bool use_scores = MODE != 0 && is_ret;

  // queries of the group, pre-scaled to log2 units: dims 8*sub..8*sub+7
  float qf[NEED_K ? G : 1][8];
  if (NEED_K && !use_scores) {
#pragma unroll
    for (int g = 0; g < (NEED_K ? G : 1); ++g) {
      const size_t qo = ((size_t)b * p.Hq + h * G + g) * D + 8 * sub;
      if (p.qrot != nullptr) {
        const float4 a = *reinterpret_cast<const float4*>(p.qrot + qo);
        const float4 c = *reinterpret_cast<const float4*>(p.qrot + qo + 4);
        qf[g][0] = a.x; qf[g][1] = a.y; qf[g][2] = a.z; qf[g][3] = a.w;
        qf[g][4] = c.x; qf[g][5] = c.y; qf[g][6] = c.z; qf[g][7] = c.w;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(p.q + qo);
        qf[g][0] = bf16_lo(u.x); qf[g][1] = bf16_hi(u.x); qf[g][2] = bf16_lo(u.y); qf[g][3] = bf16_hi(u.y);
        qf[g][4] = bf16_lo(u.z); qf[g][5] = bf16_hi(u.z); qf[g][6] = bf16_lo(u.w); qf[g][7] = bf16_hi(u.w);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[g][j] *= p.c2_attn;
    }
  }
  const float* sc = use_scores ? p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G : nullptr;
  // the rows' pools: the pages (Hp heads each, this head at pool_slot[h]) or
  // the local ring (one head per page)
  const bool ring = !is_ret && p.ring_rows > 0;
  const void* kpool = ring ? p.lk_pool : p.k_pool;
  const void* vpool = ring ? p.lv_pool : p.v_pool;
  const int hstride = ring ? 1 : p.Hp;
  const int hslot = ring ? 0 : p.pool_slot[h];
  const unsigned plim = ring ? (unsigned)p.ring_pages : (unsigned)p.num_blocks;
  if (init) {                                    // else: more rows of the same head
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = NEG_INF;
      l[g] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
    }
  }

  for (int r0 = r_begin; r0 < nrows; r0 += r_step) {
    int ii[RB], pg[RB];
    bool ok[RB];
    if (is_ret && rows != nullptr) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int off = rows[min(r0 + u, nrows - 1)];
        ii[u] = lo + off;
        pg[u] = pages[off >> 4];
      }
    } else {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int rc = min(r0 + u, nrows - 1);
        ii[u] = ltok[rc];
        pg[u] = lpg[rc];
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      ok[u] = r0 + u < nrows && (unsigned)pg[u] < plim;
      if (!ok[u]) { pg[u] = 0; ii[u] = 0; }
    }
    // debug: count each row this processor reads at its position (ring rows
    // are indexed by ring row, not position, and are not counted)
    if (p.rows_read != nullptr && sub == 0 && !ring) {
      int* rr = p.rows_read + (size_t)(b * p.Hkv + h) * p.Nmax;
#pragma unroll
      for (int u = 0; u < RB; ++u)
        if (ok[u]) atomicAdd(rr + ii[u], 1);
    }

    // every load of the batch
    float vv[RB][8];
    float z[RB][G];
    float kx[NEED_K ? RB : 1][8];
    float ks[RB], vs[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u)
      load_row8<FP8>(vpool, ((size_t)pg[u] * hstride + hslot) * BS + (ii[u] & 15), sub, vv[u]);
    if (FP8) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const float2 s2 = *reinterpret_cast<const float2*>(p.kv_scales + ((size_t)pg[u] * hstride + hslot) * 2);
        ks[u] = s2.x;
        vs[u] = s2.y;
      }
    }
    if (use_scores && lds_logits != nullptr) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int rc = min(r0 + u, nrows - 1);
#pragma unroll
        for (int g = 0; g < G; ++g) z[u][g] = lds_logits[(size_t)rc * G + g];
      }
    } else if (use_scores) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        if (G >= 4) {
#pragma unroll
          for (int q4 = 0; q4 < G / 4; ++q4) {
            const float4 v = *reinterpret_cast<const float4*>(sc + (size_t)ii[u] * G + 4 * q4);
            z[u][4 * q4 + 0] = v.x; z[u][4 * q4 + 1] = v.y; z[u][4 * q4 + 2] = v.z; z[u][4 * q4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) z[u][g] = sc[(size_t)ii[u] * G + g];
        }
      }
    } else if (NEED_K) {
#pragma unroll
      for (int u = 0; u < RB; ++u)
        load_krow8<FP8>(kpool, (size_t)pg[u] * hstride + hslot, ii[u] & 15, sub, kx[NEED_K ? u : 0]);
    }

    // logits (log2 units), masked rows at -inf
    if (use_scores) {
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) z[u][g] = ok[u] ? z[u][g] * p.c2_score : NEG_INF;
    } else if (NEED_K) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = qf[NEED_K ? g : 0][0] * kx[NEED_K ? u : 0][0];
#pragma unroll
          for (int j = 1; j < 8; ++j) a = fmaf(qf[NEED_K ? g : 0][j], kx[NEED_K ? u : 0][j], a);
          a = row16_sum(a);
          z[u][g] = ok[u] ? (FP8 ? a * ks[u] : a) : NEG_INF;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vv[u][j] = ok[u] ? (FP8 ? vv[u][j] * vs[u] : vv[u][j]) : 0.f;
    }
    if (is_ret && row_mask != nullptr) {         // heads that do not keep a row skip it
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const unsigned int mk = row_mask[min(r0 + u, nrows - 1)];
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (!((mk >> g) & 1u)) z[u][g] = NEG_INF;
      }
    }

    // one rescale per batch, then the rows in order.  ROW_ORDER walks row by
    // row (fewer values live at once: the fp8 kernels fit one more wave per
    // SIMD), otherwise head by head (more independent work in flight); per
    // head and dim both add the same terms in the same order.
    if constexpr (ROW_ORDER) {
      bool live[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mn = m[g];
#pragma unroll
        for (int u = 0; u < RB; ++u) mn = fmaxf(mn, z[u][g]);
        live[g] = mn != NEG_INF;                     // uniform over the processor
        if (!live[g]) continue;
        const float cf = fast_exp2(m[g] - mn);
        l[g] *= cf;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] *= cf;
        m[g] = mn;
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (!live[g]) continue;
          const float pz = fast_exp2(z[u][g] - m[g]);
          l[g] += pz;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pz, vv[u][j], o[g][j]);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mn = m[g];
#pragma unroll
        for (int u = 0; u < RB; ++u) mn = fmaxf(mn, z[u][g]);
        if (mn == NEG_INF) continue;                 // uniform over the processor
        const float cf = fast_exp2(m[g] - mn);
        l[g] *= cf;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] *= cf;
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const float pz = fast_exp2(z[u][g] - mn);
          l[g] += pz;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pz, vv[u][j], o[g][j]);
        }
        m[g] = mn;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gathered attention with the next batch in flight.  The rows' (index, page)
// coordinates are in LDS (tok[r], pgs[r] for r < nrows, filled by the
// caller); processor `proc` takes batches of RB rows, batch j being rows
// (16 j + proc) RB .. + RB - 1.  The K/V words (and fp8 scales) of batch j+1
// are loaded, undecoded, before batch j is decoded and folded in, so a
// processor always has a batch of loads outstanding while it computes.
// Rows past the end (or on an out-of-range page) load row 0 of page 0 and are
// masked.  Logits are q.k from the K rows (index scores), online softmax in
// log2 units as in accumulate_rows.
// ---------------------------------------------------------------------------
template <bool FP8, int RB>
struct RawBatch {
  using W = typename std::conditional<FP8, uint2, uint4>::type;
  W k[RB], v[RB];
  float2 sc[FP8 ? RB : 1];
  bool ok[RB];
};

template <bool FP8>
__device__ __forceinline__ void decode8(uint4 w, float* x) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}
template <bool FP8>
__device__ __forceinline__ void decode8(uint2 w, float* x) {
  f32x2 t;
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false); x[0] = t.x; x[1] = t.y;
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);  x[2] = t.x; x[3] = t.y;
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false); x[4] = t.x; x[5] = t.y;
  t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);  x[6] = t.x; x[7] = t.y;
}

// Where the gather reads: the pools, heads per page, this head's slot, page limit.
struct GatherSrc {
  const void* kpool;
  const void* vpool;
  const float* scales;
  int hstride, hslot;
  unsigned plim;
};

// MARK: count each row read in rr at its position (debug).
template <bool FP8, int RB, bool MARK>
__device__ __forceinline__ void issue_batch(const GatherSrc& src, const int* tok, const int* pgs, int nrows,
                                            int r0, int sub, RawBatch<FP8, RB>& rb, int* rr) {
  using W = typename RawBatch<FP8, RB>::W;
  constexpr int EB = FP8 ? 1 : 2;                       // bytes per element
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int rc = min(r0 + u, nrows - 1);
    int ii = tok[rc], pg = pgs[rc];
    rb.ok[u] = r0 + u < nrows && (unsigned)pg < src.plim;
    if (!rb.ok[u]) { pg = 0; ii = 0; }
    const size_t page = (size_t)pg * src.hstride + src.hslot;
    const size_t koff = page * (BS * D) + (size_t)((((sub >> 2) << 4) + (ii & 15)) * 32 + 8 * (sub & 3));
    const size_t voff = page * (BS * D) + (size_t)((ii & 15) * D + 8 * sub);
    rb.k[u] = *reinterpret_cast<const W*>(reinterpret_cast<const unsigned char*>(src.kpool) + koff * EB);
    rb.v[u] = *reinterpret_cast<const W*>(reinterpret_cast<const unsigned char*>(src.vpool) + voff * EB);
    if (FP8) rb.sc[FP8 ? u : 0] = *reinterpret_cast<const float2*>(src.scales + page * 2);
    if (MARK && sub == 0 && rb.ok[u]) atomicAdd(rr + ii, 1);
  }
}

template <int G, bool FP8, int RB>
__device__ __forceinline__ void fold_batch(const RawBatch<FP8, RB>& rb, const float (&qf)[G][8], float (&m)[G],
                                           float (&l)[G], float (&o)[G][8]) {
  float z[RB][G];
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    float kx[8];
    decode8<FP8>(rb.k[u], kx);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = qf[g][0] * kx[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) a = fmaf(qf[g][j], kx[j], a);
      a = row16_sum(a);
      z[u][g] = rb.ok[u] ? (FP8 ? a * rb.sc[FP8 ? u : 0].x : a) : NEG_INF;
    }
  }
  // one rescale per batch (branch-free: a head with nothing yet keeps
  // m = -inf, and its factors come out as 0)
  float ms[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mn = m[g];
#pragma unroll
    for (int u = 0; u < RB; ++u) mn = fmaxf(mn, z[u][g]);
    ms[g] = mn == NEG_INF ? 0.f : mn;
    const float cf = fast_exp2(m[g] - ms[g]);
    l[g] *= cf;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] *= cf;
    m[g] = mn;
  }
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    float vv[8];
    decode8<FP8>(rb.v[u], vv);
    const float vs = FP8 ? rb.sc[FP8 ? u : 0].y : 1.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = rb.ok[u] ? (FP8 ? vv[j] * vs : vv[j]) : 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pz = fast_exp2(z[u][g] - ms[g]);
      l[g] += pz;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pz, vv[j], o[g][j]);
    }
  }
}

// The group's queries, dims 8*sub..8*sub+7, pre-scaled to log2 units: the
// rotated fp32 queries when RoPE is on (K rows are stored rotated), else the
// bf16 queries.
template <int G>
__device__ __forceinline__ void load_group_q(const DecodeParams& p, int b, int h, int sub, float (&qf)[G][8]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t qo = ((size_t)b * p.Hq + h * G + g) * D + 8 * sub;
    if (p.qrot != nullptr) {
      const float4 a = *reinterpret_cast<const float4*>(p.qrot + qo);
      const float4 c = *reinterpret_cast<const float4*>(p.qrot + qo + 4);
      qf[g][0] = a.x; qf[g][1] = a.y; qf[g][2] = a.z; qf[g][3] = a.w;
      qf[g][4] = c.x; qf[g][5] = c.y; qf[g][6] = c.z; qf[g][7] = c.w;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(p.q + qo);
      qf[g][0] = bf16_lo(u.x); qf[g][1] = bf16_hi(u.x); qf[g][2] = bf16_lo(u.y); qf[g][3] = bf16_hi(u.y);
      qf[g][4] = bf16_lo(u.z); qf[g][5] = bf16_hi(u.z); qf[g][6] = bf16_lo(u.w); qf[g][7] = bf16_hi(u.w);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[g][j] *= p.c2_attn;
  }
}

// Rows 0..nrows-1 of the LDS list into (m, l, o) of processor `proc`
// (continuing the values it holds).  qf: the group's queries in log2 units.
// MARK: count every row read in rr[position] (debug; not for ring rows).
template <int G, bool FP8, int RB, bool MARK = false>
__device__ __forceinline__ void gather_pipelined(const GatherSrc& src, const int* tok, const int* pgs, int nrows,
                                                 int proc, int sub, const float (&qf)[G][8], float (&m)[G],
                                                 float (&l)[G], float (&o)[G][8], int* rr = nullptr) {
  const int nb = (nrows + 16 * RB - 1) / (16 * RB);   // batches of the workgroup (uniform)
  if (nb == 0) return;
  // batches past the last are all masked rows: issuing them anyway keeps the
  // loop free of branches, so the compiler waits only for the batch it folds
  // (the scheduling barriers keep the compiler from pulling a batch's use
  // up to its loads, which would leave nothing in flight)
  RawBatch<FP8, RB> a, c;
  issue_batch<FP8, RB, MARK>(src, tok, pgs, nrows, proc * RB, sub, a, rr);
#pragma clang loop unroll(disable)
  for (int j = 0; j < nb; j += 2) {
    issue_batch<FP8, RB, MARK>(src, tok, pgs, nrows, ((j + 1) * 16 + proc) * RB, sub, c, rr);
    __builtin_amdgcn_sched_barrier(0);
    fold_batch<G, FP8, RB>(a, qf, m, l, o);
    __builtin_amdgcn_sched_barrier(0);
    issue_batch<FP8, RB, MARK>(src, tok, pgs, nrows, ((j + 2) * 16 + proc) * RB, sub, a, rr);
    __builtin_amdgcn_sched_barrier(0);
    fold_batch<G, FP8, RB>(c, qf, m, l, o);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One combine step of the processors in lanes i and i^X: symmetric in the
// two lanes, so both end with the same (m, l, o).
template <int G, int X>
__device__ __forceinline__ void combine_lane_pairs(float (&m)[G], float (&l)[G], float (&o)[G][8]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float ma, mb, la, lb;
    lane_pair<X>(m[g], ma, mb);
    lane_pair<X>(l[g], la, lb);
    const float mn = fmaxf(ma, mb);
    const float ca = (mn == NEG_INF) ? 0.f : fast_exp2(ma - mn);
    const float cb = (mn == NEG_INF) ? 0.f : fast_exp2(mb - mn);
    l[g] = la * ca + lb * cb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float oa, ob;
      lane_pair<X>(o[g][j], oa, ob);
      o[g][j] = oa * ca + ob * cb;
    }
    m[g] = mn;
  }
}

// Combine the 4 processors of a wave (lanes sub, sub+16, sub+32, sub+48).
template <int G>
__device__ __forceinline__ void combine_wave_procs(float (&m)[G], float (&l)[G], float (&o)[G][8]) {
  combine_lane_pairs<G, 16>(m, l, o);
  combine_lane_pairs<G, 32>(m, l, o);
}

// ---------------------------------------------------------------------------
// Rows with K at G = 8 (index scores or local heads), bf16 rows, queries not
// rotated.  The 8 dot products per row are a dense contraction of the rows
// with the group's queries, so they run on the matrix cores: a wave takes 32
// rows per batch as two 16-row A operands of v_mfma_f32_16x16x32_bf16 (lane
// (col, quad) loads the 8 dims 32 st + 8 quad of row col, 16 bytes of the
// page-blocked K layout), B = the queries (column g < 8 = query head g, the
// other 8 columns zero), 4 MFMAs per 16 rows over the 128 dims.  Lane
// (col, quad) then holds the logits of query head col for rows 4 quad .. +3
// of each tile: the wave's online softmax per head runs there (max and sum
// over the four lane groups by lane swaps), and the weights go through LDS to
// the row processors (16 lanes, dims 8 sub .. 8 sub + 7, 8 rows each), which
// add p v on the vector ALUs.  Every processor of a wave shares the wave's
// running max, so the processors' partials differ only in o: on return m is
// the wave's max, l the wave's sum in processor 0 and 0 in the others, which
// combine_wave_procs adds up exactly.  With one set per query head
// (row_mask: each listed row's head bits), a row outside head g's set gets
// the logit -inf for that head.  wscr: 288 floats of LDS owned by the wave.
// Products of bf16 values are exact in fp32; only the order of the fp32 sums
// differs from the vector path.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void accumulate_rows_mfma8(const DecodeParams& p, int b, int h, int hr, int lo, int nrows,
                                                      const unsigned short* rows, const int* pages, const int* ltok,
                                                      const int* lpg, float* wscr, float (&m)[8], float (&l)[8],
                                                      float (&o)[8][8], const unsigned char* row_mask = nullptr) {
  constexpr int G = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int col = lane & 15, quad = lane >> 4;   // MFMA operand lane; also (sub, proc) of the row processors
  const bool is_ret = hr >= 0;
  const bool ring = !is_ret && p.ring_rows > 0;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(ring ? p.lk_pool : p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(ring ? p.lv_pool : p.v_pool);
  const int hstride = ring ? 1 : p.Hp;
  const int hslot = ring ? 0 : p.pool_slot[h];
  const unsigned plim = ring ? (unsigned)p.ring_pages : (unsigned)p.num_blocks;
  int* rr = (p.rows_read != nullptr && col == 0 && !ring) ? p.rows_read + (size_t)(b * p.Hkv + h) * p.Nmax : nullptr;

  bf16x8 qb[4];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + h * G + (col & 7)) * D + 8 * quad;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * st);
      qb[st] = __builtin_bit_cast(bf16x8, col < G ? w : u32x4{0u, 0u, 0u, 0u});
    }
  }
  // row r of the list: its position and page; false (position 0, page 0,
  // loaded but masked) past the list or for a page outside the pool
  auto row_at = [&](int r, int& ii, int& pg) {
    const int rc = min(r, nrows - 1);
    if (is_ret) {
      const int off = rows[rc];
      ii = lo + off;
      pg = pages[off >> 4];
    } else {
      ii = ltok[rc];
      pg = lpg[rc];
    }
    const bool ok = r < nrows && (unsigned)pg < plim;
    if (!ok) { ii = 0; pg = 0; }
    return ok;
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  float m_run = NEG_INF, l_run = 0.f;            // query head col (col < 8), over the wave's rows
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.f;

  for (int r0 = wave * 32; r0 < nrows; r0 += nwaves * 32) {
    int iiA[2], pgA[2], iiV[8], pgV[8];
    bool okA[2], okV[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) okA[t] = row_at(r0 + 16 * t + col, iiA[t], pgA[t]);
#pragma unroll
    for (int u = 0; u < 8; ++u) okV[u] = row_at(r0 + 8 * quad + u, iiV[u], pgV[u]);
    if (rr != nullptr) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (okV[u]) atomicAdd(rr + iiV[u], 1);
    }
    // every load of the batch: 8 V chunks (processor rows), 8 K chunks (A rows)
    u32x4 vw[8], kw[2][4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      vw[u] = *reinterpret_cast<const u32x4*>(vpool + (((size_t)pgV[u] * hstride + hslot) * BS + (iiV[u] & 15)) * D +
                                              8 * col);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kw[t][st] = *reinterpret_cast<const u32x4*>(kpool + ((size_t)pgA[t] * hstride + hslot) * (BS * D) +
                                                    (size_t)(st * 16 + (iiA[t] & 15)) * 32 + 8 * quad);
    const unsigned okb0 = (unsigned)__ballot(okA[0]) & 0xFFFFu, okb1 = (unsigned)__ballot(okA[1]) & 0xFFFFu;

    // logits in log2 units: z[t][i] = row 16 t + 4 quad + i, query head col
    float z[2][4];
    float mx = NEG_INF;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[t][st]), qb[st], acc, 0, 0, 0);
      const unsigned okb = t ? okb1 : okb0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool keep = (okb >> (4 * quad + i)) & 1u;
        if (is_ret && row_mask != nullptr)         // one set per query head: the row's head bits
          keep = keep && ((row_mask[min(r0 + 16 * t + 4 * quad + i, nrows - 1)] >> col) & 1u);
        z[t][i] = keep ? acc[i] * p.c2_attn : NEG_INF;
        mx = fmaxf(mx, z[t][i]);
      }
    }
    float a, c;
    lane_pair<16>(mx, a, c);
    mx = fmaxf(a, c);
    lane_pair<32>(mx, a, c);
    mx = fmaxf(a, c);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[t][i] = fast_exp2(z[t][i] - m_use);
        ps += z[t][i];
      }
    lane_pair<16>(ps, a, c);
    ps = a + c;
    lane_pair<32>(ps, a, c);
    ps = a + c;
    l_run = l_run * alpha + ps;

    // weights [row][head] and the heads' rescale factors to the wave's LDS
    wave_sync();                                 // the previous batch's reads are done
    if (col < G) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) wscr[(16 * t + 4 * quad + i) * G + col] = z[t][i];
      if (quad == 0) wscr[256 + col] = alpha;
    }
    wave_sync();
    {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(wscr + 256), a1 = *reinterpret_cast<const f32x4*>(wscr + 260);
      const float al[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] *= al[g];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(wscr + (8 * quad + u) * G);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(wscr + (8 * quad + u) * G + 4);
      const float pw[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      const u32x4 w = vw[u];
      float vv[8] = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]),
                     bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
#pragma unroll
      for (int j = 0; j < 8; ++j) vv[j] = okV[u] ? vv[j] : 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pw[g], vv[j], o[g][j]);
    }
  }
  // every lane: the wave's (m, l) per head, l counted once (processor 0)
  wave_sync();
  if (col < G && quad == 0) {
    wscr[272 + col] = m_run;
    wscr[280 + col] = l_run;
  }
  wave_sync();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = wscr[272 + g];
    l[g] = quad == 0 ? wscr[280 + g] : 0.f;
  }
}

}  // namespace hws

