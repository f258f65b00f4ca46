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
// page is pages[offset / 16]; local rows are at index ltok[r] of page lpg[r]
// (local_row_at), in the ring pools when there is a ring.
// MODE 0: logits q.k from K rows; MODE 1: retrieval heads only, logits from
// the stored full-dim scores; MODE 2: both (scores for retrieval heads).
// RET: the rows are known to be a retrieval head's (no K path compiled in).
// lds_logits (full-dim scores only): the scores of row r at lds_logits[r*G];
// null reads them from the scores buffer at the row's position.
// row_mask (retrieval rows, one set per query head): bit g of row_mask[r] says
// whether query head g keeps row r; null means every head keeps every row.
template <int G, bool FP8, int MODE, int RB, bool RET = false, bool ROW_ORDER = FP8>
__device__ __forceinline__ void accumulate_rows(const DecodeParams& p, int b, int h, int hr, int lo, int nrows,
                                                int r_begin, int r_step, int sub, const unsigned short* rows,
                                                const int* pages, const int* ltok, const int* lpg,
                                                const float* lds_logits, float (&m)[G], float (&l)[G],
                                                float (&o)[G][8], const unsigned char* row_mask = nullptr) {
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
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = NEG_INF;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
  }

  for (int r0 = r_begin; r0 < nrows; r0 += r_step) {
    int ii[RB], pg[RB];
    bool ok[RB];
    if (is_ret) {
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

}  // namespace hws
