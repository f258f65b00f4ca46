// Split-K decode attention over a token set, and the log-sum-exp merge of the
// splits.
//
// Retrieval heads ([ICS] "Inference-time context sparsity: illusion or
// opportunity?", §3c: sparse decode reads only the selected rows, O(k d)
// instead of O(N d)): a workgroup owns a chunk of positions, keeps the tokens
// of the chunk that pass the threshold found by the selection passes
// (a_i > t*, or a_i == t* -- for top-k only the lowest-position ties up to the
// budget), and gathers their K/V rows through the block table.  In FULL score
// mode the attention logits are the stored full-dim scores, so only V rows
// are read.
//
// Local heads ([RTPurbo] "Full attention returns in force ...", Methodology §1;
// [AoH] "Autonomy-of-Heads ...", Methodology §4): the rows are the sinks
// 0..n_sink-1 followed by the window N-w..N-1 (a position in both once),
// split into chunks of LOCAL_CHUNK rows.
//
// Each workgroup produces (max, sum, unnormalised output) per query head in
// log2 units; merge_kernel combines them.
#include <algorithm>
#include <mutex>
#include <vector>

#include "attend_rows.h"

namespace hws {

constexpr int ATT_ROWS_MAX = 4096;   // largest retrieval chunk (LDS row list)

// Exclusive scan of a per-thread count over a 256-thread block; total in tmp[4].
__device__ __forceinline__ unsigned int block_excl_scan256(unsigned int v, unsigned int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  unsigned int off = 0;
  for (int w = 0; w < wave; ++w) off += tmp[w];
  const unsigned int tot = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  if (tid == 0) tmp[4] = tot;
  __syncthreads();
  return off + inc - v;
}

// Ties at t* in positions [0, lo) of one (b, retrieval head).  Only reached
// for top-k when the ties at the threshold exceed the budget.
__device__ unsigned int ties_before(const float* agg, int lo, unsigned int tstar, unsigned int* tmp) {
  unsigned int cnt = 0;
  for (int i = threadIdx.x; i < lo; i += 256) cnt += (__float_as_uint(agg[i]) == tstar) ? 1u : 0u;
  block_excl_scan256(cnt, tmp);
  const unsigned int tot = tmp[4];
  __syncthreads();
  return tot;
}

// MODE 0: rows need K (index scoring or local heads); MODE 1: FULL scoring and
// retrieval heads only (logits from the stored scores, V rows only);
// MODE 2: FULL scoring with local heads present (both paths).
template <int G, bool FP8, int MODE>
__global__ __launch_bounds__(256) void attend_kernel(DecodeParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int proc = tid >> 4, sub = tid & 15;     // 16 row processors of 16 lanes
  const int w = blockIdx.x;
  const int nret = p.B * p.nR * p.ncR;
  int b, h, split, hr = -1, lh = 0;              // lh: local head number
  if (w < nret) {
    split = w % p.ncR;
    const int t = w / p.ncR;
    hr = t % p.nR;
    b = t / p.nR;
    h = p.ret_head[hr];
  } else {
    const int w2 = w - nret;
    split = w2 % p.ncL;
    const int t = w2 / p.ncL;
    b = t / p.nL;
    lh = t % p.nL;
    h = p.loc_head[lh];
  }
  const bool is_ret = hr >= 0;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int* bt = p.block_tables + (size_t)b * p.max_blocks;

  __shared__ unsigned short rows_s[ATT_ROWS_MAX];   // retrieval: offset in the chunk
  __shared__ unsigned char rmask_s[ATT_ROWS_MAX];   // retrieval, one set per query head: head bits
  __shared__ int pages_s[LOCAL_CHUNK];              // retrieval: chunk pages; local: row pages
  __shared__ int ltok_s[LOCAL_CHUNK];               // local: row tokens
  __shared__ unsigned int tmp[8];
  __shared__ float wm[4][MAX_G], wl[4][MAX_G];
  __shared__ __align__(16) float wo[4][MAX_G][D];   // (also the MFMA path's per-wave weights)

  int nrows = 0, lo = 0;
  if (is_ret) {
    const int chunk = p.att_chunk_R;
    const int per = chunk / 256;                 // 4, 8 or 16 positions per thread
    lo = split * chunk;
    const int hi = min(N, lo + chunk);
    if (lo < hi) {
      const int i0 = lo + tid * per;
      const int npg = (hi - lo + BS - 1) / BS;
      if (tid < npg) pages_s[tid] = bt[(lo >> 4) + tid];
      // kept by any of the GS sets; with one set per query head, hb holds
      // each position's head bits (one byte per position, 4 per word)
      unsigned int keep_any = 0u, hb[4] = {0u, 0u, 0u, 0u};
      for (int gs = 0; gs < p.GS; ++gs) {
        const size_t srow = ((size_t)b * p.nR + hr) * p.GS + gs;
        SelState* st = p.sel + srow;
        const unsigned int tstar = st->tstar, flags = st->flags;
        const float* agg = p.agg + srow * p.Nagg;
        float av[16];
        if (i0 + per <= hi) {
          for (int j = 0; j < per; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(agg + i0 + j);
            av[j] = v.x; av[j + 1] = v.y; av[j + 2] = v.z; av[j + 3] = v.w;
          }
        } else {
          for (int j = 0; j < per; ++j) av[j] = (i0 + j < hi) ? agg[i0 + j] : -1.0f;
        }
        unsigned int gt_mask = 0, eq_mask = 0;
        for (int j = 0; j < per; ++j) {
          const unsigned int bits = __float_as_uint(av[j]);
          if (i0 + j < hi) {
            if (bits > tstar) gt_mask |= 1u << j;
            else if (bits == tstar) eq_mask |= 1u << j;
          }
        }
        if (flags & SEL_TIE) {
          // keep a tie only while its position-ordered rank stays below the quota
          const unsigned int before = ties_before(agg, lo, tstar, tmp);
          const unsigned int quota = st->quota;
          const unsigned int myrank = block_excl_scan256((unsigned int)__popc(eq_mask), tmp) + before;
          unsigned int r = myrank, keep = 0;
          for (int j = 0; j < per; ++j)
            if (eq_mask & (1u << j)) { if (r < quota) keep |= 1u << j; ++r; }
          eq_mask = keep;
        }
        const unsigned int kept = gt_mask | eq_mask;
        // kept mass, unless the single-launch selection already summed it
        if (p.sel_mass != nullptr && !p.agg_out) add_kept_mass(&st->kept_mass, av, kept);
        if (p.select_mode == 0) {                  // top-p: |S| summed over chunks
          block_excl_scan256((unsigned int)__popc(kept), tmp);
          if (tid == 0 && tmp[4] > 0u) atomicAdd(&st->nsel, tmp[4]);
          __syncthreads();
        }
        if (p.GS > 1) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if ((kept >> j) & 1u) hb[j >> 2] |= (1u << gs) << ((j & 3) * 8);
        }
        keep_any |= kept;
      }
      const unsigned int off = block_excl_scan256((unsigned int)__popc(keep_any), tmp);
      nrows = (int)tmp[4];
      unsigned int k = off;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < per && (keep_any & (1u << j))) {
          rows_s[k] = (unsigned short)(i0 + j - lo);
          rmask_s[k] = (unsigned char)((hb[j >> 2] >> ((j & 3) * 8)) & 0xFFu);
          ++k;
        }
      __syncthreads();
    }
  } else if (MODE != 1) {
    const int L1 = min(p.n_sink, N);
    const int start2 = max(L1, N - p.window);
    const int L = L1 + (N - start2);
    const int llo = split * LOCAL_CHUNK;
    const int hi = min(L, llo + LOCAL_CHUNK);
    const int r = llo + tid;
    if (r < hi) {
      local_row_at(p, b, lh, r < L1 ? r : start2 + (r - L1), ltok_s[tid], pages_s[tid]);
    }
    nrows = max(0, hi - llo);
    __syncthreads();
  }

  float2* ml = p.apart_ml + ((size_t)(b * p.Hkv + h) * p.max_splits + split) * G;
  float* po = p.apart_o + (((size_t)(b * p.Hkv + h) * p.max_splits + split) * G) * D;
  if (nrows == 0) {
    if (tid < G) ml[tid] = make_float2(NEG_INF, 0.f);
    return;
  }
  float m[G], l[G], o[G][8];
  // (G = 8 with K rows: 4 rows per processor per batch here, where the
  // kernel has the registers for them; the single launches keep 2)
  constexpr int RB = (G == 8 && MODE == 0) ? 4 : AttRB<G, MODE>::value;
  // (G = 8, bf16 rows, queries not rotated: the dot products on the matrix
  // cores; with one set per query head each row's head bits mask its logits)
  bool mfma_rows = false;
  if constexpr (G == 8 && MODE == 0 && !FP8) {
    if (p.qrot == nullptr) {
      accumulate_rows_mfma8(p, b, h, hr, lo, nrows, rows_s, pages_s, ltok_s, pages_s, &wo[wave][0][0], m, l, o,
                            p.GS > 1 ? rmask_s : nullptr);
      mfma_rows = true;
    }
  }
  if (mfma_rows) {
  } else if (FP8 && !is_ret && p.ring_rows > 0)  // the ring holds bf16 rows
    accumulate_rows<G, false, MODE, RB, false, true>(p, b, h, hr, lo, nrows, proc * RB, 16 * RB, sub, rows_s,
                                                     pages_s, ltok_s, pages_s, nullptr, m, l, o, nullptr);
  else
    accumulate_rows<G, FP8, MODE, RB>(p, b, h, hr, lo, nrows, proc * RB, 16 * RB, sub, rows_s, pages_s, ltok_s,
                                      pages_s, nullptr, m, l, o, p.GS > 1 ? rmask_s : nullptr);
  combine_wave_procs<G>(m, l, o);
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
#pragma unroll
      for (int j = 0; j < 8; ++j) wo[wave][g][8 * sub + j] = o[g][j];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, d = e % D;
    float mm = NEG_INF;
    for (int k = 0; k < 4; ++k) mm = fmaxf(mm, wm[k][g]);
    float ll = 0.f, oo = 0.f;
    for (int k = 0; k < 4; ++k) {
      if (wm[k][g] == NEG_INF) continue;
      const float cf = fast_exp2(wm[k][g] - mm);
      ll += wl[k][g] * cf;
      oo += wo[k][g][d] * cf;
    }
    po[(size_t)g * D + d] = oo;
    if (d == 0) ml[g] = make_float2(mm, ll);
  }
}

// out_g = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M);  lse = (M + log2 L) ln 2.
// One workgroup per (sequence, KV head, query head): MERGE_GROUPS groups of D
// threads (one per dim) fold every MERGE_GROUPS-th split online, 16 (32 with
// 8 groups) splits' partials loaded at once, then group 0 combines the groups'
// results.

__device__ __forceinline__ void merge_fold(float& M, float& L, float& O, float m2, float l2, float o2) {
  if (!(l2 > 0.f)) return;                              // empty splits left no output
  const float mt = fmaxf(M, m2);
  const float c1 = fast_exp2(M - mt), c2 = fast_exp2(m2 - mt);   // c1 = 0 while nothing was folded in
  L = L * c1 + l2 * c2;
  O = O * c1 + o2 * c2;
  M = mt;
}

template <int G, int MERGE_GROUPS>
__global__ __launch_bounds__(D * MERGE_GROUPS) void merge_kernel(DecodeParams p) {
  constexpr int SB = MERGE_GROUPS >= 8 ? 32 : 16;
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int d = threadIdx.x % D, grp = threadIdx.x / D;
  const int hr = p.ret_slot[h];
  const int N = min(p.seq_lens[b], p.Nmax);
  int nspl;
  const float2* ml;                                     // split s at ml[s * G]
  const float* po;                                      // split s at po[s * G * D]
  if (p.item_base != nullptr) {                         // balanced attention: this pair's pieces
    const int pi = b * p.Hkv + h;
    const int x0 = p.item_base[pi] + BAL_PIECE_COST, x1 = p.item_base[pi + 1], len = p.item_base[p.B * p.Hkv + 1];
    const int w0 = x0 / len;                            // the workgroups holding its rows' cost units
    nspl = x1 > x0 ? (x1 - 1) / len - w0 + 1 : 0;
    ml = p.bal_ml + (size_t)(w0 + pi) * G + g;
    po = p.bal_o + ((size_t)(w0 + pi) * G + g) * D + d;
  } else {
    nspl = hr >= 0 ? p.ncR : p.ncL;
    const size_t base = (size_t)(b * p.Hkv + h) * p.max_splits * G + g;
    ml = p.apart_ml + base;
    po = p.apart_o + base * D + d;
  }
  float M = NEG_INF, L = 0.f, O = 0.f;
  for (int s0 = grp; s0 < nspl; s0 += SB * MERGE_GROUPS) {
    float2 v[SB];
    float ov[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      // unconditional loads (clamped split, masked after): a load behind a
      // per-lane branch would be waited for before the next one is issued
      const int sp = s0 + u * MERGE_GROUPS;
      const bool in = sp < nspl;
      const int spc = min(sp, nspl - 1);
      const float2 mv = ml[(size_t)spc * G];
      const float pv = po[(size_t)spc * G * D];
      v[u] = in ? mv : make_float2(NEG_INF, 0.f);
      ov[u] = in ? pv : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) merge_fold(M, L, O, v[u].x, v[u].y, ov[u]);
  }
  __shared__ float gm[MERGE_GROUPS], gl[MERGE_GROUPS], go[MERGE_GROUPS][D];
  if (d == 0) { gm[grp] = M; gl[grp] = L; }
  go[grp][d] = O;
  __syncthreads();
  if (grp != 0) return;
  for (int k = 1; k < MERGE_GROUPS; ++k) merge_fold(M, L, O, gm[k], gl[k], go[k][d]);
  // (a single-launch selection that gave up a wait leaves the error word set)
  const bool bad = p.agg_out && __hip_atomic_load(&p.tail_sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
  const float nan = __builtin_nanf("");
  p.out[((size_t)b * p.Hq + h * G + g) * D + d] = bad ? nan : (L > 0.f ? O / L : 0.f);
  if (d == 0 && p.lse != nullptr) p.lse[(size_t)b * p.Hq + h * G + g] = bad ? nan : (M + log2f(L)) * LN2;
  // |S| per KV head, or per query head with one set per query head
  if ((g == 0 || p.GS > 1) && d == 0 && p.sel_counts != nullptr) {
    int cnt;
    if (hr >= 0) {
      cnt = (int)p.sel[((size_t)b * p.nR + hr) * p.GS + (p.GS > 1 ? g : 0)].nsel;
    } else {
      const int L1 = min(p.n_sink, N);
      cnt = L1 + (N - max(L1, N - p.window));
    }
    if (p.GS > 1) p.sel_counts[(size_t)b * p.Hq + h * G + g] = cnt;
    else p.sel_counts[(size_t)b * p.Hkv + h] = cnt;
  }
  if ((g == 0 || p.GS > 1) && d == 0 && p.sel_mass != nullptr) {
    const float mv = hr >= 0 ? mass_value(p.sel[((size_t)b * p.nR + hr) * p.GS + (p.GS > 1 ? g : 0)].kept_mass)
                             : __builtin_nanf("");
    if (p.GS > 1) p.sel_mass[(size_t)b * p.Hq + h * G + g] = mv;
    else p.sel_mass[(size_t)b * p.Hkv + h] = mv;
  }
}

// ---------------------------------------------------------------------------
// Attention balanced by kept rows ([ICS] §2: the sparsity is irregular per
// token, query and head, so chunks cut by position leave a few dense ones as
// the long pole).  The (sequence, KV head) pairs -- pair i = b * Hkv + h has
// c_i rows, the kept rows the selection listed (retrieval; tile j's rows at
// j * TAIL_TILE in the head's list) or its sinks and window (local) -- are
// laid end to end in pair order in cost units, pair i
// costing BAL_PIECE_COST + c_i (its rows take the last c_i units), and the
// total is cut into equal segments, one per resident workgroup: so a segment
// that covers several pairs, each a piece with its own list, queries and
// partial, gathers fewer rows.  A workgroup walks its pieces, loads each
// piece's (position, page) list into LDS, gathers it with the next batch of
// loads in flight, and stores one partial per piece.  Pieces form a monotone
// path over (workgroup w, pair i), so w + i numbers them without collisions;
// pair i's partials are w_first(i) + i .. w_last(i) + i, the workgroups that
// hold its first and last row.  Workgroup 0 writes the pair offsets and the
// segment length for the merge.  Index scores only (the rows carry K and V),
// one set per KV head.
// ---------------------------------------------------------------------------
constexpr int BAL_THREADS = 256;
constexpr int BAL_LIST = 1024;                // rows per (position, page) list in LDS
constexpr int BAL_TABLE = BAL_MAX_HEADS;      // pairs the LDS table holds

// In-place exclusive scan of x[0..n) (n <= BAL_TABLE) over a 256-thread
// block; returns the total.
__device__ int block_scan_excl(int* x, int n, int* tmp) {
  constexpr int PER = BAL_TABLE / BAL_THREADS;  // 8 entries per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[PER], run = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    v[k] = i < n ? x[i] : 0;
    run += v[k];
  }
  int inc = run;
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int base = inc - run;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  const int total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    if (i < n) x[i] = base;
    base += v[k];
  }
  __syncthreads();
  return total;
}

// Rows of pair (b, h): the kept rows the selection listed (the sum over the
// head's selection tiles), or the sinks and window.
__device__ __forceinline__ int pair_row_count(const DecodeParams& p, int b, int h) {
  const int hr = p.ret_slot[h];
  if (hr >= 0) {
    const unsigned int* tc = p.tile_cnt + ((size_t)b * p.nR + hr) * p.tail_tph;
    int c = 0;
    for (int j = 0; j < p.tail_tph; ++j) c += (int)tc[j];
    return c;
  }
  const int N = min(p.seq_lens[b], p.Nmax);
  const int L1 = min(p.n_sink, N);
  return L1 + (N - max(L1, N - p.window));
}



// RING_BF16: fp8 pools with the local heads in a (bf16) ring.  MARK: count
// the rows read (debug).  The fp8 gather at G <= 4 is held to 3 waves per
// SIMD (it fits in 168 registers; one wave more in flight per SIMD).
template <int G, bool FP8, bool RING_BF16, bool MARK>
struct BalWaves { static constexpr int value = (FP8 && G <= 4 && !RING_BF16 && !MARK) ? 3 : 1; };

template <int G, bool FP8, bool RING_BF16, bool MARK>
__global__ __launch_bounds__(BAL_THREADS) __attribute__((amdgpu_waves_per_eu(BalWaves<G, FP8, RING_BF16, MARK>::value)))
void attend_balanced_kernel(DecodeParams p) {
  constexpr int RB = AttRB<G, 0>::value;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int proc = tid >> 4, sub = tid & 15;
  const int npairs = p.B * p.Hkv;
  __shared__ int base_s[BAL_TABLE + 1];
  __shared__ int tmp[8];
  __shared__ int tok_s[BAL_LIST], pg_s[BAL_LIST];
  __shared__ int tpre_s[BAL_MAX_TPH + 1];       // retrieval piece: kept rows before each selection tile
  __shared__ float wm[4][MAX_G], wl[4][MAX_G];
  __shared__ float wo[4][MAX_G][D];

  stamp_phase(p, 0);
  // ---- pair offsets in cost units (the same in every workgroup): a pair
  // with c rows costs BAL_PIECE_COST + c, its rows taking the last c units ----
  for (int i = tid; i < npairs; i += BAL_THREADS) {
    const int c = pair_row_count(p, i / p.Hkv, i % p.Hkv);
    base_s[i] = c > 0 ? c + BAL_PIECE_COST : 0;
  }
  __syncthreads();
  const int C = block_scan_excl(base_s, npairs, tmp);
  if (tid == 0) base_s[npairs] = C;
  __syncthreads();
  const int per = (C + (int)gridDim.x - 1) / (int)gridDim.x;
  const int len = max(BAL_RMIN, (per + 16 * RB - 1) / (16 * RB) * (16 * RB));
  if (blockIdx.x == 0) {
    for (int i = tid; i <= npairs; i += BAL_THREADS) p.item_base[i] = base_s[i];
    if (tid == 0) p.item_base[npairs + 1] = len;
  }
  const int x0 = (int)blockIdx.x * len;
  const int x1 = min(C, x0 + len);
  stamp_phase(p, 1);
  if (x0 >= x1) return;
  // the pair holding cost unit x0: the last i with base_s[i] <= x0 (empty pairs skipped)
  int pi = 0;
  {
    int lo_i = 0, hi_i = npairs;
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (base_s[mid] <= x0) lo_i = mid; else hi_i = mid;
    }
    pi = lo_i;
  }
  for (int x = x0; x < x1; ++pi) {
    if (base_s[pi + 1] <= x) continue;              // empty pair
    const int rb = base_s[pi] + BAL_PIECE_COST;     // cost unit of the pair's row 0
    if (x1 <= rb) break;                            // the segment ends before the pair's rows
    const int r0 = max(x, rb) - rb, r1 = min(x1, base_s[pi + 1]) - rb;
    x = base_s[pi + 1];
    // ---- one piece: rows r0..r1-1 of pair pi ----
    const int b = pi / p.Hkv, h = pi % p.Hkv, hr = p.ret_slot[h];
    const int N = min(p.seq_lens[b], p.Nmax);
    const int L1 = min(p.n_sink, N), start2 = max(L1, N - p.window);
    const bool ring = hr < 0 && p.ring_rows > 0;
    GatherSrc src;
    src.kpool = ring ? p.lk_pool : p.k_pool;
    src.vpool = ring ? p.lv_pool : p.v_pool;
    src.scales = p.kv_scales;
    src.hstride = ring ? 1 : p.Hp;
    src.hslot = ring ? 0 : p.pool_slot[h];
    src.plim = ring ? (unsigned)p.ring_pages : (unsigned)p.num_blocks;
    const int2* list = hr >= 0 ? p.row_list + ((size_t)b * p.nR + hr) * p.Nmax : nullptr;
    const int tph = p.tail_tph;
    if (hr >= 0) {                                  // where each tile's rows start in the pair's order
      const unsigned int* tc = p.tile_cnt + ((size_t)b * p.nR + hr) * tph;
      for (int j = tid; j < tph; j += BAL_THREADS) tpre_s[j + 1] = (int)tc[j];
      __syncthreads();
      if (tid == 0) {
        tpre_s[0] = 0;
        for (int j = 1; j <= tph; ++j) tpre_s[j] += tpre_s[j - 1];
      }
      __syncthreads();
    }
    float qf[G][8], m[G], l[G], o[G][8];
    load_group_q<G>(p, b, h, sub, qf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = NEG_INF;
      l[g] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
    }
    for (int rs = r0; rs < r1; rs += BAL_LIST) {
      const int nl = min(BAL_LIST, r1 - rs);
      for (int q = tid; q < nl; q += BAL_THREADS) {
        const int r = rs + q;
        if (hr >= 0) {                              // row r lies in tile j: the last with tpre_s[j] <= r
          int lo_j = 0, hi_j = tph;
          while (hi_j - lo_j > 1) {
            const int mid = (lo_j + hi_j) >> 1;
            if (tpre_s[mid] <= r) lo_j = mid; else hi_j = mid;
          }
          const int2 e = list[(size_t)lo_j * TAIL_TILE + (r - tpre_s[lo_j])];
          tok_s[q] = e.x;
          pg_s[q] = e.y;
        } else {
          local_row_at(p, b, p.loc_slot[h], r < L1 ? r : start2 + (r - L1), tok_s[q], pg_s[q]);
        }
      }
      __syncthreads();
      stamp_phase(p, 8);
      if (RING_BF16 && ring) {                      // the ring holds bf16 rows (not counted)
        gather_pipelined<G, false, RB>(src, tok_s, pg_s, nl, proc, sub, qf, m, l, o);
      } else {
        int* rr = MARK ? p.rows_read + (size_t)(b * p.Hkv + h) * p.Nmax : nullptr;
        gather_pipelined<G, FP8, RB, MARK>(src, tok_s, pg_s, nl, proc, sub, qf, m, l, o, rr);
      }
      __syncthreads();                              // the list is reused
      stamp_phase(p, 9);
    }
    // the piece's partial at slot w + i
    combine_wave_procs<G>(m, l, o);
    if (lane < 16) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
#pragma unroll
        for (int j = 0; j < 8; ++j) wo[wave][g][8 * sub + j] = o[g][j];
      }
    }
    __syncthreads();
    const size_t slot = (size_t)blockIdx.x + pi;
    float2* ml = p.bal_ml + slot * G;
    float* po = p.bal_o + slot * G * D;
    for (int e = tid; e < G * D; e += BAL_THREADS) {
      const int g = e / D, d = e % D;
      float mm = NEG_INF;
      for (int k = 0; k < 4; ++k) mm = fmaxf(mm, wm[k][g]);
      float ll = 0.f, oo = 0.f;
      for (int k = 0; k < 4; ++k) {
        if (wm[k][g] == NEG_INF) continue;
        const float cf = fast_exp2(wm[k][g] - mm);
        ll += wl[k][g] * cf;
        oo += wo[k][g][d] * cf;
      }
      po[(size_t)g * D + d] = oo;
      if (d == 0) ml[g] = make_float2(mm, ll);
    }
    __syncthreads();                                // wm / wo are reused by the next piece
  }
  stamp_phase(p, 10);
}

// ---------------------------------------------------------------------------
// Dense log-sum-exp (diagnostic): every cached row of every KV head, q.k for
// the group's query heads, online (max, sum of 2^x) per query head.  One
// workgroup per (DENSE_CHUNK rows, KV head, sequence); its 16 processors take
// every 16th row, RB rows per batch with all loads in flight.
// ---------------------------------------------------------------------------
template <int G, bool FP8>
__global__ __launch_bounds__(256) void dense_lse_kernel(DecodeParams p) {
  constexpr int RB = 4;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, proc = tid >> 4, sub = tid & 15, lane = tid & 63, wave = tid >> 6;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int lo = c * DENSE_CHUNK, hi = min(N, lo + DENSE_CHUNK);
  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  float qf[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t qo = ((size_t)b * p.Hq + h * G + g) * D + 8 * sub;
    if (p.qrot != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[g][j] = p.qrot[qo + j];
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(p.q + qo);
      qf[g][0] = bf16_lo(u.x); qf[g][1] = bf16_hi(u.x); qf[g][2] = bf16_lo(u.y); qf[g][3] = bf16_hi(u.y);
      qf[g][4] = bf16_lo(u.z); qf[g][5] = bf16_hi(u.z); qf[g][6] = bf16_lo(u.w); qf[g][7] = bf16_hi(u.w);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[g][j] *= p.c2_attn;
  }
  float m[G], s[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = NEG_INF; s[g] = 0.f; }
  const int hslot = p.pool_slot[h];
  for (int r0 = lo + proc * RB; r0 < hi; r0 += 16 * RB) {
    float kx[RB][8], ks[RB];
    bool ok[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int i = min(r0 + u, hi - 1);
      int pg = bt[i >> 4];
      ok[u] = r0 + u < hi && (unsigned)pg < (unsigned)p.num_blocks;
      if (!ok[u]) pg = 0;
      load_krow8<FP8>(p.k_pool, (size_t)pg * p.Hp + hslot, i & 15, sub, kx[u]);
      ks[u] = FP8 ? p.kv_scales[((size_t)pg * p.Hp + hslot) * 2] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = qf[g][0] * kx[u][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) a = fmaf(qf[g][j], kx[u][j], a);
        a = row16_sum(a) * ks[u];
        if (ok[u]) {
          const float mn = fmaxf(m[g], a);
          s[g] = s[g] * fast_exp2(m[g] - mn) + fast_exp2(a - mn);
          m[g] = mn;
        }
      }
    }
  }
  // the 64 lanes of a wave hold 4 processors (every lane of a processor the
  // same values), then the 4 waves
  __shared__ float wm[4][MAX_G], ws[4][MAX_G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    for (int off = 16; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m[g], off), s2 = __shfl_xor(s[g], off);
      lse_combine(m[g], s[g], m2, s2);
    }
    if (lane == 0) { wm[wave][g] = m[g]; ws[wave][g] = s[g]; }
  }
  __syncthreads();
  if (tid < G) {
    float mm = wm[0][tid], ss = ws[0][tid];
    for (int w = 1; w < 4; ++w) lse_combine(mm, ss, wm[w][tid], ws[w][tid]);
    p.spart[(((size_t)b * p.Hkv + h) * p.n_score_chunks + c) * G + tid] = make_float2(mm, ss);
  }
}

template <int G>
__global__ __launch_bounds__(64) void dense_lse_reduce_kernel(DecodeParams p, float* lse_full) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nch = (N + DENSE_CHUNK - 1) / DENSE_CHUNK;
  for (int g = 0; g < G; ++g) {
    float m = NEG_INF, s = 0.f;
    for (int c = lane; c < nch; c += 64) {
      const float2 v = p.spart[(((size_t)b * p.Hkv + h) * p.n_score_chunks + c) * G + g];
      lse_combine(m, s, v.x, v.y);
    }
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      lse_combine(m, s, m2, s2);
    }
    if (lane == 0) lse_full[(size_t)b * p.Hq + h * G + g] = (m + log2f(s)) * LN2;
  }
}

template <int G>
static hipError_t launch_dense_lse_g(const DecodeParams& p, float* lse_full, hipStream_t s) {
  const dim3 grid(p.n_score_chunks, p.Hkv, p.B);
  if (p.kv_scales != nullptr) hipLaunchKernelGGL((dense_lse_kernel<G, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((dense_lse_kernel<G, false>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_lse_reduce_kernel<G>, dim3(p.Hkv, p.B), dim3(64), 0, s, p, lse_full);
  return hipGetLastError();
}

hipError_t launch_dense_lse(const DecodeParams& p, float* lse_full, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_dense_lse_g<1>(p, lse_full, s);
    case 2: return launch_dense_lse_g<2>(p, lse_full, s);
    case 4: return launch_dense_lse_g<4>(p, lse_full, s);
    case 8: return launch_dense_lse_g<8>(p, lse_full, s);
  }
  return hipErrorInvalidValue;
}

// Debug row-read counters back to zero before a step (n int32 values).
__global__ __launch_bounds__(256) void clear_i32_kernel(int* x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0;
}

// The step's status: whether a hand-off wait of the single launch gave up.
__global__ void step_status_kernel(const unsigned int* err, int* status, int waited) {
  if (threadIdx.x == 0)
    *status = (waited && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) ? 1 : 0;
}

// Rotated fp32 queries at position N-1 (rotate-half pairs (j, j+64)); the
// angle and rotation are evaluated in fp64.
__global__ __launch_bounds__(64) void prep_q_kernel(DecodeParams p) {
  const int hq = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const double inv = pow((double)p.rope_theta, -2.0 * (double)j / (double)D);
  const double ang = (double)(N - 1) * inv;
  double sn, cs;
  sincos(ang, &sn, &cs);
  const size_t o = ((size_t)b * p.Hq + hq) * D;
  const double x1 = bf16_to_f32(p.q[o + j]);
  const double x2 = bf16_to_f32(p.q[o + j + D / 2]);
  p.qrot[o + j] = (float)(x1 * cs - x2 * sn);
  p.qrot[o + j + D / 2] = (float)(x2 * cs + x1 * sn);
}

template <int G, bool FP8>
static hipError_t launch_attend_g(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nwg = p.B * (p.nR * p.ncR + p.nL * p.ncL);
  const dim3 grid(nwg), blk(256);
  if (p.score_mode != 1) return launch_kernel(attend_kernel<G, FP8, 0>, grid, blk, s, e0, e1, p);
  if (p.nL == 0) return launch_kernel(attend_kernel<G, FP8, 1>, grid, blk, s, e0, e1, p);
  return launch_kernel(attend_kernel<G, FP8, 2>, grid, blk, s, e0, e1, p);
}

template <int G>
static hipError_t launch_attend_fp(const DecodeParams& p, hipStream_t s, bool fp8, hipEvent_t e0, hipEvent_t e1) {
  return fp8 ? launch_attend_g<G, true>(p, s, e0, e1) : launch_attend_g<G, false>(p, s, e0, e1);
}

hipError_t launch_attend(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const bool fp8 = p.kv_scales != nullptr;
  switch (p.G) {
    case 1: return launch_attend_fp<1>(p, s, fp8, e0, e1);
    case 2: return launch_attend_fp<2>(p, s, fp8, e0, e1);
    case 4: return launch_attend_fp<4>(p, s, fp8, e0, e1);
    case 8: return launch_attend_fp<8>(p, s, fp8, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int MG>
static hipError_t launch_merge_mg(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.G, p.Hkv, p.B), blk(D * MG);
  switch (p.G) {
    case 1: return launch_kernel(merge_kernel<1, MG>, grid, blk, s, e0, e1, p);
    case 2: return launch_kernel(merge_kernel<2, MG>, grid, blk, s, e0, e1, p);
    case 4: return launch_kernel(merge_kernel<4, MG>, grid, blk, s, e0, e1, p);
    case 8: return launch_kernel(merge_kernel<8, MG>, grid, blk, s, e0, e1, p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // many splits (a long context in few workgroups' worth of heads): 8 groups
  // of threads per output row halve the serial load rounds; otherwise 4
  // (the balanced attention spreads the dense head of a small batch over
  // most workgroups; a large batch leaves every head a few pieces)
  const bool many = p.max_splits >= 128 || (p.item_base != nullptr && p.B * p.Hkv < BAL_AUTO_PAIRS);
  return many ? launch_merge_mg<8>(p, s, e0, e1) : launch_merge_mg<4>(p, s, e0, e1);
}

// Workgroups of `fn` the device holds at once (cached per kernel and device).
static int resident_wgs(const void* fn, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  struct Entry { const void* fn; int dev; int nwg; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.fn == fn && e.dev == dev) return e.nwg;
  int ncu = 0, occ = 0, nwg = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads, 0) == hipSuccess)
    nwg = ncu * occ;
  cache.push_back(Entry{fn, dev, nwg});
  return nwg;
}

template <typename K>
static hipError_t launch_balanced(K kernel, const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // one segment per workgroup the device holds at once: every segment starts
  // at once and none waits for a free slot
  int nwg = resident_wgs(reinterpret_cast<const void*>(kernel), BAL_THREADS);
  if (nwg <= 0) nwg = 512;
  const dim3 grid(std::max(1, std::min(nwg, BAL_ITEMS))), blk(BAL_THREADS);
  return launch_kernel(kernel, grid, blk, s, e0, e1, p);
}

template <int G>
static hipError_t launch_attend_balanced_g(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const bool mark = p.rows_read != nullptr;
  if (p.kv_scales == nullptr)
    return mark ? launch_balanced(attend_balanced_kernel<G, false, false, true>, p, s, e0, e1)
                : launch_balanced(attend_balanced_kernel<G, false, false, false>, p, s, e0, e1);
  if (p.ring_rows > 0 && p.nL > 0)
    return mark ? launch_balanced(attend_balanced_kernel<G, true, true, true>, p, s, e0, e1)
                : launch_balanced(attend_balanced_kernel<G, true, true, false>, p, s, e0, e1);
  return mark ? launch_balanced(attend_balanced_kernel<G, true, false, true>, p, s, e0, e1)
              : launch_balanced(attend_balanced_kernel<G, true, false, false>, p, s, e0, e1);
}

hipError_t launch_attend_balanced(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.B * p.Hkv > BAL_TABLE) return hipErrorInvalidValue;
  switch (p.G) {
    case 1: return launch_attend_balanced_g<1>(p, s, e0, e1);
    case 2: return launch_attend_balanced_g<2>(p, s, e0, e1);
    case 4: return launch_attend_balanced_g<4>(p, s, e0, e1);
    case 8: return launch_attend_balanced_g<8>(p, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_clear_rows_read(const DecodeParams& p, hipStream_t s) {
  const size_t n = (size_t)p.B * p.Hkv * p.Nmax;
  const int nwg = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(clear_i32_kernel, dim3(nwg), dim3(256), 0, s, p.rows_read, n);
  return hipGetLastError();
}

hipError_t launch_step_status(const DecodeParams& p, int* status, bool waited, hipStream_t s) {
  hipLaunchKernelGGL(step_status_kernel, dim3(1), dim3(64), 0, s, (const unsigned int*)p.tail_sync, status,
                     waited ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_prep_q(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(prep_q_kernel, dim3(p.Hq, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
