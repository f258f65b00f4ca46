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
  __shared__ float wo[4][MAX_G][D];

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
  constexpr int RB = AttRB<G, MODE>::value;
  if (FP8 && !is_ret && p.ring_rows > 0)         // the ring holds bf16 rows
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
// threads (one per dim) fold every MERGE_GROUPS-th split online, 16 splits'
// partials loaded at once, then group 0 combines the groups' results.

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
  constexpr int SB = 16;
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int d = threadIdx.x % D, grp = threadIdx.x / D;
  const int hr = p.ret_slot[h];
  const int nspl = hr >= 0 ? p.ncR : p.ncL;
  const int N = min(p.seq_lens[b], p.Nmax);
  const size_t base = (size_t)(b * p.Hkv + h) * p.max_splits * G + g;
  const float2* ml = p.apart_ml + base;                 // split s at ml[s * G]
  const float* po = p.apart_o + base * D + d;           // split s at po[s * G * D]
  float M = NEG_INF, L = 0.f, O = 0.f;
  for (int s0 = grp; s0 < nspl; s0 += SB * MERGE_GROUPS) {
    float2 v[SB];
    float ov[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int sp = s0 + u * MERGE_GROUPS;
      const bool in = sp < nspl;
      v[u] = in ? ml[(size_t)sp * G] : make_float2(NEG_INF, 0.f);
      ov[u] = in ? po[(size_t)sp * G * D] : 0.f;
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
  return p.max_splits >= 128 ? launch_merge_mg<8>(p, s, e0, e1) : launch_merge_mg<4>(p, s, e0, e1);
}

hipError_t launch_prep_q(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(prep_q_kernel, dim3(p.Hq, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
