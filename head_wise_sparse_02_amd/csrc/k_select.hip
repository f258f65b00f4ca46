// Threshold selection of retrieval heads without sorting.
//
// [RTPurbo] "Full attention returns in force ...", Methodology §3: attention
// mass is accumulated from the largest value down until a cumulative p is
// reached (top-p), against a fixed budget k (top-k); Methodology §5: the
// threshold is found with histograms instead of a sort.
//
// Per (sequence, retrieval head) with aggregate a_i = mean_g 2^(x_gi - LSE2_g)
// (x = log2 logits), the threshold t* is the largest value with
//   mass(a >= t*) >= p   (top-p)     or     count(a >= t*) >= k   (top-k).
// Because a_i >= 0, the uint32 pattern of a_i orders like a_i, so t* is found
// digit by digit: pass 1 bins bits 30..19, pass 2 bits 18..9 of the tokens in
// the chosen pass-1 bin, pass 3 bits 8..0.  Top-k bins hold token counts;
// top-p bins hold the mass as fixed-point round(a * 2^40) in uint64, so sums
// are exact and do not depend on the order of atomic additions.  Each pass is one kernel of
// 1024-thread workgroups that issue all their loads before using any; the
// last workgroup of a (b, head) to finish scans the merged histogram from the
// top bin down and records the bin where the cumulative sum crosses the target.
// Top-k ties at t* beyond the budget are resolved by position in the
// attention kernel, which visits positions in order.
#include "hws_device.h"

namespace hws {

constexpr int NT = SEL_THREADS;
constexpr int NWAVES = NT / 64;

__device__ __forceinline__ unsigned long long mass_fixed(float a) {
  return __float2ull_rn(a * MASS_SCALE);
}

// Block-wide exclusive scan of a (mass, count) pair in thread order.  The
// block totals are left in wm[NWAVES], wc[NWAVES].
__device__ void block_excl_scan(unsigned long long& m, unsigned int& c,
                                unsigned long long* wm, unsigned int* wc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long im = m;
  unsigned int ic = c;
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long vm = __shfl_up(im, off);
    const unsigned int vc = __shfl_up(ic, off);
    if (lane >= off) { im += vm; ic += vc; }
  }
  if (lane == 63) { wm[wave] = im; wc[wave] = ic; }
  __syncthreads();
  if (tid == 0) {
    unsigned long long am = 0ull;
    unsigned int ac = 0u;
    for (int w = 0; w < NWAVES; ++w) {
      const unsigned long long tm = wm[w];
      const unsigned int tc = wc[w];
      wm[w] = am;
      wc[w] = ac;
      am += tm;
      ac += tc;
    }
    wm[NWAVES] = am;
    wc[NWAVES] = ac;
  }
  __syncthreads();
  m = im - m + wm[wave];
  c = ic - c + wc[wave];
}

// Scan `nbins` bins from the top down, starting from `above`; find the bin
// whose inclusive cumulative value (mass if BYMASS, else count) first
// reaches `target`.  *out_bin = -1 if the total stays short.
template <bool BYMASS>
__device__ void scan_from_top(const unsigned long long* hm, const unsigned int* hc, int nbins,
                              unsigned long long above, unsigned long long target,
                              int* out_bin, unsigned long long* out_above,
                              unsigned long long* wm, unsigned int* wc) {
  const int tid = threadIdx.x;
  const int per = nbins >= NT ? nbins / NT : 1;
  const bool act = tid * per < nbins;
  const int top = nbins - 1 - tid * per;               // bins top .. top-per+1
  unsigned long long m = 0ull;
  unsigned int c = 0u;
  if (act)
    for (int k = 0; k < per; ++k) m += BYMASS ? hm[top - k] : (unsigned long long)hc[top - k];
  block_excl_scan(m, c, wm, wc);
  if (tid == 0) *out_bin = -1;
  __syncthreads();
  if (act) {
    unsigned long long cm = above + m;
    for (int k = 0; k < per; ++k) {
      const int bin = top - k;
      const unsigned long long nm = cm + (BYMASS ? hm[bin] : (unsigned long long)hc[bin]);
      if (cm < target && nm >= target) {   // exactly one bin crosses (cumulative is monotone)
        *out_bin = bin;
        *out_above = cm;
      }
      cm = nm;
    }
  }
  __syncthreads();
}

struct SelTarget {
  bool by_mass;
  bool all;                      // the whole sequence is selected
  unsigned long long target;
  unsigned int k;
};

__device__ __forceinline__ SelTarget sel_target(const DecodeParams& p, int b, int N) {
  SelTarget t;
  if (p.select_mode == 0) {
    const float pp = p.top_p[b];
    t.by_mass = true;
    t.all = !(pp < 1.0f);
    // p <= 0 behaves as the smallest positive p: the largest value alone
    const unsigned long long tg = (pp > 0.f) ? (unsigned long long)((double)pp * 1099511627776.0) : 0ull;
    t.target = tg > 0ull ? tg : 1ull;
    t.k = 0;
  } else {
    const int k = max(p.top_k[b], 1);
    t.by_mass = false;
    t.all = k >= N;
    t.target = (unsigned long long)k;
    t.k = (unsigned int)k;
  }
  return t;
}

// Last workgroup of a pass?  Every workgroup's histogram atomics are
// acknowledged before its arrival is counted; the last one then reads the
// merged bins with coherent loads.
__device__ __forceinline__ bool arrive_last(SelState* st, int nwg, int* flag_s) {
  wait_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev = atomicAdd(&st->done, 1u);
    *flag_s = (prev == (unsigned int)(nwg - 1)) ? 1 : 0;
  }
  __syncthreads();
  return *flag_s != 0;
}

template <bool BYMASS>
__device__ __forceinline__ void finish_all(SelState* st, int N) {
  st->tstar = 0u;                 // every a_i >= +0
  if (!BYMASS) st->nsel = (unsigned int)N;
  st->flags = SEL_FINISHED;
}

// Pull the merged global histogram into LDS (all loads issued before any
// use), then clear it and the arrival counter for the next pass.
template <int NB, bool BYMASS>
__device__ void gather_and_clear(SelState* st, unsigned long long* hm, unsigned int* hc) {
  constexpr int PER = NB >= NT ? NB / NT : 1;
  const int tid = threadIdx.x;
  unsigned long long vm[PER];
  unsigned int vc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * NT;
    if (i < NB) {
      if (BYMASS) vm[k] = load_u64_coherent(&st->mass[i]);
      else vc[k] = load_u32_coherent(&st->cnt[i]);
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * NT;
    if (i < NB) {
      if (BYMASS) { hm[i] = vm[k]; st->mass[i] = 0ull; }
      else { hc[i] = vc[k]; st->cnt[i] = 0u; }
    }
  }
  if (tid == 0) st->done = 0u;
  __syncthreads();
}

template <int NB, bool BYMASS>
__device__ void flush_hist(SelState* st, const unsigned long long* hm, const unsigned int* hc) {
  for (int i = threadIdx.x; i < NB; i += NT) {
    if (BYMASS) {
      const unsigned long long m = hm[i];
      if (m != 0ull) atomicAdd(&st->mass[i], m);
    } else {
      const unsigned int c = hc[i];
      if (c != 0u) atomicAdd(&st->cnt[i], c);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: a_i from the raw scores and the per-chunk (max, sum) partials;
// histogram of bits 30..19.  Top-p bins mass, top-k bins counts.
// ---------------------------------------------------------------------------
template <int G, bool BYMASS>
__global__ __launch_bounds__(NT) void select_pass1_kernel(DecodeParams p) {
  constexpr int TB = G <= 4 ? SEL_PER_THREAD : SEL_PER_THREAD / 2;   // tokens per load batch
  // blockIdx.y = hr * GS + gq: one selection state per (retrieval head, query
  // head gq) with one set per query head, else one per retrieval head (gq = 0)
  const int c = blockIdx.x, hs = blockIdx.y, b = blockIdx.z;
  const int hr = hs / p.GS, gq = hs % p.GS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nwg = (N + SEL_CHUNK - 1) / SEL_CHUNK;
  if (c >= nwg) return;
  const size_t srow = (size_t)b * p.nR * p.GS + hs;      // selection row
  SelState* st = p.sel + srow;

  __shared__ unsigned long long hm[BYMASS ? HIST_BINS : 1];
  __shared__ unsigned int hc[BYMASS ? 1 : HIST_BINS];
  __shared__ float lse_s[MAX_G];
  __shared__ unsigned long long wm[NWAVES + 1];
  __shared__ unsigned int wc[NWAVES + 1];
  __shared__ int flag_s, bin_s;
  __shared__ unsigned long long above_s;

  const size_t row = (size_t)(b * p.nR + hr);
  const float* sc = p.scores + row * p.Nmax * G;
  float* agg = p.agg + srow * p.Nagg;
  const int base = c * SEL_CHUNK;

  // log2-sum-exp2 of query head g = wave, from the scoring partials
  const int nsc = (N + p.score_chunk - 1) / p.score_chunk;
  if (wave < G) {
    const float2* sp = p.spart + row * p.n_score_chunks * G + wave;
    float m = NEG_INF, s = 0.f;
    for (int j0 = lane; j0 < nsc; j0 += 256) {
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 64 * u;
        v[u] = j < nsc ? sp[(size_t)j * G] : make_float2(NEG_INF, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) lse_combine(m, s, v[u].x, v[u].y);
    }
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      lse_combine(m, s, m2, s2);
    }
    if (lane == 0) lse_s[wave] = m + log2f(s);
  }
  for (int i = tid; i < HIST_BINS; i += NT) {
    if (BYMASS) hm[i] = 0ull;
    else hc[i] = 0u;
  }
  __syncthreads();
  if (c == 0 && tid < G) st->lse2[tid] = lse_s[tid];

  float lse[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lse[g] = lse_s[g];
  const float c2 = p.c2_score;
  const float invG = 1.0f / (float)G;
#pragma unroll
  for (int j0 = 0; j0 < SEL_PER_THREAD; j0 += TB) {
    float x[TB][G];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int i = base + (j0 + u) * NT + tid;
      if (i < N) {
        if (G >= 4) {
#pragma unroll
          for (int q4 = 0; q4 < G / 4; ++q4) {
            const float4 v = *reinterpret_cast<const float4*>(sc + (size_t)i * G + 4 * q4);
            x[u][4 * q4 + 0] = v.x; x[u][4 * q4 + 1] = v.y; x[u][4 * q4 + 2] = v.z; x[u][4 * q4 + 3] = v.w;
          }
        } else if (G == 2) {
          const float2 v = *reinterpret_cast<const float2*>(sc + (size_t)i * G);
          x[u][0] = v.x; x[u][G - 1] = v.y;
        } else {
          x[u][0] = sc[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int i = base + (j0 + u) * NT + tid;
      if (i < N) {
        float a = 0.f;
        if (p.GS == 1) {                 // mean of the group's distributions
#pragma unroll
          for (int g = 0; g < G; ++g) a += fast_exp2(x[u][g] * c2 - lse[g]);
          a *= invG;
        } else {                         // query head gq's own distribution
          float xg = x[u][0], lg = lse[0];
#pragma unroll
          for (int g = 1; g < G; ++g)
            if (g == gq) { xg = x[u][g]; lg = lse[g]; }
          a = fast_exp2(xg * c2 - lg);
        }
        agg[i] = a;
        const unsigned int bin = (__float_as_uint(a) >> P1_SHIFT) & (HIST_BINS - 1);
        if (BYMASS) atomicAdd(&hm[bin], mass_fixed(a));
        else atomicAdd(&hc[bin], 1u);
      }
    }
  }
  __syncthreads();
  flush_hist<HIST_BINS, BYMASS>(st, hm, hc);
  if (!arrive_last(st, nwg, &flag_s)) return;

  gather_and_clear<HIST_BINS, BYMASS>(st, hm, hc);
  const SelTarget tg = sel_target(p, b, N);
  if (tg.all) {
    if (tid == 0) finish_all<BYMASS>(st, N);
    return;
  }
  scan_from_top<BYMASS>(hm, hc, HIST_BINS, 0ull, tg.target, &bin_s, &above_s, wm, wc);
  if (tid == 0) {
    if (bin_s < 0) {
      finish_all<BYMASS>(st, N);  // rounding left the total short of p: keep all
    } else {
      st->prefix = (unsigned int)bin_s;
      if (BYMASS) st->mass_above = above_s;
      else st->cnt_above = (unsigned int)above_s;
    }
  }
}

// ---------------------------------------------------------------------------
// Passes 2 and 3: refine inside the chosen bin.
// ---------------------------------------------------------------------------
template <int PASS, bool BYMASS>
__global__ __launch_bounds__(NT) void select_refine_kernel(DecodeParams p) {
  constexpr int NB = PASS == 2 ? P2_BINS : P3_BINS;
  constexpr int SHIFT = PASS == 2 ? P2_SHIFT : 0;
  constexpr int KEY_SHIFT = PASS == 2 ? P1_SHIFT : P2_SHIFT;   // bits already fixed
  const int c = blockIdx.x, hs = blockIdx.y, b = blockIdx.z;     // hs = hr * GS + gq
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nwg = (N + SEL_CHUNK - 1) / SEL_CHUNK;
  if (c >= nwg) return;
  const size_t srow = (size_t)b * p.nR * p.GS + hs;
  SelState* st = p.sel + srow;

  __shared__ unsigned long long hm[BYMASS ? NB : 1];
  __shared__ unsigned int hc[BYMASS ? 1 : NB];
  __shared__ unsigned long long wm[NWAVES + 1];
  __shared__ unsigned int wc[NWAVES + 1];
  __shared__ int flag_s, bin_s;
  __shared__ unsigned long long above_s;

  const float* agg = p.agg + srow * p.Nagg;
  const int base = c * SEL_CHUNK;
  float a[SEL_PER_THREAD];
#pragma unroll
  for (int j = 0; j < SEL_PER_THREAD; ++j) {
    const int i = base + j * NT + tid;
    a[j] = i < N ? agg[i] : -1.0f;           // -1: never matches a prefix
  }
  const unsigned int flags = st->flags;
  const unsigned int prefix = st->prefix;
  for (int i = tid; i < NB; i += NT) {
    if (BYMASS) hm[i] = 0ull;
    else hc[i] = 0u;
  }
  __syncthreads();
  if (flags & SEL_FINISHED) return;           // uniform: the state was final before this pass

#pragma unroll
  for (int j = 0; j < SEL_PER_THREAD; ++j) {
    const unsigned int bits = __float_as_uint(a[j]);
    if ((bits >> KEY_SHIFT) == prefix) {
      const unsigned int bin = (bits >> SHIFT) & (NB - 1);
      if (BYMASS) atomicAdd(&hm[bin], mass_fixed(a[j]));
      else atomicAdd(&hc[bin], 1u);
    }
  }
  __syncthreads();
  flush_hist<NB, BYMASS>(st, hm, hc);
  if (!arrive_last(st, nwg, &flag_s)) return;

  gather_and_clear<NB, BYMASS>(st, hm, hc);
  const SelTarget tg = sel_target(p, b, N);
  const unsigned long long above = BYMASS ? st->mass_above : (unsigned long long)st->cnt_above;
  scan_from_top<BYMASS>(hm, hc, NB, above, tg.target, &bin_s, &above_s, wm, wc);
  if (tid == 0) {
    if (bin_s < 0) {
      finish_all<BYMASS>(st, N);
    } else if (PASS == 2) {
      st->prefix = (prefix << 10) | (unsigned int)bin_s;
      if (BYMASS) st->mass_above = above_s;
      else st->cnt_above = (unsigned int)above_s;
    } else {
      st->tstar = (prefix << 9) | (unsigned int)bin_s;
      if (BYMASS) {
        st->flags = SEL_FINISHED;                   // |S| is summed by the attention kernel
      } else {
        const unsigned int gt = (unsigned int)above_s;  // tokens strictly above t*
        const unsigned int eq = hc[bin_s];              // tokens equal to t*
        if (gt + eq <= tg.k) {
          st->nsel = gt + eq;
          st->flags = SEL_FINISHED;
        } else {
          st->quota = tg.k - gt;                    // ties to keep, lowest positions first
          st->nsel = tg.k;
          st->flags = SEL_FINISHED | SEL_TIE;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Optional ascending list of the selected positions (one workgroup per head).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int block_rank256(bool f, unsigned int* tmp) {
  // exclusive rank among flagged threads of a 256-thread block; total in tmp[4]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long bal = __ballot(f);
  const unsigned int below = __builtin_amdgcn_mbcnt_hi((unsigned int)(bal >> 32),
                                 __builtin_amdgcn_mbcnt_lo((unsigned int)bal, 0u));
  if (lane == 0) tmp[wave] = (unsigned int)__popcll(bal);
  __syncthreads();
  unsigned int off = 0;
  for (int w = 0; w < wave; ++w) off += tmp[w];
  const unsigned int tot = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  if (tid == 0) tmp[4] = tot;
  __syncthreads();
  return off + below;
}

__global__ __launch_bounds__(256) void emit_sel_kernel(DecodeParams p) {
  const int hs = blockIdx.x, b = blockIdx.y;      // hs = hr * GS + gq
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const size_t srow = (size_t)b * p.nR * p.GS + hs;
  const SelState* st = p.sel + srow;
  const unsigned int tstar = st->tstar;
  const bool tie = (st->flags & SEL_TIE) != 0;
  const unsigned int quota = tie ? st->quota : 0xFFFFFFFFu;
  const float* agg = p.agg + srow * p.Nagg;
  int* dst = p.sel_idx + srow * p.sel_cap;
  __shared__ unsigned int tmp[8];
  unsigned int written = 0, ties = 0;
  for (int base = 0; base < N; base += 256) {
    const int i = base + tid;
    const unsigned int bits = i < N ? __float_as_uint(agg[i]) : 0u;
    const bool eq = i < N && bits == tstar;
    const unsigned int trank = block_rank256(eq, tmp);
    const unsigned int nties = tmp[4];
    __syncthreads();
    const bool f = i < N && (bits > tstar || (eq && ties + trank < quota));
    const unsigned int rank = block_rank256(f, tmp);
    if (f && written + rank < (unsigned int)p.sel_cap) dst[written + rank] = i;
    written += tmp[4];
    ties += nties;
    __syncthreads();
  }
}

template <int G, bool BYMASS>
static hipError_t launch_pass1(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_kernel(select_pass1_kernel<G, BYMASS>, dim3(p.n_sel_chunks, p.nR * p.GS, p.B), dim3(NT), s, e0, e1, p);
}

template <bool BYMASS>
static hipError_t launch_select_m(const DecodeParams& p, hipStream_t s, int pass, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.n_sel_chunks, p.nR * p.GS, p.B);
  switch (pass) {
    case 1:
      switch (p.G) {
        case 1: return launch_pass1<1, BYMASS>(p, s, e0, e1);
        case 2: return launch_pass1<2, BYMASS>(p, s, e0, e1);
        case 4: return launch_pass1<4, BYMASS>(p, s, e0, e1);
        case 8: return launch_pass1<8, BYMASS>(p, s, e0, e1);
      }
      return hipErrorInvalidValue;
    case 2: return launch_kernel(select_refine_kernel<2, BYMASS>, grid, dim3(NT), s, e0, e1, p);
    case 3: return launch_kernel(select_refine_kernel<3, BYMASS>, grid, dim3(NT), s, e0, e1, p);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select(const DecodeParams& p, hipStream_t s, int pass, hipEvent_t e0, hipEvent_t e1) {
  return p.select_mode == 0 ? launch_select_m<true>(p, s, pass, e0, e1)
                            : launch_select_m<false>(p, s, pass, e0, e1);
}

hipError_t launch_emit(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(emit_sel_kernel, dim3(p.nR * p.GS, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
