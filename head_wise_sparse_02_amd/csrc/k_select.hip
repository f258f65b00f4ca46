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
// the chosen pass-1 bin, pass 3 bits 8..0.  Bins hold a token count and the
// mass as fixed-point round(a * 2^40) in uint64, so sums are exact and do not
// depend on the order of atomic additions.  Each pass is one kernel; the
// last workgroup of a (b, head) to finish scans the merged histogram from the
// top bin down and records the bin where the cumulative sum crosses the target.
#include "hws_device.h"

namespace hws {

__device__ __forceinline__ unsigned long long mass_fixed(float a) {
  return __float2ull_rn(a * MASS_SCALE);
}

// Block-wide exclusive scan (256 threads) of a (mass, count) pair in thread
// order; returns the exclusive prefix and writes the block total.
__device__ void block_excl_scan(unsigned long long& m, unsigned int& c,
                                unsigned long long* sm, unsigned int* sc,
                                unsigned long long& tot_m, unsigned int& tot_c) {
  const int tid = threadIdx.x;
  sm[tid] = m;
  sc[tid] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    unsigned long long vm = (tid >= off) ? sm[tid - off] : 0ull;
    unsigned int vc = (tid >= off) ? sc[tid - off] : 0u;
    __syncthreads();
    sm[tid] += vm;
    sc[tid] += vc;
    __syncthreads();
  }
  tot_m = sm[255];
  tot_c = sc[255];
  const unsigned long long incl_m = sm[tid];
  const unsigned int incl_c = sc[tid];
  __syncthreads();
  m = incl_m - m;
  c = incl_c - c;
}

// Scan `nbins` bins from the top down, starting from (above_m, above_c);
// find the first bin whose inclusive cumulative value reaches `target`
// (mass if by_mass, else count).  Returns the bin in *out_bin (-1 if the
// total stays short) with the cumulative sums strictly above it.
__device__ void scan_from_top(const unsigned long long* hm, const unsigned int* hc, int nbins,
                              unsigned long long above_m, unsigned int above_c,
                              unsigned long long target, bool by_mass,
                              int* out_bin, unsigned long long* out_am, unsigned int* out_ac,
                              unsigned long long* sm, unsigned int* sc) {
  const int tid = threadIdx.x;
  const int per = nbins / 256;
  const int top = nbins - 1 - tid * per;                // this thread: bins top .. top-per+1
  unsigned long long m = 0ull;
  unsigned int c = 0u;
  for (int k = 0; k < per; ++k) { m += hm[top - k]; c += hc[top - k]; }
  unsigned long long tm;
  unsigned int tc;
  block_excl_scan(m, c, sm, sc, tm, tc);
  if (tid == 0) *out_bin = -1;
  __syncthreads();
  unsigned long long cm = above_m + m;
  unsigned int cc = above_c + c;
  for (int k = 0; k < per; ++k) {
    const int bin = top - k;
    const unsigned long long nm = cm + hm[bin];
    const unsigned int nc = cc + hc[bin];
    const bool before = by_mass ? (cm >= target) : ((unsigned long long)cc >= target);
    const bool after = by_mass ? (nm >= target) : ((unsigned long long)nc >= target);
    if (!before && after) {            // exactly one bin crosses (cumulative is monotone)
      *out_bin = bin;
      *out_am = cm;
      *out_ac = cc;
    }
    cm = nm;
    cc = nc;
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
    t.target = (pp > 0.f) ? (unsigned long long)((double)pp * 1099511627776.0) : 0ull;
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

// Last workgroup of a pass?  Every workgroup publishes its atomics first.
__device__ __forceinline__ bool arrive_last(SelState* st, int nwg, int* flag_s) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev = atomicAdd(&st->done, 1u);
    *flag_s = (prev == (unsigned int)(nwg - 1)) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag_s != 0;
  if (last) __threadfence();
  return last;
}

__device__ __forceinline__ void finish_all(SelState* st, int N) {
  st->tstar = 0u;                 // every a_i >= +0
  st->icut = 0xFFFFFFFFu;
  st->nsel = (unsigned int)N;
  st->flags = SEL_FINISHED;
}

// Pull the merged global histogram into LDS and clear it for the next pass.
__device__ void gather_and_clear(SelState* st, unsigned long long* hm, unsigned int* hc, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += 256) {
    hm[i] = load_u64_coherent(&st->mass[i]);
    hc[i] = load_u32_coherent(&st->cnt[i]);
    st->mass[i] = 0ull;
    st->cnt[i] = 0u;
  }
  if (threadIdx.x == 0) st->done = 0u;
  __syncthreads();
}

__device__ void flush_hist(SelState* st, const unsigned long long* hm, const unsigned int* hc, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += 256) {
    const unsigned int c = hc[i];
    if (c != 0u) {
      atomicAdd(&st->cnt[i], c);
      atomicAdd(&st->mass[i], hm[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: a_i from the raw scores and the per-chunk (max, sum) partials;
// histogram of bits 30..19.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void select_pass1_kernel(DecodeParams p) {
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nwg = (N + SEL_CHUNK - 1) / SEL_CHUNK;
  if (c >= nwg) return;
  SelState* st = p.sel + (size_t)b * p.nR + hr;

  __shared__ unsigned long long hm[HIST_BINS];
  __shared__ unsigned int hc[HIST_BINS];
  __shared__ float lse_s[MAX_G];
  __shared__ unsigned long long scan_m[256];
  __shared__ unsigned int scan_c[256];
  __shared__ int flag_s, bin_s;
  __shared__ unsigned long long am_s;
  __shared__ unsigned int ac_s;
  for (int i = tid; i < HIST_BINS; i += 256) { hm[i] = 0ull; hc[i] = 0u; }

  // log2-sum-exp2 of every query head from the scoring partials
  const int nsc = (N + SCORE_CHUNK - 1) / SCORE_CHUNK;
  if (tid < 64) {
    const int lane = tid;
    for (int g = 0; g < G; ++g) {
      float m = NEG_INF, s = 0.f;
      for (int j = lane; j < nsc; j += 64) {
        const float2 v = p.spart[((size_t)(b * p.nR + hr) * p.n_score_chunks + j) * G + g];
        lse_combine(m, s, v.x, v.y);
      }
      for (int off = 1; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        lse_combine(m, s, m2, s2);
      }
      if (lane == 0) lse_s[g] = m + log2f(s);
    }
  }
  __syncthreads();
  if (c == 0 && tid < G) st->lse2[tid] = lse_s[tid];

  float lse[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lse[g] = lse_s[g];
  const float c2 = p.c2_score;
  const float invG = 1.0f / (float)G;
  const float* sc = p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G;
  float* agg = p.agg + (size_t)(b * p.nR + hr) * p.Nmax;
  const int base = c * SEL_CHUNK;
  for (int j = 0; j < SEL_CHUNK / 256; ++j) {
    const int i = base + j * 256 + tid;
    if (i >= N) break;
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) a += fast_exp2(sc[(size_t)i * G + g] * c2 - lse[g]);
    a *= invG;
    agg[i] = a;
    const unsigned int bin = (__float_as_uint(a) >> P1_SHIFT) & (HIST_BINS - 1);
    atomicAdd(&hc[bin], 1u);
    atomicAdd(&hm[bin], mass_fixed(a));
  }
  __syncthreads();
  flush_hist(st, hm, hc, HIST_BINS);
  if (!arrive_last(st, nwg, &flag_s)) return;

  gather_and_clear(st, hm, hc, HIST_BINS);
  const SelTarget tg = sel_target(p, b, N);
  if (tg.all) {
    if (tid == 0) finish_all(st, N);
    return;
  }
  scan_from_top(hm, hc, HIST_BINS, 0ull, 0u, tg.target, tg.by_mass, &bin_s, &am_s, &ac_s, scan_m, scan_c);
  if (tid == 0) {
    if (bin_s < 0) {
      finish_all(st, N);          // rounding left the total short of p: keep all
    } else {
      st->prefix = (unsigned int)bin_s;
      st->mass_above = am_s;
      st->cnt_above = ac_s;
    }
  }
}

// ---------------------------------------------------------------------------
// Passes 2 and 3: refine inside the chosen bin.
// ---------------------------------------------------------------------------
template <int PASS>
__global__ __launch_bounds__(256) void select_refine_kernel(DecodeParams p) {
  constexpr int NB = PASS == 2 ? P2_BINS : P3_BINS;
  constexpr int SHIFT = PASS == 2 ? P2_SHIFT : 0;
  constexpr int KEY_SHIFT = PASS == 2 ? P1_SHIFT : P2_SHIFT;   // bits already fixed
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nwg = (N + SEL_CHUNK - 1) / SEL_CHUNK;
  if (c >= nwg) return;
  SelState* st = p.sel + (size_t)b * p.nR + hr;
  if (st->flags & SEL_FINISHED) return;
  const unsigned int prefix = st->prefix;

  __shared__ unsigned long long hm[NB];
  __shared__ unsigned int hc[NB];
  __shared__ unsigned long long scan_m[256];
  __shared__ unsigned int scan_c[256];
  __shared__ int flag_s, bin_s;
  __shared__ unsigned long long am_s;
  __shared__ unsigned int ac_s;
  for (int i = tid; i < NB; i += 256) { hm[i] = 0ull; hc[i] = 0u; }
  __syncthreads();

  const float* agg = p.agg + (size_t)(b * p.nR + hr) * p.Nmax;
  const int base = c * SEL_CHUNK;
  for (int j = 0; j < SEL_CHUNK / 256; ++j) {
    const int i = base + j * 256 + tid;
    if (i >= N) break;
    const float a = agg[i];
    const unsigned int bits = __float_as_uint(a);
    if ((bits >> KEY_SHIFT) == prefix) {
      const unsigned int bin = (bits >> SHIFT) & (NB - 1);
      atomicAdd(&hc[bin], 1u);
      atomicAdd(&hm[bin], mass_fixed(a));
    }
  }
  __syncthreads();
  flush_hist(st, hm, hc, NB);
  if (!arrive_last(st, nwg, &flag_s)) return;

  gather_and_clear(st, hm, hc, NB);
  const SelTarget tg = sel_target(p, b, N);
  const unsigned long long above_m = st->mass_above;
  const unsigned int above_c = st->cnt_above;
  scan_from_top(hm, hc, NB, above_m, above_c, tg.target, tg.by_mass, &bin_s, &am_s, &ac_s, scan_m, scan_c);
  if (tid == 0) {
    if (bin_s < 0) {
      finish_all(st, N);
    } else if (PASS == 2) {
      st->prefix = (prefix << 10) | (unsigned int)bin_s;
      st->mass_above = am_s;
      st->cnt_above = ac_s;
    } else {
      const unsigned int tstar = (prefix << 9) | (unsigned int)bin_s;
      const unsigned int gt = ac_s;                 // tokens strictly above t*
      const unsigned int eq = hc[bin_s];            // tokens equal to t*
      st->tstar = tstar;
      if (tg.by_mass || gt + eq <= tg.k) {
        st->icut = 0xFFFFFFFFu;
        st->nsel = gt + eq;
        st->flags = SEL_FINISHED;
      } else {
        st->quota = tg.k - gt;                      // ties to keep, lowest positions first
        st->nsel = tg.k;
        st->flags = SEL_TIE;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k tie pass: keep the `quota` lowest positions among a_i == t*.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int block_count(bool f, unsigned int* tmp) {
  // exclusive rank of this thread among flagged threads, total in tmp[4]
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

__global__ __launch_bounds__(256) void select_tie_kernel(DecodeParams p) {
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nwg = (N + SEL_CHUNK - 1) / SEL_CHUNK;
  if (c >= nwg) return;
  SelState* st = p.sel + (size_t)b * p.nR + hr;
  if (!(st->flags & SEL_TIE)) return;
  const unsigned int tstar = st->tstar;
  __shared__ unsigned int tmp[8];
  __shared__ int flag_s;
  const float* agg = p.agg + (size_t)(b * p.nR + hr) * p.Nmax;
  const int base = c * SEL_CHUNK;
  unsigned int cnt = 0;
  for (int j = 0; j < SEL_CHUNK / 256; ++j) {
    const int i = base + j * 256 + tid;
    if (i < N && __float_as_uint(agg[i]) == tstar) ++cnt;
  }
  // per-chunk tie count into the (cleared) count array
  for (int off = 1; off < 64; off <<= 1) cnt += __shfl_xor(cnt, off);
  if ((tid & 63) == 0) tmp[tid >> 6] = cnt;
  __syncthreads();
  if (tid == 0) st->cnt[c] = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  if (!arrive_last(st, nwg, &flag_s)) return;

  __shared__ int cstar_s;
  __shared__ unsigned int need_s;
  if (tid == 0) {
    unsigned int need = st->quota;
    int cs = nwg - 1;
    for (int k = 0; k < nwg; ++k) {
      const unsigned int v = load_u32_coherent(&st->cnt[k]);
      if (v >= need) { cs = k; break; }
      need -= v;
    }
    cstar_s = cs;
    need_s = need;            // the need-th tie (1-based) of chunk cs is the last kept
  }
  __syncthreads();
  const int cb = cstar_s * SEL_CHUNK;
  unsigned int seen = 0;
  __shared__ unsigned int icut_s;
  if (tid == 0) icut_s = 0xFFFFFFFFu;
  __syncthreads();
  for (int j = 0; j < SEL_CHUNK / 256; ++j) {
    const int i = cb + j * 256 + tid;
    const bool f = (i < N) && __float_as_uint(agg[i]) == tstar;
    const unsigned int rank = block_count(f, tmp);
    if (f && seen + rank + 1 == need_s) icut_s = (unsigned int)i;
    seen += tmp[4];
    __syncthreads();
    if (seen >= need_s) break;
  }
  __syncthreads();
  if (tid == 0) {
    st->icut = icut_s;
    for (int k = 0; k < nwg; ++k) st->cnt[k] = 0u;
    st->flags = SEL_FINISHED;
  }
}

// ---------------------------------------------------------------------------
// Optional ascending list of the selected positions (one workgroup per head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void emit_sel_kernel(DecodeParams p) {
  const int hr = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int N = min(p.seq_lens[b], p.Nmax);
  const SelState* st = p.sel + (size_t)b * p.nR + hr;
  const unsigned int tstar = st->tstar, icut = st->icut;
  const float* agg = p.agg + (size_t)(b * p.nR + hr) * p.Nmax;
  int* dst = p.sel_idx + (size_t)(b * p.nR + hr) * p.sel_cap;
  __shared__ unsigned int tmp[8];
  unsigned int written = 0;
  for (int base = 0; base < N; base += 256) {
    const int i = base + tid;
    bool f = false;
    if (i < N) {
      const unsigned int bits = __float_as_uint(agg[i]);
      f = bits > tstar || (bits == tstar && (unsigned int)i <= icut);
    }
    const unsigned int rank = block_count(f, tmp);
    if (f && written + rank < (unsigned int)p.sel_cap) dst[written + rank] = i;
    written += tmp[4];
    __syncthreads();
  }
}

template <int G>
static hipError_t launch_pass1(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(select_pass1_kernel<G>, dim3(p.n_sel_chunks, p.nR, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_select(const DecodeParams& p, hipStream_t s, int pass) {
  const dim3 grid(p.n_sel_chunks, p.nR, p.B);
  switch (pass) {
    case 1:
      switch (p.G) {
        case 1: return launch_pass1<1>(p, s);
        case 2: return launch_pass1<2>(p, s);
        case 4: return launch_pass1<4>(p, s);
        case 8: return launch_pass1<8>(p, s);
      }
      return hipErrorInvalidValue;
    case 2: hipLaunchKernelGGL(select_refine_kernel<2>, grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL(select_refine_kernel<3>, grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL(select_tie_kernel, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_emit(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(emit_sel_kernel, dim3(p.nR, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
