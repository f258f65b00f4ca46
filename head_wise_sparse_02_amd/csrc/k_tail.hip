// Selection, gathered attention and merge of one decode step in a single
// launch of co-resident workgroups.
//
// The steps are those of the multi-kernel path (k_select.hip, k_attend.hip):
// [RTPurbo] "Full attention returns in force ...", Methodology §3 (top-p mass
// / top-k budget over the GQA-aggregated softmax) and §5 (histogram
// threshold instead of a sort); [ICS] "Inference-time context sparsity:
// illusion or opportunity?", §3c (attention reads only the selected rows);
// [RTPurbo] Methodology §1 and [AoH] "Autonomy-of-Heads ...", Methodology §4
// (local heads: sinks + window).  What changes is how the work is laid out:
//
// * A retrieval head's positions are cut into tiles of TAIL_TILE tokens; a
//   workgroup owns up to TAIL_MAXT tiles and keeps their aggregates a_i in
//   registers through all three radix passes, so the raw scores are read
//   once and a_i is never written out (except for the optional index list).
// * Between passes only the tiles of the same head wait for each other: each
//   tile flushes its LDS histogram into the head's global bins, bumps the
//   head's arrival counter, then spins until all tiles of the head arrived
//   and scans the merged bins itself.  Nothing waits on another head.  The
//   grid is sized to what the device holds at once (compute units times
//   occupancy), so every workgroup that is waited for is resident; the
//   cooperative form of the launch has the runtime guarantee it.
// * A tile then compacts its kept positions in position order and attends
//   over them; local-head chunks go to the workgroups without tiles first.
// * The last split of a (sequence, KV head) to finish merges all its splits.
//
// Hand-offs use only device-coherent accesses (atomics, agent-scope atomic
// loads/stores) after waiting for the writer's memory operations to be
// acknowledged; no device-wide fence is issued.  Every wait is bounded: on a
// timeout the error word is set, the kernel runs to its end and the outputs
// of the step are NaN.
#include <mutex>
#include <vector>

#include "attend_rows.h"

namespace hws {

namespace {

constexpr int TT = TAIL_THREADS;              // 512 threads
constexpr int TW = TT / 64;                   // 8 waves
constexpr int TPT = TAIL_TPT;                 // tokens per thread per tile
constexpr int MAXT = TAIL_MAXT;
constexpr int NPROC = TT / 16;                // 16-lane row processors

struct TailLds {
  union {
    unsigned long long hist[HIST_BINS];       // radix bins (pass 1 is the largest)
    unsigned short rows[TAIL_TILE];           // kept offsets of the tile, position order
    float wo[TW][MAX_G][D];                   // per-wave partial outputs
  } u;
  int pages[MAXT][TAIL_TILE / BS];            // block-table entries of the tiles
  int ltok[LOCAL_CHUNK], lpg[LOCAL_CHUNK];    // local chunk: tokens and pages
  unsigned int cnt[TPT * TW];                 // per (u, wave) counts for ordered compaction
  float lse[MAXT][MAX_G];
  float wm[TW][MAX_G], wl[TW][MAX_G];
  unsigned long long runs[TT];                // radix scan: sums of runs of nbins / TT bins
  unsigned long long above;
  unsigned int tmp[TW + 1];
  int bin;
  int flag;
};

__device__ __forceinline__ unsigned long long mass_fixed(float a) {
  return __float2ull_rn(a * MASS_SCALE);
}

__device__ __forceinline__ unsigned int lane_rank(unsigned long long bal) {
  return __builtin_amdgcn_mbcnt_hi((unsigned int)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned int)bal, 0u));
}

// Thread 0 polls `ctr` until it reaches `target`.  Returns false (and sets
// the error word) once `limit` polls have passed (checked every 256, so every
// wait ends) or another workgroup already failed.
__device__ __forceinline__ bool spin_until(const unsigned int* ctr, unsigned int target, unsigned int* err,
                                           unsigned int limit) {
  unsigned int it = 0;
  while (load_u32_coherent(ctr) < target) {
    ++it;
    if ((it & 255u) == 0u && (it >= limit || load_u32_coherent(err) != 0u)) {
      atomicOr(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Everyone waits for thread 0's spin (the host's wait bias, 0 in normal use,
// raises the target past what can arrive, for tests of the time-out path).
__device__ __forceinline__ void block_wait(const DecodeParams& p, const unsigned int* ctr, unsigned int target,
                                           unsigned int* err) {
  __syncthreads();
  if (threadIdx.x == 0) spin_until(ctr, target + p.wait_bias, err, p.spin_limit);
  __syncthreads();
}

// In-place exclusive scan of S.cnt (TPT * TW entries in position order);
// returns the total.
__device__ __forceinline__ unsigned int scan_cnt(TailLds& S) {
  constexpr int NE = TPT * TW;                // 256
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned int v = 0, inc = 0;
  if (tid < NE) {
    v = S.cnt[tid];
    inc = v;
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned int t = __shfl_up(inc, off);
      if (lane >= off) inc += t;
    }
    if (lane == 63) S.tmp[wave] = inc;
  }
  __syncthreads();
  if (tid < NE) {
    unsigned int off = 0;
    for (int w2 = 0; w2 < wave; ++w2) off += S.tmp[w2];
    S.cnt[tid] = off + inc - v;
  }
  unsigned int tot = 0;
  for (int w2 = 0; w2 < NE / 64; ++w2) tot += S.tmp[w2];
  __syncthreads();
  return tot;
}

// Token slot u of a thread: position u*TT + tid of the tile (slot-major, the
// tail's layout) or wave*SP*64 + u*64 + lane (wave-major, the fused scans':
// a wave owns SP*64 consecutive positions, SP = the slots in use).  cnt_idx
// orders the per-(u, wave) counts by position.
template <bool WM>
__device__ __forceinline__ int cnt_idx(int u, int wave) { return WM ? wave * TPT + u : u * TW + wave; }
template <bool WM, int SP = TPT>
__device__ __forceinline__ int slot_pos(int u, int tid) { return WM ? (tid >> 6) * (SP * 64) + u * 64 + (tid & 63) : u * TT + tid; }

// Count the flagged tokens per (u, wave) in S.cnt (not yet scanned).
template <bool WM>
__device__ __forceinline__ void count_flags(TailLds& S, unsigned int mask) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const unsigned long long bal = __ballot((mask >> u) & 1u);
    if (lane == 0) S.cnt[cnt_idx<WM>(u, wave)] = (unsigned int)__popcll(bal);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ unsigned long long wave_prefix(unsigned long long v, int lane) {
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Scan `nbins` LDS bins from the top down, starting from `above`; the bin
// where the cumulative sum first reaches `target` (-1 if it never does) and
// the sum strictly above it.  Lane l of wave 0 takes the l-th group of
// nbins/64 bins from the top: a wave prefix sum over the groups' sums finds
// the group that crosses the target, and a second one over that group's bins
// (one per lane) finds the bin.  With more than 8 bins per group every thread
// first sums a run of nbins/TT bins, so that a lane adds 8 run sums instead
// of reading its whole group in turn.
template <int NBINS>
__device__ __forceinline__ void scan_top(TailLds& S, unsigned long long above, unsigned long long target,
                                         int& out_bin, unsigned long long& out_above) {
  constexpr int per = NBINS / 64;             // 64, 16 or 8
  constexpr int RL = NBINS / TT;              // 8, 2 or 1
  static_assert(per == 8 * RL, "a group is 8 runs");
  const int tid = threadIdx.x;
  if constexpr (RL > 1) {
    // neighbouring threads' runs are 8*RL bytes apart: each starts at a
    // different offset of its run so that one read spreads over the banks
    unsigned long long r = 0ull;
#pragma unroll
    for (int k = 0; k < RL; ++k) r += S.u.hist[tid * RL + ((k + tid) & (RL - 1))];
    S.runs[tid] = r;
    __syncthreads();
  }
  if (tid < 64) {
    const int top = NBINS - 1 - tid * per;
    unsigned long long m = 0ull;
    if constexpr (RL > 1) {
      const int r0 = TT - 8 * (tid + 1);      // the group's lowest run
#pragma unroll
      for (int k = 0; k < 8; ++k) m += S.runs[r0 + ((k + tid) & 7)];
    } else {
#pragma unroll
      for (int k = 0; k < per; ++k) m += S.u.hist[top - ((k + tid) & (per - 1))];
    }
    const unsigned long long inc = wave_prefix(m, tid);
    const unsigned long long cm = above + inc - m;              // sum above this lane's run
    const unsigned long long run = __ballot(cm < target && cm + m >= target);   // one lane at most
    if (tid == 0) S.bin = -1;
    if (run != 0ull) {                                          // wave-uniform
      const int c = __ffsll((long long)run) - 1;
      const int ctop = NBINS - 1 - c * per;
      const unsigned long long cabove = __shfl(cm, c);
      const unsigned long long v = tid < per ? S.u.hist[ctop - tid] : 0ull;
      const unsigned long long pre = cabove + wave_prefix(v, tid);
      if (tid < per && pre - v < target && pre >= target) {      // one lane: the bin
        S.bin = ctop - tid;
        S.above = pre - v;
      }
    }
  }
  __syncthreads();
  out_bin = S.bin;
  out_above = S.above;
  __syncthreads();
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup w runs on
// XCD w mod 8).  The first n workgroups (n a multiple of 8) are renumbered so
// that consecutive ids share an XCD: the tiles of one head, which have
// consecutive ids, then stream and finish on one XCD, and a head waits only
// for the XCD it runs on.  A bijection on [0, gridDim.x).
__device__ __forceinline__ int xcd_local_id(int w, int n) {
  if (w >= n || (n & 7) != 0) return w;
  return (w & 7) * (n >> 3) + (w >> 3);
}

struct Tile {
  int t, b, hr, j, N, lo, hi;   // t < 0: no tile in this slot
};

// Per-tile selection state (uniform over the workgroup).
struct TileSel {
  bool done;                    // threshold known
  unsigned int key;             // bits of the threshold fixed so far
  unsigned long long above;     // mass / count strictly above the candidate range
  unsigned int tstar;
  bool tie;                     // top-k: keep only `quota` lowest-position ties
  unsigned int quota;
  unsigned long long target;    // mass (fixed point) or count the threshold must reach
};

// The threshold's target for sequence b, and whether the whole sequence of N
// tokens is kept (p >= 1 or k >= N).
__device__ __forceinline__ unsigned long long sel_target(const DecodeParams& p, int b, int N, bool& all) {
  if (p.select_mode == 0) {
    const float pp = p.top_p[b];
    all = N == 0 || !(pp < 1.0f);
    const unsigned long long tg = pp > 0.f ? (unsigned long long)((double)pp * 1099511627776.0) : 0ull;
    return tg > 0ull ? tg : 1ull;              // p <= 0: the largest value alone
  }
  const int k = max(p.top_k[b], 1);
  all = k >= N;
  return (unsigned long long)k;
}

// One radix pass over the workgroup's tiles: LDS histogram of the candidate
// tokens, flush into the head's bins, arrive, wait for the head, scan.
// The head's arrival counter is at `base` + (PASS - 1) * tiles per head
// before the pass.
template <int PASS, int NT>
__device__ __forceinline__ void radix_pass(const DecodeParams& p, TailLds& S, const Tile (&tl)[NT],
                                           const float (&av)[NT][TPT], TileSel (&ts)[NT], bool bymass,
                                           unsigned int* err, unsigned int base) {
  constexpr int NB = PASS == 1 ? HIST_BINS : (PASS == 2 ? P2_BINS : P3_BINS);
  constexpr int SHIFT = PASS == 1 ? P1_SHIFT : (PASS == 2 ? P2_SHIFT : 0);
  constexpr int KEY_SHIFT = PASS == 1 ? 31 : (PASS == 2 ? P1_SHIFT : P2_SHIFT);
  const int tid = threadIdx.x;
  bool any = false;
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    if (tl[k].t < 0 || ts[k].done) continue;                 // uniform
    any = true;
    SelState* st = p.sel + (size_t)tl[k].b * p.nR + tl[k].hr;
    unsigned long long* gh = PASS == 1 ? st->mass : (PASS == 2 ? st->mass2 : st->mass3);
    // LDS bins: 64-bit fixed-point mass (top-p) or 32-bit counts (top-k)
    unsigned int* h32 = reinterpret_cast<unsigned int*>(S.u.hist);
    for (int i = tid; i < NB; i += TT) S.u.hist[i] = 0ull;
    __syncthreads();
    const unsigned int key = ts[k].key;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const unsigned int bits = __float_as_uint(av[k][u]);   // sign bit: no token
      if ((bits >> KEY_SHIFT) == key) {
        const unsigned int bin = (bits >> SHIFT) & (NB - 1);
        if (bymass) atomicAdd(&S.u.hist[bin], mass_fixed(av[k][u]));
        else atomicAdd(&h32[bin], 1u);
      }
    }
    __syncthreads();
    for (int i = tid; i < NB; i += TT) {
      const unsigned long long v = bymass ? S.u.hist[i] : (unsigned long long)h32[i];
      if (v != 0ull) atomicAdd(&gh[i], v);
    }
    __syncthreads();
  }
  if (!any) return;
  wait_memory_ops();
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < NT; ++k)
      if (tl[k].t >= 0 && !ts[k].done) atomicAdd(&p.sel[(size_t)tl[k].b * p.nR + tl[k].hr].arrive, 1u);
  }
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    if (tl[k].t < 0 || ts[k].done) continue;
    SelState* st = p.sel + (size_t)tl[k].b * p.nR + tl[k].hr;
    const unsigned long long* gh = PASS == 1 ? st->mass : (PASS == 2 ? st->mass2 : st->mass3);
    block_wait(p, &st->arrive, base + (unsigned int)(PASS * p.tail_tph), err);
    unsigned long long v[NB / TT];
#pragma unroll
    for (int e = 0; e < NB / TT; ++e) v[e] = load_u64_coherent(&gh[tid + e * TT]);
#pragma unroll
    for (int e = 0; e < NB / TT; ++e) S.u.hist[tid + e * TT] = v[e];
    __syncthreads();
    const unsigned long long target = ts[k].target;
    int bin;
    unsigned long long above;
    scan_top<NB>(S, ts[k].above, target, bin, above);
    if (bin < 0) {                             // rounding left the total short: keep all
      ts[k].done = true;
      ts[k].tstar = 0u;
    } else if (PASS < 3) {
      ts[k].key = PASS == 1 ? (unsigned int)bin : ((ts[k].key << 10) | (unsigned int)bin);
      ts[k].above = above;
    } else {
      ts[k].done = true;
      ts[k].tstar = (ts[k].key << 9) | (unsigned int)bin;
      if (!bymass) {
        const unsigned long long eq = S.u.hist[bin];
        if (above + eq > target) {
          ts[k].tie = true;
          ts[k].quota = (unsigned int)(target - above);
        }
      }
    }
    __syncthreads();                           // hist is reused by the next tile
  }
}

// Attention of one workgroup over `nrows` rows of KV head h, then the split
// partial (max, sum, unnormalised output) in log2 units, coherent stores.
template <int G, bool FP8, int MODE, int RB = AttRB<G, MODE>::value, bool RET = false>
__device__ __forceinline__ void attend_rows(const DecodeParams& p, TailLds& S, int b, int h, int hr, int split, int lo,
                                            int nrows, const int* pages, const float* lds_logits = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int proc = tid >> 4, sub = tid & 15;
  const size_t pbase = (size_t)(b * p.Hkv + h) * p.max_splits + split;
  float* ml = reinterpret_cast<float*>(p.apart_ml) + pbase * G * 2;   // (max, sum) pairs
  float* po = p.apart_o + pbase * G * D;
  float m[G], l[G], o[G][8];
  if (FP8 && !RET && hr < 0 && p.ring_rows > 0)   // local rows from the ring: bf16
    accumulate_rows<G, false, MODE, RB, RET, true>(p, b, h, hr, lo, nrows, proc * RB, NPROC * RB, sub, S.u.rows,
                                                   pages, S.ltok, S.lpg, lds_logits, m, l, o);
  else
    accumulate_rows<G, FP8, MODE, RB, RET>(p, b, h, hr, lo, nrows, proc * RB, NPROC * RB, sub, S.u.rows, pages,
                                           S.ltok, S.lpg, lds_logits, m, l, o);
  combine_wave_procs<G>(m, l, o);
  __syncthreads();                               // rows / pages no longer read; wo aliases rows
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) { S.wm[wave][g] = m[g]; S.wl[wave][g] = l[g]; }
#pragma unroll
      for (int j = 0; j < 8; ++j) S.u.wo[wave][g][8 * sub + j] = o[g][j];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += TT) {
    const int g = e / D, d = e % D;
    float mm = NEG_INF;
    for (int k = 0; k < TW; ++k) mm = fmaxf(mm, S.wm[k][g]);
    float ll = 0.f, oo = 0.f;
    for (int k = 0; k < TW; ++k) {
      if (S.wm[k][g] == NEG_INF) continue;
      const float cf = fast_exp2(S.wm[k][g] - mm);
      ll += S.wl[k][g] * cf;
      oo += S.u.wo[k][g][d] * cf;
    }
    store_f32_coherent(po + (size_t)g * D + d, oo);
    if (d == 0) {
      store_f32_coherent(ml + 2 * g, mm);
      store_f32_coherent(ml + 2 * g + 1, ll);
    }
  }
}

// A split with no rows.
template <int G>
__device__ __forceinline__ void empty_split(const DecodeParams& p, int b, int h, int split) {
  float* ml = reinterpret_cast<float*>(p.apart_ml) + ((size_t)(b * p.Hkv + h) * p.max_splits + split) * G * 2;
  if (threadIdx.x < G) {
    store_f32_coherent(ml + 2 * threadIdx.x, NEG_INF);
    store_f32_coherent(ml + 2 * threadIdx.x + 1, 0.f);
  }
}

// Count this split as done; the last split of (b, h) merges all of them.
//   out_g = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M);  lse = (M + log2 L) ln 2.
template <int G>
__device__ __forceinline__ void finish_split(const DecodeParams& p, TailLds& S, int b, int h, int hr) {
  const int tid = threadIdx.x;
  const int nspl = hr >= 0 ? p.tail_tph : p.ncL;
  wait_memory_ops();
  __syncthreads();
  if (tid == 0) {
    const unsigned int prev = atomicAdd(&p.tail_sync[1 + b * p.Hkv + h], 1u);
    S.flag = prev == (unsigned int)(nspl - 1) ? 1 : 0;
  }
  __syncthreads();
  const bool last = S.flag != 0;
  __syncthreads();
  if (!last) return;

  const bool bad = load_u32_coherent(&p.tail_sync[0]) != 0u;
  const size_t base = (size_t)(b * p.Hkv + h) * p.max_splits;
  const float* mlf = reinterpret_cast<const float*>(p.apart_ml);
  const int N = min(p.seq_lens[b], p.Nmax);
  for (int e = tid; e < G * D; e += TT) {
    const int g = e / D, d = e % D;
    float M = NEG_INF, L = 0.f, O = 0.f;
    constexpr int SB = 8;
    for (int s0 = 0; s0 < nspl; s0 += SB) {
      float mv[SB], lv[SB], ov[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const bool in = s0 + u < nspl;
        const size_t sp = base + s0 + u;
        mv[u] = in ? load_f32_coherent(mlf + (sp * G + g) * 2) : NEG_INF;
        lv[u] = in ? load_f32_coherent(mlf + (sp * G + g) * 2 + 1) : 0.f;
        ov[u] = in ? load_f32_coherent(p.apart_o + (sp * G + g) * D + d) : 0.f;
      }
      float mt = M;
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (lv[u] > 0.f) mt = fmaxf(mt, mv[u]);
      if (mt == NEG_INF) continue;
      const float cf = fast_exp2(M - mt);
      L *= cf;
      O *= cf;
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        if (lv[u] > 0.f) {
          const float wgt = fast_exp2(mv[u] - mt);
          L = fmaf(lv[u], wgt, L);
          O = fmaf(ov[u], wgt, O);
        }
      }
      M = mt;
    }
    const float nan = __builtin_nanf("");
    p.out[((size_t)b * p.Hq + h * G + g) * D + d] = bad ? nan : (L > 0.f ? O / L : 0.f);
    if (d == 0 && p.lse != nullptr) p.lse[(size_t)b * p.Hq + h * G + g] = bad ? nan : (M + log2f(L)) * LN2;
  }
  if (tid == 0 && p.sel_counts != nullptr) {
    int cnt;
    if (hr >= 0) {
      cnt = (int)load_u32_coherent(&p.sel[(size_t)b * p.nR + hr].nsel);
    } else {
      const int L1 = min(p.n_sink, N);
      cnt = L1 + (N - max(L1, N - p.window));
    }
    p.sel_counts[(size_t)b * p.Hkv + h] = cnt;
  }
  if (tid == 0 && p.sel_mass != nullptr)
    p.sel_mass[(size_t)b * p.Hkv + h] =
        hr >= 0 ? mass_value(load_u64_coherent(&p.sel[(size_t)b * p.nR + hr].kept_mass)) : __builtin_nanf("");
}

// Rows of one local-head chunk of LOCAL_CHUNK rows (sinks first, then the
// window) into S.ltok / S.lpg; returns the row count.
__device__ __forceinline__ int local_rows(const DecodeParams& p, TailLds& S, int item, int& b, int& h, int& c) {
  c = item % p.ncL;
  const int t = item / p.ncL;
  b = t / p.nL;
  h = p.loc_head[t % p.nL];
  const int N = min(p.seq_lens[b], p.Nmax);
  const int L1 = min(p.n_sink, N);
  const int start2 = max(L1, N - p.window);
  const int L = L1 + (N - start2);
  const int llo = c * LOCAL_CHUNK;
  const int nrows = max(0, min(L, llo + LOCAL_CHUNK) - llo);
  const int tid = threadIdx.x;
  if (tid < nrows) {
    const int r = llo + tid;
    local_row_at(p, b, t % p.nL, r < L1 ? r : start2 + (r - L1), S.ltok[tid], S.lpg[tid]);
  }
  return nrows;
}

// Top-k ties at t*, then the kept-token masks: a_i > t*, and for top-k the
// ties at t* that rank below the quota in position order.  Every tile of a
// tie head publishes its tie count first and only then waits for the counts
// of the head's other tiles, so the hand-off has no cycles.
template <int NT, bool WM>
__device__ __forceinline__ void tie_keep(const DecodeParams& p, TailLds& S, const Tile (&tl)[NT],
                                         const float (&av)[NT][TPT], const TileSel (&ts)[NT],
                                         unsigned int (&keepm)[NT], unsigned int* err) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned int before[NT];
  bool any_tie = false;
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    before[k] = 0u;
    if (tl[k].t < 0 || !ts[k].tie) continue;
    any_tie = true;
    unsigned int c = 0u;
#pragma unroll
    for (int u = 0; u < TPT; ++u) c += __float_as_uint(av[k][u]) == ts[k].tstar ? 1u : 0u;
    for (int off = 1; off < 64; off <<= 1) c += __shfl_xor(c, off);
    __syncthreads();
    if (lane == 0) S.tmp[wave] = c;
    __syncthreads();
    if (tid == 0) {
      unsigned int tot = 0u;
      for (int w2 = 0; w2 < TW; ++w2) tot += S.tmp[w2];
      __hip_atomic_store(&p.tail_ties[tl[k].t], tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (any_tie) {
    wait_memory_ops();
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int k = 0; k < NT; ++k)
        if (tl[k].t >= 0 && ts[k].tie) atomicAdd(&p.sel[(size_t)tl[k].b * p.nR + tl[k].hr].tie_arrive, 1u);
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if (tl[k].t < 0 || !ts[k].tie) continue;
      block_wait(p, &p.sel[(size_t)tl[k].b * p.nR + tl[k].hr].tie_arrive, (unsigned int)p.tail_tph, err);
      if (tid == 0) {
        unsigned int sum = 0u;
        const int t0 = tl[k].t - tl[k].j;
        for (int jj = 0; jj < tl[k].j; ++jj) sum += load_u32_coherent(&p.tail_ties[t0 + jj]);
        S.tmp[TW] = sum;
      }
      __syncthreads();
      before[k] = S.tmp[TW];
      __syncthreads();
    }
  }

  // ---- kept tokens: a_i > t*, and for top-k the ties at t* that rank below
  // the quota in position order ----
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    keepm[k] = 0u;
    if (tl[k].t < 0) continue;
    SelState* st = p.sel + (size_t)tl[k].b * p.nR + tl[k].hr;
    const unsigned int tstar = ts[k].tstar;
    if (tl[k].j == 0 && tid == 0) {
      st->tstar = tstar;
      st->quota = ts[k].quota;
      st->flags = SEL_FINISHED | (ts[k].tie ? SEL_TIE : 0u);
      // selection alone (the per-stage attention follows): top-k keeps
      // min(k, N) tokens (the tie quota tops the set up to k); top-p sets
      // are counted by the attention
      if (p.agg_out && p.select_mode != 0) st->nsel = (unsigned int)min((unsigned long long)tl[k].N, ts[k].target);
    }
    unsigned int gt = 0u, eq = 0u;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const unsigned int bits = __float_as_uint(av[k][u]);
      if (!(bits >> 31)) {
        if (bits > tstar) gt |= 1u << u;
        else if (bits == tstar) eq |= 1u << u;
      }
    }
    if (ts[k].tie) {
      __syncthreads();
      count_flags<WM>(S, eq);
      __syncthreads();
      scan_cnt(S);
      unsigned int kept = 0u;
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const unsigned long long bal = __ballot((eq >> u) & 1u);
        const unsigned int rank = before[k] + S.cnt[cnt_idx<WM>(u, wave)] + lane_rank(bal);
        if (((eq >> u) & 1u) && rank < ts[k].quota) kept |= 1u << u;
      }
      eq = kept;
      __syncthreads();
    }
    keepm[k] = gt | eq;
  }
}

// Kept positions of a tile (bit u of `keep` = slot u of this thread) into
// S.u.rows in position order; returns their number.
template <bool WM>
__device__ __forceinline__ int compact_rows(TailLds& S, unsigned int keep) {
  const int tid = threadIdx.x, wave = tid >> 6;
  count_flags<WM>(S, keep);
  __syncthreads();
  const int nrows = (int)scan_cnt(S);
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const unsigned long long bal = __ballot((keep >> u) & 1u);
    if ((keep >> u) & 1u) S.u.rows[S.cnt[cnt_idx<WM>(u, wave)] + lane_rank(bal)] = (unsigned short)slot_pos<WM>(u, tid);
  }
  return nrows;
}

// Selection for the tiles of workgroup w (its XCD-local id, tile t = w + k *
// gridDim.x): a_i of every token, the three radix passes, top-k ties.  Leaves
// the tiles in tl, their kept-token masks in keepm and the block-table
// entries in S.pages.
template <int G>
__device__ __forceinline__ void select_tiles(const DecodeParams& p, TailLds& S, Tile (&tl)[MAXT], unsigned int (&keepm)[MAXT],
                             int& my_tiles, unsigned int* err) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwg = gridDim.x, w = xcd_local_id(blockIdx.x, min(p.tail_ntiles, nwg));
  const bool bymass = p.select_mode == 0;
  TileSel ts[MAXT];
  float av[MAXT][TPT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int t = w + k * nwg;
    ts[k] = TileSel{false, 0u, 0ull, 0u, false, 0u, 0ull};
    if (t >= p.tail_ntiles) {
      tl[k] = Tile{-1, 0, 0, 0, 0, 0, 0};
      continue;
    }
    const int head = t / p.tail_tph;
    tl[k].t = t;
    tl[k].j = t % p.tail_tph;
    tl[k].b = head / p.nR;
    tl[k].hr = head % p.nR;
    tl[k].N = min(p.seq_lens[tl[k].b], p.Nmax);
    tl[k].lo = tl[k].j * TAIL_TILE;
    tl[k].hi = min(tl[k].N, tl[k].lo + TAIL_TILE);
  }

  // ---- a_i = mean_g 2^(x_gi - LSE2_g) for the tokens of each tile ----
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    if (tl[k].t < 0) {
#pragma unroll
      for (int u = 0; u < TPT; ++u) av[k][u] = -1.0f;
      continue;
    }
    const int b = tl[k].b, hr = tl[k].hr, N = tl[k].N, lo = tl[k].lo, hi = tl[k].hi;
    const size_t row = (size_t)(b * p.nR + hr);
    const int* bt = p.block_tables + (size_t)b * p.max_blocks;
    const int npg = hi > lo ? (hi - lo + BS - 1) / BS : 0;
    for (int e = tid; e < npg; e += TT) S.pages[k][e] = bt[(lo >> 4) + e];
    const int nsc = (N + p.score_chunk - 1) / p.score_chunk;
    if (wave < G) {
      const float2* sp = p.spart + row * p.n_score_chunks * G + wave;
      float m = NEG_INF, s = 0.f;
      for (int j0 = lane; j0 < nsc; j0 += 256) {
        float2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = j0 + 64 * u;
          v[u] = jj < nsc ? sp[(size_t)jj * G] : make_float2(NEG_INF, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) lse_combine(m, s, v[u].x, v[u].y);
      }
      for (int off = 1; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        lse_combine(m, s, m2, s2);
      }
      if (lane == 0) S.lse[k][wave] = m + log2f(s);
    }
    __syncthreads();
    if (tl[k].j == 0 && tid < G) p.sel[row].lse2[tid] = S.lse[k][tid];
    float lse[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lse[g] = S.lse[k][g];
    const float c2 = p.c2_score;
    const float invG = 1.0f / (float)G;
    const float* sc = p.scores + row * p.Nmax * G;
    // a_i goes out for the sel_idx output and for the per-stage attention
    // (the balanced attention reads the kept lists instead)
    float* agg = (p.sel_idx != nullptr || (p.agg_out && p.row_list == nullptr)) ? p.agg + row * p.Nagg : nullptr;
    // loads of UB tokens in flight at once; positions past the end re-read
    // the last token and are masked, so no load sits behind a per-lane branch
    constexpr int UB = G <= 2 ? 32 : (G == 4 ? 16 : 8);
#pragma unroll
    for (int u = 0; u < TPT; ++u) av[k][u] = -1.0f;
    if (hi > lo) {
#pragma unroll
      for (int u0 = 0; u0 < TPT; u0 += UB) {
        float x[UB][G];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int i = min(lo + (u0 + u) * TT + tid, hi - 1);
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
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int i = lo + (u0 + u) * TT + tid;
          float a = 0.f;
#pragma unroll
          for (int g = 0; g < G; ++g) a += fast_exp2(x[u][g] * c2 - lse[g]);
          a *= invG;
          if (i < hi) {
            av[k][u0 + u] = a;
            if (agg != nullptr) agg[i] = a;
          }
        }
      }
    }
    // the whole sequence kept: no threshold to find
    bool all;
    ts[k].target = sel_target(p, tl[k].b, N, all);
    if (all) {
      ts[k].done = true;
      ts[k].tstar = 0u;
    }
  }

  // ---- three radix passes; the tiles of a head wait only for each other ----
  radix_pass<1, MAXT>(p, S, tl, av, ts, bymass, err, 0u);
  radix_pass<2, MAXT>(p, S, tl, av, ts, bymass, err, 0u);
  radix_pass<3, MAXT>(p, S, tl, av, ts, bymass, err, 0u);
  tie_keep<MAXT, false>(p, S, tl, av, ts, keepm, err);
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    my_tiles += tl[k].t >= 0 ? 1 : 0;
    if (p.sel_mass != nullptr && tl[k].t >= 0)
      add_kept_mass(&p.sel[(size_t)tl[k].b * p.nR + tl[k].hr].kept_mass, av[k], keepm[k]);
  }
}

template <int G, bool FP8, int MODE>
__global__ __launch_bounds__(TT) void tail_kernel(DecodeParams p) {
  static_assert(MAXT == 2, "the work loop picks tile slots 0 / 1");
  __shared__ TailLds S;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nwg = gridDim.x, w = xcd_local_id(blockIdx.x, min(p.tail_ntiles, nwg));
  unsigned int* err = p.tail_sync;

  // Local-head chunks: item i goes to workgroup (ntiles + i) mod nwg, so the
  // workgroups without a tile take the first ones and start on them at once.
  const int nitems = (MODE == 1) ? 0 : p.B * p.nL * p.ncL;
  const int first_item = ((w - p.tail_ntiles) % nwg + nwg) % nwg;
  const int my_items = first_item < nitems ? (nitems - first_item + nwg - 1) / nwg : 0;
  int my_tiles = 0;
  unsigned int keepm[MAXT];                     // kept tokens of each tile, bit u = slot u
  Tile tl[MAXT];
  if (w < p.tail_ntiles) select_tiles<G>(p, S, tl, keepm, my_tiles, err);

  // ---- work list: this workgroup's tiles, then its local-head chunks ----
  for (int wi = 0; wi < my_tiles + my_items; ++wi) {
    int b, h, hr, split, lo = 0, nrows;
    const int* pages = nullptr;
    __syncthreads();                            // LDS of the previous item is free
    if (wi < my_tiles) {
      const Tile t = wi == 0 ? tl[0] : tl[MAXT - 1];
      const unsigned int keep = wi == 0 ? keepm[0] : keepm[MAXT - 1];
      b = t.b;
      hr = t.hr;
      h = p.ret_head[hr];
      split = t.j;
      lo = t.lo;
      pages = S.pages[wi == 0 ? 0 : MAXT - 1];
      nrows = compact_rows<false>(S, keep);
      if (tid == 0 && nrows > 0) atomicAdd(&p.sel[(size_t)b * p.nR + hr].nsel, (unsigned int)nrows);
    } else {
      hr = -1;
      if constexpr (MODE != 1) nrows = local_rows(p, S, first_item + (wi - my_tiles) * nwg, b, h, split);
      else { b = h = split = 0; nrows = 0; }     // no local heads in this mode
    }
    __syncthreads();
    if (nrows > 0) attend_rows<G, FP8, MODE>(p, S, b, h, hr, split, lo, nrows, pages);
    else empty_split<G>(p, b, h, split);
    finish_split<G>(p, S, b, h, hr);
  }
}

// Selection only: a_i of every token (written to agg), the threshold and the
// top-k tie quota of every retrieval head (written to its state), in one
// launch; the attention and merge follow.  With p.row_list set (the attention
// balanced by kept rows follows, and agg is written only for the sel_idx
// output), every tile writes its kept rows,
// (position, page) in position order, into its own region of the head's list
// and their count to tile_cnt (no exchange between tiles), and top-p sets are
// counted here.
template <int G>
__global__ __launch_bounds__(TT) void select_single_kernel(DecodeParams p) {
  __shared__ TailLds S;
  Tile tl[MAXT];
  unsigned int keepm[MAXT];
  int my_tiles = 0;
  if (xcd_local_id(blockIdx.x, min(p.tail_ntiles, (int)gridDim.x)) >= p.tail_ntiles) return;
  unsigned int* err = p.tail_sync;
  select_tiles<G>(p, S, tl, keepm, my_tiles, err);
  if (p.row_list == nullptr) return;
  const int tid = threadIdx.x;
  // ---- each tile: its kept rows, (position, page) in position order, at the
  // start of its own region of the head's list (region j holds positions
  // j * TAIL_TILE ..), and their count ----
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    if (tl[k].t < 0) continue;
    SelState* st = p.sel + (size_t)tl[k].b * p.nR + tl[k].hr;
    __syncthreads();                                  // S.u of the previous tile is free
    const int nrows = compact_rows<false>(S, keepm[k]);
    __syncthreads();
    int2* dst = p.row_list + ((size_t)tl[k].b * p.nR + tl[k].hr) * p.Nmax + tl[k].lo;
    for (int r = tid; r < nrows; r += TT) {
      const int o16 = S.u.rows[r];
      dst[r] = make_int2(tl[k].lo + o16, S.pages[k][o16 >> 4]);
    }
    if (tid == 0) {
      p.tile_cnt[tl[k].t] = (unsigned int)nrows;
      if (p.select_mode == 0 && nrows > 0) atomicAdd(&st->nsel, (unsigned int)nrows);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused decode: full-dim scores, G = 4.  The scoring scan runs inside the
// same launch, one tile per workgroup, and the tile's 16384 x 4 scores stay
// in registers: wave w scans pages w*128 .. w*128+127 of the tile, four at a
// time (the MFMA layout of the scoring kernel: lane quad u takes page u, so
// each lane owns one token of every 4-page group, 32 tokens in all).  The
// query rows of the A operand repeat the group's four heads four times.
// FP8: e4m3 pages read 16 codes per lane load (the dims of the MFMA steps
// permuted to match, in the query operand too), widened to bf16 (exact), two
// groups of loads in flight (the bytes of one bf16 group), each page's
// products times its K scale.  SPLITQ (rotated fp32 queries): rows 0-3 carry each query's bf16
// part and rows 4-7 the bf16 rounding of the rest, so a page's MFMAs give
// both products and the lanes of quads 2k and 2k+1 add them with one swap.
// The scores equal the per-stage scan's bit for bit (the same products,
// additions and scaling).  The log-sum-exp of every query head is exchanged
// between the tiles of the head like a radix pass; then a_i, the passes, the
// compaction and the attention follow as in the tail.  Only the kept
// tokens' scores are written out (the attention reads its logits from
// there), unless all scores were asked for.
// ---------------------------------------------------------------------------
constexpr int FPW = TAIL_TILE / BS / TW;     // pages per wave: 128
static_assert(FPW == 4 * TPT, "a lane owns one token of every 4-page group");

constexpr int FUSED_LOGITS = 2048;          // kept rows whose logits stay in LDS
constexpr int FUSED_RB = 12;                 // rows per processor per gather batch

template <int MODE, bool FP8, bool SPLITQ>
__device__ __forceinline__ void fused_tile(const DecodeParams& p, TailLds& S, f32x4* logits, unsigned int* err,
                                           int t) {
  constexpr int G = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, quad = lane >> 4;
  const bool bymass = p.select_mode == 0;
  Tile tl[1];
  TileSel ts[1];
  {
    const int head = t / p.tail_tph;
    tl[0].t = t;
    tl[0].j = t % p.tail_tph;
    tl[0].b = head / p.nR;
    tl[0].hr = head % p.nR;
    tl[0].N = min(p.seq_lens[tl[0].b], p.Nmax);
    tl[0].lo = tl[0].j * TAIL_TILE;
    tl[0].hi = min(tl[0].N, tl[0].lo + TAIL_TILE);
    ts[0] = TileSel{false, 0u, 0ull, 0u, false, 0u, 0ull};
    bool all;
    ts[0].target = sel_target(p, tl[0].b, tl[0].N, all);
    ts[0].done = all;                           // the whole sequence kept: no threshold to find
  }
  const int b = tl[0].b, hr = tl[0].hr, j = tl[0].j, N = tl[0].N, lo = tl[0].lo, hi = tl[0].hi;
  const int h = p.ret_head[hr];
  const size_t hrow = (size_t)(b * p.nR + hr);
  SelState* st = p.sel + hrow;

  // ---- scoring scan: x[u] = the 4 raw scores q_g . k of this lane's token u ----
  bf16x8 afrag[4];
  if constexpr (SPLITQ) {
    const float* qg = p.qrot + ((size_t)b * p.Hq + h * G + (row & 3)) * D;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xq = qg[mfma_dim0<FP8>(s2, quad) + e];
        const float hiq = bf16_to_f32(f32_to_bf16_rne(xq));
        afrag[s2][e] = (__bf16)((row & 4) ? xq - hiq : hiq);
      }
    }
  } else {
    const uint16_t* qg = p.q + ((size_t)b * p.Hq + h * G + (row & 3)) * D;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      afrag[s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qg + mfma_dim0<FP8>(s2, quad)));
  }
  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const int page0 = (lo >> 4) + wave * FPW;                // sequence page of this wave's first page
  const int blkA = (page0 + lane) * BS < N ? bt[page0 + lane] : -1;
  const int blkB = (page0 + 64 + lane) * BS < N ? bt[page0 + 64 + lane] : -1;
  S.pages[0][wave * FPW + lane] = blkA;
  S.pages[0][wave * FPW + 64 + lane] = blkB;
  const int ngroups = min(TPT, max(0, (N - page0 * BS + 4 * BS - 1) / (4 * BS)));
  const uint16_t* kbase =
      reinterpret_cast<const uint16_t*>(p.k_pool) + (size_t)p.pool_slot[h] * (BS * D) + (size_t)row * 32 + 8 * quad;
  const size_t page_stride = (size_t)p.Hp * (BS * D);
  const float c2 = p.c2_score;
  float x[TPT][G];
  float m[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = NEG_INF; sm[g] = 0.f; }
  // SPLITQ: in page p's accumulator, 16-lane rows 0 and 2 hold the products
  // of the queries' bf16 parts and rows 1 and 3 those of the rest.  One
  // v_permlane16_swap of pages (0, 1) and one of pages (2, 3) exchange rows
  // 1 <-> 0 and 3 <-> 2 across the pair, so that the two results hold, in
  // every lane, the two kinds of the lane's own page; their sum is hi + lo.
  auto fold_split = [&](const f32x4 (&acc)[4]) -> f32x4 {
    f32x4 v;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[0][g]), __float_as_uint(acc[1][g]),
                                                      false, false);
      const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[2][g]), __float_as_uint(acc[3][g]),
                                                      false, false);
      const float r01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const float r23 = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      v[g] = quad < 2 ? r01 : r23;
    }
    return v;
  };

  auto online = [&](int u, const f32x4& v) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[u][g] = v[g];
    if (lo + wave * (TPT * 64) + u * 64 + lane < hi) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float z = v[g] * c2;
        const float mn = fmaxf(m[g], z);
        sm[g] = sm[g] * fast_exp2(m[g] - mn) + fast_exp2(z - mn);
        m[g] = mn;
      }
    }
  };
  if constexpr (FP8) {
    // K scale of the lane's pages (1 for a page out of range: its products are zeroed)
    const size_t hs = (size_t)p.pool_slot[h];
    const float scA = (unsigned)blkA < (unsigned)p.num_blocks ? p.kv_scales[((size_t)blkA * p.Hp + hs) * 2] : 1.f;
    const float scB = (unsigned)blkB < (unsigned)p.num_blocks ? p.kv_scales[((size_t)blkB * p.Hp + hs) * 2] : 1.f;
    // this lane's two 16-code loads of a page: at kb8 and kb8 + 1024
    const char* kb8 = reinterpret_cast<const char*>(p.k_pool) + hs * (BS * D) + fp8_page_lane_off(row, quad);
#pragma unroll
    for (int u0 = 0; u0 < TPT; u0 += 2) {
      u32x4 f[2][4][2];
      unsigned valid[2] = {0u, 0u};
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (u0 + uu < ngroups) {                           // wave-uniform
#pragma unroll
          for (int pg = 0; pg < 4; ++pg) {
            const int idx = 4 * (u0 + uu) + pg;
            const int blk = __builtin_amdgcn_readlane(idx < 64 ? blkA : blkB, idx & 63);
            const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
            valid[uu] |= ok ? (1u << pg) : 0u;
            const char* src = kb8 + (size_t)(ok ? blk : 0) * page_stride;
            f[uu][pg][0] = load_nt16(src);
            f[uu][pg][1] = load_nt16(src + 1024);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = u0 + uu;
#pragma unroll
        for (int g = 0; g < G; ++g) x[u][g] = 0.f;
        if (u >= ngroups) continue;                        // wave-uniform
        f32x4 acc[4];
#pragma unroll
        for (int pg = 0; pg < 4; ++pg) {
          acc[pg] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            acc[pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[s2], fp8_step(f[uu][pg][s2 >> 1], s2), acc[pg], 0, 0, 0);
          if (!((valid[uu] >> pg) & 1u)) acc[pg] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        f32x4 v;
        if constexpr (SPLITQ) {
          v = fold_split(acc);
        } else {
          v = acc[0];
          v = quad == 1 ? acc[1] : v;
          v = quad == 2 ? acc[2] : v;
          v = quad == 3 ? acc[3] : v;
        }
        // this lane's page 4u + quad: the four scales read as wave-uniform values
        const int scw = __float_as_int(u < 16 ? scA : scB);
        const float s0 = __int_as_float(__builtin_amdgcn_readlane(scw, (4 * u) & 63));
        const float s1 = __int_as_float(__builtin_amdgcn_readlane(scw, (4 * u + 1) & 63));
        const float s2 = __int_as_float(__builtin_amdgcn_readlane(scw, (4 * u + 2) & 63));
        const float s3 = __int_as_float(__builtin_amdgcn_readlane(scw, (4 * u + 3) & 63));
        float ks = s0;
        ks = quad == 1 ? s1 : ks;
        ks = quad == 2 ? s2 : ks;
        ks = quad == 3 ? s3 : ks;
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] *= ks;
        online(u, v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[u][g] = 0.f;
    if (u < ngroups) {                                     // wave-uniform
      bf16x8 f[4][4];
      unsigned valid = 0u;
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
        const int idx = 4 * u + pg;
        const int blk = __builtin_amdgcn_readlane(idx < 64 ? blkA : blkB, idx & 63);
        const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
        valid |= ok ? (1u << pg) : 0u;
        const uint16_t* src = kbase + (size_t)(ok ? blk : 0) * page_stride;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) f[pg][s2] = __builtin_bit_cast(bf16x8, load_nt16(src + 512 * s2));
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc[4];
#pragma unroll
      for (int pg = 0; pg < 4; ++pg) {
        acc[pg] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          acc[pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[s2], f[pg][s2], acc[pg], 0, 0, 0);
        if (!((valid >> pg) & 1u)) acc[pg] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      f32x4 v;
      if constexpr (SPLITQ) {
        v = fold_split(acc);
      } else {
        v = acc[0];
        v = quad == 1 ? acc[1] : v;
        v = quad == 2 ? acc[2] : v;
        v = quad == 3 ? acc[3] : v;
      }
      online(u, v);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }

  stamp_phase(p, 1);
  // ---- log-sum-exp of the head: this tile's partial, exchanged between tiles ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m[g], off), s2 = __shfl_xor(sm[g], off);
      lse_combine(m[g], sm[g], m2, s2);
    }
    if (lane == 0) { S.wm[wave][g] = m[g]; S.wl[wave][g] = sm[g]; }
  }
  __syncthreads();
  // this tile's share of the head's radix bins back to zero (device-coherent
  // stores, acknowledged before the arrival that every flush waits for)
  {
    constexpr int NBIN = HIST_BINS + P2_BINS + P3_BINS;
    for (int e = j * TT + tid; e < NBIN; e += p.tail_tph * TT) {
      unsigned long long* bin = e < HIST_BINS ? &st->mass[e]
                              : (e < HIST_BINS + P2_BINS ? &st->mass2[e - HIST_BINS] : &st->mass3[e - HIST_BINS - P2_BINS]);
      __hip_atomic_store(bin, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  float* spf = reinterpret_cast<float*>(p.spart) + hrow * p.n_score_chunks * G * 2;   // [tile][g] (max, sum)
  if (tid < G) {
    float mm = S.wm[0][tid], ss = S.wl[0][tid];
    for (int w2 = 1; w2 < TW; ++w2) lse_combine(mm, ss, S.wm[w2][tid], S.wl[w2][tid]);
    store_f32_coherent(spf + ((size_t)j * G + tid) * 2, mm);
    store_f32_coherent(spf + ((size_t)j * G + tid) * 2 + 1, ss);
  }
  wait_memory_ops();
  __syncthreads();
  if (tid == 0) atomicAdd(&st->arrive, 1u);
  block_wait(p, &st->arrive, (unsigned int)p.tail_tph, err);
  if (wave < G) {
    float mm = NEG_INF, ss = 0.f;
    for (int jj = lane; jj < p.tail_tph; jj += 64)
      lse_combine(mm, ss, load_f32_coherent(spf + ((size_t)jj * G + wave) * 2),
                  load_f32_coherent(spf + ((size_t)jj * G + wave) * 2 + 1));
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(mm, off), s2 = __shfl_xor(ss, off);
      lse_combine(mm, ss, m2, s2);
    }
    if (lane == 0) S.lse[0][wave] = mm + log2f(ss);
  }
  __syncthreads();
  float lse[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lse[g] = S.lse[0][g];
  if (j == 0 && tid < G) st->lse2[tid] = S.lse[0][tid];
  stamp_phase(p, 2);

  // ---- a_i = mean_g 2^(x_gi - LSE2_g) ----
  float av[1][TPT];
  float* agg = p.sel_idx != nullptr ? p.agg + hrow * p.Nagg : nullptr;
  float* sc = p.scores + hrow * p.Nmax * G;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int i = lo + wave * (TPT * 64) + u * 64 + lane;
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) a += fast_exp2(x[u][g] * c2 - lse[g]);
    a *= 0.25f;
    av[0][u] = i < hi ? a : -1.0f;
    if (i < hi) {
      if (agg != nullptr) agg[i] = a;
      if (p.scores_out) *reinterpret_cast<f32x4*>(sc + (size_t)i * G) = (f32x4){x[u][0], x[u][1], x[u][2], x[u][3]};
    }
  }

  // ---- radix passes (the arrival counter already holds the exchange) ----
  const unsigned int base = (unsigned int)p.tail_tph;
  stamp_phase(p, 3);
  radix_pass<1, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 4);
  radix_pass<2, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 5);
  radix_pass<3, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 6);
  unsigned int keepm[1];
  tie_keep<1, true>(p, S, tl, av, ts, keepm, err);
  const unsigned int keep = keepm[0];
  if (p.sel_mass != nullptr) add_kept_mass(&st->kept_mass, av[0], keep);
  stamp_phase(p, 7);

  // ---- ordered compaction; the kept tokens' scores (the attention's logits)
  // go to LDS next to the row list, or to the scores buffer if too many ----
  // A wave owns 2048 consecutive positions (slot u, lane): its kept tokens
  // go after those of the waves before it, in (u, lane) order.
  unsigned int wcount = 0u;
#pragma unroll
  for (int u = 0; u < TPT; ++u) wcount += (unsigned int)__popcll(__ballot((keep >> u) & 1u));
  if (lane == 0) S.tmp[wave] = wcount;
  __syncthreads();
  unsigned int run = 0u, total = 0u;
#pragma unroll
  for (int w2 = 0; w2 < TW; ++w2) {
    const unsigned int c = S.tmp[w2];
    run += w2 < wave ? c : 0u;
    total += c;
  }
  const int nrows = (int)total;
  const bool lds = nrows <= FUSED_LOGITS;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const unsigned long long bal = __ballot((keep >> u) & 1u);
    const unsigned int slot0 = run;
    run += (unsigned int)__popcll(bal);
    if ((keep >> u) & 1u) {
      const int slot = slot0 + lane_rank(bal);
      const int off = slot_pos<true>(u, tid);
      S.u.rows[slot] = (unsigned short)off;
      const f32x4 v = (f32x4){x[u][0], x[u][1], x[u][2], x[u][3]};
      if (lds) logits[slot] = v;
      else if (!p.scores_out) *reinterpret_cast<f32x4*>(sc + (size_t)(lo + off) * G) = v;
    }
  }
  if (!lds) wait_memory_ops();
  if (tid == 0 && nrows > 0) atomicAdd(&st->nsel, (unsigned int)nrows);
  __syncthreads();
  stamp_phase(p, 8);
  if (nrows > 0)
    attend_rows<G, FP8, MODE, FUSED_RB, true>(p, S, b, h, hr, j, lo, nrows, S.pages[0],
                                                lds ? reinterpret_cast<const float*>(logits) : nullptr);
  else
    empty_split<G>(p, b, h, j);
  stamp_phase(p, 9);
  finish_split<G>(p, S, b, h, hr);
  stamp_phase(p, 10);
}

template <int MODE, bool FP8, bool SPLITQ>
__global__ __launch_bounds__(TT) void fused_g4_kernel(DecodeParams p) {
  __shared__ TailLds S;
  __shared__ f32x4 logits[FUSED_LOGITS];
  const int nwg = gridDim.x, w = xcd_local_id(blockIdx.x, min(p.tail_ntiles, nwg));
  unsigned int* err = p.tail_sync;
  stamp_phase(p, 0);
  if (w < p.tail_ntiles) fused_tile<MODE, FP8, SPLITQ>(p, S, logits, err, w);
  if constexpr (MODE != 1) {
    // local-head chunks: item i goes to workgroup (ntiles + i) mod nwg
    const int nitems = p.B * p.nL * p.ncL;
    const int first_item = ((w - p.tail_ntiles) % nwg + nwg) % nwg;
    for (int it = first_item; it < nitems; it += nwg) {
      int b, h, c;
      __syncthreads();
      const int nrows = local_rows(p, S, it, b, h, c);
      __syncthreads();
      if (nrows > 0) attend_rows<4, FP8, MODE>(p, S, b, h, -1, c, 0, nrows, nullptr);
      else empty_split<4>(p, b, h, c);
      finish_split<4>(p, S, b, h, -1);
    }
  }
  stamp_phase(p, 11);
}

// ---------------------------------------------------------------------------
// Fused decode with r = 16 index scores ([RTPurbo] Methodology §2: the index
// scan streams 64 B (fp32) or 32 B (bf16) per token and retrieval head): the
// scan runs inside the launch, one tile of TT * SP tokens per workgroup, and
// the tile's scores stay in registers.  Wave w scans the tile's pages
// w*4*SP .. w*4*SP + 4*SP - 1, four pages per slot u.  fp32 index: a page
// (16 tokens x 16 dims, 1 KiB) is one wave load, lane l holding four dims of
// token l % 16 -- 16-lane group j holds dims 4*s(j) .. +3 with s = (0, 2, 1, 3)
// -- and the four pages' partial dot products are summed over the groups by
// one x32 and one x16 lane swap, which leave lane l with the scores of token
// l of the slot's 64 positions; the additions pair the same terms as the
// per-stage scan (dims 0-3 with 4-7, 8-11 with 12-15, then the two halves),
// so both give the same scores.  bf16 index: one wave load covers two 512 B
// pages (lanes 0-31 and 32-63), a lane holding eight dims, and the x16 swap
// alone completes the sums.  Then, as in the full-dim fused launch: the
// log-sum-exp exchange between the tiles of the head, a_i, the radix passes,
// ties, the ordered compaction, and the gathered attention over the kept
// rows (K and V rows, logits from q.k) with the last split merging.
// ---------------------------------------------------------------------------
// The local-head chunks of workgroup w (item i goes to workgroup
// (ntiles + i) mod nwg), each gathered and finished as a split of its head.
template <int G, bool FP8>
__device__ __forceinline__ void local_items(const DecodeParams& p, TailLds& S, int w, int nwg) {
  const int nitems = p.B * p.nL * p.ncL;
  const int first_item = ((w - p.tail_ntiles) % nwg + nwg) % nwg;
  for (int it = first_item; it < nitems; it += nwg) {
    int b, h, c;
    __syncthreads();
    const int nrows = local_rows(p, S, it, b, h, c);
    __syncthreads();
    if (nrows > 0) attend_rows<G, FP8, 0>(p, S, b, h, -1, c, 0, nrows, nullptr);
    else empty_split<G>(p, b, h, c);
    finish_split<G>(p, S, b, h, -1);
  }
}

template <int G, bool FP8, int SP>
__device__ __forceinline__ void fused_index_tile(const DecodeParams& p, TailLds& S, unsigned int* err, int t) {
  static_assert(SP <= TPT && SP % 4 == 0 && 4 * SP <= 64, "slots in use; a page id per lane");
  constexpr int FPW_I = 4 * SP;                          // pages per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, slot = lane & 15;
  const bool bymass = p.select_mode == 0;
  const bool bf16 = p.index_bf16 != 0;
  Tile tl[1];
  TileSel ts[1];
  {
    const int head = t / p.tail_tph;
    tl[0].t = t;
    tl[0].j = t % p.tail_tph;
    tl[0].b = head / p.nR;
    tl[0].hr = head % p.nR;
    tl[0].N = min(p.seq_lens[tl[0].b], p.Nmax);
    tl[0].lo = tl[0].j * (TT * SP);
    tl[0].hi = min(tl[0].N, tl[0].lo + TT * SP);
    ts[0] = TileSel{false, 0u, 0ull, 0u, false, 0u, 0ull};
    bool all;
    ts[0].target = sel_target(p, tl[0].b, tl[0].N, all);
    ts[0].done = all;
  }
  const int b = tl[0].b, hr = tl[0].hr, j = tl[0].j, N = tl[0].N, lo = tl[0].lo, hi = tl[0].hi;
  const int h = p.ret_head[hr];
  const size_t hrow = (size_t)(b * p.nR + hr);
  SelState* st = p.sel + hrow;

  // ---- page ids of this wave (one per lane), then every index load of the
  // first group of slots, before the projected queries are formed ----
  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const int page0 = (lo >> 4) + wave * FPW_I;
  const int my_blk = (lane < FPW_I && (page0 + lane) * BS < N) ? bt[page0 + lane] : -1;
  if (lane < FPW_I) S.pages[0][wave * FPW_I + lane] = my_blk;
  const int nslots = min(SP, max(0, (N - page0 * BS + 4 * BS - 1) / (4 * BS)));
  const char* ipool = reinterpret_cast<const char*>(p.index_pool);
  const size_t page_bytes = (size_t)BS * R * (bf16 ? 2 : 4);
  // lane's byte offset in a page: fp32: token `slot`, dims 4*s(grp); bf16:
  // token `slot`, dims 8*(grp & 1) of the half's page
  const int sgrp = ((grp & 1) << 1) | (grp >> 1);       // s = (0, 2, 1, 3)
  const int lane_off = bf16 ? slot * 32 + (grp & 1) * 16 : slot * 64 + sgrp * 16;
  // the index load of page q (0..3) of slot u for this lane: fp32 every lane
  // reads page q; bf16 lanes 0-31 read page q and lanes 32-63 page q + 2.
  // Bit q (and q + 2) of `valid` records whether the page id is in range;
  // an out-of-range page reads page 0 and its scores are zeroed.
  auto load_page = [&](int u, int q, unsigned& valid) -> u32x4 {
    const int pg = 4 * u + q;
    const int blk_a = __builtin_amdgcn_readlane(my_blk, pg);
    const int blk_b = __builtin_amdgcn_readlane(my_blk, bf16 ? pg + 2 : pg);
    const bool ok_a = (unsigned)blk_a < (unsigned)p.num_blocks;
    const bool ok_b = (unsigned)blk_b < (unsigned)p.num_blocks;
    valid |= (ok_a ? 1u : 0u) << q;
    if (bf16) valid |= (ok_b ? 1u : 0u) << (q + 2);
    const bool upper = bf16 && lane >= 32;
    const int blk = upper ? (ok_b ? blk_b : 0) : (ok_a ? blk_a : 0);
    return load_nt16(ipool + ((size_t)blk * p.nR + hr) * page_bytes + lane_off);
  };

  // ---- projected queries q~ = P q, split like the per-stage scan's (the
  // first 256 threads, the same partial sums), then this lane's dims ----
  __shared__ float qt_s[MAX_G][R];
  if (tid < 256) {
    constexpr int TPD = 256 / (G * R);
    constexpr int EPT = D / TPD;
    const int dot = tid / TPD, part = tid % TPD;
    const int g = dot / R, jj = dot % R;
    const float4* prow = reinterpret_cast<const float4*>(p.proj + ((size_t)h * R + jj) * D + part * EPT);
    const u32x4* qrow = reinterpret_cast<const u32x4*>(p.q + ((size_t)b * p.Hq + h * G + g) * D + part * EPT);
    float acc = 0.f;
#pragma unroll
    for (int e8 = 0; e8 < EPT / 8; ++e8) {
      const u32x4 w = qrow[e8];
      const float4 pa = prow[2 * e8], pb = prow[2 * e8 + 1];
      acc = fmaf(pa.x, bf16_lo(w[0]), acc);
      acc = fmaf(pa.y, bf16_hi(w[0]), acc);
      acc = fmaf(pa.z, bf16_lo(w[1]), acc);
      acc = fmaf(pa.w, bf16_hi(w[1]), acc);
      acc = fmaf(pb.x, bf16_lo(w[2]), acc);
      acc = fmaf(pb.y, bf16_hi(w[2]), acc);
      acc = fmaf(pb.z, bf16_lo(w[3]), acc);
      acc = fmaf(pb.w, bf16_hi(w[3]), acc);
    }
#pragma unroll
    for (int off = 1; off < TPD; off <<= 1) acc += __shfl_xor(acc, off);
    if (part == 0) qt_s[g][jj] = acc;
  }
  __syncthreads();
  float qv[G][8];
  {
    const int d0 = bf16 ? 8 * (grp & 1) : 4 * sgrp;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[g][e] = (bf16 || e < 4) ? qt_s[g][min(d0 + e, R - 1)] : 0.f;
  }

  // ---- scan: x[u][g] = raw index score of this lane's token of slot u ----
  const float c2 = p.c2_score;
  float x[SP][G];
  float m[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = NEG_INF; sm[g] = 0.f; }
#pragma unroll
  for (int u0 = 0; u0 < SP; u0 += 4) {
    u32x4 kw[4][4];
    unsigned valid[4];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      valid[uu] = 0u;
      if (u0 + uu < nslots) {                               // wave-uniform
        if (bf16) {
          kw[uu][0] = load_page(u0 + uu, 0, valid[uu]);
          kw[uu][1] = load_page(u0 + uu, 1, valid[uu]);
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) kw[uu][q4] = load_page(u0 + uu, q4, valid[uu]);
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int u = u0 + uu;
#pragma unroll
      for (int g = 0; g < G; ++g) x[u][g] = 0.f;
      if (u >= nslots) continue;                            // wave-uniform
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float v;
        if (bf16) {
          // X = pages 0 | 2 (the two halves), Y = pages 1 | 3
          float part[2];
#pragma unroll
          for (int ld = 0; ld < 2; ++ld) {
            const u32x4 w = kw[uu][ld];
            float a = qv[g][0] * bf16_lo(w[0]);
            a = fmaf(qv[g][1], bf16_hi(w[0]), a);
            a = fmaf(qv[g][2], bf16_lo(w[1]), a);
            a = fmaf(qv[g][3], bf16_hi(w[1]), a);
            a = fmaf(qv[g][4], bf16_lo(w[2]), a);
            a = fmaf(qv[g][5], bf16_hi(w[2]), a);
            a = fmaf(qv[g][6], bf16_lo(w[3]), a);
            a = fmaf(qv[g][7], bf16_hi(w[3]), a);
            part[ld] = a;
          }
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                           false, false);
          v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        } else {
          float part[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4 w = kw[uu][q4];
            float a = qv[g][0] * __uint_as_float(w[0]);
            a = fmaf(qv[g][1], __uint_as_float(w[1]), a);
            a = fmaf(qv[g][2], __uint_as_float(w[2]), a);
            a = fmaf(qv[g][3], __uint_as_float(w[3]), a);
            part[q4] = a;
          }
          // pages (0, 2) and (1, 3) over the x32 pairs of groups, then the
          // x16 pairs
          const auto r02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]),
                                                             false, false);
          const auto r13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]),
                                                             false, false);
          const float a0 = __uint_as_float(r02[0]) + __uint_as_float(r02[1]);
          const float a1 = __uint_as_float(r13[0]) + __uint_as_float(r13[1]);
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
          v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        x[u][g] = ((valid[uu] >> grp) & 1u) ? v : 0.f;      // an invalid page scores 0
      }
      if (lo + wave * (SP * 64) + u * 64 + lane < hi) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float z = x[u][g] * c2;
          const float mn = fmaxf(m[g], z);
          sm[g] = sm[g] * fast_exp2(m[g] - mn) + fast_exp2(z - mn);
          m[g] = mn;
        }
      }
    }
  }

  stamp_phase(p, 1);
  // ---- log-sum-exp of the head: this tile's partial, exchanged between tiles ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m[g], off), s2 = __shfl_xor(sm[g], off);
      lse_combine(m[g], sm[g], m2, s2);
    }
    if (lane == 0) { S.wm[wave][g] = m[g]; S.wl[wave][g] = sm[g]; }
  }
  __syncthreads();
  {
    constexpr int NBIN = HIST_BINS + P2_BINS + P3_BINS;
    for (int e = j * TT + tid; e < NBIN; e += p.tail_tph * TT) {
      unsigned long long* bin = e < HIST_BINS ? &st->mass[e]
                              : (e < HIST_BINS + P2_BINS ? &st->mass2[e - HIST_BINS] : &st->mass3[e - HIST_BINS - P2_BINS]);
      __hip_atomic_store(bin, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  float* spf = reinterpret_cast<float*>(p.spart) + hrow * p.n_score_chunks * G * 2;   // [tile][g] (max, sum)
  if (tid < G) {
    float mm = S.wm[0][tid], ss = S.wl[0][tid];
    for (int w2 = 1; w2 < TW; ++w2) lse_combine(mm, ss, S.wm[w2][tid], S.wl[w2][tid]);
    store_f32_coherent(spf + ((size_t)j * G + tid) * 2, mm);
    store_f32_coherent(spf + ((size_t)j * G + tid) * 2 + 1, ss);
  }
  wait_memory_ops();
  __syncthreads();
  if (tid == 0) atomicAdd(&st->arrive, 1u);
  block_wait(p, &st->arrive, (unsigned int)p.tail_tph, err);
  if (wave < G) {
    float mm = NEG_INF, ss = 0.f;
    for (int jj = lane; jj < p.tail_tph; jj += 64)
      lse_combine(mm, ss, load_f32_coherent(spf + ((size_t)jj * G + wave) * 2),
                  load_f32_coherent(spf + ((size_t)jj * G + wave) * 2 + 1));
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(mm, off), s2 = __shfl_xor(ss, off);
      lse_combine(mm, ss, m2, s2);
    }
    if (lane == 0) S.lse[0][wave] = mm + log2f(ss);
  }
  __syncthreads();
  float lse[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lse[g] = S.lse[0][g];
  if (j == 0 && tid < G) st->lse2[tid] = S.lse[0][tid];
  stamp_phase(p, 2);

  // ---- a_i = mean_g 2^(x_gi - LSE2_g); slots past SP hold no token ----
  float av[1][TPT];
  float* agg = p.sel_idx != nullptr ? p.agg + hrow * p.Nagg : nullptr;
  float* sc = p.scores + hrow * p.Nmax * G;
  const float invG = 1.0f / (float)G;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    if (u >= SP) { av[0][u] = -1.0f; continue; }
    const int i = lo + wave * (SP * 64) + u * 64 + lane;
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) a += fast_exp2(x[u < SP ? u : 0][g] * c2 - lse[g]);
    a *= invG;
    av[0][u] = i < hi ? a : -1.0f;
    if (i < hi) {
      if (agg != nullptr) agg[i] = a;
      if (p.scores_out) {
#pragma unroll
        for (int g = 0; g < G; ++g) sc[(size_t)i * G + g] = x[u < SP ? u : 0][g];
      }
    }
  }

  // ---- radix passes (the arrival counter already holds the exchange) ----
  const unsigned int base = (unsigned int)p.tail_tph;
  stamp_phase(p, 3);
  radix_pass<1, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 4);
  radix_pass<2, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 5);
  radix_pass<3, 1>(p, S, tl, av, ts, bymass, err, base);
  stamp_phase(p, 6);
  unsigned int keepm[1];
  tie_keep<1, true>(p, S, tl, av, ts, keepm, err);
  const unsigned int keep = keepm[0];
  if (p.sel_mass != nullptr) add_kept_mass(&st->kept_mass, av[0], keep);
  stamp_phase(p, 7);

  // ---- ordered compaction: a wave's kept tokens after those of the waves
  // before it, in (u, lane) order ----
  unsigned int wcount = 0u;
#pragma unroll
  for (int u = 0; u < SP; ++u) wcount += (unsigned int)__popcll(__ballot((keep >> u) & 1u));
  if (lane == 0) S.tmp[wave] = wcount;
  __syncthreads();
  unsigned int run = 0u, total = 0u;
#pragma unroll
  for (int w2 = 0; w2 < TW; ++w2) {
    const unsigned int c = S.tmp[w2];
    run += w2 < wave ? c : 0u;
    total += c;
  }
  const int nrows = (int)total;
#pragma unroll
  for (int u = 0; u < SP; ++u) {
    const unsigned long long bal = __ballot((keep >> u) & 1u);
    const unsigned int slot0 = run;
    run += (unsigned int)__popcll(bal);
    if ((keep >> u) & 1u) S.u.rows[slot0 + lane_rank(bal)] = (unsigned short)slot_pos<true, SP>(u, tid);
  }
  if (tid == 0 && nrows > 0) atomicAdd(&st->nsel, (unsigned int)nrows);
  __syncthreads();
  stamp_phase(p, 8);
  if (nrows > 0)
    attend_rows<G, FP8, 0>(p, S, b, h, hr, j, lo, nrows, S.pages[0]);
  else
    empty_split<G>(p, b, h, j);
  stamp_phase(p, 9);
  finish_split<G>(p, S, b, h, hr);
  stamp_phase(p, 10);
}

template <int G, bool FP8, int SP>
__global__ __launch_bounds__(TT) void fused_index_kernel(DecodeParams p) {
  __shared__ TailLds S;
  const int nwg = gridDim.x, w = xcd_local_id(blockIdx.x, min(p.tail_ntiles, nwg));
  unsigned int* err = p.tail_sync;
  stamp_phase(p, 0);
  if (w < p.tail_ntiles) fused_index_tile<G, FP8, SP>(p, S, err, w);
  local_items<G, FP8>(p, S, w, nwg);
  stamp_phase(p, 11);
}

// Counters back to zero before a fused launch (the radix bins are cleared by
// the tiles themselves before their first hand-off).
__global__ __launch_bounds__(256) void reset_state_kernel(DecodeParams p) {
  for (int i = threadIdx.x; i < p.B * p.nR; i += 256) {
    SelState* st = p.sel + i;
    st->arrive = 0u;
    st->tie_arrive = 0u;
    st->nsel = 0u;
    st->kept_mass = 0ull;
  }
  for (int i = threadIdx.x; i < 1 + p.B * p.Hkv; i += 256) p.tail_sync[i] = 0u;
}

template <int G, bool FP8, int MODE>
struct TailKernel {
  static void* fn() { return reinterpret_cast<void*>(&tail_kernel<G, FP8, MODE>); }
};

template <int G>
void* pick_mode(const DecodeParams& p) {
  const bool fp8 = p.kv_scales != nullptr;
  if (p.score_mode != 1) return fp8 ? TailKernel<G, true, 0>::fn() : TailKernel<G, false, 0>::fn();
  if (fp8) return nullptr;                       // full-dim scores need a bf16 cache
  return p.nL == 0 ? TailKernel<G, false, 1>::fn() : TailKernel<G, false, 2>::fn();
}

void* pick_kernel(const DecodeParams& p, bool select_only) {
  switch (p.G) {
    case 1: return select_only ? reinterpret_cast<void*>(&select_single_kernel<1>) : pick_mode<1>(p);
    case 2: return select_only ? reinterpret_cast<void*>(&select_single_kernel<2>) : pick_mode<2>(p);
    case 4: return select_only ? reinterpret_cast<void*>(&select_single_kernel<4>) : pick_mode<4>(p);
    case 8: return select_only ? reinterpret_cast<void*>(&select_single_kernel<8>) : pick_mode<8>(p);
  }
  return nullptr;
}

template <int G, bool FP8>
void* pick_index_sp(int sp) {
  switch (sp) {
    case 4: return reinterpret_cast<void*>(&fused_index_kernel<G, FP8, 4>);
    // (G = 8 with 16 slots would spill: only the 2048-position tiles)
    case 16: return G == 8 ? nullptr : reinterpret_cast<void*>(&fused_index_kernel<G, FP8, G == 8 ? 4 : 16>);
  }
  return nullptr;
}

template <int G>
void* pick_index_g(const DecodeParams& p, int sp) {
  return p.kv_scales != nullptr ? pick_index_sp<G, true>(sp) : pick_index_sp<G, false>(sp);
}

}  // namespace

// Workgroups of `fn` (TT threads each) that the current device holds at once,
// looked up once per (kernel, device); 0 when `cooperative` and the device
// has no cooperative launches.
static int resident_grid(void* fn, bool cooperative) {
  if (fn == nullptr) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  struct Entry { void* fn; int dev; int nwg; int coop; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  const Entry* hit = nullptr;
  for (const Entry& e : cache)
    if (e.fn == fn && e.dev == dev) hit = &e;
  if (hit == nullptr) {
    int ncu = 0, occ = 0, coop = 0;
    int nwg = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(fn), TT, 0) == hipSuccess)
      nwg = ncu * occ;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) coop = 0;
    cache.push_back(Entry{fn, dev, nwg, coop});
    hit = &cache.back();
  }
  return (cooperative && hit->coop == 0) ? 0 : hit->nwg;
}

int tail_grid(const DecodeParams& p, bool cooperative, bool select_only) {
  return resident_grid(pick_kernel(p, select_only), cooperative);
}

template <bool FP8, bool SPLITQ>
void* pick_fused_mode(const DecodeParams& p) {
  return p.nL == 0 ? reinterpret_cast<void*>(&fused_g4_kernel<1, FP8, SPLITQ>)
                   : reinterpret_cast<void*>(&fused_g4_kernel<2, FP8, SPLITQ>);
}

void* pick_fused(const DecodeParams& p) {
  if (p.G != 4 || p.score_mode != 1) return nullptr;
  const bool fp8 = p.kv_scales != nullptr, rot = p.qrot != nullptr;
  if (fp8) return rot ? pick_fused_mode<true, true>(p) : pick_fused_mode<true, false>(p);
  return rot ? pick_fused_mode<false, true>(p) : pick_fused_mode<false, false>(p);
}

int fused_grid(const DecodeParams& p, bool cooperative) { return resident_grid(pick_fused(p), cooperative); }

void* pick_fused_index(const DecodeParams& p, int sp) {
  if (p.score_mode != 0 || p.GS != 1) return nullptr;
  switch (p.G) {
    case 1: return pick_index_g<1>(p, sp);
    case 2: return pick_index_g<2>(p, sp);
    case 4: return pick_index_g<4>(p, sp);
    case 8: return pick_index_g<8>(p, sp);
  }
  return nullptr;
}

int fused_index_grid(const DecodeParams& p, int sp, bool cooperative) {
  return resident_grid(pick_fused_index(p, sp), cooperative);
}

// Launch `fn` on nwg workgroups; e0 / e1 (optional) time the dispatch itself.
hipError_t launch_single(void* fn, const DecodeParams& p, int nwg, bool cooperative, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1) {
  DecodeParams arg = p;
  void* args[] = {&arg};
  hipError_t e;
  if (cooperative) {
    if (e0 != nullptr && (e = hipEventRecord(e0, s)) != hipSuccess) return e;
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(nwg), dim3(TT), args, 0, s);
    if (e == hipSuccess && e1 != nullptr) e = hipEventRecord(e1, s);
    return e;
  }
  if (e0 != nullptr || e1 != nullptr)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(nwg), dim3(TT), args, 0, s, e0, e1, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(nwg), dim3(TT), args, 0, s);
}

hipError_t launch_fused(const DecodeParams& p, int nwg, bool cooperative, hipStream_t s, hipEvent_t e0,
                        hipEvent_t e1) {
  void* fn = pick_fused(p);
  if (fn == nullptr || nwg < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reset_state_kernel, dim3(1), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_single(fn, p, nwg, cooperative, s, e0, e1);
}

hipError_t launch_fused_index(const DecodeParams& p, int sp, int nwg, bool cooperative, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  void* fn = pick_fused_index(p, sp);
  if (fn == nullptr || nwg < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reset_state_kernel, dim3(1), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_single(fn, p, nwg, cooperative, s, e0, e1);
}

hipError_t launch_tail(const DecodeParams& p, int nwg, bool cooperative, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1, bool select_only) {
  void* fn = pick_kernel(p, select_only);
  if (fn == nullptr || nwg < 1) return hipErrorInvalidValue;
  return launch_single(fn, p, nwg, cooperative, s, e0, e1);
}

}  // namespace hws
