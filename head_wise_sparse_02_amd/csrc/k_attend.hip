// Split-K decode attention over a token set, and the log-sum-exp merge.
//
// Retrieval heads ([ICS] "Inference-time context sparsity: illusion or
// opportunity?", §3c: sparse decode reads only the selected rows, O(k d)
// instead of O(N d)): a workgroup owns a chunk of positions, keeps the tokens
// of the chunk that pass the threshold found by the selection passes
// (a_i > t*, or a_i == t* and position <= icut), and gathers their K/V rows
// through the block table.  In FULL score mode the attention logits are the
// stored full-dim scores, so only V rows are read.
//
// Local heads ([RTPurbo] "Full attention returns in force ...", Methodology §1;
// [AoH] "Autonomy-of-Heads ...", Methodology §4): the rows are the sinks
// 0..n_sink-1 followed by the window N-w..N-1 (a position in both once),
// split into chunks of LOCAL_CHUNK rows.
//
// Each workgroup emits (max, sum, unnormalised output) per query head in
// log2 units; merge_kernel combines the splits.
#include "hws_device.h"

namespace hws {

constexpr int ATT_ROWS_MAX = 4096;   // largest retrieval chunk (LDS row list)
constexpr int RB = 4;                // rows per 16-lane processor per batch

__device__ __forceinline__ unsigned int block_rank(bool f, unsigned int* tmp) {
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

// Load 8 consecutive elements of a K or V row as fp32 (bf16 or e4m3 codes).
template <bool FP8>
__device__ __forceinline__ void load_row8(const void* pool, size_t row_off, int sub, float* x) {
  if (!FP8) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(pool) + row_off * D + 8 * sub);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint8_t*>(pool) + row_off * D + 8 * sub);
    f32x2 t;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false); x[0] = t.x; x[1] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);  x[2] = t.x; x[3] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false); x[4] = t.x; x[5] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);  x[6] = t.x; x[7] = t.y;
  }
}

template <int G, bool FP8, bool FULL, bool ROPE>
__global__ __launch_bounds__(256) void attend_kernel(DecodeParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int proc = tid >> 4, sub = tid & 15;     // 16 row processors of 16 lanes
  const int w = blockIdx.x;
  const int nret = p.B * p.nR * p.ncR;
  int b, h, split, hr = -1;
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
    h = p.loc_head[t % p.nL];
  }
  const bool is_ret = hr >= 0;
  const int N = min(p.seq_lens[b], p.Nmax);

  __shared__ int rows_s[ATT_ROWS_MAX];
  __shared__ unsigned int tmp[8];
  __shared__ float wm[4][MAX_G], wl[4][MAX_G];
  __shared__ float wo[4][MAX_G][D];

  int nrows = 0;
  if (is_ret) {
    const int lo = split * p.att_chunk_R;
    const int hi = min(N, lo + p.att_chunk_R);
    if (lo < hi) {
      const SelState* st = p.sel + (size_t)b * p.nR + hr;
      const unsigned int tstar = st->tstar, icut = st->icut;
      const float* agg = p.agg + (size_t)(b * p.nR + hr) * p.Nmax;
      for (int base = lo; base < hi; base += 256) {
        const int i = base + tid;
        bool f = false;
        if (i < hi) {
          const unsigned int bits = __float_as_uint(agg[i]);
          f = bits > tstar || (bits == tstar && (unsigned int)i <= icut);
        }
        const unsigned int rank = block_rank(f, tmp);
        if (f) rows_s[nrows + rank] = i;
        nrows += (int)tmp[4];
        __syncthreads();
      }
    }
  } else {
    const int L1 = min(p.n_sink, N);
    const int start2 = max(L1, N - p.window);
    const int L = L1 + (N - start2);
    const int lo = split * LOCAL_CHUNK;
    const int hi = min(L, lo + LOCAL_CHUNK);
    for (int r = lo + tid; r < hi; r += 256) rows_s[r - lo] = r < L1 ? r : start2 + (r - L1);
    nrows = max(0, hi - lo);
    __syncthreads();
  }

  float2* ml = p.apart_ml + ((size_t)(b * p.Hkv + h) * p.max_splits + split) * G;
  if (nrows == 0) {
    if (tid < G) ml[tid] = make_float2(NEG_INF, 0.f);
    return;
  }

  const bool use_scores = FULL && is_ret;
  // queries of the group, pre-scaled to log2 units: dims 8*sub..8*sub+7
  float qf[G][8];
  if (!use_scores) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t qo = ((size_t)b * p.Hq + h * G + g) * D + 8 * sub;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = ROPE ? p.qrot[qo + j] : bf16_to_f32(p.q[qo + j]);
        qf[g][j] = x * p.c2_attn;
      }
    }
  }

  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const float* sc = use_scores ? p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G : nullptr;
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = NEG_INF;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
  }

  for (int r0 = proc * RB; r0 < nrows; r0 += 16 * RB) {
    float z[RB][G];
    float vv[RB][8];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = r0 + u;
      const bool valid = r < nrows;
      const int i = valid ? rows_s[r] : 0;
      const int pg = bt[i >> 4];
      const bool ok = valid && (unsigned)pg < (unsigned)p.num_blocks;
      const size_t row_off = ((size_t)(ok ? pg : 0) * p.Hkv + h) * BS + (i & 15);
      float ks = 1.f, vs = 1.f;
      if (FP8 && ok) {
        ks = p.kv_scales[((size_t)pg * p.Hkv + h) * 2 + 0];
        vs = p.kv_scales[((size_t)pg * p.Hkv + h) * 2 + 1];
      }
      if (ok) {
        load_row8<FP8>(p.v_pool, row_off, sub, vv[u]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) vv[u][j] = 0.f;
      }
      if (FP8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) vv[u][j] *= vs;
      }
      if (use_scores) {
#pragma unroll
        for (int g = 0; g < G; ++g) z[u][g] = ok ? sc[(size_t)i * G + g] * p.c2_score : NEG_INF;
      } else {
        float kx[8];
        if (ok) {
          load_row8<FP8>(p.k_pool, row_off, sub, kx);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) kx[j] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = qf[g][0] * kx[0];
#pragma unroll
          for (int j = 1; j < 8; ++j) a = fmaf(qf[g][j], kx[j], a);
          a += __shfl_xor(a, 1);
          a += __shfl_xor(a, 2);
          a += __shfl_xor(a, 4);
          a += __shfl_xor(a, 8);
          z[u][g] = ok ? a * ks : NEG_INF;
        }
      }
    }
    // one rescale per batch of RB rows
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mn = m[g];
#pragma unroll
      for (int u = 0; u < RB; ++u) mn = fmaxf(mn, z[u][g]);
      if (mn == NEG_INF) continue;                   // uniform over the processor
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

  // combine the 4 processors of each wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], m2);
      const float c1 = (mn == NEG_INF) ? 0.f : fast_exp2(m[g] - mn);
      const float c2 = (mn == NEG_INF) ? 0.f : fast_exp2(m2 - mn);
      l[g] = l[g] * c1 + l2 * c2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o2 = __shfl_xor(o[g][j], off);
        o[g][j] = o[g][j] * c1 + o2 * c2;
      }
      m[g] = mn;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
#pragma unroll
      for (int j = 0; j < 8; ++j) wo[wave][g][8 * sub + j] = o[g][j];
    }
  }
  __syncthreads();
  float* po = p.apart_o + (((size_t)(b * p.Hkv + h) * p.max_splits + split) * G) * D;
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

// out_g = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M);  lse = (M + log2 L) ln 2
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = p.G;
  const int hr = p.ret_slot[h];
  const int nspl = hr >= 0 ? p.ncR : p.ncL;
  const int N = min(p.seq_lens[b], p.Nmax);
  const float2* ml = p.apart_ml + (size_t)(b * p.Hkv + h) * p.max_splits * G;
  const float* po = p.apart_o + (size_t)(b * p.Hkv + h) * p.max_splits * G * D;
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, d = e % D;
    float M = NEG_INF;
    for (int s = 0; s < nspl; ++s) {
      const float2 v = ml[s * G + g];
      if (v.y > 0.f) M = fmaxf(M, v.x);
    }
    float L = 0.f, O = 0.f;
    for (int s = 0; s < nspl; ++s) {
      const float2 v = ml[s * G + g];
      if (v.y > 0.f) {
        const float wgt = fast_exp2(v.x - M);
        L += v.y * wgt;
        O += po[((size_t)s * G + g) * D + d] * wgt;
      }
    }
    p.out[((size_t)b * p.Hq + h * G + g) * D + d] = L > 0.f ? O / L : 0.f;
    if (d == 0 && p.lse != nullptr) p.lse[(size_t)b * p.Hq + h * G + g] = (M + log2f(L)) * LN2;
  }
  if (tid == 0 && p.sel_counts != nullptr) {
    int cnt;
    if (hr >= 0) {
      cnt = (int)p.sel[(size_t)b * p.nR + hr].nsel;
    } else {
      const int L1 = min(p.n_sink, N);
      cnt = L1 + (N - max(L1, N - p.window));
    }
    p.sel_counts[(size_t)b * p.Hkv + h] = cnt;
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
static hipError_t launch_attend_g(const DecodeParams& p, hipStream_t s) {
  const int nwg = p.B * (p.nR * p.ncR + p.nL * p.ncL);
  if (nwg == 0) return hipSuccess;
  const bool full = p.score_mode == 1, rope = p.qrot != nullptr;
  if (full && rope) hipLaunchKernelGGL((attend_kernel<G, FP8, true, true>), dim3(nwg), dim3(256), 0, s, p);
  else if (full) hipLaunchKernelGGL((attend_kernel<G, FP8, true, false>), dim3(nwg), dim3(256), 0, s, p);
  else if (rope) hipLaunchKernelGGL((attend_kernel<G, FP8, false, true>), dim3(nwg), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((attend_kernel<G, FP8, false, false>), dim3(nwg), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_attend_fp(const DecodeParams& p, hipStream_t s, bool fp8) {
  return fp8 ? launch_attend_g<G, true>(p, s) : launch_attend_g<G, false>(p, s);
}

hipError_t launch_attend(const DecodeParams& p, hipStream_t s) {
  const bool fp8 = p.kv_scales != nullptr;
  switch (p.G) {
    case 1: return launch_attend_fp<1>(p, s, fp8);
    case 2: return launch_attend_fp<2>(p, s, fp8);
    case 4: return launch_attend_fp<4>(p, s, fp8);
    case 8: return launch_attend_fp<8>(p, s, fp8);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(p.Hkv, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prep_q(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(prep_q_kernel, dim3(p.Hq, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
