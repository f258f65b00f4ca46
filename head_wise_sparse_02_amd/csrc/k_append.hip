// Cache append: write new K/V rows into their pages and, for retrieval heads,
// the projected pre-RoPE key k~ = P_h k into the index pool.
//
// [RTPurbo] "Full attention returns in force ...", Methodology §2: the index
// projection is applied before RoPE.  [AoH] "Autonomy-of-Heads ...", Problem
// statement: the KV cache grows by one row per token.
//
// One workgroup per (sequence, page touched, KV head).  With RoPE on, K is
// rotated at its position (angle and rotation in fp64) and rounded once to
// bf16.  FP8 pages hold OCP e4m3fn codes of x / scale; a call that writes
// slot 0 of a page sets that page's scale to amax/448 over the rows it
// writes there (1.0 if they are all zero); later calls keep the scale.
//
// Local ring ([RTPurbo] Methodology §1: a local head attends to its sinks and
// its window only): local heads write the sequence's ring slot instead of the
// pages, and only the rows a decode or a prefill chunk can still read: the
// first ring_sink positions (the sinks, rounded up to a 64-key tile) and the
// last ring_mod positions of the call (window + slack, in distinct ring rows,
// so no two writers meet); older rows are overwritten as the sequence grows.
#include "hws_device.h"

namespace hws {

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

template <bool FP8, bool ROPE>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int jb = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int p0 = p.start_pos[s];
  if (p0 < 0) return;
  const int blk_l = p0 / BS + jb;
  const int lo = max(p0, blk_l * BS), hi = min(p0 + p.n_tok, blk_l * BS + BS);
  if (lo >= hi || blk_l >= p.max_blocks) return;
  const int hr = p.ret_slot[h];
  const bool ring = p.ring_rows > 0 && hr < 0;
  int phys = 0, seq_slot = 0;
  if (ring) {
    seq_slot = p.seq_slots[s];
    if ((unsigned)seq_slot >= (unsigned)p.max_seqs) return;
    if (lo >= p.ring_sink && hi <= p0 + p.n_tok - p.ring_mod) return;   // no row of this page is kept
  } else {
    phys = p.block_tables[(size_t)s * p.max_blocks + blk_l];
    if ((unsigned)phys >= (unsigned)p.num_blocks) return;
  }
  const int nrows = hi - lo, slot0 = lo - blk_l * BS;

  __shared__ float ks[BS][D], vs[BS][D];
  __shared__ float red[4];
  for (int e = tid; e < nrows * D; e += 256) {
    const int r = e / D, d = e % D;
    const size_t src = (((size_t)s * p.n_tok + (lo - p0 + r)) * p.Hkv + h) * D + d;
    ks[r][d] = bf16_to_f32(p.k[src]);
    vs[r][d] = bf16_to_f32(p.v[src]);
  }
  __syncthreads();

  if (hr >= 0) {
    const int r = tid >> 4, j = tid & 15;
    if (r < nrows) {
      const float* prow = p.proj + ((size_t)h * R + j) * D;
      const size_t o = (((size_t)phys * p.nR + hr) * BS + slot0 + r) * R + j;
      if (p.index_bf16) {           // P k in fp64, rounded once to bf16
        double acc = 0.0;
        for (int e = 0; e < D; ++e) acc = fma((double)prow[e], (double)ks[r][e], acc);
        reinterpret_cast<uint16_t*>(p.index_pool)[o] = f64_to_bf16_rne(acc);
      } else {
        float acc = 0.f;
        for (int e = 0; e < D; ++e) acc = fmaf(prow[e], ks[r][e], acc);
        reinterpret_cast<float*>(p.index_pool)[o] = acc;
      }
    }
  }
  __syncthreads();

  if (ROPE) {
    for (int e = tid; e < nrows * (D / 2); e += 256) {
      const int r = e / (D / 2), j = e % (D / 2);
      const double inv = pow((double)p.rope_theta, -2.0 * (double)j / (double)D);
      const double ang = (double)(lo + r) * inv;
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double x1 = ks[r][j], x2 = ks[r][j + D / 2];
      ks[r][j] = bf16_to_f32(f64_to_bf16_rne(x1 * cs - x2 * sn));
      ks[r][j + D / 2] = bf16_to_f32(f64_to_bf16_rne(x2 * cs + x1 * sn));
    }
    __syncthreads();
  }

  if (ring) {                       // bf16 rows, whatever the page type
    uint16_t* kp = reinterpret_cast<uint16_t*>(p.lk_pool);
    uint16_t* vp = reinterpret_cast<uint16_t*>(p.lv_pool);
    // positions below ring_sink, and the last ring_mod positions of the call
    const int keep_from = p0 + p.n_tok - p.ring_mod;
    const size_t ring0 = ((size_t)seq_slot * (p.Hkv - p.nR) + p.loc_slot[h]) * p.ring_rows;
    for (int e = tid; e < nrows * D; e += 256) {
      const int r = e / D, d = e % D, t = lo + r;
      if (t >= p.ring_sink && t < keep_from) continue;
      const int rr = ring_row(t, p.ring_sink, p.ring_mod);
      const size_t grow = ring0 + rr;
      kp[(grow >> 4) * (BS * D) + kpage_off(rr & 15, d)] = f32_to_bf16_rne(ks[r][d]);
      vp[grow * D + d] = f32_to_bf16_rne(vs[r][d]);
    }
    return;
  }

  const size_t row0 = ((size_t)phys * p.Hp + p.pool_slot[h]) * BS + slot0;
  const size_t page0 = ((size_t)phys * p.Hp + p.pool_slot[h]) * BS * D;      // K page (blocked layout)
  if (!FP8) {
    uint16_t* kp = reinterpret_cast<uint16_t*>(p.k_pool);
    uint16_t* vp = reinterpret_cast<uint16_t*>(p.v_pool);
    for (int e = tid; e < nrows * D; e += 256) {
      const int r = e / D, d = e % D;
      kp[page0 + kpage_off(slot0 + r, d)] = f32_to_bf16_rne(ks[r][d]);
      vp[(row0 + r) * D + d] = f32_to_bf16_rne(vs[r][d]);
    }
  } else {
    float* sc = p.kv_scales + ((size_t)phys * p.Hp + p.pool_slot[h]) * 2;
    float kscale, vscale;
    if (slot0 == 0) {
      float ka = 0.f, va = 0.f;
      for (int e = tid; e < nrows * D; e += 256) {
        ka = fmaxf(ka, fabsf(ks[e / D][e % D]));
        va = fmaxf(va, fabsf(vs[e / D][e % D]));
      }
      ka = block_max(ka, red);
      va = block_max(va, red);
      kscale = ka > 0.f ? ka / 448.0f : 1.0f;
      vscale = va > 0.f ? va / 448.0f : 1.0f;
      if (tid == 0) { sc[0] = kscale; sc[1] = vscale; }
    } else {
      kscale = sc[0];
      vscale = sc[1];
    }
    uint8_t* kp = reinterpret_cast<uint8_t*>(p.k_pool);
    uint8_t* vp = reinterpret_cast<uint8_t*>(p.v_pool);
    for (int e = tid; e < nrows * D; e += 256) {
      const int r = e / D, d = e % D;
      kp[page0 + kpage_off(slot0 + r, d)] = e4m3_encode(ks[r][d] / kscale);
      vp[(row0 + r) * D + d] = e4m3_encode(vs[r][d] / vscale);
    }
  }
}

hipError_t launch_append(const AppendParams& p, int kv_fp8, hipStream_t s) {
  const dim3 grid((p.n_tok + BS - 1) / BS + 1, p.Hkv, p.n_seq);
  const bool rope = p.rope_theta > 0.f;
  if (kv_fp8 && rope) hipLaunchKernelGGL((append_kernel<true, true>), grid, dim3(256), 0, s, p);
  else if (kv_fp8) hipLaunchKernelGGL((append_kernel<true, false>), grid, dim3(256), 0, s, p);
  else if (rope) hipLaunchKernelGGL((append_kernel<false, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((append_kernel<false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hws
