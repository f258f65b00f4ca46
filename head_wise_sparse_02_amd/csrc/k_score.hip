// Scoring scans of retrieval heads: one pass over every cached token.
//
// INDEX mode ([RTPurbo] "Full attention returns in force ...", Methodology §2:
// a 16-dim projection of the pre-RoPE query and key estimates relevance):
// s_{g,i} = (P_h q_g) . k~_i with k~_i = P_h k_i stored in the index pool,
// 64 bytes per token and head, streamed with one 16-byte load per lane.
//
// FULL mode ([ICS] "Inference-time context sparsity: illusion or
// opportunity?", §2 "Oracle Top-K"): s_{g,i} = q_g . k_i over all 128 dims,
// reading every K row once.  The G x 16-token x 128 tile is a dense bf16
// contraction, done with v_mfma_f32_16x16x32_bf16; e4m3 pages are widened to
// bf16 codes (exactly) and each 16-token page's products multiplied by its K
// scale.
//
// Both write the raw scores to [B][nR][Nmax][G] and, per workgroup chunk,
// the (max, sum) of 2^(c2 * s) for each query head, so that the selection
// pass can form the per-head log-sum-exp without another scan.
#include "hws_device.h"

namespace hws {

// Zero this chunk's share of the (b, hr) selection states (GS of them).
__device__ __forceinline__ void zero_state_share(const DecodeParams& p, SelState* st, int b, int hr, int c,
                                                 int nchunks) {
  // the chunks that exist share the work; chunk 0 also runs for an empty sequence
  const int nz = nchunks > 0 ? nchunks : 1;
  if (c >= nz) return;
  unsigned int* w = reinterpret_cast<unsigned int*>(st);
  const int words = SELSTATE_WORDS * p.GS;
  for (int i = c * 256 + (int)threadIdx.x; i < words; i += nz * 256) w[i] = 0u;
  // split arrival counters of the single-launch tail (and its error word)
  if (p.tail_sync != nullptr && c == 0 && hr == 0) {
    for (int h = threadIdx.x; h < p.Hkv; h += 256) p.tail_sync[1 + b * p.Hkv + h] = 0u;
    if (b == 0 && threadIdx.x == 0) p.tail_sync[0] = 0u;
  }
}

// Reduce (max, sum) over lanes sharing the same (lane & (span-1)) pattern.
__device__ __forceinline__ void wave_lse_reduce(float& m, float& s, int from_mask, int to_mask) {
  for (int off = from_mask; off <= to_mask; off <<= 1) {
    float m2 = __shfl_xor(m, off);
    float s2 = __shfl_xor(s, off);
    lse_combine(m, s, m2, s2);
  }
}

// ---------------------------------------------------------------------------
// INDEX mode.  A wave scores 256 consecutive tokens (16 pages) with coalesced
// 1 KiB loads: fp32 index (1 KiB per page): lane l holds token slot l/4 of
// the page and index dims 4*(l%4)..+3, a 2-step butterfly over the 4 lanes of
// a token leaves lane l with the score of query head g = l%4 (+4 for G = 8).
// bf16 index (512 B per page, two pages per load): lane l holds page l/32 of
// the pair, token slot (l%32)/2 and dims 8*(l%2)..+7; one butterfly step
// leaves lane l with query heads g = l%2, +2, +4, ...  The wave's page ids
// come in with one load and are read back wave-uniform, so no load waits on
// another; pages past the end read page 0 and are masked.
// ---------------------------------------------------------------------------
template <int G, bool BF16>
__global__ __launch_bounds__(256) void score_index_kernel(DecodeParams p) {
  constexpr int LPT = BF16 ? 2 : 4;                   // lanes per token
  constexpr int DPL = R / LPT;                        // index dims per lane
  constexpr int NOWN = (G + LPT - 1) / LPT;           // scores owned per lane per token
  constexpr int TPL = 64 / LPT;                       // tokens per wave load
  constexpr int NLD = 256 / TPL;                      // loads per wave: 16 (fp32) or 8 (bf16)
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nchunks = (N + SCORE_CHUNK - 1) / SCORE_CHUNK;  // == p.score_chunk here
  SelState* st = p.sel + ((size_t)b * p.nR + hr) * p.GS;
  zero_state_share(p, st, b, hr, c, nchunks);
  if (c >= nchunks) return;

  const int h = p.ret_head[hr];
  __shared__ float qt_s[G][R];
  __shared__ float red_m[4][G], red_s[4][G];

  const int tok0 = c * SCORE_CHUNK + wave * 256;
  const int page0 = tok0 >> 4;
  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const int my_blk = (lane < 16 && (page0 + lane) * BS < N) ? bt[page0 + lane] : -1;
  const int sub = lane % LPT;
  const int pin = BF16 ? (lane >> 5) : 0;             // page of the pair (bf16)
  const size_t page_elems = (size_t)BS * R;
  u32x4 kw[NLD];
  unsigned valid = 0u;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    // load i covers page i (fp32) or pages 2i, 2i+1 (bf16); every lane reads
    // both candidates wave-uniformly and picks its own
    const int pa = BF16 ? 2 * i : i;
    const int blk_a = __builtin_amdgcn_readlane(my_blk, pa);
    const int blk_b = BF16 ? __builtin_amdgcn_readlane(my_blk, pa + 1) : blk_a;
    const bool ok_a = (unsigned)blk_a < (unsigned)p.num_blocks;
    const bool ok_b = (unsigned)blk_b < (unsigned)p.num_blocks;
    valid |= (ok_a ? 1u : 0u) << (2 * i);
    valid |= (ok_b ? 1u : 0u) << (2 * i + 1);
    const int blk = pin ? (ok_b ? blk_b : 0) : (ok_a ? blk_a : 0);
    const char* pg = reinterpret_cast<const char*>(p.index_pool) +
                     (((size_t)blk * p.nR + hr) * page_elems) * (BF16 ? 2 : 4);
    kw[i] = load_nt16(pg + (BF16 ? (lane & 31) : lane) * 16);
  }
  // the projected queries q~ = P q, while the index loads are in flight:
  // each of the G*R dot products is split over 256/(G*R) neighbouring lanes
  {
    constexpr int TPD = 256 / (G * R);                // lanes per dot product: 16, 8, 4 or 2
    constexpr int EPT = D / TPD;                      // dims per lane: 8..64
    const int dot = tid / TPD, part = tid % TPD;
    const int g = dot / R, j = dot % R;
    const float4* prow = reinterpret_cast<const float4*>(p.proj + ((size_t)h * R + j) * D + part * EPT);
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
    if (part == 0) qt_s[g][j] = acc;
  }
  __syncthreads();                                    // qt_s ready
  float qv[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < DPL; ++j) qv[g][j] = qt_s[g][sub * DPL + j];

  float* out = p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G;
  float m[NOWN], s[NOWN];
#pragma unroll
  for (int k = 0; k < NOWN; ++k) { m[k] = NEG_INF; s[k] = 0.f; }
  const float c2 = p.c2_score;

#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int t = tok0 + i * TPL + (BF16 ? pin * BS + ((lane & 31) >> 1) : (lane >> 2));
    const bool ok = ((valid >> (BF16 ? 2 * i + pin : 2 * i)) & 1u) != 0u;
    float kx[DPL];
    if (BF16) {
      kx[0] = bf16_lo(kw[i].x); kx[1] = bf16_hi(kw[i].x); kx[2] = bf16_lo(kw[i].y); kx[3] = bf16_hi(kw[i].y);
      kx[4] = bf16_lo(kw[i].z); kx[5] = bf16_hi(kw[i].z); kx[6] = bf16_lo(kw[i].w); kx[DPL - 1] = bf16_hi(kw[i].w);
    } else {
      kx[0] = __uint_as_float(kw[i].x); kx[1] = __uint_as_float(kw[i].y);
      kx[2] = __uint_as_float(kw[i].z); kx[DPL - 1] = __uint_as_float(kw[i].w);
    }
    float part[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = qv[g][0] * kx[0];
#pragma unroll
      for (int j = 1; j < DPL; ++j) a = fmaf(qv[g][j], kx[j], a);
      a += __shfl_xor(a, 1);
      if (!BF16) a += __shfl_xor(a, 2);
      part[g] = ok ? a : 0.f;                          // an invalid page scores 0
    }
#pragma unroll
    for (int k = 0; k < NOWN; ++k) {
      const int g = sub + LPT * k;
      float v = part[0];
#pragma unroll
      for (int gg = 1; gg < G; ++gg) v = (g == gg) ? part[gg] : v;
      if (t < N && g < G) {
        out[(size_t)t * G + g] = v;
        const float x = v * c2;
        const float mn = fmaxf(m[k], x);
        s[k] = s[k] * fast_exp2(m[k] - mn) + fast_exp2(x - mn);
        m[k] = mn;
      }
    }
  }
  // lanes with equal (lane % LPT) hold the same query heads
#pragma unroll
  for (int k = 0; k < NOWN; ++k) {
    wave_lse_reduce(m[k], s[k], LPT, 32);
    const int g = sub + LPT * k;
    if (lane < LPT && g < G) { red_m[wave][g] = m[k]; red_s[wave][g] = s[k]; }
  }
  __syncthreads();
  if (tid < G) {
    float mm = red_m[0][tid], ss = red_s[0][tid];
    for (int w = 1; w < 4; ++w) lse_combine(mm, ss, red_m[w][tid], red_s[w][tid]);
    p.spart[((size_t)(b * p.nR + hr) * p.n_score_chunks + c) * G + tid] = make_float2(mm, ss);
  }
}

// ---------------------------------------------------------------------------
// FULL mode (MFMA).  A = query tile: row g < G holds q_g (bf16); with RoPE on
// rows G..2G-1 hold the bf16 residual q_g - bf16(q_g) of the rotated fp32
// query, so hi + lo carries ~16 mantissa bits.  B = 32 dims x 16 tokens of
// one page, read from the dim-blocked K page as one contiguous 1 KiB run per
// step with non-temporal loads.  Lane l supplies row/column l%16 and the 8 consecutive
// contraction elements 8*(l/16)..+7 of each 32-wide step; both operands use
// the same dim for the same (lane, element), so the product sums over all
// 128 dims.  C[row][col] sits in lane col + 16*(row/4), element row%4.
// ---------------------------------------------------------------------------
template <int G, bool SPLITQ, bool FP8>
__global__ __launch_bounds__(256) void score_full_kernel(DecodeParams p) {
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nchunks = (N + SCORE_CHUNK - 1) / SCORE_CHUNK;  // == p.score_chunk here
  SelState* st = p.sel + ((size_t)b * p.nR + hr) * p.GS;
  zero_state_share(p, st, b, hr, c, nchunks);
  if (c >= nchunks) return;

  const int h = p.ret_head[hr];
  const int row = lane & 15, quad = lane >> 4;
  __shared__ float red_m[4][MAX_G], red_s[4][MAX_G];

  // A operand (query tile), 4 contraction steps of 32 dims.
  bf16x8 afrag[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = mfma_dim0<FP8>(s, quad) + j;
      float v = 0.f;
      if (SPLITQ) {
        const int g = row < G ? row : row - G;
        if (row < 2 * G) {
          const float x = p.qrot[((size_t)b * p.Hq + h * G + g) * D + d];
          const float hi = bf16_to_f32(f32_to_bf16_rne(x));
          v = row < G ? hi : (x - hi);
        }
      } else if (row < G) {
        v = bf16_to_f32(p.q[((size_t)b * p.Hq + h * G + row) * D + d]);
      }
      afrag[s][j] = (__bf16)v;
    }
  }

  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  constexpr int ES = FP8 ? 1 : 2;                          // bytes per stored element
  float* out = p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G;
  const float c2 = p.c2_score;
  float m[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = NEG_INF; sm[i] = 0.f; }

  const int page0 = c * (SCORE_CHUNK / BS) + wave * 16;   // 16 pages per wave
  // pages in flight: e4m3 pages are held as raw codes (8 registers a page)
  // until their MFMAs, so twice as many fit
  constexpr int U = FP8 ? 8 : 4;
#pragma unroll 1
  for (int i0 = 0; i0 < 16; i0 += U) {
    bf16x8 bfrag[FP8 ? 1 : U][4];
    u32x4 raw[FP8 ? U : 1][2];
    int tpage[U];
    float ksc[U];                                          // FP8: the page's K scale
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pg = page0 + i0 + u;
      tpage[u] = pg * BS;
      ksc[u] = 1.f;
      int blk = -1;
      if (tpage[u] < N) blk = bt[pg];
      if ((unsigned)blk < (unsigned)p.num_blocks) {
        // blocked page: step s of all 16 rows is one contiguous run (1 KiB bf16, 512 B e4m3)
        const size_t page = (size_t)blk * p.Hp + p.pool_slot[h];
        if constexpr (FP8) {
          // e4m3 codes widened to bf16 (exact); the product is scaled after the MFMAs
          ksc[u] = p.kv_scales[page * 2];
          const char* src8 = kpool + page * (BS * D) + fp8_page_lane_off(row, quad);
          raw[FP8 ? u : 0][0] = load_nt16(src8);
          raw[FP8 ? u : 0][1] = load_nt16(src8 + 1024);
        } else {
          const char* src = kpool + (page * (BS * D) + row * 32 + 8 * quad) * ES;
#pragma unroll
          for (int s = 0; s < 4; ++s) bfrag[FP8 ? 0 : u][s] = __builtin_bit_cast(bf16x8, load_nt16(src + 2 * 512 * s));
        }
      } else if constexpr (FP8) {
        raw[FP8 ? u : 0][0] = (u32x4){0u, 0u, 0u, 0u};    // e4m3 code 0 is +0
        raw[FP8 ? u : 0][1] = (u32x4){0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) bfrag[FP8 ? 0 : u][s] = (bf16x8)(__bf16)0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tpage[u] >= N) continue;                         // wave-uniform
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 bk = FP8 ? fp8_step(raw[FP8 ? u : 0][s >> 1], s) : bfrag[FP8 ? 0 : u][s];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[s], bk, acc, 0, 0, 0);
      }
      // Fold the lo rows onto the hi rows and keep the G scores of token `row`.
      float v[4] = {acc[0], acc[1], acc[2], acc[3]};
      if (SPLITQ) {
        if (G == 1) { v[0] += v[1]; }
        else if (G == 2) { v[0] += v[2]; v[1] += v[3]; }
        else {
          const int off = 16 * (G / 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += __shfl_down(v[i], off);
        }
      }
      if (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= ksc[u];
      }
      // Lanes holding query heads: quad < G/4 (G >= 4) or quad 0 (G < 4).
      const bool owner = (G >= 4) ? (quad < G / 4) : (quad == 0);
      const int t = tpage[u] + row;
      if (owner && t < N) {
        float* dst = out + (size_t)t * G + ((G >= 4) ? 4 * quad : 0);
        if (G >= 4) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else if (G == 2) {
          *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
        } else {
          dst[0] = v[0];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < G) {
            const float x = v[i] * c2;
            const float mn = fmaxf(m[i], x);
            sm[i] = sm[i] * fast_exp2(m[i] - mn) + fast_exp2(x - mn);
            m[i] = mn;
          }
        }
      }
    }
  }
  // reduce over the 16 lanes of each quad (token columns)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wave_lse_reduce(m[i], sm[i], 1, 8);
    const int g = ((G >= 4) ? 4 * quad : 0) + i;
    const bool owner = (G >= 4) ? (quad < G / 4) : (quad == 0);
    if (row == 0 && owner && i < G && g < G) { red_m[wave][g] = m[i]; red_s[wave][g] = sm[i]; }
  }
  __syncthreads();
  if (tid < G) {
    float mm = red_m[0][tid], ss = red_s[0][tid];
    for (int w = 1; w < 4; ++w) lse_combine(mm, ss, red_m[w][tid], red_s[w][tid]);
    p.spart[((size_t)(b * p.nR + hr) * p.n_score_chunks + c) * G + tid] = make_float2(mm, ss);
  }
}

// FULL mode, G = 4 query heads per KV head, unrotated (exact bf16) queries.
// The query tile is replicated into all four 4-row groups of the 16-row A
// operand, and four pages are multiplied into four accumulators, so lane l
// (quad u = l/16) keeps accumulator u: the 4 scores of token l%16 of page u.
// Every lane then owns one token, and a wave's 64 tokens x 4 scores are one
// contiguous 1 KiB block.  The blocks are staged in LDS and the workgroup
// writes its CH x 16 bytes of scores in one burst after its last page:
// interleaving small writes with the K stream costs read bandwidth.
template <int CH, int GP, bool PF>
__global__ __launch_bounds__(256) void score_full_g4_kernel(DecodeParams p) {
  constexpr int G = 4;
  constexpr int PW = CH / BS / 4;                          // pages per wave
  static_assert(PW <= 64 && PW % GP == 0, "one page id per lane, whole groups");
  const int c = blockIdx.x, hr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
  const int N = min(p.seq_lens[b], p.Nmax);
  const int nchunks = (N + CH - 1) / CH;
  SelState* st = p.sel + ((size_t)b * p.nR + hr) * p.GS;
  zero_state_share(p, st, b, hr, c, nchunks);
  if (c >= nchunks) return;

  const int h = p.ret_head[hr];
  const int row = lane & 15, quad = lane >> 4;
  __shared__ float red_m[4][G], red_s[4][G];
  __shared__ f32x4 stage[CH];                              // this chunk's scores

  bf16x8 afrag[4];
  {
    const uint16_t* qg = p.q + ((size_t)b * p.Hq + h * G + (row & 3)) * D + 8 * quad;
#pragma unroll
    for (int s = 0; s < 4; ++s) afrag[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qg + 32 * s));
  }

  const int* bt = p.block_tables + (size_t)b * p.max_blocks;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const float c2 = p.c2_score;
  float m[4], sm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = NEG_INF; sm[i] = 0.f; }

  // page ids of this wave's pages, one per lane; read back wave-uniform with
  // readlane so that page addresses are scalar and no load waits on another
  const int page0 = c * (CH / BS) + wave * PW;
  const int my_blk = (lane < PW && (page0 + lane) * BS < N) ? bt[page0 + lane] : -1;
  const int npages = min(PW, max(0, (N - page0 * BS + BS - 1) / BS));
  const size_t page_stride = (size_t)p.Hp * (BS * D);
  const uint16_t* kbase = kpool + (size_t)p.pool_slot[h] * (BS * D) + (size_t)row * 32 + 8 * quad;

  // GP pages per step; invalid pages read page 0 and are zeroed after the MFMA
  bf16x8 cur[GP][4], nxt[GP][4];
  unsigned vcur = 0u, vnxt = 0u;
  auto load_group = [&](int pg, bf16x8 (&f)[GP][4], unsigned& valid) {
    valid = 0u;
#pragma unroll
    for (int u = 0; u < GP; ++u) {
      const int blk = __builtin_amdgcn_readlane(my_blk, pg + u);
      const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
      valid |= ok ? (1u << u) : 0u;
      const uint16_t* src = kbase + (size_t)(ok ? blk : 0) * page_stride;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) f[u][s2] = __builtin_bit_cast(bf16x8, load_nt16(src + 512 * s2));
    }
  };
  if (PF && npages > 0) load_group(0, cur, vcur);
  for (int pg = 0; pg < npages; pg += GP) {
    if (!PF) load_group(pg, cur, vcur);
    else if (pg + GP < npages) load_group(pg + GP, nxt, vnxt);
    // 4 pages per MFMA group: lane quad u keeps page u's accumulator
#pragma unroll
    for (int u0 = 0; u0 < GP; u0 += 4) {
      f32x4 acc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (u0 + u < GP) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[s2], cur[u0 + u < GP ? u0 + u : 0][s2], acc[u], 0, 0, 0);
          if (!((vcur >> (u0 + u)) & 1u)) acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      }
      // GP < 4: quads beyond GP hold no page this step
      const int npg_here = GP < 4 ? GP : 4;
      if (quad < npg_here) {
        f32x4 v = acc[0];
        v = quad == 1 ? acc[1] : v;
        v = quad == 2 ? acc[2] : v;
        v = quad == 3 ? acc[3] : v;
        stage[(wave * PW + pg + u0) * BS + lane] = v;
        const int t = (page0 + pg + u0) * BS + lane;     // token of this lane
        if (t < N) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = v[i] * c2;
            const float mn = fmaxf(m[i], x);
            sm[i] = sm[i] * fast_exp2(m[i] - mn) + fast_exp2(x - mn);
            m[i] = mn;
          }
        }
      }
    }
    if (PF) {
#pragma unroll
      for (int u = 0; u < GP; ++u)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) cur[u][s2] = nxt[u][s2];
      vcur = vnxt;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wave_lse_reduce(m[i], sm[i], 1, 32);
    if (lane == 0) { red_m[wave][i] = m[i]; red_s[wave][i] = sm[i]; }
  }
  __syncthreads();
  float* out = p.scores + ((size_t)(b * p.nR + hr) * p.Nmax) * G;
  const int t0 = c * CH;
#pragma unroll
  for (int k = 0; k < CH / 256; ++k) {
    const int e = k * 256 + tid;
    if (t0 + e < N) __builtin_nontemporal_store(stage[e], reinterpret_cast<f32x4*>(out + (size_t)(t0 + e) * G));
  }
  if (tid < G) {
    float mm = red_m[0][tid], ss = red_s[0][tid];
    for (int w = 1; w < 4; ++w) lse_combine(mm, ss, red_m[w][tid], red_s[w][tid]);
    p.spart[((size_t)(b * p.nR + hr) * p.n_score_chunks + c) * G + tid] = make_float2(mm, ss);
  }
}

constexpr int G4_GP = 1;          // pages per load step of the G=4 scan
constexpr bool G4_PF = true;      // issue the next step's loads before this step's MFMAs

template <int G>
static hipError_t launch_score_g(const DecodeParams& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.n_score_chunks, p.nR, p.B), blk(256);
  if (p.score_mode == 0) {
    if (p.index_bf16) return launch_kernel(score_index_kernel<G, true>, grid, blk, st, e0, e1, p);
    return launch_kernel(score_index_kernel<G, false>, grid, blk, st, e0, e1, p);
  }
  if (p.kv_scales != nullptr) {                  // fp8 cache
    if (p.qrot != nullptr) return launch_kernel(score_full_kernel<G, true, true>, grid, blk, st, e0, e1, p);
    return launch_kernel(score_full_kernel<G, false, true>, grid, blk, st, e0, e1, p);
  }
  if (p.qrot != nullptr) return launch_kernel(score_full_kernel<G, true, false>, grid, blk, st, e0, e1, p);
  if (G == 4) return launch_kernel(score_full_g4_kernel<G4_SCORE_CHUNK, G4_GP, G4_PF>, grid, blk, st, e0, e1, p);
  return launch_kernel(score_full_kernel<G, false, false>, grid, blk, st, e0, e1, p);
}

hipError_t launch_score(const DecodeParams& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (p.G) {
    case 1: return launch_score_g<1>(p, st, e0, e1);
    case 2: return launch_score_g<2>(p, st, e0, e1);
    case 4: return launch_score_g<4>(p, st, e0, e1);
    case 8: return launch_score_g<8>(p, st, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace hws
