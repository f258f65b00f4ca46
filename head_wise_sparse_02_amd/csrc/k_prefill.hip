// Head-wise chunked prefill attention on the paged cache.
//
// [RTPurbo] Methodology §1: during prefill a retrieval head keeps its whole
// cache (causal attention over every earlier position) while a local head
// attends to its sinks and its sliding window; the prefill speed-up of the
// method comes from the local heads ([RTPurbo] Results; [AoH] Results).
// Query position i of a local head sees keys 0..n_sink-1 and i-window+1..i.
//
// One workgroup per (sequence, KV head, tile of 128 query rows), a query row
// being one (position, query head of the group) pair, so the G query heads of
// a KV head share every K/V tile.  Key tiles of 64 keys (4 pages) go through
// LDS, double-buffered: K in its page-blocked layout with the 16-byte chunks
// of each row swizzled, V row-major (read back transposed by the gfx950
// transposing LDS read); each tile's loads are issued two tiles ahead, so
// they are in flight during two tiles' products.  Each wave owns 32 query
// rows and computes
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims from LDS,
//                  B = the wave's queries, kept in registers)
//   O^T += V^T P^T (v_mfma_f32_16x16x32_f16: A = 16 dims x 32 keys of V^T,
//                  B = P, both fp16),
// with the online softmax in log2 units between the two.  The S^T layout
// leaves each lane with 4 keys of one query per 16-key block, which is the
// B-operand shape of P^T once both operands enumerate the 32 keys of a step
// in the same (permuted) order.  A retrieval head walks key tiles 0..last;
// a local head walks its sink tile(s) and the tiles its window touches.
// Masks are evaluated only on tiles that cross a boundary.  With a local
// ring, a local head's tiles come from its ring slot instead of the pages:
// every 16 positions from a multiple of 16 sit in one ring page.
//
// With RoPE on, queries are rotated in fp64 at their position and split as
// q = hi + lo (two bf16 parts), so S keeps fp32-level accuracy.  The P V
// product runs in fp16: V enters LDS as fp16 (exact for bf16 values of
// magnitude 2^-14 .. 65504; smaller ones keep an absolute error below
// 2^-25), and the softmax weights P in (0, 1] are rounded once to fp16
// (2^-11 relative, where bf16 would give 2^-9 and move outputs by up to a few
// 1e-3), with fp32 accumulation.
//
// FP8 pages: the e4m3 K codes are widened to bf16 on their way into LDS
// (exact: every e4m3 value is a bf16 value), so S holds the products on the
// codes and each 16-key block of S is multiplied by its page's K scale
// (which enters the exponent: exp2(s * c2 * ks - m) for raw product s and
// the running max m); the V codes enter LDS already multiplied by their
// page's V scale, as fp16.
#include "mfma_tile.h"

namespace hws {

namespace {

// Waves per workgroup, 32 query rows each (8 waves sharing each tile measured
// no faster: the loop is bound by its softmax and LDS reads, not by the tile
// loads it shares).
template <bool ROPE> struct PfShape {
  static constexpr int WAVES = 4;
  static constexpr int QB = 2;                   // 16-row query blocks per wave
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 16 * QB * WAVES;
};
constexpr int PF_KT = 64;         // keys per tile

struct alignas(16) PfLds {        // 16-byte aligned: the tile moves as 16-byte LDS accesses
  uint16_t k[2][4 * BS * D];      // 4 pages, page-blocked layout (16 KiB each)
  uint16_t v[2][PF_KT * V_STRIDE]; // V [key][dim], rows padded (18 KiB each)
  float sc[2][8];                 // FP8: K scales of the 4 pages, then V scales
};

template <int G, bool ROPE, bool FP8>
__global__ __launch_bounds__(PfShape<ROPE>::THREADS, ROPE ? 1 : 2) void prefill_kernel(PrefillParams p) {
  constexpr int PF_THREADS = PfShape<ROPE>::THREADS;
  constexpr int QP = PfShape<ROPE>::ROWS / G;      // query positions per tile
  constexpr int QB = PfShape<ROPE>::QB;
  __shared__ PfLds S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;

  // work item -> (sequence, KV head, query tile); retrieval items first and
  // the tiles with the most keys first
  int item = blockIdx.x + p.item0;
  const int nret = p.n_seq * p.nR * p.ntq;
  bool ret;
  int s, h, qt, lh = 0;                            // lh: local head number
  if (item < nret) {
    ret = true;
    const int per = p.n_seq * p.nR;
    qt = p.ntq - 1 - item / per;
    const int rem = item % per;
    s = rem / p.nR;
    h = p.ret_head[rem % p.nR];
  } else {
    item -= nret;
    ret = false;
    const int per = p.n_seq * p.nL;
    qt = p.ntq - 1 - item / per;
    const int rem = item % per;
    s = rem / p.nL;
    lh = rem % p.nL;
    h = p.loc_head[lh];
  }
  const int start = p.start_pos[s];
  if (start < 0) return;
  const int t0l = qt * QP;                         // first position of the tile within the chunk
  const int nq = min(QP, p.n_tok - t0l);
  const int t0 = start + t0l, tl = t0 + nq - 1;    // first / last query position

  // key tiles: [0, ns_t) sink tiles, then [lo_t, last_t]
  const int last_t = tl / PF_KT;
  int ns_t = 0, lo_t = 0;
  if (!ret) {
    ns_t = p.n_sink > 0 ? min((p.n_sink - 1) / PF_KT + 1, last_t + 1) : 0;
    lo_t = max(ns_t, max(0, t0 - p.window + 1) / PF_KT);
  }
  // a local head with a ring reads its rows from the sequence's ring slot
  // (positions below ring_sink in their own rows, later ones modulo
  // ring_mod); a slot out of range reads nothing (output 0, lse -inf)
  const bool ring = !ret && p.ring_rows > 0;
  const int rslot = ring ? p.seq_slots[s] : 0;
  const bool slot_ok = !ring || (unsigned)rslot < (unsigned)p.max_seqs;
  const int n_tiles = slot_ok ? ns_t + max(0, last_t - lo_t + 1) : 0;

  // queries of this wave: rows 32*wave + 16*qb + col = (position, head) pairs
  int qpos[QB];
  bool qok[QB];
  bf16x8 qf[QB][4], ql[ROPE ? QB : 1][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = 16 * (QB * wave + qb) + col;
    const int pl = r / G, g = r % G;
    qok[qb] = pl < nq;
    qpos[qb] = t0 + pl;
    const uint16_t* qrow = p.q + (((size_t)s * p.n_tok + t0l + (qok[qb] ? pl : 0)) * p.Hq + h * G + g) * D;
    if (!ROPE) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
        qf[qb][st] = qok[qb] ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * st + 8 * quad))
                             : zero8();
    } else {
      // dims 32*st + 8*quad + e (st = 0, 1) pair with the same dims + 64 (st + 2)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + 32 * st + 8 * quad);
        const u32x4 b = *reinterpret_cast<const u32x4*>(qrow + 32 * (st + 2) + 8 * quad);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double x1 = (e & 1) ? bf16_hi(a[e >> 1]) : bf16_lo(a[e >> 1]);
          const double x2 = (e & 1) ? bf16_hi(b[e >> 1]) : bf16_lo(b[e >> 1]);
          const int j = 32 * st + 8 * quad + e;
          const double inv = pow((double)p.rope_theta, -2.0 * (double)j / (double)D);
          double sn, cs;
          sincos((double)qpos[qb] * inv, &sn, &cs);
          const double r1 = qok[qb] ? x1 * cs - x2 * sn : 0.0;
          const double r2 = qok[qb] ? x2 * cs + x1 * sn : 0.0;
          const float h1 = bf16_to_f32(f64_to_bf16_rne(r1)), h2 = bf16_to_f32(f64_to_bf16_rne(r2));
          qf[qb][st][e] = (__bf16)h1;
          qf[qb][st + 2][e] = (__bf16)h2;
          ql[ROPE ? qb : 0][st][e] = (__bf16)bf16_to_f32(f64_to_bf16_rne(r1 - (double)h1));
          ql[ROPE ? qb : 0][st + 2][e] = (__bf16)bf16_to_f32(f64_to_bf16_rne(r2 - (double)h2));
        }
      }
    }
  }

  const int* bt = p.block_tables + (size_t)s * p.max_blocks;
  typedef typename KvChunk<FP8>::T Chunk;
  constexpr int ES = FP8 ? 1 : 2;                  // bytes per stored element
  const char* kpool = reinterpret_cast<const char*>(ring ? p.lk_pool : p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(ring ? p.lv_pool : p.v_pool);
  const int hslot = ring ? 0 : p.pool_slot[h];
  const int hp = ring ? 1 : p.Hp;                  // heads per page of the pool read
  const size_t rbase = ring ? ((size_t)(slot_ok ? rslot : 0) * p.nL + lh) * (size_t)(p.ring_rows / BS) : 0;
  const float* scales = FP8 ? p.kv_scales + 2 * hslot : nullptr;   // (K, V) scale of page 0 of this head
  // Tile loaders: a tile is 4 pages x 256 16-byte chunks of K and 64 keys x
  // 16 chunks of 8 dims of V.  Each thread moves KC chunks of each (chunk
  // tid + PF_THREADS * u: page c / 256; for V key c / 16, dims 8 (c % 16)).
  constexpr int KC = 1024 / PF_THREADS;
  // K in LDS: the 16-byte chunk q of row r (of a 32-dim block) is stored at
  // chunk q ^ ((r >> 1) & 3), so the 8 lanes of an A-operand read (rows 0..7,
  // one chunk) fall in 8 different bank groups
  const int kcp = tid & 255;                       // chunk within its page
  const int kw_row = (kcp >> 2) & 15;
  const int kw_off = (kcp >> 6) * 512 + kw_row * 32 + 8 * ((kcp & 3) ^ ((kw_row >> 1) & 3));
  const int kr_off = col * 32 + 8 * (quad ^ ((col >> 1) & 3));

  // global -> registers -> LDS for key tile kt.  Page ids are fetched one
  // tile ahead (scalar loads, unconditional so none waits behind a branch);
  // entries past the last query's page read page 0.  The registers are not
  // touched until the tile is stored after the compute of the current tile,
  // so the loads overlap it; V rows of keys past the last query are zeroed
  // there, so stale slots never reach P V.  FP8: the page scales travel with
  // the tile (1 for entries past the last query's page, whose keys are all
  // masked, so that no unwritten scale reaches the softmax).
  Chunk kA[KC], vA[KC], kB[KC], vB[KC];        // two tiles in flight
  float scA[FP8 ? 8 : 1], scB[FP8 ? 8 : 1];
  const int lp_max = min(p.max_blocks - 1, tl / BS);
  int live = 0;                                // FP8: bit u set if page u of the tile is before lp_max
  auto tile_pages = [&](int kt, int (&ids)[4]) {
    live = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int lp = kt * 4 + u;
      if (ring) {                                  // wave-uniform
        const int pos = lp * BS;
        const int rp = pos < p.ring_sink ? lp
                     : (p.ring_mod > 0 ? (p.ring_sink + pos % p.ring_mod) / BS : 0);
        ids[u] = (int)rbase + (lp <= lp_max ? rp : 0);
      } else {
        const int blk = bt[min(lp, lp_max)];
        ids[u] = ((lp <= lp_max) & ((unsigned)blk < (unsigned)p.num_blocks)) ? blk : 0;
      }
      live |= (lp <= lp_max) << u;
    }
  };
  auto pick = [](const int (&ids)[4], int i) { return i == 0 ? ids[0] : (i == 1 ? ids[1] : (i == 2 ? ids[2] : ids[3])); };
  auto load_tile = [&](const int (&ids)[4], Chunk (&kreg)[KC], Chunk (&vreg)[KC], float (&sc)[FP8 ? 8 : 1]) {
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int c = tid + PF_THREADS * u;
      const size_t page = (size_t)pick(ids, c >> 8) * hp + hslot;   // wave-uniform
      kreg[u] = *reinterpret_cast<const Chunk*>(kpool + (page * (BS * D) + kcp * 8) * ES);
      vreg[u] = *reinterpret_cast<const Chunk*>(vpool + ((page * BS + ((c >> 4) & 15)) * D + 8 * (c & 15)) * ES);
    }
    if constexpr (FP8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x2 s2 = *reinterpret_cast<const f32x2*>(scales + (size_t)ids[u] * (2 * hp));
        sc[u] = (live >> u) & 1 ? s2.x : 1.f;
        sc[4 + u] = (live >> u) & 1 ? s2.y : 1.f;
      }
    }
  };
  auto store_tile = [&](int buf, int kt, Chunk (&kreg)[KC], Chunk (&vreg)[KC], float (&sc)[FP8 ? 8 : 1]) {
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int c = tid + PF_THREADS * u;
      *reinterpret_cast<u32x4*>(&S.k[buf][(c >> 8) * (BS * D) + kw_off]) = chunk_bf16(kreg[u]);
      const int key = c >> 4;
      // V as fp16 (fp8: the code times its page's V scale); keys past the
      // chunk's last position as +0
      *reinterpret_cast<u32x4*>(&S.v[buf][key * V_STRIDE + 8 * (c & 15)]) =
          chunk_v_f16(kt * PF_KT + key <= tl ? vreg[u] : Chunk{}, FP8 ? sc[4 + (key >> 4)] : 1.f);
    }
    if constexpr (FP8) {
      if (tid == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) S.sc[buf][i] = sc[i];
      }
    }
  };

  float m[QB], lsum[QB];
  f32x4 o[8][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = NEG_INF; lsum[qb] = 0.f; }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c2 = p.c2;

  auto tile_at = [&](int it) { return it < ns_t ? it : lo_t + (it - ns_t); };
  // compute on tile kt in LDS buffer buf
  auto compute = [&](int buf, int kt) {
    // S^T = K Q^T for the 4 key blocks x 2 query blocks of this wave
    f32x4 sacc[4][QB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&S.k[buf][kb * (BS * D) + st * 512 + kr_off]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sacc[kb][qb] = mfma(a, qf[qb][st], sacc[kb][qb]);
          if (ROPE) sacc[kb][qb] = mfma(a, ql[ROPE ? qb : 0][st], sacc[kb][qb]);
        }
      }
    }

    // FP8: per 16-key page, c2 times its K scale, log2 of its V scale and the
    // reciprocal of that scale (the scales are positive)
    float ksc[4], c2k[4];
    if constexpr (FP8) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(&S.sc[buf][0]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        ksc[kb] = kv[kb];
        c2k[kb] = p.c2 * kv[kb];
      }
    }

    // masks, only where the tile crosses the causal edge, the window's lower
    // edge or the end of the sinks
    const int key0 = kt * PF_KT;
    const bool inside = key0 + PF_KT - 1 <= t0 &&
                        (ret || key0 + PF_KT - 1 < p.n_sink || key0 > tl - p.window);
    f16x8 ph[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // (rows past the chunk's end hold zero queries: finite, and never written)
      if (!inside) {                                   // wave-uniform
        const int rel = qpos[qb] - key0 - 4 * quad;    // key offset 16*kb + i is causal iff <= rel
        const int wlo = rel - p.window;                // ... and in the window iff > wlo
        const int slim = ret ? 0x7FFFFFFF : p.n_sink - key0 - 4 * quad;   // ... or a sink iff < slim
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jo = 16 * kb + i;
            const bool ok = (jo <= rel) & ((jo > wlo) | (jo < slim) | ret);
            sacc[kb][qb][i] = ok ? sacc[kb][qb][i] : NEG_INF;
          }
      }
      float mx = NEG_INF;
      if constexpr (FP8) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float mk = sacc[kb][qb][0];
#pragma unroll
          for (int i = 1; i < 4; ++i) mk = fmaxf(mk, sacc[kb][qb][i]);
          mx = fmaxf(mx, mk * ksc[kb]);
        }
      } else {
        mx = sacc[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
      }
      mx = max_x16_x32(mx);
      const float m_new = fmaxf(m[qb], mx * c2);
      const float m_use = m_new == NEG_INF ? 0.f : m_new;
      const float alpha = fast_exp2(m[qb] - m_use);
      m[qb] = m_new;
      float ps = 0.f;
      float pv[4][4];
      if constexpr (FP8) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[kb][i] = fast_exp2(fmaf(sacc[kb][qb][i], c2k[kb], -m_use));
            ps += pv[kb][i];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[kb][i] = fast_exp2(fmaf(sacc[kb][qb][i], c2, -m_use));
            ps += pv[kb][i];
          }
      }
      lsum[qb] = lsum[qb] * alpha + ps;
      if (__any(alpha != 1.f)) {                       // rescale only when a max moved
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[qb][ks][i] = (_Float16)pv[2 * ks][i];
          ph[qb][ks][4 + i] = (_Float16)pv[2 * ks + 1][i];
        }
    }

    // O^T += V^T P^T, each V^T fragment read one step ahead of its products
    // (the LDS read then overlaps the previous step's MFMAs: -3.5 %)
    f16x8 a_cur = vt_frag(S.v[buf], 0, 0, col, quad);
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int db = step >> 1, ks = step & 1;
      f16x8 a_next = a_cur;
      if (step + 1 < 16) a_next = vt_frag(S.v[buf], (step + 1) & 1, (step + 1) >> 1, col, quad);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma(a_cur, ph[qb][ks], o[db][qb]);
      a_cur = a_next;
    }

  };

  // Tile t is loaded into register set t % 2 two tiles ahead of its use and
  // stored to LDS buffer t % 2 after the compute of tile t - 1, so each load
  // has the compute of two tiles to arrive.
  int ids[4];
  if (n_tiles > 0) {
    tile_pages(tile_at(0), ids);
    load_tile(ids, kA, vA, scA);
    store_tile(0, tile_at(0), kA, vA, scA);
  }
  if (n_tiles > 1) { tile_pages(tile_at(1), ids); load_tile(ids, kB, vB, scB); }
  if (n_tiles > 2) { tile_pages(tile_at(2), ids); load_tile(ids, kA, vA, scA); }
  if (n_tiles > 3) tile_pages(tile_at(3), ids);
  __syncthreads();
  for (int it = 0; it < n_tiles; it += 2) {
    compute(0, tile_at(it));                          // even tile in buffer 0
    if (it + 1 < n_tiles) store_tile(1, tile_at(it + 1), kB, vB, scB);
    if (it + 3 < n_tiles) {
      load_tile(ids, kB, vB, scB);                    // tile it + 3
      if (it + 4 < n_tiles) tile_pages(tile_at(it + 4), ids);
    }
    __syncthreads();
    if (it + 1 >= n_tiles) break;
    compute(1, tile_at(it + 1));                      // odd tile in buffer 1
    if (it + 2 < n_tiles) store_tile(0, tile_at(it + 2), kA, vA, scA);
    if (it + 4 < n_tiles) {
      load_tile(ids, kA, vA, scA);                    // tile it + 4
      if (it + 5 < n_tiles) tile_pages(tile_at(it + 5), ids);
    }
    __syncthreads();
  }

  // normalise and write: lane holds dims 16*db + 4*quad + i of its query row
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_x16_x32(lsum[qb]);
    if (!qok[qb]) continue;
    const int r = 16 * (QB * wave + qb) + col;
    const int pl = r / G, g = r % G;
    const size_t orow = ((size_t)s * p.n_tok + t0l + pl) * p.Hq + h * G + g;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = o[db][qb] * inv;
      *reinterpret_cast<float4*>(p.out + orow * D + 16 * db + 4 * quad) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (quad == 0 && p.lse != nullptr) p.lse[orow] = (m[qb] + log2f(l)) * LN2;
  }
}

template <int G, bool FP8>
hipError_t launch_gf(const PrefillParams& p, int nwg, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.rope_theta > 0.f)
    return launch_kernel(prefill_kernel<G, true, FP8>, dim3(nwg), dim3(PfShape<true>::THREADS), s, e0, e1, p);
  return launch_kernel(prefill_kernel<G, false, FP8>, dim3(nwg), dim3(PfShape<false>::THREADS), s, e0, e1, p);
}

// All work items in one launch; with fp8 pages and a ring, the retrieval
// items (fp8 pages) and the local items (bf16 ring rows) in two launches,
// timed from the first one's start to the second one's end.
template <int G>
hipError_t launch_g(const PrefillParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const long long nret = (long long)p.n_seq * p.nR * p.ntq;
  const long long nall = (long long)p.n_seq * (p.nR + p.nL) * p.ntq;
  if (p.kv_scales == nullptr) return launch_gf<G, false>(p, (int)nall, s, e0, e1);
  if (p.ring_rows == 0 || nret == nall) return launch_gf<G, true>(p, (int)nall, s, e0, e1);
  hipError_t e = hipSuccess;
  if (nret > 0 && (e = launch_gf<G, true>(p, (int)nret, s, e0, nullptr)) != hipSuccess) return e;
  PrefillParams q = p;
  q.item0 = (int)nret;
  return launch_gf<G, false>(q, (int)(nall - nret), s, nret > 0 ? nullptr : e0, e1);
}

}  // namespace

int prefill_rows_per_tile(bool rope) { return rope ? PfShape<true>::ROWS : PfShape<false>::ROWS; }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const long long nwg = (long long)p.n_seq * (p.nR + p.nL) * p.ntq;
  if (nwg <= 0) return hipSuccess;
  switch (p.G) {
    case 1: return launch_g<1>(p, s, e0, e1);
    case 2: return launch_g<2>(p, s, e0, e1);
    case 4: return launch_g<4>(p, s, e0, e1);
    default: return launch_g<8>(p, s, e0, e1);
  }
}

}  // namespace hws
