// Host side of libhws: the C ABI declared in include/hws.h.
//
// Validation runs before any HIP call, so every error status can be produced
// without a GPU.  Device work is only kernel launches on the caller's stream;
// nothing here allocates device memory or synchronises (except
// hws_profile_read, which waits for its own timing events).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "hws.h"
#include "hws_internal.h"

using namespace hws;

static_assert(PHASES == HWS_PHASES, "phase count of the profiling hook");

namespace {

constexpr int NUM_STAGES = 9;
const char* const STAGE_NAMES[NUM_STAGES] = {"score", "select", "attend", "merge", "tail", "fused", "prefill",
                                             "fused_index", "attend_balanced"};

struct EvPair {
  hipEvent_t a, b;
  int stage;
};

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions of one decode call.
struct Layout {
  size_t scores, agg, spart, sel, apart_ml, apart_o, qrot, tail_sync, tail_ties, total;
  size_t row_list, tile_cnt, item_base, bal_ml, bal_o;   // attention balanced by kept rows
  int Nagg;
  int score_chunk, n_score_chunks, n_sel_chunks, ncR, ncL, att_chunk_R, max_splits;
  int tail_tph, tail_ntiles;
};

}  // namespace

struct hws_ctx {
  hws_config cfg;
  int G = 1;
  uint8_t kinds[MAX_KV] = {};
  int nR = 0, nL = 0;
  signed char ret_slot[MAX_KV];
  signed char ret_head[MAX_KV];
  signed char loc_head[MAX_KV];
  signed char pool_slot[MAX_KV];   // head -> index within a page (-1: local head in the ring)
  signed char loc_slot[MAX_KV];    // head -> local head number (-1: retrieval head)
  int Hp = 0;                      // heads per page
  int ring_rows = 0;               // local ring rows per (slot, local head); 0 = no ring
  int ring_sink = 0, ring_mod = 0; // ring geometry: first positions, then positions modulo ring_mod
  bool appended = false, bound = false;
  hws_buffers buf{};
  std::string err;
  int launch_mode = HWS_LAUNCH_AUTO;
  unsigned int spin_limit = 1u << 20;  // polls per hand-off wait (~1 us each)
  unsigned int wait_bias = 0;
  bool prof = false;
  uint64_t* phase_t = nullptr;     // phase timestamps of the single launches (profiling aid)
  int phase_wgs = 0;
  std::vector<EvPair> recorded;
  std::vector<hipEvent_t> pool;
};

namespace {

hws_status fail(hws_ctx* ctx, hws_status st, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
hws_status fail(hws_ctx* ctx, hws_status st, const char* fmt, ...) {
  if (ctx != nullptr) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof(msg), fmt, ap);
    va_end(ap);
    ctx->err = msg;
  }
  return st;
}

hws_status hip_fail(hws_ctx* ctx, hipError_t e, const char* what) {
  return fail(ctx, HWS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Head numbering: retrieval and local heads in KV-head order; with a local
// ring the pages hold only the retrieval heads.
void rebuild_slots(hws_ctx* c) {
  c->nR = c->nL = 0;
  for (int h = 0; h < MAX_KV; ++h) {
    c->ret_slot[h] = c->ret_head[h] = c->loc_head[h] = c->pool_slot[h] = c->loc_slot[h] = -1;
  }
  for (int h = 0; h < c->cfg.num_kv_heads; ++h) {
    if (c->kinds[h] == HWS_HEAD_RETRIEVAL) {
      c->ret_slot[h] = (signed char)c->nR;
      c->ret_head[c->nR++] = (signed char)h;
    } else {
      c->loc_slot[h] = (signed char)c->nL;
      c->loc_head[c->nL++] = (signed char)h;
    }
  }
  const bool ring = c->cfg.local_ring != 0;
  c->Hp = ring ? c->nR : c->cfg.num_kv_heads;
  for (int h = 0; h < c->cfg.num_kv_heads; ++h) c->pool_slot[h] = ring ? c->ret_slot[h] : (signed char)h;
  // positions below ring_sink (the sinks, rounded up to a 64-key tile) keep
  // their own rows; later positions cycle through ring_mod rows (window +
  // slack, rounded up to a page)
  c->ring_sink = ring ? (c->cfg.n_sink + 63) / 64 * 64 : 0;
  c->ring_mod = ring ? (int)(((long long)c->cfg.window + c->cfg.ring_slack + BS - 1) / BS * BS) : 0;
  c->ring_rows = ring ? c->ring_sink + c->ring_mod : 0;
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Longest context for which AUTO prefers the single launch after the scan.
constexpr int AUTO_TAIL_MAX_LEN = 4096;

// GS: selection states per retrieval head (1, or G with one set per query head).
Layout make_layout(const hws_ctx* c, int B, int Nmax, bool rope, int score_mode, int GS) {
  Layout L{};
  const int G = c->G;
  // The G=4 full-dim scan (bf16 queries, RoPE off) uses longer chunks.
  L.score_chunk = (score_mode == HWS_SCORE_FULL && G == 4 && !rope && c->cfg.kv_dtype == HWS_KV_BF16)
                      ? G4_SCORE_CHUNK : SCORE_CHUNK;
  L.n_score_chunks = cdiv(Nmax, L.score_chunk);
  L.n_sel_chunks = cdiv(Nmax, SEL_CHUNK);
  // Retrieval attention chunk: long enough that the split partials stay small
  // next to the gathered rows, short enough that the chunks of the whole batch
  // give about two workgroups per compute unit (a few sequences and heads at a
  // long context would otherwise leave most of the chip idle).
  {
    const long long units = (long long)B * std::max(c->nR, 1) * Nmax;
    int chunk = 1024;
    while (chunk < 4096 && units / (2 * chunk) >= 2 * 256) chunk *= 2;
    L.att_chunk_R = chunk;
  }
  L.ncR = cdiv(Nmax, L.att_chunk_R);
  const long long local_rows = std::min<long long>(Nmax, (long long)c->cfg.n_sink + c->cfg.window);
  L.ncL = std::max(1, cdiv(local_rows, LOCAL_CHUNK));
  // (the single launch with the index scan inside has one split per tile, of
  // at least FI_TILE_MIN positions)
  L.max_splits = std::max(c->nR > 0 ? std::max(L.ncR, cdiv(Nmax, FI_TILE_MIN)) : 1, c->nL > 0 ? L.ncL : 1);
  const size_t nRb = (size_t)B * c->nR;
  size_t off = 0;
  L.scores = off;   off = align_up(off + nRb * Nmax * G * sizeof(float));
  L.Nagg = (Nmax + 63) & ~63;
  L.agg = off;      off = align_up(off + nRb * GS * L.Nagg * sizeof(float));
  L.spart = off;    off = align_up(off + nRb * L.n_score_chunks * G * sizeof(float2));
  L.sel = off;      off = align_up(off + nRb * GS * sizeof(SelState));
  const size_t nsp = (size_t)B * c->cfg.num_kv_heads * L.max_splits * G;
  L.apart_ml = off; off = align_up(off + nsp * sizeof(float2));
  L.apart_o = off;  off = align_up(off + nsp * D * sizeof(float));
  L.qrot = off;     off = align_up(off + (rope ? (size_t)B * c->cfg.num_q_heads * D * sizeof(float) : 0));
  // single-launch tail: tiles of TAIL_TILE positions per retrieval head
  L.tail_tph = cdiv(Nmax, TAIL_TILE);
  L.tail_ntiles = (int)(nRb * L.tail_tph);
  L.tail_sync = off; off = align_up(off + (1 + (size_t)B * c->cfg.num_kv_heads) * sizeof(unsigned int));
  // tie counts per tile: for the smallest tiles any single launch uses
  L.tail_ties = off; off = align_up(off + nRb * cdiv(Nmax, FI_TILE_MIN) * sizeof(unsigned int));
  // attention balanced by kept rows (index scores, one set per KV head)
  if (score_mode == HWS_SCORE_INDEX && GS == 1) {
    // pieces: at most one per workgroup, min(BAL_ITEMS, cost units / BAL_RMIN),
    // plus one per pair
    const size_t npairs = (size_t)B * c->cfg.num_kv_heads;
    const size_t nitems = std::min<size_t>(BAL_ITEMS, (npairs * ((size_t)Nmax + BAL_PIECE_COST) + BAL_RMIN - 1) / BAL_RMIN) + npairs;
    L.row_list = off;  off = align_up(off + nRb * Nmax * sizeof(int2));
    L.tile_cnt = off;  off = align_up(off + (size_t)L.tail_ntiles * sizeof(unsigned int));
    L.item_base = off; off = align_up(off + (npairs + 2) * sizeof(int));
    L.bal_ml = off;    off = align_up(off + nitems * G * sizeof(float2));
    L.bal_o = off;     off = align_up(off + nitems * G * D * sizeof(float));
  }
  L.total = off;
  return L;
}

bool finite_f(float x) { return std::isfinite(x); }

hws_status check_ctx(hws_ctx* ctx) {
  return ctx == nullptr ? HWS_ERR_INVALID_ARG : HWS_OK;
}

// Timing events of one stage (both null when profiling is off).  The events
// are taken by the first / last dispatch of the stage itself.
struct StageEv {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipEvent_t pool_event(hws_ctx* ctx) {
  hipEvent_t e = nullptr;
  if (ctx->pool.empty()) {
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
  } else {
    e = ctx->pool.back();
    ctx->pool.pop_back();
  }
  return e;
}

StageEv stage_events(hws_ctx* ctx, int stage) {
  StageEv ev;
  if (!ctx->prof) return ev;
  ev.start = pool_event(ctx);
  ev.stop = pool_event(ctx);
  if (ev.start == nullptr || ev.stop == nullptr) {
    if (ev.start) ctx->pool.push_back(ev.start);
    if (ev.stop) ctx->pool.push_back(ev.stop);
    return StageEv{};
  }
  ctx->recorded.push_back(EvPair{ev.start, ev.stop, stage});
  return ev;
}

// Last launch of a decode step: the status word, when the caller asked for it
// (`waited`: a single launch with hand-off waits ran in this step).
hws_status finish_step(hws_ctx* ctx, const DecodeParams& p, const hws_decode_args* a, bool waited, hipStream_t s) {
  if (a->status == nullptr) return HWS_OK;
  const hipError_t e = launch_step_status(p, a->status, waited, s);
  return e == hipSuccess ? HWS_OK : hip_fail(ctx, e, "status launch");
}

// Workspace of hws_decode_noalloc: one static device array, which every GPU
// that loads the library holds its own copy of.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device.
__device__ __align__(256) unsigned char scratch[HWS_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
  int dev;
  char* ptr;
};
std::mutex scratch_mu;
std::vector<ScratchAddr> scratch_addrs;

hws_status scratch_of_current_device(hws_ctx* ctx, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(scratch_mu);
  for (const ScratchAddr& s : scratch_addrs)
    if (s.dev == dev) {
      *out = s.ptr;
      return HWS_OK;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) return hip_fail(ctx, e, "hipGetSymbolAddress(scratch)");
  scratch_addrs.push_back(ScratchAddr{dev, static_cast<char*>(ptr)});
  *out = static_cast<char*>(ptr);
  return HWS_OK;
}

hws_status decode_step(hws_ctx* ctx, const hws_decode_args* a, void* stream, bool noalloc);

}  // namespace

extern "C" {

int32_t hws_abi_version(void) { return HWS_ABI_VERSION; }

const char* hws_status_string(hws_status s) {
  switch (s) {
    case HWS_OK: return "ok";
    case HWS_ERR_INVALID_ARG: return "invalid argument";
    case HWS_ERR_STATE: return "call out of order";
    case HWS_ERR_CAPACITY: return "capacity exceeded";
    case HWS_ERR_WORKSPACE: return "workspace too small";
    case HWS_ERR_UNSUPPORTED: return "unsupported shape";
    case HWS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* hws_last_error(const hws_ctx* ctx) { return ctx == nullptr ? "" : ctx->err.c_str(); }

hws_status hws_create(const hws_config* cfg, hws_ctx** out) {
  if (cfg == nullptr || out == nullptr) return HWS_ERR_INVALID_ARG;
  *out = nullptr;
  const hws_config& c = *cfg;
  if (c.num_q_heads < 1 || c.num_kv_heads < 1 || c.num_q_heads % c.num_kv_heads != 0) return HWS_ERR_INVALID_ARG;
  const int G = c.num_q_heads / c.num_kv_heads;
  if (c.num_kv_heads > MAX_KV || (G != 1 && G != 2 && G != 4 && G != 8)) return HWS_ERR_UNSUPPORTED;
  if (c.head_dim != D || c.index_dim != R || c.block_size != BS) return HWS_ERR_UNSUPPORTED;
  if (c.num_blocks < 1 || c.max_blocks_per_seq < 1 || c.max_blocks_per_seq > (1 << 26)) return HWS_ERR_INVALID_ARG;
  if (c.kv_dtype != HWS_KV_BF16 && c.kv_dtype != HWS_KV_FP8_E4M3) return HWS_ERR_INVALID_ARG;
  if (c.index_dtype != HWS_INDEX_F32 && c.index_dtype != HWS_INDEX_BF16) return HWS_ERR_INVALID_ARG;
  if (c.n_sink < 0 || c.window < 0 || (long long)c.n_sink + c.window < 1) return HWS_ERR_INVALID_ARG;
  if (c.local_ring != 0 && c.local_ring != 1) return HWS_ERR_INVALID_ARG;
  if (c.local_ring) {
    if (c.max_seqs < 1 || c.ring_slack < 0 || (long long)c.n_sink + c.window + c.ring_slack > (1 << 26))
      return HWS_ERR_INVALID_ARG;
    const long long rows = ((long long)c.n_sink + 63) / 64 * 64 + ((long long)c.window + c.ring_slack + BS - 1) / BS * BS;
    if ((long long)c.max_seqs * c.num_kv_heads * rows / BS >= (1LL << 31)) return HWS_ERR_INVALID_ARG;
  }
  if (!finite_f(c.attn_scale) || !(c.attn_scale > 0.f) || !finite_f(c.index_scale) ||
      !finite_f(c.rope_theta) || c.rope_theta < 0.f)
    return HWS_ERR_INVALID_ARG;
  hws_ctx* ctx = new (std::nothrow) hws_ctx();
  if (ctx == nullptr) return HWS_ERR_INVALID_ARG;
  ctx->cfg = c;
  ctx->G = G;
  rebuild_slots(ctx);
  *out = ctx;
  return HWS_OK;
}

hws_status hws_destroy(hws_ctx* ctx) {
  if (ctx == nullptr) return HWS_OK;
  for (auto& p : ctx->recorded) { hipEventDestroy(p.a); hipEventDestroy(p.b); }
  for (auto e : ctx->pool) hipEventDestroy(e);
  delete ctx;
  return HWS_OK;
}

hws_status hws_set_head_kinds(hws_ctx* ctx, const uint8_t* kinds) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (kinds == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "kinds is NULL");
  if (ctx->appended) return fail(ctx, HWS_ERR_STATE, "head kinds are fixed after the first append");
  for (int h = 0; h < ctx->cfg.num_kv_heads; ++h)
    if (kinds[h] != HWS_HEAD_LOCAL && kinds[h] != HWS_HEAD_RETRIEVAL)
      return fail(ctx, HWS_ERR_INVALID_ARG, "kinds[%d] = %d is not a head kind", h, (int)kinds[h]);
  std::memcpy(ctx->kinds, kinds, (size_t)ctx->cfg.num_kv_heads);
  rebuild_slots(ctx);
  return HWS_OK;
}

hws_status hws_classify_by_scores(hws_ctx* ctx, const float* q_head_scores, int32_t n_retrieval_kv,
                                  int32_t lower_is_retrieval) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (q_head_scores == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "scores is NULL");
  const int Hkv = ctx->cfg.num_kv_heads, G = ctx->G;
  if (n_retrieval_kv < 0 || n_retrieval_kv > Hkv)
    return fail(ctx, HWS_ERR_INVALID_ARG, "n_retrieval_kv = %d outside [0, %d]", n_retrieval_kv, Hkv);
  if (ctx->appended) return fail(ctx, HWS_ERR_STATE, "head kinds are fixed after the first append");
  std::vector<double> pooled(Hkv);
  for (int h = 0; h < Hkv; ++h) {
    double s = 0.0;
    for (int g = 0; g < G; ++g) {
      const float v = q_head_scores[h * G + g];
      if (!finite_f(v)) return fail(ctx, HWS_ERR_INVALID_ARG, "score of query head %d is not finite", h * G + g);
      s += v;
    }
    pooled[h] = s / G;                       // mean pooling over the GQA group
  }
  std::vector<int> order(Hkv);
  for (int h = 0; h < Hkv; ++h) order[h] = h;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return lower_is_retrieval ? pooled[a] < pooled[b] : pooled[a] > pooled[b];
  });
  uint8_t kinds[MAX_KV] = {};
  for (int i = 0; i < n_retrieval_kv; ++i) kinds[order[i]] = HWS_HEAD_RETRIEVAL;
  std::memcpy(ctx->kinds, kinds, (size_t)Hkv);
  rebuild_slots(ctx);
  return HWS_OK;
}

hws_status hws_get_head_kinds(const hws_ctx* ctx, uint8_t* kinds) {
  if (ctx == nullptr || kinds == nullptr) return HWS_ERR_INVALID_ARG;
  std::memcpy(kinds, ctx->kinds, (size_t)ctx->cfg.num_kv_heads);
  return HWS_OK;
}

hws_status hws_bind(hws_ctx* ctx, const hws_buffers* buf) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (buf == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "buffers is NULL");
  if (buf->k_pool == nullptr || buf->v_pool == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "k_pool / v_pool is NULL");
  if (ctx->cfg.kv_dtype == HWS_KV_FP8_E4M3 && buf->kv_scales == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "fp8 cache needs kv_scales");
  if (ctx->cfg.local_ring && (buf->local_k_pool == nullptr || buf->local_v_pool == nullptr))
    return fail(ctx, HWS_ERR_INVALID_ARG, "local_ring needs local_k_pool and local_v_pool");
  ctx->buf = *buf;
  ctx->bound = true;
  return HWS_OK;
}

hws_status hws_workspace_size(const hws_ctx* ctx, int32_t batch, int32_t max_seq_len, int32_t score_mode,
                              int32_t select_scope, size_t* bytes) {
  if (ctx == nullptr || bytes == nullptr) return HWS_ERR_INVALID_ARG;
  if (batch < 1 || max_seq_len < 1) return HWS_ERR_INVALID_ARG;
  if (score_mode != HWS_SCORE_INDEX && score_mode != HWS_SCORE_FULL) return HWS_ERR_INVALID_ARG;
  if (select_scope != HWS_SCOPE_KV_HEAD && select_scope != HWS_SCOPE_QUERY_HEAD) return HWS_ERR_INVALID_ARG;
  if ((long long)max_seq_len > (long long)ctx->cfg.max_blocks_per_seq * BS) return HWS_ERR_CAPACITY;
  *bytes = make_layout(ctx, batch, max_seq_len, ctx->cfg.rope_theta > 0.f, score_mode,
                       select_scope == HWS_SCOPE_QUERY_HEAD ? ctx->G : 1).total;
  return HWS_OK;
}

hws_status hws_append(hws_ctx* ctx, int32_t n_seq, int32_t n_tok, const int32_t* block_tables,
                      const int32_t* start_pos, const int32_t* seq_slots, const void* k, const void* v,
                      void* stream) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, HWS_ERR_STATE, "append before bind");
  if (n_seq < 1 || n_tok < 1) return fail(ctx, HWS_ERR_INVALID_ARG, "n_seq = %d, n_tok = %d", n_seq, n_tok);
  if (block_tables == nullptr || start_pos == nullptr || k == nullptr || v == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "null device pointer");
  if ((long long)n_tok > (long long)ctx->cfg.max_blocks_per_seq * BS)
    return fail(ctx, HWS_ERR_CAPACITY, "n_tok = %d exceeds the block table", n_tok);
  if (ctx->nR > 0 && (ctx->buf.index_pool == nullptr || ctx->buf.proj == nullptr))
    return fail(ctx, HWS_ERR_INVALID_ARG, "retrieval heads need index_pool and proj");
  if (ctx->ring_rows > 0 && ctx->nL > 0 && seq_slots == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "local_ring needs seq_slots");
  AppendParams p{};
  p.n_seq = n_seq;
  p.n_tok = n_tok;
  p.Hkv = ctx->cfg.num_kv_heads;
  p.nR = ctx->nR;
  p.max_blocks = ctx->cfg.max_blocks_per_seq;
  p.num_blocks = ctx->cfg.num_blocks;
  p.rope_theta = ctx->cfg.rope_theta;
  p.block_tables = block_tables;
  p.start_pos = start_pos;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.k_pool = ctx->buf.k_pool;
  p.v_pool = ctx->buf.v_pool;
  p.kv_scales = ctx->buf.kv_scales;
  p.Hp = ctx->Hp;
  p.n_sink = ctx->cfg.n_sink;
  p.window = ctx->cfg.window;
  p.ring_rows = ctx->ring_rows;
  p.ring_sink = ctx->ring_sink;
  p.ring_mod = ctx->ring_mod;
  p.max_seqs = ctx->cfg.max_seqs;
  p.seq_slots = seq_slots;
  p.lk_pool = ctx->buf.local_k_pool;
  p.lv_pool = ctx->buf.local_v_pool;
  p.index_pool = ctx->buf.index_pool;
  p.index_bf16 = ctx->cfg.index_dtype == HWS_INDEX_BF16 ? 1 : 0;
  p.proj = ctx->buf.proj;
  std::memcpy(p.ret_slot, ctx->ret_slot, sizeof(p.ret_slot));
  std::memcpy(p.pool_slot, ctx->pool_slot, sizeof(p.pool_slot));
  std::memcpy(p.loc_slot, ctx->loc_slot, sizeof(p.loc_slot));
  ctx->appended = true;
  const hipError_t e = launch_append(p, ctx->cfg.kv_dtype == HWS_KV_FP8_E4M3, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(ctx, e, "append launch");
  return HWS_OK;
}

hws_status hws_decode(hws_ctx* ctx, const hws_decode_args* a, void* stream) {
  return decode_step(ctx, a, stream, false);
}

hws_status hws_decode_noalloc(hws_ctx* ctx, const hws_decode_args* a, void* stream) {
  return decode_step(ctx, a, stream, true);
}

}  // extern "C"

namespace {

// One decode step; `noalloc` takes the workspace from the static scratch
// array of the current device instead of the caller's.
hws_status decode_step(hws_ctx* ctx, const hws_decode_args* a, void* stream, bool noalloc) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (a == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "args is NULL");
  if (!ctx->bound) return fail(ctx, HWS_ERR_STATE, "decode before bind");
  const hws_config& c = ctx->cfg;
  if (a->batch < 1 || a->max_seq_len < 1)
    return fail(ctx, HWS_ERR_INVALID_ARG, "batch = %d, max_seq_len = %d", a->batch, a->max_seq_len);
  if ((long long)a->max_seq_len > (long long)c.max_blocks_per_seq * BS)
    return fail(ctx, HWS_ERR_CAPACITY, "max_seq_len = %d exceeds %d pages of 16", a->max_seq_len, c.max_blocks_per_seq);
  if (a->select_mode != HWS_SELECT_TOP_P && a->select_mode != HWS_SELECT_TOP_K)
    return fail(ctx, HWS_ERR_INVALID_ARG, "select_mode = %d", a->select_mode);
  if (a->score_mode != HWS_SCORE_INDEX && a->score_mode != HWS_SCORE_FULL)
    return fail(ctx, HWS_ERR_INVALID_ARG, "score_mode = %d", a->score_mode);
  if (a->select_scope != HWS_SCOPE_KV_HEAD && a->select_scope != HWS_SCOPE_QUERY_HEAD)
    return fail(ctx, HWS_ERR_INVALID_ARG, "select_scope = %d", a->select_scope);
  if (a->q == nullptr || a->block_tables == nullptr || a->seq_lens == nullptr || a->out == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "null device pointer (q, block_tables, seq_lens or out)");
  if (ctx->nR > 0) {
    if (a->select_mode == HWS_SELECT_TOP_P && a->top_p == nullptr)
      return fail(ctx, HWS_ERR_INVALID_ARG, "top-p selection needs top_p");
    if (a->select_mode == HWS_SELECT_TOP_K && a->top_k == nullptr)
      return fail(ctx, HWS_ERR_INVALID_ARG, "top-k selection needs top_k");
    if (a->score_mode == HWS_SCORE_INDEX && (ctx->buf.index_pool == nullptr || ctx->buf.proj == nullptr))
      return fail(ctx, HWS_ERR_INVALID_ARG, "index scoring needs index_pool and proj");
  }
  if (a->sel_idx != nullptr && a->sel_cap < 1) return fail(ctx, HWS_ERR_INVALID_ARG, "sel_cap = %d", a->sel_cap);
  if (ctx->ring_rows > 0 && ctx->nL > 0 && a->seq_slots == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "local_ring needs seq_slots");
  const bool rope = c.rope_theta > 0.f;
  const int GS = a->select_scope == HWS_SCOPE_QUERY_HEAD ? ctx->G : 1;
  const Layout L = make_layout(ctx, a->batch, a->max_seq_len, rope, a->score_mode, GS);
  char* ws = nullptr;
  if (noalloc) {
    if (L.total > (size_t)HWS_NOALLOC_SCRATCH_BYTES)
      return fail(ctx, HWS_ERR_CAPACITY, "step needs %zu bytes of workspace; the static scratch array holds %u",
                  L.total, (unsigned)HWS_NOALLOC_SCRATCH_BYTES);
    const hws_status st = scratch_of_current_device(ctx, &ws);
    if (st != HWS_OK) return st;
  } else {
    if (a->workspace == nullptr || a->workspace_bytes < L.total)
      return fail(ctx, HWS_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", a->workspace_bytes, L.total);
    ws = static_cast<char*>(a->workspace);
  }
  DecodeParams p{};
  p.B = a->batch;
  p.Hq = c.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = ctx->G;
  p.GS = GS;
  p.nR = ctx->nR;
  p.nL = ctx->nL;
  p.Nmax = a->max_seq_len;
  p.Nagg = L.Nagg;
  p.max_blocks = c.max_blocks_per_seq;
  p.num_blocks = c.num_blocks;
  p.select_mode = a->select_mode;
  p.score_mode = a->score_mode;
  p.n_sink = c.n_sink;
  p.window = c.window;
  p.attn_scale = c.attn_scale;
  p.index_scale = c.index_scale;
  p.rope_theta = c.rope_theta;
  p.c2_attn = (float)((double)c.attn_scale * 1.4426950408889634);
  p.c2_score = a->score_mode == HWS_SCORE_FULL ? p.c2_attn : (float)((double)c.index_scale * 1.4426950408889634);
  p.q = static_cast<const uint16_t*>(a->q);
  p.block_tables = a->block_tables;
  p.seq_lens = a->seq_lens;
  p.top_p = a->top_p;
  p.top_k = a->top_k;
  p.k_pool = ctx->buf.k_pool;
  p.v_pool = ctx->buf.v_pool;
  p.kv_scales = c.kv_dtype == HWS_KV_FP8_E4M3 ? ctx->buf.kv_scales : nullptr;
  p.Hp = ctx->Hp;
  p.ring_rows = ctx->ring_rows;
  p.ring_sink = ctx->ring_sink;
  p.ring_mod = ctx->ring_mod;
  p.ring_pages = (int)((long long)c.max_seqs * ctx->nL * ctx->ring_rows / BS);
  p.max_seqs = c.max_seqs;
  p.seq_slots = a->seq_slots;
  p.lk_pool = ctx->buf.local_k_pool;
  p.lv_pool = ctx->buf.local_v_pool;
  p.index_pool = ctx->buf.index_pool;
  p.index_bf16 = ctx->cfg.index_dtype == HWS_INDEX_BF16 ? 1 : 0;
  p.proj = ctx->buf.proj;
  p.scores = a->scores != nullptr ? a->scores : reinterpret_cast<float*>(ws + L.scores);
  p.scores_out = a->scores != nullptr ? 1 : 0;
  p.agg = reinterpret_cast<float*>(ws + L.agg);
  p.spart = reinterpret_cast<float2*>(ws + L.spart);
  p.sel = reinterpret_cast<SelState*>(ws + L.sel);
  p.apart_ml = reinterpret_cast<float2*>(ws + L.apart_ml);
  p.apart_o = reinterpret_cast<float*>(ws + L.apart_o);
  p.qrot = rope ? reinterpret_cast<float*>(ws + L.qrot) : nullptr;
  p.out = a->out;
  p.lse = a->lse;
  p.sel_counts = a->sel_counts;
  p.sel_idx = a->sel_idx;
  p.sel_cap = a->sel_cap;
  p.rows_read = a->rows_read;
  p.sel_mass = a->sel_mass;
  p.score_chunk = L.score_chunk;
  p.n_score_chunks = L.n_score_chunks;
  p.n_sel_chunks = L.n_sel_chunks;
  p.ncR = L.ncR;
  p.ncL = L.ncL;
  p.att_chunk_R = L.att_chunk_R;
  p.max_splits = L.max_splits;
  p.tail_tph = L.tail_tph;
  p.tail_ntiles = L.tail_ntiles;
  p.tail_sync = reinterpret_cast<unsigned int*>(ws + L.tail_sync);
  p.tail_ties = reinterpret_cast<unsigned int*>(ws + L.tail_ties);
  p.spin_limit = ctx->spin_limit;
  p.wait_bias = ctx->wait_bias;
  p.phase_t = reinterpret_cast<unsigned long long*>(ctx->phase_t);
  p.phase_wgs = ctx->phase_wgs;
  std::memcpy(p.ret_slot, ctx->ret_slot, sizeof(p.ret_slot));
  std::memcpy(p.ret_head, ctx->ret_head, sizeof(p.ret_head));
  std::memcpy(p.loc_head, ctx->loc_head, sizeof(p.loc_head));
  std::memcpy(p.pool_slot, ctx->pool_slot, sizeof(p.pool_slot));
  std::memcpy(p.loc_slot, ctx->loc_slot, sizeof(p.loc_slot));

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (p.rows_read != nullptr && (e = launch_clear_rows_read(p, s)) != hipSuccess)
    return hip_fail(ctx, e, "rows_read clear launch");
  if (rope && (e = launch_prep_q(p, s)) != hipSuccess) return hip_fail(ctx, e, "prep_q launch");
  // Single launch after the scoring scan (or with the scan inside, one tile
  // per workgroup, for full-dim G = 4 scoring) when every tile fits the
  // grid the device holds at once; otherwise one kernel per stage.
  const int mode = ctx->launch_mode;
  const bool coop = mode == HWS_LAUNCH_COOPERATIVE;
  // (one set per query head runs in the per-stage kernels)
  const bool single = ctx->nR > 0 && mode != HWS_LAUNCH_MULTI && GS == 1;
  // the scan inside the single launch: AUTO, SINGLE and COOPERATIVE
  const bool scan_inside = single && (mode == HWS_LAUNCH_AUTO || mode == HWS_LAUNCH_SINGLE || coop);
  // AUTO takes the single launch after the scan only for short contexts (one
  // 4096-position stretch per head: there the per-stage launches' latency
  // dominates; measured 40.5 against 44.1 us at 4096, slower from 8192 on)
  const bool tail_ok = mode == HWS_LAUNCH_SINGLE || coop || mode == HWS_LAUNCH_SCAN_SINGLE ||
                       (mode == HWS_LAUNCH_AUTO && a->max_seq_len <= AUTO_TAIL_MAX_LEN);
  const int nwf = scan_inside ? fused_grid(p, coop) : 0;
  if (nwf > 0 && L.tail_ntiles <= nwf) {
    p.n_score_chunks = L.tail_tph;                 // one (max, sum) partial per tile
    const StageEv ef = stage_events(ctx, 5);
    if ((e = launch_fused(p, nwf, coop, s, ef.start, ef.stop)) != hipSuccess) return hip_fail(ctx, e, "fused launch");
    if (a->sel_idx != nullptr && (e = launch_emit(p, s)) != hipSuccess) return hip_fail(ctx, e, "emit launch");
    return finish_step(ctx, p, a, true, s);
  }
  // index scores: the scan inside the launch too, in tiles of 2048 positions,
  // or 8192 where 2048 would need more workgroups than the device holds
  // (measured: 2048-position tiles beat 8192 at the 8B layer shape, 53.8
  // against 74.4 us, the scan of a tile being bound by one workgroup's loads
  // in flight).  AUTO takes it for G <= 4: a dense G = 8 selection gathers
  // too few rows per workgroup at once (256K-token workload: 107 against
  // 90.8 us for the per-stage attention).
  if (scan_inside && a->score_mode == HWS_SCORE_INDEX && (mode != HWS_LAUNCH_AUTO || ctx->G <= 4)) {
    int pick = 0, pick_nw = 0;
    for (const int sp : {4, 16}) {
      const long long ntiles = (long long)a->batch * ctx->nR * cdiv(a->max_seq_len, (long long)TAIL_THREADS * sp);
      const int nwi = fused_index_grid(p, sp, coop);
      if (pick == 0 && nwi > 0 && ntiles <= nwi) { pick = sp; pick_nw = nwi; }
    }
    if (pick > 0) {
      const int tph = cdiv(a->max_seq_len, (long long)TAIL_THREADS * pick);
      p.tail_tph = tph;
      p.tail_ntiles = a->batch * ctx->nR * tph;
      p.n_score_chunks = tph;                        // one (max, sum) partial per tile
      const StageEv ef = stage_events(ctx, 7);
      if ((e = launch_fused_index(p, pick, pick_nw, coop, s, ef.start, ef.stop)) != hipSuccess)
        return hip_fail(ctx, e, "fused index launch");
      if (a->sel_idx != nullptr && (e = launch_emit(p, s)) != hipSuccess) return hip_fail(ctx, e, "emit launch");
      return finish_step(ctx, p, a, true, s);
    }
  }
  const int nwg = (single && tail_ok) ? tail_grid(p, coop) : 0;
  const bool tail = nwg > 0 && (long long)L.tail_ntiles <= (long long)TAIL_MAXT * nwg;
  if (tail) {
    const StageEv es = stage_events(ctx, 0);
    if ((e = launch_score(p, s, es.start, es.stop)) != hipSuccess) return hip_fail(ctx, e, "score launch");
    const StageEv et = stage_events(ctx, 4);
    if ((e = launch_tail(p, nwg, coop, s, et.start, et.stop)) != hipSuccess) return hip_fail(ctx, e, "tail launch");
    if (a->sel_idx != nullptr && (e = launch_emit(p, s)) != hipSuccess) return hip_fail(ctx, e, "emit launch");
    return finish_step(ctx, p, a, true, s);
  }
  // AUTO otherwise: the whole selection in one launch (its workgroups hand
  // the radix passes to each other, as in the single launch) when its tiles
  // fit, then the per-stage attention and merge.
  const int nws = (single && (mode == HWS_LAUNCH_AUTO || mode == HWS_LAUNCH_SCAN_SELECT)) ? tail_grid(p, false, true) : 0;
  const bool sel1 = nws > 0 && (long long)L.tail_ntiles <= (long long)TAIL_MAXT * nws;
  // Index scores: the attention balanced by kept rows (the selection lists
  // each head's kept rows) with SCAN_SELECT, and with AUTO for batches of
  // many (sequence, KV head) pairs, where position chunks leave a few dense
  // ones as the long pole (ragged fp8 workload, 256 pairs: attention 57 us
  // against 83, at 10 us more for the lists in the selection).  With few
  // pairs AUTO keeps the per-stage attention (256K-token workload, 8 pairs:
  // attention 35 us either way, selection 30 against 37, merge 9 against 14).
  const long long npairs = (long long)a->batch * c.num_kv_heads;
  const bool balanced = sel1 && a->score_mode == HWS_SCORE_INDEX && L.bal_o != 0 && npairs <= BAL_MAX_HEADS &&
                        npairs * ((long long)a->max_seq_len + BAL_PIECE_COST) < (1LL << 31) && L.tail_tph <= BAL_MAX_TPH &&
                        (mode == HWS_LAUNCH_SCAN_SELECT || (mode == HWS_LAUNCH_AUTO && npairs >= BAL_AUTO_PAIRS));
  if (ctx->nR > 0) {
    const StageEv es = stage_events(ctx, 0);
    if ((e = launch_score(p, s, es.start, es.stop)) != hipSuccess) return hip_fail(ctx, e, "score launch");
    const StageEv ev = stage_events(ctx, 1);
    if (sel1) {
      p.agg_out = 1;
      if (balanced) {
        p.row_list = reinterpret_cast<int2*>(ws + L.row_list);
        p.tile_cnt = reinterpret_cast<unsigned int*>(ws + L.tile_cnt);
      }
      if ((e = launch_tail(p, nws, false, s, ev.start, ev.stop, true)) != hipSuccess)
        return hip_fail(ctx, e, "select launch");
    } else {
      for (int pass = 1; pass <= 3; ++pass) {
        if ((e = launch_select(p, s, pass, pass == 1 ? ev.start : nullptr, pass == 3 ? ev.stop : nullptr)) != hipSuccess)
          return hip_fail(ctx, e, "select launch");
      }
    }
  }
  const StageEv ea = stage_events(ctx, balanced ? 8 : 2);
  if (balanced) {
    p.row_list = reinterpret_cast<int2*>(ws + L.row_list);
    p.item_base = reinterpret_cast<int*>(ws + L.item_base);
    p.bal_ml = reinterpret_cast<float2*>(ws + L.bal_ml);
    p.bal_o = reinterpret_cast<float*>(ws + L.bal_o);
    if ((e = launch_attend_balanced(p, s, ea.start, ea.stop)) != hipSuccess) return hip_fail(ctx, e, "attend launch");
  } else if ((e = launch_attend(p, s, ea.start, ea.stop)) != hipSuccess) {
    return hip_fail(ctx, e, "attend launch");
  }
  const StageEv em = stage_events(ctx, 3);
  if ((e = launch_merge(p, s, em.start, em.stop)) != hipSuccess) return hip_fail(ctx, e, "merge launch");
  if (ctx->nR > 0 && a->sel_idx != nullptr && (e = launch_emit(p, s)) != hipSuccess)
    return hip_fail(ctx, e, "emit launch");
  return finish_step(ctx, p, a, sel1, s);
}

}  // namespace

extern "C" {

hws_status hws_prefill(hws_ctx* ctx, const hws_prefill_args* a, void* stream) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (a == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "args is NULL");
  if (!ctx->bound) return fail(ctx, HWS_ERR_STATE, "prefill before bind");
  const hws_config& c = ctx->cfg;
  if (a->n_seq < 1 || a->n_tok < 1)
    return fail(ctx, HWS_ERR_INVALID_ARG, "n_seq = %d, n_tok = %d", a->n_seq, a->n_tok);
  if (a->dense != 0 && a->dense != 1) return fail(ctx, HWS_ERR_INVALID_ARG, "dense = %d", a->dense);
  if (a->q == nullptr || a->block_tables == nullptr || a->start_pos == nullptr || a->out == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "null device pointer (q, block_tables, start_pos or out)");
  if ((long long)a->n_tok > (long long)c.max_blocks_per_seq * BS)
    return fail(ctx, HWS_ERR_CAPACITY, "n_tok = %d exceeds the block table", a->n_tok);
  if (ctx->ring_rows > 0 && ctx->nL > 0) {
    if (a->dense) return fail(ctx, HWS_ERR_UNSUPPORTED, "dense prefill needs every row of the local heads (no local_ring)");
    if (a->seq_slots == nullptr) return fail(ctx, HWS_ERR_INVALID_ARG, "local_ring needs seq_slots");
    if ((long long)a->n_tok > (long long)c.ring_slack + 1)
      return fail(ctx, HWS_ERR_CAPACITY, "n_tok = %d exceeds ring_slack + 1 = %lld", a->n_tok,
                  (long long)c.ring_slack + 1);
  }
  const int rows = prefill_rows_per_tile(c.rope_theta > 0.f);
  const int qp = rows / ctx->G;
  const long long ntq = (a->n_tok + qp - 1) / qp;
  if ((long long)a->n_seq * c.num_kv_heads * ntq >= (1LL << 31))
    return fail(ctx, HWS_ERR_CAPACITY, "too many query tiles");
  PrefillParams p{};
  p.n_seq = a->n_seq;
  p.n_tok = a->n_tok;
  p.Hq = c.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = ctx->G;
  p.max_blocks = c.max_blocks_per_seq;
  p.num_blocks = c.num_blocks;
  p.Hp = ctx->Hp;
  p.n_sink = c.n_sink;
  p.window = c.window;
  p.ntq = (int)ntq;
  p.c2 = (float)((double)c.attn_scale * 1.4426950408889634);
  p.rope_theta = c.rope_theta;
  p.q = static_cast<const uint16_t*>(a->q);
  p.block_tables = a->block_tables;
  p.start_pos = a->start_pos;
  p.k_pool = ctx->buf.k_pool;
  p.v_pool = ctx->buf.v_pool;
  p.kv_scales = c.kv_dtype == HWS_KV_FP8_E4M3 ? ctx->buf.kv_scales : nullptr;
  if (ctx->ring_rows > 0 && ctx->nL > 0) {
    p.ring_rows = ctx->ring_rows;
    p.ring_sink = ctx->ring_sink;
    p.ring_mod = ctx->ring_mod;
    p.max_seqs = c.max_seqs;
    p.seq_slots = a->seq_slots;
    p.lk_pool = ctx->buf.local_k_pool;
    p.lv_pool = ctx->buf.local_v_pool;
  }
  p.out = a->out;
  p.lse = a->lse;
  std::memcpy(p.pool_slot, ctx->pool_slot, sizeof(p.pool_slot));
  for (int h = 0; h < MAX_KV; ++h) { p.ret_head[h] = -1; p.loc_head[h] = -1; }
  if (a->dense) {
    p.nR = c.num_kv_heads;
    p.nL = 0;
    for (int h = 0; h < c.num_kv_heads; ++h) p.ret_head[h] = (signed char)h;
  } else {
    p.nR = ctx->nR;
    p.nL = ctx->nL;
    std::memcpy(p.ret_head, ctx->ret_head, sizeof(p.ret_head));
    std::memcpy(p.loc_head, ctx->loc_head, sizeof(p.loc_head));
  }
  const StageEv ev = stage_events(ctx, 6);
  const hipError_t e = launch_prefill(p, static_cast<hipStream_t>(stream), ev.start, ev.stop);
  if (e != hipSuccess) return hip_fail(ctx, e, "prefill launch");
  return HWS_OK;
}

namespace {

// Workspace of hws_dense_lse: rotated queries (RoPE on), then the chunk partials.
struct DenseLayout {
  size_t qrot, spart, total;
  int nch;
};

DenseLayout dense_layout(const hws_ctx* c, int B, int Nmax) {
  DenseLayout L{};
  L.nch = cdiv(Nmax, DENSE_CHUNK);
  size_t off = 0;
  L.qrot = off;
  off = align_up(off + (c->cfg.rope_theta > 0.f ? (size_t)B * c->cfg.num_q_heads * D * sizeof(float) : 0));
  L.spart = off;
  off = align_up(off + (size_t)B * c->cfg.num_kv_heads * L.nch * c->G * sizeof(float2));
  L.total = off;
  return L;
}

}  // namespace

hws_status hws_dense_lse_workspace(const hws_ctx* ctx, int32_t batch, int32_t max_seq_len, size_t* bytes) {
  if (ctx == nullptr || bytes == nullptr || batch < 1 || max_seq_len < 1) return HWS_ERR_INVALID_ARG;
  if ((long long)max_seq_len > (long long)ctx->cfg.max_blocks_per_seq * BS) return HWS_ERR_CAPACITY;
  *bytes = dense_layout(ctx, batch, max_seq_len).total;
  return HWS_OK;
}

hws_status hws_dense_lse(hws_ctx* ctx, int32_t batch, int32_t max_seq_len, const void* q,
                         const int32_t* block_tables, const int32_t* seq_lens, float* lse_full, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (!ctx->bound) return fail(ctx, HWS_ERR_STATE, "dense lse before bind");
  const hws_config& c = ctx->cfg;
  if (batch < 1 || max_seq_len < 1) return fail(ctx, HWS_ERR_INVALID_ARG, "batch = %d, max_seq_len = %d", batch, max_seq_len);
  if ((long long)max_seq_len > (long long)c.max_blocks_per_seq * BS)
    return fail(ctx, HWS_ERR_CAPACITY, "max_seq_len = %d exceeds %d pages of 16", max_seq_len, c.max_blocks_per_seq);
  if (q == nullptr || block_tables == nullptr || seq_lens == nullptr || lse_full == nullptr)
    return fail(ctx, HWS_ERR_INVALID_ARG, "null device pointer (q, block_tables, seq_lens or lse_full)");
  if (ctx->ring_rows > 0 && ctx->nL > 0)
    return fail(ctx, HWS_ERR_UNSUPPORTED, "local heads in a ring keep only their sinks and window");
  const DenseLayout L = dense_layout(ctx, batch, max_seq_len);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(ctx, HWS_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  DecodeParams p{};
  p.B = batch;
  p.Hq = c.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = ctx->G;
  p.Nmax = max_seq_len;
  p.max_blocks = c.max_blocks_per_seq;
  p.num_blocks = c.num_blocks;
  p.rope_theta = c.rope_theta;
  p.c2_attn = (float)((double)c.attn_scale * 1.4426950408889634);
  p.q = static_cast<const uint16_t*>(q);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.k_pool = ctx->buf.k_pool;
  p.kv_scales = c.kv_dtype == HWS_KV_FP8_E4M3 ? ctx->buf.kv_scales : nullptr;
  p.Hp = ctx->Hp;
  std::memcpy(p.pool_slot, ctx->pool_slot, sizeof(p.pool_slot));
  p.qrot = c.rope_theta > 0.f ? reinterpret_cast<float*>(ws + L.qrot) : nullptr;
  p.spart = reinterpret_cast<float2*>(ws + L.spart);
  p.n_score_chunks = L.nch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (p.qrot != nullptr && (e = launch_prep_q(p, s)) != hipSuccess) return hip_fail(ctx, e, "prep_q launch");
  if ((e = launch_dense_lse(p, lse_full, s)) != hipSuccess) return hip_fail(ctx, e, "dense lse launch");
  return HWS_OK;
}

hws_status hws_effective_rank_workspace(int32_t num_q_heads, int32_t num_kv_heads, size_t* bytes) {
  if (bytes == nullptr || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return HWS_ERR_INVALID_ARG;
  *bytes = rank_workspace_bytes(num_q_heads, num_kv_heads);
  return HWS_OK;
}

hws_status hws_effective_rank(int32_t num_q_heads, int32_t num_kv_heads, int32_t d_model, const float* w_q,
                              const float* w_k, float* eff_rank, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 || d_model < 1)
    return HWS_ERR_INVALID_ARG;
  if (w_q == nullptr || w_k == nullptr || eff_rank == nullptr) return HWS_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < rank_workspace_bytes(num_q_heads, num_kv_heads))
    return HWS_ERR_WORKSPACE;
  const hipError_t e = launch_effective_rank(num_q_heads, num_kv_heads, d_model, w_q, w_k, eff_rank, workspace,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HWS_OK : HWS_ERR_HIP;
}

hws_status hws_set_launch_mode(hws_ctx* ctx, int32_t mode) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (mode < HWS_LAUNCH_AUTO || mode > HWS_LAUNCH_SCAN_SINGLE)
    return fail(ctx, HWS_ERR_INVALID_ARG, "launch mode = %d", mode);
  ctx->launch_mode = mode;
  return HWS_OK;
}

hws_status hws_set_wait_limit(hws_ctx* ctx, uint32_t max_polls, int32_t unreachable) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (max_polls > (1u << 24))
    return fail(ctx, HWS_ERR_INVALID_ARG, "max_polls = %u (at most 2^24)", max_polls);
  // waits check the limit every 256 polls
  ctx->spin_limit = max_polls == 0 ? (1u << 20) : ((max_polls + 255u) & ~255u);
  ctx->wait_bias = unreachable != 0 ? 1u : 0u;
  return HWS_OK;
}

hws_status hws_profile_enable(hws_ctx* ctx, int32_t enable) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  ctx->prof = enable != 0;
  return HWS_OK;
}

hws_status hws_profile_read(hws_ctx* ctx, double* ms, int32_t* calls, int32_t n) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (n < 0 || (n > 0 && (ms == nullptr || calls == nullptr))) return fail(ctx, HWS_ERR_INVALID_ARG, "bad output arrays");
  for (int i = 0; i < n; ++i) { ms[i] = 0.0; calls[i] = 0; }
  hws_status st = HWS_OK;
  for (auto& pr : ctx->recorded) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(pr.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, pr.a, pr.b);
    if (e != hipSuccess) {
      st = hip_fail(ctx, e, "profile read");
    } else if (pr.stage < n) {
      ms[pr.stage] += t;
      calls[pr.stage] += 1;
    }
    ctx->pool.push_back(pr.a);
    ctx->pool.push_back(pr.b);
  }
  ctx->recorded.clear();
  return st;
}

hws_status hws_profile_phases(hws_ctx* ctx, uint64_t* buf, int32_t max_workgroups) {
  if (check_ctx(ctx)) return HWS_ERR_INVALID_ARG;
  if (buf != nullptr && max_workgroups < 1)
    return fail(ctx, HWS_ERR_INVALID_ARG, "max_workgroups = %d", max_workgroups);
  ctx->phase_t = buf;
  ctx->phase_wgs = buf != nullptr ? max_workgroups : 0;
  return HWS_OK;
}

const char* hws_profile_stage_name(int32_t i) {
  return (i >= 0 && i < NUM_STAGES) ? STAGE_NAMES[i] : "";
}

}  // extern "C"
