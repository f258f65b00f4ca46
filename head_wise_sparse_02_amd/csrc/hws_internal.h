// Internal definitions shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hws {

constexpr int D = 128;            // head dim
constexpr int R = 16;             // index dim
constexpr int BS = 16;            // tokens per page
constexpr int MAX_KV = 64;        // KV heads per layer
constexpr int MAX_G = 8;          // query heads per KV head

constexpr int SCORE_CHUNK = 1024; // tokens per scoring workgroup (4 waves x 256)
constexpr int G4_SCORE_CHUNK = 4096;  // tokens per workgroup of the G=4 full-dim scan
constexpr int SEL_THREADS = 1024; // threads per selection workgroup
constexpr int SEL_PER_THREAD = 16;
constexpr int SEL_CHUNK = SEL_THREADS * SEL_PER_THREAD;   // 16384 tokens
constexpr int HIST_BINS = 4096;   // pass 1 bins: bits 30..19 of the fp32 pattern
constexpr int LOCAL_CHUNK = 256;  // rows per local-head attention workgroup
constexpr int PHASES = 12;        // phase timestamps per workgroup (HWS_PHASES)
// Attention balanced by kept rows: at most BAL_ITEMS workgroups, each a
// segment of at least BAL_RMIN cost units (a pair of c rows costs
// BAL_PIECE_COST + c); a segment leaves one partial per (sequence, KV head)
// piece it covers.
constexpr int BAL_ITEMS = 2048;
constexpr int BAL_RMIN = 64;
constexpr int BAL_PIECE_COST = 128;  // a piece's fixed cost in rows (its list, queries and partial)
constexpr int BAL_AUTO_PAIRS = 64;   // AUTO balances the attention from this many (sequence, KV head) pairs
constexpr int BAL_MAX_HEADS = 2048;
constexpr int BAL_MAX_TPH = 256;    // selection tiles per head the balanced attention maps rows over  // (sequence, KV head) pairs the item table holds in LDS

// Single-launch tail (selection + attention + merge in one cooperative launch)
constexpr int TAIL_THREADS = 512;
constexpr int TAIL_TPT = 32;                             // tokens per thread per tile
constexpr int TAIL_TILE = TAIL_THREADS * TAIL_TPT;       // 16384 tokens
constexpr int TAIL_MAXT = 2;                             // tiles a workgroup keeps in registers

// Bit split of the non-negative fp32 aggregate a_i (bit 31 is always 0):
// pass 1 bins bits 30..19 (12 bits), pass 2 bits 18..9 (10), pass 3 bits 8..0 (9).
constexpr int P1_SHIFT = 19, P2_SHIFT = 9;
constexpr int P2_BINS = 1024, P3_BINS = 512;

constexpr uint32_t SEL_FINISHED = 1u;   // tstar is final
constexpr uint32_t SEL_TIE = 2u;        // top-k: keep only the `quota` lowest-position ties

// Fixed-point mass: round(a * 2^40) as uint64.  Integer bins make the
// threshold independent of the order in which workgroups add their counts.
constexpr float MASS_SCALE = 1099511627776.0f;   // 2^40

// Selection state of one (sequence, retrieval head).  Zeroed by the scoring
// kernel of each decode call; histograms are cleared by the last workgroup
// of each pass for the next one.
struct alignas(256) SelState {
  unsigned long long mass[HIST_BINS];
  unsigned int cnt[HIST_BINS];
  unsigned int done;        // arrivals in the current pass
  unsigned int flags;       // SEL_*
  unsigned int prefix;      // known high bits of the threshold pattern
  unsigned int tstar;       // threshold pattern (valid once FINISHED)
  unsigned long long mass_above;  // mass strictly above the candidate bin range
  unsigned int cnt_above;   // count strictly above the candidate bin range
  unsigned int nsel;        // |S| (top-p: summed by the attention kernel)
  unsigned int quota;       // top-k with SEL_TIE: ties at tstar to keep
  float lse2[MAX_G];        // per query head log2-sum-exp2 of the logits
  // Single-launch tail: every radix pass has its own bins (top-p: fixed-point
  // mass, top-k: counts; pass 1 uses `mass` above), and the tiles of the
  // head count their arrivals here.
  unsigned int arrive;      // tiles done with a radix pass (monotonic over passes)
  unsigned int tie_arrive;  // tiles that published their tie count
  unsigned int cnt_arrive;  // tiles that published their kept count (row lists for the attention)
  unsigned long long kept_mass;  // fixed-point sum of a_i over the kept tokens (only when asked for)
  unsigned long long mass2[P2_BINS];
  unsigned long long mass3[P3_BINS];
};
constexpr int SELSTATE_WORDS = (int)(sizeof(SelState) / 4);

// Everything a decode kernel needs, passed by value.
struct DecodeParams {
  int B, Hq, Hkv, G, nR, nL, Nmax, max_blocks, num_blocks;
  int GS;                       // selection states per retrieval head: 1, or G (one per query head)
  int Nagg;                     // row stride of agg (Nmax rounded up to 64)
  int select_mode, score_mode;
  int n_sink, window;
  float attn_scale, index_scale, rope_theta;
  float c2_attn;    // attn_scale * log2(e)
  float c2_score;   // scale of raw scores to log2 logits (index or attention)
  const uint16_t* q;            // [B][Hq][D] bf16
  const int* block_tables;      // [B][max_blocks]
  const int* seq_lens;          // [B]
  const float* top_p;           // [B]
  const int* top_k;             // [B]
  const void* k_pool;           // [blocks][Hp][16 x 128] (pages hold Hp heads)
  const void* v_pool;
  const float* kv_scales;
  int Hp;                       // heads per page: Hkv, or nR with a local ring
  int ring_rows;                // local ring: rows per (slot, local head) = ring_sink + ring_mod; 0 = no ring
  int ring_sink, ring_mod;      // local ring: rows of positions 0..ring_sink-1, then position t at
                                // ring_sink + t % ring_mod (ring_sink a multiple of 64, ring_mod of 16)
  int ring_pages;               // local ring: 16-row pages in each ring pool
  int max_seqs;
  const int* seq_slots;         // [B] ring slot of each sequence (ring only)
  const void* lk_pool;          // [max_seqs][nL][ring_rows][128] ring pools (K in 16-row pages)
  const void* lv_pool;
  const void* index_pool;       // [blocks][nR][16][16] fp32, or bf16 when index_bf16
  int index_bf16;
  const float* proj;
  float* scores;                // [B][nR][Nmax][G]
  int scores_out;               // the caller asked for every score (else only kept ones may be written)
  float* agg;                   // [B][nR][GS][Nagg]
  float2* spart;                // [B][nR][n_score_chunks][G]  (max, sum) in log2 units
  SelState* sel;                // [B][nR][GS]
  float2* apart_ml;             // [B][Hkv][max_splits][G]  (max, sum)
  float* apart_o;               // [B][Hkv][max_splits][G][D]
  float* qrot;                  // [B][Hq][D] fp32 rotated queries (RoPE on) or null
  float* out;
  float* lse;
  int* sel_counts;
  int* sel_idx;
  int sel_cap;
  int* rows_read;               // debug [B][Hkv][Nmax]: reads of each cached row by the attention, or null
  float* sel_mass;              // [B][Hkv] or [B][Hq]: kept aggregate mass, or null
  int score_chunk;              // tokens per scoring workgroup
  int tail_tph, tail_ntiles;    // tail: tiles per retrieval head, total tiles
  unsigned int* tail_sync;      // [0] error word, [1 + b*Hkv + h] split arrivals (zeroed by the scan)
  unsigned int* tail_ties;      // [tail_ntiles] ties at t* per tile
  unsigned int spin_limit;      // polls before a hand-off wait gives up (multiple of 256)
  unsigned int wait_bias;       // added to every hand-off target (0; 1 makes each wait give up)
  unsigned long long* phase_t;  // [phase_wgs][HWS_PHASES] phase timestamps of the single launches, or null
  int phase_wgs;
  int n_score_chunks, n_sel_chunks, ncR, ncL, att_chunk_R, max_splits;
  int agg_out;                  // the single-launch selection ran: a_i is in agg, and the merge
                                // checks the hand-off error word
  // Attention balanced by kept rows (after the one-launch selection): the
  // selection writes each retrieval head's kept rows as one list in position
  // order; the attention cuts every head's rows into items of about the same
  // number of rows.
  int2* row_list;               // [B][nR][Nmax] (position, page) of the kept rows, tile j's at
                                //   j * TAIL_TILE.., or null
  unsigned int* tile_cnt;       // [tail_ntiles] kept rows of each selection tile
  int* item_base;               // [B * Hkv + 2] first listed row of each (sequence, KV head), the
                                //   total, then the rows per workgroup of the balanced attention
  float2* bal_ml;               // [BAL_ITEMS + B * Hkv][G] (max, sum) of each piece
  float* bal_o;                 // [BAL_ITEMS + B * Hkv][G][D] unnormalised output of each piece
  signed char ret_slot[MAX_KV];
  signed char ret_head[MAX_KV];
  signed char loc_head[MAX_KV];
  signed char pool_slot[MAX_KV];  // head's index within a page (-1: not in the pages)
  signed char loc_slot[MAX_KV];   // head's number among the local heads (-1: retrieval head)
};

struct AppendParams {
  int n_seq, n_tok, Hkv, nR, max_blocks, num_blocks;
  float rope_theta;
  const int* block_tables;
  const int* start_pos;
  const uint16_t* k;
  const uint16_t* v;
  void* k_pool;
  void* v_pool;
  float* kv_scales;
  int Hp;                       // heads per page
  int n_sink, window;
  int ring_rows, max_seqs;      // local ring (ring_rows = 0: none)
  int ring_sink, ring_mod;      // ring geometry (as in DecodeParams)
  const int* seq_slots;         // [n_seq] ring slots
  void* lk_pool;
  void* lv_pool;
  void* index_pool;             // fp32, or bf16 when index_bf16
  int index_bf16;
  const float* proj;
  signed char ret_slot[MAX_KV];
  signed char pool_slot[MAX_KV];
  signed char loc_slot[MAX_KV];   // local head's index among the local heads
};

// One chunked-prefill call: n_tok query positions per sequence from start_pos.
struct PrefillParams {
  int n_seq, n_tok, Hq, Hkv, G, max_blocks, num_blocks, Hp;
  int n_sink, window;
  int nR, nL;                   // heads walked as retrieval (all keys) / local (sinks + window)
  int ntq;                      // query tiles per (sequence, KV head)
  float c2;                     // attn_scale * log2(e)
  float rope_theta;
  const uint16_t* q;            // [n_seq][n_tok][Hq][D] bf16, pre-RoPE
  const int* block_tables;      // [n_seq][max_blocks]
  const int* start_pos;         // [n_seq]
  const void* k_pool;
  const void* v_pool;
  const float* kv_scales;       // FP8 pages: [blocks][Hp][2]; null for bf16
  float* out;                   // [n_seq][n_tok][Hq][D]
  float* lse;                   // [n_seq][n_tok][Hq] or null
  int ring_rows, ring_sink, ring_mod, max_seqs;   // local ring (ring_rows = 0: none)
  const int* seq_slots;         // [n_seq] ring slots
  const void* lk_pool;          // ring pools (bf16)
  const void* lv_pool;
  int item0;                    // work item of workgroup 0 (a launch may cover a range of items)
  signed char ret_head[MAX_KV];
  signed char loc_head[MAX_KV];
  signed char pool_slot[MAX_KV];
};

// Ring row of position t (ring_sink rows of the first positions, then t
// modulo ring_mod); the caller checks that the ring still holds t.
__host__ __device__ __forceinline__ int ring_row(int t, int ring_sink, int ring_mod) {
  return t < ring_sink ? t : (ring_mod > 0 ? ring_sink + t % ring_mod : 0);
}

// Launch a kernel; with timing events the start/stop timestamps are taken
// by the dispatch packet itself (no extra barrier packets in the stream).
template <typename K, typename... A>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1, A... args) {
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
  return hipGetLastError();
}

// Kernel launchers (one translation unit each); return the launch status.
// e0 / e1: optional timing events recorded at the start / end of the launch.
hipError_t launch_prep_q(const DecodeParams& p, hipStream_t s);
hipError_t launch_score(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_select(const DecodeParams& p, hipStream_t s, int pass, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_attend(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_merge(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
// Attention balanced by kept rows (index scores, one set per KV head, after
// the one-launch selection wrote sel_rows / tile_cnt) and its merge.
hipError_t launch_attend_balanced(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_merge_balanced(const DecodeParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_emit(const DecodeParams& p, hipStream_t s);
// Debug row-read counters to zero; the step's status word (waited: a single
// launch with hand-off waits ran in this step).
hipError_t launch_clear_rows_read(const DecodeParams& p, hipStream_t s);
// Dense log-sum-exp over every cached row (diagnostic): chunk partials of
// DENSE_CHUNK rows into p.spart ([B][Hkv][chunks][G], log2 units), then the
// reduction into lse_full [B][Hq] (natural log).
constexpr int DENSE_CHUNK = 1024;
hipError_t launch_dense_lse(const DecodeParams& p, float* lse_full, hipStream_t s);
hipError_t launch_step_status(const DecodeParams& p, int* status, bool waited, hipStream_t s);
// Single launch for select + attend + merge.  tail_grid() is the number of
// workgroups of the instantiation `p` needs that the device holds at once (0
// if there is no such instantiation, or `cooperative` and the device has no
// cooperative launches).
// select_only: the launch stops after the selection (threshold, top-k ties,
// a_i in agg), for the per-stage attention and merge to follow.
int tail_grid(const DecodeParams& p, bool cooperative, bool select_only = false);
hipError_t launch_tail(const DecodeParams& p, int nwg, bool cooperative, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1, bool select_only = false);
// The same with the scoring scan inside (full-dim scores, G = 4, bf16, no
// RoPE: 0 workgroups otherwise); launch_fused also resets the selection state.
int fused_grid(const DecodeParams& p, bool cooperative);
hipError_t launch_fused(const DecodeParams& p, int nwg, bool cooperative, hipStream_t s, hipEvent_t e0,
                        hipEvent_t e1);
// The same with the r = 16 index scan inside (KV-scope sets), in tiles of
// TAIL_THREADS * sp positions (sp = 4 or 16); p.tail_tph / tail_ntiles /
// n_score_chunks must describe those tiles.
constexpr int FI_TILE_MIN = TAIL_THREADS * 4;            // smallest index tile: 2048 positions
int fused_index_grid(const DecodeParams& p, int sp, bool cooperative);
hipError_t launch_fused_index(const DecodeParams& p, int sp, int nwg, bool cooperative, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1);
hipError_t launch_append(const AppendParams& p, int kv_fp8, hipStream_t s);
// Effective rank of the query-key kernels (fp64 Gram, Cholesky, Jacobi).
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
int prefill_rows_per_tile(bool rope);
size_t rank_workspace_bytes(int hq, int hkv);
hipError_t launch_effective_rank(int hq, int hkv, int d_model, const float* w_q, const float* w_k,
                                 float* eff_rank, void* workspace, hipStream_t s);

}  // namespace hws
