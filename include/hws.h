/*
 * hws.h — C ABI of libhws: head-wise sparse decode attention on AMD MI355X (gfx950).
 *
 * One context serves one attention layer.  Attention heads are split into
 * retrieval heads and local heads:
 *   - a retrieval KV head scores every cached token through a 16-dim pre-RoPE
 *     key index (or, in FULL mode, through the full-dim keys), keeps a dynamic
 *     top-p or fixed top-k token set and attends over only those rows;
 *   - a local KV head attends to its attention-sink tokens plus a sliding window.
 *
 * Sources (gist.science summary pages; titles as shown on the pages, the first
 * translated from Arabic):
 *   [RTPurbo] "Full attention returns in force: converting full attention to
 *             sparse attention within hundreds of training steps" (arXiv 2605.16928)
 *   [ICS]     "Inference-time context sparsity: illusion or opportunity?" (arXiv 2605.24168)
 *   [NHA]     "Native Hybrid Attention for Efficient Sequence Modeling" (arXiv 2510.07019)
 *   [AoH]     "Autonomy-of-Heads: Data-Free Sparse Attention from Frozen Query-Key
 *             Geometry" (arXiv 2608.06849)
 *
 * Conventions that hold for every call:
 *   - Return codes only (hws_status); nothing throws or aborts across the ABI.
 *     hws_last_error(ctx) holds a message for the last failing call on ctx.
 *   - Every argument is validated on the host before any HIP call, so all
 *     validation errors are reported without touching a GPU.
 *   - All device memory is caller-owned and passed as raw device pointers; the
 *     library never allocates device memory.  Host arrays and structs are
 *     copied before the call returns.
 *   - Device work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*, NULL = the default stream) and is asynchronous: device buffers
 *     must stay valid until the stream has finished.  No call synchronises.
 *   - A launch failure returns HWS_ERR_HIP with the HIP error text; a fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - A context is not thread-safe: use one context per stream.
 *   - hws_append, hws_decode and hws_prefill enqueue kernel launches only (no
 *     allocation, memset or synchronisation), so a call can be captured into
 *     a HIP graph on the caller's stream, with profile timing off; a decode
 *     step's own kernels reset its selection state in the workspace, so
 *     replays need nothing else.
 *
 * Supported shapes: head_dim 128, index_dim 16, block_size 16, GQA group
 * G = num_q_heads / num_kv_heads in {1, 2, 4, 8}, num_kv_heads <= 64.
 * Other values give HWS_ERR_UNSUPPORTED.
 */
#ifndef HWS_H
#define HWS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HWS_ABI_VERSION 5

typedef int32_t hws_status;
enum {
  HWS_OK = 0,
  HWS_ERR_INVALID_ARG = -1, /* null pointer, out-of-range value             */
  HWS_ERR_STATE = -2,       /* call out of order (e.g. decode before bind)    */
  HWS_ERR_CAPACITY = -3,    /* sequence longer than the block table allows    */
  HWS_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required     */
  HWS_ERR_UNSUPPORTED = -5, /* shape outside the supported set                */
  HWS_ERR_HIP = -6          /* a HIP launch or runtime call failed            */
};

/* KV storage type.  FP8 is OCP e4m3fn with one fp32 scale per
 * (block, KV head, K|V); see hws_append for how scales are set. */
enum { HWS_KV_BF16 = 0, HWS_KV_FP8_E4M3 = 1 };

/* Head kinds ([RTPurbo] Methodology §1: retrieval heads vs local heads). */
enum { HWS_HEAD_LOCAL = 0, HWS_HEAD_RETRIEVAL = 1 };

/* Selection rule of retrieval heads ([RTPurbo] Methodology §3). */
enum { HWS_SELECT_TOP_P = 0, HWS_SELECT_TOP_K = 1 };

/* Selection score: INDEX = 16-dim pre-RoPE index ([RTPurbo] Methodology §2);
 * FULL = full-dim q.k, i.e. exact "oracle top-k" ([ICS] §2). */
enum { HWS_SCORE_INDEX = 0, HWS_SCORE_FULL = 1 };
/* Storage of the r = 16 index k~ = P k: fp32 as computed (64 B per token and
 * retrieval head), or bf16 of P k evaluated in fp64 and rounded once (32 B). */
enum { HWS_INDEX_F32 = 0, HWS_INDEX_BF16 = 1 };
/* Selection scope: one set per KV head shared by its query heads, or one set
 * per query head ([ICS] §2: sparsity differs per token, query and head). */
enum { HWS_SCOPE_KV_HEAD = 0, HWS_SCOPE_QUERY_HEAD = 1 };
enum { HWS_LAUNCH_AUTO = 0, HWS_LAUNCH_MULTI = 1, HWS_LAUNCH_COOPERATIVE = 2, HWS_LAUNCH_SINGLE = 3,
       HWS_LAUNCH_SCAN_SELECT = 4, HWS_LAUNCH_SCAN_SINGLE = 5 };

typedef struct hws_ctx hws_ctx; /* opaque host object, owned by the library */

typedef struct {
  int32_t num_q_heads;        /* Hq                                          */
  int32_t num_kv_heads;       /* Hkv; query head g uses KV head g / (Hq/Hkv) */
  int32_t head_dim;           /* d, must be 128                              */
  int32_t index_dim;          /* r, must be 16                               */
  int32_t block_size;         /* tokens per KV page, must be 16              */
  int32_t num_blocks;         /* pages in the pools                          */
  int32_t max_blocks_per_seq; /* row length of every block table             */
  int32_t kv_dtype;           /* HWS_KV_*                                    */
  int32_t index_dtype;        /* HWS_INDEX_*: fp32 (64 B/token) or bf16      */
  int32_t n_sink;             /* local heads: sink tokens 0..n_sink-1        */
  int32_t window;             /* local heads: last `window` tokens           */
  int32_t local_ring;         /* 1: local heads keep only sinks + window rows
                                 in per-sequence ring pools (bf16 rows, also
                                 with fp8 pages); 0: every head keeps every
                                 row in the pages                           */
  int32_t max_seqs;           /* local_ring: sequence slots in the ring pools */
  int32_t ring_slack;         /* local_ring: rows kept beyond the window, >= 0;
                                 hws_prefill takes chunks of at most
                                 ring_slack + 1 positions                    */
  float attn_scale;           /* softmax scale of attention, e.g. 1/sqrt(d)  */
  float index_scale;          /* logit = index_scale * (P q).(P k)           */
  float rope_theta;           /* > 0: rotate-half RoPE with this base; 0: off */
} hws_config;

/* Caller-owned device buffers.  Layouts (row-major); Hp is the number of
 * heads a page holds: Hkv, or n_retrieval with local_ring (then the pages hold
 * the retrieval heads only, in KV-head order):
 *   k_pool:         [num_blocks][Hp][4][16][32] bf16 (or e4m3 bytes for FP8):
 *                   each 16-token page is stored in four 32-dim blocks, i.e.
 *                   element (slot r, dim d) of a page is at ((d/32)*16 + r)*32
 *                   + d%32; K is stored after RoPE (when rope_theta > 0).
 *   v_pool:         [num_blocks][Hp][16][128] bf16 or e4m3 bytes, row-major.
 *   kv_scales:      [num_blocks][Hp][2] fp32 (K scale, V scale); FP8 only.
 *   local_k_pool,   local_ring only: [max_seqs][n_local][W][128] bf16 (also
 *   local_v_pool:   when kv_dtype is FP8: the ring keeps exact rows) with the
 *                   local heads in KV-head order, W = S + M, S = n_sink rounded
 *                   up to a multiple of 64 and M = window + ring_slack rounded
 *                   up to a multiple of 16.  Position t of a sequence sits in
 *                   ring row t (t < S) or S + t % M.  K rows are grouped in
 *                   16-row pages laid out like k_pool pages, V rows are plain
 *                   rows.  [RTPurbo] Methodology §1: a local head only ever
 *                   reads its sinks and window, so older rows need not be kept
 *                   ([AoH] Results: the KV memory saving of local heads).
 *   index_pool:     [num_blocks][n_retrieval][16][16] fp32 or bf16 (index_dtype),
 *                   the projected pre-RoPE keys of retrieval heads in KV-head
 *                   order; may be NULL when no head is a retrieval head.
 *   proj:           [Hkv][16][128] fp32 index projections (rows of local
 *                   heads are ignored); may be NULL when no head is retrieval. */
typedef struct {
  void* k_pool;
  void* v_pool;
  float* kv_scales;
  void* index_pool;
  const float* proj;
  void* local_k_pool;
  void* local_v_pool;
} hws_buffers;

/* One decode step for a batch.  Device pointers unless noted. */
typedef struct {
  int32_t batch;             /* B >= 1 (host)                                 */
  int32_t max_seq_len;       /* host upper bound of seq_lens (sizes grids)    */
  int32_t select_mode;       /* HWS_SELECT_*                                  */
  int32_t score_mode;        /* HWS_SCORE_*                                   */
  int32_t select_scope;      /* HWS_SCOPE_* (0 = one set per KV head)         */
  const void* q;             /* [B][Hq][128] bf16, pre-RoPE queries           */
  const int32_t* block_tables; /* [B][max_blocks_per_seq] page ids            */
  const int32_t* seq_lens;   /* [B] context lengths incl. the current token;
                                with local_ring, the appended length          */
  const int32_t* seq_slots;  /* [B] ring slot of each sequence (local_ring),
                                or NULL                                       */
  const float* top_p;        /* [B] (TOP_P); p >= 1 keeps every token         */
  const int32_t* top_k;      /* [B] (TOP_K); k >= N keeps every token         */
  float* out;                /* [B][Hq][128] fp32 attention output            */
  float* lse;                /* [B][Hq] natural-log LSE over the set, or NULL */
  int32_t* sel_counts;       /* [B][Hkv] |S| per KV head (KV scope) or
                                [B][Hq] per query head (query scope; a local
                                head's query heads all report its set), or
                                NULL                                          */
  int32_t* sel_idx;          /* [B][n_retrieval][sel_cap] (KV scope) or
                                [B][n_retrieval][G][sel_cap] (query scope)
                                ascending positions, or NULL                  */
  int32_t sel_cap;           /* row length of sel_idx (host)                  */
  float* scores;             /* [B][n_retrieval][max_seq_len][G] raw scores
                                (P q).(P k) or q.k, or NULL (then kept in the
                                workspace)                                    */
  void* workspace;           /* hws_workspace_size() bytes                    */
  size_t workspace_bytes;
  /* ABI 5 (all optional, NULL = not wanted): */
  int32_t* rows_read;        /* debug: [B][Hkv][max_seq_len] int32, how many
                                times the attention read the cached row of
                                each position for each KV head (K and V, or V
                                alone when FULL scores give the logits).  The
                                step clears it first.  Rows of local heads
                                kept in a ring are not counted.               */
  float* sel_mass;           /* [B][Hkv] (KV scope) or [B][Hq] (query scope):
                                the aggregate mass the selected set keeps,
                                sum of a_i over S (a query head's own
                                probabilities in the query scope), in
                                [0, 1]; NaN for local heads ([RTPurbo] Main
                                results: attention mass retained)             */
  int32_t* status;           /* device int32: HWS_STEP_OK, or
                                HWS_STEP_WAIT_TIMEOUT when a hand-off wait of
                                the single launch gave up (the affected
                                outputs are then NaN)                         */
} hws_decode_args;

/* Values of hws_decode_args.status (written on the device by the step). */
enum { HWS_STEP_OK = 0, HWS_STEP_WAIT_TIMEOUT = 1 };

/* ABI version of the loaded library (HWS_ABI_VERSION). */
int32_t hws_abi_version(void);

/* Static text for a status code. */
const char* hws_status_string(hws_status s);

/* Message of the last failing call on ctx ("" if none; ctx may be NULL). */
const char* hws_last_error(const hws_ctx* ctx);

/* Create a context from cfg (copied).  All heads start as local heads. */
hws_status hws_create(const hws_config* cfg, hws_ctx** out);

/* Destroy a context (NULL is accepted).  Device buffers are not touched. */
hws_status hws_destroy(hws_ctx* ctx);

/* Set the head kinds: kinds[Hkv] (host) of HWS_HEAD_*.  Must precede the
 * first hws_append, because only retrieval heads keep an index
 * ([RTPurbo] Methodology §1: heads are split offline into H_ret and H_loc). */
hws_status hws_set_head_kinds(hws_ctx* ctx, const uint8_t* kinds);

/* Classify heads from per-query-head scores (host, [Hq]): scores are
 * mean-pooled over each GQA group ([AoH] Methodology §4) and the
 * n_retrieval_kv groups ranked first become retrieval heads.  With
 * lower_is_retrieval = 1 the lowest scores win (effective rank, [AoH]
 * Methodology §4); with 0 the highest win (needle calibration, [RTPurbo]
 * Methodology §1).  Equal scores go to the lower head index.  Same ordering
 * rule as hws_set_head_kinds. */
hws_status hws_classify_by_scores(hws_ctx* ctx, const float* q_head_scores,
                                  int32_t n_retrieval_kv, int32_t lower_is_retrieval);

/* Effective rank of every query head's query-key kernel, from frozen
 * weights and no data ([AoH] Methodology §1-§3): M_g = W_K^T W_Q of query
 * head g and its KV head (d_model x d_model); eff_rank = exp of the Shannon
 * entropy of its singular values normalised to sum 1.  A low value marks a
 * concentrated spectrum, i.e. a retrieval head: pass the values (copied to the
 * host) to hws_classify_by_scores with lower_is_retrieval = 1.  Computed in
 * fp64 from the d_head x d_head matrices W_Q W_Q^T and W_K W_K^T.
 * w_q: [num_q_heads][128][d_model] fp32, w_k: [num_kv_heads][128][d_model]
 * fp32 (device, rows are the head's output dims); eff_rank: [num_q_heads]
 * fp32 (device); workspace: hws_effective_rank_workspace() bytes (device).
 * No context is needed.  Asynchronous on `stream`. */
hws_status hws_effective_rank_workspace(int32_t num_q_heads, int32_t num_kv_heads, size_t* bytes);
hws_status hws_effective_rank(int32_t num_q_heads, int32_t num_kv_heads, int32_t d_model,
                              const float* w_q, const float* w_k, float* eff_rank,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Copy the current head kinds into kinds[Hkv] (host). */
hws_status hws_get_head_kinds(const hws_ctx* ctx, uint8_t* kinds);

/* Bind the caller's pools (pointers copied; memory stays caller-owned). */
hws_status hws_bind(hws_ctx* ctx, const hws_buffers* buf);

/* Workspace bytes that hws_decode needs for this batch, length bound, score
 * mode and selection scope (the query scope keeps G selection states and
 * aggregates per retrieval head). */
hws_status hws_workspace_size(const hws_ctx* ctx, int32_t batch, int32_t max_seq_len,
                              int32_t score_mode, int32_t select_scope, size_t* bytes);

/* Append n_tok tokens to each of n_seq sequences: token t of sequence s goes to
 * position start_pos[s] + t, i.e. slot pos % 16 of page
 * block_tables[s][pos / 16].  k, v: [n_seq][n_tok][Hkv][128] bf16, pre-RoPE.
 * With local_ring, local heads write ring slot seq_slots[s] instead (device
 * [n_seq], each in [0, max_seqs), NULL otherwise): the positions below S and
 * the last M positions of the call (the ring layout above), so a sequence
 * must be appended in position order and a later call overwrites the rows
 * that left the window and the slack; a slot out of range skips that
 * sequence's local rows.
 * For each retrieval head the projected key P_h k (fp32, before RoPE) goes to
 * the index pool ([RTPurbo] Methodology §2).  With RoPE on, K is rotated at its
 * position and rounded to bf16 before it is stored.  FP8: when a call writes
 * slot 0 of a page, that page's scale becomes amax/448 over the rows this call
 * writes into it (1.0 if all zero); later appends into the open page keep the
 * scale and saturate at +-448.  The KV cache grows by one row per token
 * ([AoH] Problem statement).  block_tables and start_pos are device arrays;
 * max_blocks_per_seq (from the config) is the row stride of block_tables. */
hws_status hws_append(hws_ctx* ctx, int32_t n_seq, int32_t n_tok, const int32_t* block_tables,
                      const int32_t* start_pos, const int32_t* seq_slots, const void* k, const void* v,
                      void* stream);

/* One decode step ([RTPurbo] Methodology §1: retrieval heads switch to dynamic
 * sparse selection during decoding, local heads use sinks plus a window).
 * Retrieval head h with query heads g: logits l_{g,i} = index_scale (P q_g).(P k_i)
 * (INDEX) or attn_scale q_g.k_i (FULL, rotated vectors); a_i = mean_g
 * softmax_i(l_g); S = top-p set (smallest descending prefix with mass >= p,
 * all ties at the threshold kept) or top-k set (ties at the k-th value by
 * lowest position).  Local head: S = {0..n_sink-1} U {N-window..N-1}.  Then
 * out_g = sum_{i in S} softmax_S(attn_scale q_g.k_i) v_i.  With local_ring
 * the local heads read their rows from ring slot seq_slots[b]; a slot out of
 * range reads no rows (that sequence's local heads output 0 with lse -inf). */
hws_status hws_decode(hws_ctx* ctx, const hws_decode_args* args, void* stream);

/* Largest workspace (hws_workspace_size bytes) hws_decode_noalloc can serve:
 * the size of the library's static device scratch array. */
#define HWS_NOALLOC_SCRATCH_BYTES (32u << 20)

/* hws_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * same step with the same kernels and results, but its workspace is a
 * library-owned static device array of HWS_NOALLOC_SCRATCH_BYTES on each GPU
 * (held by the loaded library until the process ends); args->workspace and
 * args->workspace_bytes are ignored.  A step whose hws_workspace_size exceeds
 * HWS_NOALLOC_SCRATCH_BYTES returns HWS_ERR_CAPACITY (host check, before any
 * HIP call).  The first call on a device looks up that device's copy of the
 * array (with the device current; make one call before capturing a graph).
 * Nothing is allocated, set or synchronised: the step's own kernels reset
 * every counter and state they read, so each call starts clean whatever the
 * previous call left in the array.  Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (two streams, or two host threads)
 * race: the caller must order them on one stream. */
hws_status hws_decode_noalloc(hws_ctx* ctx, const hws_decode_args* args, void* stream);
/* (FULL scoring of an fp8 cache multiplies each page's products of the e4m3
 * codes, widened exactly to bf16, by the page's K scale; it runs in the
 * per-stage kernels, as HWS_LAUNCH_MULTI or AUTO's one-launch selection.) */

/* Dense log-sum-exp of every query head over its whole cache: a diagnostic
 * beside the decode step, not part of it.  lse_full[b][g] = ln sum_{i < N_b}
 * exp(attn_scale q_g . k_i) over every cached row of sequence b (rotated q
 * and k when rope_theta > 0; fp8 rows as stored, code times page scale), for
 * every query head, retrieval and local.  With the decode's lse over the
 * kept set S, exp(lse - lse_full) is the full-dim attention mass that S
 * keeps ([RTPurbo] Main results: retained attention mass; the index mass is
 * hws_decode_args.sel_mass).  q: [B][Hq][128] bf16, block_tables, seq_lens
 * as for hws_decode; lse_full: [B][Hq] fp32 (device); workspace:
 * hws_dense_lse_workspace() bytes.  HWS_ERR_UNSUPPORTED with a local ring
 * that has local heads (their older rows are gone). */
hws_status hws_dense_lse_workspace(const hws_ctx* ctx, int32_t batch, int32_t max_seq_len, size_t* bytes);
hws_status hws_dense_lse(hws_ctx* ctx, int32_t batch, int32_t max_seq_len, const void* q,
                         const int32_t* block_tables, const int32_t* seq_lens, float* lse_full, void* workspace,
                         size_t workspace_bytes, void* stream);

/* One chunked-prefill attention call ([RTPurbo] Methodology §1: during
 * prefill a retrieval head keeps its whole cache while a local head attends
 * to its sinks and window; [AoH] Methodology §4: this fits chunked prefill).
 * For query position i = start_pos[s] + t of sequence s and query head g of
 * KV head h: out = sum_j softmax_j(attn_scale q_g.k_j) v_j over j <= i
 * (retrieval head, or every head with dense = 1) or over j in
 * {0..n_sink-1} U {i-window+1..i}, j <= i (local head); q and k rotated at
 * their positions when rope_theta > 0.  K/V are read from the pages, so the
 * chunk must have been appended first (the cache holds positions
 * 0..start_pos[s]+n_tok-1).  Computed with bf16 MFMA products: logits in
 * fp32 (the rotated query is split into two bf16 parts), softmax weights
 * rounded to bf16 for the weighted sum of V.  FP8 cache: the products run on
 * the e4m3 codes (exact in bf16), logits are then multiplied by the page's
 * K scale and weights by its V scale before that rounding.  A negative
 * start_pos[s] skips that sequence.  With local_ring the local heads read
 * ring slot seq_slots[s] (device [n_seq]; a slot out of range gives that
 * sequence's local heads output 0 and lse -inf), which still holds every
 * row a chunk needs when n_tok <= ring_slack + 1 (HWS_ERR_CAPACITY
 * otherwise).  No workspace. */
typedef struct {
  int32_t n_seq;               /* sequences (host), >= 1                       */
  int32_t n_tok;               /* query positions per sequence (host), >= 1    */
  int32_t dense;               /* 1: every head attends to all of j <= i       */
  const void* q;               /* [n_seq][n_tok][Hq][128] bf16, pre-RoPE       */
  const int32_t* block_tables; /* [n_seq][max_blocks_per_seq]                  */
  const int32_t* start_pos;    /* [n_seq] position of each sequence's first query */
  const int32_t* seq_slots;    /* [n_seq] ring slots (local_ring), else NULL    */
  float* out;                  /* [n_seq][n_tok][Hq][128] fp32                 */
  float* lse;                  /* [n_seq][n_tok][Hq] natural-log LSE, or NULL  */
} hws_prefill_args;
hws_status hws_prefill(hws_ctx* ctx, const hws_prefill_args* args, void* stream);

/* Launch shape of hws_decode.
 *  HWS_LAUNCH_MULTI: one kernel per stage (score, select passes, attend,
 *    merge); no workgroup waits for another.
 *  HWS_LAUNCH_SINGLE: everything after the scoring scan runs as ONE launch
 *    whose workgroups hand results to each other through device memory and
 *    wait for each other (bounded spins); the scan itself runs inside it too,
 *    with each tile's scores in registers, for full-dim scores with G = 4, a
 *    bf16 cache and RoPE off (one 16384-position tile per workgroup) and for
 *    r = 16 index scores with one set per KV head (tiles of 2048 positions,
 *    or 8192 when that needs fewer workgroups than the device holds; G = 8
 *    takes 2048 only).
 *  HWS_LAUNCH_SCAN_SINGLE: the scoring scan as its own kernel, then the rest
 *    as the single launch (the shape HWS_LAUNCH_SINGLE falls back to).
 *  HWS_LAUNCH_SCAN_SELECT: the scoring scan, then the selection alone as one
 *    launch of the single-launch kind, then the attention and merge: with
 *    index scores the attention balanced by kept rows (the selection lists
 *    each head's kept rows; the rows of all heads, kept or sinks + window,
 *    laid end to end with a fixed charge per head, are cut into one equal
 *    segment per resident workgroup, for up to 2048 (sequence, KV head)
 *    pairs), else the per-stage attention.
 *    The grid is sized to what the device holds at once (compute units x
 *    occupancy) and launched as an ordinary dispatch: it relies on this
 *    process having the device's compute units (no CU masking); a kernel
 *    running concurrently on another stream only delays it.  A launch that
 *    cannot make progress ends after about a second per wait (by default;
 *    hws_set_wait_limit) with NaN outputs.  Used when the device supports it and the tiles fit the grid
 *    (one tile per workgroup with the scan inside, else two); otherwise the
 *    decode runs as HWS_LAUNCH_MULTI.
 *  HWS_LAUNCH_COOPERATIVE: HWS_LAUNCH_SINGLE as a cooperative launch, so the
 *    runtime guarantees that all workgroups are resident (costs a few tens of
 *    microseconds of launch latency per call).
 *  HWS_LAUNCH_AUTO (the default): HWS_LAUNCH_SINGLE where the scan runs
 *    inside the launch (full-dim scores; index scores with G <= 4) or where
 *    max_seq_len <= 4096 (short contexts, where launch latency dominates);
 *    otherwise the scoring scan, the one-launch selection (same waits and
 *    time-out; one set per KV head, when its tiles fit the device), the
 *    per-stage attention and merge -- with index scores and at least 64
 *    (sequence, KV head) pairs the attention balanced by kept rows, as in
 *    HWS_LAUNCH_SCAN_SELECT --; otherwise HWS_LAUNCH_MULTI.  (The
 *    single launch without the scan gathers each tile's kept rows in one
 *    workgroup, which loses to the per-stage attention when many rows are
 *    kept or many local-head chunks run beside it.)
 * All shapes select the same token sets; outputs differ only by the fp32
 * rounding order of the attention splits.  Returns HWS_ERR_INVALID_ARG for an
 * unknown mode. */
hws_status hws_set_launch_mode(hws_ctx* ctx, int32_t mode);

/* Time-out of the single launch's hand-off waits (the selection launch of
 * HWS_LAUNCH_AUTO, HWS_LAUNCH_SINGLE and HWS_LAUNCH_COOPERATIVE; the
 * per-stage kernels of HWS_LAUNCH_MULTI never wait).  Not part of the method:
 * a control for callers that want a shorter bound and for tests of the
 * failure path.  A waiting workgroup gives up after max_polls polls of its
 * counter (about a microsecond each; rounded up to a multiple of 256; 0
 * restores the default 2^20, at most 2^24), sets an error word, and every
 * other wait then gives up too; the step still runs to its end and writes
 * NaN into out and lse of every retrieval head whose selection gave up (of
 * every head when the per-stage attention follows the selection).  unreachable != 0 raises every wait's
 * target by one, so each wait gives up: every kernel still exits normally
 * and the next step with unreachable = 0 is correct again (the step resets
 * its own selection state).  Applies to later hws_decode calls on ctx.
 * Returns HWS_ERR_INVALID_ARG for max_polls > 2^24. */
hws_status hws_set_wait_limit(hws_ctx* ctx, uint32_t max_polls, int32_t unreachable);

/* Optional per-stage timing with HIP events on the decode stream.
 * hws_profile_enable(ctx, 1) starts recording one event pair per stage per
 * decode call; hws_profile_read(ctx, ms, calls, n) waits for the recorded
 * events, writes the summed milliseconds of stage i to ms[i] and the number
 * of timed calls to calls[i] for i < n, then clears the record.  The stage
 * names come from hws_profile_stage_name(i) ("" past the last stage):
 * score, select, attend, merge, tail (the single launch that replaces
 * select, attend and merge), fused (the single launch that also does the
 * full-dim scoring scan), prefill, fused_index (the single launch that also
 * does the r = 16 index scan) and attend_balanced (the attention balanced by
 * kept rows, in place of attend). */
hws_status hws_profile_enable(hws_ctx* ctx, int32_t enable);
hws_status hws_profile_read(hws_ctx* ctx, double* ms, int32_t* calls, int32_t n);
const char* hws_profile_stage_name(int32_t i);

/* Optional phase timestamps of the single launches (a profiling aid, off by
 * default): with buf != NULL, thread 0 of workgroup w of every later
 * single-launch decode on ctx writes the device's constant 100 MHz clock
 * (s_memrealtime) at the end of phase k to buf[w * HWS_PHASES + k] (device
 * memory, uint64, max_workgroups * HWS_PHASES entries; workgroups beyond
 * max_workgroups write nothing; a phase a workgroup does not run stays as the
 * caller left it).  Phases: 0 start, 1 scan, 2 log-sum-exp exchange, 3 a_i,
 * 4-6 radix passes 1-3, 7 ties, 8 compaction, 9 attention, 10 merge,
 * 11 local-head chunks.  The attention balanced by kept rows (launch mode
 * HWS_LAUNCH_SCAN_SELECT) stamps 0 start, 1 segment table, 8 row list
 * loaded, 9 rows gathered (the last list of its segment), 10 end.
 * buf = NULL turns it off. */
#define HWS_PHASES 12
hws_status hws_profile_phases(hws_ctx* ctx, uint64_t* buf, int32_t max_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* HWS_H */
