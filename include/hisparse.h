/*
 * hisparse.h -- C ABI of the HiSparse swap-in hot path for MI355X (gfx950).
 *
 * What the path computes (per decode step, per layer): every request's top-k
 * token indices from a sparse-attention indexer are resolved against that
 * request's hot cache in HBM.  A hit returns the token's resident device row.
 * Misses are deduplicated (across speculative steps in the multi-step call),
 * given victim slots (LRU for the single-step call, CLOCK for the multi-step
 * call), and their KV entries are copied from pinned host memory into those
 * slots; the token->slot table and the policy state are then committed.  The
 * result is the sparse row (or page) table that decode attention consumes.
 *
 * Sources of the operations (page title, section):
 *   - sglang PR #20343 summary, "Implementation breakdown": the single-step
 *     swap-in kernel with a token->slot hash table, hit/miss handling and an
 *     LRU cache; host memory holds the idle KV ("Features and motivation").
 *   - PR #32162 report "[HiSparse] Support hisparse multi-step swap io
 *     kernel", "Implementation breakdown" items 1-2: multi-step gather/commit
 *     over a [batch, steps, top_k] working set with cross-step miss dedup and
 *     a CLOCK cache; steps limited to 2..4; optional miss_src/miss_dst/
 *     miss_count plan; "Risks and impact": hot_buffer_size up to 32768.
 *   - "SGLang HiSparse" blog, section 2.1: swap_in_selected_pages takes
 *     req_pool_indices, seq_lens, topk_indices and the layer id and returns a
 *     sparse page table; sections 1.3 and 2.3: token indices become a page
 *     load list, a token is found by page plus in-page offset.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless the name ends in "_h" (host).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Swap and reset calls only enqueue work on `stream`: they never allocate
 *     and never synchronise the host.  Calls marked "synchronous" wait for
 *     `stream` to drain.
 *   - Return value: HISPARSE_OK (0) or a negative HISPARSE_E_* code, decided
 *     on the host from scalar arguments only.  Problems only the device can
 *     see (bad indices, a request named twice, page overflow) write -1 to the
 *     affected outputs and OR a HISPARSE_ERR_* bit into the state's sticky
 *     error word (hisparse_get_error_flags).
 *   - A state is used from one stream at a time; the calls that touch it are
 *     ordered by that stream.
 *   - All functions are callable from any host thread; no exceptions cross
 *     the ABI.
 */
#ifndef HISPARSE_H_
#define HISPARSE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side status codes. */
#define HISPARSE_OK 0
#define HISPARSE_E_INVAL (-1)       /* an argument is out of range or NULL */
#define HISPARSE_E_NOMEM (-2)       /* a device or pinned host allocation failed */
#define HISPARSE_E_HIP (-3)         /* a HIP runtime call failed */
#define HISPARSE_E_UNSUPPORTED (-4) /* valid request outside what this library supports */

/* Device-side error bits (sticky; see hisparse_get_error_flags). */
#define HISPARSE_ERR_BAD_INDEX 1u     /* top-k entry outside [0, seq_len), not -1 */
#define HISPARSE_ERR_DUP_REQUEST 2u   /* one request index twice in one batch */
#define HISPARSE_ERR_PAGE_OVERFLOW 4u /* a row needs more distinct pages than hot pages */
#define HISPARSE_ERR_BAD_ROW 8u       /* request index or seq_len out of range */
#define HISPARSE_ERR_BAD_PLAN 16u     /* a replayed plan entry, or a top-k plan entry,
                                         outside the buffers */

/* Replacement policies. */
#define HISPARSE_POLICY_LRU 0   /* single-step calls (PR #20343 summary) */
#define HISPARSE_POLICY_CLOCK 1 /* multi-step calls (PR #32162 report, item 1) */

/* Which misses a multi-step call admits when they outnumber the unpinned
 * slots (PR #32162 report, "Risks and impact": admission is approximate under
 * overflow; the pages name no rule).  Ties go to the first occurrence. */
#define HISPARSE_ADMIT_RECENT 0   /* latest step naming the key first (default) */
#define HISPARSE_ADMIT_FREQUENT 1 /* most steps naming the key first */
#define HISPARSE_ADMIT_FIRST 2    /* first occurrence alone */

/* Limits of this library. */
#define HISPARSE_MAX_HOT 32768        /* hot_buffer_size bound (PR #32162, "Risks and impact") */
#define HISPARSE_MIN_STEPS 2          /* multi-step range (PR #32162, item 2) */
#define HISPARSE_MAX_STEPS 4
#define HISPARSE_MAX_WORKING_SET 8192 /* top_k (x num_steps) entries per row */
#define HISPARSE_MAX_SEQ_LEN ((1 << 28) - 2)
#define HISPARSE_MAX_PAGES_PER_REQUEST (1 << 18)
#define HISPARSE_MAX_BATCH 16000        /* rows of one call (the copy's per-row prefix in LDS) */

typedef struct hisparse_state* hisparse_state_t;

/*
 * Creation parameters (PR #32162 report, "Implementation breakdown" item 2
 * lists the compile-time knobs block_size, num_top_k, hot_buffer_size,
 * item_size_bytes, num_steps, record_miss_plan; here they are runtime fields).
 *
 *   max_requests     R: request pool size; requests are 0..R-1.
 *   num_layers       L: layers; each (request, layer) pair is an independent
 *                    cache instance.
 *   hot_buffer_size  H: hot slots per instance (pages when page_size > 1),
 *                    1..HISPARSE_MAX_HOT.
 *   top_k            K: entries per row and step.  Token LRU needs K <= H.
 *   max_steps        1 for LRU states; 2..4 for CLOCK states (the largest
 *                    num_steps a multi-step call may use).
 *   page_size        P: 1 = token mode; P > 1 = page mode (LRU only), which
 *                    needs max_seq_len % P == 0.
 *   item_size_bytes  I: bytes of one token's KV entry, a multiple of 16 (e.g.
 *                    1152 for a 576-dim bf16 MLA entry, 656 for the fp8 layout).
 *   max_seq_len      N: host tokens per request.
 *   policy           HISPARSE_POLICY_LRU or HISPARSE_POLICY_CLOCK.
 *   max_batch        largest batch of one call, 1..min(R, HISPARSE_MAX_BATCH);
 *                    above HISPARSE_MAX_BATCH: HISPARSE_E_UNSUPPORTED.
 *   host_kv          host array of L pointers; layer l's host KV tier,
 *                    row-major [R][N][I] bytes, in pinned host memory the
 *                    device can read (hisparse_host_alloc or any hipHostMalloc
 *                    buffer).  Owned by the caller; must outlive the state and
 *                    every enqueued call.
 *   dev_kv           host array of L device pointers; layer l's hot KV
 *                    buffer: token mode [R][H + X + E][I] bytes with
 *                    X = max(0, max_steps*K - H) scratch rows for CLOCK states
 *                    (0 for LRU) and E extra rows; page mode [R][H][P][I]
 *                    bytes.  Owned by the caller (for example torch tensors).
 *   admission        HISPARSE_ADMIT_*: which misses of a multi-step call
 *                    take hot slots when they outnumber the unpinned slots
 *                    (CLOCK states; ignored for LRU).  Zero-initialised
 *                    configs get HISPARSE_ADMIT_RECENT.
 *   extra_rows       E >= 0, token mode only: the extra-page lookup (PR
 *                    #32162 report, item 1, before the hash lookup).  Each
 *                    request keeps its newest E tokens on the device in a ring
 *                    of E rows after its hot and scratch rows: token t lives
 *                    in row H + X + t % E, written by the caller's decode, never
 *                    by this library.  A top-k entry t with seq_len - E <= t <
 *                    seq_len resolves to its ring row: no probe, no miss, no
 *                    copy, no change to the cache state.
 */
typedef struct hisparse_config {
  int32_t max_requests;
  int32_t num_layers;
  int32_t hot_buffer_size;
  int32_t top_k;
  int32_t max_steps;
  int32_t page_size;
  int32_t item_size_bytes;
  int32_t max_seq_len;
  int32_t policy;
  int32_t max_batch;
  const void* const* host_kv;
  void* const* dev_kv;
  int32_t admission;
  int32_t extra_rows;
} hisparse_config_t;

/*
 * Optional miss plan written by a swap call (PR #32162 report, item 2 and
 * "Risks and impact": the miss_src / miss_dst / miss_count protocol of the
 * prefetch replay path).  Arrays are device int32 [batch][capacity]; row b's
 * first miss_count[b] entries are written, the rest are left untouched.
 * The protocol's miss_count is the swap call's own `miss_count` output (device
 * int32 [batch]), which hisparse_copy_planned takes beside the plan, so the
 * struct carries no count array of its own.
 *   miss_src  host row copied: r*N + t (token mode) or host page r*(N/P) + p.
 *   miss_dst  device row written: r*(H+X+E) + slot, or r*H + page slot.
 *   victim    key (token or page) evicted from that slot, or -1.
 * capacity must be >= hisparse_plan_capacity(state).
 */
typedef struct hisparse_miss_plan {
  int32_t* miss_src;
  int32_t* miss_dst;
  int32_t* victim;
  int32_t capacity;
  int32_t flags; /* 0 or HISPARSE_PLAN_DEFER_COPY; other bits: HISPARSE_E_INVAL */
} hisparse_miss_plan_t;

/*
 * hisparse_miss_plan_t.flags: the swap call resolves the rows and commits the
 * cache state (outputs, miss_count and the plan are written) but does not
 * copy; the caller enqueues hisparse_copy_planned(layer, batch, miss_count,
 * plan) itself, on any stream ordered after the swap call.  This splits the
 * swap-in into the plan and the IO prefetch/replay of that plan (PR #32162
 * report, "Risks and impact": the miss_src / miss_dst / miss_count protocol
 * of the prefetch path), so that one layer's plan kernel can run while the
 * previous layer's rows are still crossing the host link.  The caller owns
 * the synchronisation the overlap needs (PR #20343 summary, review comments:
 * a missing stream wait under overlapped scheduling crashed with an illegal
 * address):
 *   - nothing may read the layer's hot rows named by the plan (attention, a
 *     copy of the buffer) before that copy has run;
 *   - miss_count and the plan arrays must stay unchanged until it has run;
 *   - copies of one layer must run in the order of their swap calls (a later
 *     call may take as victim a slot an earlier call filled); later swap
 *     calls themselves need no wait, they read and write only cache state.
 */
#define HISPARSE_PLAN_DEFER_COPY 1

/* Accumulated kernel timings (see hisparse_profile_enable). */
typedef struct hisparse_profile {
  int64_t calls;  /* swap calls timed */
  double plan_ms; /* summed duration of the lookup/victim/commit kernel,
                     with its copies when the call copies inside it */
  double copy_ms; /* summed duration of the separate miss-copy kernel */
  int64_t fused_calls; /* calls among them that copied inside the lookup kernel */
} hisparse_profile_t;

/*
 * Device rows per request of a layer's hot KV buffer for `cfg`: H + X + E in
 * token mode, H in page mode (each row then holds P*I bytes).  Returns a
 * negative HISPARSE_E_* code when `cfg` is invalid (E_INVAL for an admission
 * outside HISPARSE_ADMIT_* or extra_rows outside [0, N]; E_UNSUPPORTED for
 * extra_rows > 0 in page mode).
 */
int64_t hisparse_device_rows_per_request(const hisparse_config_t* cfg);

/*
 * Creates a state on the current HIP device: validates `cfg`, allocates the
 * per-instance token->slot table, slot->key table, policy state (LRU order and
 * timestamps, or CLOCK reference bits and hand) and the miss workspace in
 * HBM, and enqueues their initialisation (every cache empty) on `stream`.
 * Synchronous.  On success *out owns the device memory it allocated.
 * Errors: HISPARSE_E_INVAL for a bad field or a host_kv pointer the device
 * cannot read; HISPARSE_E_NOMEM; HISPARSE_E_HIP.
 */
int hisparse_state_create(const hisparse_config_t* cfg, void* stream, hisparse_state_t* out);

/* Frees what the state allocated (not the caller's KV buffers).  The caller
 * must have drained every stream that used the state.  NULL is a no-op. */
void hisparse_state_destroy(hisparse_state_t st);

/*
 * Single-step swap-in of one layer (PR #20343 summary, "Implementation
 * breakdown"; "SGLang HiSparse" blog, section 2.1).  LRU states only.
 *
 *   layer_id          0..L-1.
 *   batch             rows, 0..max_batch (0 is a no-op).
 *   req_pool_indices  int32 [batch]: request of each row.
 *   seq_lens          int32 [batch]: valid token range [0, seq_len) per row.
 *   topk_indices      int32 [batch][K]: token indices; -1 is padding.
 *   out_locs          int32 [batch][K], written:
 *                       token mode: device row r*(H+X+E) + slot of the token,
 *                       or r*(H+X+E) + H + X + t % E for a token t among the
 *                       newest E (extra_rows);
 *                       page mode: j*P + (t mod P), j = index of the token's
 *                       page among the row's distinct pages (ascending);
 *                       -1 for padding, invalid entries and rejected rows.
 *   miss_count        int32 [batch], written: distinct keys (tokens, or pages)
 *                     of the row that were not resident and were copied.
 *   page_table        page mode only (NULL in token mode): int32 [batch][H],
 *                     written: device page row r*H + slot of the j-th distinct
 *                     page, -1 from num_pages[b] on.
 *   num_pages         page mode only: int32 [batch], distinct pages per row.
 *   plan              NULL or a miss plan (see hisparse_miss_plan_t).
 *
 * Ordering rules: misses are placed in first-occurrence order of their
 * tokens (ascending page order in page mode) into victims taken in LRU order
 * (timestamp, slot) with EMPTY slots first; keys of the call are never
 * evicted.  A row whose request is out of range or whose seq_len is outside
 * [0, N] is rejected (ERR_BAD_ROW); a request named by two rows rejects both
 * (ERR_DUP_REQUEST); page mode with more than H distinct pages rejects the row
 * (ERR_PAGE_OVERFLOW); rejected rows leave their cache untouched.
 * Launches: token-mode calls of at least 16 rows copy inside the lookup
 * kernel (each row's workgroup moves its own misses after its commit); page
 * mode and smaller batches add a second, miss-copy kernel.  Either way the
 * copies are complete when the call's work on `stream` is.
 * Errors: HISPARSE_E_INVAL (NULL pointer, range, policy mismatch, plan
 * capacity), HISPARSE_E_HIP.
 */
int hisparse_swap_in_selected(hisparse_state_t st, int32_t layer_id, int32_t batch,
                              const int32_t* req_pool_indices, const int32_t* seq_lens,
                              const int32_t* topk_indices, int32_t* out_locs,
                              int32_t* miss_count, int32_t* page_table, int32_t* num_pages,
                              const hisparse_miss_plan_t* plan, void* stream);

/*
 * Multi-step swap-in of one layer (PR #32162 report, "Implementation
 * breakdown" items 1-2).  CLOCK states only; token mode.
 *
 *   num_steps     S, 2..max_steps.
 *   topk_indices  int32 [batch][S][K]; -1 is padding.
 *   out_locs      int32 [batch][S][K], written: device row of each token, a
 *                 hot slot, on overflow a scratch row r*(H+X+E) + H + j, or
 *                 a ring row r*(H+X+E) + H + X + t % E for the newest E tokens.
 *   miss_count    int32 [batch]: distinct missing tokens over all S steps.
 *   plan          NULL or a miss plan; admitted misses first, then scratch.
 *
 * The S rows of a request form one working set: duplicates across steps
 * resolve to one row and one copy.  Resident keys of the call are pinned;
 * victims come from a CLOCK sweep (reference bit set on hit and insert, hand
 * persists per instance, stops after the last victim).  When the misses
 * exceed the unpinned slots, the misses ranked first by the state's admission
 * priority (default: seen in the latest steps) are admitted and the rest are
 * copied to scratch rows without entering the cache (the
 * pages call this admission approximate; the data of the call stays exact).
 * Row rejection rules, launches and errors as for hisparse_swap_in_selected.
 */
int hisparse_swap_in_spec_multistep(hisparse_state_t st, int32_t layer_id, int32_t batch,
                                    int32_t num_steps, const int32_t* req_pool_indices,
                                    const int32_t* seq_lens, const int32_t* topk_indices,
                                    int32_t* out_locs, int32_t* miss_count,
                                    const hisparse_miss_plan_t* plan, void* stream);

/*
 * Replays a miss plan: for every row b < batch, copies the first
 * min(miss_count[b], plan->capacity) pairs (miss_src, miss_dst) of `plan`
 * from layer `layer_id`'s host tier into its hot KV buffer -- the copy half
 * of a swap call on its own, so a plan recorded by a swap call can be
 * replayed later or on another stream (PR #32162 report, item 2 and "Risks
 * and impact": the plan stays compatible with the prefetch replay path).
 * The victim array and plan->flags are not read; this is the call that
 * completes a swap call made with HISPARSE_PLAN_DEFER_COPY.  Entries outside
 * the layer's host rows
 * ([0, R*N) tokens or [0, R*N/P) pages) or device rows are skipped and raise
 * HISPARSE_ERR_BAD_PLAN.  miss_count: device int32 [batch].  Enqueued on
 * `stream`; errors: HISPARSE_E_INVAL, HISPARSE_E_UNSUPPORTED (batch above
 * HISPARSE_MAX_BATCH), HISPARSE_E_HIP.
 */
int hisparse_copy_planned(hisparse_state_t st, int32_t layer_id, int32_t batch,
                          const int32_t* miss_count, const hisparse_miss_plan_t* plan,
                          void* stream);

/*
 * Sparse MLA decode attention over the rows a swap call returned ("SGLang
 * HiSparse" blog, section 1: attention is exact over the selected positions;
 * section 2.1: the sparse table goes straight to decode attention).  For
 * batch row b and head h, over the valid entries i of locs[b]:
 *   s_i = softmax_scale * (q[b][h][0:512] . c_i + q[b][h][512:576] . r_i)
 *   out[b][h] = sum_i softmax(s)_i * c_i,   lse[b][h] = ln sum_i exp(s_i)
 * where c_i (512-dim latent, also the value) and r_i (64-dim rope key) are
 * decoded from the KV row of location i in layer `layer_id`'s hot buffer.
 * Row formats by item_size_bytes: 1152 = 576 bf16; 656 = 512 fp8 e4m3fn
 * latent, 4 fp32 scales (one per 128 latent dims), 64 bf16 rope.  Other
 * item sizes, and a layer's hot buffer of 2 GiB or more (rows are addressed
 * by 32-bit offsets): HISPARSE_E_UNSUPPORTED.
 *
 *   q           bf16 [batch][num_heads][576] (device).
 *   locs        int32 [batch][n_locs]: token mode, device rows as returned in
 *               out_locs; page mode, j*P + offset with page_table.  -1 entries
 *               are skipped; an entry that resolves outside the buffer is
 *               skipped and raises HISPARSE_ERR_BAD_INDEX.
 *   page_table  page mode only: int32 [batch][H] as returned; NULL otherwise.
 *   out         fp32 [batch][num_heads][512]; a row with no valid entry gets 0.
 *   lse         fp32 [batch][num_heads] (natural log; -inf when empty), or NULL.
 *   workspace   device scratch of at least
 *               hisparse_sparse_mla_workspace_bytes(st, batch, num_heads,
 *               n_locs) bytes (split partials), NULL when that is 0.
 * softmax_scale must be positive and finite (else HISPARSE_E_INVAL).
 * Computes in bf16 MFMA with fp32 accumulation (fp8 latents are dequantised
 * by one fp32 product and rounded to bf16); the softmax weights are rounded
 * to bf16 for the weighted sum, while their normaliser and lse sum the fp32
 * weights.  When the locations are split over several workgroups, each
 * split's normalised output is kept in fp16 (relative 2^-11) until the
 * splits are merged by their log-sum-exp; a 32-dim block whose largest
 * |value| exceeds fp16's range is kept scaled by a power of two, so fp16
 * sets no range limit.  The softmax itself stays exact while |latent| < 2^53.
 * Enqueued on `stream`; allocates nothing.  Errors: HISPARSE_E_INVAL,
 * HISPARSE_E_UNSUPPORTED, HISPARSE_E_HIP.
 */
size_t hisparse_sparse_mla_workspace_bytes(hisparse_state_t st, int32_t batch, int32_t num_heads,
                                           int32_t n_locs);
int hisparse_sparse_mla_decode(hisparse_state_t st, int32_t layer_id, int32_t batch,
                               int32_t num_heads, int32_t n_locs, const void* q,
                               const int32_t* locs, const int32_t* page_table,
                               float softmax_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * ---- Top-k selection fused with the index-table build ----
 * ("SGLang HiSparse" blog, section 2.2: a plan computed once per decode step
 * from the sequence lengths alone, then one kernel per layer that selects
 * the top-k positions from the indexer scores and builds the index table in
 * the same pass; section 2.3: PAGED and RAGGED index tables.)
 *
 * Selection: for row b, the min(k, seq_lens[b]) positions of
 * [0, seq_lens[b]) with the largest logits; equal logits go to the lower
 * position; NaN ranks below every number.  `indices[b]` lists them in
 * ascending position order, then -1 up to k: the top-k input of
 * hisparse_swap_in_selected.  A row with seq_lens[b] < 0 or > max_len gets
 * all -1 and raises HISPARSE_ERR_BAD_ROW.
 * Index table (`locs`, same shape and order):
 *   HISPARSE_INDEX_PAGED   locs = page_table[b][p / page_size] * page_size
 *                          + p % page_size; a position whose page entry is
 *                          negative or at or beyond pt_stride gets -1 and
 *                          raises HISPARSE_ERR_BAD_INDEX;
 *   HISPARSE_INDEX_RAGGED  locs = row_offsets[b] + p;
 *   HISPARSE_INDEX_NONE    locs unused (may be NULL).
 * -1 entries of `indices` give -1 in `locs`.
 */
#define HISPARSE_INDEX_NONE 0
#define HISPARSE_INDEX_PAGED 1
#define HISPARSE_INDEX_RAGGED 2
#define HISPARSE_TOPK_CHUNK 32768            /* positions per workgroup; longer rows are split */
#define HISPARSE_TOPK_MAX_CANDIDATES 32768   /* chunks x k merged per split row */
#define HISPARSE_TOPK_MAX_CHUNKS 64

typedef struct hisparse_topk_call {
  int32_t batch;               /* rows, >= 1 */
  int32_t max_len;             /* logits row length (stride) >= 1 */
  int32_t k;                   /* 1 .. 32768; if max_len > 32768: ceil(max_len / 32768)
                                  <= 64 and ceil(max_len / 32768) * k <= 32768 */
  const float* logits;         /* device fp32 [batch][max_len], caller-owned */
  const int32_t* seq_lens;     /* device int32 [batch] */
  const int32_t* plan;         /* device plan from hisparse_topk_plan for the same
                                  batch, max_len and seq_lens (read only) */
  size_t plan_ints;            /* size of `plan` in int32 */
  int32_t mode;                /* HISPARSE_INDEX_* */
  const int32_t* page_table;   /* PAGED: device int32 [batch][pt_stride] */
  int32_t pt_stride;           /* PAGED: >= 1 */
  int32_t page_size;           /* PAGED: >= 1 */
  const int32_t* row_offsets;  /* RAGGED: device int32 [batch] */
  int32_t* indices;            /* device int32 [batch][k], written */
  int32_t* locs;               /* device int32 [batch][k], written (PAGED/RAGGED) */
  void* workspace;             /* device scratch of hisparse_topk_workspace_bytes
                                  (NULL when that is 0) */
  size_t workspace_bytes;
  uint32_t* error_word;        /* device uint32; HISPARSE_ERR_* bits are OR-ed in */
} hisparse_topk_call_t;

/*
 * Plan of the work split: int32 words needed for `batch` rows of length up
 * to max_len (0 if the sizes are invalid), and the plan itself (device
 * seq_lens in, device plan out: n_items, max_len, per row (first item,
 * n_chunks), per item (row, chunk, start, length)).  A row of s positions is
 * split into n = max(1, ceil(s / 32768)) chunks of 1024 * ceil(ceil(s / n) /
 * 1024) positions (the last shorter); rows outside [0, max_len] get one empty
 * chunk.  The plan depends on seq_lens only: one plan serves every layer of a
 * decode step.  Enqueued on `stream`; allocates nothing.
 * Errors: HISPARSE_E_INVAL (bad sizes, NULL pointers, plan_ints too small),
 * HISPARSE_E_HIP.
 */
size_t hisparse_topk_plan_ints(int32_t batch, int32_t max_len);
int hisparse_topk_plan(int32_t batch, int32_t max_len, const int32_t* seq_lens, int32_t* plan,
                       size_t plan_ints, void* stream);
/*
 * Scratch bytes for hisparse_topk_index_build: 0 when no row can be split
 * (max_len <= 32768), else 8 * k + 4 bytes per plan item for the chunks'
 * candidates.  0 as well for unsupported (max_len, k).
 */
size_t hisparse_topk_workspace_bytes(int32_t batch, int32_t max_len, int32_t k);
/*
 * One layer's selection and index table (see above) on `stream`: one kernel
 * launch, plus a second one that merges the chunks of rows longer than 32768
 * positions; reads each logit once.  Allocates nothing.  A plan entry that
 * lies outside batch, max_len or the plan (a plan made for other sizes) is
 * skipped and raises HISPARSE_ERR_BAD_PLAN; its row's outputs are then not
 * written.
 * Errors: HISPARSE_E_INVAL (NULL pointers, bad sizes or mode, plan or
 * workspace too small), HISPARSE_E_UNSUPPORTED (k or max_len beyond the
 * limits above), HISPARSE_E_HIP.
 */
int hisparse_topk_index_build(const hisparse_topk_call_t* call, void* stream);

/*
 * hisparse_topk_index_build for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same selection and index table, with the split rows'
 * candidates kept in a fixed array the library holds on every device it runs
 * on (HISPARSE_TOPK_STATIC_SCRATCH_BYTES, 16 MiB, for the life of the
 * process) instead of call->workspace, which is ignored along with
 * call->workspace_bytes.  The call allocates nothing; the caller still passes
 * every input and output.  The first call on a device looks the array's
 * address up once (no allocation).  Nothing in the array needs clearing:
 * each call's chunk kernel writes every candidate and count its merge kernel
 * reads.  Every call on one device shares that device's array, so calls that
 * may overlap on one device (on different streams, or from different host
 * threads without stream ordering) race; calls on one stream are ordered.
 * Errors: those of hisparse_topk_index_build, except that a call needing
 * more than HISPARSE_TOPK_STATIC_SCRATCH_BYTES of candidates
 * (hisparse_topk_workspace_bytes) returns HISPARSE_E_UNSUPPORTED before any
 * launch.
 */
#define HISPARSE_TOPK_STATIC_SCRATCH_BYTES (16u << 20)
int hisparse_topk_index_build_noalloc(const hisparse_topk_call_t* call, void* stream);

/*
 * Empties the caches of `n` requests in every layer: a request newly admitted
 * to a pool slot starts from an empty hot cache (sglang PR #20343 summary,
 * "Risks and impact": admit_request_into_staging is where the coordinator
 * admits a request; "Review highlights": the race there was fixed by a stream
 * wait, which is why this call is ordered on the same stream as the swap
 * calls instead of running on a side stream).  req_pool_indices: device int32
 * [n]; out-of-range entries set ERR_BAD_ROW and are skipped.  Enqueued on
 * `stream`; allocates nothing.  Errors: HISPARSE_E_INVAL (NULL state, n < 0,
 * NULL indices with n > 0), HISPARSE_E_HIP.
 */
int hisparse_request_reset(hisparse_state_t st, int32_t n, const int32_t* req_pool_indices,
                           void* stream);

/* Per-row miss capacity a plan must provide: S*K (token mode) or H (page mode). */
int32_t hisparse_plan_capacity(hisparse_state_t st);

/*
 * Copies one instance's state to host memory (the inspection side of the
 * pages' tests, PR #32162 report, "Key files": the correctness test builds a
 * cache index and state up front and checks them after the swap).
 * Synchronous; HISPARSE_E_INVAL for a NULL pointer or (req, layer) out of
 * range, HISPARSE_E_HIP if a copy fails.
 *   slot_key_h  int32 [H]: key held by each slot, -1 if empty.
 *   policy_h    int32 [H]: LRU timestamp of each slot (-1 if empty), or the
 *               CLOCK reference bit (0/1).
 *   ctrl_h      int32 [2]: {LRU call counter, CLOCK hand}.
 *   key_slot_h  NULL or int32 [N] (token mode) / [N/P] (page mode): slot of
 *               every key, -1 if not resident.
 */
int hisparse_state_export(hisparse_state_t st, int32_t req, int32_t layer, int32_t* slot_key_h,
                          int32_t* policy_h, int32_t* ctrl_h, int32_t* key_slot_h, void* stream);

/*
 * Overwrites one instance's state from host memory (same layouts as export):
 * a resident set built up front, as the pages' tests do with
 * _make_cache_index / _make_state (PR #32162 report, "Key files").  The caller
 * fills the matching device KV rows.  Synchronous.  HISPARSE_E_INVAL, with the
 * state unchanged, if a key is out of range or resident twice; for LRU, if the
 * call counter ctrl_h[0] is negative, an occupied slot's timestamp is outside
 * [0, ctrl_h[0]) or an empty slot's is not -1; for CLOCK, if a reference bit
 * is not 0 or 1 or the hand ctrl_h[1] is outside [0, H).
 */
int hisparse_state_import(hisparse_state_t st, int32_t req, int32_t layer,
                          const int32_t* slot_key_h, const int32_t* policy_h,
                          const int32_t* ctrl_h, void* stream);

/* Reads the sticky error word into *flags_h; clears it when `clear` != 0.
 * The word carries the HISPARSE_ERR_* conditions the pages' risk sections
 * name as silent failure modes -- a wrong cache-index mapping (sglang PR
 * #20343 summary, "Risks and impact") shows up as rejected rows and indices
 * instead of wrong rows.  Synchronous; HISPARSE_E_INVAL for a NULL pointer,
 * HISPARSE_E_HIP if the read fails. */
int hisparse_get_error_flags(hisparse_state_t st, uint32_t* flags_h, int32_t clear, void* stream);

/* Static description of a status code. */
const char* hisparse_strerror(int code);

/*
 * Pinned, device-readable host memory for the host KV tier, where the idle KV
 * lives (sglang PR #20343 summary, "Features and motivation"): hipHostMalloc
 * with hipHostMallocMapped and the runtime's default coherence.  *out_h
 * receives the host address, usable directly as a host_kv pointer.  Free with
 * hisparse_host_free.  HISPARSE_E_INVAL for bytes == 0 or a NULL out_h,
 * HISPARSE_E_NOMEM if the allocation fails.
 */
int hisparse_host_alloc(size_t bytes, void** out_h);
int hisparse_host_free(void* p_h);

/*
 * Kernel timing with HIP events recorded on the call's stream around the
 * kernels of every swap call while enabled: the lookup kernel, then the
 * miss-copy kernel (a call that copies inside its lookup kernel, or one made
 * with HISPARSE_PLAN_DEFER_COPY, adds a zero copy interval; a replay by
 * hisparse_copy_planned is not timed).  hisparse_profile_read is
 * synchronous: it waits for the recorded events, returns the sums since the
 * last read and resets them.
 */
int hisparse_profile_enable(hisparse_state_t st, int32_t enable);
int hisparse_profile_read(hisparse_state_t st, hisparse_profile_t* out_h);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H_ */
