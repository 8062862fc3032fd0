/*
 * spkv.h -- C ABI of the SP-KV hot path on MI355X (gfx950).
 *
 * SP-KV ("Self-Pruned Key-Value Attention: learning when to write by
 * predicting future utility", arXiv 2605.14037) gives every (token, key head)
 * a learned utility u = sigmoid(f(h)) (section 2.1, Eq. 1), keeps the pair in
 * a persistent cache only when u >= tau (Eq. 2), and attends over the union
 * of a causal local window of w tokens and the kept pairs (Eq. 3-4).  At
 * deployment the cache holds only the kept pairs and may be built
 * incrementally or chunk by chunk (section 2.1, deployment paragraph); the
 * threshold can be changed after training (section 3.3, threshold paragraph).
 *
 * Four calls implement that path:
 *   spkv_gate            hidden states -> utilities u and keep bits z   (Eq. 1-2)
 *   spkv_compact_append  keep bits + K/V -> order-preserving append to the
 *                        paged per-head cache, and the window ring buffer
 *   spkv_decode_attn     one query per sequence over window + kept pairs (Eq. 3-4)
 *   spkv_prefill_attn    a chunk of queries of one sequence over window + kept
 *                        pairs (Eq. 3-4), for chunked prefill
 * and spkv_decode_step runs gate, append and decode attention of one decode
 * step in a single launch.  spkv_cache_rethreshold rebuilds a cache at a new,
 * higher threshold from the utilities stored with its entries, and
 * spkv_head_stats gives per-head density and mean-utility sums.
 * spkv_prefill_attn_soft is the forward of the soft relaxation of Eq. (5)-(6).
 *
 * Conventions
 *   - Every call returns an int status (SPKV_OK or a negative SPKV_E_*).
 *     Argument checks happen before any launch; on failure nothing is
 *     launched and spkv_last_error() (per thread) holds a message.
 *   - Every device pointer is caller-owned and must stay valid until the work
 *     queued on `stream` completes.  The library allocates no memory and keeps
 *     no state between calls except the per-thread error text and the wait
 *     limit of spkv_set_wait_limit.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     queued; no call synchronises, except spkv_cache_check.
 *   - Device pointers must be 16-byte aligned; row strides (`ld_*`) are in
 *     elements and must be multiples of 8 (bf16) or 4 (f32).
 *   - dtype applies to hidden, W1, Q, K, V and the cache; b1, W2, b2 are f32;
 *     outputs are f32.
 *   - Errors found on the device (capacity, bad row offsets) are recorded as
 *     sticky bits in cache->status and reported by spkv_cache_check.
 */
#ifndef SPKV_H
#define SPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPKV_VERSION 2

enum {
    SPKV_OK = 0,
    SPKV_E_INVALID = -1,     /* null pointer, bad size or stride, misalignment */
    SPKV_E_UNSUPPORTED = -2, /* head_dim, dtype, group size or d_hidden not supported */
    SPKV_E_HIP = -3,         /* a HIP runtime call or launch failed */
    SPKV_E_CAPACITY = -4,    /* device flag: page pool or page table exhausted */
    SPKV_E_WORKSPACE = -5,   /* workspace smaller than the *_ws_bytes figure */
    SPKV_E_ROWS = -6,        /* device flag: row_offsets inconsistent with n_rows / max_rows */
    SPKV_E_TIMEOUT = -7      /* device flag: a wait inside a launch ran out */
};

/* device status bits written by the kernels into cache->status[0] */
enum {
    SPKV_STATUS_POOL_FULL = 1,  /* pool_next ran past n_pages; rows were dropped */
    SPKV_STATUS_TABLE_FULL = 2, /* a head needed more than max_pages_per_head pages */
    SPKV_STATUS_BAD_ROWS = 4,   /* row_offsets not monotone, a sequence longer than max_rows,
                                   or a negative position; that sequence's rows were skipped */
    SPKV_STATUS_STEP_TIMEOUT = 8 /* a wait inside a launch ran out: in spkv_decode_step the
                                   arrivals it waits for did not come (fewer workgroups resident
                                   than it needs) and the step's append or new lengths were not
                                   stored; in spkv_compact_append a tile's predecessor or a page
                                   claim never published (a workspace not at zero) and the
                                   append was dropped */
};

typedef enum { SPKV_F32 = 0, SPKV_BF16 = 1 } spkv_dtype;

enum { SPKV_APPEND_GLOBAL = 1, SPKV_APPEND_WINDOW = 2 };

/*
 * The utility predictor f of Eq. (1): d_model -> d_hidden (ReLU) -> n_kv,
 * one output per key head.
 *   w1 [d_hidden, d_model] dtype (row j = weights of hidden unit j)
 *   b1 [d_hidden] f32, w2 [n_kv, d_hidden] f32, b2 [n_kv] f32
 * Supported: d_hidden in {16, 32, 48, ..., 256}, d_model a multiple of 32,
 * n_kv <= 16.
 */
typedef struct spkv_gate_desc {
    int32_t d_model;
    int32_t d_hidden;
    int32_t n_kv;
    int32_t dtype; /* spkv_dtype */
    const void *w1;
    const float *b1;
    const float *w2;
    const float *b2;
} spkv_gate_desc;

/*
 * One attention layer's SP-KV cache for `batch` sequences.  POD; every
 * pointer is a caller-owned device buffer.
 *
 * Persistent (global) cache, paged per (sequence b, key head g):
 *   k_pages    n_pages x page_size x head_dim keys   (storage order below)
 *   v_pages    n_pages x page_size x head_dim values (storage order below)
 *   pos_pages  [n_pages, page_size] int32       token position of each entry
 *   page_table [batch, n_kv, max_pages_per_head] int32: page id of the i-th
 *              page of (b, g); entry j of (b, g) is slot j % page_size of
 *              page page_table[b][g][j / page_size]
 *   lengths    [batch, n_kv] int32: kept entries appended so far, in token
 *              order (kept entries still inside the window are counted; the
 *              attention calls skip them by position)
 *   pool_next  [1] int32: next free page (device bump allocator)
 *   status     [1] int32: sticky SPKV_STATUS_* bits
 * Window ring of the last `window` tokens of every (b, g):
 *   ring_k     batch x n_kv x window x head_dim keys, slot = position % window
 *   ring_v     batch x n_kv x window x head_dim values (storage order below)
 * Storage order of keys and values: a page (and the ring of one (b, g)) is a
 * run of blocks of 32 consecutive slots, block k holding slots 32k .. 32k+31
 * at element offset 32k * head_dim.  Within a block, the key of slot r,
 * dimension d sits at element
 *     (d / 32) * 1024 + row(r) * 32 + d % 32,
 *     row(r) = 16 * ((r / 4) % 2) + 4 * (r / 8) + r % 4,
 * and its value at element d * 32 + r (transposed).  So the keys of a block
 * are head_dim / 32 tiles of 32 rows x 32 dimensions, each half-tile of 16
 * rows one contiguous 1 KB run at bf16 (the operand of one 16 x 16 x 32 MFMA
 * of the decode kernel), and the values 64 contiguous bytes per dimension.
 * The appends, re-threshold and attention calls all use this order; a
 * caller that reads the buffers itself has to undo it.
 * Optional:
 *   u_pages    [n_pages, page_size] f32 or NULL: the utility u of each entry,
 *              stored by the appends when set (spkv_compact_append needs its
 *              utility argument then); spkv_cache_rethreshold reads it.
 * A fresh cache has lengths = 0, pool_next = 0, status = 0 (spkv_cache_reset).
 * Supported: head_dim in {64, 128}; page_size a power of two in [32, 1024];
 * window a multiple of 32 in [32, 1024].
 */
typedef struct spkv_cache {
    int32_t batch;
    int32_t n_kv;
    int32_t head_dim;
    int32_t window;
    int32_t page_size;
    int32_t n_pages;
    int32_t max_pages_per_head;
    int32_t dtype; /* spkv_dtype */
    void *k_pages;
    void *v_pages;
    int32_t *pos_pages;
    int32_t *page_table;
    int32_t *lengths;
    int32_t *pool_next;
    int32_t *status;
    void *ring_k;
    void *ring_v;
    float *u_pages; /* may be NULL */
} spkv_cache;

/*
 * spkv_gate -- Eq. (1)-(2) for n_rows independent rows (rows may mix
 * sequences and positions).
 *   a = ReLU(W1 h + b1) (kept in f32), logit = W2 a + b2, u = sigmoid(logit),
 *   keep = (u >= tau).  A NaN utility gives keep = 0.
 *   hidden  [n_rows, ld_hidden] dtype (first d_model entries of each row)
 *   utility [n_rows, n_kv] f32, may be NULL;  keep [n_rows, n_kv] uint8
 *   ws      workspace of at least spkv_gate_ws_bytes(g, n_rows) bytes
 *           (may be NULL when that figure is 0).  Its first 256 bytes hold
 *           an arrival counter that must be zero before the first call that
 *           uses ws (zero-fill it once after allocation); every call leaves
 *           it at zero.  Calls sharing one ws must not overlap.
 *   Launches: up to 16 rows, one kernel (one workgroup per hidden unit; the
 *   last to finish adds the per-unit shares of each logit in unit order);
 *   bf16 up to 64 rows, two kernels (d_model split, then the epilogue);
 *   otherwise one kernel.  Results do not depend on scheduling.
 * tau is a runtime argument: the threshold may be changed at inference.
 */
int spkv_gate(const spkv_gate_desc *g, const void *hidden, int64_t n_rows,
              int64_t ld_hidden, float tau, float *utility, uint8_t *keep,
              void *ws, size_t ws_bytes, void *stream);
size_t spkv_gate_ws_bytes(const spkv_gate_desc *g, int64_t n_rows);

/*
 * The sink-attention gate, an alternative predictor f in front of the same
 * keep decision (the gate of Fast KVzip: page "Fast KVzip: efficient and
 * accurate LLM inference with gated KV eviction", section "core method";
 * S = 16 and d_key = 16 in section "reproduction").  The page gives it in
 * words; the reading implemented:
 *   per key head h, with G = group query heads per key head:
 *     q_{h,g} = Wq_{h,g} x (d_key values), k_h = Wk_h x (d_key values),
 *     a_{h,g} = softmax over {k_h, sink_{h,1..S}} of q_{h,g} . key / sqrt(d_key),
 *               taken at k_h (the weight of the token's own key),
 *     u_h = max_g a_{h,g},  keep = (u_h >= tau).
 *   w      [n_kv][(group + 1) * d_key][d_model] dtype: per head the group
 *          query blocks (g-major), then the key block
 *   sinks  [n_kv][n_sinks][d_key] f32
 * Supported: bf16, d_model a multiple of 64, n_kv <= 16, group in
 * {1, 2, 4, 8}, d_key = 16, n_sinks <= 64.
 */
typedef struct spkv_sink_gate_desc {
    int32_t d_model;
    int32_t n_kv;
    int32_t group;
    int32_t d_key;
    int32_t n_sinks;
    int32_t dtype; /* spkv_dtype */
    const void *w;
    const float *sinks;
} spkv_sink_gate_desc;

/*
 * spkv_gate_sink -- the sink-attention gate for n_rows independent rows.
 *   hidden  [n_rows, ld_hidden] bf16 (first d_model entries of each row)
 *   utility [n_rows, n_kv] f32, may be NULL;  keep [n_rows, n_kv] uint8
 * One launch (a workgroup per 256 rows and 1, 2 or 4 key heads: the
 * projections on v_mfma_f32_16x16x32_bf16 accumulate in f32, the sink scores
 * on the f32 MFMA, then the softmax and maximum in f32); no workspace.  A NaN
 * gives keep = 0.
 */
int spkv_gate_sink(const spkv_sink_gate_desc *g, const void *hidden, int64_t n_rows, int64_t ld_hidden,
                   float tau, float *utility, uint8_t *keep, void *stream);

/*
 * spkv_compact_append -- append one batch of rows to the cache.
 *   Rows of sequence b are rows row_offsets[b] .. row_offsets[b+1]-1 of k, v
 *   and keep, at token positions pos0[b], pos0[b]+1, ... (consecutive).
 *   k, v     row r, key head g at  k + r*ld_kv + g*head_dim  (dtype)
 *   keep     [n_rows, n_kv] uint8; read only with SPKV_APPEND_GLOBAL
 *   utility  [n_rows, n_kv] f32 (spkv_gate's output), read only with
 *            SPKV_APPEND_GLOBAL and only when c->u_pages is set, and then
 *            required: the utility of each kept row is stored with its entry.
 *   row_offsets [batch+1], pos0 [batch]: int32 device arrays
 *   max_rows_per_seq: host-side bound on row_offsets[b+1]-row_offsets[b]
 *   flags: SPKV_APPEND_GLOBAL -- for each (b, g), the rows with keep = 1 are
 *            appended in row order (stable compaction): key row, value row and
 *            position copied exactly, lengths[b][g] += count, pages taken from
 *            the pool as needed;
 *          SPKV_APPEND_WINDOW -- every row is written to ring slot
 *            position % window (only the last `window` rows of a sequence
 *            matter and only those are written).
 *   append_offsets [batch, n_kv] int32, may be NULL: receives the length of
 *            each (b, g) before this append.
 *   ws  at least spkv_compact_ws_bytes(...) bytes (0 when max_rows_per_seq
 *       <= 256), 16-byte aligned.  Appends of up to 256 rows per sequence
 *       take one workgroup per (b, g); larger GLOBAL appends run as one
 *       launch of 256-row tiles that find their output offsets from each
 *       other (each tile adds the counts its predecessors publish) and
 *       share new pages through claim words, all kept in ws: it must be
 *       zero-filled once after allocation, every call leaves it at zero, and
 *       calls that share it must not overlap (calls on one stream do not).
 *       Physical page ids then depend on timing; list contents never do.
 * Capacity overflow drops the rows that do not fit and sets a status bit
 * (the list keeps the entries before the first one that did not fit).
 */
int spkv_compact_append(const spkv_cache *c, const uint8_t *keep,
                        const float *utility, const void *k,
                        const void *v, int64_t ld_kv, const int32_t *row_offsets,
                        const int32_t *pos0, int32_t n_rows,
                        int32_t max_rows_per_seq, int32_t flags,
                        int32_t *append_offsets, void *ws, size_t ws_bytes,
                        void *stream);
size_t spkv_compact_ws_bytes(const spkv_cache *c, int32_t n_rows,
                             int32_t max_rows_per_seq);

/*
 * spkv_decode_attn -- one query row per sequence, Eq. (3)-(4).
 *   Query head h of sequence b at position t[b] reads key head g = h / G
 *   (G = n_q_heads / n_kv; contiguous groups) and attends over
 *     window: positions max(0, t-w+1) .. t, read from the ring, and
 *     global: cached entries of (b, g) with position <= t - w.
 *   Preconditions: position t[b] (and the w-1 before it) were WINDOW-appended,
 *   and no entry of (b, g) has a position > t[b] (appends come in token
 *   order), so only the last `window` entries can fall inside the window.
 *   q   [batch, n_q_heads, head_dim] dtype (row b at q + b*ld_q)
 *   t   [batch] int32 device array
 *   out [batch, n_q_heads, head_dim] f32; lse [batch, n_q_heads] f32 or NULL
 *       (natural-log normaliser of each softmax row)
 *   scale: score multiplier (1/sqrt(head_dim) for Eq. 3)
 *   ws  at least spkv_decode_ws_bytes(c, n_q_heads) bytes of scratch
 *       (0 for f32 caches).  Its head holds one arrival counter per (b, g)
 *       and the rest holds split-K partials.  The counters must be zero
 *       before the first call that uses ws (zero-fill it once after
 *       allocation); every call leaves them at zero again.  Calls that share
 *       one ws must not overlap (queue them on one stream).
 *   Launches one kernel.  bf16: a persistent grid (compute units x resident
 *   workgroups) splits the concatenated per-(b, g) key lists evenly; the
 *   last workgroup to finish a (b, g) merges its partials in a fixed order,
 *   so results are deterministic.  f32: one wavefront per (b, query head).
 * Supported: G in {1, 2, 4, 8, 16}.
 */
int spkv_decode_attn(const spkv_cache *c, int32_t n_q_heads, const void *q,
                     int64_t ld_q, const int32_t *t, float scale, float *out,
                     float *lse, void *ws, size_t ws_bytes, void *stream);
size_t spkv_decode_ws_bytes(const spkv_cache *c, int32_t n_q_heads);

/*
 * spkv_decode_attn_noalloc -- spkv_decode_attn without a workspace argument,
 *   for callers that cannot allocate device memory (code under HIP graph
 *   capture, serving loops or harnesses that forbid allocation).  Same
 *   arguments, results and errors as spkv_decode_attn (the same kernel runs;
 *   outputs are bit-identical for the same inputs), but the split-K partials
 *   and arrival counters live in a built-in device array of 4 MiB per GPU,
 *   held from the first call on that GPU until the process ends.  The call
 *   allocates nothing.
 *   Limit: the bf16 path needs 512.5 KiB of counters plus
 *   (compute units + batch * n_kv) * (G * head_dim + 32) * 4 bytes of
 *   partials (about 1.2 MiB for batch 8, 8 key heads, G 4, head_dim 128 on
 *   256 compute units); a cache beyond 4 MiB is refused with
 *   SPKV_E_WORKSPACE before any launch.  f32 caches need no scratch.
 *   The first call on a GPU queues a zero fill of the array on `stream`
 *   ahead of its launch; every launch leaves the counters at zero again.
 *   All calls on one GPU share the array: calls that overlap in time on one
 *   GPU (other streams, other threads) race and give wrong results; queue
 *   them on one stream or order them.
 */
int spkv_decode_attn_noalloc(const spkv_cache *c, int32_t n_q_heads,
                             const void *q, int64_t ld_q, const int32_t *t,
                             float scale, float *out, float *lse,
                             void *stream);

/*
 * spkv_decode_step -- one whole decode step of one layer in one launch:
 *   spkv_gate on the new token's hidden state of every sequence (Eq. 1-2),
 *   spkv_compact_append of its key/value row with
 *   SPKV_APPEND_GLOBAL | SPKV_APPEND_WINDOW at position t[b] (only kept
 *   pairs enter the persistent cache: section 2.1, deployment paragraph),
 *   and spkv_decode_attn of its query at t[b] (Eq. 3-4).
 *   The appended global entries have position t > t - w, so they are not
 *   part of this step's attention (the new row is seen through the window);
 *   the attention plans from the lengths before the step.
 *   Launches one kernel on the resident decode grid: the last workgroup
 *   finishes the gate, appends the kept rows and stores the new lengths once
 *   every other workgroup has read the old ones; it waits for the others'
 *   arrivals (bounded polls: if they never come -- fewer workgroups resident
 *   than the grid, e.g. compute units reserved by another process -- it sets
 *   SPKV_STATUS_STEP_TIMEOUT and leaves the append or lengths undone).
 *   hidden [batch, d_model] dtype (row b at hidden + b*ld_hidden)
 *   k, v   [batch, n_kv, head_dim] dtype (row b at k + b*ld_kv)
 *   q, t, scale, out, lse: as for spkv_decode_attn
 *   utility [batch, n_kv] f32 or NULL; keep [batch, n_kv] uint8.  When
 *       c->u_pages is set, the utility of each appended entry is stored
 *       there whether or not `utility` is given.
 *   ws  at least spkv_decode_step_ws_bytes(c, g, n_q_heads) bytes, zero-filled
 *       once after allocation (a ws of this size also serves
 *       spkv_decode_attn).  Its two step counters only grow, with the totals
 *       they must reach kept beside them, so a call after a step timeout
 *       waits for its own arrivals on top of the late ones of the timed-out
 *       call: the ws needs no new zero fill.  Calls sharing a ws must not
 *       overlap.
 *   Results: utility, keep, the cache contents, lengths and the ring are
 *   those of the three separate calls, bit for bit; out and lse differ from
 *   spkv_decode_attn's only in the rounding of the split-K merge (the keys
 *   are split among workgroups at other points), and are deterministic.
 * Supported: a bf16 cache with batch <= 16, n_kv <= 16, the gate shapes of
 *   spkv_gate, G as for spkv_decode_attn; otherwise
 *   SPKV_E_UNSUPPORTED (make the three calls instead).
 * Capacity overflow drops the row and sets a status bit, and a negative
 * t[b] writes nothing for that sequence and sets SPKV_STATUS_BAD_ROWS, as
 * for spkv_compact_append.
 * g == NULL: no gate and no GLOBAL append -- the step writes the new rows to
 *   the ring (spkv_compact_append(WINDOW)) and attends, for a schedule that
 *   gates buffered hidden states later (Fast KVzip method section, decode
 *   buffer; SP-KV Eq. 4 needs a token in the persistent cache only once it
 *   leaves the window).  hidden, tau, utility and keep are ignored; any
 *   batch size; out and lse are bit-identical to
 *   spkv_compact_append(WINDOW) followed by spkv_decode_attn; ws as for
 *   spkv_decode_attn (spkv_decode_step_ws_bytes(c, NULL, n_q_heads)).
 */
int spkv_decode_step(const spkv_cache *c, const spkv_gate_desc *g,
                     int32_t n_q_heads, const void *hidden, int64_t ld_hidden,
                     float tau, const void *k, const void *v, int64_t ld_kv,
                     const void *q, int64_t ld_q, const int32_t *t,
                     float scale, float *utility, uint8_t *keep, float *out,
                     float *lse, void *ws, size_t ws_bytes, void *stream);
size_t spkv_decode_step_ws_bytes(const spkv_cache *c, const spkv_gate_desc *g,
                                 int32_t n_q_heads);

/*
 * spkv_prefill_attn -- n_rows consecutive query rows of sequence b, Eq. (3)-(4).
 *   Row i is at position t = pos0 + i and attends over
 *     window: positions max(0, t-w+1) .. t, taken from this chunk's k, v for
 *             positions >= pos0 and from the ring for positions < pos0;
 *     global: cached entries of (b, g) with position <= t - w.
 *   Required order for a chunk: spkv_gate -> spkv_compact_append(GLOBAL) ->
 *   spkv_prefill_attn -> spkv_compact_append(WINDOW) (so that the ring still
 *   holds the previous chunk's tail, and kept rows of this chunk are visible
 *   to later rows of the same chunk).
 *   q   row i, head h at q + i*ld_q + h*head_dim; k, v row i, key head g at
 *       k + i*ld_kv + g*head_dim (dtype)
 *   out [n_rows, n_q_heads, head_dim] f32; lse [n_rows, n_q_heads] f32 or NULL
 *   ws  at least spkv_prefill_ws_bytes(c, n_q_heads, n_rows) bytes.
 */
int spkv_prefill_attn(const spkv_cache *c, int32_t n_q_heads, int32_t b,
                      const void *q, int64_t ld_q, const void *k, const void *v,
                      int64_t ld_kv, int32_t pos0, int32_t n_rows, float scale,
                      float *out, float *lse, void *ws, size_t ws_bytes,
                      void *stream);
size_t spkv_prefill_ws_bytes(const spkv_cache *c, int32_t n_q_heads,
                             int32_t n_rows);

/*
 * spkv_prefill_attn_soft -- spkv_prefill_attn with the training-time soft
 *   relaxation of the gate (SP-KV section 2.1, Eq. 5-6) in place of the hard
 *   mask of Eq. (4): every cached entry with position <= t - w takes part
 *   with the additive score c * (alpha - 1), alpha = sigmoid((u - tau) / beta)
 *   from its stored utility u (c->u_pages, required); window keys take part
 *   with no added score.  With every token of the sequence in the cache
 *   (appended with keep = 1 and its utility), this is the attention over all
 *   causal keys with the mask of Eq. (6).  Forward only.
 *   tau (finite), beta > 0 (the pages use 0.01), c_mask >= 0 (the pages use
 *   1e6), with log2(e) / beta and c_mask / scale finite in float; other
 *   arguments and call order as for spkv_prefill_attn.
 *   Utilities must not be NaN.
 * Supported: a bf16 cache, G <= 16.
 */
int spkv_prefill_attn_soft(const spkv_cache *c, int32_t n_q_heads, int32_t b,
                           const void *q, int64_t ld_q, const void *k,
                           const void *v, int64_t ld_kv, int32_t pos0,
                           int32_t n_rows, float scale, float tau, float beta,
                           float c_mask, float *out, float *lse, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * spkv_cache_rethreshold -- rebuild the persistent cache at a new threshold.
 *   SP-KV lets the sparse cache be rebuilt periodically (section 2.1,
 *   deployment paragraph) and its sparsity be moved after training by
 *   changing the threshold (section 3.3, hybrids paragraph).  For every
 *   (b, g), dst's list becomes the entries of src's list whose stored utility
 *   satisfies u >= tau, in the same (token) order, with key, value, position
 *   and utility copied exactly; a NaN utility is dropped.  With tau at or
 *   above the threshold src was built with, the result is the cache that
 *   gating at tau and compacting would have built; entries dropped from src
 *   earlier cannot come back, so a lower tau keeps only what src holds.
 *   src   a cache with u_pages set; read only.
 *   dst   same batch, n_kv, head_dim, page_size and dtype.  Its page tables
 *         and lengths are overwritten; pages are taken from its pool from
 *         dst->pool_next on (reset dst first to reuse its pool), capacity
 *         overflow drops entries and sets bits in dst->status as for
 *         spkv_compact_append.  dst->u_pages may be NULL (the utilities are
 *         then not kept).  The ring is not touched: point dst's ring at
 *         src's, or copy it, before attending over dst.  No buffer dst
 *         writes may overlap a buffer of src.
 *   tau   the new threshold (not NaN).
 *   Supported: src->max_pages_per_head * page_size <= 65535 * 256.
 *   ws    at least spkv_rethreshold_ws_bytes(src) bytes.
 *   Launches three kernels: kept counts per tile of 256 entries, a scan and
 *   page allocation per (b, g), the copies per tile.
 */
int spkv_cache_rethreshold(const spkv_cache *src, const spkv_cache *dst,
                           float tau, void *ws, size_t ws_bytes, void *stream);
size_t spkv_rethreshold_ws_bytes(const spkv_cache *src);

/*
 * spkv_head_stats -- per key head statistics of gate outputs: the measure of
 *   density SP-KV reports (share of the pairs outside the local window that
 *   are kept: Table 1 caption) and the mean learned utility it ranks heads by
 *   to choose the global heads of a local/global hybrid (section 1,
 *   contribution 2; section 4).  For the rows of utility / keep (spkv_gate's
 *   outputs, [n_rows, n_kv]) it adds, for each key head g,
 *     u_sum[g]  += sum over rows of utility[., g]   (double)
 *     n_kept[g] += number of rows with keep[., g] != 0
 *   so that a sequence can be fed in chunks; mean utility = u_sum / rows,
 *   density = n_kept / rows (feed only the rows outside the window for the
 *   density of Table 1).  utility or keep may be NULL (not both; that sum is
 *   then left alone); u_sum, n_kept are device arrays of n_kv entries.  A
 *   NaN utility makes its head's sum NaN.  n_rows = 0 adds nothing and
 *   reads no pointer.
 *   ws  at least spkv_head_stats_ws_bytes(n_rows, n_kv) bytes (8-byte
 *       aligned; 0 when n_rows = 0).  Its first 4352 bytes hold arrival
 *       counters that must be zero before the first call that uses ws
 *       (zero-fill it once after allocation); every call leaves them at
 *       zero.  Calls sharing one ws must not overlap.
 *   Launches one kernel: each workgroup sums a band of rows, the last to
 *   finish adds the band sums in band order.  The sums are deterministic;
 *   they may differ from a sequential sum in the last bits.
 * Supported: n_kv <= 16, n_rows < 2^31.
 */
int spkv_head_stats(const float *utility, const uint8_t *keep, int64_t n_rows,
                    int32_t n_kv, double *u_sum, int64_t *n_kept, void *ws,
                    size_t ws_bytes, void *stream);
size_t spkv_head_stats_ws_bytes(int64_t n_rows, int32_t n_kv);

/* Polls after which the bounded waits inside spkv_decode_step (its
 * finisher's waits for the gate's and the plan's arrivals) give up and set
 * SPKV_STATUS_STEP_TIMEOUT.  polls >= 0 sets the limit (0: the waits give
 * up at once, without polling -- a forced timeout for tests of its
 * handling); a negative value restores the default (2^20 polls, about a
 * second).  Applies to launches queued after the call (process-wide, not
 * synchronised with calls in flight on other threads).  Returns SPKV_OK. */
int spkv_set_wait_limit(int32_t polls);

/* Streaming read of `bytes` bytes at `src` (device memory): the measured
 * bandwidth ceiling that the decode attention kernel is compared with.  It
 * reads every byte once with 16-byte loads and writes nothing (one word of
 * `sink` only in a case that data cannot produce).  It measures the
 * hardware and computes nothing of the method.
 *   flags  SPKV_READ_NONTEMPORAL: loads carry the non-temporal hint;
 *          SPKV_READ_RUNS: each of the grid x 4 waves streams its own
 *          contiguous run of 16 KB blocks (the decode kernel's order);
 *          otherwise every thread steps through the buffer by the whole grid.
 *   grid   workgroups of 256 threads (1..65536).
 *   sink   device word, 4-byte aligned (not read).
 * src must be 16-byte aligned and bytes a multiple of 16384, flags only the
 * two bits above (SPKV_E_INVALID otherwise); bytes = 0 launches nothing. */
enum { SPKV_READ_NONTEMPORAL = 1, SPKV_READ_RUNS = 2 };
int spkv_hbm_read(const void *src, size_t bytes, int32_t flags, int32_t grid, void *sink, void *stream);

/* Sizes in bytes of each cache buffer (k_pages, v_pages, pos_pages,
 * page_table, lengths, ring_k, ring_v) for the dimensions in *c; returns the
 * sum.  `sizes` may be NULL.  u_pages, when used, adds n_pages * page_size
 * * 4 bytes, not included. */
size_t spkv_cache_bytes(const spkv_cache *c, size_t sizes[7]);

/* Queue a reset of lengths, pool_next and status to 0 (page contents are left
 * as they are; they are unreachable once lengths are 0). */
int spkv_cache_reset(const spkv_cache *c, void *stream);

/* Synchronise `stream`, read the sticky status and map it to SPKV_OK,
 * SPKV_E_CAPACITY, SPKV_E_ROWS or SPKV_E_TIMEOUT; *status_bits (may be NULL)
 * receives the bits. */
int spkv_cache_check(const spkv_cache *c, void *stream, int32_t *status_bits);

const char *spkv_status_str(int status);
const char *spkv_last_error(void);
int spkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPKV_H */
