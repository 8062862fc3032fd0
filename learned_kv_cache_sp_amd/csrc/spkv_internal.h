// Internal declarations shared by the host API and the HIP kernels of libspkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "spkv.h"

namespace spkv {

// Kernel-side view of an spkv_cache (passed by value to kernels).
struct CacheView {
    int32_t batch, n_kv, head_dim, window, page_size, n_pages, max_pages, dtype;
    int32_t page_shift;  // log2(page_size)
    char *k_pages;
    char *v_pages;
    int32_t *pos_pages;
    int32_t *page_table;
    int32_t *lengths;
    int32_t *pool_next;
    int32_t *status;
    char *ring_k;
    char *ring_v;
    float *u_pages;      // utility of each entry, or NULL
};

inline CacheView make_view(const spkv_cache *c) {
    CacheView v;
    v.batch = c->batch;
    v.n_kv = c->n_kv;
    v.head_dim = c->head_dim;
    v.window = c->window;
    v.page_size = c->page_size;
    v.n_pages = c->n_pages;
    v.max_pages = c->max_pages_per_head;
    v.dtype = c->dtype;
    int s = 0;
    while ((1 << s) < c->page_size) ++s;
    v.page_shift = s;
    v.k_pages = (char *)c->k_pages;
    v.v_pages = (char *)c->v_pages;
    v.pos_pages = c->pos_pages;
    v.page_table = c->page_table;
    v.lengths = c->lengths;
    v.pool_next = c->pool_next;
    v.status = c->status;
    v.ring_k = (char *)c->ring_k;
    v.ring_v = (char *)c->ring_v;
    v.u_pages = c->u_pages;
    return v;
}

inline int elem_bytes(int dtype) { return dtype == SPKV_BF16 ? 2 : 4; }

// ---- storage order of the key and value entries ------------------------------
// A page of P slots (and the ring of one (b, g), w slots) is stored as blocks
// of 32 consecutive slots, each block 32 x head_dim keys followed by nothing
// else (the values live in their own pages, in blocks at the same offsets).
// Within a block:
//   keys   [head_dim / 32][32 rows][32 dims], row p holding slot
//          kv_slot_of_row(p): rows 16t .. 16t+15 are the A operand of the
//          t-th 16 x 16 x 32 MFMA tile of the decode step, so that each
//          16-byte lane load of the tile's operand falls in one contiguous
//          1 KB run (whole 128-byte lines, read once);
//   values [head_dim][32 slots] (transposed), 64 bytes per dimension at bf16:
//          the 16 dimensions of one V^T operand tile are again one 1 KB run.
// Indices are in elements, relative to the page (page * P * head_dim) or the
// ring of (b, g) ((b * n_kv + g) * w * head_dim).
__host__ __device__ inline int kv_row_of_slot(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }
__host__ __device__ inline int kv_slot_of_row(int p) { return 8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3); }
__host__ __device__ inline int64_t kv_k_index(int64_t j, int d, int hd) {
    return (j >> 5) * 32 * hd + (int64_t)((((d >> 5) << 5) + kv_row_of_slot((int)(j & 31))) * 32 + (d & 31));
}
__host__ __device__ inline int64_t kv_v_index(int64_t j, int d, int hd) {
    return (j >> 5) * 32 * hd + (int64_t)d * 32 + (int)(j & 31);
}
// A slot index may also count from the start of the pool (page * P + j) or
// of the ring (bg * w + slot): P and w are multiples of 32.

// ---- streaming-read ceiling ---------------------------------------------------
hipError_t launch_hbm_read(const void *src, size_t bytes, bool nontemporal, bool runs, uint32_t *sink, int grid,
                           hipStream_t s);

// ---- gate ------------------------------------------------------------------
struct GateArgs {
    int32_t d_model, d_hidden, n_kv, dtype;
    const void *w1;
    const float *b1, *w2, *b2;
    const void *hidden;
    int64_t n_rows, ld_hidden;
    float tau;
    float *utility;
    uint8_t *keep;
    float *ws;          // 256-byte header (arrival counter) + partial sums
    int32_t n_split;    // number of slices of d_model (1 = no workspace)
    // sink-attention gate: w1 = [n_kv][(group + 1) * 16][d_model] projections,
    // sinks [n_kv][n_sinks][16]
    const float *sinks;
    int32_t n_sinks, group;
};
size_t gate_ws_bytes(int d_model, int d_hidden, int n_kv, int dtype, int64_t n_rows);
int gate_split_for(int d_model, int dtype, int64_t n_rows);
hipError_t launch_gate(const GateArgs &a, hipStream_t s);
hipError_t launch_sink_gate(const GateArgs &a, hipStream_t s);

// ---- compaction ------------------------------------------------------------
struct CompactArgs {
    CacheView c;
    const uint8_t *keep;
    const float *utility;  // [n_rows, n_kv]; stored into c.u_pages when both are set
    const char *k;
    const char *v;
    int64_t ld_kv;  // elements
    const int32_t *row_offsets;
    const int32_t *pos0;
    int32_t n_rows, max_rows, flags;
    int32_t *append_offsets;
    int32_t *ws;  // large path: per (b, g) tile numbering, look-back status and page claims
};
size_t compact_ws_bytes(int batch, int n_kv, int page_size, int32_t max_rows);
hipError_t launch_compact(const CompactArgs &a, hipStream_t s);

// ---- decode ----------------------------------------------------------------
struct DecodeArgs {
    CacheView c;
    int32_t n_q, group;
    const char *q;
    int64_t ld_q;
    const int32_t *t;
    float scale;
    float *out, *lse;
    // workspace pieces (decode_ws_assign): arrival counters, the fused
    // step's gate sums, split-K partials
    int32_t *cnt;
    float *gshare;
    float *part;
    int32_t grid;       // persistent workgroups
    int32_t max_items;  // partial slots
    // fused step (spkv_decode_step): the gate of the batch's new rows and
    // their append run inside the attention launch
    int32_t share_cut;  // fused step: attention steps fewer for the workgroups that run a gate item
    int32_t wait_limit; // fused step: polls before its finisher's waits give up
    GateArgs gate;      // n_rows = batch; outputs utility / keep
    const char *k_new, *v_new;  // new rows: row b, key head g at + (b*ld_new + g*hd) elements
    int64_t ld_new;
};
// fused_model / fused_hidden: the gate's d_model and d_hidden for spkv_decode_step (0: plain attention);
// fixed_counters: counters laid out for the largest batch * n_kv (spkv_decode_attn_noalloc's scratch)
size_t decode_ws_bytes(const spkv_cache *c, int n_q, int grid, int *max_items_out, int fused_model = 0,
                       int fused_hidden = 0, bool fixed_counters = false);
// points a's workspace pieces into ws (laid out as decode_ws_bytes counts it)
void decode_ws_assign(DecodeArgs &a, const spkv_cache *c, int n_q, int grid, int fused_model, int fused_hidden,
                      bool fixed_counters, char *ws);
bool decode_fused_ok(const spkv_cache *c, int d_hidden, int grid);
int decode_blocks_per_cu();
constexpr int kDefaultWaitLimit = 1 << 20;  // about a second of device-scope polls
extern int g_wait_limit;  // polls before a bounded wait of the fused step gives up
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// ---- prefill ---------------------------------------------------------------
struct PrefillArgs {
    CacheView c;
    int32_t n_q, group, b;
    const char *q;
    int64_t ld_q;
    const char *k, *v;
    int64_t ld_kv;
    int32_t pos0, n_rows;
    float scale;
    float *out, *lse;
    char *ws;
    // soft mode (spkv_prefill_attn_soft): cached keys outside the window get
    // -soft_cs / (1 + 2^((u - soft_tau) * soft_k1)) added to their raw score
    int32_t soft;
    float soft_tau, soft_k1, soft_cs;  // tau, log2(e) / beta, c / scale
};
size_t prefill_ws_bytes(const spkv_cache *c, int n_q, int n_rows);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

hipError_t launch_cache_reset(const CacheView &c, hipStream_t s);

// ---- re-threshold (spkv_cache_rethreshold) ---------------------------------
struct RethreshArgs {
    CacheView src, dst;
    float tau;
    int32_t *ws;        // tile counts/offsets [B*Hkv*max_tiles] + new lengths [B*Hkv]
    int32_t max_tiles;  // tiles of 256 entries in the longest possible list
};
size_t rethresh_ws_bytes(const spkv_cache *src);
hipError_t launch_rethresh(const RethreshArgs &a, hipStream_t s);

// ---- per-head statistics (spkv_head_stats) ---------------------------------
struct StatsArgs {
    const float *utility;   // [n_rows, n_kv] or NULL
    const uint8_t *keep;    // [n_rows, n_kv] or NULL
    int64_t n_rows;
    int32_t n_kv;
    double *u_sum;          // [n_kv], accumulated
    int64_t *n_kept;        // [n_kv], accumulated
    void *ws;
    // set by the launcher
    int *cnt;               // arrival counter (zero between calls)
    double *ws_u;
    int64_t *ws_k;
    int64_t band_rows;      // rows (row path) or elements (vector path) per band
    int32_t n_bands;
};
size_t stats_ws_bytes(int64_t n_rows, int n_kv);
hipError_t launch_stats(const StatsArgs &a, hipStream_t s);

}  // namespace spkv
