// C ABI of libspkv: argument checks, workspace sizing and launches.
// Every check happens before anything is queued; kernels run on the caller's
// stream and the library allocates nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "spkv.h"
#include "spkv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(SPKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check_cache(const spkv_cache *c) {
    if (!c) return fail(SPKV_E_INVALID, "cache is NULL");
    if (c->dtype != SPKV_F32 && c->dtype != SPKV_BF16)
        return fail(SPKV_E_UNSUPPORTED, "cache dtype %d", c->dtype);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(SPKV_E_UNSUPPORTED, "head_dim %d (64 or 128)", c->head_dim);
    if (c->batch < 1 || c->n_kv < 1 || c->n_kv > 16)
        return fail(SPKV_E_INVALID, "batch %d / n_kv %d (n_kv in 1..16)", c->batch, c->n_kv);
    if ((int64_t)c->batch * c->n_kv > 2048)
        return fail(SPKV_E_UNSUPPORTED, "batch * n_kv = %lld exceeds 2048",
                    (long long)c->batch * c->n_kv);
    if (c->window < 32 || c->window > 1024 || c->window % 32)
        return fail(SPKV_E_UNSUPPORTED, "window %d (multiple of 32 in [32, 1024])", c->window);
    if (!pow2(c->page_size) || c->page_size < 32 || c->page_size > 1024)
        return fail(SPKV_E_UNSUPPORTED, "page_size %d (power of two in [32, 1024])", c->page_size);
    if (c->n_pages < 0 || c->max_pages_per_head < 0)
        return fail(SPKV_E_INVALID, "negative n_pages / max_pages_per_head");
    if ((int64_t)c->max_pages_per_head * c->page_size > INT32_MAX)
        return fail(SPKV_E_INVALID, "max_pages_per_head * page_size overflows int32");
    const void *ptrs[] = {c->k_pages, c->v_pages, c->pos_pages, c->page_table, c->lengths,
                          c->pool_next, c->status, c->ring_k, c->ring_v};
    const char *names[] = {"k_pages", "v_pages", "pos_pages", "page_table", "lengths",
                           "pool_next", "status", "ring_k", "ring_v"};
    for (int i = 0; i < 9; ++i) {
        if (!ptrs[i]) return fail(SPKV_E_INVALID, "cache->%s is NULL", names[i]);
        if (!aligned16(ptrs[i]) && i != 5 && i != 6)
            return fail(SPKV_E_INVALID, "cache->%s is not 16-byte aligned", names[i]);
    }
    if (c->u_pages && !aligned16(c->u_pages)) return fail(SPKV_E_INVALID, "cache->u_pages is not 16-byte aligned");
    return SPKV_OK;
}

int check_ld(int64_t ld, int64_t min_ld, int dtype, const char *what) {
    const int q = dtype == SPKV_BF16 ? 8 : 4;
    if (ld < min_ld) return fail(SPKV_E_INVALID, "%s = %lld < %lld", what, (long long)ld, (long long)min_ld);
    if (ld % q) return fail(SPKV_E_INVALID, "%s = %lld is not a multiple of %d", what, (long long)ld, q);
    return SPKV_OK;
}

// persistent grid for the decode kernel: CUs x resident workgroups per CU
int g_decode_grid = 0;

// Scratch of spkv_decode_attn_noalloc, for callers that cannot allocate
// (code under graph capture, serving loops that forbid it).  Each GPU the
// library runs on holds its own copy until the process ends; host code only
// ever uses the device address hipGetSymbolAddress gives for it.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

__global__ void scratch_zero_kernel(uint4 *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

// Device address of the current device's scratch.  The first call on a
// device looks it up and queues a zero fill of it on `stream` (the decode
// kernel's counters must start at zero; every launch leaves them at zero).
int noalloc_scratch(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SPKV_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        hipLaunchKernelGGL(scratch_zero_kernel, dim3(256), dim3(256), 0, stream, (uint4 *)p,
                           kNoAllocScratchBytes / sizeof(uint4));
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch zero fill");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPKV_OK;
}

}  // namespace

extern "C" {

int spkv_version(void) { return SPKV_VERSION; }

const char *spkv_last_error(void) { return g_err; }

const char *spkv_status_str(int status) {
    switch (status) {
    case SPKV_OK: return "ok";
    case SPKV_E_INVALID: return "invalid argument";
    case SPKV_E_UNSUPPORTED: return "unsupported configuration";
    case SPKV_E_HIP: return "HIP runtime error";
    case SPKV_E_CAPACITY: return "cache capacity exhausted (rows dropped)";
    case SPKV_E_WORKSPACE: return "workspace too small";
    case SPKV_E_ROWS: return "row offsets inconsistent with n_rows / max_rows_per_seq";
    case SPKV_E_TIMEOUT: return "a wait inside a fused decode step ran out";
    default: return "unknown status";
    }
}

// ----------------------------------------------------------------------------
size_t spkv_gate_ws_bytes(const spkv_gate_desc *g, int64_t n_rows) {
    if (!g) return 0;
    return spkv::gate_ws_bytes(g->d_model, g->d_hidden, g->n_kv, g->dtype, n_rows);
}

int spkv_gate(const spkv_gate_desc *g, const void *hidden, int64_t n_rows, int64_t ld_hidden,
              float tau, float *utility, uint8_t *keep, void *ws, size_t ws_bytes, void *stream) {
    if (!g) return fail(SPKV_E_INVALID, "gate descriptor is NULL");
    if (g->dtype != SPKV_F32 && g->dtype != SPKV_BF16)
        return fail(SPKV_E_UNSUPPORTED, "gate dtype %d", g->dtype);
    if (g->d_model < 32 || g->d_model % 32)
        return fail(SPKV_E_UNSUPPORTED, "d_model %d (a positive multiple of 32)", g->d_model);
    if (g->d_hidden < 16 || g->d_hidden > 256 || g->d_hidden % 16)
        return fail(SPKV_E_UNSUPPORTED, "d_hidden %d (multiple of 16 in [16, 256])", g->d_hidden);
    if (g->n_kv < 1 || g->n_kv > 16) return fail(SPKV_E_UNSUPPORTED, "n_kv %d (1..16)", g->n_kv);
    if (!g->w1 || !g->b1 || !g->w2 || !g->b2) return fail(SPKV_E_INVALID, "gate weights NULL");
    if (!aligned16(g->w1)) return fail(SPKV_E_INVALID, "w1 not 16-byte aligned");
    if (n_rows < 0 || n_rows > (int64_t)INT32_MAX) return fail(SPKV_E_INVALID, "n_rows %lld", (long long)n_rows);
    if (n_rows == 0) return SPKV_OK;
    if (!hidden || !keep) return fail(SPKV_E_INVALID, "hidden / keep is NULL");
    if (!aligned16(hidden)) return fail(SPKV_E_INVALID, "hidden not 16-byte aligned");
    if (int r = check_ld(ld_hidden, g->d_model, g->dtype, "ld_hidden")) return r;
    if (std::isnan(tau)) return fail(SPKV_E_INVALID, "tau is NaN");
    const size_t need = spkv::gate_ws_bytes(g->d_model, g->d_hidden, g->n_kv, g->dtype, n_rows);
    if (need && (!ws || ws_bytes < need))
        return fail(SPKV_E_WORKSPACE, "gate workspace %zu < %zu bytes", ws_bytes, need);
    spkv::GateArgs a = {};
    a.d_model = g->d_model;
    a.d_hidden = g->d_hidden;
    a.n_kv = g->n_kv;
    a.dtype = g->dtype;
    a.w1 = g->w1;
    a.b1 = g->b1;
    a.w2 = g->w2;
    a.b2 = g->b2;
    a.hidden = hidden;
    a.n_rows = n_rows;
    a.ld_hidden = ld_hidden;
    a.tau = tau;
    a.utility = utility;
    a.keep = keep;
    a.ws = (float *)ws;
    a.n_split = spkv::gate_split_for(g->d_model, g->dtype, n_rows);
    hipError_t e = spkv::launch_gate(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gate launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
int spkv_gate_sink(const spkv_sink_gate_desc *g, const void *hidden, int64_t n_rows, int64_t ld_hidden, float tau,
                   float *utility, uint8_t *keep, void *stream) {
    if (!g) return fail(SPKV_E_INVALID, "gate descriptor is NULL");
    if (g->dtype != SPKV_BF16) return fail(SPKV_E_UNSUPPORTED, "sink gate dtype %d (bf16 only)", g->dtype);
    if (g->d_model < 64 || g->d_model % 64)
        return fail(SPKV_E_UNSUPPORTED, "d_model %d (a positive multiple of 64)", g->d_model);
    if (g->n_kv < 1 || g->n_kv > 16) return fail(SPKV_E_UNSUPPORTED, "n_kv %d (1..16)", g->n_kv);
    if (g->group != 1 && g->group != 2 && g->group != 4 && g->group != 8)
        return fail(SPKV_E_UNSUPPORTED, "group %d (1, 2, 4 or 8)", g->group);
    if (g->d_key != 16) return fail(SPKV_E_UNSUPPORTED, "d_key %d (16)", g->d_key);
    if (g->n_sinks < 0 || g->n_sinks > 64) return fail(SPKV_E_UNSUPPORTED, "n_sinks %d (0..64)", g->n_sinks);
    if (!g->w || (g->n_sinks && !g->sinks)) return fail(SPKV_E_INVALID, "gate weights NULL");
    if (!aligned16(g->w)) return fail(SPKV_E_INVALID, "w not 16-byte aligned");
    if (n_rows < 0 || n_rows > (int64_t)INT32_MAX) return fail(SPKV_E_INVALID, "n_rows %lld", (long long)n_rows);
    if (n_rows == 0) return SPKV_OK;
    if (!hidden || !keep) return fail(SPKV_E_INVALID, "hidden / keep is NULL");
    if (!aligned16(hidden)) return fail(SPKV_E_INVALID, "hidden not 16-byte aligned");
    if (int r = check_ld(ld_hidden, g->d_model, g->dtype, "ld_hidden")) return r;
    if (std::isnan(tau)) return fail(SPKV_E_INVALID, "tau is NaN");
    spkv::GateArgs a = {};
    a.d_model = g->d_model;
    a.d_hidden = (g->group + 1) * g->d_key;
    a.n_kv = g->n_kv;
    a.dtype = g->dtype;
    a.w1 = g->w;
    a.sinks = g->sinks;
    a.n_sinks = g->n_sinks;
    a.group = g->group;
    a.hidden = hidden;
    a.n_rows = n_rows;
    a.ld_hidden = ld_hidden;
    a.tau = tau;
    a.utility = utility;
    a.keep = keep;
    a.n_split = 1;
    hipError_t e = spkv::launch_sink_gate(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sink gate launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
size_t spkv_compact_ws_bytes(const spkv_cache *c, int32_t n_rows, int32_t max_rows_per_seq) {
    (void)n_rows;
    if (!c || c->page_size < 1 || c->batch < 1 || c->n_kv < 1 || max_rows_per_seq < 0) return 0;
    return spkv::compact_ws_bytes(c->batch, c->n_kv, c->page_size, max_rows_per_seq);
}

int spkv_compact_append(const spkv_cache *c, const uint8_t *keep, const float *utility, const void *k,
                        const void *v,
                        int64_t ld_kv, const int32_t *row_offsets, const int32_t *pos0,
                        int32_t n_rows, int32_t max_rows_per_seq, int32_t flags,
                        int32_t *append_offsets, void *ws, size_t ws_bytes, void *stream) {
    if (int r = check_cache(c)) return r;
    if (flags & ~(SPKV_APPEND_GLOBAL | SPKV_APPEND_WINDOW))
        return fail(SPKV_E_INVALID, "unknown flags 0x%x", flags);
    if (n_rows < 0 || max_rows_per_seq < 0) return fail(SPKV_E_INVALID, "negative n_rows / max_rows");
    if (n_rows == 0 || flags == 0) return SPKV_OK;
    if (max_rows_per_seq == 0) return fail(SPKV_E_INVALID, "max_rows_per_seq is 0 with n_rows > 0");
    if (!k || !v || !row_offsets || !pos0) return fail(SPKV_E_INVALID, "k / v / row_offsets / pos0 NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(SPKV_E_INVALID, "k / v not 16-byte aligned");
    if ((flags & SPKV_APPEND_GLOBAL) && !keep) return fail(SPKV_E_INVALID, "keep is NULL with GLOBAL");
    if ((flags & SPKV_APPEND_GLOBAL) && c->u_pages && !utility)
        return fail(SPKV_E_INVALID, "the cache stores utilities (u_pages) but utility is NULL");
    if (int r = check_ld(ld_kv, (int64_t)c->n_kv * c->head_dim, c->dtype, "ld_kv")) return r;
    const size_t need = spkv::compact_ws_bytes(c->batch, c->n_kv, c->page_size, max_rows_per_seq);
    if (need && (!ws || ws_bytes < need))
        return fail(SPKV_E_WORKSPACE, "compaction workspace %zu < %zu bytes", ws_bytes, need);
    if (need && ((uintptr_t)ws & 15)) return fail(SPKV_E_INVALID, "compaction workspace not 16-byte aligned");
    spkv::CompactArgs a;
    a.c = spkv::make_view(c);
    a.keep = keep;
    a.utility = utility;
    a.k = (const char *)k;
    a.v = (const char *)v;
    a.ld_kv = ld_kv;
    a.row_offsets = row_offsets;
    a.pos0 = pos0;
    a.n_rows = n_rows;
    a.max_rows = max_rows_per_seq;
    a.flags = flags;
    a.append_offsets = append_offsets;
    a.ws = (int32_t *)ws;
    hipError_t e = spkv::launch_compact(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "compaction launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
static int decode_grid() {
    if (g_decode_grid > 0) return g_decode_grid;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 512;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    int per_cu = spkv::decode_blocks_per_cu();
    if (per_cu < 1) per_cu = 1;
    g_decode_grid = cus * per_cu;
    return g_decode_grid;
}

size_t spkv_decode_ws_bytes(const spkv_cache *c, int32_t n_q_heads) {
    if (!c || c->n_kv <= 0 || n_q_heads <= 0) return 0;
    return spkv::decode_ws_bytes(c, n_q_heads, decode_grid(), nullptr);
}

static int decode_attn_impl(const spkv_cache *c, int32_t n_q_heads, const void *q, int64_t ld_q,
                            const int32_t *t, float scale, float *out, float *lse, void *ws,
                            size_t ws_bytes, bool noalloc, void *stream) {
    if (int r = check_cache(c)) return r;
    if (n_q_heads < 1 || n_q_heads % c->n_kv) return fail(SPKV_E_INVALID, "n_q_heads %d vs n_kv %d", n_q_heads, c->n_kv);
    const int G = n_q_heads / c->n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(SPKV_E_UNSUPPORTED, "group size %d (1, 2, 4, 8 or 16)", G);
    if (!q || !t || !out) return fail(SPKV_E_INVALID, "q / t / out NULL");
    if (!aligned16(q)) return fail(SPKV_E_INVALID, "q not 16-byte aligned");
    if (int r = check_ld(ld_q, (int64_t)n_q_heads * c->head_dim, c->dtype, "ld_q")) return r;
    if (!std::isfinite(scale)) return fail(SPKV_E_INVALID, "scale not finite");
    const int grid = decode_grid();
    const size_t need = spkv::decode_ws_bytes(c, n_q_heads, grid, nullptr, 0, 0, noalloc);
    if (noalloc) {
        if (need > kNoAllocScratchBytes)
            return fail(SPKV_E_WORKSPACE, "decode needs %zu bytes of scratch; the built-in scratch holds %zu "
                                          "(use spkv_decode_attn with a workspace)", need, kNoAllocScratchBytes);
        if (need) {
            if (int r = noalloc_scratch((hipStream_t)stream, &ws)) return r;
        }
    } else {
        if (need && (!ws || ws_bytes < need))
            return fail(SPKV_E_WORKSPACE, "decode workspace %zu < %zu bytes", ws_bytes, need);
        if (need && !aligned16(ws)) return fail(SPKV_E_INVALID, "ws not 16-byte aligned");
    }
    spkv::DecodeArgs a = {};
    a.c = spkv::make_view(c);
    a.n_q = n_q_heads;
    a.group = G;
    a.q = (const char *)q;
    a.ld_q = ld_q;
    a.t = t;
    a.scale = scale;
    a.out = out;
    a.lse = lse;
    a.grid = grid;
    spkv::decode_ws_assign(a, c, n_q_heads, grid, 0, 0, noalloc, (char *)ws);
    hipError_t e = spkv::launch_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return SPKV_OK;
}

int spkv_decode_attn(const spkv_cache *c, int32_t n_q_heads, const void *q, int64_t ld_q,
                     const int32_t *t, float scale, float *out, float *lse, void *ws,
                     size_t ws_bytes, void *stream) {
    return decode_attn_impl(c, n_q_heads, q, ld_q, t, scale, out, lse, ws, ws_bytes, false, stream);
}

int spkv_decode_attn_noalloc(const spkv_cache *c, int32_t n_q_heads, const void *q, int64_t ld_q,
                             const int32_t *t, float scale, float *out, float *lse, void *stream) {
    return decode_attn_impl(c, n_q_heads, q, ld_q, t, scale, out, lse, nullptr, 0, true, stream);
}

// ----------------------------------------------------------------------------
// attention steps the gate workgroups give up in the fused step (they spend
// about that long on their gate item before planning)
static const int kFusedShareCut = 10;

size_t spkv_decode_step_ws_bytes(const spkv_cache *c, const spkv_gate_desc *g, int32_t n_q_heads) {
    if (!c || c->n_kv <= 0 || n_q_heads <= 0) return 0;
    return spkv::decode_ws_bytes(c, n_q_heads, decode_grid(), nullptr, g ? g->d_model : 0, g ? g->d_hidden : 0);
}

int spkv_decode_step(const spkv_cache *c, const spkv_gate_desc *g, int32_t n_q_heads, const void *hidden,
                     int64_t ld_hidden, float tau, const void *k, const void *v, int64_t ld_kv, const void *q,
                     int64_t ld_q, const int32_t *t, float scale, float *utility, uint8_t *keep, float *out,
                     float *lse, void *ws, size_t ws_bytes, void *stream) {
    if (int r = check_cache(c)) return r;
    if (!g) {
        // no gate: the new rows go to the ring only (their kept pairs are
        // appended later, e.g. when a gating buffer is flushed)
        if (c->dtype != SPKV_BF16) return fail(SPKV_E_UNSUPPORTED, "a step without gate needs a bf16 cache");
        if (n_q_heads < 1 || n_q_heads % c->n_kv)
            return fail(SPKV_E_INVALID, "n_q_heads %d vs n_kv %d", n_q_heads, c->n_kv);
        const int G = n_q_heads / c->n_kv;
        if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
            return fail(SPKV_E_UNSUPPORTED, "group size %d (1, 2, 4, 8 or 16)", G);
        if (!k || !v || !q || !t || !out) return fail(SPKV_E_INVALID, "k / v / q / t / out NULL");
        if (!aligned16(k) || !aligned16(v) || !aligned16(q)) return fail(SPKV_E_INVALID, "k / v / q not 16-byte aligned");
        if (int r = check_ld(ld_kv, (int64_t)c->n_kv * c->head_dim, c->dtype, "ld_kv")) return r;
        if (int r = check_ld(ld_q, (int64_t)n_q_heads * c->head_dim, c->dtype, "ld_q")) return r;
        if (!std::isfinite(scale)) return fail(SPKV_E_INVALID, "scale not finite");
        const int grid = decode_grid();
        const size_t need = spkv::decode_ws_bytes(c, n_q_heads, grid, nullptr);
        if (!ws || ws_bytes < need) return fail(SPKV_E_WORKSPACE, "decode step workspace %zu < %zu bytes", ws_bytes, need);
        if (!aligned16(ws)) return fail(SPKV_E_INVALID, "ws not 16-byte aligned");
        spkv::DecodeArgs a = {};
        a.c = spkv::make_view(c);
        a.n_q = n_q_heads;
        a.group = G;
        a.q = (const char *)q;
        a.ld_q = ld_q;
        a.t = t;
        a.scale = scale;
        a.out = out;
        a.lse = lse;
        a.grid = grid;
        spkv::decode_ws_assign(a, c, n_q_heads, grid, 0, 0, false, (char *)ws);
        a.k_new = (const char *)k;
        a.v_new = (const char *)v;
        a.ld_new = ld_kv;
        hipError_t e = spkv::launch_decode(a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "decode step launch");
        return SPKV_OK;
    }
    if (g->dtype != c->dtype) return fail(SPKV_E_INVALID, "gate dtype %d differs from the cache's", g->dtype);
    if (g->n_kv != c->n_kv) return fail(SPKV_E_INVALID, "gate n_kv %d vs cache n_kv %d", g->n_kv, c->n_kv);
    if (g->d_model < 32 || g->d_model % 32)
        return fail(SPKV_E_UNSUPPORTED, "d_model %d (a positive multiple of 32)", g->d_model);
    if (g->d_hidden < 16 || g->d_hidden > 256 || g->d_hidden % 16)
        return fail(SPKV_E_UNSUPPORTED, "d_hidden %d (multiple of 16 in [16, 256])", g->d_hidden);
    if (!g->w1 || !g->b1 || !g->w2 || !g->b2) return fail(SPKV_E_INVALID, "gate weights NULL");
    if (!aligned16(g->w1)) return fail(SPKV_E_INVALID, "w1 not 16-byte aligned");
    if (n_q_heads < 1 || n_q_heads % c->n_kv) return fail(SPKV_E_INVALID, "n_q_heads %d vs n_kv %d", n_q_heads, c->n_kv);
    const int G = n_q_heads / c->n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(SPKV_E_UNSUPPORTED, "group size %d (1, 2, 4, 8 or 16)", G);
    const int grid = decode_grid();
    if (!spkv::decode_fused_ok(c, g->d_hidden, grid))
        return fail(SPKV_E_UNSUPPORTED, "fused step needs a bf16 cache and batch <= 16; "
                                        "use spkv_gate, spkv_compact_append and spkv_decode_attn");
    if (!hidden || !k || !v || !q || !t || !keep || !out)
        return fail(SPKV_E_INVALID, "hidden / k / v / q / t / keep / out NULL");
    if (!aligned16(hidden) || !aligned16(k) || !aligned16(v) || !aligned16(q))
        return fail(SPKV_E_INVALID, "hidden / k / v / q not 16-byte aligned");
    if (int r = check_ld(ld_hidden, g->d_model, g->dtype, "ld_hidden")) return r;
    if (int r = check_ld(ld_kv, (int64_t)c->n_kv * c->head_dim, c->dtype, "ld_kv")) return r;
    if (int r = check_ld(ld_q, (int64_t)n_q_heads * c->head_dim, c->dtype, "ld_q")) return r;
    if (std::isnan(tau)) return fail(SPKV_E_INVALID, "tau is NaN");
    if (!std::isfinite(scale)) return fail(SPKV_E_INVALID, "scale not finite");
    const size_t need = spkv::decode_ws_bytes(c, n_q_heads, grid, nullptr, g->d_model, g->d_hidden);
    if (!ws || ws_bytes < need) return fail(SPKV_E_WORKSPACE, "decode step workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned16(ws)) return fail(SPKV_E_INVALID, "ws not 16-byte aligned");
    spkv::DecodeArgs a = {};
    a.c = spkv::make_view(c);
    a.n_q = n_q_heads;
    a.group = G;
    a.q = (const char *)q;
    a.ld_q = ld_q;
    a.t = t;
    a.scale = scale;
    a.out = out;
    a.lse = lse;
    a.grid = grid;
    spkv::decode_ws_assign(a, c, n_q_heads, grid, g->d_model, g->d_hidden, false, (char *)ws);
    a.share_cut = kFusedShareCut;
    a.wait_limit = spkv::g_wait_limit;
    a.gate.d_model = g->d_model;
    a.gate.d_hidden = g->d_hidden;
    a.gate.n_kv = g->n_kv;
    a.gate.dtype = g->dtype;
    a.gate.w1 = g->w1;
    a.gate.b1 = g->b1;
    a.gate.w2 = g->w2;
    a.gate.b2 = g->b2;
    a.gate.hidden = hidden;
    a.gate.n_rows = c->batch;
    a.gate.ld_hidden = ld_hidden;
    a.gate.tau = tau;
    a.gate.utility = utility;
    a.gate.keep = keep;
    a.k_new = (const char *)k;
    a.v_new = (const char *)v;
    a.ld_new = ld_kv;
    hipError_t e = spkv::launch_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode step launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
size_t spkv_prefill_ws_bytes(const spkv_cache *c, int32_t n_q_heads, int32_t n_rows) {
    if (!c) return 0;
    return spkv::prefill_ws_bytes(c, n_q_heads, n_rows);
}

}  // extern "C"

namespace {
struct SoftArgs {
    bool on;
    float tau, beta, c;
};

int prefill_common(const spkv_cache *c, int32_t n_q_heads, int32_t b, const void *q, int64_t ld_q,
                   const void *k, const void *v, int64_t ld_kv, int32_t pos0, int32_t n_rows, float scale,
                   float *out, float *lse, void *ws, size_t ws_bytes, void *stream, SoftArgs soft) {
    if (int r = check_cache(c)) return r;
    if (n_q_heads < 1 || n_q_heads % c->n_kv) return fail(SPKV_E_INVALID, "n_q_heads %d vs n_kv %d", n_q_heads, c->n_kv);
    const int G = n_q_heads / c->n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(SPKV_E_UNSUPPORTED, "group size %d (1, 2, 4, 8 or 16)", G);
    if (b < 0 || b >= c->batch) return fail(SPKV_E_INVALID, "sequence %d of %d", b, c->batch);
    if (pos0 < 0 || n_rows < 0) return fail(SPKV_E_INVALID, "pos0 %d / n_rows %d", pos0, n_rows);
    if (n_rows == 0) return SPKV_OK;
    if ((int64_t)pos0 + n_rows > INT32_MAX) return fail(SPKV_E_INVALID, "positions overflow int32");
    if (!q || !k || !v || !out) return fail(SPKV_E_INVALID, "q / k / v / out NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(SPKV_E_INVALID, "q / k / v not 16-byte aligned");
    if (int r = check_ld(ld_q, (int64_t)n_q_heads * c->head_dim, c->dtype, "ld_q")) return r;
    if (int r = check_ld(ld_kv, (int64_t)c->n_kv * c->head_dim, c->dtype, "ld_kv")) return r;
    if (!std::isfinite(scale)) return fail(SPKV_E_INVALID, "scale not finite");
    const size_t need = spkv::prefill_ws_bytes(c, n_q_heads, n_rows);
    if (need && (!ws || ws_bytes < need))
        return fail(SPKV_E_WORKSPACE, "prefill workspace %zu < %zu bytes", ws_bytes, need);
    spkv::PrefillArgs a;
    a.c = spkv::make_view(c);
    a.n_q = n_q_heads;
    a.group = G;
    a.b = b;
    a.q = (const char *)q;
    a.ld_q = ld_q;
    a.k = (const char *)k;
    a.v = (const char *)v;
    a.ld_kv = ld_kv;
    a.pos0 = pos0;
    a.n_rows = n_rows;
    a.scale = scale;
    a.out = out;
    a.lse = lse;
    a.ws = (char *)ws;
    a.soft = soft.on ? 1 : 0;
    a.soft_tau = soft.tau;
    a.soft_k1 = soft.on ? (float)(1.4426950408889634 / (double)soft.beta) : 0.f;
    a.soft_cs = soft.on ? (float)((double)soft.c / (double)scale) : 0.f;
    hipError_t e = spkv::launch_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return SPKV_OK;
}
}  // namespace

extern "C" {

int spkv_prefill_attn(const spkv_cache *c, int32_t n_q_heads, int32_t b, const void *q, int64_t ld_q,
                      const void *k, const void *v, int64_t ld_kv, int32_t pos0, int32_t n_rows,
                      float scale, float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return prefill_common(c, n_q_heads, b, q, ld_q, k, v, ld_kv, pos0, n_rows, scale, out, lse, ws, ws_bytes,
                          stream, SoftArgs{false, 0.f, 0.f, 0.f});
}

int spkv_prefill_attn_soft(const spkv_cache *c, int32_t n_q_heads, int32_t b, const void *q, int64_t ld_q,
                           const void *k, const void *v, int64_t ld_kv, int32_t pos0, int32_t n_rows,
                           float scale, float tau, float beta, float c_mask, float *out, float *lse, void *ws,
                           size_t ws_bytes, void *stream) {
    if (int r = check_cache(c)) return r;
    if (!c->u_pages) return fail(SPKV_E_INVALID, "soft mask needs stored utilities (cache->u_pages)");
    if (c->dtype != SPKV_BF16) return fail(SPKV_E_UNSUPPORTED, "soft mask needs a bf16 cache");
    if (n_q_heads < 1 || n_q_heads % c->n_kv || n_q_heads / c->n_kv > 16)
        return fail(SPKV_E_UNSUPPORTED, "soft mask: group size must be 1..16");
    if (!std::isfinite(tau) || !(beta > 0.f) || !std::isfinite(beta) || !(c_mask >= 0.f) || !std::isfinite(c_mask))
        return fail(SPKV_E_INVALID, "soft mask: tau finite, beta > 0 and c >= 0 finite");
    if (!std::isfinite(scale) || scale == 0.f) return fail(SPKV_E_INVALID, "scale not finite or zero");
    // the kernel works with log2(e) / beta and c / scale: both must be finite
    if (!std::isfinite((float)(1.4426950408889634 / (double)beta)) ||
        !std::isfinite((float)((double)c_mask / (double)scale)))
        return fail(SPKV_E_INVALID, "soft mask: beta too small or c / scale too large for float");
    return prefill_common(c, n_q_heads, b, q, ld_q, k, v, ld_kv, pos0, n_rows, scale, out, lse, ws, ws_bytes,
                          stream, SoftArgs{true, tau, beta, c_mask});
}

// ----------------------------------------------------------------------------
size_t spkv_rethreshold_ws_bytes(const spkv_cache *src) {
    if (!src) return 0;
    return spkv::rethresh_ws_bytes(src);
}

namespace {
struct Span {
    const char *p;
    size_t n;
};
bool overlap(Span a, Span b) { return a.n && b.n && a.p < b.p + b.n && b.p < a.p + a.n; }
}  // namespace

int spkv_cache_rethreshold(const spkv_cache *src, const spkv_cache *dst, float tau, void *ws, size_t ws_bytes,
                           void *stream) {
    if (int r = check_cache(src)) return r;
    if (int r = check_cache(dst)) return r;
    if (src->batch != dst->batch || src->n_kv != dst->n_kv || src->head_dim != dst->head_dim ||
        src->page_size != dst->page_size || src->dtype != dst->dtype)
        return fail(SPKV_E_INVALID, "src and dst differ in batch, n_kv, head_dim, page_size or dtype");
    if (!src->u_pages) return fail(SPKV_E_INVALID, "src->u_pages is NULL (no stored utilities)");
    if (std::isnan(tau)) return fail(SPKV_E_INVALID, "tau is NaN");
    if (((int64_t)src->max_pages_per_head * src->page_size + 255) / 256 > 65535)
        return fail(SPKV_E_UNSUPPORTED, "src lists may exceed 65535 x 256 entries (max_pages_per_head * page_size)");
    // dst's writes must not reach anything src's lists are read from
    size_t ss[7], ds[7];
    spkv_cache_bytes(src, ss);
    spkv_cache_bytes(dst, ds);
    const size_t su = (size_t)(src->n_pages > 0 ? src->n_pages : 0) * src->page_size * 4;
    const size_t du = (size_t)(dst->n_pages > 0 ? dst->n_pages : 0) * dst->page_size * 4;
    const Span rd[] = {{(const char *)src->k_pages, ss[0]}, {(const char *)src->v_pages, ss[1]},
                       {(const char *)src->pos_pages, ss[2]}, {(const char *)src->page_table, ss[3]},
                       {(const char *)src->lengths, ss[4]}, {(const char *)src->u_pages, su}};
    const Span wr[] = {{(const char *)dst->k_pages, ds[0]}, {(const char *)dst->v_pages, ds[1]},
                       {(const char *)dst->pos_pages, ds[2]}, {(const char *)dst->page_table, ds[3]},
                       {(const char *)dst->lengths, ds[4]}, {(const char *)dst->u_pages, dst->u_pages ? du : 0},
                       {(const char *)dst->pool_next, 4}, {(const char *)dst->status, 4}};
    for (const Span &w : wr)
        for (const Span &r : rd)
            if (overlap(w, r)) return fail(SPKV_E_INVALID, "a dst buffer overlaps a src buffer");
    const size_t need = spkv::rethresh_ws_bytes(src);
    if (!ws || ws_bytes < need) return fail(SPKV_E_WORKSPACE, "re-threshold workspace %zu < %zu bytes", ws_bytes, need);
    spkv::RethreshArgs a;
    a.src = spkv::make_view(src);
    a.dst = spkv::make_view(dst);
    a.tau = tau;
    a.ws = (int32_t *)ws;
    a.max_tiles = 0;
    hipError_t e = spkv::launch_rethresh(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "re-threshold launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
size_t spkv_head_stats_ws_bytes(int64_t n_rows, int32_t n_kv) {
    if (n_rows < 0 || n_kv < 1 || n_kv > 16) return 0;
    return spkv::stats_ws_bytes(n_rows, n_kv);
}

int spkv_head_stats(const float *utility, const uint8_t *keep, int64_t n_rows, int32_t n_kv, double *u_sum,
                    int64_t *n_kept, void *ws, size_t ws_bytes, void *stream) {
    if (n_kv < 1 || n_kv > 16) return fail(SPKV_E_UNSUPPORTED, "n_kv %d (1..16)", n_kv);
    if (n_rows < 0 || n_rows > (int64_t)INT32_MAX) return fail(SPKV_E_INVALID, "n_rows %lld", (long long)n_rows);
    if (n_rows == 0) return SPKV_OK;  // nothing to add
    if (!utility && !keep) return fail(SPKV_E_INVALID, "utility and keep are both NULL");
    if (utility && !u_sum) return fail(SPKV_E_INVALID, "u_sum is NULL with utility given");
    if (keep && !n_kept) return fail(SPKV_E_INVALID, "n_kept is NULL with keep given");
    if ((u_sum && ((uintptr_t)u_sum & 7)) || (n_kept && ((uintptr_t)n_kept & 7)) || (utility && ((uintptr_t)utility & 3)))
        return fail(SPKV_E_INVALID, "u_sum / n_kept not 8-byte or utility not 4-byte aligned");
    const size_t need = spkv::stats_ws_bytes(n_rows, n_kv);
    if (need && (!ws || ws_bytes < need))
        return fail(SPKV_E_WORKSPACE, "statistics workspace %zu < %zu bytes", ws_bytes, need);
    if (need && ((uintptr_t)ws & 7)) return fail(SPKV_E_INVALID, "ws not 8-byte aligned");
    spkv::StatsArgs a = {};
    a.utility = utility;
    a.keep = keep;
    a.n_rows = n_rows;
    a.n_kv = n_kv;
    a.u_sum = u_sum;
    a.n_kept = n_kept;
    a.ws = ws;
    hipError_t e = spkv::launch_stats(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "statistics launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
int spkv_set_wait_limit(int32_t polls) {
    spkv::g_wait_limit = polls >= 0 ? polls : spkv::kDefaultWaitLimit;
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
int spkv_hbm_read(const void *src, size_t bytes, int32_t flags, int32_t grid, void *sink, void *stream) {
    if (bytes == 0) return SPKV_OK;
    if (!src || !sink) return fail(SPKV_E_INVALID, "src / sink NULL");
    if (((uintptr_t)src & 15) || (bytes & 16383))
        return fail(SPKV_E_INVALID, "src not 16-byte aligned or bytes %zu not a multiple of 16384", bytes);
    if ((uintptr_t)sink & 3) return fail(SPKV_E_INVALID, "sink not 4-byte aligned");
    if (flags & ~(SPKV_READ_NONTEMPORAL | SPKV_READ_RUNS)) return fail(SPKV_E_INVALID, "flags 0x%x", flags);
    if (grid < 1 || grid > 65536) return fail(SPKV_E_INVALID, "grid %d (1..65536)", grid);
    hipError_t e = spkv::launch_hbm_read(src, bytes, (flags & SPKV_READ_NONTEMPORAL) != 0, (flags & SPKV_READ_RUNS) != 0,
                                         (uint32_t *)sink, grid, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "streaming-read launch");
    return SPKV_OK;
}

// ----------------------------------------------------------------------------
size_t spkv_cache_bytes(const spkv_cache *c, size_t sizes[7]) {
    if (!c) return 0;
    const size_t es = c->dtype == SPKV_BF16 ? 2 : 4;
    const size_t np = (size_t)(c->n_pages > 0 ? c->n_pages : 0);
    const size_t bg = (size_t)c->batch * c->n_kv;
    size_t s[7];
    s[0] = np * c->page_size * c->head_dim * es;
    s[1] = s[0];
    s[2] = np * c->page_size * 4;
    s[3] = bg * (size_t)c->max_pages_per_head * 4;
    s[4] = bg * 4;
    s[5] = bg * (size_t)c->window * c->head_dim * es;
    s[6] = s[5];
    size_t tot = 0;
    for (int i = 0; i < 7; ++i) {
        tot += s[i];
        if (sizes) sizes[i] = s[i];
    }
    return tot;
}

int spkv_cache_reset(const spkv_cache *c, void *stream) {
    if (int r = check_cache(c)) return r;
    hipError_t e = spkv::launch_cache_reset(spkv::make_view(c), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "reset launch");
    return SPKV_OK;
}

int spkv_cache_check(const spkv_cache *c, void *stream, int32_t *status_bits) {
    if (!c || !c->status) return fail(SPKV_E_INVALID, "cache / status NULL");
    int32_t bits = 0;
    hipError_t e = hipMemcpyAsync(&bits, c->status, sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "status copy");
    e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    if (status_bits) *status_bits = bits;
    if (bits & (SPKV_STATUS_POOL_FULL | SPKV_STATUS_TABLE_FULL))
        return fail(SPKV_E_CAPACITY, "cache status bits 0x%x", bits);
    if (bits & SPKV_STATUS_BAD_ROWS) return fail(SPKV_E_ROWS, "cache status bits 0x%x", bits);
    if (bits & SPKV_STATUS_STEP_TIMEOUT) return fail(SPKV_E_TIMEOUT, "cache status bits 0x%x", bits);
    return SPKV_OK;
}

}  // extern "C"
