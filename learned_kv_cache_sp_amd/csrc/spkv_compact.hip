// Order-preserving compaction of kept (token, key head) pairs into the paged
// persistent cache, and the window ring write.
//
// SP-KV (arXiv 2605.14037), section 2.1, deployment paragraph: the persistent
// cache holds only the pairs with z = 1 and may be built incrementally or per
// chunk; the local window (Eq. 4, indicator 1_win) is always available.
//
// For each (sequence b, key head g) the kept rows of one append get ranks by
// an exclusive prefix count over the keep bits in row order (wavefront ballot
// + mbcnt inside a tile, a scan over tiles across the sequence), so entry
// lengths[b][g] + rank receives the rank-th kept row: token order is kept no
// matter how the work is spread over workgroups.  Pages come from a device
// bump allocator (one atomic per (b, g) and append); physical page ids may
// differ between runs, the logical content never does.
//
// Layout written: key rows [page][slot][hd] (16-byte coalesced copies), value
// rows transposed [page][hd][slot] (transposed in registers: consecutive
// lanes write consecutive slots), positions [page][slot], and when the cache
// keeps them, utilities [page][slot].
//
// The same file holds the re-threshold of a cache (SP-KV section 2.1,
// deployment paragraph: the cache may be rebuilt from time to time; section
// 3.3, hybrids paragraph: sparsity can be changed after training through the
// threshold): a stable filter of every (b, g) list on its stored utilities,
// ranked the same way and copied page to page.
#include "spkv_internal.h"
#include "spkv_device.h"

namespace spkv {
namespace {

constexpr int NT = 256;     // threads per workgroup
constexpr int TILE = 256;   // rows per tile (one row per thread)

// 16-byte pieces are handled as a native 4 x u32 vector: copies of the
// library's struct-based vector type, or through a local element array, keep
// the loaded pieces in scratch memory instead of registers.
typedef uint32_t piece_t __attribute__((ext_vector_type(4)));

// element i of a piece
template <typename T>
__device__ inline T piece_elem(const piece_t &v, int i) {
    const uint32_t w = v[(i * (int)sizeof(T)) >> 2];
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, w);
    } else {
        static_assert(sizeof(T) == 2, "16- or 32-bit elements");
        return __builtin_bit_cast(T, (uint16_t)(w >> (16 * (i & 1))));
    }
}


__device__ inline int block_rank(bool flag, int *lds_waves, int *total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    __syncthreads();
    if (lane == 0) lds_waves[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int cnt = lds_waves[w];
        before += (w < wave) ? cnt : 0;
        tot += cnt;
    }
    *total = tot;
    return before + rank;
}

// Rows of sequence b; returns false (and flags the cache) when row_offsets
// are inconsistent with n_rows / max_rows.
__device__ inline bool seq_rows(const CompactArgs &a, int b, int *r0, int *nb, bool report) {
    const int lo = a.row_offsets[b];
    const int hi = a.row_offsets[b + 1];
    const int n = hi - lo;
    const int p0 = a.pos0[b];
    if (lo < 0 || n < 0 || n > a.max_rows || hi > a.n_rows || p0 < 0 || p0 > INT32_MAX - n) {
        if (report && threadIdx.x == 0) atomicOr(a.c.status, SPKV_STATUS_BAD_ROWS);
        return false;
    }
    *r0 = lo;
    *nb = n;
    return true;
}

// Take pages so that (b, g) can hold want_len entries; returns the new length
// (clipped when the page table or the pool runs out).  Called by all threads
// of the workgroup; thread 0 does the atomic, everyone writes table entries.
__device__ int grow_head(const CacheView &c, int b, int g, int old_len, int want_len, int *lds) {
    if (threadIdx.x == 0) {
        const int P = c.page_size;
        const int first = (old_len + P - 1) >> c.page_shift;
        int last = (want_len + P - 1) >> c.page_shift;
        int new_len = want_len;
        int bits = 0;
        if (last > c.max_pages) {
            last = c.max_pages;
            new_len = min(new_len, last * P);
            bits |= SPKV_STATUS_TABLE_FULL;
        }
        const int need = last - first;
        int base = 0, granted = 0;
        if (need > 0) {
            base = atomicAdd(c.pool_next, need);
            granted = need;
            if (base + need > c.n_pages) {
                granted = max(0, c.n_pages - base);
                new_len = min(new_len, (first + granted) * P);
                bits |= SPKV_STATUS_POOL_FULL;
            }
        }
        if (bits) atomicOr(c.status, bits);
        lds[0] = max(new_len, old_len);
        lds[1] = first;
        lds[2] = base;
        lds[3] = granted;
    }
    __syncthreads();
    const int first = lds[1], base = lds[2], granted = lds[3];
    int32_t *pt = c.page_table + ((int64_t)b * c.n_kv + g) * c.max_pages;
    for (int i = threadIdx.x; i < granted; i += NT) pt[first + i] = base + i;
    const int new_len = lds[0];
    __syncthreads();
    return new_len;
}

// Copy n rows (source row ids in src_rows[]) of key head g:
//   key rows   -> kdst(kk) (row-major, 16-byte chunks)
//   value rows -> vdst(kk, e) (transposed: one element each)
// Each thread loads KB 16-byte pieces before storing any: the stores could
// alias the sources as far as the compiler knows, so a load-store loop would
// wait for every load in turn.  Values are transposed in registers: the 64
// lanes of a wave take one 16-byte piece of 64 consecutive rows, and each of
// the piece's elements goes to its value row with one store instruction that
// writes consecutive slots.  Ends with a barrier (src_rows may be refilled).
template <typename T, typename KDst, typename VDst>
__device__ void copy_rows(const CompactArgs &a, int g, int n, const int *src_rows, KDst kdst, VDst vdst) {
    constexpr int ES = sizeof(T);
    constexpr int EPC = 16 / ES;   // elements per piece
    constexpr int KB = 8;
    const int hd = a.c.head_dim;
    const int cpr = hd / EPC;      // pieces per row
    const int64_t ld_bytes = a.ld_kv * ES;
    const int np = n * cpr;
    // keys: piece idx = row * cpr + chunk (a row's pieces on neighbouring
    // lanes); values: piece idx = chunk * n + row (consecutive rows on
    // neighbouring lanes).  Both batches are loaded before either is stored.
    for (int base = 0; base < np; base += NT * KB) {
        piece_t kv[KB], vv[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int idx = base + u * NT + (int)threadIdx.x;
            if (idx < np) {
                const int kk = idx / cpr;
                const int ch = idx - kk * cpr;
                kv[u] = *(const piece_t *)(a.k + (int64_t)src_rows[kk] * ld_bytes + (int64_t)g * hd * ES + ch * 16);
                const int vc = idx / n;
                const int vk = idx - vc * n;
                vv[u] = *(const piece_t *)(a.v + (int64_t)src_rows[vk] * ld_bytes + (int64_t)g * hd * ES + vc * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int idx = base + u * NT + (int)threadIdx.x;
            if (idx < np) {
                const int kk = idx / cpr;
                const int ch = idx - kk * cpr;
                *(piece_t *)kdst(kk, ch * EPC) = kv[u];
                const int vc = idx / n;
                const int vk = idx - vc * n;
#pragma unroll
                for (int i = 0; i < EPC; ++i) *vdst(vk, vc * EPC + i) = piece_elem<T>(vv[u], i);
            }
        }
    }
    __syncthreads();
}

// Append the kept rows [row_lo, row_hi) of sequence b, key head g, whose
// first kept row has destination entry dst0 (entries beyond new_len are
// dropped).  Rows are ranked inside the tile.
template <typename T>
__device__ void scatter_tile(const CompactArgs &a, int b, int g, int r0, int row_lo, int row_hi,
                             int dst0, int new_len, int pos_base, int *lds_rows, int *lds_waves,
                             int *lds_pages) {
    const CacheView &c = a.c;
    const int i = row_lo + threadIdx.x;
    const bool flag = (i < row_hi) && a.keep[(int64_t)(r0 + i) * c.n_kv + g] != 0;
    int total;
    const int rank = block_rank(flag, lds_waves, &total);
    if (flag) lds_rows[rank] = r0 + i;
    __syncthreads();
    const int n = max(0, min(total, new_len - dst0));
    if (n == 0) return;
    const int hd = c.head_dim;
    const int P = c.page_size;
    const int32_t *pt = c.page_table + ((int64_t)b * c.n_kv + g) * c.max_pages;
    constexpr int ES = sizeof(T);
    // page ids of the destination entries, read once (the copies below store
    // through char pointers, which may alias the table as far as the
    // compiler knows: a table read per store would wait for every load)
    const int pg0 = dst0 >> c.page_shift;
    const int npg = ((dst0 + n - 1) >> c.page_shift) - pg0 + 1;  // <= TILE / 32 + 1
    if ((int)threadIdx.x < npg) lds_pages[threadIdx.x] = pt[pg0 + threadIdx.x];
    __syncthreads();
    const bool store_u = c.u_pages != nullptr && a.utility != nullptr;
    for (int kk = threadIdx.x; kk < n; kk += NT) {
        const int j = dst0 + kk;
        const int page = lds_pages[(j >> c.page_shift) - pg0];
        const int64_t slot = (int64_t)page * P + (j & (P - 1));
        c.pos_pages[slot] = pos_base + (lds_rows[kk] - r0);
        if (store_u) c.u_pages[slot] = a.utility[(int64_t)lds_rows[kk] * c.n_kv + g];
    }
    auto kdst = [&](int kk, int d) -> char * {
        const int j = dst0 + kk;
        const int page = lds_pages[(j >> c.page_shift) - pg0];
        return c.k_pages + ((int64_t)page * P * hd + kv_k_index(j & (P - 1), d, hd)) * ES;
    };
    auto vdst = [&](int kk, int e) -> T * {
        const int j = dst0 + kk;
        const int page = lds_pages[(j >> c.page_shift) - pg0];
        return (T *)c.v_pages + (int64_t)page * P * hd + kv_v_index(j & (P - 1), e, hd);
    };
    copy_rows<T>(a, g, n, lds_rows, kdst, vdst);
}

// Write rows [row_lo, row_hi) of sequence b (key head g) into the ring.
template <typename T>
__device__ void window_rows(const CompactArgs &a, int b, int g, int r0, int row_lo, int row_hi,
                            int pos_base, int *lds_rows) {
    const CacheView &c = a.c;
    const int hd = c.head_dim;
    const int w = c.window;
    constexpr int ES = sizeof(T);
    const int64_t bg = (int64_t)b * c.n_kv + g;
    // at most TILE rows (lds_rows) at a time; a window may hold up to 1024
    for (int lo = row_lo; lo < row_hi; lo += TILE) {
        const int n = min(TILE, row_hi - lo);
        for (int kk = threadIdx.x; kk < n; kk += NT) lds_rows[kk] = r0 + lo + kk;
        __syncthreads();
        const int first_pos = pos_base + lo;
        auto kdst = [&](int kk, int d) -> char * {
            const int slot = (first_pos + kk) % w;
            return c.ring_k + (bg * w * hd + kv_k_index(slot, d, hd)) * ES;
        };
        auto vdst = [&](int kk, int e) -> T * {
            const int slot = (first_pos + kk) % w;
            return (T *)c.ring_v + bg * w * hd + kv_v_index(slot, e, hd);
        };
        copy_rows<T>(a, g, n, lds_rows, kdst, vdst);  // ends with a barrier
    }
}

// ---------------------------------------------------------------------------
// Small appends (every sequence has at most TILE rows): one workgroup per
// (b, g) does ranking, page allocation and the copies.
template <typename T>
__global__ void __launch_bounds__(NT) compact_small_kernel(CompactArgs a) {
    __shared__ int lds_rows[TILE];
    __shared__ int lds_waves[NT / 64];
    __shared__ int lds_pages[16];
    __shared__ int lds_misc[4];
    const int b = blockIdx.x;
    const int g = blockIdx.y;
    int r0, nb;
    if (!seq_rows(a, b, &r0, &nb, g == 0)) return;
    const int p0 = a.pos0[b];
    const CacheView &c = a.c;
    if (a.flags & SPKV_APPEND_GLOBAL) {
        const int64_t bg = (int64_t)b * c.n_kv + g;
        // count the kept rows first (needed for the page allocation)
        const bool flag = threadIdx.x < nb && a.keep[(int64_t)(r0 + threadIdx.x) * c.n_kv + g] != 0;
        int total;
        (void)block_rank(flag, lds_waves, &total);
        const int old_len = c.lengths[bg];
        const int new_len = grow_head(c, b, g, old_len, old_len + total, lds_misc);
        if (threadIdx.x == 0) {
            c.lengths[bg] = new_len;
            if (a.append_offsets) a.append_offsets[bg] = old_len;
        }
        scatter_tile<T>(a, b, g, r0, 0, nb, old_len, new_len, p0, lds_rows, lds_waves, lds_pages);
    }
    if (a.flags & SPKV_APPEND_WINDOW) {
        __syncthreads();
        window_rows<T>(a, b, g, r0, max(0, nb - c.window), nb, p0, lds_rows);
    }
}

// One row per sequence (decode): one wavefront per (b, g).  Row offsets,
// position, length and the page-table entry of the next slot are read
// together; the key/value row and the keep bit in a second round; then the
// ring and (when kept) the cache entry are written.  A new page costs one
// more round trip (the pool atomic) once every page_size kept rows.
template <typename T>
__global__ void __launch_bounds__(64) compact_row_kernel(CompactArgs a) {
    const CacheView &c = a.c;
    const int b = blockIdx.x;
    const int g = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t bg = (int64_t)b * c.n_kv + g;
    const bool global = (a.flags & SPKV_APPEND_GLOBAL) != 0;
    const int lo = a.row_offsets[b];
    const int hi = a.row_offsets[b + 1];
    const int pos = a.pos0[b];
    const int old_len = global ? c.lengths[bg] : 0;
    int32_t *pt = c.page_table + bg * c.max_pages;
    const int P = c.page_size;
    const int pidx = min(old_len >> c.page_shift, c.max_pages - 1);
    const int cur_page = (global && (old_len & (P - 1)) != 0) ? pt[pidx] : -1;
    const int n = hi - lo;
    if (lo < 0 || n < 0 || n > a.max_rows || hi > a.n_rows || pos < 0 || pos > INT32_MAX - n) {
        if (g == 0 && lane == 0) atomicOr(c.status, SPKV_STATUS_BAD_ROWS);
        return;
    }
    if (global && lane == 0 && a.append_offsets) a.append_offsets[bg] = old_len;
    if (n == 0) return;

    constexpr int ES = sizeof(T);
    constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
    const int hd = c.head_dim;
    const int cpr = hd / EPC;     // chunks per row (<= 32)
    const bool kept = global && a.keep[(int64_t)lo * c.n_kv + g] != 0;
    const bool store_u = global && c.u_pages != nullptr && a.utility != nullptr;
    const float u = store_u ? a.utility[(int64_t)lo * c.n_kv + g] : 0.f;
    const int64_t src = (int64_t)lo * a.ld_kv * ES + (int64_t)g * hd * ES + lane * 16;
    piece_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (lane < cpr) {
        kv = *(const piece_t *)(a.k + src);
        vv = *(const piece_t *)(a.v + src);
    }

    if (a.flags & SPKV_APPEND_WINDOW) {
        const int w = c.window;
        const int slot = pos % w;
        if (lane < cpr) {
            *(piece_t *)(c.ring_k + (bg * w * hd + kv_k_index(slot, lane * EPC, hd)) * ES) = kv;
            T *rv = (T *)c.ring_v + bg * w * hd + kv_v_index(slot, lane * EPC, hd);
#pragma unroll
            for (int e = 0; e < EPC; ++e) rv[32 * e] = piece_elem<T>(vv, e);
        }
    }
    if (!kept) return;
    int page = cur_page;
    if ((old_len & (P - 1)) == 0) {
        // the entry opens a new page
        int got = -1;
        if (lane == 0) {
            const int first = old_len >> c.page_shift;
            if (first >= c.max_pages) {
                atomicOr(c.status, SPKV_STATUS_TABLE_FULL);
            } else {
                const int base = atomicAdd(c.pool_next, 1);
                if (base >= c.n_pages) {
                    atomicOr(c.status, SPKV_STATUS_POOL_FULL);
                } else {
                    pt[first] = base;
                    got = base;
                }
            }
        }
        page = __shfl(got, 0);
        if (page < 0) return;  // dropped: no room
    }
    const int j = old_len & (P - 1);
    if (lane < cpr) {
        *(piece_t *)(c.k_pages + ((int64_t)page * P * hd + kv_k_index(j, lane * EPC, hd)) * ES) = kv;
        T *dv = (T *)c.v_pages + (int64_t)page * P * hd + kv_v_index(j, lane * EPC, hd);
#pragma unroll
        for (int e = 0; e < EPC; ++e) dv[32 * e] = piece_elem<T>(vv, e);
    }
    if (lane == 0) {
        c.pos_pages[(int64_t)page * P + j] = pos;
        if (store_u) c.u_pages[(int64_t)page * P + j] = u;
        c.lengths[bg] = old_len + 1;
    }
}

// ---------------------------------------------------------------------------
// Large appends, one launch.  A workgroup takes one tile of TILE rows of one
// (b, g); tiles of a (b, g) are numbered in the order their workgroups start
// (a counter), so that a tile only ever waits for tiles that are already
// running.  Each tile
//   1. ranks its kept rows (ballot) and publishes its count,
//   2. starts loading the first batch of those rows' key/value pieces,
//   3. finds the count of all tiles before it (decoupled look-back: one
//      wave reads the status of its 64 predecessors at a time, adding counts
//      back to the nearest tile that has published its inclusive prefix)
//      and publishes its own inclusive prefix,
//   4. gets the pages its destination entries fall in: a page already in the
//      list is read from the page table; a new page is claimed by whichever
//      tile touching it gets there first (compare-and-swap on a claim word),
//      which takes an id from the pool and publishes it; the others read it,
//   5. stores the rows, positions and utilities (and ring rows).
// The last workgroup of a (b, g) to finish sets its new length -- cut at the
// first entry whose page could not be had, so the list stays a prefix -- and
// returns the (b, g)'s workspace words to zero.
//
// Workspace per (b, g), int32 words: CH_HDR header words (next tile id,
// arrivals, first dropped entry encoded as INT32_MAX - entry, 0 = none), then
// one status word per tile (0, ST_A | count or ST_P | inclusive count), then
// one claim word per new page (0 free, CLAIMING, NO_PAGE or page id + 1).
constexpr int CH_HDR = 16;
constexpr uint32_t ST_A = 1u << 30, ST_P = 2u << 30, ST_VAL = (1u << 30) - 1;
constexpr int CLAIMING = -1, NO_PAGE = -2;
constexpr int KB = 8;                 // 16-byte pieces per thread and tensor in one batch
constexpr int WAIT_LIMIT = 1 << 20;   // polls before a wait gives up (about a second)

struct OnepassWs {
    int64_t stride;     // int32 words per (b, g)
    int32_t max_tiles, max_claims;
};

__host__ __device__ inline OnepassWs onepass_ws(int32_t max_rows, int page_size) {
    OnepassWs w;
    w.max_tiles = (max_rows + TILE - 1) / TILE;
    w.max_claims = (max_rows + page_size - 1) / page_size + 1;
    w.stride = ((int64_t)CH_HDR + w.max_tiles + w.max_claims + 15) / 16 * 16;
    return w;
}

__device__ inline uint32_t load_st(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_st(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive count of the tiles before t (wave 0).  false if a predecessor
// never published (a workspace not left at zero by the previous call).
__device__ inline bool look_back(const uint32_t *st, int t, int *excl_out) {
    const int lane = threadIdx.x & 63;
    int excl = 0;
    int k = t - 1;
    int polls = 0;
    while (k >= 0) {
        const int idx = k - lane;
        const uint32_t s = idx >= 0 ? load_st(st + idx) : ST_P;  // before tile 0: prefix 0
        const uint32_t kind = s >> 30;
        const uint64_t is_p = __ballot(kind == 2);
        const uint64_t not_ready = __ballot(kind == 0);
        const int last = is_p ? __builtin_ctzll(is_p) : 63;   // lanes 0..last count
        const uint64_t need = last == 63 ? ~0ull : ((2ull << last) - 1);
        if (not_ready & need) {
            if (++polls > WAIT_LIMIT) return false;
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        int v = lane <= last ? (int)(s & ST_VAL) : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        excl += v;
        if (is_p) break;
        k -= 64;
    }
    *excl_out = excl;
    return true;
}

// Page ids of the list pages pg0 .. pg0+npg-1 of (b, g) into lds_pages (-1:
// none could be had).  Wave 0; npg <= 64.  Winners of a claim first take and
// publish their ids, then the others wait: a winner never waits in between,
// so every wait ends.  false if a wait ran out.
__device__ inline bool claim_pages(const CacheView &c, int64_t bg, int pg0, int npg, int first_new,
                                   int32_t *claim, int32_t *hdr, int *lds_pages) {
    const int lane = threadIdx.x & 63;
    const int pidx = pg0 + lane;
    int32_t *pt = c.page_table + bg * c.max_pages;
    int id = -1;
    bool win = false, wait = false;
    int bits = 0;
    if (lane < npg) {
        if (pidx < first_new) {
            id = pt[pidx];                       // the list's last page, partly filled
        } else if (pidx >= c.max_pages) {
            bits = SPKV_STATUS_TABLE_FULL;
        } else {
            const int prev = atomicCAS(claim + (pidx - first_new), 0, CLAIMING);
            win = prev == 0;
            wait = !win;
            if (wait && prev != CLAIMING) {
                id = prev > 0 ? prev - 1 : -1;
                wait = false;
            }
        }
    }
    const uint64_t wins = __ballot(win);
    if (wins) {
        int base = 0;
        if (lane == 0) base = atomicAdd(c.pool_next, __popcll(wins));
        base = __shfl(base, 0);
        if (win) {
            id = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(wins >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)wins, 0u));
            if (id >= c.n_pages) {
                id = -1;
                bits = SPKV_STATUS_POOL_FULL;
                __hip_atomic_store(claim + (pidx - first_new), NO_PAGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                pt[pidx] = id;
                __hip_atomic_store(claim + (pidx - first_new), id + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    bool ok = true;
    if (wait) {
        int polls = 0;
        int v;
        while ((v = __hip_atomic_load(claim + (pidx - first_new), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ==
               CLAIMING) {
            if (++polls > WAIT_LIMIT) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (v == CLAIMING) ok = false;
        id = v > 0 ? v - 1 : -1;
    }
    if (bits) {
        atomicOr(c.status, bits);
        // the entries from this page on cannot be stored: the list ends before it
        atomicMax(hdr + 2, INT32_MAX - pidx * c.page_size);
    }
    if (lane < npg) lds_pages[lane] = id;
    return __ballot(!ok) == 0;
}

// The key/value pieces of kept rows 0 .. nrow-1 (source rows in rows[]),
// spread over threads tid = 0 .. nth-1: keys by piece idx = row * cpr +
// chunk, values by idx = chunk * nrow + row (consecutive rows on
// neighbouring lanes, for the transposed value store).
template <typename T>
__device__ __attribute__((always_inline)) inline void load_batch(const CompactArgs &a, int g, const int *rows,
                                                                   int nrow, piece_t (&kv)[KB], piece_t (&vv)[KB],
                                                                   int tid, int nth) {
    constexpr int ES = sizeof(T);
    const int hd = a.c.head_dim;
    const int cpr = hd * ES / 16;
    const int64_t ld_bytes = a.ld_kv * ES;
    const int64_t goff = (int64_t)g * hd * ES;
    const int np = nrow * cpr;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        const int idx = u * nth + tid;
        if (idx < np) {
            const int kk = idx / cpr, ch = idx - kk * cpr;
            kv[u] = *(const piece_t *)(a.k + rows[kk] * ld_bytes + goff + ch * 16);
            const int vc = idx / nrow, vk = idx - vc * nrow;
            vv[u] = *(const piece_t *)(a.v + rows[vk] * ld_bytes + goff + vc * 16);
        }
    }
}

// Store them to list entries e0 .. e0+nrow-1 (pages in lds_pages, relative to pg0).
template <typename T>
__device__ __attribute__((always_inline)) inline void store_batch(const CacheView &c, int e0, int nrow, int pg0,
                                                                    const int *lds_pages, const piece_t (&kv)[KB],
                                                                    const piece_t (&vv)[KB], int tid, int nth) {
    constexpr int ES = sizeof(T);
    constexpr int EPC = 16 / ES;
    const int hd = c.head_dim;
    const int cpr = hd / EPC;
    const int P = c.page_size;
    const int np = nrow * cpr;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
        const int idx = u * nth + tid;
        if (idx < np) {
            const int kk = idx / cpr, ch = idx - kk * cpr;
            const int jk = e0 + kk;
            const int pk = lds_pages[(jk >> c.page_shift) - pg0];
            if (pk >= 0) *(piece_t *)(c.k_pages + ((int64_t)pk * P * hd + kv_k_index(jk & (P - 1), ch * EPC, hd)) * ES) = kv[u];
            const int vc = idx / nrow, vk = idx - vc * nrow;
            const int jv = e0 + vk;
            const int pv = lds_pages[(jv >> c.page_shift) - pg0];
            if (pv >= 0) {
                T *dv = (T *)c.v_pages + (int64_t)pv * P * hd + kv_v_index(jv & (P - 1), vc * EPC, hd);
#pragma unroll
                for (int i = 0; i < EPC; ++i) dv[32 * i] = piece_elem<T>(vv[u], i);
            }
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(NT) compact_onepass_kernel(CompactArgs a) {
    __shared__ int lds_rows[TILE];
    __shared__ int lds_waves[NT / 64];
    __shared__ int lds_pages[16];
    __shared__ int lds_misc[4];
    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int bg = (int)(blockIdx.x % (uint32_t)BG);
    const int b = bg / c.n_kv, g = bg - b * c.n_kv;
    const OnepassWs W = onepass_ws(a.max_rows, c.page_size);
    int32_t *hdr = a.ws + (int64_t)bg * W.stride;
    uint32_t *st = (uint32_t *)(hdr + CH_HDR);
    int32_t *claim = hdr + CH_HDR + W.max_tiles;
    if (threadIdx.x == 0) lds_misc[0] = arrive_dev(hdr);  // this workgroup's tile
    __syncthreads();
    const int t = lds_misc[0];
    int r0 = 0, nb = 0;
    const bool rows_ok = seq_rows(a, b, &r0, &nb, g == 0 && t == 0);
    const int n_tiles = rows_ok ? (nb + TILE - 1) / TILE : 0;
    const int old_len = c.lengths[bg];
    const int P = c.page_size;
    const int first_new = (old_len + P - 1) >> c.page_shift;
    const bool global = (a.flags & SPKV_APPEND_GLOBAL) != 0;
    if (t < n_tiles) {
        const int row_lo = t * TILE, row_hi = min(nb, row_lo + TILE);
        const int p0 = a.pos0[b];
        if (global) {
            const int i = row_lo + threadIdx.x;
            const bool flag = i < row_hi && a.keep[(int64_t)(r0 + i) * c.n_kv + g] != 0;
            int agg;
            const int rank = block_rank(flag, lds_waves, &agg);
            if (flag) lds_rows[rank] = r0 + i;
            if (threadIdx.x == 0) store_st(st + t, (t == 0 ? ST_P : ST_A) | (uint32_t)agg);
            __syncthreads();
            // the first batch of the kept rows' pieces is loaded by waves 1-3
            // while wave 0 finds the prefix and the pages (its own loads would
            // hold up its polls: loads complete in order)
            const int cpr = c.head_dim * (int)sizeof(T) / 16;
            const int RB1 = (NT - 64) * KB / cpr, RB = NT * KB / cpr;  // rows per batch
            piece_t kv[KB], vv[KB];
            if (threadIdx.x >= 64) load_batch<T>(a, g, lds_rows, min(RB1, agg), kv, vv, threadIdx.x - 64, NT - 64);
            if (threadIdx.x < 64) {
                int excl = 0;
                bool ok = true;
                if (t > 0) {
                    ok = look_back(st, t, &excl);
                    if (threadIdx.x == 0 && ok) store_st(st + t, ST_P | (uint32_t)(excl + agg));
                }
                const int e0 = old_len + excl;
                const int pg0 = e0 >> c.page_shift;
                const int npg = agg ? ((e0 + agg - 1) >> c.page_shift) - pg0 + 1 : 0;
                if (ok && npg) ok = claim_pages(c, bg, pg0, npg, first_new, claim, hdr, lds_pages);
                if (!ok && threadIdx.x == 0) {
                    atomicOr(c.status, SPKV_STATUS_STEP_TIMEOUT);
                    atomicMax(hdr + 2, INT32_MAX - old_len);  // the append is dropped
                }
                if (threadIdx.x == 0) {
                    lds_misc[1] = e0;
                    lds_misc[2] = ok ? agg : 0;
                }
            }
            __syncthreads();
            const int e0 = lds_misc[1], n = lds_misc[2];
            const int pg0 = e0 >> c.page_shift;
            if (n) {
                if (threadIdx.x >= 64)
                    store_batch<T>(c, e0, min(RB1, n), pg0, lds_pages, kv, vv, threadIdx.x - 64, NT - 64);
                for (int rb = RB1; rb < n; rb += RB) {
                    load_batch<T>(a, g, lds_rows + rb, min(RB, n - rb), kv, vv, threadIdx.x, NT);
                    store_batch<T>(c, e0 + rb, min(RB, n - rb), pg0, lds_pages, kv, vv, threadIdx.x, NT);
                }
                const bool store_u = c.u_pages != nullptr && a.utility != nullptr;
                for (int kk = threadIdx.x; kk < n; kk += NT) {
                    const int j = e0 + kk;
                    const int page = lds_pages[(j >> c.page_shift) - pg0];
                    if (page < 0) continue;
                    const int64_t slot = (int64_t)page * P + (j & (P - 1));
                    c.pos_pages[slot] = p0 + (lds_rows[kk] - r0);
                    if (store_u) c.u_pages[slot] = a.utility[(int64_t)lds_rows[kk] * c.n_kv + g];
                }
            }
            __syncthreads();  // lds_rows is reused below
        }
        if (a.flags & SPKV_APPEND_WINDOW) {
            const int w_lo = max(row_lo, nb - c.window);
            if (w_lo < row_hi) window_rows<T>(a, b, g, r0, w_lo, row_hi, p0, lds_rows);
        }
    }
    // arrival: the status and claim words this workgroup wrote are complete
    // (wave 0 wrote them all) before it counts itself in
    if (threadIdx.x == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        lds_misc[3] = arrive_dev(hdr + 1) == W.max_tiles - 1;
    }
    __syncthreads();
    if (!lds_misc[3]) return;
    // the last of the (b, g): new length, then the workspace words back to zero
    if (threadIdx.x == 0) {
        if (global && rows_ok) {
            const int total = n_tiles ? (int)(load_st(st + n_tiles - 1) & ST_VAL) : 0;
            const int enc = load_dev(hdr + 2);
            const int limit = enc ? INT32_MAX - enc : INT32_MAX;
            const int new_len = max(old_len, min(old_len + total, limit));
            c.lengths[bg] = new_len;
            if (a.append_offsets) a.append_offsets[bg] = old_len;
            lds_misc[1] = min(W.max_claims, max(0, ((old_len + total + P - 1) >> c.page_shift) - first_new));
        } else {
            lds_misc[1] = 0;
        }
    }
    __syncthreads();
    const int n_claims = lds_misc[1];
    for (int i = threadIdx.x; i < n_tiles; i += NT) store_st(st + i, 0u);
    for (int i = threadIdx.x; i < n_claims; i += NT) reset_dev(claim + i);
    if (threadIdx.x < 3) reset_dev(hdr + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Re-threshold: src list of (b, g) -> dst list of the entries with u >= tau.
// Entry e of a list is slot e % P of page page_table[b][g][e / P]; tiles are
// 256 consecutive entries (one per thread).

// Entries of the (b, g) list, clipped to what its page table can address.
__device__ inline int list_len(const CacheView &c, int64_t bg) {
    return min(max(c.lengths[bg], 0), c.max_pages * c.page_size);
}

// Stored utility of entry e of (b, g) passes tau (NaN fails).  Returns the
// flat slot (page * P + e % P) through *slot.
__device__ inline bool passes(const RethreshArgs &a, int64_t bg, int e, int len, int *slot) {
    const CacheView &c = a.src;
    if (e >= len) return false;
    const int page = c.page_table[bg * c.max_pages + (e >> c.page_shift)];
    *slot = page * c.page_size + (e & (c.page_size - 1));
    return c.u_pages[*slot] >= a.tau;
}

// Grids of the count and scatter kernels run (b, g) fastest: the tiles that
// exist (short lists end early) are dispatched first, the empty ones last.
__global__ void __launch_bounds__(NT) rethresh_count_kernel(RethreshArgs a) {
    __shared__ int lds_waves[NT / 64];
    const int j = blockIdx.y;
    const int64_t bg = blockIdx.x;
    const int len = list_len(a.src, bg);
    if (j * TILE >= len) return;
    int slot = 0;
    const bool flag = passes(a, bg, j * TILE + (int)threadIdx.x, len, &slot);
    int total;
    (void)block_rank(flag, lds_waves, &total);
    if (threadIdx.x == 0) a.ws[bg * a.max_tiles + j] = total;
}

__global__ void __launch_bounds__(NT) rethresh_plan_kernel(RethreshArgs a) {
    __shared__ int lds_scan[NT];
    __shared__ int lds_misc[4];
    const int64_t bg = blockIdx.x;
    const CacheView &d = a.dst;
    const int b = (int)(bg / d.n_kv);
    const int g = (int)(bg - (int64_t)b * d.n_kv);
    int32_t *cnt = a.ws + bg * a.max_tiles;
    const int n_tiles = (list_len(a.src, bg) + TILE - 1) / TILE;
    int carry = 0;
    for (int base = 0; base < n_tiles; base += NT) {
        const int j = base + threadIdx.x;
        const int x = j < n_tiles ? cnt[j] : 0;
        lds_scan[threadIdx.x] = x;
        __syncthreads();
        for (int off = 1; off < NT; off <<= 1) {
            const int y = threadIdx.x >= off ? lds_scan[threadIdx.x - off] : 0;
            __syncthreads();
            lds_scan[threadIdx.x] += y;
            __syncthreads();
        }
        if (j < n_tiles) cnt[j] = carry + lds_scan[threadIdx.x] - x;  // exclusive offset
        carry += lds_scan[NT - 1];
        __syncthreads();
    }
    const int new_len = grow_head(d, b, g, 0, carry, lds_misc);
    if (threadIdx.x == 0) {
        d.lengths[bg] = new_len;
        a.ws[(int64_t)d.batch * d.n_kv * a.max_tiles + bg] = new_len;
    }
}

// Copies of one tile.  Values are transposed in both caches ([page][hd][slot]):
// the tile's value columns are staged in LDS with 16-byte loads (every column
// of the tile: a cache line holds many slots, so the dropped entries' bytes
// come along anyway), then each value row of the destination is written in
// 16-byte pieces; only the pieces at the two ends of the tile's destination
// range, shared with the neighbouring tiles, are written element by element.
// Each thread takes its own entry's position, utility and (bf16) key row as
// soon as its keep decision is known and stores them once its rank is known,
// so that a tile costs few dependent trips to memory.  RT_SPLIT workgroups
// can share a tile (blockIdx.z), each with 1 / RT_SPLIT of the value rows and
// of every key row (less LDS per workgroup, more of them resident); on the
// decode_32k cache one workgroup per tile measured fastest (89 us against
// 134 us with two).
constexpr int RT_SPLIT = 1;

template <typename T>
__global__ void __launch_bounds__(NT) rethresh_scatter_kernel(RethreshArgs a) {
    constexpr int ES = sizeof(T);
    constexpr int EPC = 16 / ES;          // elements per 16-byte piece
    constexpr int MAXHD = 128;
    __shared__ int lds_src[TILE];         // flat source slot of each kept entry, in order
    __shared__ int lds_loc[TILE];         // its index inside the tile
    __shared__ int lds_waves[NT / 64];
    __shared__ int lds_pages[16];         // destination pages of the tile's range
    __shared__ int lds_spages[16];        // source pages of the tile
    __shared__ __attribute__((aligned(16))) T lds_v[MAXHD / RT_SPLIT][TILE];  // this half's value rows
    const int j = blockIdx.y;
    const int64_t bg = blockIdx.x;
    const int half = blockIdx.z;
    const CacheView &s = a.src;
    const CacheView &d = a.dst;
    const int len = list_len(s, bg);
    const int dst0 = a.ws[bg * a.max_tiles + j];
    const int new_len = a.ws[(int64_t)d.batch * d.n_kv * a.max_tiles + bg];
    const int e0 = j * TILE;
    if (e0 >= len) return;
    const int hd = d.head_dim;            // 64 or 128
    const int hh = hd / RT_SPLIT;         // value rows of this half: [half * hh, half * hh + hh)
    const int P = d.page_size;
    const int cnt = min(TILE, len - e0);
    const int sp0 = e0 >> s.page_shift;
    const int nsp = ((e0 + cnt - 1) >> s.page_shift) - sp0 + 1;  // <= TILE / 32
    // the destination range is at most [dst0, dst0 + min(cnt, new_len - dst0))
    const int nmax = max(0, min(cnt, new_len - dst0));
    const int pg0 = dst0 >> d.page_shift;
    const int npg = nmax > 0 ? ((dst0 + nmax - 1) >> d.page_shift) - pg0 + 1 : 0;  // <= TILE / 32 + 1
    if ((int)threadIdx.x < nsp) lds_spages[threadIdx.x] = s.page_table[bg * s.max_pages + sp0 + threadIdx.x];
    if ((int)threadIdx.x >= 64 && (int)threadIdx.x < 64 + npg)
        lds_pages[threadIdx.x - 64] = d.page_table[bg * d.max_pages + pg0 + threadIdx.x - 64];
    __syncthreads();
    const int me = e0 + (int)threadIdx.x;
    const bool mine = me < len;
    const int slot = mine ? lds_spages[(me >> s.page_shift) - sp0] * P + (me & (P - 1)) : 0;
    const float u = mine ? s.u_pages[slot] : 0.f;
    const int pos = mine ? s.pos_pages[slot] : 0;
    // stage the value columns of the tile: row e, entries [e0, e0 + cnt)
    // rounded up to a piece (a piece never crosses a page: P >= 32); every
    // load is issued before the first LDS store
    constexpr int NPT = MAXHD / RT_SPLIT * TILE / EPC / NT;  // pieces per thread at most
    const int ncol = (cnt + EPC - 1) / EPC;       // pieces per row
    piece_t x[NPT];
#pragma unroll
    for (int q = 0; q < NPT; ++q) {
        const int idx = q * NT + (int)threadIdx.x;
        if (idx < hh * ncol) {
            const int r = idx / ncol;
            const int e = half * hh + r;
            const int ent = e0 + (idx - r * ncol) * EPC;
            const int page = lds_spages[(ent >> s.page_shift) - sp0];
            // every line of the tile's value columns is read once, here
            x[q] = __builtin_nontemporal_load((const piece_t *)((const T *)s.v_pages + kv_v_index(page * P + (ent & (P - 1)), e, hd)));
        }
    }
    const bool flag = mine && u >= a.tau;  // NaN fails
    const int k0 = half * hh;             // first key element of this half
#pragma unroll
    for (int q = 0; q < NPT; ++q) {
        const int idx = q * NT + (int)threadIdx.x;
        if (idx < hh * ncol) {
            const int r = idx / ncol;
            *(piece_t *)&lds_v[r][(idx - r * ncol) * EPC] = x[q];
        }
    }
    int total;
    const int rank = block_rank(flag, lds_waves, &total);  // its barriers also cover the staging
    if (flag) {
        lds_src[rank] = slot;
        lds_loc[rank] = threadIdx.x;
    }
    const int n = max(0, min(total, new_len - dst0));
    if (n == 0) return;  // uniform: no barrier below is skipped by part of the block
    auto dslot = [&](int kk) -> int64_t {
        const int e = dst0 + kk;
        return (int64_t)lds_pages[(e >> d.page_shift) - pg0] * P + (e & (P - 1));
    };
    if (flag && rank < n) {
        const int64_t ds = dslot(rank);
        if (half == 0) {
            d.pos_pages[ds] = pos;
            if (d.u_pages) d.u_pages[ds] = u;
        }
    }
    __syncthreads();  // lds_src / lds_loc complete
    {
        // keys: 16-byte pieces, a row's pieces on neighbouring lanes, so every
        // load instruction reads whole 128-byte lines and every store
        // instruction writes consecutive rows (one row per entry and thread
        // would touch 64 lines of 16 bytes per instruction, about a third of
        // the throughput); a batch of loads is issued before its stores
        constexpr int KB = 8;
        const int cpr = hh / EPC;         // this half's pieces of a key row
        const int npk = n * cpr;
        for (int base = 0; base < npk; base += NT * KB) {
            piece_t kv[KB];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int idx = base + q * NT + (int)threadIdx.x;
                if (idx < npk) {
                    const int kk = idx / cpr;
                    const int ch = idx - kk * cpr;
                    kv[q] = *(const piece_t *)(s.k_pages + kv_k_index(lds_src[kk], k0 + ch * EPC, hd) * ES);
                }
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int idx = base + q * NT + (int)threadIdx.x;
                if (idx < npk) {
                    const int kk = idx / cpr;
                    const int ch = idx - kk * cpr;
                    *(piece_t *)(d.k_pages + kv_k_index(dslot(kk), k0 + ch * EPC, hd) * ES) = kv[q];
                }
            }
        }
    }
    // values: destination pieces c cover entries [c * EPC, c * EPC + EPC) of
    // the (b, g) list; those inside [dst0, dst0 + n) are whole
    const int c_lo = dst0 / EPC;
    const int c_hi = (dst0 + n - 1) / EPC;  // inclusive
    const int nch = c_hi - c_lo + 1;
    for (int idx = threadIdx.x; idx < hh * nch; idx += NT) {
        const int r = idx / nch;
        const int e = half * hh + r;
        const int c = c_lo + (idx - r * nch);
        const int first = c * EPC;                       // list entry of the piece's element 0
        const int64_t row = kv_v_index(lds_pages[(first >> d.page_shift) - pg0] * P + (first & (P - 1)), e, hd);
        T *dv = (T *)d.v_pages + row;
        if (first >= dst0 && first + EPC <= dst0 + n) {
            piece_t y;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (ES == 4) {
                    y[w] = __builtin_bit_cast(uint32_t, lds_v[r][lds_loc[first - dst0 + w]]);
                } else {
                    const uint32_t lo = __builtin_bit_cast(uint16_t, lds_v[r][lds_loc[first - dst0 + 2 * w]]);
                    const uint32_t hi = __builtin_bit_cast(uint16_t, lds_v[r][lds_loc[first - dst0 + 2 * w + 1]]);
                    y[w] = lo | (hi << 16);
                }
            }
            *(piece_t *)dv = y;
        } else {
            for (int q = 0; q < EPC; ++q) {
                const int kk = first + q - dst0;
                if (kk >= 0 && kk < n) dv[q] = lds_v[r][lds_loc[kk]];
            }
        }
    }
}

__global__ void cache_reset_kernel(CacheView c) {
    const int n = c.batch * c.n_kv;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        c.lengths[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *c.pool_next = 0;
        *c.status = 0;
    }
}

}  // namespace

size_t compact_ws_bytes(int batch, int n_kv, int page_size, int32_t max_rows) {
    if (max_rows <= TILE) return 0;
    return (size_t)((int64_t)batch * n_kv * onepass_ws(max_rows, page_size).stride) * sizeof(int32_t);
}

hipError_t launch_compact(const CompactArgs &a, hipStream_t s) {
    const CacheView &c = a.c;
    const bool bf16 = c.dtype == SPKV_BF16;
    if (a.max_rows == 1) {
        dim3 grid(c.batch, c.n_kv);
        if (bf16)
            hipLaunchKernelGGL(compact_row_kernel<uint16_t>, grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL(compact_row_kernel<float>, grid, dim3(64), 0, s, a);
        return hipGetLastError();
    }
    if (a.max_rows <= TILE || !(a.flags & SPKV_APPEND_GLOBAL)) {
        // one workgroup per (b, g); a window-only append of any size copies
        // just the last `window` rows of each sequence there
        dim3 grid(c.batch, c.n_kv);
        if (bf16)
            hipLaunchKernelGGL(compact_small_kernel<uint16_t>, grid, dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL(compact_small_kernel<float>, grid, dim3(NT), 0, s, a);
        return hipGetLastError();
    }
    // one workgroup per tile and (b, g), (b, g) fastest
    const int64_t n_wg = (int64_t)onepass_ws(a.max_rows, c.page_size).max_tiles * c.batch * c.n_kv;
    if (bf16)
        hipLaunchKernelGGL(compact_onepass_kernel<uint16_t>, dim3((uint32_t)n_wg), dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL(compact_onepass_kernel<float>, dim3((uint32_t)n_wg), dim3(NT), 0, s, a);
    return hipGetLastError();
}

size_t rethresh_ws_bytes(const spkv_cache *src) {
    const int64_t max_entries = (int64_t)src->max_pages_per_head * src->page_size;
    const int64_t max_tiles = (max_entries + TILE - 1) / TILE;
    return (size_t)((int64_t)src->batch * src->n_kv * (max_tiles + 1)) * sizeof(int32_t);
}

hipError_t launch_rethresh(const RethreshArgs &a0, hipStream_t s) {
    RethreshArgs a = a0;
    const int64_t max_entries = (int64_t)a.src.max_pages * a.src.page_size;
    a.max_tiles = (int32_t)((max_entries + TILE - 1) / TILE);
    const int BG = a.src.batch * a.src.n_kv;
    if (a.max_tiles == 0) {
        // nothing can be stored: every dst list is empty
        hipLaunchKernelGGL(rethresh_plan_kernel, dim3(BG), dim3(NT), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(rethresh_count_kernel, dim3(BG, a.max_tiles), dim3(NT), 0, s, a);
    hipLaunchKernelGGL(rethresh_plan_kernel, dim3(BG), dim3(NT), 0, s, a);
    if (a.src.dtype == SPKV_BF16)
        hipLaunchKernelGGL(rethresh_scatter_kernel<uint16_t>, dim3(BG, a.max_tiles, RT_SPLIT), dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL(rethresh_scatter_kernel<float>, dim3(BG, a.max_tiles, RT_SPLIT), dim3(NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cache_reset(const CacheView &c, hipStream_t s) {
    hipLaunchKernelGGL(cache_reset_kernel, dim3(1), dim3(256), 0, s, c);
    return hipGetLastError();
}

}  // namespace spkv
