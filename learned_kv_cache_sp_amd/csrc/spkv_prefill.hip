// Chunked-prefill attention of SP-KV (arXiv 2605.14037), section 2.1,
// Eq. (3)-(4), for the rows t = pos0 .. pos0 + n_rows - 1 of one sequence:
//   window keys  max(0, t-w+1) .. t   -- from this chunk's K/V when >= pos0,
//                                        from the ring when < pos0
//   global keys  cached entries with position <= t - w
// The chunk's kept rows were appended to the cache before this call, so a
// row also sees kept keys of its own chunk once they leave its window (Eq. 4
// is per token).
//
// bf16 (MFMA): a workgroup of 8 waves (2 per SIMD; 4 waves and two
// workgroups per compute unit at hd = 64) takes 32 (row, query head) pairs
// of one key head per wave -- 32 / G query positions, all G heads of the
// group -- and walks one list of 64-key blocks: the cached
// entries visible to its first row (no mask), the staircase of cached
// entries that only later rows see (mask pos <= t - w), and the window band
// (mask 0 <= t - s < w).  Whole cached blocks stream into LDS through a
// pipeline of direct global->LDS loads, two blocks per barrier into four
// buffers (keys row-major, values already transposed in the cache); the
// last, partial cached block and the
// band blocks go through registers (zeroing invalid slots, transposing chunk
// values).  Both layouts are XOR-swizzled so MFMA operand reads are free of
// bank conflicts.  Per wave and 32 keys:
//   S^T[32 keys x 16 pairs] = K . Q^T       (v_mfma_f32_16x16x32_bf16)
//   O^T[hd x 16 pairs]     += V^T . P^T     (P rounded to bf16, f32 accumulate)
// for each of its 2 pair tiles, online softmax with a lazily updated max.
// The weights P enter the second product as bf16 (relative error <= 2^-9 per
// weight; the normaliser l sums them in f32): this kernel is MFMA-bound, and
// a bf16 hi/lo pair (f32-accurate, as the memory-bound decode kernel uses)
// would cost half as many MFMAs again.
// Row tiles are handed out last-first: later rows see more keys.
//
// f32 (and a fallback for shapes the MFMA tiling does not take): VALU, one
// wave per (row, query head), online softmax over the key list.
#include "spkv_internal.h"

namespace spkv {
namespace {

template <typename T, int HD>
__global__ void __launch_bounds__(64) prefill_valu_kernel(PrefillArgs a) {
    const CacheView &c = a.c;
    const int i = blockIdx.x;
    const int h = blockIdx.y;
    const int g = h / a.group;
    const int b = a.b;
    const int bg = b * c.n_kv + g;
    const int lane = threadIdx.x;
    constexpr int PER = HD / 64;
    const int t = a.pos0 + i;
    const int w = c.window;
    const T *qp = (const T *)a.q + (int64_t)i * a.ld_q + (int64_t)h * HD;
    float q[PER], o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        q[e] = (float)qp[lane + 64 * e];
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    // j < 0: k, v point at a row of the chunk; else k, v are a page or ring
    // region and j the slot (block storage order)
    auto kat = [&](const T *k, int j, int d) -> float { return (float)(j < 0 ? k[d] : k[kv_k_index(j, d, HD)]); };
    auto vat = [&](const T *v, int j, int d) -> float { return (float)(j < 0 ? v[d] : v[kv_v_index(j, d, HD)]); };
    auto visit = [&](const T *k, const T *v, int j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) s = fmaf(q[e], kat(k, j, lane + 64 * e), s);
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        s *= a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = o[e] * alpha + p * vat(v, j, lane + 64 * e);
        m = m_new;
    };
    // window band
    const int s_lo = max(0, t - w + 1);
    for (int s = s_lo; s <= t; ++s) {
        if (s >= a.pos0) {
            const int64_t r = (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD;
            visit((const T *)a.k + r, (const T *)a.v + r, -1);
        } else {
            visit((const T *)c.ring_k + (int64_t)bg * w * HD, (const T *)c.ring_v + (int64_t)bg * w * HD, s % w);
        }
    }
    // kept entries older than the window
    const int len = c.lengths[bg];
    const int P = c.page_size;
    const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
    for (int j = 0; j < len; ++j) {
        const int page = pt[j >> c.page_shift];
        const int slot = j & (P - 1);
        if (c.pos_pages[(int64_t)page * P + slot] > t - w) break;  // positions increase
        visit((const T *)c.k_pages + (int64_t)page * P * HD, (const T *)c.v_pages + (int64_t)page * P * HD, slot);
    }
    float *op = a.out + ((int64_t)i * a.n_q + h) * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[lane + 64 * e] = l > 0.f ? o[e] / l : 0.f;
    if (lane == 0 && a.lse) a.lse[(int64_t)i * a.n_q + h] = l > 0.f ? m + logf(l) : -INFINITY;
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Workgroup shape per head size.  hd = 128: 8 waves (2 per SIMD) share one
// workgroup's key/value buffers (148 KB of LDS).  hd = 64: 4 waves, and two
// workgroups per compute unit (78 KB of LDS each, 2048 page-table entries),
// so that the two waves of a SIMD belong to different barriers and their
// phases need not line up: 9 % faster at hd = 64, while at hd = 128 the
// doubled key/value traffic per flop of half-size workgroups costs more
// than that (4 % slower) and two would not fit in LDS.
template <int HD>
struct PfShape {
    static constexpr int NW = HD == 64 ? 4 : 8;          // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int PTMAX = HD == 64 ? 2048 : 4096;  // page-table entries staged in LDS
};
constexpr int PF_PT = 2;           // 16-pair MFMA column tiles per wave
constexpr int PF_KB = 64;          // keys per block
constexpr int PF_ST = 4;           // LDS buffers of the direct-load pipeline (two blocks per barrier)
constexpr float PF_LOG2E = 1.4426950408889634f;
constexpr float PF_LN2 = 0.6931471805599453f;

__device__ inline int pf_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// raw buffer descriptor over `bytes` bytes at base (gfx9 family dword 3)
__device__ inline __amdgpu_buffer_rsrc_t pf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void;
// direct buffer -> LDS loads of 16 and 4 bytes per lane (lane l writes
// dst + size * l).  The builtin is left out of the host pass, whose checks
// reject it inside the kernel template.
__device__ inline void pf_buffer_lds16(__amdgpu_buffer_rsrc_t r, lds_void *dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
#endif
}
__device__ inline void pf_buffer_lds4(__amdgpu_buffer_rsrc_t r, lds_void *dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
#endif
}

// position of cached entry j of (b, g)
__device__ inline int entry_pos(const CacheView &c, const int32_t *pt, int j) {
    const int page = pt[j >> c.page_shift];
    return c.pos_pages[(int64_t)page * c.page_size + (j & (c.page_size - 1))];
}

// number of cached entries of (b, g) with position <= x (positions increase
// along the list), by two rounds of parallel probes
template <int NT>
__device__ int count_upto(const CacheView &c, const int32_t *pt, int len, int x, int *lds_cnt) {
    if (len <= 0 || x < 0) return 0;
    // round 1: NT evenly spaced probes -> a bracket of at most ceil(len/NT) entries
    const int step = (len + NT - 1) / NT;
    const int j = threadIdx.x * step;
    const bool le = j < len && entry_pos(c, pt, j) <= x;
    __syncthreads();
    if (threadIdx.x == 0) lds_cnt[0] = 0;
    __syncthreads();
    const uint64_t bal = __ballot(le);
    if ((threadIdx.x & 63) == 0) atomicAdd(&lds_cnt[0], __popcll(bal));
    __syncthreads();
    const int k = lds_cnt[0];  // probes 0..k-1 are <= x (a prefix)
    if (k == 0) return 0;
    const int lo = (k - 1) * step;  // entry lo is <= x
    const int hi = min(len, k * step);
    // round 2: the entries lo+1 .. hi-1
    __syncthreads();
    if (threadIdx.x == 0) lds_cnt[1] = 0;
    __syncthreads();
    for (int jj = lo + 1 + threadIdx.x; jj - threadIdx.x < hi; jj += NT) {
        const bool le2 = jj < hi && entry_pos(c, pt, jj) <= x;
        const uint64_t bal2 = __ballot(le2);
        if ((threadIdx.x & 63) == 0 && bal2) atomicAdd(&lds_cnt[1], __popcll(bal2));
    }
    __syncthreads();
    return lo + 1 + lds_cnt[1];
}

// LDS layouts of one 64-key block (byte offsets), XOR-swizzled so that the
// 16 lanes that read one MFMA operand row group hit 16 different 16-byte
// bank groups:
//   keys:   row r (HD bf16), 16-byte chunk c at r*2*HD + 16*(c ^ swz_k(r))
//   values: transposed, row e (64 keys), chunk c at e*128 + 16*(c ^ swz_v(e))
template <int HD>
__device__ inline int swz_k(int r) {
    return HD == 128 ? ((r & 3) | (((r >> 3) & 3) << 2)) : (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
}
__device__ inline int swz_v(int e) { return (e >> 1) & 7; }
template <int HD>
__device__ inline int koff(int r, int c) { return r * (2 * HD) + ((c ^ swz_k<HD>(r)) << 4); }
__device__ inline int voff(int e, int c) { return e * (2 * PF_KB) + ((c ^ swz_v(e)) << 4); }


// SOFT: the training-time relaxation of SP-KV (section 2.1, Eq. 5-6) --
// every cached key outside the window gets the additive score
// c (alpha - 1) = -c sigmoid((tau - u) / beta), u its stored utility, formed
// here as -c / (1 + exp((u - tau) / beta)) (the same value without the loss
// of precision of 1 - alpha near alpha = 1); window keys get none.
template <int HD, bool SOFT>
__global__ void __launch_bounds__(PfShape<HD>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(PrefillArgs a) {
    constexpr int PF_NW = PfShape<HD>::NW;
    constexpr int PF_NT = PfShape<HD>::NT;
    constexpr int PF_PTMAX = PfShape<HD>::PTMAX;
    constexpr int CPR = HD / 8;                  // 16-byte chunks per key row
    constexpr int KBYTES = PF_KB * 2 * HD;       // key block
    constexpr int VBYTES = HD * 2 * PF_KB;       // transposed value block
    constexpr int KI = KBYTES / 1024;            // 1 KB direct loads per key block
    constexpr int VI = VBYTES / 1024;
    constexpr int KRPI = 1024 / (2 * HD);        // key rows per direct load
    // one array per stage: with every stage index a compile-time constant in
    // the pipeline loop, the compiler can tell that reading one stage does
    // not touch the direct loads in flight into another (with one indexed
    // array it waits for all of them before every read)
    static_assert(PF_ST == 4, "four buffers");
    __shared__ __attribute__((aligned(1024))) char lds_kb0[KBYTES], lds_kb1[KBYTES], lds_kb2[KBYTES], lds_kb3[KBYTES];
    __shared__ __attribute__((aligned(1024))) char lds_vb0[VBYTES], lds_vb1[VBYTES], lds_vb2[VBYTES], lds_vb3[VBYTES];
    __shared__ __attribute__((aligned(16))) int lds_pos0[PF_KB], lds_pos1[PF_KB], lds_pos2[PF_KB], lds_pos3[PF_KB];
    constexpr int UN = SOFT ? PF_KB : 4;  // stored utilities of a block (soft mode)
    __shared__ __attribute__((aligned(16))) float lds_u0[UN], lds_u1[UN], lds_u2[UN], lds_u3[UN];
    __shared__ __attribute__((aligned(16))) float lds_bias[SOFT ? PF_NW : 1][UN];  // per wave: a block's key scores
    __shared__ int lds_pt[PF_PTMAX];
    __shared__ int lds_cnt[2];

    const CacheView &c = a.c;
    const int G = a.group;
    // Workgroups are dealt to the 8 XCDs in launch order (linear id mod 8).
    // When n_kv divides 8, the linear id is read as (row tile, key head) with
    // the head fastest, so every workgroup of head g runs on the XCDs
    // congruent to g: the workgroups that stream the same cached blocks at
    // about the same time share an L2.
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const bool xcd_map = (8 % a.c.n_kv) == 0;
    const int g = xcd_map ? lin % a.c.n_kv : (int)blockIdx.y;
    const int tile = xcd_map ? lin / a.c.n_kv : (int)blockIdx.x;
    const int b = a.b;
    const int bg = b * c.n_kv + g;
    const int w = c.window;
    const int P = c.page_size;
    const int rows_wave = (16 * PF_PT) / G;           // query positions per wave
    const int rows_wg = rows_wave * PF_NW;
    // the last row tiles see the most keys: hand them out first
    const int r_base = (gridDim.x - 1 - tile) * rows_wg;  // chunk-relative first row
    const int t_min = a.pos0 + r_base;
    const int t_max = a.pos0 + min(a.n_rows, r_base + rows_wg) - 1;
    const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
    const int len = c.lengths[bg];

    // ---- the block list of this workgroup -----------------------------------
    const int n_full = count_upto<PF_NT>(c, pt, len, t_min - w, lds_cnt);  // visible to every row
    const int n_part = count_upto<PF_NT>(c, pt, len, t_max - w, lds_cnt);  // visible to the last row
    const int s_lo = max(0, t_min - w + 1);                          // window band
    const int nb_d = n_part / PF_KB;                        // whole cached blocks (direct loads)
    const int nb_g = (n_part + PF_KB - 1) / PF_KB;          // all cached blocks
    const int nb_b = (t_max - s_lo + 1 + PF_KB - 1) / PF_KB;  // band blocks

    const int lane = threadIdx.x & 63;
    const int wave = pf_uniform(threadIdx.x >> 6);
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const float sl2 = a.scale * PF_LOG2E;

    // ---- this wave's query operand: pair p = pt * 16 + i16 -> (row, head) ----
    bf16x8 qr[PF_PT][HD / 32];
    int trow[PF_PT];   // position of this lane's pair in each tile
#pragma unroll
    for (int ptl = 0; ptl < PF_PT; ++ptl) {
        const int p = ptl * 16 + i16;
        const int row = wave * rows_wave + p / G;       // workgroup-relative
        const int h = g * G + (p % G);
        const int r = r_base + row;                     // chunk-relative
        trow[ptl] = a.pos0 + r;
        const bool ok = r < a.n_rows;
        const __bf16 *qp = (const __bf16 *)a.q + (int64_t)(ok ? r : 0) * a.ld_q + (int64_t)h * HD + 8 * q4;
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc) qr[ptl][cc] = ok ? *(const bf16x8 *)(qp + 32 * cc) : bf16x8{};
    }
    // ---- whole cached blocks: direct global -> LDS loads ---------------------
    // Page ids come from LDS (lds_pt holds a window of the page table): a page
    // id read from global memory just before each load would make every issue
    // wait for all loads in flight, the pipeline's included.
    int pg_base = 0;  // page index held by lds_pt[0]
    auto page_of = [&](int ent) -> int { return lds_pt[(ent >> c.page_shift) - pg_base]; };
    // Pages of at least one block (the usual case): a block lies in one page,
    // so its loads are buffer loads from the page with a scalar base and
    // per-lane offsets fixed for the whole launch -- no address arithmetic
    // per block.
    const bool page_blocks = P >= PF_KB;
    int dk_off[KI / PF_NW], dv_off[VI / PF_NW];
#pragma unroll
    for (int u = 0; u < KI / PF_NW; ++u) {
        const int i = wave + PF_NW * u;
        const int r = i * KRPI + lane / CPR;
        dk_off[u] = (int)kv_k_index(r, 8 * ((lane % CPR) ^ swz_k<HD>(r)), HD) * 2;
    }
#pragma unroll
    for (int u = 0; u < VI / PF_NW; ++u) {
        const int i = wave + PF_NW * u;
        const int e = i * 8 + (lane >> 3);
        dv_off[u] = (int)kv_v_index(8 * ((lane & 7) ^ swz_v(e)), e, HD) * 2;
    }
    auto issue_direct = [&](int j, char *kbuf, char *vbuf, int *pbuf, float *ubuf) {
        const int e0 = j * PF_KB;
        if (page_blocks) {
            const int page = pf_uniform(page_of(e0));
            const int slot0 = e0 & (P - 1);
            const __amdgpu_buffer_rsrc_t rk =
                pf_rsrc(c.k_pages + ((int64_t)page * P + slot0) * HD * 2, PF_KB * HD * 2);
            const __amdgpu_buffer_rsrc_t rv =
                pf_rsrc(c.v_pages + ((int64_t)page * P + slot0) * HD * 2, PF_KB * HD * 2);
            const __amdgpu_buffer_rsrc_t rp = pf_rsrc(c.pos_pages + (int64_t)page * P + slot0, PF_KB * 4);
#pragma unroll
            for (int u = 0; u < KI / PF_NW; ++u)
                pf_buffer_lds16(rk, (lds_void *)(kbuf + (wave + PF_NW * u) * 1024), dk_off[u]);
#pragma unroll
            for (int u = 0; u < VI / PF_NW; ++u)
                pf_buffer_lds16(rv, (lds_void *)(vbuf + (wave + PF_NW * u) * 1024), dv_off[u]);
            pf_buffer_lds4(rp, (lds_void *)pbuf, lane * 4);
            if constexpr (SOFT) {
                const __amdgpu_buffer_rsrc_t ru = pf_rsrc(c.u_pages + (int64_t)page * P + slot0, PF_KB * 4);
                pf_buffer_lds4(ru, (lds_void *)ubuf, lane * 4);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < KI / PF_NW; ++u) {
            const int i = wave + PF_NW * u;
            const int r = i * KRPI + lane / CPR;
            const int cch = (lane % CPR) ^ swz_k<HD>(r);
            const int ent = e0 + r;
            const char *src = c.k_pages + ((int64_t)page_of(ent) * P * HD + kv_k_index(ent & (P - 1), 8 * cch, HD)) * 2;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(kbuf + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < VI / PF_NW; ++u) {
            const int i = wave + PF_NW * u;
            const int e = i * 8 + (lane >> 3);
            const int cch = (lane & 7) ^ swz_v(e);
            const int ent = e0 + 8 * cch;
            const char *src = c.v_pages + ((int64_t)page_of(ent) * P * HD + kv_v_index(ent & (P - 1), e, HD)) * 2;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(vbuf + i * 1024), 16, 0, 0);
        }
        {
            // positions of the 64 entries (every wave loads the same values)
            const int ent = e0 + lane;
            const int32_t *src = c.pos_pages + (int64_t)page_of(ent) * P + (ent & (P - 1));
            __builtin_amdgcn_global_load_lds(src, (lds_void *)pbuf, 4, 0, 0);
            if constexpr (SOFT) {
                const float *usrc = c.u_pages + (int64_t)page_of(ent) * P + (ent & (P - 1));
                __builtin_amdgcn_global_load_lds(usrc, (lds_void *)ubuf, 4, 0, 0);
            }
        }
    };

    // ---- the partial cached block and the band: staged through registers ----
    constexpr int KCH = PF_KB * CPR / PF_NT;        // key chunks per thread
    constexpr int VCH = HD * (PF_KB / 8) / PF_NT;   // value chunks per thread
    i32x4 kst[KCH], vst[VCH];
    int pst = 0;
    float ust = 0.f;
    // This rarely run path (a few blocks per workgroup) forms its index
    // arithmetic from opaque copies of the thread index and the window, at
    // each call: otherwise the compiler hoists that arithmetic out of the
    // whole kernel and holds it in registers across the main pipeline.
    auto load_staged = [&](int blk) {
        int tid = threadIdx.x, w = c.window;
        asm volatile("" : "+v"(tid), "+s"(w));
        if (blk < nb_g) {
            // cached block with n_ok < 64 valid entries: invalid keys get zero
            // values (their slots may hold anything) and position INT_MAX
            const int j0 = blk * PF_KB;
            const int n_ok = min(PF_KB, n_part - j0);
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int id = tid + u * PF_NT;
                const int kk = id / CPR, ch = id % CPR;
                const int ent = j0 + kk;
                kst[u] = kk < n_ok ? *(const i32x4 *)((const __bf16 *)c.k_pages + (int64_t)pt[ent >> c.page_shift] * P * HD +
                                                      kv_k_index(ent & (P - 1), 8 * ch, HD))
                                   : i32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = tid + u * PF_NT;
                const int e = id / (PF_KB / 8), kc = id % (PF_KB / 8);
                const int ent = j0 + 8 * kc;
                i32x4 v = i32x4{0, 0, 0, 0};
                if (8 * kc < n_ok) {
                    v = *(const i32x4 *)((const __bf16 *)c.v_pages + (int64_t)pt[ent >> c.page_shift] * P * HD +
                                         kv_v_index(ent & (P - 1), e, HD));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int k0 = 8 * kc + 2 * q;
                        const uint32_t mk = (k0 < n_ok ? 0x0000ffffu : 0u) | (k0 + 1 < n_ok ? 0xffff0000u : 0u);
                        v[q] &= (int32_t)mk;
                    }
                }
                vst[u] = v;
            }
            if (tid < PF_KB) {
                const int ent = j0 + tid;
                pst = tid < n_ok ? c.pos_pages[(int64_t)pt[ent >> c.page_shift] * P + (ent & (P - 1))] : INT_MAX;
                if constexpr (SOFT)
                    ust = tid < n_ok ? c.u_pages[(int64_t)pt[ent >> c.page_shift] * P + (ent & (P - 1))] : 0.f;
            }
        } else {
            const int s0 = s_lo + (blk - nb_g) * PF_KB;
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int id = tid + u * PF_NT;
                const int kk = id / CPR, ch = id % CPR;
                const int s = s0 + kk;
                i32x4 kv = i32x4{0, 0, 0, 0};
                if (s <= t_max) {
                    if (s >= a.pos0)
                        kv = *(const i32x4 *)((const __bf16 *)a.k + (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD + 8 * ch);
                    else
                        kv = *(const i32x4 *)((const __bf16 *)c.ring_k + kv_k_index((int64_t)bg * w + (s % w), 8 * ch, HD));
                }
                kst[u] = kv;
            }
            // values: key kk2, dims 8*dc .. 8*dc+7 (row-major source, or 8
            // gathers from the transposed ring), scattered on store
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = tid + u * PF_NT;
                const int kk2 = id / CPR, dc = id % CPR;
                const int s = s0 + kk2;
                i32x4 vv = i32x4{0, 0, 0, 0};
                if (s <= t_max) {
                    if (s >= a.pos0) {
                        vv = *(const i32x4 *)((const __bf16 *)a.v + (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD + 8 * dc);
                    } else {
                        const __bf16 *rv = (const __bf16 *)c.ring_v + kv_v_index((int64_t)bg * w + (s % w), 8 * dc, HD);
                        __bf16 tmp[8];
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) tmp[e2] = rv[32 * e2];
                        vv = __builtin_bit_cast(i32x4, *(bf16x8 *)tmp);
                    }
                }
                vst[u] = vv;
            }
            if (tid < PF_KB) pst = s0 + tid;
        }
    };
    auto store_staged = [&](int blk, char *kbuf, char *vbuf, int *pbuf, float *ubuf) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int id = tid + u * PF_NT;
            const int kk = id / CPR, ch = id % CPR;
            *(i32x4 *)(kbuf + koff<HD>(kk, ch)) = kst[u];
        }
        if (blk < nb_g) {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = tid + u * PF_NT;
                const int e = id / (PF_KB / 8), kc = id % (PF_KB / 8);
                *(i32x4 *)(vbuf + voff(e, kc)) = vst[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = tid + u * PF_NT;
                const int kk2 = id / CPR, dc = id % CPR;
                const bf16x8 vv = __builtin_bit_cast(bf16x8, vst[u]);
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2)
                    *(__bf16 *)(vbuf + voff(8 * dc + e2, kk2 >> 3) + 2 * (kk2 & 7)) = vv[e2];
            }
        }
        if (tid < PF_KB) pbuf[tid] = pst;
        if constexpr (SOFT)
            if (tid < PF_KB) ubuf[tid] = ust;
    };

    // ---- per-wave online softmax state over its pair tiles -------------------
    f32x4 o[PF_PT][HD / 16];
    float m[PF_PT], l[PF_PT];
#pragma unroll
    for (int ptl = 0; ptl < PF_PT; ++ptl) {
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) o[ptl][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[ptl] = -INFINITY;
        l[ptl] = 0.f;
    }

    // LDS operand addresses: with the swizzles above, the XOR term of every
    // operand row a lane reads is a lane constant
    //   key row 32*hh + 8*(i16/4) + 4*tt + i16%4, chunk 4*cc + q4
    //   value row 16*nt + i16, chunk 4*hh + q4
    const int k_lane = (8 * (i16 >> 2) + (i16 & 3)) * (2 * HD);
    const int k_x = swz_k<HD>(8 * (i16 >> 2) + (i16 & 3));
    const int v_lane = i16 * (2 * PF_KB);
    const int v_x = swz_v(i16);

    // one 64-key block from stage st; kind 0: every key visible to every row,
    // 1: cached keys visible iff position <= t - w, 2: band keys visible iff
    // 0 <= t - position < w.  The scores of both 32-key halves are formed
    // first (score tiles accumulating side by side), then one max check per
    // pair tile for the whole block, then exponentials and value products
    // without branches, the products of the pair tiles alternating so that
    // no MFMA waits on the one before.
    // soft mode: -c / (1 + 2^((u - tau) * log2(e) / beta)), divided by the
    // score scale (the scores are scaled with the exponent's argument below)
    auto soft_bias = [&](float u) -> float {
        return -a.soft_cs / (1.f + __builtin_amdgcn_exp2f((u - a.soft_tau) * a.soft_k1));
    };
    // Issue priority: a wave in a matrix-core phase of a block (the scores,
    // the value products) runs at priority 1, in its exponential / mask
    // phases at 0, so that of the two waves of a SIMD the one with matrix
    // work gets the issue slots (soft mode, with more vector work per block:
    // 2.7 % faster; the plain mode unchanged).
    auto prio_hi = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto prio_lo = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute_block = [&](const char *kb, const char *vb, const int *pb_pos, const float *pb_u, int kind) {
        f32x4 sc[2][PF_PT][2];
        prio_hi();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            bf16x8 ka[2][HD / 32];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int cc = 0; cc < HD / 32; ++cc)
                    ka[tt][cc] = *(const bf16x8 *)(kb + k_lane + (32 * hh + 4 * tt) * (2 * HD) +
                                                   (((4 * cc + q4) ^ k_x) << 4));
#pragma unroll
            for (int ptl = 0; ptl < PF_PT; ++ptl)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) sc[hh][ptl][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < HD / 32; ++cc)
#pragma unroll
                for (int ptl = 0; ptl < PF_PT; ++ptl)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        sc[hh][ptl][tt] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][cc], qr[ptl][cc], sc[hh][ptl][tt], 0, 0, 0);
        }
        prio_lo();
        // soft mode: the mask of Eq. (6) on cached keys (kinds 0 and 1).
        // Lane l forms the added score of key l once and parks it in the
        // wave's LDS row (LDS operations of one wave complete in order);
        // every lane then reads the 16 it needs.
        if constexpr (SOFT) {
            if (kind != 2) {
                float *wb = lds_bias[wave];
                wb[lane] = soft_bias(pb_u[lane]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const f32x4 b0 = *(const f32x4 *)&wb[32 * hh + 8 * q4];
                    const f32x4 b1 = *(const f32x4 *)&wb[32 * hh + 8 * q4 + 4];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float bias = e < 4 ? b0[e] : b1[e - 4];
#pragma unroll
                        for (int ptl = 0; ptl < PF_PT; ++ptl) sc[hh][ptl][e >> 2][e & 3] += bias;
                    }
                }
            }
        }
        // masks; this lane's keys are 32*hh + 8*q4 + e
        if (kind != 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const i32x4 p0 = *(const i32x4 *)&pb_pos[32 * hh + 8 * q4];
                const i32x4 p1 = *(const i32x4 *)&pb_pos[32 * hh + 8 * q4 + 4];
#pragma unroll
                for (int ptl = 0; ptl < PF_PT; ++ptl) {
                    const int t = trow[ptl];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kp = e < 4 ? p0[e] : p1[e - 4];
                        const bool vis = kind == 1 ? (kp <= t - w) : ((unsigned)(t - kp) < (unsigned)w);
                        if (!vis) sc[hh][ptl][e >> 2][e & 3] = -INFINITY;
                    }
                }
            }
        }
        // lazily updated reference max, one check per pair tile and block
        // (exact result; see the decode kernel)
        float nbase[PF_PT];
#pragma unroll
        for (int ptl = 0; ptl < PF_PT; ++ptl) {
            float mraw = -INFINITY;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e) mraw = fmaxf(mraw, sc[hh][ptl][e >> 2][e & 3]);
            float mloc = mraw * sl2;  // log2 domain
            if (__ballot(mloc > m[ptl] + 8.f) != 0) {
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
                const float m_new = fmaxf(m[ptl], mloc);
                if (m_new != m[ptl]) {
                    const float alpha = __builtin_amdgcn_exp2f(m[ptl] - m_new);
#pragma unroll
                    for (int nt = 0; nt < HD / 16; ++nt) o[ptl][nt] *= alpha;
                    l[ptl] *= alpha;
                    m[ptl] = m_new;
                }
            }
            nbase[ptl] = (m[ptl] == -INFINITY) ? 0.f : -m[ptl];
        }
        auto exp_half = [&](int hh, bf16x8 (&pb)[PF_PT]) {
#pragma unroll
            for (int ptl = 0; ptl < PF_PT; ++ptl) {
                float psum = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(fmaf(sc[hh][ptl][e >> 2][e & 3], sl2, nbase[ptl]));  // -inf -> 0
                    psum += pe;
                    pb[ptl][e] = (__bf16)pe;
                }
                l[ptl] += psum;
            }
        };
        // O^T += V^T . P^T; the V^T operand is shared by the pair tiles
        auto pv_half = [&](int hh, const bf16x8 (&pb)[PF_PT]) {
#pragma unroll
            for (int nt = 0; nt < HD / 16; ++nt) {
                const bf16x8 va = *(const bf16x8 *)(vb + v_lane + nt * 16 * (2 * PF_KB) + (((4 * hh + q4) ^ v_x) << 4));
#pragma unroll
                for (int ptl = 0; ptl < PF_PT; ++ptl)
                    o[ptl][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ptl], o[ptl][nt], 0, 0, 0);
            }
        };
        bf16x8 pb0[PF_PT], pb1[PF_PT];
        exp_half(0, pb0);
        prio_hi();
        // the first half's value products with the second half's
        // exponentials between them (VALU work under the MFMAs)
        pv_half(0, pb0);
        exp_half(1, pb1);
        __builtin_amdgcn_sched_group_barrier(0x100, HD / 16, 0);  // the value operand reads first
#pragma unroll
        for (int i = 0; i < (HD / 16) * PF_PT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then some VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        pv_half(1, pb1);
        prio_lo();
    };

    // ---- phase 1: whole cached blocks, two per barrier ----------------------
    // Windows of blocks whose page ids fit lds_pt (one window unless the list
    // is very long).  Blocks jj, jj + 1 of a window live in buffers 0, 1 or
    // 2, 3 (jj / 2 even or odd).  Before computing them a wave waits for its
    // own loads of both (the only ones in flight); then a plain barrier -- a
    // fenced one would wait on the direct-load counter too -- makes every
    // wave's loads of the pair visible and guarantees that every wave is done
    // reading the previous pair (its reads were consumed by its MFMAs), whose
    // buffers then receive jj + 2 and jj + 3, loading while the pair is
    // computed.  One barrier per 128 keys: against one per 64 keys with a
    // 3-stage ring, 2.5 % more throughput on the 8B layer's chunks.
    constexpr int WAIT_ALL = (7 << 4) | (15 << 8);  // vmcnt(0)
    const int win_blocks = (PF_PTMAX << c.page_shift) / PF_KB;  // >= 1024 (page size >= 32)
    __syncthreads();  // query operands loaded, lds_cnt no longer read
    for (int wb0 = 0; wb0 < nb_d; wb0 += win_blocks) {
        const int wb1 = min(nb_d, wb0 + win_blocks);
        pg_base = (wb0 * PF_KB) >> c.page_shift;
        const int np_ = (((wb1 * PF_KB) - 1) >> c.page_shift) + 1 - pg_base;
        for (int i = threadIdx.x; i < np_; i += PF_NT) lds_pt[i] = pt[pg_base + i];
        __syncthreads();  // page ids staged (no direct loads in flight here)
        const int n = wb1 - wb0;
        issue_direct(wb0, lds_kb0, lds_vb0, lds_pos0, lds_u0);
        if (n > 1) issue_direct(wb0 + 1, lds_kb1, lds_vb1, lds_pos1, lds_u1);
        // blocks jj, jj + 1 in buffers X0, X1; Y0, Y1 receive jj + 2, jj + 3
        auto pair = [&](int jj, char *kx0, char *vx0, int *px0, float *ux0, char *kx1, char *vx1, int *px1,
                        float *ux1, char *ky0, char *vy0, int *py0, float *uy0, char *ky1, char *vy1, int *py1,
                        float *uy1) {
            __builtin_amdgcn_sched_barrier(0);  // no scheduling across blocks (register pressure)
            const int j = wb0 + jj;
            __builtin_amdgcn_s_waitcnt(WAIT_ALL);  // this wave's loads of jj and jj + 1
            __builtin_amdgcn_s_barrier();
            if (jj + 2 < n) issue_direct(j + 2, ky0, vy0, py0, uy0);
            if (jj + 3 < n) issue_direct(j + 3, ky1, vy1, py1, uy1);
            compute_block(kx0, vx0, px0, ux0, (j + 1) * PF_KB <= n_full ? 0 : 1);
            __builtin_amdgcn_sched_barrier(0);
            if (jj + 1 < n) compute_block(kx1, vx1, px1, ux1, (j + 2) * PF_KB <= n_full ? 0 : 1);
        };
        for (int jj = 0; jj < n; jj += 4) {
            pair(jj, lds_kb0, lds_vb0, lds_pos0, lds_u0, lds_kb1, lds_vb1, lds_pos1, lds_u1,
                 lds_kb2, lds_vb2, lds_pos2, lds_u2, lds_kb3, lds_vb3, lds_pos3, lds_u3);
            if (jj + 2 < n)
                pair(jj + 2, lds_kb2, lds_vb2, lds_pos2, lds_u2, lds_kb3, lds_vb3, lds_pos3, lds_u3,
                     lds_kb0, lds_vb0, lds_pos0, lds_u0, lds_kb1, lds_vb1, lds_pos1, lds_u1);
        }
        __syncthreads();  // every stage and lds_pt are free again (nothing in flight)
    }

    // ---- phase 2: partial cached block and band blocks (a few per
    // workgroup), staged through registers; the stores of block blk + 1 go
    // to the other stage while blk is computed from its stage ---------------
    const int b0 = nb_d, nb = nb_g + nb_b;
    if (b0 < nb) {
        load_staged(b0);
        store_staged(b0, lds_kb0, lds_vb0, lds_pos0, lds_u0);
    }
    __syncthreads();
    for (int blk = b0; blk < nb; ++blk) {
        const bool odd = ((blk - b0) & 1) != 0;
        if (blk + 1 < nb) {
            load_staged(blk + 1);
            store_staged(blk + 1, odd ? lds_kb0 : lds_kb1, odd ? lds_vb0 : lds_vb1, odd ? lds_pos0 : lds_pos1,
                         odd ? lds_u0 : lds_u1);
        }
        compute_block(odd ? lds_kb1 : lds_kb0, odd ? lds_vb1 : lds_vb0, odd ? lds_pos1 : lds_pos0,
                      odd ? lds_u1 : lds_u0, blk < nb_g ? 1 : 2);
        __syncthreads();
    }

    // ---- outputs ------------------------------------------------------------
#pragma unroll
    for (int ptl = 0; ptl < PF_PT; ++ptl) {
        float lsum = l[ptl];
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        const int p = ptl * 16 + i16;
        const int row = wave * rows_wave + p / G;
        const int h = g * G + (p % G);
        const int r = r_base + row;
        if (r < a.n_rows) {
            float *op = a.out + ((int64_t)r * a.n_q + h) * HD;
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int nt = 0; nt < HD / 16; ++nt)
                *(f32x4 *)(op + 16 * nt + 4 * q4) = o[ptl][nt] * inv;
            if (q4 == 0 && a.lse) a.lse[(int64_t)r * a.n_q + h] = lsum > 0.f ? (m[ptl] + log2f(lsum)) * PF_LN2 : -INFINITY;
        }
    }
}

}  // namespace

size_t prefill_ws_bytes(const spkv_cache *c, int n_q, int n_rows) {
    (void)c;
    (void)n_q;
    (void)n_rows;
    return 0;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    const CacheView &c = a.c;
    const dim3 grid(a.n_rows, a.n_q);
    if (c.dtype == SPKV_BF16 && a.group <= 16) {
        auto go = [&](auto kernel, int nw) {
            const int rows_wg = (16 * PF_PT / a.group) * nw;
            const dim3 g2((a.n_rows + rows_wg - 1) / rows_wg, c.n_kv);
            hipLaunchKernelGGL(kernel, g2, dim3(nw * 64), 0, s, a);
        };
        if (c.head_dim == 128) {
            if (a.soft) go(prefill_bf16_kernel<128, true>, PfShape<128>::NW);
            else go(prefill_bf16_kernel<128, false>, PfShape<128>::NW);
        } else {
            if (a.soft) go(prefill_bf16_kernel<64, true>, PfShape<64>::NW);
            else go(prefill_bf16_kernel<64, false>, PfShape<64>::NW);
        }
        return hipGetLastError();
    }
    if (c.dtype == SPKV_BF16) {
        if (c.head_dim == 128)
            hipLaunchKernelGGL((prefill_valu_kernel<__bf16, 128>), grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_valu_kernel<__bf16, 64>), grid, dim3(64), 0, s, a);
    } else {
        if (c.head_dim == 128)
            hipLaunchKernelGGL((prefill_valu_kernel<float, 128>), grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_valu_kernel<float, 64>), grid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace spkv
