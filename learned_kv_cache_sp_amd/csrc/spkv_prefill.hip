// Chunked-prefill attention of SP-KV (arXiv 2605.14037), section 2.1,
// Eq. (3)-(4), for the rows t = pos0 .. pos0 + n_rows - 1 of one sequence:
//   window keys  max(0, t-w+1) .. t   -- from this chunk's K/V when >= pos0,
//                                        from the ring when < pos0
//   global keys  cached entries with position <= t - w
// The chunk's kept rows were appended to the cache before this call, so a
// row also sees kept keys of its own chunk once they leave its window (Eq. 4
// is per token).
//
// bf16 (MFMA): a workgroup of 4 waves takes 256 (row, query head) pairs of
// one key head -- 64 / G query positions per wave, all G heads of the group --
// and walks one list of 32-key blocks: the cached entries visible to its
// first row (no mask), the staircase of cached entries that only later rows
// see (mask pos <= t - w), and the window band (mask 0 <= t - s < w).  Each
// block is staged once in LDS (keys row-major, values transposed, rows padded
// against bank conflicts) and read by all four waves; the next block's loads
// are in flight while the current one is computed.  Per wave and block:
//   S^T[32 keys x 16 pairs] = K . Q^T       (v_mfma_f32_16x16x32_bf16)
//   O^T[hd x 16 pairs]     += V^T . P^T     (P as a bf16 pair, f32-accurate)
// for each of its 4 pair tiles, online softmax with a lazily updated max.
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
    auto visit = [&](const T *k, const T *v, int64_t vstride) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) s = fmaf(q[e], (float)k[lane + 64 * e], s);
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        s *= a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = o[e] * alpha + p * (float)v[(int64_t)(lane + 64 * e) * vstride];
        m = m_new;
    };
    // window band
    const int s_lo = max(0, t - w + 1);
    for (int s = s_lo; s <= t; ++s) {
        if (s >= a.pos0) {
            const int64_t r = (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD;
            visit((const T *)a.k + r, (const T *)a.v + r, 1);
        } else {
            const int slot = s % w;
            visit((const T *)c.ring_k + ((int64_t)bg * w + slot) * HD,
                  (const T *)c.ring_v + (int64_t)bg * HD * w + slot, w);
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
        visit((const T *)c.k_pages + ((int64_t)page * P + slot) * HD,
              (const T *)c.v_pages + (int64_t)page * HD * P + slot, P);
    }
    float *op = a.out + ((int64_t)i * a.n_q + h) * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[lane + 64 * e] = l > 0.f ? o[e] / l : 0.f;
    if (lane == 0 && a.lse) a.lse[(int64_t)i * a.n_q + h] = l > 0.f ? m + logf(l) : -INFINITY;
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int PF_NW = 4;           // waves per workgroup
constexpr int PF_NT = PF_NW * 64;
constexpr int PF_PT = 4;           // 16-pair MFMA column tiles per wave
constexpr int PF_KB = 32;          // keys per block
constexpr float PF_LOG2E = 1.4426950408889634f;
constexpr float PF_LN2 = 0.6931471805599453f;

__device__ inline int pf_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// position of cached entry j of (b, g)
__device__ inline int entry_pos(const CacheView &c, const int32_t *pt, int j) {
    const int page = pt[j >> c.page_shift];
    return c.pos_pages[(int64_t)page * c.page_size + (j & (c.page_size - 1))];
}

// number of cached entries of (b, g) with position <= x (positions increase
// along the list), by two rounds of parallel probes
__device__ int count_upto(const CacheView &c, const int32_t *pt, int len, int x, int *lds_cnt) {
    if (len <= 0 || x < 0) return 0;
    // round 1: NT evenly spaced probes -> a bracket of at most ceil(len/NT) entries
    const int step = (len + PF_NT - 1) / PF_NT;
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
    for (int jj = lo + 1 + threadIdx.x; jj - threadIdx.x < hi; jj += PF_NT) {
        const bool le2 = jj < hi && entry_pos(c, pt, jj) <= x;
        const uint64_t bal2 = __ballot(le2);
        if ((threadIdx.x & 63) == 0 && bal2) atomicAdd(&lds_cnt[1], __popcll(bal2));
    }
    __syncthreads();
    return lo + 1 + lds_cnt[1];
}

template <int HD>
__global__ void __launch_bounds__(PF_NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_bf16_kernel(PrefillArgs a) {
    constexpr int KROW = HD + 8;         // padded key row (elements)
    constexpr int VROW = PF_KB + 8;      // padded transposed value row
    constexpr int CPR = HD / 8;          // 16-byte chunks per key row
    __shared__ __bf16 lds_k[2][PF_KB][KROW];
    __shared__ __bf16 lds_vt[2][HD][VROW];
    __shared__ int lds_pos[2][PF_KB];
    __shared__ int lds_cnt[2];

    const CacheView &c = a.c;
    const int G = a.group;
    const int g = blockIdx.y;
    const int b = a.b;
    const int bg = b * c.n_kv + g;
    const int w = c.window;
    const int P = c.page_size;
    const int rows_wave = (16 * PF_PT) / G;           // query positions per wave
    const int rows_wg = rows_wave * PF_NW;
    const int r_base = blockIdx.x * rows_wg;           // chunk-relative first row
    const int t_min = a.pos0 + r_base;
    const int t_max = a.pos0 + min(a.n_rows, r_base + rows_wg) - 1;
    const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
    const int len = c.lengths[bg];

    // ---- the block list of this workgroup -----------------------------------
    const int n_full = count_upto(c, pt, len, t_min - w, lds_cnt);  // visible to every row
    const int n_part = count_upto(c, pt, len, t_max - w, lds_cnt);  // visible to the last row
    const int s_lo = max(0, t_min - w + 1);                          // window band
    const int nb_g = (n_part + PF_KB - 1) / PF_KB;
    const int nb_b = (t_max - s_lo + 1 + PF_KB - 1) / PF_KB;
    const int nb = nb_g + nb_b;

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

    // ---- staging: thread (key kk = tid / CPR, chunk ch = tid % CPR) for keys,
    // and (dim row e = tid / 4, chunk of 8 keys) for the transposed values ----
    // Each block needs 32 x CPR key chunks and HD x 4 value chunks; with 256
    // threads and HD = 128 that is two of each per thread.
    constexpr int KCH = PF_KB * CPR / PF_NT;     // key chunks per thread
    constexpr int VCH = HD * (PF_KB / 8) / PF_NT; // value chunks per thread
    i32x4 kst[KCH], vst[VCH];
    int pst = 0;
    // value staging for band keys taken from this chunk's rows (row-major V):
    // thread loads V[key][8 dims] and scatters it into 8 transposed rows
    auto load_block = [&](int blk) {
        if (blk < nb_g) {
            const int j0 = blk * PF_KB;
            const int page = pt[j0 >> c.page_shift];
            const int slot0 = j0 & (P - 1);
            const int n_ok = min(PF_KB, n_part - j0);
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                const int kk = id / CPR, ch = id % CPR;
                kst[u] = kk < n_ok ? *(const i32x4 *)((const __bf16 *)c.k_pages + ((int64_t)page * P + slot0 + kk) * HD + 8 * ch)
                                   : i32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                const int e = id / (PF_KB / 8), kc = id % (PF_KB / 8);
                i32x4 v = *(const i32x4 *)((const __bf16 *)c.v_pages + ((int64_t)page * HD + e) * P + slot0 + 8 * kc);
                // keys beyond n_part hold other data: zero them
                const int first = 8 * kc;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = first + 2 * q;
                    const uint32_t mk = (k0 < n_ok ? 0x0000ffffu : 0u) | (k0 + 1 < n_ok ? 0xffff0000u : 0u);
                    v[q] &= (int32_t)mk;
                }
                vst[u] = v;
            }
            if (threadIdx.x < PF_KB) pst = threadIdx.x < n_ok ? c.pos_pages[(int64_t)page * P + slot0 + threadIdx.x] : INT_MAX;
        } else {
            const int s0 = s_lo + (blk - nb_g) * PF_KB;
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                const int kk = id / CPR, ch = id % CPR;
                const int s = s0 + kk;
                i32x4 kv = i32x4{0, 0, 0, 0};
                if (s <= t_max) {
                    if (s >= a.pos0)
                        kv = *(const i32x4 *)((const __bf16 *)a.k + (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD + 8 * ch);
                    else
                        kv = *(const i32x4 *)((const __bf16 *)c.ring_k + ((int64_t)bg * w + (s % w)) * HD + 8 * ch);
                }
                kst[u] = kv;
            }
            // values: from chunk rows (row-major) -> chunk of 8 dims of one key;
            // from the ring (transposed) -> 8 keys of one dim.  Band keys below
            // pos0 come first in the band, so a block mixes the two only once.
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                // row-major source: key kk2, dims 8*dc .. 8*dc+7
                const int kk2 = id / CPR, dc = id % CPR;
                const int s = s0 + kk2;
                i32x4 vv = i32x4{0, 0, 0, 0};
                if (s <= t_max) {
                    if (s >= a.pos0) {
                        vv = *(const i32x4 *)((const __bf16 *)a.v + (int64_t)(s - a.pos0) * a.ld_kv + (int64_t)g * HD + 8 * dc);
                    } else {
                        const __bf16 *rv = (const __bf16 *)c.ring_v + (int64_t)bg * HD * w + (s % w);
                        __bf16 tmp[8];
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) tmp[e2] = rv[(int64_t)(8 * dc + e2) * w];
                        vv = __builtin_bit_cast(i32x4, *(bf16x8 *)tmp);
                    }
                }
                vst[u] = vv;
            }
            if (threadIdx.x < PF_KB) pst = s0 + threadIdx.x;
        }
    };
    auto store_block = [&](int blk, int buf) {
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int id = threadIdx.x + u * PF_NT;
            const int kk = id / CPR, ch = id % CPR;
            *(i32x4 *)&lds_k[buf][kk][8 * ch] = kst[u];
        }
        if (blk < nb_g) {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                const int e = id / (PF_KB / 8), kc = id % (PF_KB / 8);
                *(i32x4 *)&lds_vt[buf][e][8 * kc] = vst[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int id = threadIdx.x + u * PF_NT;
                const int kk2 = id / CPR, dc = id % CPR;
                const bf16x8 vv = __builtin_bit_cast(bf16x8, vst[u]);
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) lds_vt[buf][8 * dc + e2][kk2] = vv[e2];
            }
        }
        if (threadIdx.x < PF_KB) lds_pos[buf][threadIdx.x] = pst;
    };

    // ---- per-wave online softmax state over its 4 pair tiles ----------------
    f32x4 o[PF_PT][HD / 16];
    float m[PF_PT], l[PF_PT];
#pragma unroll
    for (int ptl = 0; ptl < PF_PT; ++ptl) {
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) o[ptl][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[ptl] = -INFINITY;
        l[ptl] = 0.f;
    }

    if (nb > 0) {
        load_block(0);
        store_block(0, 0);
    }
    __syncthreads();
    for (int blk = 0; blk < nb; ++blk) {
        const int buf = blk & 1;
        if (blk + 1 < nb) load_block(blk + 1);
        // kind of block: 0 fully visible cached, 1 staircase cached, 2 band
        const int kind = blk < nb_g ? ((blk + 1) * PF_KB <= n_full ? 0 : 1) : 2;
        // key rows of the A operand: tile tt row i -> key 8*(i/4) + 4*tt + i%4
        bf16x8 ka[2][HD / 32];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int key = 8 * (i16 >> 2) + 4 * tt + (i16 & 3);
#pragma unroll
            for (int cc = 0; cc < HD / 32; ++cc) ka[tt][cc] = *(const bf16x8 *)&lds_k[buf][key][32 * cc + 8 * q4];
        }
        // this lane's 8 keys: 8*q4 + e (positions / entry positions)
        int kpos[8];
        if (kind != 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kpos[e] = lds_pos[buf][8 * q4 + e];
        }
        bf16x8 pb[PF_PT], pl[PF_PT];
#pragma unroll
        for (int ptl = 0; ptl < PF_PT; ++ptl) {
            f32x4 sacc[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int cc = 0; cc < HD / 32; ++cc)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][cc], qr[ptl][cc], acc, 0, 0, 0);
                sacc[tt] = acc;
            }
            const int t = trow[ptl];
            float x[8];
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = sacc[e >> 2][e & 3] * sl2;
                if (kind == 1) v = (kpos[e] <= t - w) ? v : -INFINITY;
                else if (kind == 2) v = (t - kpos[e] >= 0 && t - kpos[e] < w) ? v : -INFINITY;
                x[e] = v;
                mloc = fmaxf(mloc, v);
            }
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
            const float base = (m[ptl] == -INFINITY) ? 0.f : m[ptl];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(x[e] - base);
                psum += pe;
                pb[ptl][e] = (__bf16)pe;
                pl[ptl][e] = (__bf16)(pe - (float)pb[ptl][e]);
            }
            l[ptl] += psum;
        }
        // O^T += V^T . P^T; the V^T operand is shared by the 4 pair tiles
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) {
            const bf16x8 va = *(const bf16x8 *)&lds_vt[buf][16 * nt + i16][8 * q4];
#pragma unroll
            for (int ptl = 0; ptl < PF_PT; ++ptl) {
                o[ptl][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ptl], o[ptl][nt], 0, 0, 0);
                o[ptl][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[ptl], o[ptl][nt], 0, 0, 0);
            }
        }
        if (blk + 1 < nb) store_block(blk + 1, buf ^ 1);
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
        const int rows_wg = (16 * PF_PT / a.group) * PF_NW;
        const dim3 g2((a.n_rows + rows_wg - 1) / rows_wg, c.n_kv);
        if (c.head_dim == 128)
            hipLaunchKernelGGL(prefill_bf16_kernel<128>, g2, dim3(PF_NT), 0, s, a);
        else
            hipLaunchKernelGGL(prefill_bf16_kernel<64>, g2, dim3(PF_NT), 0, s, a);
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
