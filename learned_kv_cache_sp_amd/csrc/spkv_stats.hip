// Per-head utility statistics of the gate's outputs.
//
// SP-KV (arXiv 2605.14037) measures a model's density as the share of the
// pairs outside the local window that the gate keeps (Table 1 caption) and
// picks the heads that stay global in a local/global hybrid by their mean
// learned utility (section 1, contribution 2; section 4).  For n rows of gate
// output u [n, n_kv] f32 and keep [n, n_kv] u8 this adds, per key head g, the
// sum of u[., g] (in double) and the count of keep[., g] != 0 to the caller's
// accumulators.
//
// One launch: workgroup b sums a fixed band of the data per head (thread
// partials in order, then a fixed-shape reduction across the workgroup),
// stores the band's sums device-wide and counts itself (in one of 16 group
// counters, the last of each group at a top counter); the workgroup that
// arrives last adds the band sums to the accumulators in a fixed order.  The
// band layout depends only on the sizes (and on whether the vector path is
// taken), so results are deterministic.  HBM-bound: 5 bytes per (row, head),
// read once.
//
// Vector path (n_kv a power of two, utility and keep 16-byte aligned): the
// data are read as one flat array, 1024 elements per wave and step in 1 KB
// loads; bands start at multiples of 4096 elements, so the head of an element
// follows from its lane and slot alone.  Otherwise one row per thread and
// step.
#include "spkv_internal.h"
#include "spkv_device.h"

namespace spkv {
namespace {

constexpr int NT = 256;
constexpr int MAX_KV = 16;
constexpr int MAX_BANDS = 256;  // one workgroup per compute unit
// workspace: a header of 1 + ARRIVE_GROUPS 256-byte lines holding the arrival
// counters, then the band sums
constexpr int ARRIVE_GROUPS = 16;
constexpr size_t STATS_HEADER = 256 * (1 + ARRIVE_GROUPS);

__device__ inline double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ inline int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Band sums of the vector path, left in lds_u / lds_k [NT / 64][MAX_KV] (one
// entry per wave and head).  Per step a wave reads 1024 consecutive elements
// with five load instructions of 1 KB each: four of utilities (lane l holds
// elements 256 i + 4 l + c, head (4 l + c) mod n_kv) and one of keep bytes
// (lane l holds elements 16 l + q, head q mod n_kv); the loads of U steps are
// issued before any is used.
__device__ void band_vec(const StatsArgs &a, double *lds_u, int *lds_k) {
    constexpr int U = 8;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int nkv = a.n_kv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t total = a.n_rows * nkv;
    const int64_t f0 = (int64_t)blockIdx.x * a.band_rows;  // band length in elements here
    const int64_t f1 = min(total, f0 + a.band_rows);
    double acc[4][4];
    int cnt[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) cnt[q] = 0;
    for (int64_t base = f0 + 1024 * wave; base < f1; base += U * 4096) {
        f32x4 x[U][4];
        u32x4 k[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t f = base + (int64_t)u * 4096;
            const bool full = f + 1024 <= f1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[u][i] = (a.utility && full) ? __builtin_nontemporal_load((const f32x4 *)(a.utility + f + 256 * i) + lane)
                                              : f32x4{0.f, 0.f, 0.f, 0.f};
            k[u] = (a.keep && full) ? __builtin_nontemporal_load((const u32x4 *)(a.keep + f) + lane) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t f = base + (int64_t)u * 4096;
            if (f + 1024 <= f1) {
                if (a.utility) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[i][c] += (double)x[u][i][c];
                }
                if (a.keep) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) cnt[q] += ((k[u][q >> 2] >> (8 * (q & 3))) & 0xffu) != 0;
                }
            } else if (f < f1) {
                for (int i = 0; i < 4; ++i)
                    for (int c = 0; c < 4; ++c) {
                        const int64_t e = f + 256 * i + 4 * lane + c;
                        if (a.utility && e < f1) acc[i][c] += (double)a.utility[e];
                    }
                for (int q = 0; q < 16; ++q) {
                    const int64_t e = f + 16 * lane + q;
                    if (a.keep && e < f1) cnt[q] += a.keep[e] != 0;
                }
            }
        }
    }
    // per head: the thread's slots in slot order, then a fixed butterfly over
    // the wave, then (by the caller) the waves in order
    double hu[MAX_KV];
    int hk[MAX_KV];
#pragma unroll
    for (int g = 0; g < MAX_KV; ++g) {
        hu[g] = 0.0;
        hk[g] = 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int hg = (4 * lane + c) & (nkv - 1);
#pragma unroll
            for (int g = 0; g < MAX_KV; ++g)
                if (g == hg) hu[g] += acc[i][c];
        }
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int g = 0; g < MAX_KV; ++g)
            if (g == (q & (nkv - 1))) hk[g] += cnt[q];
#pragma unroll
    for (int g = 0; g < MAX_KV; ++g) {
        if (g < nkv) {
            const double su = wave_sum(hu[g]);
            const int sk = wave_sum(hk[g]);
            if (lane == 0) {
                lds_u[wave * MAX_KV + g] = su;
                lds_k[wave * MAX_KV + g] = sk;
            }
        }
    }
    __syncthreads();
}

// Band sums of the row path, left in lds_u / lds_k [NT / 64][MAX_KV] (one
// entry per wave and head).
__device__ void band_rows(const StatsArgs &a, double (*lds_u)[MAX_KV], int (*lds_k)[MAX_KV]) {
    const int nkv = a.n_kv;
    const int64_t r0 = (int64_t)blockIdx.x * a.band_rows;
    const int64_t r1 = min(a.n_rows, r0 + a.band_rows);
    double acc[MAX_KV];
    int cnt[MAX_KV];
#pragma unroll
    for (int g = 0; g < MAX_KV; ++g) {
        acc[g] = 0.0;
        cnt[g] = 0;
    }
#pragma unroll 4
    for (int64_t r = r0 + threadIdx.x; r < r1; r += NT) {
#pragma unroll
        for (int g = 0; g < MAX_KV; ++g) {
            if (g < nkv) {
                if (a.utility) acc[g] += (double)a.utility[r * nkv + g];
                if (a.keep) cnt[g] += a.keep[r * nkv + g] != 0;
            }
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int g = 0; g < MAX_KV; ++g) {
        if (g < nkv) {
            const double su = wave_sum(acc[g]);
            const int sk = wave_sum(cnt[g]);
            if (lane == 0) {
                lds_u[wave][g] = su;
                lds_k[wave][g] = sk;
            }
        }
    }
    __syncthreads();
}

// Band sums of each head added up, by the workgroup that arrived last:
// thread t takes head t mod n_kv and the bands part, part + per, ... (part =
// t / n_kv, per = NT / n_kv threads per head) in order; then, per head, the
// per-thread sums in part order.  The band sums were stored device-wide by
// their workgroups and are read device-wide here.
__device__ void stats_finish(const StatsArgs &a, double *lds_u, int64_t *lds_k) {
    const int nkv = a.n_kv;
    const int per = NT / nkv;
    const int t = threadIdx.x;
    if (t < per * nkv) {
        const int g = t % nkv;
        const int part = t / nkv;
        double su = 0.0;
        int64_t sk = 0;
#pragma unroll 8
        for (int b = part; b < a.n_bands; b += per) {
            su += __hip_atomic_load(a.ws_u + (int64_t)b * nkv + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sk += __hip_atomic_load(a.ws_k + (int64_t)b * nkv + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        lds_u[t] = su;
        lds_k[t] = sk;
    }
    __syncthreads();
    if (t < nkv) {
        double tu = 0.0;
        int64_t tk = 0;
        for (int p = 0; p < per; ++p) {
            tu += lds_u[p * nkv + t];
            tk += lds_k[p * nkv + t];
        }
        if (a.utility) a.u_sum[t] += tu;
        if (a.keep) a.n_kept[t] += tk;
    }
}

template <bool VEC>
__global__ void __launch_bounds__(NT) stats_kernel(StatsArgs a) {
    __shared__ double lds_u[NT];   // band sums per (wave, head), then the finish's per-thread sums
    __shared__ int64_t lds_k8[NT];
    __shared__ int lds_k[NT];
    __shared__ int lds_last;
    const int nkv = a.n_kv;
    double su = 0.0;
    int64_t sk = 0;
    double (*lu)[MAX_KV] = (double (*)[MAX_KV])lds_u;
    int (*lk)[MAX_KV] = (int (*)[MAX_KV])lds_k;
    if constexpr (VEC) band_vec(a, lds_u, lds_k);
    else band_rows(a, lu, lk);
    if ((int)threadIdx.x < nkv)
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            su += lu[w][threadIdx.x];
            sk += lk[w][threadIdx.x];
        }
    // this band's sums, device-wide; each storing thread waits for its stores
    // before the workgroup counts itself
    if ((int)threadIdx.x < nkv) {
        __hip_atomic_store(a.ws_u + (int64_t)blockIdx.x * nkv + threadIdx.x, su, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.ws_k + (int64_t)blockIdx.x * nkv + threadIdx.x, sk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    // arrival in two levels, so that the bands finishing together do not all
    // queue on one word: band b counts in group b mod ARRIVE_GROUPS (a
    // 256-byte line each), the last of a group counts at the top
    if (threadIdx.x == 0) {
        const int grp = (int)blockIdx.x % ARRIVE_GROUPS;
        const int in_grp = (a.n_bands - grp + ARRIVE_GROUPS - 1) / ARRIVE_GROUPS;
        int *gc = a.cnt + 64 * (1 + grp);
        bool last = arrive_dev(gc) == in_grp - 1;
        if (last) {
            reset_dev(gc);
            last = arrive_dev(a.cnt) == min(a.n_bands, ARRIVE_GROUPS) - 1;
            if (last) reset_dev(a.cnt);  // every counter is back to zero for the next call
        }
        lds_last = last;
    }
    __syncthreads();
    if (!lds_last) return;
    stats_finish(a, lds_u, lds_k8);
}

bool use_vec(const StatsArgs &a) {
    const int k = a.n_kv;
    return (k & (k - 1)) == 0 && ((uintptr_t)a.utility & 15) == 0 && ((uintptr_t)a.keep & 15) == 0;
}

// vector path: bands of whole multiples of 16 NT elements; otherwise of NT
// rows; at most MAX_BANDS of them
void plan(int64_t n_rows, int n_kv, bool vec, int64_t *band, int *n_bands) {
    const int64_t n = vec ? n_rows * n_kv : n_rows;
    const int64_t unit = vec ? 16 * NT : NT;
    const int64_t per = (n + MAX_BANDS - 1) / MAX_BANDS;
    int64_t br = ((per + unit - 1) / unit) * unit;
    if (br < unit) br = unit;
    *band = br;
    *n_bands = (int)((n + br - 1) / br);
}

}  // namespace

size_t stats_ws_bytes(int64_t n_rows, int n_kv) {
    if (n_rows <= 0) return 0;
    // the larger of the two layouts' needs (at most MAX_BANDS bands each)
    int64_t br;
    int nb0, nb1;
    plan(n_rows, n_kv, false, &br, &nb0);
    plan(n_rows, n_kv, true, &br, &nb1);
    return STATS_HEADER + (size_t)(nb0 > nb1 ? nb0 : nb1) * n_kv * (sizeof(double) + sizeof(int64_t));
}

hipError_t launch_stats(const StatsArgs &a0, hipStream_t s) {
    StatsArgs a = a0;
    const bool vec = use_vec(a);
    plan(a.n_rows, a.n_kv, vec, &a.band_rows, &a.n_bands);
    a.cnt = (int *)a.ws;
    a.ws_u = (double *)((char *)a.ws + STATS_HEADER);
    a.ws_k = (int64_t *)(a.ws_u + (int64_t)a.n_bands * a.n_kv);
    if (vec)
        hipLaunchKernelGGL(stats_kernel<true>, dim3(a.n_bands), dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL(stats_kernel<false>, dim3(a.n_bands), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace spkv
