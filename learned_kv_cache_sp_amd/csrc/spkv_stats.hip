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
// Two launches: workgroup b sums a fixed band of the data per head (thread
// partials in order, then a fixed-shape reduction across the workgroup) into
// the workspace; one workgroup adds the band sums to the accumulators in a
// fixed order.  The band layout depends only on the sizes (and on whether
// the vector path is taken), so results are deterministic.  HBM-bound: 5
// bytes per (row, head), read once.
//
// Vector path (n_kv a power of two, utility 16-byte and keep 4-byte
// aligned): the data are read as one flat array, 4 elements (16 + 4 bytes)
// per thread and step; bands start at multiples of 1024 elements, so element
// q of thread t always belongs to head (4 t + q) mod n_kv.  Otherwise one row
// per thread and step.
#include "spkv_internal.h"

namespace spkv {
namespace {

constexpr int NT = 256;
constexpr int MAX_KV = 16;
constexpr int MAX_BANDS = 1024;

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

__global__ void __launch_bounds__(NT) stats_band_vec_kernel(StatsArgs a) {
    __shared__ double lds_u[4 * NT];
    __shared__ int lds_k[4 * NT];
    const int nkv = a.n_kv;
    const int64_t total = a.n_rows * nkv;
    const int64_t f0 = (int64_t)blockIdx.x * a.band_rows;  // band length in elements here
    const int64_t f1 = min(total, f0 + a.band_rows);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    int cnt[4] = {0, 0, 0, 0};
    typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll 4
    for (int64_t f = f0 + 4 * (int)threadIdx.x; f < f1; f += 4 * NT) {
        if (f + 4 <= f1) {
            if (a.utility) {
                const f32x4 x = *(const f32x4 *)(a.utility + f);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] += (double)x[q];
            }
            if (a.keep) {
                const uint32_t k = *(const uint32_t *)(a.keep + f);
#pragma unroll
                for (int q = 0; q < 4; ++q) cnt[q] += ((k >> (8 * q)) & 0xffu) != 0;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (f + q < f1) {
                    if (a.utility) acc[q] += (double)a.utility[f + q];
                    if (a.keep) cnt[q] += a.keep[f + q] != 0;
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        lds_u[4 * threadIdx.x + q] = acc[q];
        lds_k[4 * threadIdx.x + q] = cnt[q];
    }
    __syncthreads();
    if ((int)threadIdx.x < nkv) {
        double su = 0.0;
        int64_t sk = 0;
        for (int i = threadIdx.x; i < 4 * NT; i += nkv) {
            su += lds_u[i];
            sk += lds_k[i];
        }
        a.ws_u[(int64_t)blockIdx.x * nkv + threadIdx.x] = su;
        a.ws_k[(int64_t)blockIdx.x * nkv + threadIdx.x] = sk;
    }
}

__global__ void __launch_bounds__(NT) stats_band_kernel(StatsArgs a) {
    __shared__ double lds_u[NT / 64][MAX_KV];
    __shared__ int lds_k[NT / 64][MAX_KV];
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
    if ((int)threadIdx.x < nkv) {
        double su = 0.0;
        int64_t sk = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            su += lds_u[w][threadIdx.x];
            sk += lds_k[w][threadIdx.x];
        }
        a.ws_u[(int64_t)blockIdx.x * nkv + threadIdx.x] = su;
        a.ws_k[(int64_t)blockIdx.x * nkv + threadIdx.x] = sk;
    }
}

// Band sums of each head added up: thread t takes head t mod n_kv and the
// bands part, part + per, ... (part = t / n_kv, per = NT / n_kv threads per
// head) in order; then, per head, the per-thread sums in part order.
__global__ void __launch_bounds__(NT) stats_total_kernel(StatsArgs a) {
    __shared__ double lds_u[NT];
    __shared__ int64_t lds_k[NT];
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
            su += a.ws_u[(int64_t)b * nkv + g];
            sk += a.ws_k[(int64_t)b * nkv + g];
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

bool use_vec(const StatsArgs &a) {
    const int k = a.n_kv;
    return (k & (k - 1)) == 0 && ((uintptr_t)a.utility & 15) == 0 && ((uintptr_t)a.keep & 3) == 0;
}

// vector path: bands of whole multiples of 4 NT elements; otherwise of NT
// rows; at most MAX_BANDS of them
void plan(int64_t n_rows, int n_kv, bool vec, int64_t *band, int *n_bands) {
    const int64_t n = vec ? n_rows * n_kv : n_rows;
    const int64_t unit = vec ? 4 * NT : NT;
    const int64_t per = (n + MAX_BANDS - 1) / MAX_BANDS;
    int64_t br = ((per + unit - 1) / unit) * unit;
    if (br < unit) br = unit;
    *band = br;
    *n_bands = (int)((n + br - 1) / br);
}

}  // namespace

size_t stats_ws_bytes(int64_t n_rows, int n_kv) {
    // the larger of the two layouts' needs (at most MAX_BANDS bands each)
    int64_t br;
    int nb0, nb1;
    plan(n_rows, n_kv, false, &br, &nb0);
    plan(n_rows, n_kv, true, &br, &nb1);
    return (size_t)(nb0 > nb1 ? nb0 : nb1) * n_kv * (sizeof(double) + sizeof(int64_t));
}

hipError_t launch_stats(const StatsArgs &a0, hipStream_t s) {
    StatsArgs a = a0;
    const bool vec = use_vec(a);
    plan(a.n_rows, a.n_kv, vec, &a.band_rows, &a.n_bands);
    a.ws_u = (double *)a.ws;
    a.ws_k = (int64_t *)(a.ws_u + (int64_t)a.n_bands * a.n_kv);
    if (a.n_bands > 0) {
        if (vec)
            hipLaunchKernelGGL(stats_band_vec_kernel, dim3(a.n_bands), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL(stats_band_kernel, dim3(a.n_bands), dim3(NT), 0, s, a);
    }
    hipLaunchKernelGGL(stats_total_kernel, dim3(1), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace spkv
