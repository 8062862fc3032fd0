// Device pieces of the few-row gate (SP-KV, arXiv 2605.14037, section 2.1,
// Eq. (1)-(2)), shared by the gate kernel and the fused decode step:
//   gate_unit_share  -- workgroup j: hidden unit j for every row, its share
//                       W2[k][j] * a_j of every logit stored device-wide
//   gate_finish      -- the last workgroup: shares added in unit order,
//                       sigmoid and threshold
#pragma once

#include "spkv_internal.h"
#include "spkv_device.h"

namespace spkv {

__device__ inline float gate_sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ inline float gate_relu(float x) { return x < 0.f ? 0.f : x; }  // NaN passes

// All threads of the workgroup (NT threads, NT / 64 waves).  Rows past
// n_rows re-read the last row (their shares are stored but never used), so
// every load is unconditional and all are in flight at once.  part is
// [d_hidden][NR][n_kv] floats; red is LDS scratch of NT / 64 x NR floats.
template <typename T, int NR, int NT>
__device__ void gate_unit_share(const GateArgs &a, int j, float *part, float *red) {
    constexpr int V = 16 / sizeof(T);
    typedef T tvec __attribute__((ext_vector_type(V)));
    const int n = (int)a.n_rows;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nkv = a.n_kv;
    const T *w = (const T *)a.w1 + (int64_t)j * a.d_model;
    const T *h = (const T *)a.hidden;
    const int my_k = threadIdx.x % nkv;
    const float w2j = a.w2[(size_t)my_k * a.d_hidden + j];
    const float b1j = a.b1[j];
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
    int64_t roff[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) roff[r] = (int64_t)(r < n ? r : n - 1) * a.ld_hidden;
    const int nvec = a.d_model / V;
#pragma unroll 2
    for (int c = threadIdx.x; c < nvec; c += NT) {
        const tvec wv = *(const tvec *)(w + (int64_t)c * V);
        tvec hv[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) hv[r] = *(const tvec *)(h + roff[r] + (int64_t)c * V);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int e = 0; e < V; ++e) acc[r] = fmaf((float)wv[e], (float)hv[r][e], acc[r]);
    }
    // butterfly over the wave, all rows interleaved so the lane exchanges overlap
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] += __shfl_xor(acc[r], off);
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < NR; ++r) red[wave * NR + r] = acc[r];
    __syncthreads();
    if (threadIdx.x < NR * nkv) {
        const int r = threadIdx.x / nkv;
        const int k = threadIdx.x - r * nkv;  // == my_k
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < NT / 64; ++v) s += red[v * NR + r];
        const float act = gate_relu(s + b1j);
        store_dev(part + ((size_t)j * NR + r) * nkv + k, w2j * act);
    }
}

// All threads of the (last) workgroup: logit (r, k) = sum over units j in
// order of the shares, then u = sigmoid(logit + b2), keep = u >= tau (NaN ->
// 0).  TPO threads per logit each add a strided subset (all loads issued
// before any add), the TPO sums then added in a fixed tree.  keep_out may be
// NULL; keep_lds (NR * n_kv bytes, may be NULL) receives the bits as well.
template <int NR, int NT>
__device__ void gate_finish(const GateArgs &a, const float *part, uint8_t *keep_lds) {
    const int n = (int)a.n_rows;
    const int nkv = a.n_kv;
    const int outs = n * nkv;
    int tpo = 1;
    while (tpo * 2 * outs <= NT && tpo < 32) tpo *= 2;
    const int o = threadIdx.x / tpo;
    const int q = threadIdx.x - o * tpo;
    const float b2o = o < outs ? a.b2[o % nkv] : 0.f;
    float s = 0.f;
    if (o < outs) {
        const int r = o / nkv;
        const int k = o - r * nkv;
        const float *p = part + (size_t)r * nkv + k;
        const size_t stride = (size_t)NR * nkv;
        const int hg = a.d_hidden;
        for (int j0 = q; j0 < hg; j0 += 32 * tpo) {
            float v[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int jj = j0 + e * tpo;
                v[e] = jj < hg ? load_dev(p + (size_t)jj * stride) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 32; ++e) s += v[e];
        }
    }
    // lanes of a logit are consecutive and TPO <= 32 divides the wave
    for (int off = 1; off < tpo; off <<= 1) {
        const float y = __shfl_down(s, off);
        if ((q & (2 * off - 1)) == 0) s += y;
    }
    if (o < outs && q == 0) {
        const float u = gate_sigmoid(s + b2o);
        const uint8_t z = (u >= a.tau) ? 1 : 0;  // NaN -> 0
        if (a.utility) a.utility[o] = u;
        if (a.keep) a.keep[o] = z;
        if (keep_lds) keep_lds[o] = z;
    }
}

}  // namespace spkv
