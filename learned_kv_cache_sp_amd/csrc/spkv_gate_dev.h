// Device pieces of the few-row gate (SP-KV, arXiv 2605.14037, section 2.1,
// Eq. (1)-(2)), shared by the gate kernels and the fused decode step:
//   gate_unit_share / gate_finish (f32): workgroup j takes hidden unit j for
//     every row and stores its share W2[k][j] * a_j of every logit; the last
//     workgroup adds the shares in unit order, then sigmoid and threshold
//   gate_tile_share / gate_tile_finish (bf16): workgroups take 16-unit tiles
//     of the first layer on MFMA; the finishing workgroup adds the parts,
//     then ReLU, the second layer, sigmoid and threshold
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

// ---------------------------------------------------------------------------
// Few rows (<= 16), bf16, on MFMA.  Work item (tile, kpart): the first-layer
// pre-activations W1 h of hidden units 16*tile .. 16*tile+15 for every row,
// summed over the kpart-th part of d_model.  v_mfma_f32_16x16x32_bf16 with
// A = the hidden rows (row = lane % 16) and B = the W1 rows (unit = lane %
// 16), both read K-contiguous straight from memory: each lane loads 16 bytes
// per 32-wide slice.  A part is at most 4 waves x GT_SLICES slices, so every
// load of a wave is in flight at once.
constexpr int GT_SLICES = 16;

__host__ __device__ inline int gate_tile_kparts(int d_model) {
    const int steps = d_model / 32;
    return (steps + 4 * GT_SLICES - 1) / (4 * GT_SLICES);
}
__host__ __device__ inline int gate_tile_items(int d_model, int d_hidden) {
    return (d_hidden / 16) * gate_tile_kparts(d_model);
}

typedef __bf16 gt_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gt_f32x4 __attribute__((ext_vector_type(4)));

// All 256 threads.  part: [items][16 rows][16 units] floats, stored
// device-wide (rows past n_rows hold sums of a repeated row, never used);
// red: LDS scratch of 4 x 16 x 17 floats.
__device__ inline void gate_tile_share(const GateArgs &a, int item, float *part, float *red) {
    const int kparts = gate_tile_kparts(a.d_model);
    const int tile = item / kparts;
    const int kpart = item - tile * kparts;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const int steps = a.d_model / 32;
    const int spk = (steps + kparts - 1) / kparts;
    const int s_lo = kpart * spk;
    const int s_hi = min(steps, s_lo + spk);
    const int n = (int)a.n_rows;
    const int row = i16 < n ? i16 : n - 1;
    const __bf16 *hrow = (const __bf16 *)a.hidden + (int64_t)row * a.ld_hidden + 8 * q4;
    const __bf16 *wrow = (const __bf16 *)a.w1 + (int64_t)(16 * tile + i16) * a.d_model + 8 * q4;
    gt_bf16x8 av[GT_SLICES], bv[GT_SLICES];
#pragma unroll
    for (int u = 0; u < GT_SLICES; ++u) {
        const int s = s_lo + wave + 4 * u;
        const int se = s < s_hi ? s : s_lo;  // in bounds; zeroed below
        av[u] = *(const gt_bf16x8 *)(hrow + 32 * se);
        bv[u] = *(const gt_bf16x8 *)(wrow + 32 * se);
    }
    gt_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < GT_SLICES; ++u) {
        const int s = s_lo + wave + 4 * u;
        const gt_bf16x8 ab = s < s_hi ? av[u] : gt_bf16x8{};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bv[u], acc, 0, 0, 0);
    }
    // D: row 4*q4 + r, unit i16; the 4 waves' sums added in wave order
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * q4 + r) * 17 + i16] = acc[r];
    __syncthreads();
    {
        const int r = threadIdx.x >> 4;
        const int j = threadIdx.x & 15;
        const float v = ((red[(0 * 16 + r) * 17 + j] + red[(1 * 16 + r) * 17 + j]) + red[(2 * 16 + r) * 17 + j]) +
                        red[(3 * 16 + r) * 17 + j];
        store_dev(part + (size_t)item * 256 + r * 16 + j, v);
    }
}

// All 256 threads of the finishing workgroup, once every item is stored:
// a_j = ReLU(sum over parts in order + b1_j) staged in act (LDS, n_rows x
// d_hidden floats), then logit (r, k) = sum over j in order of W2[k][j] a_j,
// + b2, u = sigmoid(logit), keep = u >= tau (NaN -> 0).  utility / keep in
// a may be NULL; keep_lds and u_lds (may be NULL) receive the bits and the
// utilities too.
__device__ inline void gate_tile_finish(const GateArgs &a, const float *part, float *act, uint8_t *keep_lds,
                                        float *u_lds = nullptr) {
    const int kparts = gate_tile_kparts(a.d_model);
    const int n = (int)a.n_rows;
    const int hg = a.d_hidden;
    const int nkv = a.n_kv;
    for (int idx = threadIdx.x; idx < n * hg; idx += 256) {
        const int r = idx / hg;
        const int j = idx - r * hg;
        const float *p = part + (size_t)(j >> 4) * kparts * 256 + r * 16 + (j & 15);
        float pre = 0.f;
        for (int kp = 0; kp < kparts; ++kp) pre += load_dev(p + (size_t)kp * 256);
        act[idx] = gate_relu(pre + a.b1[j]);
    }
    __syncthreads();
    for (int o = threadIdx.x; o < n * nkv; o += 256) {
        const int r = o / nkv;
        const int k = o - r * nkv;
        const float *w2 = a.w2 + (size_t)k * hg;
        const float *ar = act + r * hg;
        float s = 0.f;
#pragma unroll 16
        for (int j = 0; j < hg; ++j) s = fmaf(w2[j], ar[j], s);
        const float u = gate_sigmoid(s + a.b2[k]);
        const uint8_t z = (u >= a.tau) ? 1 : 0;  // NaN -> 0
        if (a.utility) a.utility[o] = u;
        if (a.keep) a.keep[o] = z;
        if (keep_lds) keep_lds[o] = z;
        if (u_lds) u_lds[o] = u;
    }
}

}  // namespace spkv
