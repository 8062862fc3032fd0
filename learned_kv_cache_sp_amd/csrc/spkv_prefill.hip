// Chunked-prefill attention of SP-KV (arXiv 2605.14037), section 2.1,
// Eq. (3)-(4), for the rows t = pos0 .. pos0 + n_rows - 1 of one sequence:
//   window keys  max(0, t-w+1) .. t   -- from this chunk's K/V when >= pos0,
//                                        from the ring when < pos0
//   global keys  cached entries with position <= t - w
// The chunk's kept rows were appended to the cache before this call, so a
// row also sees kept keys of its own chunk once they leave its window (Eq. 4
// is per token).
//
// This file holds the VALU form: one wave per (row, query head), online
// softmax over the key list.  It serves f32 caches and bf16 chunks.
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
