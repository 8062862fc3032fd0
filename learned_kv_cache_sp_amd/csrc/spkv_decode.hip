// Decode attention over the window ring plus the kept (global) entries.
//
// SP-KV (arXiv 2605.14037), section 2.1, Eq. (3)-(4): query t of head h sees
// the keys of its key head g = h / G that are inside the causal window
// (0 <= t - s < w) or were kept (z_s = 1, s <= t); softmax with scale
// 1/sqrt(d_k).  At deployment the kept keys live in the persistent cache and
// the window in a ring (section 2.1, deployment paragraph); a kept key still
// inside the window is read from the ring only (its cache entry is skipped by
// position), so every visible key counts once.  Decode is bound by the
// KV-cache read (sections 1 and 3.4), so this kernel is built to stream it.
//
// Work decomposition (flat split-K list, built on the device):
//   every (b, g) owns ceil(len[b][g] / C) chunks of C cached entries plus one
//   window item; the chunk size C is chosen by every workgroup from the
//   lengths, the same way, so that the list has about 2x as many items as the
//   grid has workgroups.  Persistent workgroups walk the list; each item is
//   split over the 4 waves, merged in LDS and written as a partial
//   (max, sum, unnormalised output) per query head; the last workgroup to
//   finish an item of (b, g) (device-scope counter) merges its partials in
//   item order -- deterministic -- and writes out and lse.
//
// Inner loop (bf16, one wave, 32 keys per step):
//   S[32 keys x 16 heads] = K . Q^T   two v_mfma_f32_16x16x32_bf16 tiles x hd/32
//   O^T[hd x 16 heads]   += V^T . P   2 x hd/16 MFMAs (V pages are stored
//                                      transposed, so both operands load as
//                                      16-byte rows; P is split into a bf16
//                                      pair so the product is f32-accurate)
//   The G query heads of the key head share every K/V load (rows >= G of the
//   query operand are zero).  Online softmax in the log2 domain.
#include "spkv_internal.h"

namespace spkv {
namespace {

constexpr int NT = 256;
constexpr int NW = 4;
constexpr int KSTEP = 32;
constexpr int MAX_BG = 2048;
constexpr int MAX_ITEMS_PER_BG = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct Plan {
    int chunk;      // C
    int total;      // items
};

// Every workgroup derives the same work list from lengths[].
__device__ Plan build_plan(const DecodeArgs &a, int *lds_first /*[MAX_BG+1]*/, int *lds_red) {
    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    int tot_len = 0, max_len = 0;
    for (int i = threadIdx.x; i < BG; i += NT) {
        const int l = c.lengths[i];
        tot_len += l;
        max_len = max(max_len, l);
    }
    // block reduce (sum, max)
    for (int off = 32; off > 0; off >>= 1) {
        tot_len += __shfl_xor(tot_len, off);
        max_len = max(max_len, __shfl_xor(max_len, off));
    }
    if ((threadIdx.x & 63) == 0) {
        lds_red[threadIdx.x >> 6] = tot_len;
        lds_red[NW + (threadIdx.x >> 6)] = max_len;
    }
    __syncthreads();
    int64_t T = 0;
    int M = 0;
    for (int w = 0; w < NW; ++w) {
        T += lds_red[w];
        M = max(M, lds_red[NW + w]);
    }
    const int64_t target = 2 * (int64_t)gridDim.x;
    int C = 128;
    while ((int64_t)C * target < T && C < (1 << 20)) C <<= 1;
    while ((int64_t)C * (MAX_ITEMS_PER_BG - 1) < M && C < (1 << 20)) C <<= 1;
    // inclusive prefix of items per (b, g): serial over chunks of NT with a
    // block scan (BG is at most a few thousand)
    int carry = 0;
    for (int base = 0; base < BG; base += NT) {
        const int i = base + threadIdx.x;
        const int n = i < BG ? (c.lengths[i] + C - 1) / C + 1 : 0;
        // wave inclusive scan
        int x = n;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if ((threadIdx.x & 63) >= off) x += y;
        }
        __syncthreads();
        if ((threadIdx.x & 63) == 63) lds_red[2 * NW + (threadIdx.x >> 6)] = x;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < (threadIdx.x >> 6); ++w) before += lds_red[2 * NW + w];
        if (i < BG) lds_first[i + 1] = before + x;
        int step_total = 0;
        for (int w = 0; w < NW; ++w) step_total += lds_red[2 * NW + w];
        carry += step_total;
    }
    if (threadIdx.x == 0) lds_first[0] = 0;
    __syncthreads();
    Plan p;
    p.chunk = C;
    p.total = carry;
    return p;
}

__device__ inline int find_bg(const int *first, int BG, int item) {
    // largest bg with first[bg] <= item
    int lo = 0, hi = BG - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// One wave's pass over `n_steps` steps of 32 keys.  The key block of step i
// starts at entry e0 + 32 i of the list described by the callbacks.
template <int HD>
struct WaveState {
    f32x4 o[HD / 16];
    float m;     // running max (log2 domain), identical across the 4 lane groups
    float l;     // this lane's partial sum
};

template <int HD>
__device__ inline void load_step(const __bf16 *kblk, const __bf16 *vblk, int vstride,
                                 bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int q4 = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int key = 8 * (i >> 2) + 4 * t + (i & 3);
        const bf16x8 *src = (const bf16x8 *)(kblk + key * HD + (HD / 4) * q4);
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc) kr[t][cc] = src[cc];
    }
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt)
        vr[nt] = *(const bf16x8 *)(vblk + (int64_t)(16 * nt + i) * vstride + 8 * q4);
}

// valid: bit e set when key 8*(lane/16)+e of the step is visible (used only
// when MASKED; the unmasked form is taken for steps that are entirely visible,
// a wave-uniform decision).
template <int HD, bool MASKED>
__device__ inline void compute_step(WaveState<HD> &st, const bf16x8 (&qr)[HD / 32],
                                    const bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16],
                                    uint32_t valid, float sl2) {
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[t][cc], qr[cc], acc, 0, 0, 0);
        s[t] = acc;
    }
    float x[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = s[e >> 2][e & 3] * sl2;
        if (MASKED) x[e] = ((valid >> e) & 1u) ? x[e] : -INFINITY;
        mloc = fmaxf(mloc, x[e]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(st.m, mloc);
    // m_new == -inf only if nothing was visible so far: keep everything at 0
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    if (__builtin_expect(__ballot(m_new != st.m) != 0, 0)) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - base);  // st.m = -inf -> 0
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) st.o[nt] *= alpha;
        st.l *= alpha;
    }
    st.m = m_new;
    // P = P_hi + P_lo, both bf16: the value product is then exact to ~2^-17
    // relative (V is bf16, the MFMA accumulates in f32)
    bf16x8 pb, pl;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(x[e] - base);
        psum += p;
        pb[e] = (__bf16)p;
        pl[e] = (__bf16)(p - (float)pb[e]);
    }
    st.l += psum;
    if (MASKED) {
        // zero the values of invisible keys (their slots may hold anything):
        // element pair w of a lane's 8 keys is 32-bit word w
        uint32_t keepw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            keepw[w] = (((valid >> (2 * w)) & 1u) ? 0x0000ffffu : 0u) |
                       (((valid >> (2 * w + 1)) & 1u) ? 0xffff0000u : 0u);
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) {
            i32x4 wv = __builtin_bit_cast(i32x4, vr[nt]);
#pragma unroll
            for (int w = 0; w < 4; ++w) wv[w] &= (int32_t)keepw[w];
            vr[nt] = __builtin_bit_cast(bf16x8, wv);
        }
    }
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) {
        st.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[nt], pb, st.o[nt], 0, 0, 0);
        st.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[nt], pl, st.o[nt], 0, 0, 0);
    }
}

template <int HD>
__device__ inline void step(WaveState<HD> &st, const bf16x8 (&qr)[HD / 32],
                            const bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16],
                            uint32_t valid, bool all_visible, float sl2) {
    if (all_visible) compute_step<HD, false>(st, qr, kr, vr, 0xffu, sl2);
    else compute_step<HD, true>(st, qr, kr, vr, valid, sl2);
}

template <int HD>
__global__ void __launch_bounds__(NT) decode_bf16_kernel(DecodeArgs a) {
    __shared__ int lds_first[MAX_BG + 1];
    __shared__ int lds_red[3 * NW];
    __shared__ float lds_m[NW][16];
    __shared__ float lds_l[NW][16];
    __shared__ float lds_o[NW][16][HD];
    __shared__ int lds_flag;

    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int G = a.group;
    const Plan plan = build_plan(a, lds_first, lds_red);
    const int C = plan.chunk;
    if (plan.total > a.max_items) {  // cannot happen for caches below 2^30 entries
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(c.status, SPKV_STATUS_TABLE_FULL);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int head = lane & 15;
    const int q4 = lane >> 4;
    const float sl2 = a.scale * LOG2E;
    const int rec = G * (HD + 2);  // floats per partial
    int32_t *cnt = (int32_t *)a.ws;
    float *part = (float *)(a.ws + (((size_t)BG * 4 + 255) & ~(size_t)255));

    for (int item = blockIdx.x; item < plan.total; item += gridDim.x) {
        const int bg = find_bg(lds_first, BG, item);
        const int b = bg / c.n_kv;
        const int g = bg - b * c.n_kv;
        const int first = lds_first[bg];
        const int n_items = lds_first[bg + 1] - first;
        const int ci = item - first;
        const bool is_window = (ci == n_items - 1);
        const int t = a.t[b];
        const int len = c.lengths[bg];

        // query operand: head `head` of this group, zero rows beyond G
        bf16x8 qr[HD / 32];
        {
            const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.ld_q + (int64_t)(g * G + head) * HD +
                               (HD / 4) * q4;
#pragma unroll
            for (int cc = 0; cc < HD / 32; ++cc) {
                if (head < G) qr[cc] = *(const bf16x8 *)(qp + 8 * cc);
                else qr[cc] = bf16x8{};
            }
        }
        WaveState<HD> st;
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) st.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;

        if (is_window) {
            const int w = c.window;
            const int n_steps = w / KSTEP;
            const __bf16 *kb = (const __bf16 *)c.ring_k + (int64_t)bg * w * HD;
            const __bf16 *vb = (const __bf16 *)c.ring_v + (int64_t)bg * HD * w;
            for (int sidx = wave; sidx < n_steps; sidx += NW) {
                bf16x8 kr[2][HD / 32];
                bf16x8 vr[HD / 16];
                load_step<HD>(kb + (int64_t)sidx * KSTEP * HD, vb + sidx * KSTEP, w, kr, vr);
                // slot s holds position t - ((t - s) mod w); it is visible iff
                // that position is >= 0, i.e. s <= t
                uint32_t valid = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int slot = sidx * KSTEP + 8 * q4 + e;
                    valid |= (slot <= t ? 1u : 0u) << e;
                }
                step<HD>(st, qr, kr, vr, valid, t >= sidx * KSTEP + KSTEP - 1, sl2);
            }
        } else {
            const int e_lo = ci * C;
            const int e_hi = min(len, e_lo + C);
            const int n_steps_all = (e_hi - e_lo + KSTEP - 1) / KSTEP;
            // contiguous share of the steps for this wave
            const int per = (n_steps_all + NW - 1) / NW;
            const int s_lo = wave * per;
            const int s_hi = min(n_steps_all, s_lo + per);
            const int limit = t - c.window;  // cached entries need pos <= limit
            const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
            const int P = c.page_size;
            // two register buffers: the loads of step i+1 are in flight while
            // step i is computed
            bf16x8 kA[2][HD / 32], kB[2][HD / 32];
            bf16x8 vA[HD / 16], vB[HD / 16];
            auto issue = [&](int sidx, bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
                const int j0 = e_lo + sidx * KSTEP;
                const int page = pt[j0 >> c.page_shift];
                const int slot0 = j0 & (P - 1);
                const __bf16 *kb = (const __bf16 *)c.k_pages + ((int64_t)page * P + slot0) * HD;
                const __bf16 *vb = (const __bf16 *)c.v_pages + (int64_t)page * HD * P + slot0;
                load_step<HD>(kb, vb, P, kr, vr);
            };
            // entries below len - w are older than the window (positions
            // strictly increase and at most w entries lie inside it), so only
            // steps reaching past len - w (or past the item) read positions
            auto all_visible = [&](int sidx) -> bool {
                const int j0 = e_lo + sidx * KSTEP;
                return j0 + KSTEP <= e_hi && j0 + KSTEP <= len - c.window && limit >= 0;
            };
            auto visible = [&](int sidx) -> uint32_t {
                const int j0 = e_lo + sidx * KSTEP;
                const int jl = j0 + 8 * q4;  // this lane's first key
                const int page = pt[j0 >> c.page_shift];
                const i32x4 *pp = (const i32x4 *)(c.pos_pages + (int64_t)page * P + (jl & (P - 1)));
                const i32x4 p0 = pp[0], p1 = pp[1];
                uint32_t valid = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int pe = e < 4 ? p0[e] : p1[e - 4];
                    const bool ok = (jl + e < e_hi) && (pe <= limit);
                    valid |= (ok ? 1u : 0u) << e;
                }
                return valid;
            };
            if (s_lo < s_hi) issue(s_lo, kA, vA);
            for (int sidx = s_lo; sidx < s_hi; sidx += 2) {
                const bool two = sidx + 1 < s_hi;
                if (two) issue(sidx + 1, kB, vB);
                {
                    const bool av = all_visible(sidx);
                    step<HD>(st, qr, kA, vA, av ? 0xffu : visible(sidx), av, sl2);
                }
                if (sidx + 2 < s_hi) issue(sidx + 2, kA, vA);
                if (two) {
                    const bool av = all_visible(sidx + 1);
                    step<HD>(st, qr, kB, vB, av ? 0xffu : visible(sidx + 1), av, sl2);
                }
            }
        }

        // ---- merge the 4 waves of this item --------------------------------
        float lsum = st.l;
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        __syncthreads();
        if (q4 == 0) {
            lds_m[wave][head] = st.m;
            lds_l[wave][head] = lsum;
        }
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) lds_o[wave][head][16 * nt + 4 * q4 + r] = st.o[nt][r];
        __syncthreads();
        float *my = part + (size_t)item * rec;
        for (int idx = threadIdx.x; idx < G * HD; idx += NT) {
            const int h = idx / HD;
            const int d = idx - h * HD;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][h]);
            const float base = (M == -INFINITY) ? 0.f : M;
            float O = 0.f, L = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = exp2f(lds_m[w][h] - base);
                O += f * lds_o[w][h][d];
                L += f * lds_l[w][h];
            }
            my[2 * G + h * HD + d] = O;
            if (d == 0) {
                my[h] = M;
                my[G + h] = L;
            }
        }
        // ---- completion counter; the last item of (b, g) combines ----------
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const int prev = atomicAdd(&cnt[bg], 1);
            lds_flag = (prev == n_items - 1);
        }
        __syncthreads();
        if (lds_flag) {
            __threadfence();
            const float *pb = part + (size_t)first * rec;
            for (int idx = threadIdx.x; idx < G * HD; idx += NT) {
                const int h = idx / HD;
                const int d = idx - h * HD;
                float M = -INFINITY;
                for (int k = 0; k < n_items; ++k) M = fmaxf(M, __builtin_nontemporal_load(pb + (size_t)k * rec + h));
                const float base = (M == -INFINITY) ? 0.f : M;
                float O = 0.f, L = 0.f;
#pragma unroll 4
                for (int k = 0; k < n_items; ++k) {
                    const float *pk = pb + (size_t)k * rec;
                    const float f = exp2f(__builtin_nontemporal_load(pk + h) - base);
                    O += f * __builtin_nontemporal_load(pk + 2 * G + h * HD + d);
                    L += f * __builtin_nontemporal_load(pk + G + h);
                }
                const int64_t oidx = ((int64_t)b * a.n_q + g * G + h);
                a.out[oidx * HD + d] = L > 0.f ? O / L : 0.f;
                if (d == 0 && a.lse) a.lse[oidx] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
            }
            if (threadIdx.x == 0) cnt[bg] = 0;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// f32 caches: one wave per (b, query head), plain online softmax on VALU.
template <int HD>
__global__ void __launch_bounds__(64) decode_f32_kernel(DecodeArgs a) {
    const CacheView &c = a.c;
    const int bh = blockIdx.x;
    const int b = bh / a.n_q;
    const int h = bh - b * a.n_q;
    const int g = h / a.group;
    const int bg = b * c.n_kv + g;
    const int lane = threadIdx.x;
    constexpr int PER = HD / 64;
    const float *qp = (const float *)a.q + (int64_t)b * a.ld_q + (int64_t)h * HD;
    float q[PER], o[PER];
    for (int i = 0; i < PER; ++i) {
        q[i] = qp[lane + 64 * i];
        o[i] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int t = a.t[b];
    auto visit = [&](const float *k, const float *v, int vstride) {
        float s = 0.f;
        for (int i = 0; i < PER; ++i) s += q[i] * k[lane + 64 * i];
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        s *= a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
        for (int i = 0; i < PER; ++i) o[i] = o[i] * alpha + p * v[(int64_t)(lane + 64 * i) * vstride];
        m = m_new;
    };
    const int w = c.window;
    const float *rk = (const float *)c.ring_k + (int64_t)bg * w * HD;
    const float *rv = (const float *)c.ring_v + (int64_t)bg * HD * w;
    for (int slot = 0; slot < w; ++slot)
        if (slot <= t) visit(rk + slot * HD, rv + slot, w);
    const int len = c.lengths[bg];
    const int P = c.page_size;
    const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
    for (int j = 0; j < len; ++j) {
        const int page = pt[j >> c.page_shift];
        const int slot = j & (P - 1);
        if (c.pos_pages[(int64_t)page * P + slot] > t - w) break;  // positions increase
        visit((const float *)c.k_pages + ((int64_t)page * P + slot) * HD,
              (const float *)c.v_pages + (int64_t)page * HD * P + slot, P);
    }
    float *op = a.out + ((int64_t)b * a.n_q + h) * HD;
    for (int i = 0; i < PER; ++i) op[lane + 64 * i] = l > 0.f ? o[i] / l : 0.f;
    if (lane == 0 && a.lse) a.lse[(int64_t)b * a.n_q + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

size_t decode_ws_bytes(const spkv_cache *c, int n_q, int grid, int *max_items_out) {
    if (c->dtype != SPKV_BF16) {
        if (max_items_out) *max_items_out = 0;
        return 0;
    }
    const int BG = c->batch * c->n_kv;
    const int G = n_q / c->n_kv;
    // items <= lengths / C + 2 * BG with C * (2 * grid) >= sum of lengths
    const int max_items = 2 * grid + 2 * BG + 8;
    if (max_items_out) *max_items_out = max_items;
    const size_t cnt_bytes = ((size_t)BG * 4 + 255) & ~(size_t)255;
    return cnt_bytes + (size_t)max_items * G * (c->head_dim + 2) * sizeof(float);
}

int decode_blocks_per_cu() {
    int n128 = 0, n64 = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n128, decode_bf16_kernel<128>, NT, 0) != hipSuccess)
        n128 = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n64, decode_bf16_kernel<64>, NT, 0) != hipSuccess)
        n64 = 1;
    return max(1, min(n128, n64));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const CacheView &c = a.c;
    if (c.dtype == SPKV_BF16) {
        if (c.head_dim == 128)
            hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3(a.grid), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3(a.grid), dim3(NT), 0, s, a);
    } else {
        const dim3 grid(c.batch * a.n_q);
        if (c.head_dim == 128)
            hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace spkv
