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
// Work decomposition (built on the device from the cache lengths):
//   every (b, g) owns a list of 32-key steps -- w/32 ring steps, then
//   ceil(len[b][g] / 32) steps over its cached entries.  The lists of all
//   (b, g) are laid end to end and every wave of the (resident, persistent)
//   grid takes an equal contiguous share of that flat list: the load is
//   balanced whatever the per-head lengths (they differ by 30x in the skewed
//   workloads), and a wave streams its share with two steps in flight, never
//   draining its pipeline between work items.  Where its share crosses from
//   one (b, g) to the next, a wave writes a partial (max, sum, unnormalised
//   output) per query head.  A second, small kernel merges the partials of
//   every (b, g) in wave order -- deterministic -- and writes out and lse (the
//   kernel boundary makes the partials visible, with no cache flush).
//   Page ids and the number of visible entries of each step are staged in
//   LDS per wave before its steps run, so the streaming loop issues no vector
//   loads other than the key/value loads themselves.
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
constexpr int ROUND = 256;             // steps staged per wave at a time
constexpr int MAX_SLOTS_PER_BG = 256;  // partials merged per pass of the combine
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// floats per partial: G x HD outputs, then G maxima and G sums (padded so
// every record starts 16-byte aligned)
__host__ __device__ inline int rec_floats(int G, int HD) { return G * HD + 32; }

// workspace: one arrival counter per (b, g) (ints, padded; zero between
// calls), then the partials
__host__ __device__ inline size_t ws_header_bytes(int BG) { return ((size_t)(BG + 1) * 4 + 255) & ~(size_t)255; }

// Inclusive block scan of val(i), i < n, into out[1..n] (out[0] = 0); returns the total.
template <typename Fn>
__device__ int block_scan(int n, Fn val, int *out, int *lds_red) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int carry = 0;
    for (int base = 0; base < n; base += NT) {
        const int i = base + threadIdx.x;
        int x = i < n ? val(i) : 0;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        __syncthreads();
        if (lane == 63) lds_red[wave] = x;
        __syncthreads();
        int before = carry, tot = 0;
        for (int w = 0; w < NW; ++w) {
            const int v = lds_red[w];
            before += (w < wave) ? v : 0;
            tot += v;
        }
        if (i < n) out[i + 1] = before + x;
        carry += tot;
    }
    if (threadIdx.x == 0) out[0] = 0;
    __syncthreads();
    return carry;
}

// largest i in [0, n) with first[i] <= s (first[] non-decreasing, first[0] = 0)
__device__ inline int find_owner(const int *first, int n, int s) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= s) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// One wave's online-softmax state for the query heads of one (b, g).
template <int HD>
struct WaveState {
    f32x4 o[HD / 16];  // O^T tiles: lane holds rows 16*nt + 4*(lane/16) + r, head lane % 16
    float m;           // running max (log2 domain), identical across the 4 lane groups
    float l;           // this lane's partial sum
};

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    // raw buffer descriptor (gfx9 family dword 3); reads beyond `bytes` return 0
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Loads of one 32-key step into registers, as buffer loads with one 32-bit
// lane offset per operand (constant parts go to the instruction offset or a
// scalar offset), so that two steps in flight fit the register budget.
//   K operand (two 16-key tiles t): lane (i = lane % 16, q = lane / 16)
//     reads key 8*(i/4) + 4t + i%4, elements 32*cc + 8*q .. +8 for MFMA
//     step cc -- a 64-byte run of each key row per instruction
//   V^T operand (hd/16 tiles nt): lane reads V^T row 16*nt + i, keys
//     8*q .. 8*q+7 of the step (16 bytes)
template <int HD>
struct StepLanes {
    int k_off[2];  // byte offsets in the key block
    int v_off;     // byte offset in the V^T block (row i, key 8q)
};

template <int HD>
__device__ inline StepLanes<HD> step_lanes(int vstride) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int q4 = lane >> 4;
    StepLanes<HD> o;
#pragma unroll
    for (int t = 0; t < 2; ++t) o.k_off[t] = ((8 * (i >> 2) + 4 * t + (i & 3)) * HD + 8 * q4) * 2;
    o.v_off = (i * vstride + 8 * q4) * 2;
    return o;
}

template <int HD>
__device__ inline void load_step(const __bf16 *kblk, const __bf16 *vblk, int vstride, const StepLanes<HD> &ln,
                                 bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kblk, KSTEP * HD * 2);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vblk, (uint32_t)(HD * vstride * 2));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc)
            kr[t][cc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ln.k_off[t] + 64 * cc, 0, 0));
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt)
        vr[nt] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, ln.v_off, nt * 16 * vstride * 2, 0));
}

// valid: bit e set when key 8*(lane/16)+e of the step is visible (used only
// when MASKED; the unmasked form is taken for steps that are entirely visible,
// a wave-uniform decision).
template <int HD, bool MASKED>
__device__ inline void compute_step(WaveState<HD> &st, const bf16x8 *qlds,
                                    const bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16],
                                    uint32_t valid, float sl2) {
    // qlds: this lane's query operand pieces (MFMA step cc at qlds[64 * cc]),
    // re-read from LDS each step to keep registers for loads in flight
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[t][cc], qlds[64 * cc], acc, 0, 0, 0);
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
    // Lazily updated reference max: the exponentials below are taken
    // relative to st.m, which only has to bound the scores from above up to
    // a factor 2^8 (P <= 256 is exact enough in the bf16 pair and in f32).
    // Only when some lane sees a score beyond st.m + 8 is the exact max of
    // the head (over the 4 lane groups) formed and the sums rescaled -- after
    // the first step of a head that is rare, and the common step needs no
    // cross-lane traffic.  The result does not depend on the reference.
    if (__ballot(mloc > st.m + 8.f) != 0) {
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(st.m, mloc);
        if (m_new != st.m) {
            const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // st.m = -inf -> 0
#pragma unroll
            for (int nt = 0; nt < HD / 16; ++nt) st.o[nt] *= alpha;
            st.l *= alpha;
            st.m = m_new;
        }
    }
    // st.m == -inf only if nothing was visible so far (then every x is -inf)
    const float base = (st.m == -INFINITY) ? 0.f : st.m;
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
    if (MASKED && valid != 0xffu) {
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


// device-scope (L2-bypassing) accesses used to hand partials between
// workgroups: stores complete at the device-coherent level before the
// counter is bumped (s_waitcnt), and the merging workgroup reads them back
// past its own L2, so no cache-wide flush or invalidate is needed
__device__ inline void store_dev(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float load_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


template <int HD>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) decode_bf16_kernel(DecodeArgs a) {
    __shared__ int lds_F[MAX_BG + 1];     // first flat step of each (b, g)
    __shared__ int lds_len[MAX_BG];
    __shared__ int lds_t[MAX_BG];
    __shared__ int lds_red[NW];
    __shared__ int lds_flag;
    __shared__ int lds_sbg[NW][ROUND];    // per wave: (b, g) of each staged step
    __shared__ int lds_spg[NW][ROUND];    //           page id (-1: ring step)
    __shared__ int lds_snv[NW][ROUND];    //           visible keys (a prefix of the step)
    __shared__ bf16x8 lds_q[NW][HD / 32][64];  // per wave: query operand of each lane
    __shared__ float lds_wm[NW][16], lds_wl[NW][16];
    __shared__ float lds_o[NW][16][HD];   // wave states at a (b, g) boundary; merge scratch
    __shared__ float lds_sc[16];

    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int G = a.group;
    const int w = c.window;
    const int nws = w / KSTEP;  // ring steps per (b, g)
    const int P = c.page_size;

    // ---- flat step list; every workgroup derives it identically ------------
    for (int i = threadIdx.x; i < BG; i += NT) lds_len[i] = c.lengths[i];
    for (int i = threadIdx.x; i < c.batch; i += NT) lds_t[i] = a.t[i];
    __syncthreads();
    const int total = uniform(block_scan(BG, [&](int i) { return nws + (lds_len[i] + KSTEP - 1) / KSTEP; },
                                         lds_F, lds_red));
    const int spg = (total + gridDim.x - 1) / gridDim.x;  // steps per workgroup
    // One partial per (workgroup, (b, g)) that meet, at slot workgroup + bg:
    // ranges are contiguous and in order, so if workgroup x meets (b, g) then
    // x+1 cannot meet an earlier (b, g) -- the slots are distinct, and those
    // of one (b, g) are consecutive, from F[bg]/spg + bg to (F[bg+1]-1)/spg + bg.
    const int W0 = blockIdx.x * spg;
    const int W1 = min(total, W0 + spg);
    if (W0 >= W1) return;  // (uniform over the workgroup)

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int head = lane & 15;
    const int q4 = lane >> 4;
    const float sl2 = a.scale * LOG2E;
    const int rec = rec_floats(G, HD);
    int32_t *cnt = (int32_t *)a.ws;
    float *part = (float *)(a.ws + ws_header_bytes(BG));
    const StepLanes<HD> lanes_ring = step_lanes<HD>(w);
    const StepLanes<HD> lanes_page = step_lanes<HD>(P);
    // this wave's steps: W0 + wave + NW * k (the 4 waves of the workgroup
    // walk neighbouring steps, i.e. neighbouring memory)
    const int nk = max(0, (W1 - W0 - wave + NW - 1) / NW);
    const int bg_first = uniform(find_owner(lds_F, BG, W0));
    const int bg_last = uniform(find_owner(lds_F, BG, W1 - 1));

    WaveState<HD> st;
    auto reset = [&](int bg) {
        const int b = bg / c.n_kv;
        const int g = bg - b * c.n_kv;
        const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.ld_q + (int64_t)(g * G + head) * HD + 8 * q4;
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc)
            lds_q[wave][cc][lane] = head < G ? *(const bf16x8 *)(qp + 32 * cc) : bf16x8{};
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) st.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
    };

    // ---- per-wave staging of (b, g), page and visible count of its steps ----
    int r0 = 0, r1 = 0;
    auto stage = [&](int from) {
        r0 = from;
        r1 = min(nk, from + ROUND);
        for (int k = r0 + lane; k < r1; k += 64) {
            const int s = W0 + wave + NW * k;
            const int bg = find_owner(lds_F, BG, s);
            const int ls = s - lds_F[bg];
            const int len = lds_len[bg];
            const int t = lds_t[bg / c.n_kv];
            const int limit = t - w;
            int page = -1, nv;
            if (ls < nws) {
                // ring slot s holds position t - ((t - s) mod w): visible iff s <= t
                nv = min(KSTEP, max(0, t - ls * KSTEP + 1));
            } else {
                const int j0 = (ls - nws) * KSTEP;
                page = c.page_table[(int64_t)bg * c.max_pages + (j0 >> c.page_shift)];
                if (limit >= 0 && j0 + KSTEP <= len - w) {
                    nv = KSTEP;  // older than the window: every entry visible
                } else {
                    // visible = index < len and position <= t - w: a prefix,
                    // since positions increase along the list; the 32
                    // positions of the step are one aligned 128-byte run
                    const i32x4 *pp = (const i32x4 *)(c.pos_pages + (int64_t)page * P + (j0 & (P - 1)));
                    const int lim_n = min(KSTEP, len - j0);
                    i32x4 pv[KSTEP / 4];
#pragma unroll
                    for (int u = 0; u < KSTEP / 4; ++u) pv[u] = pp[u];
                    nv = 0;
#pragma unroll
                    for (int u = 0; u < KSTEP; ++u) nv += (u < lim_n && pv[u >> 2][u & 3] <= limit) ? 1 : 0;
                }
            }
            lds_sbg[wave][k - r0] = bg;
            lds_spg[wave][k - r0] = page;
            lds_snv[wave][k - r0] = nv;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    };

    bf16x8 kA[2][HD / 32], kB[2][HD / 32];
    bf16x8 vA[HD / 16], vB[HD / 16];
    auto issue = [&](int k, bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
        const int bg = uniform(lds_sbg[wave][k - r0]);
        const int page = uniform(lds_spg[wave][k - r0]);
        const int ls = W0 + wave + NW * k - uniform(lds_F[bg]);
        if (page < 0) {
            const __bf16 *kb = (const __bf16 *)c.ring_k + ((int64_t)bg * w + ls * KSTEP) * HD;
            const __bf16 *vb = (const __bf16 *)c.ring_v + (int64_t)bg * HD * w + ls * KSTEP;
            load_step<HD>(kb, vb, w, lanes_ring, kr, vr);
        } else {
            const int slot0 = ((ls - nws) * KSTEP) & (P - 1);
            const __bf16 *kb = (const __bf16 *)c.k_pages + ((int64_t)page * P + slot0) * HD;
            const __bf16 *vb = (const __bf16 *)c.v_pages + (int64_t)page * HD * P + slot0;
            load_step<HD>(kb, vb, P, lanes_page, kr, vr);
        }
    };
    auto compute = [&](int k, bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
        // the visible keys of a step are its first nv keys; this lane's keys
        // are 8*q4 .. 8*q4+7
        const int nv = uniform(lds_snv[wave][k - r0]);
        const uint32_t valid = (uint32_t)((1u << min(8, max(0, nv - 8 * q4))) - 1u);
        compute_step<HD, true>(st, &lds_q[wave][0][lane], kr, vr, valid, sl2);
    };

    // ---- the (b, g) segments of this workgroup's range -----------------------
    reset(bg_first);
    int k = 0;  // next step of this wave to compute (its loads are in flight)
    if (nk > 0) {
        stage(0);
        issue(0, kA, vA);
    }
    for (int bg = bg_first; bg <= bg_last; ++bg) {
        const int seg_end = min(W1, lds_F[bg + 1]);
        while (k < nk && W0 + wave + NW * k < seg_end) {
            const bool more = k + 1 < r1;  // prefetch stays inside the staged round
            if ((k & 1) == 0) {
                if (more) issue(k + 1, kB, vB);
                compute(k, kA, vA);
            } else {
                if (more) issue(k + 1, kA, vA);
                compute(k, kB, vB);
            }
            ++k;
            if (k < nk && k == r1) {
                stage(k);
                if ((k & 1) == 0) issue(k, kA, vA); else issue(k, kB, vB);
            }
        }
        // ---- end of this (b, g) in the workgroup: merge the 4 wave states ----
        {
            float lsum = st.l;
            lsum += __shfl_xor(lsum, 16);
            lsum += __shfl_xor(lsum, 32);
            if (q4 == 0) {
                lds_wm[wave][head] = st.m;
                lds_wl[wave][head] = lsum;
            }
#pragma unroll
            for (int nt = 0; nt < HD / 16; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) lds_o[wave][head][16 * nt + 4 * q4 + r] = st.o[nt][r];
        }
        __syncthreads();
        const int slot = blockIdx.x + bg;
        const int part0 = lds_F[bg] / spg + bg;                  // first slot of (b, g)
        const int n_parts = (lds_F[bg + 1] - 1) / spg + bg - part0 + 1;
        float *my = part + (size_t)slot * rec;
        for (int idx = threadIdx.x; idx < G * HD; idx += NT) {
            const int h = idx / HD;
            const int d = idx - h * HD;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < NW; ++v) M = fmaxf(M, lds_wm[v][h]);
            const float bse = (M == -INFINITY) ? 0.f : M;
            float O = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) O += exp2f(lds_wm[v][h] - bse) * lds_o[v][h][d];
            store_dev(my + h * HD + d, O);
            if (d == 0) {
                float L = 0.f;
#pragma unroll
                for (int v = 0; v < NW; ++v) L += exp2f(lds_wm[v][h] - bse) * lds_wl[v][h];
                store_dev(my + G * HD + h, M);
                store_dev(my + G * HD + G + h, L);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
        __syncthreads();
        if (threadIdx.x == 0)
            lds_flag = __hip_atomic_fetch_add(&cnt[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_parts - 1;
        __syncthreads();
        if (lds_flag) {
            // the last workgroup of (b, g): merge its partials in slot order.
            // Partials are taken MB at a time; every load of a batch (maxima,
            // sums and outputs) is issued before any is used, so a batch costs
            // one trip to memory.
            constexpr int MB = 8;
            constexpr int PER = (16 * HD + NT - 1) / NT;  // outputs per thread
            const float *pb = part + (size_t)part0 * rec;
            float *cm = &lds_o[0][0][0];  // [MB][16] maxima -> weights
            float *cl = cm + MB * 16;     // [MB][16] sums
            float Oacc[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) Oacc[j] = 0.f;
            float Mrun = -INFINITY, Lrun = 0.f;  // (threads < G: head threadIdx.x)
            for (int c0 = 0; c0 < n_parts; c0 += MB) {
                const int m_n = min(MB, n_parts - c0);
                float ov[MB][PER];
#pragma unroll
                for (int kk = 0; kk < MB; ++kk)
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        const int idx = threadIdx.x + j * NT;
                        ov[kk][j] = (kk < m_n && idx < G * HD) ? load_dev(pb + (size_t)(c0 + kk) * rec + idx) : 0.f;
                    }
                if (threadIdx.x < m_n * G) {
                    const int kk = threadIdx.x / G;
                    const int h = threadIdx.x - kk * G;
                    cm[kk * 16 + h] = load_dev(pb + (size_t)(c0 + kk) * rec + G * HD + h);
                    cl[kk * 16 + h] = load_dev(pb + (size_t)(c0 + kk) * rec + G * HD + G + h);
                }
                __syncthreads();
                if (threadIdx.x < G) {
                    const int h = threadIdx.x;
                    float M = Mrun;
                    for (int kk = 0; kk < m_n; ++kk) M = fmaxf(M, cm[kk * 16 + h]);
                    const float bse = (M == -INFINITY) ? 0.f : M;
                    const float so = exp2f(Mrun - bse);
                    float L = Lrun * so;
                    for (int kk = 0; kk < m_n; ++kk) {
                        const float f = exp2f(cm[kk * 16 + h] - bse);
                        cm[kk * 16 + h] = f;
                        L += f * cl[kk * 16 + h];
                    }
                    lds_sc[h] = so;
                    Mrun = M;
                    Lrun = L;
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int idx = threadIdx.x + j * NT;
                    if (idx < G * HD) {
                        const int h = idx / HD;
                        float O = Oacc[j] * lds_sc[h];
#pragma unroll
                        for (int kk = 0; kk < MB; ++kk)
                            if (kk < m_n) O += cm[kk * 16 + h] * ov[kk][j];
                        Oacc[j] = O;
                    }
                }
                __syncthreads();
            }
            if (threadIdx.x < G) {
                lds_wm[0][threadIdx.x] = Mrun;
                lds_wl[0][threadIdx.x] = Lrun;
            }
            __syncthreads();
            const int b = bg / c.n_kv;
            const int g = bg - b * c.n_kv;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int idx = threadIdx.x + j * NT;
                if (idx < G * HD) {
                    const int h = idx / HD;
                    const int d = idx - h * HD;
                    const float L = lds_wl[0][h];
                    const int64_t oidx = (int64_t)b * a.n_q + g * G + h;
                    a.out[oidx * HD + d] = L > 0.f ? Oacc[j] / L : 0.f;
                    if (d == 0 && a.lse) a.lse[oidx] = L > 0.f ? (lds_wm[0][h] + log2f(L)) * LN2 : -INFINITY;
                }
            }
            if (threadIdx.x == 0) __hip_atomic_store(&cnt[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (bg < bg_last) reset(bg + 1);
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
    // a workgroup's contiguous range meets each (b, g) in at most one
    // segment, and consecutive (b, g) share at most one workgroup
    const int max_slots = grid + BG;
    if (max_items_out) *max_items_out = max_slots;
    return ws_header_bytes(BG) + (size_t)max_slots * rec_floats(G, c->head_dim) * sizeof(float);
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
