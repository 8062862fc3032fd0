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
//   workloads).  The grid is persistent (compute units x resident
//   workgroups); workgroup x takes a contiguous share of the list and its 4
//   waves interleave over it, two steps in flight each.  The shares are
//   equal once every (b, g) is charged a few extra steps for the hand-over
//   or output write that a workgroup starting it inside its share pays.
//   A (b, g) wholly inside one share is finished by that workgroup (the 4
//   wave states combined in LDS, output written).  A (b, g) spread over
//   several shares gets one partial (max, sum, unnormalised output per query
//   head) from each; a workgroup publishes its (at most two) partials after
//   its last step, with device-scope stores, then bumps the (b, g) arrival
//   counter; the workgroup that arrives last merges the partials in share
//   order -- deterministic -- and writes out and lse.
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
#include "spkv_device.h"
#include "spkv_gate_dev.h"

namespace spkv {
namespace {

constexpr int NT = 256;
constexpr int NW = 4;
constexpr int KSTEP = 32;
constexpr int MAX_BG = 2048;
constexpr int ROUND = 256;             // steps staged per wave at a time
// extra (virtual) steps charged to every (b, g) when the shares are cut:
// starting a (b, g) inside a share costs its workgroup a hand-over or an
// output write, about 12 steps of streaming time (12 measured best of 4, 8,
// 12, 16 on the 32K-, 131K-context and ragged batch-32 decode workloads)
constexpr int BG_COST = 12;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// floats per partial: G x HD outputs, then G maxima and G sums (padded so
// every record starts 16-byte aligned)
__host__ __device__ inline int rec_floats(int G, int HD) { return G * HD + 32; }

// workspace head: one arrival counter per (b, g), each in its own 256-byte
// line (the end-of-launch arrivals of all workgroups would otherwise queue on
// a few lines), then the fused step's two counters (gate units stored,
// workgroups that have read the lengths), a line each, with the running total
// each has to reach 16 words after it.  Every call leaves the per-(b, g)
// counters at zero; the fused step's two only grow (see fused_finisher), so
// one workspace may serve both entry points.
constexpr int CNT_STRIDE = 64;  // ints
__host__ __device__ inline size_t ws_header_bytes(int BG) { return ((size_t)BG * CNT_STRIDE + 2 * 64) * 4; }
// then, for the fused step only, the gate's partial first-layer sums
// ([items][16 rows][16 units] floats, rounded to 256 bytes); then the split-K
// partials
constexpr int FUSED_ROWS = 16;  // batch rows the fused gate takes
__host__ __device__ inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t fused_bytes(int d_model, int d_hidden) {
    return d_hidden <= 0 ? 0 : round256((size_t)gate_tile_items(d_model, d_hidden) * 256 * 4);
}

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
// lane offset (the constant parts go to the scalar offset).  A step is one
// 32-slot block of the cache (see the storage order in spkv_internal.h):
//   K operand (two 16-key tiles t, MFMA step cc): lane (i = lane % 16,
//     q = lane / 16) reads row 16t + i of the block's dims 32cc .. 32cc+31,
//     elements 8q .. 8q+7 -- the 64 lanes read one contiguous 1 KB run
//   V^T operand (hd/16 tiles nt): lane reads dimension 16nt + i, slots
//     8q .. 8q+7 -- again one 1 KB run
// Every byte of a step is read by exactly one load, with the non-temporal
// hint: the blocks are streamed once per launch.
constexpr int CPOL_NT = 2;

__device__ inline int step_lane_offset() {
    const int lane = threadIdx.x & 63;
    return (lane & 15) * 64 + (lane >> 4) * 16;
}

template <int HD, int CPOL = 0>
__device__ inline void load_step(const __bf16 *kblk, const __bf16 *vblk, int lo,
                                 bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kblk, KSTEP * HD * 2);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vblk, KSTEP * HD * 2);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc)
            kr[t][cc] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, lo, 1024 * t + 2048 * cc, CPOL | CPOL_NT));
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt)
        vr[nt] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, lo, 1024 * nt, CPOL | CPOL_NT));
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



// Fused step: append the new row of every (b, g) whose keep bit is set
// (SP-KV section 2.1, deployment paragraph: only kept pairs enter the
// persistent cache), as spkv_compact_append does for one row per sequence.
// 16 threads per (b, g); the new lengths go to new_len (LDS).  u (LDS) holds
// the utilities, stored with the entries when the cache keeps them.
template <int HD>
__device__ void append_new_rows(const DecodeArgs &a, const uint8_t *keep, const float *u, int *new_len) {
    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int P = c.page_size;
    constexpr int TPP = 16;
    const int sub = threadIdx.x % TPP;
    for (int p0 = 0; p0 < BG; p0 += NT / TPP) {
        const int bg = p0 + (int)threadIdx.x / TPP;
        if (bg < BG) {
            const int old = c.lengths[bg];
            const int tb = a.t[bg / c.n_kv];
            int newlen = old;
            if (tb < 0) {
                // a negative position is refused, as spkv_compact_append does
                if (sub == 0) atomicOr(c.status, SPKV_STATUS_BAD_ROWS);
            } else if (keep[bg]) {
                int32_t *ptab = c.page_table + (int64_t)bg * c.max_pages;
                int page = -1;
                if ((old & (P - 1)) == 0) {
                    // the entry opens a new page
                    if (sub == 0) {
                        const int first = old >> c.page_shift;
                        if (first >= c.max_pages) {
                            atomicOr(c.status, SPKV_STATUS_TABLE_FULL);
                        } else {
                            const int base = atomicAdd(c.pool_next, 1);
                            if (base >= c.n_pages) {
                                atomicOr(c.status, SPKV_STATUS_POOL_FULL);
                            } else {
                                ptab[first] = base;
                                page = base;
                            }
                        }
                    }
                    page = __shfl(page, (int)(threadIdx.x & 63) & ~(TPP - 1));
                } else {
                    page = ptab[old >> c.page_shift];
                }
                if (page >= 0) {
                    const int b = bg / c.n_kv;
                    const int g = bg - b * c.n_kv;
                    const __bf16 *kn = (const __bf16 *)a.k_new + (int64_t)b * a.ld_new + (int64_t)g * HD;
                    const __bf16 *vn = (const __bf16 *)a.v_new + (int64_t)b * a.ld_new + (int64_t)g * HD;
                    const int j = old & (P - 1);
                    if (sub < HD / 8)
                        *(bf16x8 *)((__bf16 *)c.k_pages + kv_k_index((int64_t)page * P + j, 8 * sub, HD)) =
                            *(const bf16x8 *)(kn + 8 * sub);
                    for (int e = sub; e < HD; e += TPP) ((__bf16 *)c.v_pages)[kv_v_index((int64_t)page * P + j, e, HD)] = vn[e];
                    if (sub == 0) {
                        c.pos_pages[(int64_t)page * P + j] = tb;
                        if (c.u_pages) c.u_pages[(int64_t)page * P + j] = u[bg];
                    }
                    newlen = old + 1;
                }
            }
            if (sub == 0) new_len[bg] = newlen;
        }
    }
}

// Fused step, the last workgroup of the launch (it takes no attention work):
// once every gate unit's shares are stored, finish the gate (utilities, keep
// bits), append the kept rows, and once every other workgroup has read the
// lengths for its plan, store the new lengths.  The two arrival counters only
// ever grow; the workspace keeps, beside each, the total its arrivals have
// reached once every call so far has completed, and each call raises that
// total by its own count before it waits.  The waits are bounded: if one
// runs out, the step's append or lengths are left undone and a status bit
// says so -- and the next call on the workspace still waits for its own
// arrivals on top of this call's late ones, so nothing has to be reset.
template <int HD>
__device__ void fused_finisher(const DecodeArgs &a, const float *gshare, int *gate_cnt, int *plan_cnt,
                               float *lds_act, uint8_t *lds_keep, int *lds_new_len, int *lds_flag) {
    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int items = gate_tile_items(a.gate.d_model, a.gate.d_hidden);
    int *gate_total = gate_cnt + 16, *plan_total = plan_cnt + 16;
    int gate_target = 0, plan_target = 0;
    if (threadIdx.x == 0) {
        gate_target = (int)((unsigned)load_dev(gate_total) + (unsigned)items);
        plan_target = (int)((unsigned)load_dev(plan_total) + (unsigned)(gridDim.x - 1));
        __hip_atomic_store(gate_total, gate_target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(plan_total, plan_target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_flag[0] = wait_reach_dev(gate_cnt, gate_target, a.wait_limit);
    }
    __syncthreads();
    if (!lds_flag[0]) {
        if (threadIdx.x == 0) atomicOr(c.status, SPKV_STATUS_STEP_TIMEOUT);
        return;
    }
    // the utilities go after the staged activations (at most FUSED_ROWS
    // rows of d_hidden <= 256 floats)
    float *lds_u = lds_act + FUSED_ROWS * 256;
    gate_tile_finish(a.gate, gshare, lds_act, lds_keep, lds_u);
    __syncthreads();
    append_new_rows<HD>(a, lds_keep, lds_u, lds_new_len);
    __syncthreads();
    if (threadIdx.x == 0) lds_flag[1] = wait_reach_dev(plan_cnt, plan_target, a.wait_limit);
    __syncthreads();
    if (!lds_flag[1]) {
        if (threadIdx.x == 0) atomicOr(c.status, SPKV_STATUS_STEP_TIMEOUT);
        return;
    }
    for (int i = threadIdx.x; i < BG; i += NT) c.lengths[i] = lds_new_len[i];
}

// MODE 0: attention only (spkv_decode_attn); MODE_STEP: the whole decode
// step (gate, append, ring, attention); MODE_RING: the new rows' ring write
// and attention (spkv_decode_step without a gate)
constexpr int MODE_STEP = 1;
constexpr int MODE_RING = 2;

template <int HD, int MODE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) decode_bf16_kernel(DecodeArgs a) {
    constexpr bool FUSED = MODE == MODE_STEP;  // gate + append + finisher
    constexpr bool RING = MODE != 0;           // the new rows go into the ring here
    __shared__ int lds_F[MAX_BG + 1];     // first flat step of each (b, g)
    __shared__ int lds_len[MAX_BG];
    __shared__ int lds_t[MAX_BG];
    __shared__ int lds_red[NW];
    __shared__ int lds_flag[2];
    __shared__ uint8_t lds_keep[FUSED_ROWS * 16];  // fused step: keep bits of the new rows
    __shared__ int lds_sbg[NW][ROUND];    // per wave: (b, g) of each staged step
    __shared__ int lds_spg[NW][ROUND];    //           page id (-1: ring step)
    __shared__ int lds_snv[NW][ROUND];    //           visible keys (a prefix of the step)
    __shared__ bf16x8 lds_q[NW][HD / 32][64];  // per wave: query operand of each lane
    // wave states at (b, g) boundaries, two slots (slot 0 doubles as merge scratch)
    __shared__ float lds_wm[2][NW][16], lds_wl[2][NW][16];
    __shared__ __attribute__((aligned(16))) float lds_o[2][NW][16][HD];

    const CacheView &c = a.c;
    const int BG = c.batch * c.n_kv;
    const int G = a.group;
    const int w = c.window;
    const int nws = w / KSTEP;  // ring steps per (b, g)
    const int P = c.page_size;
    int32_t *cnt = a.cnt;
    const int g_items = FUSED ? gate_tile_items(a.gate.d_model, a.gate.d_hidden) : 0;
    int32_t *gate_cnt = cnt + (size_t)BG * CNT_STRIDE;  // fused: gate units stored
    int32_t *plan_cnt = gate_cnt + 64;                  // fused: workgroups that read the lengths
    float *gshare = a.gshare;
    float *part = a.part;
    // attention workgroups (the fused step keeps the last one for its finisher)
    const int n_att = FUSED ? (int)gridDim.x - 1 : (int)gridDim.x;

    if constexpr (FUSED) {
        // The new rows' gate: workgroup x stores the partial sums of gate
        // items x, x + n_att, ... (16-unit tiles of the first layer over a
        // part of d_model) and counts them, without waiting; the finisher
        // completes the gate and appends the kept rows.  It stores the new lengths only after
        // every workgroup has read the old ones for its plan (the appended
        // entries, at position t, are outside this step's global set).
        if ((int)blockIdx.x == n_att) {
            // lds_o holds the staged activations and the utilities
            static_assert(2 * NW * 16 * HD >= FUSED_ROWS * 256 + FUSED_ROWS * 16, "finisher LDS");
            fused_finisher<HD>(a, gshare, gate_cnt, plan_cnt, &lds_o[0][0][0][0], lds_keep, lds_len, lds_flag);
            return;
        }
        if ((int)blockIdx.x < g_items) {
            float *red = &lds_o[0][0][0][0];
            int units = 0;
            for (int j = blockIdx.x; j < g_items; j += n_att) {
                if (units++) __syncthreads();  // red is reused
                gate_tile_share(a.gate, j, gshare, red);
            }
            __builtin_amdgcn_s_waitcnt(0);  // this thread's shares are stored
            __syncthreads();
            if (threadIdx.x == 0) arrive_nr_dev(gate_cnt, units);
        }
    }

    // ---- flat step list; every workgroup derives it identically ------------
    for (int i = threadIdx.x; i < BG; i += NT) lds_len[i] = c.lengths[i];
    for (int i = threadIdx.x; i < c.batch; i += NT) lds_t[i] = a.t[i];
    __syncthreads();
    if (FUSED && threadIdx.x == 0) arrive_nr_dev(plan_cnt);  // the lengths are read
    const int total = uniform(block_scan(BG, [&](int i) { return nws + (lds_len[i] + KSTEP - 1) / KSTEP; },
                                         lds_F, lds_red));
    // Shares are cut from a list in which every (b, g) is charged BGC extra
    // steps ahead of its own (a workgroup that starts a (b, g) inside its
    // share also hands a partial over or writes an output there, which
    // costs it about that much streaming time): the virtual position of
    // step s of (b, g) is s + BGC * (bg + 1).  Workgroup x takes the virtual
    // range [w0(x), w0(x+1)); the first n_cut workgroups (in a fused step
    // they ran a gate unit first) take cut virtual steps fewer.
    constexpr int BGC = BG_COST;
    const int total_v = total + BGC * BG;
    const int spg0 = (total_v + n_att - 1) / n_att;
    const int n_cut = FUSED ? min(g_items, n_att) : 0;
    const int cut = FUSED ? min(a.share_cut, spg0 / 2) : 0;
    const int spg = (total_v + n_cut * cut + n_att - 1) / n_att;  // >= 2 * cut
    const int cut_end = n_cut * (spg - cut);
    auto w0 = [&](int x) -> int { return min(total_v, x * spg - min(x, n_cut) * cut); };
    auto owner_v = [&](int v) -> int { return v < cut_end ? v / (spg - cut) : n_cut + (v - cut_end) / spg; };
    auto owner = [&](int s, int bg) -> int { return owner_v(s + BGC * (bg + 1)); };  // s a step of (b, g)
    // first real step at or after virtual position v
    auto real_of = [&](int v) -> int {
        int lo = 0, hi = BG - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds_F[mid] + BGC * mid <= v) lo = mid; else hi = mid - 1;
        }
        return lds_F[lo] + max(0, v - lds_F[lo] - BGC * (lo + 1));
    };
    // One partial per (workgroup, (b, g)) that meet, at slot workgroup + bg:
    // ranges are contiguous and in order, so if workgroup x meets (b, g) then
    // x+1 cannot meet an earlier (b, g) -- the slots are distinct, and those
    // of one (b, g) are consecutive, from owner(F[bg]) + bg to owner(F[bg+1]-1) + bg.
    const int W0 = uniform(real_of(w0(blockIdx.x)));
    const int W1 = uniform(real_of(w0(blockIdx.x + 1)));
    if (W0 >= W1) return;  // (uniform over the workgroup)

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int head = lane & 15;
    const int q4 = lane >> 4;
    const float sl2 = a.scale * LOG2E;
    const int rec = rec_floats(G, HD);
    const int step_lo = step_lane_offset();
    // this wave's steps: W0 + wave + NW * k (the 4 waves of the workgroup
    // walk neighbouring steps, i.e. neighbouring memory)
    const int nk = max(0, (W1 - W0 - wave + NW - 1) / NW);
    const int bg_first = uniform(find_owner(lds_F, BG, W0));
    const int bg_last = uniform(find_owner(lds_F, BG, W1 - 1));

    WaveState<HD> st;
    // The query operand of (b, g): every lane loads (lanes of heads >= G
    // read head 0's row and store zeros), so the HD/32 loads go out together
    // and are waited for once -- a load per condition would cost a memory
    // round trip each.
    auto q_load = [&](int bg, bf16x8 (&qv)[HD / 32]) {
        const int b = bg / c.n_kv;
        const int g = bg - b * c.n_kv;
        const int hq = head < G ? head : 0;
        const __bf16 *qp = (const __bf16 *)a.q + (int64_t)b * a.ld_q + (int64_t)(g * G + hq) * HD + 8 * q4;
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc) qv[cc] = *(const bf16x8 *)(qp + 32 * cc);
    };
    auto q_store = [&](const bf16x8 (&qv)[HD / 32]) {
#pragma unroll
        for (int cc = 0; cc < HD / 32; ++cc) lds_q[wave][cc][lane] = head < G ? qv[cc] : bf16x8{};
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt) st.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
    };
    auto reset = [&](int bg) {
        bf16x8 qv[HD / 32];
        q_load(bg, qv);
        q_store(qv);
    };

    // ---- per-wave staging of (b, g), page and visible count of its steps ----
    // Phase A (page ids) comes before the first loads of a round; phase B
    // (visible counts, which need the positions of the last entries of each
    // (b, g)) runs while those loads are in flight.
    int r0 = 0, r1 = 0;
    auto stage_pages = [&](int from) {
        r0 = from;
        r1 = min(nk, from + ROUND);
        for (int k = r0 + lane; k < r1; k += 64) {
            const int s = W0 + wave + NW * k;
            const int bg = find_owner(lds_F, BG, s);
            const int ls = s - lds_F[bg];
            int page = -1;
            if (ls >= nws) page = c.page_table[(int64_t)bg * c.max_pages + (((ls - nws) * KSTEP) >> c.page_shift)];
            lds_sbg[wave][k - r0] = bg;
            lds_spg[wave][k - r0] = page;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    };
    auto stage_counts = [&]() {
        for (int k = r0 + lane; k < r1; k += 64) {
            const int s = W0 + wave + NW * k;
            const int bg = lds_sbg[wave][k - r0];
            const int ls = s - lds_F[bg];
            const int len = lds_len[bg];
            const int t = lds_t[bg / c.n_kv];
            const int limit = t - w;
            int nv;
            if (ls < nws) {
                // ring slot s holds position t - ((t - s) mod w): visible iff s <= t
                nv = min(KSTEP, max(0, t - ls * KSTEP + 1));
            } else {
                const int j0 = (ls - nws) * KSTEP;
                if (limit >= 0 && j0 + KSTEP <= len - w) {
                    nv = KSTEP;  // older than the window: every entry visible
                } else {
                    // visible = index < len and position <= t - w: a prefix,
                    // since positions increase along the list; the 32
                    // positions of the step are one aligned 128-byte run
                    const int page = lds_spg[wave][k - r0];
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
            const __bf16 *vb = (const __bf16 *)c.ring_v + ((int64_t)bg * w + ls * KSTEP) * HD;
            if constexpr (RING) {
                const int tb = uniform(lds_t[bg / c.n_kv]);
                if (tb >= 0 && ls == (tb % w) / KSTEP) {
                    // the step holding the new token (this wave wrote it into
                    // the ring before its first loads): read past the L1 cache
                    load_step<HD, 1>(kb, vb, step_lo, kr, vr);
                    return;
                }
            }
            load_step<HD>(kb, vb, step_lo, kr, vr);
        } else {
            const int slot0 = ((ls - nws) * KSTEP) & (P - 1);
            const __bf16 *kb = (const __bf16 *)c.k_pages + ((int64_t)page * P + slot0) * HD;
            const __bf16 *vb = (const __bf16 *)c.v_pages + ((int64_t)page * P + slot0) * HD;
            load_step<HD>(kb, vb, step_lo, kr, vr);
        }
    };
    auto compute = [&](int k, bf16x8 (&kr)[2][HD / 32], bf16x8 (&vr)[HD / 16]) {
        // the visible keys of a step are its first nv keys; this lane's keys
        // are 8*q4 .. 8*q4+7
        const int nv = uniform(lds_snv[wave][k - r0]);
        const uint32_t valid = (uint32_t)((1u << min(8, max(0, nv - 8 * q4))) - 1u);
        compute_step<HD, true>(st, &lds_q[wave][0][lane], kr, vr, valid, sl2);
    };
    // this wave's state -> LDS state slot `sl` (the lane groups' sums added)
    auto save_state = [&](int sl) {
        float lsum = st.l;
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (q4 == 0) {
            lds_wm[sl][wave][head] = st.m;
            lds_wl[sl][wave][head] = lsum;
        }
#pragma unroll
        for (int nt = 0; nt < HD / 16; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) lds_o[sl][wave][head][16 * nt + 4 * q4 + r] = st.o[nt][r];
    };
    // combination of the NW wave states of slot sl for outputs (h, d..d+3):
    // M and O, L relative to 2^M
    auto combine4 = [&](int sl, int h, int d, float &M, f32x4 &O, float &L) {
        M = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, lds_wm[sl][v][h]);
        const float bse = (M == -INFINITY) ? 0.f : M;
        O = f32x4{0.f, 0.f, 0.f, 0.f};
        L = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float f = exp2f(lds_wm[sl][v][h] - bse);
            O += f * *(const f32x4 *)&lds_o[sl][v][h][d];
            L += f * lds_wl[sl][v][h];
        }
    };
    auto out_index = [&](int bg, int h) -> int64_t {
        const int b = bg / c.n_kv;
        return (int64_t)b * a.n_q + (bg - b * c.n_kv) * G + h;
    };
    auto parts_of = [&](int bg, int &part0, int &n_parts) {
        part0 = owner(lds_F[bg], bg) + bg;  // first slot of (b, g)
        n_parts = owner(lds_F[bg + 1] - 1, bg) + bg - part0 + 1;
    };
    // Partials are handed between workgroups with 16-byte device-scope
    // (sc1) buffer stores and loads: they bypass the non-coherent per-XCD L2
    // copies, so the only ordering needed is the producer's s_waitcnt before
    // its arrival atomic.
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(part, (uint32_t)((size_t)a.max_items * rec * sizeof(float)));
    constexpr int CPOL_SC1 = 16;
    // publish the combined state of slot sl as the partial of (b, g) at slot
    // blockIdx + bg; threads t0, t0 + stride, ... take one float4 each
    auto publish = [&](int sl, int bg, int t0, int stride) {
        const uint32_t base = (uint32_t)((size_t)(blockIdx.x + bg) * rec * sizeof(float));
        for (int f = t0; f < G * HD / 4; f += stride) {
            const int h = (4 * f) / HD;
            const int d = 4 * f - h * HD;
            float M, L;
            f32x4 O;
            combine4(sl, h, d, M, O, L);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, O), prs, base + 16 * f, 0, CPOL_SC1);
            if (d == 0) {
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, M), prs, base + 4 * (G * HD + h), 0, CPOL_SC1);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, L), prs, base + 4 * (G * HD + G + h), 0, CPOL_SC1);
            }
        }
    };
    // Merge of the partials of one (b, g) (this workgroup arrived last), in
    // slot order -- deterministic.  Per batch of MB slots, the maxima and
    // sums go to LDS and each thread loads the float4 outputs it owns, all
    // loads issued before any is used: a batch costs one trip to memory and
    // one barrier (a (b, g) spread over many shares, as the long heads of a
    // skewed cache are, takes ceil(parts / MB) batches).  Uses state slot 0
    // of LDS as scratch.
    auto merge = [&](int bg) {
        constexpr int MB = 16;
        constexpr int MAXC = (16 * HD / 4 + NT - 1) / NT;  // float4 chunks per thread
        const int GH = G * HD;
        const int n4 = GH / 4;
        int p0, np;
        parts_of(bg, p0, np);
        float *cm = &lds_o[0][0][0][0];  // [MB][16] maxima
        float *cl = cm + MB * 16;         // [MB][16] sums
        f32x4 Oa[MAXC];
        float Ma[MAXC], La[MAXC];
#pragma unroll
        for (int ch = 0; ch < MAXC; ++ch) {
            Oa[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
            Ma[ch] = -INFINITY;
            La[ch] = 0.f;
        }
        for (int c0 = 0; c0 < np; c0 += MB) {
            if (c0 > 0) __syncthreads();  // the previous batch's maxima are consumed
            f32x4 ov[MAXC][MB];
#pragma unroll
            for (int ch = 0; ch < MAXC; ++ch) {
                if (ch * NT >= n4) break;  // uniform
                const int f = ch * NT + threadIdx.x;
                const uint32_t off = (uint32_t)(((size_t)p0 * rec + 4 * f) * sizeof(float));
#pragma unroll
                for (int kk = 0; kk < MB; ++kk)
                    ov[ch][kk] = (f < n4 && c0 + kk < np)
                                     ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    prs, off + (uint32_t)((c0 + kk) * rec * 4), 0, CPOL_SC1))
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (threadIdx.x < MB * G) {
                const int kk = threadIdx.x / G;
                const int h = threadIdx.x % G;
                const bool ok = c0 + kk < np;
                const uint32_t off = (uint32_t)(((size_t)(p0 + c0 + kk) * rec + GH + h) * sizeof(float));
                const float mv = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, off, 0, CPOL_SC1)) : -INFINITY;
                const float lv = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, off + 4 * G, 0, CPOL_SC1)) : 0.f;
                cm[kk * 16 + h] = mv;
                cl[kk * 16 + h] = lv;
            }
            __syncthreads();
#pragma unroll
            for (int ch = 0; ch < MAXC; ++ch) {
                if (ch * NT >= n4) break;
                const int f = ch * NT + threadIdx.x;
                if (f < n4) {
                    const int h = (4 * f) / HD;
                    const float *mk = cm + h;
                    const float *lk = cl + h;
                    float M = Ma[ch];
#pragma unroll
                    for (int kk = 0; kk < MB; ++kk) M = fmaxf(M, mk[kk * 16]);
                    const float bse = (M == -INFINITY) ? 0.f : M;
                    const float so = exp2f(Ma[ch] - bse);
                    f32x4 O = Oa[ch] * so;
                    float L = La[ch] * so;
#pragma unroll
                    for (int kk = 0; kk < MB; ++kk) {
                        const float fw = exp2f(mk[kk * 16] - bse);  // empty slot: -inf -> 0
                        O += fw * ov[ch][kk];
                        L += fw * lk[kk * 16];
                    }
                    Oa[ch] = O;
                    La[ch] = L;
                    Ma[ch] = M;
                }
            }
        }
#pragma unroll
        for (int ch = 0; ch < MAXC; ++ch) {
            if (ch * NT >= n4) break;
            const int f = ch * NT + threadIdx.x;
            if (f < n4) {
                const int h = (4 * f) / HD;
                const int d = 4 * f - h * HD;
                const float L = La[ch];
                const int64_t oi = out_index(bg, h);
                *(f32x4 *)(a.out + oi * HD + d) = L > 0.f ? Oa[ch] * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
                if (d == 0 && a.lse) a.lse[oi] = L > 0.f ? (Ma[ch] + log2f(L)) * LN2 : -INFINITY;
            }
        }
        if (threadIdx.x == 0) reset_dev(&cnt[bg * CNT_STRIDE]);
    };

    // ---- the (b, g) segments of this workgroup's range -----------------------
    // A (b, g) that lies wholly inside the range is finished here (its output
    // written from the 4 wave states).  At most two are shared with other
    // workgroups: the first (it starts before W0) and the last (it goes on
    // past W1).  Each is published (4 wave states combined, stored as one
    // partial) and counted as soon as this workgroup is done with it.
    const bool first_split = lds_F[bg_first] < W0;
    const bool last_split = lds_F[bg_last + 1] > W1;
    const bool one = bg_first == bg_last;
    const bool pub_first = !one && first_split;                            // slot 1
    const bool pub_last = one ? (first_split || last_split) : last_split;  // slot 0
    if constexpr (RING) {
        // the new token's row goes into ring slot t % w; the wave that reads
        // that ring step writes it now, so that the wait at the end of its
        // first staging covers these stores
        for (int bg = bg_first; bg <= bg_last; ++bg) {
            const int b = bg / c.n_kv;
            const int tb = lds_t[b];
            if (tb < 0) continue;
            const int sn = lds_F[bg] + (tb % w) / KSTEP;
            if (sn < W0 || sn >= W1 || (sn - W0) % NW != wave) continue;
            const int g = bg - b * c.n_kv;
            const int slot = tb % w;
            const __bf16 *kn = (const __bf16 *)a.k_new + (int64_t)b * a.ld_new + (int64_t)g * HD;
            const __bf16 *vn = (const __bf16 *)a.v_new + (int64_t)b * a.ld_new + (int64_t)g * HD;
            if (lane < HD / 8)
                *(bf16x8 *)((__bf16 *)c.ring_k + kv_k_index((int64_t)bg * w + slot, 8 * lane, HD)) =
                    *(const bf16x8 *)(kn + 8 * lane);
            for (int e = lane; e < HD; e += 64) ((__bf16 *)c.ring_v)[kv_v_index((int64_t)bg * w + slot, e, HD)] = vn[e];
        }
    }
    int k = 0;  // next step of this wave to compute (its loads are in flight)
    {
        // the first (b, g)'s query goes out with the page-id loads of the
        // first staging, whose wait covers both
        bf16x8 qv[HD / 32];
        q_load(bg_first, qv);
        if (nk > 0) stage_pages(0);
        q_store(qv);
    }
    if (nk > 0) {
        issue(0, kA, vA);
        stage_counts();
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
                stage_pages(k);
                if ((k & 1) == 0) issue(k, kA, vA); else issue(k, kB, vB);
                stage_counts();
            }
        }
        if (bg == bg_first && pub_first) {
            // publish and arrive now, so that arrivals are spread over the
            // launch instead of all falling at its end
            save_state(1);
            __syncthreads();
            publish(1, bg_first, threadIdx.x, NT);
            __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
            __syncthreads();
            if (threadIdx.x == 0) {
                int p0, np;
                parts_of(bg_first, p0, np);
                lds_flag[0] = arrive_dev(&cnt[bg_first * CNT_STRIDE]) == np - 1;
            }
            __syncthreads();
            if (lds_flag[0]) {
                merge(bg_first);
                __syncthreads();
            }
        } else if (bg == bg_last && pub_last) {
            save_state(0);
        } else {
            // whole (b, g) in this workgroup: normalise and write the output
            save_state(0);
            __syncthreads();
            for (int f = threadIdx.x; f < G * HD / 4; f += NT) {
                const int h = (4 * f) / HD;
                const int d = 4 * f - h * HD;
                float M, L;
                f32x4 O;
                combine4(0, h, d, M, O, L);
                const int64_t oi = out_index(bg, h);
                *(f32x4 *)(a.out + oi * HD + d) = L > 0.f ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
                if (d == 0 && a.lse) a.lse[oi] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
            }
            __syncthreads();
        }
        if (bg < bg_last) reset(bg + 1);
    }

    // ---- the last (b, g), if shared: publish, arrive, the last arrival merges
    if (!pub_last) return;
    __syncthreads();
    publish(0, bg_last, threadIdx.x, NT);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        int p0, np;
        parts_of(bg_last, p0, np);
        lds_flag[1] = arrive_dev(&cnt[bg_last * CNT_STRIDE]) == np - 1;
    }
    __syncthreads();
    if (lds_flag[1]) merge(bg_last);
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
    // key and value of slot j of a page or ring region (block storage order)
    auto visit = [&](const float *kreg, const float *vreg, int j) {
        float s = 0.f;
        for (int i = 0; i < PER; ++i) s += q[i] * kreg[kv_k_index(j, lane + 64 * i, HD)];
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        s *= a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
        for (int i = 0; i < PER; ++i) o[i] = o[i] * alpha + p * vreg[kv_v_index(j, lane + 64 * i, HD)];
        m = m_new;
    };
    const int w = c.window;
    const float *rk = (const float *)c.ring_k + (int64_t)bg * w * HD;
    const float *rv = (const float *)c.ring_v + (int64_t)bg * HD * w;
    for (int slot = 0; slot < w; ++slot)
        if (slot <= t) visit(rk, rv, slot);
    const int len = c.lengths[bg];
    const int P = c.page_size;
    const int32_t *pt = c.page_table + (int64_t)bg * c.max_pages;
    for (int j = 0; j < len; ++j) {
        const int page = pt[j >> c.page_shift];
        const int slot = j & (P - 1);
        if (c.pos_pages[(int64_t)page * P + slot] > t - w) break;  // positions increase
        visit((const float *)c.k_pages + (int64_t)page * P * HD, (const float *)c.v_pages + (int64_t)page * P * HD, slot);
    }
    float *op = a.out + ((int64_t)b * a.n_q + h) * HD;
    for (int i = 0; i < PER; ++i) op[lane + 64 * i] = l > 0.f ? o[i] / l : 0.f;
    if (lane == 0 && a.lse) a.lse[(int64_t)b * a.n_q + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

namespace {

// Workspace of the bf16 kernel: arrival counters (one 256-byte line per
// (b, g), then the fused step's two counters), the fused step's gate sums,
// then the split-K partials.
// With fixed_counters the counters are laid out for the largest batch * n_kv,
// so that they sit at the same place whatever the cache.
struct WsLayout {
    size_t gshare, part, total;
    int max_items;
};

WsLayout ws_layout(const spkv_cache *c, int n_q, int grid, int fused_model, int fused_hidden, bool fixed_counters) {
    const int BG = c->batch * c->n_kv;
    const int G = n_q / c->n_kv;
    WsLayout L;
    L.gshare = round256(ws_header_bytes(fixed_counters ? MAX_BG : BG));
    L.part = L.gshare + fused_bytes(fused_model, fused_hidden);
    // a workgroup's contiguous range meets each (b, g) in at most one
    // segment, and consecutive (b, g) share at most one workgroup
    L.max_items = grid + BG;
    L.total = L.part + (size_t)L.max_items * rec_floats(G, c->head_dim) * sizeof(float);
    return L;
}

}  // namespace

size_t decode_ws_bytes(const spkv_cache *c, int n_q, int grid, int *max_items_out, int fused_model, int fused_hidden,
                       bool fixed_counters) {
    if (c->dtype != SPKV_BF16) {
        if (max_items_out) *max_items_out = 0;
        return 0;
    }
    const WsLayout L = ws_layout(c, n_q, grid, fused_model, fused_hidden, fixed_counters);
    if (max_items_out) *max_items_out = L.max_items;
    return L.total;
}

void decode_ws_assign(DecodeArgs &a, const spkv_cache *c, int n_q, int grid, int fused_model, int fused_hidden,
                      bool fixed_counters, char *ws) {
    if (c->dtype != SPKV_BF16 || !ws) {
        a.cnt = nullptr;
        a.gshare = nullptr;
        a.part = nullptr;
        a.max_items = 0;
        return;
    }
    const WsLayout L = ws_layout(c, n_q, grid, fused_model, fused_hidden, fixed_counters);
    a.cnt = (int32_t *)ws;
    a.gshare = (float *)(ws + L.gshare);
    a.part = (float *)(ws + L.part);
    a.max_items = L.max_items;
}

bool decode_fused_ok(const spkv_cache *c, int d_hidden, int grid) {
    // the last workgroup is the finisher; the gate units go to the others
    return c->dtype == SPKV_BF16 && c->batch <= FUSED_ROWS && d_hidden >= 1 && grid >= 2 && c->n_kv <= 16;
}

// polls of the fused step's waits before they give up (each poll takes a
// device-scope round trip, about a microsecond; the waits normally end within
// tens of microseconds)
int g_wait_limit = kDefaultWaitLimit;

int decode_blocks_per_cu() {
    int n = 1 << 20;
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<128, 0>, NT, 0) == hipSuccess) n = min(n, v);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<64, 0>, NT, 0) == hipSuccess) n = min(n, v);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<128, MODE_STEP>, NT, 0) == hipSuccess) n = min(n, v);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<64, MODE_STEP>, NT, 0) == hipSuccess) n = min(n, v);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<128, MODE_RING>, NT, 0) == hipSuccess) n = min(n, v);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, decode_bf16_kernel<64, MODE_RING>, NT, 0) == hipSuccess) n = min(n, v);
    return max(1, n == (1 << 20) ? 1 : n);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const CacheView &c = a.c;
    const int mode = a.gate.d_hidden > 0 ? MODE_STEP : (a.k_new ? MODE_RING : 0);
    if (c.dtype == SPKV_BF16) {
        const dim3 grid(a.grid);
        if (c.head_dim == 128) {
            if (mode == MODE_STEP) hipLaunchKernelGGL((decode_bf16_kernel<128, MODE_STEP>), grid, dim3(NT), 0, s, a);
            else if (mode == MODE_RING) hipLaunchKernelGGL((decode_bf16_kernel<128, MODE_RING>), grid, dim3(NT), 0, s, a);
            else hipLaunchKernelGGL((decode_bf16_kernel<128, 0>), grid, dim3(NT), 0, s, a);
        } else {
            if (mode == MODE_STEP) hipLaunchKernelGGL((decode_bf16_kernel<64, MODE_STEP>), grid, dim3(NT), 0, s, a);
            else if (mode == MODE_RING) hipLaunchKernelGGL((decode_bf16_kernel<64, MODE_RING>), grid, dim3(NT), 0, s, a);
            else hipLaunchKernelGGL((decode_bf16_kernel<64, 0>), grid, dim3(NT), 0, s, a);
        }
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
