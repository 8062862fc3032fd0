// The utility gate of SP-KV (arXiv 2605.14037), section 2.1, Eq. (1)-(2):
//   a = ReLU(W1 h + b1), logit = W2 a + b2, u = sigmoid(logit), z = [u >= tau]
// one output per key head.  The hidden activation a stays in f32 between the
// two layers (a bf16 rounding there could move u by ~1e-3).
//
// bf16: the first layer is a GEMM [rows x d_model] . [d_model x d_hidden] on
// v_mfma_f32_16x16x32_bf16; both operands are K-contiguous rows (hidden
// states, W1 rows), so lanes load 16-byte pieces straight from memory.  The
// epilogue (bias, ReLU, second layer, sigmoid, threshold) runs from LDS in
// the same kernel.  For up to 64 rows d_model is split over several
// workgroups that write partial sums; a second small kernel adds the slices
// in a fixed order and runs the epilogue.
// Up to 16 rows (decode), one launch: bf16 -- one workgroup per 16-unit tile
// and d_model part on MFMA, storing its partial first-layer sums; f32 -- one
// workgroup per hidden unit, storing its share W2[:, j] a_j of every logit.
// The workgroup that finishes last adds the pieces in a fixed order, so the
// result does not depend on scheduling.
// f32 with more rows, or d_hidden outside {32, 64, 128, 256}: a plain VALU
// kernel.
#include "spkv_internal.h"
#include "spkv_device.h"
#include "spkv_gate_dev.h"

namespace spkv {
namespace {

constexpr int NT = 256;
// the workspace starts with a 256-byte header holding the arrival counter of
// the few-row kernel; partial sums follow it
constexpr int WS_HEADER_FLOATS = 64;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// Second layer + sigmoid + threshold for `rows` rows whose activations
// (after bias and ReLU) are in act[r * ld + j].  W2 and b2 are staged in LDS
// first (one coalesced pass), so the dot products never wait on memory.
template <int HG>
__device__ void gate_epilogue(const GateArgs &a, const float *act, int ld, int64_t row0, int rows,
                              float *lds_w2 /* [n_kv][HG + 1] */) {
    const int nkv = a.n_kv;
    for (int i = threadIdx.x; i < nkv * HG; i += blockDim.x) {
        const int k = i / HG;
        lds_w2[k * (HG + 1) + (i - k * HG)] = a.w2[i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * nkv; idx += blockDim.x) {
        const int r = idx / nkv;
        const int k = idx - r * nkv;
        const int64_t row = row0 + r;
        if (row >= a.n_rows) continue;
        const float *w2 = lds_w2 + k * (HG + 1);
        const float *ar = act + r * ld;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 16
        for (int j = 0; j < HG; j += 2) {
            acc0 = fmaf(w2[j], ar[j], acc0);
            acc1 = fmaf(w2[j + 1], ar[j + 1], acc1);
        }
        const float logit = (acc0 + acc1) + a.b2[k];
        const float u = sigmoid_f(logit);
        if (a.utility) a.utility[row * nkv + k] = u;
        a.keep[row * nkv + k] = (u >= a.tau) ? 1 : 0;  // NaN -> 0
    }
}

__device__ inline float relu_keep_nan(float x) { return x < 0.f ? 0.f : x; }

// ---------------------------------------------------------------------------
// bf16, many rows (d_model a multiple of 64): 64 rows x all HG hidden units per
// workgroup, one 16-row MFMA tile per wave; iteration j covers d_model
// columns [64 j, 64 j + 64).  The hidden rows -- the HBM stream, each row
// read by one wave only -- go straight into registers, P iterations ahead of
// their use.  W1 -- the same for every workgroup and L2-resident -- is shared
// by the 4 waves through a ring of P + 1 LDS stages filled P iterations
// ahead by direct global -> LDS loads (unit u's 64 columns = 128 bytes:
// 16-byte chunk c at u*128 + 16*(c ^ ((u >> 1) & 7)), so the 16 lanes that
// read one operand group hit 16 different bank groups).
typedef __attribute__((address_space(3))) void lds_void;

template <int HG, int JC> struct GatePipe {
    // One depth for both streams: vector-memory loads complete in issue
    // order, so waiting for W1's pieces of iteration j also waits for every
    // hidden-row load issued before them -- a deeper register prefetch than
    // the W1 ring would not keep more bytes in flight.  The W1 ring (HG / 64
    // times the hidden-row bytes of an iteration) is what fills the LDS.
    static constexpr int P = HG <= 128 ? 8 : 3;
    static constexpr int NSTAGE = P + 1;
    static constexpr int SBYTES = HG * 128;              // W1 stage: HG units x 64 columns
    static constexpr int LB = SBYTES / 1024 / 4;         // direct loads per wave and stage
    static constexpr int LA = 2;                         // hidden-row loads per wave and iteration
    static constexpr int EPI = 64 * (HG + 1) * 4 + 16 * (HG + 1) * 4;
    static constexpr int LDS = NSTAGE * SBYTES > EPI ? NSTAGE * SBYTES : EPI;
};

// s_waitcnt vmcnt(n), n in [0, N] (the immediate must be a constant)
template <int N>
__device__ inline void wait_vm(int n) {
    if constexpr (N > 0) {
        if (n >= N) {
            __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
            return;
        }
        wait_vm<N - 1>(n);
    } else {
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    }
}

// JC > 0: d_model = 64 JC fixed at compile time, so the loop unrolls fully,
// the wait counts fold to constants and the compiler tracks each hidden-row
// load to its use (a run-time trip count makes it wait for every load at the
// top of each unrolled block).
template <int HG, int JC>
__global__ void __launch_bounds__(NT) gate_pipe_kernel(GateArgs a) {
    using C = GatePipe<HG, JC>;
    constexpr int P = C::P;
    constexpr int NTL = HG / 16;  // unit tiles
    static_assert((P - 1) * (C::LB + C::LA) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * 64;
    const int J = JC > 0 ? JC : a.d_model / 64;  // iterations
    const int64_t my_row = min(row0 + wave * 16 + i16, a.n_rows - 1);  // rows past n re-read the last
    const __bf16 *hrow = (const __bf16 *)a.hidden + my_row * a.ld_hidden + 8 * q4;
    const char *w1 = (const char *)a.w1;
    const int64_t w1_row_bytes = (int64_t)a.d_model * 2;

    // W1 columns [64 j, 64 j + 64) of all units -> stage st
    auto issue_w1 = [&](int j, int st) {
#pragma unroll
        for (int u = 0; u < C::LB; ++u) {
            const int i = wave + 4 * u;         // 1 KB piece: units 8 i .. 8 i + 7
            const int unit = 8 * i + (lane >> 3);
            const int c = (lane & 7) ^ ((unit >> 1) & 7);
            const char *src = w1 + unit * w1_row_bytes + (int64_t)(64 * j + 8 * c) * 2;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds + st * C::SBYTES + i * 1024), 16, 0, 0);
        }
    };
    bf16x8 av[P][2];
    auto issue_h = [&](int j, bf16x8 (&dst)[2]) {
        dst[0] = *(const bf16x8 *)(hrow + 64 * j);
        dst[1] = *(const bf16x8 *)(hrow + 64 * j + 32);
    };

    f32x4 acc[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: iterations 0 .. P-1 in flight (W1 then hidden rows, per iteration)
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (i < J) {
            issue_w1(i, i);
            issue_h(i, av[i]);
        }
    }
#pragma unroll
    for (int j0 = 0; j0 < (JC > 0 ? JC : J); j0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int j = j0 + u;
            if (j < J) {
                // this wave's loads of iteration j are done once at most the
                // younger iterations' loads are outstanding
                wait_vm<63>(min(P - 1, J - 1 - j) * (C::LB + C::LA));
                // every wave's W1 pieces of j have landed, and every wave is
                // done reading stage (j - 1) (its reads were consumed by its
                // MFMAs): a plain barrier, no fence (a fence would also wait
                // for the hidden-row loads still in flight)
                __builtin_amdgcn_s_barrier();
                if (j + P < J) issue_w1(j + P, (j + P) % C::NSTAGE);
                const char *st = lds + (j % C::NSTAGE) * C::SBYTES;
                // all operand reads of the iteration first, so that their
                // latencies overlap each other and the MFMAs
                bf16x8 bv[2][NTL];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int n = 0; n < NTL; ++n) {
                        const int unit = 16 * n + i16;
                        bv[ks][n] = *(const bf16x8 *)(st + unit * 128 + (((4 * ks + q4) ^ ((unit >> 1) & 7)) << 4));
                    }
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int n = 0; n < NTL; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][ks], bv[ks][n], acc[n], 0, 0, 0);
                if (j + P < J) issue_h(j + P, av[u]);
            }
        }
    }
    __syncthreads();  // the stages become the epilogue's scratch
    float *act = (float *)lds;                       // [64][HG + 1]
    float *lds_w2 = act + 64 * (HG + 1);             // [16][HG + 1]
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
        const int jj = 16 * n + i16;
        const float bias = a.b1[jj];
#pragma unroll
        for (int r = 0; r < 4; ++r) act[(wave * 16 + 4 * q4 + r) * (HG + 1) + jj] = relu_keep_nan(acc[n][r] + bias);
    }
    __syncthreads();
    gate_epilogue<HG>(a, act, HG + 1, row0, 64, lds_w2);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  Workgroup tile: (16 * WM) rows x HG hidden units; waves
// are arranged WM (rows) x (4 / WM) (hidden units).  blockIdx.y = d_model
// slice when n_split > 1.
template <int WM, int HG>
__global__ void __launch_bounds__(NT) gate_bf16_kernel(GateArgs a) {
    constexpr int WN = 4 / WM;
    constexpr int BM = 16 * WM;
    constexpr int NTW = HG / 16 / WN;  // 16-wide unit tiles per wave
    static_assert(NTW >= 1, "d_hidden too small for this wave layout");
    __shared__ float act[BM][HG + 1];
    __shared__ float lds_w2[16 * (HG + 1)];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * BM;
    const int split = blockIdx.y;
    const int steps_total = a.d_model / 32;
    const int steps = steps_total / a.n_split;
    const int k_lo = split * steps * 32;

    f32x4 acc[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t my_row = row0 + wm * 16 + i16;
    const bool row_ok = my_row < a.n_rows;
    const __bf16 *hrow = (const __bf16 *)a.hidden + (row_ok ? my_row : 0) * a.ld_hidden + k_lo + 8 * q4;
    const __bf16 *w1 = (const __bf16 *)a.w1;
    const __bf16 *wrow[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n)
        wrow[n] = w1 + (int64_t)((wn * NTW + n) * 16 + i16) * a.d_model + k_lo + 8 * q4;

    for (int s = 0; s < steps; ++s) {
        bf16x8 av = row_ok ? *(const bf16x8 *)(hrow + 32 * s) : bf16x8{};
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const bf16x8 bv = *(const bf16x8 *)(wrow[n] + 32 * s);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
        }
    }

    if (a.n_split == 1) {
        // D layout: lane holds rows 4*q4 + r, unit 16*tile + i16
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            const int j = (wn * NTW + n) * 16 + i16;
            const float bias = a.b1[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) act[wm * 16 + 4 * q4 + r][j] = relu_keep_nan(acc[n][r] + bias);
        }
        __syncthreads();
        gate_epilogue<HG>(a, &act[0][0], HG + 1, row0, BM, lds_w2);
        return;
    }

    // split d_model: write this slice's sums; gate_split_epilogue adds them
    const int n_tiles = gridDim.x;
    float *part = a.ws + WS_HEADER_FLOATS;  // [n_split][n_tiles * BM][HG]
    const size_t slab = (size_t)n_tiles * BM * HG;
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
        const int j = (wn * NTW + n) * 16 + i16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = (int)(blockIdx.x * BM) + wm * 16 + 4 * q4 + r;
            part[split * slab + (size_t)rr * HG + j] = acc[n][r];
        }
    }
}

// Sum of the d_model slices in slice order (deterministic), then bias, ReLU
// and the epilogue.  One workgroup per row tile of the split launch.
template <int BM, int HG>
__global__ void __launch_bounds__(NT) gate_split_epilogue(GateArgs a) {
    __shared__ float act[BM][HG + 1];
    __shared__ float lds_w2[16 * (HG + 1)];
    const size_t slab = (size_t)gridDim.x * BM * HG;
    const float *part = a.ws + WS_HEADER_FLOATS;
    for (int idx = threadIdx.x; idx < BM * HG; idx += NT) {
        const int r = idx / HG;
        const int j = idx - r * HG;
        const size_t off = (size_t)(blockIdx.x * BM + r) * HG + j;
        float sum = 0.f;
#pragma unroll 16
        for (int sp = 0; sp < a.n_split; ++sp) sum += part[sp * slab + off];
        act[r][j] = relu_keep_nan(sum + a.b1[j]);
    }
    __syncthreads();
    gate_epilogue<HG>(a, &act[0][0], HG + 1, (int64_t)blockIdx.x * BM, BM, lds_w2);
}

// ---------------------------------------------------------------------------
// f32 (and any d_hidden) VALU kernel: one workgroup per row.
template <typename T>
__global__ void __launch_bounds__(NT) gate_valu_kernel(GateArgs a) {
    __shared__ float part[NT];
    __shared__ float act[256];
    const int64_t row = blockIdx.x;
    const int hg = a.d_hidden;
    const int per = NT / hg;  // threads per hidden unit (>= 1 since hg <= 256)
    const int j = threadIdx.x % hg;
    const int p = threadIdx.x / hg;
    float acc = 0.f;
    if (p < per) {
        const T *h = (const T *)a.hidden + row * a.ld_hidden;
        const T *w = (const T *)a.w1 + (int64_t)j * a.d_model;
        for (int i = p; i < a.d_model; i += per) acc = fmaf((float)w[i], (float)h[i], acc);
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < hg) {
        float s = 0.f;
        for (int q = 0; q < per; ++q) s += part[q * hg + threadIdx.x];
        act[threadIdx.x] = relu_keep_nan(s + a.b1[threadIdx.x]);
    }
    __syncthreads();
    if (threadIdx.x < a.n_kv) {
        const int k = threadIdx.x;
        const float *w2 = a.w2 + (int64_t)k * hg;
        float acc = 0.f;
        for (int j = 0; j < hg; ++j) acc = fmaf(w2[j], act[j], acc);
        const float u = sigmoid_f(acc + a.b2[k]);
        if (a.utility) a.utility[row * a.n_kv + k] = u;
        a.keep[row * a.n_kv + k] = (u >= a.tau) ? 1 : 0;  // NaN -> 0
    }
}

// ---------------------------------------------------------------------------
// Few rows (n_rows <= NR <= 16): workgroup j computes hidden unit j for every
// row over the whole d_model and stores its share W2[k][j] * a_j of logit
// (row, k); the last workgroup to arrive adds the shares in unit order, then
// sigmoid and threshold (gate_unit_share / gate_finish).
template <typename T, int NR>
__global__ void __launch_bounds__(NT) gate_tiny_kernel(GateArgs a) {
    __shared__ float red[(NT / 64) * NR];
    __shared__ int lds_last;
    int *cnt = (int *)a.ws;
    float *part = a.ws + WS_HEADER_FLOATS;  // [d_hidden][NR][n_kv]
    gate_unit_share<T, NR, NT>(a, blockIdx.x, part, red);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's share is stored
    __syncthreads();
    if (threadIdx.x == 0) lds_last = arrive_dev(cnt) == (int)gridDim.x - 1;
    __syncthreads();
    if (!lds_last) return;
    gate_finish<NR, NT>(a, part, nullptr);
    if (threadIdx.x == 0) reset_dev(cnt);
}

// bf16, up to 16 rows: one workgroup per (16-unit tile, d_model part), on
// MFMA; the last workgroup to arrive finishes (gate_tile_share /
// gate_tile_finish).
__global__ void __launch_bounds__(NT) gate_tile_kernel(GateArgs a) {
    __shared__ float red[4 * 16 * 17];
    __shared__ float act[16 * 256];
    __shared__ int lds_last;
    int *cnt = (int *)a.ws;
    float *part = a.ws + WS_HEADER_FLOATS;  // [items][16][16]
    gate_tile_share(a, blockIdx.x, part, red);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's sums are stored
    __syncthreads();
    if (threadIdx.x == 0) lds_last = arrive_dev(cnt) == (int)gridDim.x - 1;
    __syncthreads();
    if (!lds_last) return;
    gate_tile_finish(a, part, act, nullptr);
    if (threadIdx.x == 0) reset_dev(cnt);
}

constexpr int SMALL_ROWS = 64;
constexpr int TINY_ROWS = 16;

}  // namespace

int gate_split_for(int d_model, int dtype, int64_t n_rows) {
    if (dtype != SPKV_BF16 || n_rows > SMALL_ROWS || n_rows <= TINY_ROWS) return 1;
    const int steps = d_model / 32;
    int split = 1;
    while (split * 2 <= 16 && steps % (split * 2) == 0) split *= 2;
    return split;
}

static bool mfma_hidden(int hg) { return hg == 32 || hg == 64 || hg == 128 || hg == 256; }

// rows per workgroup on the small-row (split) path: 16 * WM with WM = 2 for
// d_hidden = 32 (two 16-unit tiles) and 1 otherwise
static int small_bm(int hg) { return hg == 32 ? 32 : 16; }

size_t gate_ws_bytes(int d_model, int d_hidden, int n_kv, int dtype, int64_t n_rows) {
    const size_t header = WS_HEADER_FLOATS * sizeof(float);
    if (n_rows > 0 && n_rows <= TINY_ROWS) {
        if (dtype == SPKV_BF16) return header + (size_t)gate_tile_items(d_model, d_hidden) * 256 * sizeof(float);
        return header + (size_t)d_hidden * TINY_ROWS * n_kv * sizeof(float);
    }
    const int split = gate_split_for(d_model, dtype, n_rows);
    if (split == 1 || !mfma_hidden(d_hidden)) return 0;
    const int bm = small_bm(d_hidden);
    const int64_t tiles = (n_rows + bm - 1) / bm;
    return header + (size_t)split * tiles * bm * d_hidden * sizeof(float);
}

template <typename T>
static void launch_tiny(const GateArgs &a, hipStream_t s) {
    const dim3 grid(a.d_hidden);
    if (a.n_rows <= 4)
        hipLaunchKernelGGL((gate_tiny_kernel<T, 4>), grid, dim3(NT), 0, s, a);
    else if (a.n_rows <= 8)
        hipLaunchKernelGGL((gate_tiny_kernel<T, 8>), grid, dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL((gate_tiny_kernel<T, 16>), grid, dim3(NT), 0, s, a);
}

template <int WM, int HG>
static void launch_mfma_hg(const GateArgs &a, int tiles, hipStream_t s) {
    hipLaunchKernelGGL((gate_bf16_kernel<WM, HG>), dim3(tiles, a.n_split), dim3(NT), 0, s, a);
    if (a.n_split > 1) hipLaunchKernelGGL((gate_split_epilogue<16 * WM, HG>), dim3(tiles), dim3(NT), 0, s, a);
}

template <int WM>
static void launch_mfma(const GateArgs &a, int tiles, hipStream_t s) {
    switch (a.d_hidden) {
    case 32: launch_mfma_hg<(WM < 2 ? 2 : WM), 32>(a, tiles, s); break;
    case 64: launch_mfma_hg<WM, 64>(a, tiles, s); break;
    case 128: launch_mfma_hg<WM, 128>(a, tiles, s); break;
    default: launch_mfma_hg<WM, 256>(a, tiles, s); break;
    }
}

hipError_t launch_gate(const GateArgs &a0, hipStream_t s) {
    GateArgs a = a0;
    if (a.n_rows <= TINY_ROWS) {
        if (a.dtype == SPKV_BF16)
            hipLaunchKernelGGL(gate_tile_kernel, dim3(gate_tile_items(a.d_model, a.d_hidden)), dim3(NT), 0, s, a);
        else
            launch_tiny<float>(a, s);
    } else if (a.dtype == SPKV_BF16 && mfma_hidden(a.d_hidden)) {
        if (a.n_split > 1) {
            const int bm = small_bm(a.d_hidden);
            const int tiles = (int)((a.n_rows + bm - 1) / bm);
            launch_mfma<1>(a, tiles, s);
        } else if (a.d_model % 64 == 0) {
            const dim3 grid((unsigned)((a.n_rows + 63) / 64));
            if (a.d_model == 4096) {
                switch (a.d_hidden) {
                case 32: hipLaunchKernelGGL((gate_pipe_kernel<32, 64>), grid, dim3(NT), 0, s, a); break;
                case 64: hipLaunchKernelGGL((gate_pipe_kernel<64, 64>), grid, dim3(NT), 0, s, a); break;
                case 128: hipLaunchKernelGGL((gate_pipe_kernel<128, 64>), grid, dim3(NT), 0, s, a); break;
                default: hipLaunchKernelGGL((gate_pipe_kernel<256, 64>), grid, dim3(NT), 0, s, a); break;
                }
            } else {
                switch (a.d_hidden) {
                case 32: hipLaunchKernelGGL((gate_pipe_kernel<32, 0>), grid, dim3(NT), 0, s, a); break;
                case 64: hipLaunchKernelGGL((gate_pipe_kernel<64, 0>), grid, dim3(NT), 0, s, a); break;
                case 128: hipLaunchKernelGGL((gate_pipe_kernel<128, 0>), grid, dim3(NT), 0, s, a); break;
                default: hipLaunchKernelGGL((gate_pipe_kernel<256, 0>), grid, dim3(NT), 0, s, a); break;
                }
            }
        } else {
            const int tiles = (int)((a.n_rows + 63) / 64);
            launch_mfma<4>(a, tiles, s);
        }
    } else {
        a.n_split = 1;
        if (a.dtype == SPKV_BF16)
            hipLaunchKernelGGL(gate_valu_kernel<__bf16>, dim3((unsigned)a.n_rows), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL(gate_valu_kernel<float>, dim3((unsigned)a.n_rows), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace spkv
