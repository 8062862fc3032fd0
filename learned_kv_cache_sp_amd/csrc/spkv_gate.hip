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
// the few-row kernels; partial sums follow it
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
    static constexpr int PIECES = HG / 8;                // 1 KB pieces of a W1 stage (8 units each)
    static constexpr int LB = (PIECES + 3) / 4;          // direct loads per wave and stage (at most)
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
    const int64_t w1_row_bytes = (int64_t)a.d_model * 2;
    const char *w1 = (const char *)a.w1;
    // this wave's share of a stage's pieces (pieces wave, wave + 4, ...)
    const int lbw = (C::PIECES - wave + 3) / 4;

    // W1 columns [64 j, 64 j + 64) of all units -> stage st
    auto issue_w1 = [&](int j, int st) {
#pragma unroll
        for (int u = 0; u < C::LB; ++u) {
            const int i = wave + 4 * u;         // 1 KB piece: units 8 i .. 8 i + 7
            if (C::PIECES % 4 == 0 || i < C::PIECES) {
                const int unit = 8 * i + (lane >> 3);
                const int c = (lane & 7) ^ ((unit >> 1) & 7);
                const char *src = w1 + unit * w1_row_bytes + (int64_t)(64 * j + 8 * c) * 2;
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(lds + st * C::SBYTES + i * 1024), 16, 0, 0);
            }
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
                wait_vm<63>(min(P - 1, J - 1 - j) * (lbw + C::LA));
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
// Many rows, HG in {64, 128, 256}: 64 rows per workgroup, the hidden units
// split over the 4 waves (wave w owns unit tiles w * NTW .. w * NTW + NTW - 1
// for all 64 rows).  Per 64-column iteration the workgroup's hidden tile
// (64 rows x 128 bytes, the HBM stream) lands in an LDS ring by direct
// global->LDS loads, a quarter from each wave, and every wave reads it as its
// B operands; each wave loads its own W1 rows (L2-resident) into registers
// as whole 128-byte lines, eight rows per instruction, and passes them
// through a small LDS slice of its own into the A-operand layout.  (Loading
// the operand layout directly -- 16 rows x 64 bytes per instruction -- runs
// at about a third of the rate per compute unit, and every workgroup loads
// all of W1.)  Sharing the hidden tile rather than W1 keeps the LDS traffic
// per iteration low (8 KB written + 4 x 8 KB read for the tile).
// Layer 1 is computed transposed, a^T[unit][row] = W1 . h^T, so that each
// lane ends up holding one row and four units of every 16 x 16 tile --
// exactly the B operand of the f32 16x16x4 MFMA that forms layer 2
// (logit^T[head][row] = W2 . a^T), four units per step, with no data
// movement; the 4 waves' partial logits (each over its own units) are added
// in wave order.
//
// One LDS object per ring stage: the compiler then sees the direct loads into
// one stage and the operand reads of another as disjoint (with one array it
// makes some reads wait for every load in flight).
template <int S, int SB>
__device__ __attribute__((always_inline)) inline char *stage_obj() {
    __shared__ __attribute__((aligned(1024))) char buf[SB];
    return buf;
}
template <int SB, int N>
__device__ __attribute__((always_inline)) inline char *stage_at(int st) {
    if constexpr (N > 1) {
        if (st == N - 1) return stage_obj<N - 1, SB>();
        return stage_at<SB, N - 1>(st);
    } else {
        return stage_obj<0, SB>();
    }
}

// the two W1 slices of the 64-row kernel (each its own LDS object as well)
template <int S, int SB>
__device__ __attribute__((always_inline)) inline char *wslice_obj() {
    __shared__ __attribute__((aligned(1024))) char buf[SB];
    return buf;
}
template <int SB>
__device__ __attribute__((always_inline)) inline char *wslice(int p) {
    return p ? wslice_obj<1, SB>() : wslice_obj<0, SB>();
}

template <int HG> struct UnitSplit {
    static constexpr int NTW = HG / 64;                  // 16-unit tiles per wave
    static constexpr int LW = 2 * NTW;                   // W1 register loads per wave and iteration
    static constexpr int LH = 2;                         // hidden-row direct loads per wave and iteration
    // iterations in flight: the vmcnt field (at most 63 outstanding) and the
    // W1 registers (D x 8 NTW) bound the depth; a power of two, so that with
    // d_model = 4096 the loop unrolls completely and every wait count is a
    // constant
    static constexpr int D = (LW + LH) <= 4 ? 16 : (LW + LH) <= 8 ? 8 : 4;
    static constexpr int NSTAGE = D + 1;
    static constexpr int SBYTES = 64 * 128;              // hidden stage: 64 rows x 64 columns
    // epilogue: each wave's partial logits, [4 row tiles][16 heads][16 rows]
    // floats, two waves per stage object
    static constexpr int PART_WAVE = 4 * 256 * 4;
    static_assert(2 * PART_WAVE <= SBYTES, "epilogue scratch fits two stages");
};

// JC: iterations (d_model / 64) when fixed at compile time (0: from d_model)
template <int HG, int JC>
__global__ void __launch_bounds__(NT) gate_unitsplit_kernel(GateArgs a) {
    using C = UnitSplit<HG>;
    constexpr int D = C::D;
    constexpr int NTW = C::NTW;
    static_assert((D - 1) * (C::LW + C::LH) <= 63, "vmcnt range");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * 64;
    const int J = JC > 0 ? JC : a.d_model / 64;  // iterations
    // hidden-tile loads: instruction k of this wave fills rows 16 wave + 8 k ..
    // + 7; lane -> (row, 16-byte slot), slot s of row r holds the row's
    // column chunk s ^ ((r >> 1) & 7) (conflict-free operand reads)
    const __bf16 *hsrc[C::LH];
#pragma unroll
    for (int k = 0; k < C::LH; ++k) {
        const int r = 8 * (C::LH * wave + k) + (lane >> 3);
        const int64_t grow = min(row0 + r, a.n_rows - 1);  // rows past n re-read the last
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        hsrc[k] = (const __bf16 *)a.hidden + grow * a.ld_hidden + 8 * c;
    }
    // W1 rows of this wave, loaded as whole 128-byte lines: instruction m
    // reads units 16 wave NTW + 8 m + (lane >> 3), 16-byte chunk lane & 7 of
    // the iteration's 64 columns; they go through this wave's LDS slice
    // (swizzled like the hidden tile) into the MFMA operand layout
    const __bf16 *wsrc = (const __bf16 *)a.w1 + (int64_t)(16 * wave * NTW + (lane >> 3)) * a.d_model + 8 * (lane & 7);

    // the hidden rows are read once (cache policy 2: non-temporal); W1 is
    // read by every workgroup and stays cacheable
    auto issue_h = [&](int j, int st) {
        char *dst = stage_at<C::SBYTES, C::NSTAGE>(st);
#pragma unroll
        for (int k = 0; k < C::LH; ++k)
            __builtin_amdgcn_global_load_lds((const void *)(hsrc[k] + 64 * j),
                                             (lds_void *)(dst + (C::LH * wave + k) * 1024), 16, 0, 2);
    };
    bf16x8 wv[D][NTW][2];  // [m / 2][m % 2]: instruction m = 2 nn + ks of the raw lines
    auto issue_w = [&](int j, bf16x8 (&dst)[NTW][2]) {
#pragma unroll
        for (int nn = 0; nn < NTW; ++nn)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                dst[nn][ks] = *(const bf16x8 *)(wsrc + (int64_t)8 * (2 * nn + ks) * a.d_model + 64 * j);
    };

    f32x4 acc[4][NTW];  // a^T tiles: lane (row 16 rt + i16, units 16 (wave NTW + nn) + 4 q4 + r)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int nn = 0; nn < NTW; ++nn) acc[rt][nn] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: iterations 0 .. D-1 in flight (hidden tile, then W1, per iteration)
#pragma unroll
    for (int i = 0; i < D; ++i) {
        if (i < J) {
            issue_h(i, i);
            issue_w(i, wv[i]);
        }
    }
#pragma unroll
    for (int j0 = 0; j0 < (JC > 0 ? JC : J); j0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int j = j0 + u;
            if (j < J) {
                // this wave's loads of iteration j are done once at most the
                // younger iterations' loads are outstanding
                wait_vm<63>(min(D - 1, J - 1 - j) * (C::LH + C::LW));
                // every wave's quarter of hidden tile j has landed, and every
                // wave is done reading the stage of j - 1: a plain barrier
                // (a fence would also wait for the loads still in flight)
                __builtin_amdgcn_s_barrier();
                if (j + D < J) issue_h(j + D, (j + D) % C::NSTAGE);
                const char *st = stage_at<C::SBYTES, C::NSTAGE>(j % C::NSTAGE);
                // this wave's W1 lines of j -> its LDS slice (row ur = 8 m + lane / 8)
                char *ws = wslice<NTW * 2048 * 4>(j & 1) + wave * NTW * 2048;
#pragma unroll
                for (int m = 0; m < 2 * NTW; ++m) {
                    const int ur = 8 * m + (lane >> 3);
                    *(bf16x8 *)(ws + ur * 128 + (((lane & 7) ^ ((ur >> 1) & 7)) << 4)) = wv[u][m >> 1][m & 1];
                }
                bf16x8 av[4][2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const int r = 16 * rt + i16;
                        av[rt][ks] = *(const bf16x8 *)(st + r * 128 + (((4 * ks + q4) ^ ((r >> 1) & 7)) << 4));
                    }
                bf16x8 bw[NTW][2];
#pragma unroll
                for (int nn = 0; nn < NTW; ++nn)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int ur = 16 * nn + i16;
                        bw[nn][ks] = *(const bf16x8 *)(ws + ur * 128 + (((4 * ks + q4) ^ ((ur >> 1) & 7)) << 4));
                    }
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                        for (int nn = 0; nn < NTW; ++nn)
                            acc[rt][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[nn][ks], av[rt][ks],
                                                                                  acc[rt][nn], 0, 0, 0);
                if (j + D < J) issue_w(j + D, wv[u]);
            }
        }
    }
    // layer 2 on the f32 MFMA: step (nn, c) takes units 16 (wave NTW + nn) +
    // 4 k + c, k = 0..3; the A operand is W2[head i16][that unit] (zero for
    // heads past n_kv), the B operand ReLU(a^T + b1) from register c of acc
    float w2r[NTW][4], b1r[NTW][4];
#pragma unroll
    for (int nn = 0; nn < NTW; ++nn)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int unit = 16 * (wave * NTW + nn) + 4 * q4 + c;
            w2r[nn][c] = i16 < a.n_kv ? a.w2[i16 * HG + unit] : 0.f;
            b1r[nn][c] = a.b1[unit];
        }
    f32x4 lg[4];  // partial logit^T tiles: lane (row 16 rt + i16, heads 4 q4 + r)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        lg[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nn = 0; nn < NTW; ++nn)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                lg[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w2r[nn][c], relu_keep_nan(acc[rt][nn][c] + b1r[nn][c]),
                                                               lg[rt], 0, 0, 0);
    }
    __syncthreads();  // every wave is done with the ring: its first two stages hold the partials
    float *mine = (float *)(stage_at<C::SBYTES, C::NSTAGE>(wave >> 1) + (wave & 1) * C::PART_WAVE);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[rt * 256 + (4 * q4 + r) * 16 + i16] = lg[rt][r];
    __syncthreads();
    const float *p01 = (const float *)stage_at<C::SBYTES, C::NSTAGE>(0);
    const float *p23 = (const float *)stage_at<C::SBYTES, C::NSTAGE>(1);
    constexpr int PW = C::PART_WAVE / 4;  // floats per wave
    const int nkv = a.n_kv;
    for (int idx = threadIdx.x; idx < 64 * nkv; idx += NT) {
        const int r = idx / nkv;
        const int k = idx - r * nkv;
        const int64_t row = row0 + r;
        if (row >= a.n_rows) continue;
        const int o = (r >> 4) * 256 + k * 16 + (r & 15);
        const float logit = (((p01[o] + p01[PW + o]) + p23[o]) + p23[PW + o]) + a.b2[k];
        const float u = sigmoid_f(logit);
        if (a.utility) a.utility[row * nkv + k] = u;
        a.keep[row * nkv + k] = (u >= a.tau) ? 1 : 0;  // NaN -> 0
    }
}

// ---------------------------------------------------------------------------
// Sink-attention gate (Fast KVzip page, core method): per key head, G query
// vectors and one key of 16 dimensions are projections of the hidden state;
// each query's weight on the token's own key against the n_sinks sink keys
// (scores scaled by 1/sqrt(16), softmax with its maximum subtracted) and the
// largest over the G queries is the utility (a NaN anywhere gives NaN, so
// keep = 0).  A workgroup takes 256 rows and H key heads (wave w:
// rows 64 w .. 64 w + 63), i.e. the T = H (G + 1) projections of d_key = 16
// (G queries and one key per head) as 16-unit tiles.  Every load reads whole
// 128-byte lines (8 rows x 128 bytes per instruction), P iterations ahead,
// into registers: a quarter of the iteration's projection rows of W1 per
// wave, and the wave's own hidden rows; at their iteration they are written
// to double-buffered LDS -- the W1 stage shared by the 4 waves, the hidden
// rows in the wave's slice -- and read back in the operand layout (loads in
// the operand layout, 16 rows x 64 bytes per instruction, and direct
// global->LDS loads both run at about a third of that rate per compute
// unit).  The projections are formed transposed (p^T = W1 . h^T), so a lane holds one row
// and four dimensions (4 k + r) of every tile, and the epilogue works from the
// accumulators: the own-key score is a 4-lane sum of q . k; the sink scores
// are an f32 16x16x4 MFMA of the sink keys against q^T (step c takes the
// dimensions 4 k + c, register c of the tile); then the softmax against the
// sinks, the maximum over the G queries and the threshold.  Taller tiles and
// several heads per workgroup cut the bytes each compute unit loads (the
// weights once per 256 rows, the hidden rows once per H heads).
template <int G, int H, bool FIXED> struct SinkTall {
    static constexpr int T = H * (G + 1);                // projection tiles
    static constexpr int PIECES = 2 * T;                 // 1 KB W1 pieces per stage (8 units x 128 B)
    static constexpr int LB = (PIECES + 3) / 4;          // W1 loads per wave and iteration (at most)
    static constexpr int LA = 8;                         // hidden loads per wave and iteration (64 rows x 128 B)
    // iterations in flight: 4, or 2 with 6 or more tiles in the fully
    // unrolled loop (FIXED: d_model = 4096), whose registers would spill at 4
    static constexpr int P = (T >= 6 && FIXED) ? 2 : 4;
    static constexpr int SBYTES = T * 16 * 128;          // W1 stage: T x 16 units x 64 columns
};

template <int G, int H, int JC>
__global__ void __launch_bounds__(NT) gate_sink_tall_kernel(GateArgs a) {
    using C = SinkTall<G, H, (JC > 0)>;
    constexpr int P = C::P;
    constexpr int T = C::T;
    constexpr int DK = 16;
    static_assert((P - 1) * (C::LB + C::LA) <= 63, "vmcnt range");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i16 = lane & 15;
    const int q4 = lane >> 4;
    const int ngrp = a.n_kv / H;
    const int x = (int)blockIdx.x;
    const int64_t tile = (int64_t)(x / (8 * ngrp)) * 8 + (x & 7);
    const int hgrp = (x / 8) % ngrp;
    const int64_t row0 = tile * 256;
    if (row0 >= a.n_rows) return;
    const int J = JC > 0 ? JC : a.d_model / 64;
    const int64_t w1_row_bytes = (int64_t)a.d_model * 2;
    const char *w1 = (const char *)a.w1 + (int64_t)hgrp * T * 16 * w1_row_bytes;
    // every load reads whole 128-byte lines (8 rows x 128 B per instruction):
    // W1 piece i (units 8 i .. 8 i + 7) by wave i % 4, the wave's hidden rows
    // 64 wave + 8 k + lane / 8; both are written to LDS (swizzled rows) just
    // before their iteration and read back in the operand layout
    const char *wsrc = w1 + (int64_t)(lane >> 3) * w1_row_bytes + 16 * (lane & 7);
    const __bf16 *hsrc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t r = min(row0 + 64 * wave + 8 * k + (lane >> 3), a.n_rows - 1);  // rows past n re-read the last
        hsrc[k] = (const __bf16 *)a.hidden + r * a.ld_hidden + 8 * (lane & 7);
    }
    bf16x8 wraw[P][C::LB];
    auto issue_w1 = [&](int j, bf16x8 (&dst)[C::LB]) {
#pragma unroll
        for (int u = 0; u < C::LB; ++u) {
            const int i = wave + 4 * u;
            if (C::PIECES % 4 == 0 || i < C::PIECES)
                dst[u] = *(const bf16x8 *)(wsrc + (int64_t)8 * i * w1_row_bytes + 128 * j);
        }
    };
    bf16x8 hraw[P][8];
    auto issue_h = [&](int j, bf16x8 (&dst)[8]) {
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = *(const bf16x8 *)(hsrc[k] + 64 * j);
    };

    f32x4 acc[4][T];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (i < J) {
            issue_w1(i, wraw[i]);
            issue_h(i, hraw[i]);
        }
    }
#pragma unroll
    for (int j0 = 0; j0 < (JC > 0 ? JC : J); j0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int j = j0 + u;
            if (j < J) {
                wait_vm<63>(min(P - 1, J - 1 - j) * (C::LB + C::LA));
                // buffer j & 1 was last read in iteration j - 2, before every
                // wave passed the barrier of j - 1
                char *wst = stage_at<C::SBYTES, 2>(j & 1);
#pragma unroll
                for (int uu = 0; uu < C::LB; ++uu) {
                    const int i = wave + 4 * uu;
                    if (C::PIECES % 4 == 0 || i < C::PIECES) {
                        const int unit = 8 * i + (lane >> 3);
                        *(bf16x8 *)(wst + unit * 128 + (((lane & 7) ^ ((unit >> 1) & 7)) << 4)) = wraw[u][uu];
                    }
                }
                char *hst = wslice<4 * 64 * 128>(j & 1) + wave * 64 * 128;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int r = 8 * k + (lane >> 3);
                    *(bf16x8 *)(hst + r * 128 + (((lane & 7) ^ ((r >> 1) & 7)) << 4)) = hraw[u][k];
                }
                // the W1 stage of j is complete: a barrier whose fences cover
                // LDS only (__syncthreads would also wait for every load in flight)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                if (j + P < J) {
                    issue_w1(j + P, wraw[u]);
                    issue_h(j + P, hraw[u]);
                }
                bf16x8 hv[4][2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const int r = 16 * rt + i16;
                        hv[rt][ks] = *(const bf16x8 *)(hst + r * 128 + (((4 * ks + q4) ^ ((r >> 1) & 7)) << 4));
                    }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    bf16x8 wv[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        const int unit = 16 * t + i16;
                        wv[t] = *(const bf16x8 *)(wst + unit * 128 + (((4 * ks + q4) ^ ((unit >> 1) & 7)) << 4));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < T; ++t)
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt)
                            acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[t], hv[rt][ks], acc[rt][t], 0, 0, 0);
                }
            }
        }
    }

    // epilogue, per wave from its accumulators
    const int S = a.n_sinks;
    const int nst = (S + 15) / 16;  // 16-sink tiles (S <= 64)
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const int head = hgrp * H + h;
        const float *sk = a.sinks + (int64_t)head * S * DK;
        float sa[4][4];  // A operands: sink 16 st + i16, dimension 4 q4 + c
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int sj = 16 * st + i16;
                sa[st][c] = (st < nst && sj < S) ? sk[sj * DK + 4 * q4 + c] : 0.f;
            }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 kt = acc[rt][h * (G + 1) + G];
            float umax = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const f32x4 qt = acc[rt][h * (G + 1) + g];
                float own = fmaf(qt[3], kt[3], fmaf(qt[2], kt[2], fmaf(qt[1], kt[1], qt[0] * kt[0])));
                own += __shfl_xor(own, 16);
                own += __shfl_xor(own, 32);
                own *= 0.25f;
                f32x4 sc[4];
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    sc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (st < nst) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            sc[st] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[st][c], qt[c], sc[st], 0, 0, 0);
                    }
                }
                // this lane's sinks: 16 st + 4 q4 + r
                float m = own;
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * st + 4 * q4 + r < S) m = fmaxf(m, sc[st][r] * 0.25f);
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                float den = 0.f;
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * st + 4 * q4 + r < S) den += expf(sc[st][r] * 0.25f - m);
                den += __shfl_xor(den, 16);
                den += __shfl_xor(den, 32);
                const float num = expf(own - m);
                const float ug = num / (num + den);
                umax = (g == 0 || ug != ug || ug > umax) ? ug : umax;  // NaN wins
            }
            const int64_t row = row0 + 64 * wave + 16 * rt + i16;
            if (q4 == 0 && row < a.n_rows) {
                if (a.utility) a.utility[row * a.n_kv + head] = umax;
                a.keep[row * a.n_kv + head] = (umax >= a.tau) ? 1 : 0;  // NaN -> 0
            }
        }
    }
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

template <int HG>
static void launch_unitsplit(const GateArgs &a, dim3 grid, hipStream_t s) {
    if (a.d_model == 4096) hipLaunchKernelGGL((gate_unitsplit_kernel<HG, 64>), grid, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((gate_unitsplit_kernel<HG, 0>), grid, dim3(NT), 0, s, a);
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
            const bool fixed = a.d_model == 4096;
            switch (a.d_hidden) {
            case 32:
                if (fixed) hipLaunchKernelGGL((gate_pipe_kernel<32, 64>), grid, dim3(NT), 0, s, a);
                else hipLaunchKernelGGL((gate_pipe_kernel<32, 0>), grid, dim3(NT), 0, s, a);
                break;
            case 64: launch_unitsplit<64>(a, grid, s); break;
            case 128: launch_unitsplit<128>(a, grid, s); break;
            default: launch_unitsplit<256>(a, grid, s); break;
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

template <int G, int H>
static void launch_sink_tall(const GateArgs &a, hipStream_t s) {
    const int64_t tiles = (a.n_rows + 255) / 256;
    const dim3 grid((unsigned)(((tiles + 7) / 8) * 8 * (a.n_kv / H)));
    if (a.d_model == 4096)
        hipLaunchKernelGGL((gate_sink_tall_kernel<G, H, 64>), grid, dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL((gate_sink_tall_kernel<G, H, 0>), grid, dim3(NT), 0, s, a);
}

// heads per workgroup: as many as keep the projection tiles at most 10 (the
// accumulators of 4 row tiles x 10 tiles fill 160 registers) and divide n_kv
template <int G>
static void launch_sink_g(const GateArgs &a, hipStream_t s) {
    constexpr int HMAX = 10 / (G + 1);
    if (HMAX >= 4 && a.n_kv % 4 == 0) launch_sink_tall<G, (HMAX >= 4 ? 4 : 1)>(a, s);
    else if (HMAX >= 2 && a.n_kv % 2 == 0) launch_sink_tall<G, (HMAX >= 2 ? 2 : 1)>(a, s);
    else launch_sink_tall<G, 1>(a, s);
}

hipError_t launch_sink_gate(const GateArgs &a, hipStream_t s) {
    switch (a.group) {
    case 1: launch_sink_g<1>(a, s); break;
    case 2: launch_sink_g<2>(a, s); break;
    case 4: launch_sink_g<4>(a, s); break;
    default: launch_sink_g<8>(a, s); break;
    }
    return hipGetLastError();
}

}  // namespace spkv
