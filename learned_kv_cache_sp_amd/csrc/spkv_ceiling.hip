// Streaming-read kernels: what the HBM delivers to a plain read on this GPU,
// the measured ceiling that the decode kernel's bandwidth is set beside.
//
// Two access orders, each with or without the non-temporal hint:
//   stride  every thread loads 16-byte words one grid apart, four at a time
//           (consecutive lanes read consecutive words);
//   runs    every wave streams its own contiguous run of 16 KB blocks, the
//           way a decode wave walks its share of one head's pages.
// The loaded words are folded into one value per lane, stored only if it
// equals a constant that the data never produces, so the loads cannot be
// dropped; nothing else is written.
#include "spkv_internal.h"

namespace spkv {
namespace {

constexpr int RT = 256;            // threads per workgroup
constexpr int BLK_WORDS = 1024;    // 16-byte words per 16 KB block
constexpr uint32_t NEVER = 0x9e3779b9u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ inline u32x4 ld(const u32x4 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ inline uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool NT>
__global__ void __launch_bounds__(RT) read_stride_kernel(const u32x4 *__restrict__ p, uint64_t words, uint32_t *sink) {
    // four loads in flight per thread: word i, i + step, i + 2 step, i + 3 step
    const uint64_t step = (uint64_t)gridDim.x * RT;
    uint32_t acc = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * RT + threadIdx.x; i < words; i += 4 * step) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = i + u * step < words ? ld<NT>(p + i + u * step) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= fold(v[u]);
    }
    if (acc == NEVER) sink[0] = acc;
}

template <bool NT>
__global__ void __launch_bounds__(RT) read_runs_kernel(const u32x4 *__restrict__ p, uint64_t nblk, uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    const uint64_t nw = (uint64_t)gridDim.x * (RT / 64);
    // the wave index is the same on every lane: keep it (and the run bounds) in scalar registers
    const uint64_t wave = (uint64_t)blockIdx.x * (RT / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t b0 = nblk * wave / nw, b1 = nblk * (wave + 1) / nw;
    uint32_t acc = 0;
    for (uint64_t b = b0; b < b1; ++b) {
        const u32x4 *blk = p + b * BLK_WORDS + lane;
        u32x4 v[BLK_WORDS / 64];
#pragma unroll
        for (int i = 0; i < BLK_WORDS / 64; ++i) v[i] = ld<NT>(blk + 64 * i);
#pragma unroll
        for (int i = 0; i < BLK_WORDS / 64; ++i) acc ^= fold(v[i]);
    }
    if (acc == NEVER) sink[0] = acc;
}

}  // namespace

hipError_t launch_hbm_read(const void *src, size_t bytes, bool nontemporal, bool runs, uint32_t *sink, int grid,
                           hipStream_t s) {
    const u32x4 *p = (const u32x4 *)src;
    if (runs) {
        const uint64_t nblk = bytes / (BLK_WORDS * 16);
        if (nontemporal) hipLaunchKernelGGL(read_runs_kernel<true>, dim3(grid), dim3(RT), 0, s, p, nblk, sink);
        else hipLaunchKernelGGL(read_runs_kernel<false>, dim3(grid), dim3(RT), 0, s, p, nblk, sink);
    } else {
        const uint64_t words = bytes / 16;
        if (nontemporal) hipLaunchKernelGGL(read_stride_kernel<true>, dim3(grid), dim3(RT), 0, s, p, words, sink);
        else hipLaunchKernelGGL(read_stride_kernel<false>, dim3(grid), dim3(RT), 0, s, p, words, sink);
    }
    return hipGetLastError();
}

}  // namespace spkv
