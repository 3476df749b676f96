// Device helpers shared by the gfx950 kernels of libq4stream (Q4_0 and Q8_0
// weight paths): typed global/constant loads, the activation loads, the
// cross-lane-group transpose used to build MFMA operands, and the
// per-workgroup LDS of the GEMV tiles.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "q4s_internal.h"

namespace q4s {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef u32x8 u32x8_a4 __attribute__((aligned(4)));
#define Q4S_CONST __attribute__((address_space(4)))
#define Q4S_GLOBAL __attribute__((address_space(1)))

// Pointers taken from a descriptor table are generic to the compiler; casting
// them to the global address space keeps the streaming loads global_load_*
// (a flat load would also count against the scalar-load wait counter).
template <class T>
__device__ __forceinline__ const Q4S_GLOBAL T* gp(const void* p) { return (const Q4S_GLOBAL T*)p; }
template <class T>
__device__ __forceinline__ Q4S_GLOBAL T* gwr(void* p) { return (Q4S_GLOBAL T*)p; }

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 32 int8 activation values of one block, wave-uniform -> SGPRs.
__device__ __forceinline__ u32x8 act_q(const int8_t* xq, int64_t off) {
    return *(const Q4S_CONST u32x8_a4*)(xq + off);
}

// binary16 activation scale idx, wave-uniform (dword scalar load; d_x rows are
// padded to a multiple of 8 entries, so the containing dword is in bounds).
__device__ __forceinline__ float act_d(const uint16_t* xd, int64_t idx) {
    const uint32_t v = *(const Q4S_CONST uint32_t*)(xd + (idx & ~(int64_t)1));
    const uint16_t h = (idx & 1) ? (uint16_t)(v >> 16) : (uint16_t)(v & 0xffffu);
    return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ float half_lo(uint32_t v) { return __half2float(__ushort_as_half((uint16_t)(v & 0xffffu))); }
__device__ __forceinline__ float half_hi(uint32_t v) { return __half2float(__ushort_as_half((uint16_t)(v >> 16))); }

// Segment length (in chunks) of the summation order shared by every path.
constexpr int kSegChunks = 16;


typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 4x4 dword transpose across the four 16-lane groups: on entry lane (m, j)
// holds v[0..3]; on exit lane (g, j) holds in v[m] what lane (m, j) held in v[g].
__device__ __forceinline__ void xpose4x4(uint32_t (&v)[4]) {
    auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    v[0] = a[0];
    v[2] = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    v[1] = b[0];
    v[3] = b[1];
    auto c = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    auto d = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
    v[2] = d[0];
    v[3] = d[1];
}

// A wave's LDS slice.  q: per (token t, block b, K half h) 16 bytes at
// ((t*8 + b)*2 + h)*16: q[8h..8h+7] then q[16+8h..16+8h+7]; then 16 zero bytes
// (the A operand of lanes outside their K half).  dx: d_x/16 [token][block]
// fp32.  dw: d_w [row][block] fp32 of the wave's 64 rows.
struct WaveLds {
    u32x4 q[8 * kChunkBlocks * 2 + 1];        // 16-byte slots; the last one stays zero
    f32x4 dx[8 * kChunkBlocks / 4];
    f32x4 dw[kGroupRows * kChunkBlocks / 4];
};
constexpr int kZeroSlot = 8 * kChunkBlocks * 2;

// The raw activation data of one chunk as loaded: lane (r4, j) holds bytes
// 16*(j&1) .. +15 of block j>>1 for tokens r4 and 4 + r4 (r4 = lane/16), and
// the binary16 d_x of token lane/8, block lane%8.
struct ActRaw {
    u32x4 q0, q1;
    uint32_t dxh;
};

template <int N>
__device__ __forceinline__ void load_act(ActRaw& a, const MatDesc& m, int c) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;
    const int blk = min(c * kChunkBlocks + (j >> 1), m.nb - 1);  // valid block for padding pieces
    const int64_t off = (int64_t)blk * 32 + (j & 1) * 16;
    const int last = min(N, m.n) - 1;  // token slots past the rows repeat the last row
    a.q0 = *gp<u32x4>(m.xq + (int64_t)min(lane >> 4, last) * m.cols + off);
    a.q1 = *gp<u32x4>(m.xq + (int64_t)min(4 + (lane >> 4), last) * m.cols + off);
    // d_x rows are padded to a multiple of 8 entries (zero past the last block)
    a.dxh = *gp<uint16_t>(m.xd + (int64_t)min(lane >> 3, last) * m.dstride + c * kChunkBlocks + (lane & 7));
}

// Per-workgroup LDS of the GEMV kernels: the split reduction buffer and, for
// the MFMA path, one 1 KB scale-exchange slot per wave.
template <int N>
struct TileLds {
    float red[kWaves * (N == 1 ? 1 : 16) * 64];
    WaveLds wl[N == 1 ? 1 : kWaves];
};

// Outputs are written with non-temporal stores: written into a saturated
// weight stream, y cost less that way (7B step at 1 row 595 -> 588 us, at 8
// rows 672 -> 655 us).  The 1-row split tiles keep plain stores, where the
// hint made no difference.
//
// One workgroup tile of a matrix-core path: kWaves / ks row groups, ks waves
// per group; task(g, c0, c1, acc, lds) runs one wave's chunk range and leaves
// acc[mt*4 + r] = y[token 4*(lane/16 & 1) + r][row g*64 + 16*mt + lane%16].
template <int N, class Task>
__device__ __forceinline__ void run_tile_mfma_with(const MatDesc& m, int64_t gset, float* red, WaveLds* wl,
                                                   Task&& task) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4, j = lane & 15;
    const int ks = m.ks;
    const int gpw = kWaves / ks;
    const int64_t g = gset * gpw + wave / ks;
    const int s = wave % ks;
    const int c0 = (int)((int64_t)s * m.C / ks);
    const int c1 = (int)((int64_t)(s + 1) * m.C / ks);
    float acc[16];
    task((int)g, c0, c1, acc, wl[wave]);
    if (ks > 1) {
#pragma unroll
        for (int k = 0; k < 16; ++k) red[(wave * 16 + k) * 64 + lane] = acc[k];
        __syncthreads();
        if (s != 0) return;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float v = red[(wave * 16 + k) * 64 + lane];
            for (int q = 1; q < ks; ++q) v += red[((wave + q) * 16 + k) * 64 + lane];
            acc[k] = v;
        }
    }
    if (g >= m.G || lg >= 2) return;  // lanes 32-63 hold the same sums as lanes 0-31
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int64_t row = g * kGroupRows + 16 * mt + j;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = 4 * lg + r;
            if (tok < min(N, m.n) && row < m.rows)
                __builtin_nontemporal_store(acc[mt * 4 + r], gwr<float>(m.y) + (int64_t)tok * m.rows + row);
        }
    }
}

// One workgroup tile of a lane-per-row path: kWaves / ks row groups, ks waves
// per group; task(g, c0, c1, acc) runs one wave's chunk range of row g*64 + lane.
template <int N, class Task>
__device__ __forceinline__ void run_tile_with(const MatDesc& m, int64_t gset, float* red, Task&& task) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ks = m.ks;
    const int gpw = kWaves / ks;
    const int64_t g = gset * gpw + wave / ks;
    const int s = wave % ks;
    const int c0 = (int)((int64_t)s * m.C / ks);
    const int c1 = (int)((int64_t)(s + 1) * m.C / ks);
    float acc[N];
    task((int)g, c0, c1, acc);
    const int64_t row = g * kGroupRows + lane;
    if (ks == 1) {
        if (g < m.G && row < m.rows) {
#pragma unroll
            for (int t = 0; t < N; ++t)
                __builtin_nontemporal_store(acc[t], gwr<float>(m.y) + (int64_t)t * m.rows + row);
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < N; ++t) red[(wave * N + t) * 64 + lane] = acc[t];
    __syncthreads();
    if (s == 0 && g < m.G && row < m.rows) {
#pragma unroll
        for (int t = 0; t < N; ++t) {
            float v = red[(wave * N + t) * 64 + lane];
            for (int j = 1; j < ks; ++j) v += red[((wave + j) * N + t) * 64 + lane];
            __builtin_nontemporal_store(v, gwr<float>(m.y) + (int64_t)t * m.rows + row);
        }
    }
}

}  // namespace
}  // namespace q4s
