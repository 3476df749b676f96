// gfx950 (CDNA4) kernels of libq4stream: Q4_0 weight repack, Q8_0 activation
// quantization, the Q4_0 x Q8_0 GEMV / skinny GEMM (n <= 8), the layer-stack
// sweep, the per-block integer-sum test hook and two measurement kernels.
//
// Method (the "minfer" README, nano-inference page): integer MACs over int8
// activations (milestone M3.5) with SIMD nibble masking instead of per-nibble
// extraction (M9), wide 16-byte loads (M10), weights repacked at load so a
// wavefront reads one contiguous span and each lane owns one output row
// (mega.cu bullet of "How it works"; M15), and one fp32 expression per block
// shared by every step size (M16).
//
// gfx950 design:
//  * lane = output row, wave = 64-row group; every wave-wide 16-byte load reads
//    1 KB contiguous of the packed layout;
//  * the activation is wave-uniform, so it is read with scalar loads into SGPRs
//    and fed to v_dot4 as the scalar operand (no LDS staging, no barrier);
//  * nibbles are stored in two's complement (canonical byte XOR 0x88), so one
//    AND gives the high nibbles and one shift+AND the low nibbles of 4 elements
//    as int8 values 16*(nibble-8): the dot yields 16*s exactly and the scale
//    absorbs the 1/16, with no per-block offset correction;
//  * a workgroup (4 waves) owns whole output rows: long rows are split over
//    its waves and added in LDS in split order, so no cross-workgroup
//    reduction, atomic or device-wide fence is needed.
#include <hip/hip_fp16.h>

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

// ---------------------------------------------------------------- loads

// The 9 x 16 bytes a lane reads per chunk: 8 blocks of nibbles, then its row's
// 8 binary16 scales.
struct Chunk {
    u32x4 nib[kChunkBlocks];
    u32x4 scale;
};

__device__ __forceinline__ void load_chunk(Chunk& ch, const uint8_t* p) {
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b)
        ch.nib[b] = __builtin_nontemporal_load(gp<u32x4>(p + b * (kGroupRows * kBlockNibBytes)));
    ch.scale = __builtin_nontemporal_load(gp<u32x4>(p + kChunkNibBytes));
}

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

// ---------------------------------------------------------------- block dot

// Unpacked int8 operands of one block: lo[k] holds elements 4k..4k+3 and hi[k]
// elements 16+4k..16+4k+3, each as 16*(nibble-8).
struct Unpacked {
    uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Unpacked unpack(u32x4 w) {
    Unpacked u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        u.lo[k] = (w[k] << 4) & 0xF0F0F0F0u;
        u.hi[k] = w[k] & 0xF0F0F0F0u;
    }
    return u;
}

// 16 * sum_j (nibble_j - 8) * q_j, exact in int32 (|.| <= 16 * 32512).
__device__ __forceinline__ int block_dot16(const Unpacked& u, const u32x8& q) {
    int s = __builtin_amdgcn_sdot4((int)u.lo[0], (int)q[0], 0, false);
    s = __builtin_amdgcn_sdot4((int)u.lo[1], (int)q[1], s, false);
    s = __builtin_amdgcn_sdot4((int)u.lo[2], (int)q[2], s, false);
    s = __builtin_amdgcn_sdot4((int)u.lo[3], (int)q[3], s, false);
    s = __builtin_amdgcn_sdot4((int)u.hi[0], (int)q[4], s, false);
    s = __builtin_amdgcn_sdot4((int)u.hi[1], (int)q[5], s, false);
    s = __builtin_amdgcn_sdot4((int)u.hi[2], (int)q[6], s, false);
    s = __builtin_amdgcn_sdot4((int)u.hi[3], (int)q[7], s, false);
    return s;
}

// ---------------------------------------------------------------- GEMV core

// Adds chunk `c` (held in ch) of the lane's row into acc[0..N).  The per-block
// term is fmaf(d_w/16 * d_x, (float)(16 s), part): the product of the two
// scales is exact, so this equals fmaf(d_w * d_x, (float)s, part) bit for bit.
// Within a chunk blocks 0-3 and blocks 4-7 form two chains that are added at
// the end; the MFMA path (two blocks per instruction) forms exactly the same
// chains.
template <int N>
__device__ __forceinline__ void chunk_fma(const MatDesc& m, int c, const Chunk& ch, float (&acc)[N]) {
    float pe[N], po[N];
#pragma unroll
    for (int t = 0; t < N; ++t) pe[t] = po[t] = 0.0f;
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b) {
        // padding blocks of the last chunk have zero nibbles and scale; read a
        // valid activation block for them
        const int blk = min(c * kChunkBlocks + b, m.nb - 1);
        const uint32_t sw = ch.scale[b >> 1];
        const float dw16 = ((b & 1) ? half_hi(sw) : half_lo(sw)) * 0.0625f;
        const Unpacked u = unpack(ch.nib[b]);
#pragma unroll
        for (int t = 0; t < N; ++t) {
            const u32x8 q = act_q(m.xq, (int64_t)t * m.cols + (int64_t)blk * 32);
            const int s16 = block_dot16(u, q);
            const float dx = act_d(m.xd, (int64_t)t * m.dstride + blk);
            float& p = (b < kChunkBlocks / 2) ? pe[t] : po[t];
            p = fmaf(dw16 * dx, (float)s16, p);
        }
    }
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] += pe[t] + po[t];
}

// One wave streams chunks [c0, c1) of row group g; lane = row.  Two chunks are
// in flight per wave: the next chunk's loads are issued before the current
// chunk is consumed.
template <int N>
__device__ __forceinline__ void wave_task(const MatDesc& m, int g, int c0, int c1, float (&acc)[N]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kChunkBytes + lane * kBlockNibBytes;
    Chunk a, b;
    load_chunk(a, wp);
    for (int c = c0; c < c1; c += 2) {
        const bool has_b = c + 1 < c1;
        if (has_b) load_chunk(b, wp + kChunkBytes);
        chunk_fma<N>(m, c, a, acc);
        if (!has_b) break;
        if (c + 2 < c1) load_chunk(a, wp + 2 * kChunkBytes);
        chunk_fma<N>(m, c + 1, b, acc);
        wp += 2 * kChunkBytes;
    }
}

// ---------------------------------------------------------------- MFMA path (n >= 2)
//
// For 2..8 activation rows the per-block dots run on the matrix cores with
// v_mfma_i32_16x16x64_i8, two Q4_0 blocks per instruction (blocks p and p+4
// of a chunk, p = 0..3): D = A x B with
//   A (16 x 64): rows 0-7 = token slots 0-7 of block p, rows 8-15 = token
//      slots 0-7 of block p+4; a row is non-zero only in its block's K half
//      (lane groups 0-1 carry block p, lane groups 2-3 block p+4);
//   B (64 x 16): 16 rows of the wave's 64-row group, K half 0 = block p,
//      K half 1 = block p+4;
// so D[slot][row] for slots 0-7 is block p's exact integer sum and slots 8-15
// block p+4's.  In D, lane (lg, j) = (lane/16, lane%16) holds row j and slots
// 4*lg + r: lanes 0-31 accumulate blocks 0-3 of a chunk, lanes 32-63 blocks
// 4-7, and the two chains are added at the end of the chunk, exactly as in
// the 1-row path, so each row's result is bit-identical to the 1-row call.
// Token slots >= n read a valid activation row and are never stored.

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Per-lane activation data of one chunk.  a[p]: the A operand of block pair
// (p, p+4): 16 bytes, q[8k..8k+7] and q[16+8k..16+8k+7] (k = lg & 1) of the
// lane's token and block, or zero where the lane's row lies outside its K
// half; dx[r]: the binary16 scales of token slot 4*(lg&1) + r for the four
// blocks 4*(lg>>1) .. 4*(lg>>1)+3 of the chunk that the lane accumulates.
struct ActChunk {
    u32x4 a[kChunkBlocks / 2];
    u32x2 dx[4];
};

template <int N>
__device__ __forceinline__ void load_act(ActChunk& a, const MatDesc& m, int c) {
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4, i = lane & 15;
    const int h = lg >> 1;
    const bool active = h == (i >> 3);
    const uint8_t* xa = (const uint8_t*)m.xq + (int64_t)min(i & 7, N - 1) * m.cols + 8 * (lg & 1);
#pragma unroll
    for (int p = 0; p < kChunkBlocks / 2; ++p) {
        const int blk = min(c * kChunkBlocks + p + 4 * h, m.nb - 1);
        const u32x2 lo = *gp<u32x2>(xa + (int64_t)blk * 32);
        const u32x2 hi = *gp<u32x2>(xa + (int64_t)blk * 32 + 16);
        const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
        const u32x4 z = {0u, 0u, 0u, 0u};
        a.a[p] = active ? v : z;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = min(4 * (lg & 1) + r, N - 1);
        // d_x rows are padded to a multiple of 8 entries (zero past the last
        // block), so this aligned 8-byte load stays inside row t
        a.dx[r] = *gp<u32x2>(m.xd + (int64_t)t * m.dstride + c * kChunkBlocks + 4 * h);
    }
}

template <int N>
__device__ __forceinline__ void chunk_mfma(Chunk& ch, const ActChunk& a, float (&acc)[16], u32x4* lds_sc) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, h = lane >> 5;
    // the scales of rows 16*mt + j for the lane's four blocks, exchanged
    // through the wave's own LDS slot
    lds_sc[lane] = ch.scale;
    u32x2 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sc[mt] = *((const u32x2*)&lds_sc[16 * mt + j] + h);
    float part[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) part[k] = 0.0f;
#pragma unroll
    for (int p = 0; p < kChunkBlocks / 2; ++p) {
        // B operands: lane (g, j) gets dwords 2(g&1), 2(g&1)+1 of block p + 4(g>>1)
        // of row 16*mt + j, for the 4 row tiles mt
        uint32_t e[4] = {ch.nib[p][0], ch.nib[p][2], ch.nib[p + 4][0], ch.nib[p + 4][2]};
        uint32_t o[4] = {ch.nib[p][1], ch.nib[p][3], ch.nib[p + 4][1], ch.nib[p + 4][3]};
        xpose4x4(e);
        xpose4x4(o);
        const i32x4 aop = (i32x4)a.a[p];
        const i32x4 zero = {0, 0, 0, 0};
        i32x4 d[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const i32x4 bop = {(int)((e[mt] << 4) & 0xF0F0F0F0u), (int)((o[mt] << 4) & 0xF0F0F0F0u),
                               (int)(e[mt] & 0xF0F0F0F0u), (int)(o[mt] & 0xF0F0F0F0u)};
            d[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, zero, 0, 0, 0);
        }
        float dx16[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dx16[r] = ((p & 1) ? half_hi(a.dx[r][p >> 1]) : half_lo(a.dx[r][p >> 1])) * 0.0625f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float dw = (p & 1) ? half_hi(sc[mt][p >> 1]) : half_lo(sc[mt][p >> 1]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[mt * 4 + r] = fmaf(dw * dx16[r], (float)d[mt][r], part[mt * 4 + r]);
        }
    }
    // chains of blocks 0-3 live in lanes 0-31, of blocks 4-7 in lanes 32-63
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[k]), __float_as_uint(part[k]), false, false);
        acc[k] += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
}

// acc[mt*4 + r] = y[token 4*(lg&1) + r][row g*64 + 16*mt + j]
template <int N>
__device__ __forceinline__ void wave_task_mfma(const MatDesc& m, int g, int c0, int c1, float (&acc)[16],
                                               u32x4* lds_sc) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kChunkBytes + lane * kBlockNibBytes;
    Chunk wa, wb;
    ActChunk aa, ab;
    load_chunk(wa, wp);
    load_act<N>(aa, m, c0);
    for (int c = c0; c < c1; c += 2) {
        const bool has_b = c + 1 < c1;
        if (has_b) {
            load_chunk(wb, wp + kChunkBytes);
            load_act<N>(ab, m, c + 1);
        }
        chunk_mfma<N>(wa, aa, acc, lds_sc);
        if (!has_b) break;
        if (c + 2 < c1) {
            load_chunk(wa, wp + 2 * kChunkBytes);
            load_act<N>(aa, m, c + 2);
        }
        chunk_mfma<N>(wb, ab, acc, lds_sc);
        wp += 2 * kChunkBytes;
    }
}

template <int N>
__device__ __forceinline__ void run_tile_mfma(const MatDesc& m, int64_t gset, float* red, u32x4* lds_sc) {
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
    wave_task_mfma<N>(m, (int)g, c0, c1, acc, lds_sc + wave * 64);
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
            if (tok < N && row < m.rows) gwr<float>(m.y)[(int64_t)tok * m.rows + row] = acc[mt * 4 + r];
        }
    }
}

// One workgroup tile: kWaves / ks row groups, ks waves per group.
template <int N>
__device__ __forceinline__ void run_tile(const MatDesc& m, int64_t gset, float* red) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ks = m.ks;
    const int gpw = kWaves / ks;
    const int64_t g = gset * gpw + wave / ks;
    const int s = wave % ks;
    const int c0 = (int)((int64_t)s * m.C / ks);
    const int c1 = (int)((int64_t)(s + 1) * m.C / ks);
    float acc[N];
    wave_task<N>(m, (int)g, c0, c1, acc);
    const int64_t row = g * kGroupRows + lane;
    if (ks == 1) {
        if (g < m.G && row < m.rows) {
#pragma unroll
            for (int t = 0; t < N; ++t) gwr<float>(m.y)[(int64_t)t * m.rows + row] = acc[t];
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
            gwr<float>(m.y)[(int64_t)t * m.rows + row] = v;
        }
    }
}

// Per-workgroup LDS of the GEMV kernels: the split reduction buffer and, for
// the MFMA path, one 1 KB scale-exchange slot per wave.
template <int N>
struct TileLds {
    float red[kWaves * (N == 1 ? 1 : 16) * 64];
    u32x4 sc[N == 1 ? 1 : kWaves * 64];
};

template <int N>
__device__ __forceinline__ void run_any(const MatDesc& m, int64_t gset, TileLds<N>& l) {
    if constexpr (N == 1)
        run_tile<1>(m, gset, l.red);
    else
        run_tile_mfma<N>(m, gset, l.red, l.sc);
}

template <int N>
__global__ __launch_bounds__(kThreads) void k_gemv(MatDesc m) {
    __shared__ TileLds<N> l;
    run_any<N>(m, blockIdx.x, l);
}

// The sweep: workgroup i takes tile i = (matrix, group set) of a table sorted
// by tile size, largest first, so the hardware dispatcher's in-order
// assignment to free slots is a longest-first list schedule.
template <int N>
__global__ __launch_bounds__(kThreads) void k_sweep(const MatDesc* __restrict__ mats,
                                                    const uint32_t* __restrict__ tiles) {
    __shared__ TileLds<N> l;
    const uint32_t mi = tiles[2 * (size_t)blockIdx.x];
    const uint32_t gs = tiles[2 * (size_t)blockIdx.x + 1];
    const MatDesc m = mats[mi];
    run_any<N>(m, gs, l);
}

// Test hook: the exact per-block sums, from the same loads, unpack and dot.
template <int N>
__global__ __launch_bounds__(kThreads) void k_block_sums(MatDesc m, int32_t* __restrict__ s) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    if (g >= m.G) return;
    const int64_t row = g * kGroupRows + lane;
    const uint8_t* wp = m.w + (size_t)g * m.C * kChunkBytes + lane * kBlockNibBytes;
    for (int c = 0; c < m.C; ++c, wp += kChunkBytes) {
        Chunk ch;
        load_chunk(ch, wp);
#pragma unroll
        for (int b = 0; b < kChunkBlocks; ++b) {
            const int blk = c * kChunkBlocks + b;
            if (blk >= m.nb) break;
            const Unpacked u = unpack(ch.nib[b]);
#pragma unroll
            for (int t = 0; t < N; ++t) {
                const int s16 = block_dot16(u, act_q(m.xq, (int64_t)t * m.cols + (int64_t)blk * 32));
                if (row < m.rows) s[((int64_t)t * m.rows + row) * m.nb + blk] = s16 >> 4;
            }
        }
    }
}

// ---------------------------------------------------------------- repack

// One thread per (group, chunk, block, row): writes the row's 16 nibble bytes
// (XOR 0x88) and its binary16 scale into the packed layout; padding is zero.
__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ w, uint8_t* __restrict__ out,
                                                int64_t rows, int32_t nb, int32_t C, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int r = (int)(idx & 63);
    const int b = (int)((idx >> 6) & 7);
    const int64_t gc = idx >> 9;  // g * C + c
    const int64_t g = gc / C;
    const int c = (int)(gc - g * C);
    const int64_t row = g * kGroupRows + r;
    const int64_t blk = (int64_t)c * kChunkBlocks + b;
    u32x4 nib = {0u, 0u, 0u, 0u};
    uint16_t d = 0;
    if (row < rows && blk < nb) {
        const uint16_t* src = (const uint16_t*)(w + (row * nb + blk) * 18);  // 2-byte aligned
        d = src[0];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            nib[k] = ((uint32_t)src[1 + 2 * k] | ((uint32_t)src[2 + 2 * k] << 16)) ^ 0x88888888u;
    }
    uint8_t* base = out + gc * kChunkBytes;
    *(u32x4*)(base + b * (kGroupRows * kBlockNibBytes) + r * kBlockNibBytes) = nib;
    *(uint16_t*)(base + kChunkNibBytes + r * (kChunkBlocks * 2) + b * 2) = d;
}

// ---------------------------------------------------------------- quantize

// 32 consecutive lanes quantize one block: d = max|x| / 127 (correctly rounded
// fp32 division), q = roundf(x / d) (half away from zero), d_x = binary16(d)
// rounded to nearest even.  All-zero blocks give d = 0, q = 0.
__device__ __forceinline__ void quant_block(const float* x, int8_t* q, uint16_t* d) {
    const int l = threadIdx.x & 31;
    const float v = x[l];
    float a = fabsf(v);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 32));
    const float dd = a / 127.0f;
    int qi = 0;
    if (a != 0.0f) qi = (int)roundf(v / dd);
    q[l] = (int8_t)qi;
    if (l == 0) *d = __half_as_ushort(__float2half_rn(dd));
}

__device__ __forceinline__ void quant_local(const QuantDesc& qd, int64_t lb) {
    const int nb = qd.cols / 32;
    const int64_t t = lb / nb;
    const int64_t b = lb - t * nb;
    const int64_t off = t * qd.cols + b * 32;
    quant_block(qd.x + off, qd.q + off, qd.d + t * qd.dstride + b);
    // the half-wave of a row's last block zeroes the row's padding entries
    const int l = threadIdx.x & 31;
    if (b == nb - 1 && l < qd.dstride - nb) qd.d[t * qd.dstride + nb + l] = 0;
}

__global__ __launch_bounds__(256) void k_quantize(QuantDesc qd, int64_t total_blocks) {
    const int64_t gb = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
    if (gb >= total_blocks) return;  // uniform per 32-lane half
    quant_local(qd, gb);
}

// Batched quantization for the sweep: workgroup i takes tile i = (activation,
// first block) of a host-built table and quantizes up to kQuantTileBlocks
// consecutive blocks of that activation (each 32-lane half-wave takes every
// 8th block), so no thread searches for its activation.
__global__ __launch_bounds__(256) void k_quantize_batch(const QuantDesc* __restrict__ descs,
                                                        const uint32_t* __restrict__ tiles) {
    const uint32_t di = tiles[2 * (size_t)blockIdx.x];
    const uint32_t b0 = tiles[2 * (size_t)blockIdx.x + 1];
    const QuantDesc qd = descs[di];
    const int64_t total = (int64_t)qd.n * (qd.cols / 32);
    const int64_t end = min((int64_t)b0 + kQuantTileBlocks, total);
    for (int64_t lb = (int64_t)b0 + (threadIdx.x >> 5); lb < end; lb += 8)  // uniform per half-wave
        quant_local(qd, lb);
}

// ---------------------------------------------------------------- measurement

template <int L>
__global__ __launch_bounds__(256) void k_bench_read(const u32x4* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (L - 1) * stride < n16; i += L * stride) {
        u32x4 v[L];
#pragma unroll
        for (int k = 0; k < L; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
        for (int k = 0; k < L; ++k) acc ^= v[k];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
    const uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (h == 0x9E3779B9u && acc.x == 0x7F4A7C15u) sink[0] = h;  // practically never
}

__global__ __launch_bounds__(256) void k_bench_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_repack(const uint8_t* w, uint8_t* packed, int64_t rows, int64_t cols, hipStream_t st) {
    const int64_t G = groups_of(rows), C = chunks_of(cols);
    const int64_t total = G * C * kChunkBlocks * kGroupRows;
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(k_repack, dim3((unsigned)grid), dim3(256), 0, st, w, packed, rows,
                       (int32_t)(cols / 32), (int32_t)C, total);
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantDesc& d, hipStream_t st) {
    const int64_t total = (int64_t)d.n * (d.cols / 32);
    if (total == 0) return hipSuccess;
    const int64_t grid = (total * 32 + 255) / 256;
    hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(256), 0, st, d, total);
    return hipGetLastError();
}

hipError_t launch_quantize_batch(const QuantDesc* dev_descs, const uint32_t* dev_tiles, int64_t n_tiles,
                                 hipStream_t st) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize_batch, dim3((unsigned)n_tiles), dim3(256), 0, st, dev_descs, dev_tiles);
    return hipGetLastError();
}

template <int N>
static void gemv_n(const MatDesc& m, int64_t n_gsets, hipStream_t st) {
    hipLaunchKernelGGL(k_gemv<N>, dim3((unsigned)n_gsets), dim3(kThreads), 0, st, m);
}

hipError_t launch_gemv(const MatDesc& m, int n, int64_t n_gsets, hipStream_t st) {
    if (n_gsets == 0 || n == 0) return hipSuccess;
    switch (n) {
        case 1: gemv_n<1>(m, n_gsets, st); break;
        case 2: gemv_n<2>(m, n_gsets, st); break;
        case 3: gemv_n<3>(m, n_gsets, st); break;
        case 4: gemv_n<4>(m, n_gsets, st); break;
        case 5: gemv_n<5>(m, n_gsets, st); break;
        case 6: gemv_n<6>(m, n_gsets, st); break;
        case 7: gemv_n<7>(m, n_gsets, st); break;
        case 8: gemv_n<8>(m, n_gsets, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int N>
static void sweep_n(const MatDesc* mats, const uint32_t* tiles, int64_t n_tiles, hipStream_t st) {
    hipLaunchKernelGGL(k_sweep<N>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, mats, tiles);
}

hipError_t launch_sweep(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles, int n,
                        hipStream_t st) {
    if (n_tiles == 0 || n == 0) return hipSuccess;
    switch (n) {
        case 1: sweep_n<1>(dev_mats, dev_tiles, n_tiles, st); break;
        case 2: sweep_n<2>(dev_mats, dev_tiles, n_tiles, st); break;
        case 3: sweep_n<3>(dev_mats, dev_tiles, n_tiles, st); break;
        case 4: sweep_n<4>(dev_mats, dev_tiles, n_tiles, st); break;
        case 5: sweep_n<5>(dev_mats, dev_tiles, n_tiles, st); break;
        case 6: sweep_n<6>(dev_mats, dev_tiles, n_tiles, st); break;
        case 7: sweep_n<7>(dev_mats, dev_tiles, n_tiles, st); break;
        case 8: sweep_n<8>(dev_mats, dev_tiles, n_tiles, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int N>
static void sums_n(const MatDesc& m, int32_t* s, hipStream_t st) {
    const int64_t grid = (m.G + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_block_sums<N>, dim3((unsigned)grid), dim3(kThreads), 0, st, m, s);
}

hipError_t launch_block_sums(const MatDesc& m, int n, int32_t* s, hipStream_t st) {
    if (m.G == 0 || n == 0 || m.nb == 0) return hipSuccess;
    switch (n) {
        case 1: sums_n<1>(m, s, st); break;
        case 2: sums_n<2>(m, s, st); break;
        case 3: sums_n<3>(m, s, st); break;
        case 4: sums_n<4>(m, s, st); break;
        case 5: sums_n<5>(m, s, st); break;
        case 6: sums_n<6>(m, s, st); break;
        case 7: sums_n<7>(m, s, st); break;
        case 8: sums_n<8>(m, s, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bench_read(const void* buf, size_t bytes, int lif, int n_blocks, uint32_t* sink,
                             hipStream_t st) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    if (n_blocks <= 0) n_blocks = 256 * 8;
    const u32x4* p = (const u32x4*)buf;
    switch (lif) {
        case 1: hipLaunchKernelGGL(k_bench_read<1>, dim3(n_blocks), dim3(256), 0, st, p, n16, sink); break;
        case 2: hipLaunchKernelGGL(k_bench_read<2>, dim3(n_blocks), dim3(256), 0, st, p, n16, sink); break;
        case 4: hipLaunchKernelGGL(k_bench_read<4>, dim3(n_blocks), dim3(256), 0, st, p, n16, sink); break;
        case 8: hipLaunchKernelGGL(k_bench_read<8>, dim3(n_blocks), dim3(256), 0, st, p, n16, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const int64_t grid = std::min<int64_t>((n16 + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(k_bench_copy, dim3((unsigned)grid), dim3(256), 0, st, (const u32x4*)src,
                       (u32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace q4s
