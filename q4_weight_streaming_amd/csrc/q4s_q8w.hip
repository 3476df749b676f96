// gfx950 kernels for Q8_0 weights (the 8-bit output head): repack, the
// Q8_0 x Q8_0 GEMV / skinny GEMM (n <= 8), its per-block integer-sum test
// hook, and the load-time Q8_0 -> Q4_0 requantization.
//
// Method (the "minfer" README, nano-inference page): the int8 lm_head of
// milestone M6, whose Q8_0 weights sit in a linear layout that a coalesced
// int8 GEMV streams against the same Q8_0 activation as the Q4_0 layers
// (gemv_q8_dp4a bullet of "How it works"), and the requantization of 8-bit
// heads to Q4_0 at load (milestones M14 and M18).
//
// Layout and schedule follow the Q4_0 kernels: lane = output row, wave =
// 64-row group, 8-block chunks (each stored as two 4-block pieces), the same
// K splits and 16-chunk segments.  The per-block sum needs no unpacking: the
// 32 int8 weights of a lane's row meet the wave-uniform activation in 8
// v_dot4 steps.  Chain A takes the even blocks of a chunk and chain B the odd
// ones, so the matrix-core path can pair blocks 2i and 2i+1 of one piece.
#include "q4s_lane.h"

namespace q4s {
namespace {

// The 8 x 16 + 8 bytes a lane reads per piece: [block][half] int8 values of
// its row, then the row's 4 binary16 scales.
struct Piece {
    u32x4 q[2 * kQ8PieceBlocks];
    u32x2 scale;
};

// p: start of the piece in the packed matrix
__device__ __forceinline__ void load_piece(Piece& pc, const uint8_t* p, int lane) {
#pragma unroll
    for (int k = 0; k < 2 * kQ8PieceBlocks; ++k)
        pc.q[k] = __builtin_nontemporal_load(gp<u32x4>(p + (k * kGroupRows + lane) * 16));
    pc.scale = __builtin_nontemporal_load(gp<u32x2>(p + kQ8PieceQBytes + lane * 8));
}

// sum_j w_j * q_j over one block, exact in int32 (|.| <= 32 * 128 * 127)
__device__ __forceinline__ int block_dot_q8(const u32x4& lo, const u32x4& hi, const u32x8& q) {
    int s = __builtin_amdgcn_sdot4((int)lo[0], (int)q[0], 0, false);
    s = __builtin_amdgcn_sdot4((int)lo[1], (int)q[1], s, false);
    s = __builtin_amdgcn_sdot4((int)lo[2], (int)q[2], s, false);
    s = __builtin_amdgcn_sdot4((int)lo[3], (int)q[3], s, false);
    s = __builtin_amdgcn_sdot4((int)hi[0], (int)q[4], s, false);
    s = __builtin_amdgcn_sdot4((int)hi[1], (int)q[5], s, false);
    s = __builtin_amdgcn_sdot4((int)hi[2], (int)q[6], s, false);
    s = __builtin_amdgcn_sdot4((int)hi[3], (int)q[7], s, false);
    return s;
}

// Adds piece k of chunk c into the chains: block 4k + b goes to chain A when
// it is even, to chain B when it is odd; term fmaf(d_w * d_x, (float)s, .).
template <int N>
__device__ __forceinline__ void piece_fma(const MatDesc& m, int c, int k, const Piece& pc, float (&pa)[N],
                                          float (&pb)[N]) {
#pragma unroll
    for (int b = 0; b < kQ8PieceBlocks; ++b) {
        // padding blocks of the last chunk have zero weights and scale; read a
        // valid activation block for them
        const int blk = min(c * kChunkBlocks + k * kQ8PieceBlocks + b, m.nb - 1);
        const uint32_t sw = pc.scale[b >> 1];
        const float dw = (b & 1) ? half_hi(sw) : half_lo(sw);
#pragma unroll
        for (int t = 0; t < N; ++t) {
            const u32x8 q = act_q(m.xq, (int64_t)t * m.cols + (int64_t)blk * 32);
            const int s = block_dot_q8(pc.q[2 * b], pc.q[2 * b + 1], q);
            const float dx = act_d(m.xd, (int64_t)t * m.dstride + blk);
            float& p = (b & 1) ? pb[t] : pa[t];
            p = fmaf(dw * dx, (float)s, p);
        }
    }
}

// One wave streams chunks [c0, c1) of row group g; lane = row.  The next
// piece's loads are issued before the current piece is consumed; the steady
// state prefetches unconditionally (see the Q4_0 path) and the last chunk is
// peeled.
template <int N>
__device__ __forceinline__ void wave_task_q8(const MatDesc& m, int g, int c0, int c1, float (&acc)[N]) {
    const int lane = threadIdx.x & 63;
    float pa[N], pb[N];
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = pa[t] = pb[t] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kQ8ChunkBytes;
    auto seg_end = [&](int c) {  // after chunk c: close the segment if it ends here
        if (c + 1 == c1 || (c + 1 - c0) % kSegChunks == 0) {
#pragma unroll
            for (int t = 0; t < N; ++t) {
                acc[t] += pa[t] + pb[t];
                pa[t] = pb[t] = 0.0f;
            }
        }
    };
    Piece a, b;
    load_piece(a, wp, lane);
    int c = c0;
    for (; c + 1 < c1; ++c, wp += kQ8ChunkBytes) {
        load_piece(b, wp + kQ8PieceBytes, lane);
        piece_fma<N>(m, c, 0, a, pa, pb);
        load_piece(a, wp + kQ8ChunkBytes, lane);
        piece_fma<N>(m, c, 1, b, pa, pb);
        seg_end(c);
    }
    load_piece(b, wp + kQ8PieceBytes, lane);
    piece_fma<N>(m, c, 0, a, pa, pb);
    piece_fma<N>(m, c, 1, b, pa, pb);
    seg_end(c);
}

// ---------------------------------------------------------------- MFMA path (n >= 2)
//
// v_mfma_i32_16x16x64_i8 on blocks 2i and 2i+1 of a piece (pair i = 0, 1):
//   A (16 x 64): rows 0-7 = token slots 0-7 of block 2i, rows 8-15 = token
//      slots of block 2i+1; a row is non-zero only in its block's K half
//      (lane groups 0-1 carry block 2i, lane groups 2-3 block 2i+1);
//   B (64 x 16): 16 rows of the wave's group; lane group g holds half g&1 of
//      block 2i + (g>>1), the 16 bytes lane (g, j) of a 4x4 transpose gathers
//      from the lane that owns the row;
// so in D, lanes 0-31 hold even-block sums (chain A) and lanes 32-63
// odd-block sums (chain B), each row's chains formed in the same order as in
// the 1-row path.  The activation is staged per chunk in the wave's LDS slice
// (slot ((t*8 + b)*2 + h) = bytes 16h..16h+15 of block b of token t).

__device__ __forceinline__ void stage_act_q8(const ActRaw& a, WaveLds& L) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, b = j >> 1, e = j & 1;
    L.q[((lane >> 4) * 8 + b) * 2 + e] = a.q0;
    L.q[((4 + (lane >> 4)) * 8 + b) * 2 + e] = a.q1;
    // d_x of token lane/8, block bl = lane%8, stored at [token][piece][bl&1][(bl>>1)&1]
    // so a lane reads its two blocks 2i + h (i = 0, 1) of a piece as one pair
    const int bl = lane & 7;
    const int pos = (lane & ~7) | (bl & 4) | ((bl & 1) << 1) | ((bl >> 1) & 1);
    ((float*)L.dx)[pos] = __half2float(__ushort_as_half((uint16_t)a.dxh));
}

template <int N>
__device__ __forceinline__ void piece_mfma(const Piece& pc, int k, float (&part)[16], WaveLds& L, int abase,
                                           int astep) {
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4, j = lane & 15, h = lane >> 5;
    // the lane's row scales as fp32, stored [row][h][i] for blocks 2i + h
    {
        const f32x4 v = {half_lo(pc.scale[0]), half_lo(pc.scale[1]), half_hi(pc.scale[0]), half_hi(pc.scale[1])};
        L.dw[lane] = v;
    }
    f32x2 dw[4], dx[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dw[mt] = ((const f32x2*)L.dw)[(16 * mt + j) * 2 + h];
#pragma unroll
    for (int r = 0; r < 4; ++r) dx[r] = ((const f32x2*)L.dx)[(4 * (lg & 1) + r) * 4 + 2 * k + h];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t v[4][4];  // [dword][source item]: items are (block 2i, half 0/1), (block 2i+1, half 0/1)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int it = 0; it < 4; ++it) v[w][it] = pc.q[4 * i + it][w];
            xpose4x4(v[w]);
        }
        const i32x4 aop = (i32x4)L.q[abase + (2 * k + i) * astep];
        const i32x4 zero = {0, 0, 0, 0};
        i32x4 d[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const i32x4 bop = {(int)v[0][mt], (int)v[1][mt], (int)v[2][mt], (int)v[3][mt]};
            d[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, zero, 0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[mt * 4 + r] = fmaf(dw[mt][i] * dx[r][i], (float)d[mt][r], part[mt * 4 + r]);
    }
}

template <int N>
__device__ __forceinline__ void wave_task_mfma_q8(const MatDesc& m, int g, int c0, int c1, float (&acc)[16],
                                                  WaveLds& L) {
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4, j = lane & 15, h = lane >> 5;
    float part[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = part[k] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    if (lane == 0) L.q[kZeroSlot] = (u32x4){0u, 0u, 0u, 0u};
    // A operand of lane (lg, j): token slot j, half lg&1 of block 2i + h of pair
    // i; zero unless the slot's block half (j >> 3) is the lane's (h)
    const bool active = h == (j >> 3);
    const int abase = active ? ((j & 7) * 8 + h) * 2 + (lg & 1) : kZeroSlot;
    const int astep = active ? 4 : 0;
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kQ8ChunkBytes;
    auto seg_end = [&](int c) {
        if (c + 1 == c1 || (c + 1 - c0) % kSegChunks == 0) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[k]), __float_as_uint(part[k]),
                                                           false, false);
                acc[k] += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                part[k] = 0.0f;
            }
        }
    };
    Piece a, b;
    ActRaw ar;
    load_piece(a, wp, lane);
    load_act<N>(ar, m, c0);
    int c = c0;
    for (; c + 1 < c1; ++c, wp += kQ8ChunkBytes) {
        load_piece(b, wp + kQ8PieceBytes, lane);
        stage_act_q8(ar, L);
        piece_mfma<N>(a, 0, part, L, abase, astep);
        load_piece(a, wp + kQ8ChunkBytes, lane);
        load_act<N>(ar, m, c + 1);
        piece_mfma<N>(b, 1, part, L, abase, astep);
        seg_end(c);
    }
    load_piece(b, wp + kQ8PieceBytes, lane);
    stage_act_q8(ar, L);
    piece_mfma<N>(a, 0, part, L, abase, astep);
    piece_mfma<N>(b, 1, part, L, abase, astep);
    seg_end(c);
}

template <int N>
__global__ __launch_bounds__(kThreads, N == 1 ? 1 : 2) void k_gemv_q8(MatDesc m) {
    __shared__ TileLds<N> l;
    if constexpr (N == 1)
        run_tile_with<1>(m, blockIdx.x, l.red,
                         [&](int g, int c0, int c1, float (&acc)[1]) { wave_task_q8<1>(m, g, c0, c1, acc); });
    else
        run_tile_mfma_with<N>(m, blockIdx.x, l.red, l.wl, [&](int g, int c0, int c1, float (&acc)[16], WaveLds& L) {
            wave_task_mfma_q8<N>(m, g, c0, c1, acc, L);
        });
}

// ---------------------------------------------------------------- 1-row split tiles
//
// A 1-row GEMV of a Q8_0 matrix with one K split (C <= 8 chunks), as the Q4_0
// split tiles: each 64-row group gets an 8-wave workgroup, wave w the chunks
// [ceil(wC/8), ceil((w+1)C/8)) -- one at most, both pieces loaded at once --
// whose exact block sums (int32) and binary16 d_w go to LDS, with the chunk's
// d_x when the wave quantized the activation itself (kFused: the sweep's
// in-wave quantizer, codes to every lane by lane swaps and DPP dot operands;
// 8-bit weights need no unpack, so the 32 raw int8 weights of a block meet the
// codes as they are).  Waves 0 and 1 then run chains A (even blocks) and B (odd
// blocks) over all chunks in order with wave_task_q8's fmaf, and wave 0 adds
// 0 + (A + B): bit-identical to wave_task_q8.  (For the 151936 x 1536 head:
// 38.2 us quantizing on the fly, against 39.6 us for one wave per row group
// over a quantized activation plus 2.5 us for the quantize launch.)
constexpr int kSplitWavesQ8 = 8;
struct SplitLdsQ8 {
    int32_t s[kChunkBlocks * kChunkBlocks * 64];   // [chunk][block][lane], C <= 8
    uint16_t dw[kChunkBlocks * kChunkBlocks * 64];
    uint32_t dx[kChunkBlocks * kChunkBlocks];      // fp32 bits of d_x per block (kFused)
    float chain_b[64];
};

template <bool kFused>
__device__ __forceinline__ void split_group_q8(const MatDesc& m, int g, SplitLdsQ8& l) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int C = m.C;
    const int c = (wave * C + kSplitWavesQ8 - 1) / kSplitWavesQ8;
    if (c < ((wave + 1) * C + kSplitWavesQ8 - 1) / kSplitWavesQ8) {  // the wave's one chunk
        const uint8_t* wp = m.w + ((size_t)g * C + c) * kQ8ChunkBytes;
        Piece pc[2];
        load_piece(pc[0], wp, lane);
        load_piece(pc[1], wp + kQ8PieceBytes, lane);
        ActQuant aq{m, g == 0, {}};
        if constexpr (kFused) aq.load(0, c);
        int s[kChunkBlocks];
        if constexpr (kFused) {
            const auto pr = aq.prepare(0, c);
            uint32_t y[4];
            rows4(pr.packed, y);
#pragma unroll
            for (int k = 0; k < 2; ++k) {  // piece k: blocks 4k .. 4k+3
                Unpacked u[4];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u[x].lo[j] = pc[k].q[2 * x][j];
                        u[x].hi[j] = pc[k].q[2 * x + 1][j];
                    }
                int sh[4];
                quad_dot16_rows(u, y[2 * k], y[2 * k + 1], sh);
#pragma unroll
                for (int x = 0; x < 4; ++x) s[4 * k + x] = sh[x];
            }
            if ((lane & 7) == 0) l.dx[c * kChunkBlocks + (lane >> 3)] = pr.dbits;
        } else {
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int b = 0; b < kQ8PieceBlocks; ++b) {
                    // padding blocks of the last chunk have zero weights; read a valid block
                    const int blk = min(c * kChunkBlocks + k * kQ8PieceBlocks + b, m.nb - 1);
                    s[4 * k + b] = block_dot_q8(pc[k].q[2 * b], pc[k].q[2 * b + 1], act_q(m.xq, (int64_t)blk * 32));
                }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int b = 0; b < kQ8PieceBlocks; ++b) {
                const int i = (c * kChunkBlocks + k * kQ8PieceBlocks + b) * 64 + lane;
                const uint32_t sw = pc[k].scale[b >> 1];
                l.s[i] = s[4 * k + b];
                l.dw[i] = (uint16_t)((b & 1) ? (sw >> 16) : (sw & 0xffffu));
            }
    }
    __syncthreads();
    float p = 0.0f;
    if (wave < 2) {  // wave 0: chain A, the even blocks; wave 1: chain B, the odd ones
        for (int cc = 0; cc < C; ++cc) {
#pragma unroll
            for (int j = 0; j < kChunkBlocks / 2; ++j) {
                const int b = 2 * j + wave;
                const int i = (cc * kChunkBlocks + b) * 64 + lane;
                const float dw = __half2float(__ushort_as_half(l.dw[i]));
                const float dx = kFused ? __uint_as_float(l.dx[cc * kChunkBlocks + b])
                                        : act_d(m.xd, min(cc * kChunkBlocks + b, m.nb - 1));
                p = fmaf(dw * dx, (float)l.s[i], p);
            }
        }
        if (wave == 1) l.chain_b[lane] = p;
    }
    __syncthreads();
    if (wave == 0) {
        float acc = 0.0f;
        acc += p + l.chain_b[lane];
        const int64_t row = (int64_t)g * kGroupRows + lane;
        if (row < m.rows) gwr<float>(m.y)[row] = acc;
    }
}

template <bool kFused>
__global__ __launch_bounds__(64 * kSplitWavesQ8) void k_gemv_q8_split(MatDesc m) {
    __shared__ SplitLdsQ8 l;
    split_group_q8<kFused>(m, blockIdx.x, l);
}

// Test hook: the exact per-block sums, from the same loads and dot.
template <int N>
__global__ __launch_bounds__(kThreads) void k_block_sums_q8(MatDesc m, int32_t* __restrict__ s) {
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    if (g >= m.G) return;
    const int64_t row = g * kGroupRows + lane;
    for (int c = 0; c < m.C; ++c) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            Piece pc;
            load_piece(pc, m.w + ((size_t)g * m.C + c) * kQ8ChunkBytes + k * kQ8PieceBytes, lane);
#pragma unroll
            for (int b = 0; b < kQ8PieceBlocks; ++b) {
                const int blk = c * kChunkBlocks + k * kQ8PieceBlocks + b;
                if (blk >= m.nb) break;
#pragma unroll
                for (int t = 0; t < N; ++t) {
                    const int v = block_dot_q8(pc.q[2 * b], pc.q[2 * b + 1],
                                               act_q(m.xq, (int64_t)t * m.cols + (int64_t)blk * 32));
                    if (row < m.rows) s[((int64_t)t * m.rows + row) * m.nb + blk] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- repack

// One thread per (group, chunk, block, row): the row's 32 int8 values and its
// binary16 scale into the packed layout; padding is zero.
__global__ __launch_bounds__(256) void k_repack_q8(const uint8_t* __restrict__ w, uint8_t* __restrict__ out,
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
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    uint16_t d = 0;
    if (row < rows && blk < nb) {
        const uint16_t* src = (const uint16_t*)(w + (row * nb + blk) * 34);  // 2-byte aligned
        d = src[0];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = (uint32_t)src[1 + 2 * k] | ((uint32_t)src[2 + 2 * k] << 16);
            hi[k] = (uint32_t)src[9 + 2 * k] | ((uint32_t)src[10 + 2 * k] << 16);
        }
    }
    uint8_t* base = out + gc * kQ8ChunkBytes + (b >> 2) * kQ8PieceBytes;
    const int lb = b & 3;
    *(u32x4*)(base + ((lb * 2 + 0) * kGroupRows + r) * 16) = lo;
    *(u32x4*)(base + ((lb * 2 + 1) * kGroupRows + r) * 16) = hi;
    *(uint16_t*)(base + kQ8PieceQBytes + r * 8 + lb * 2) = d;
}

// ---------------------------------------------------------------- requantize

// One thread per block.  Q4_0 rule (GGUF reference): in fp32, x_j = q_j * d8;
// vmax = the x_j of largest magnitude (first on ties); d = vmax / -8;
// id = 1 / d (correctly rounded; 0 when d == 0); nibble = min(15,
// trunc(x_j * id + 8.5)); the scale is stored as binary16(d), nearest even.
__global__ __launch_bounds__(256) void k_requant_q8_q4(const uint8_t* __restrict__ w8, uint8_t* __restrict__ w4,
                                                       int64_t n_blocks) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_blocks) return;
    const uint16_t* src = (const uint16_t*)(w8 + idx * 34);
    const float d8 = __half2float(__ushort_as_half(src[0]));
    float x[32];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint16_t u = src[1 + k];
        x[2 * k] = (float)(int8_t)(u & 0xff) * d8;
        x[2 * k + 1] = (float)(int8_t)(u >> 8) * d8;
    }
    float amax = 0.0f, vmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(x[j]);
        if (a > amax) {
            amax = a;
            vmax = x[j];
        }
    }
    float d = vmax / -8.0f;
    // Materialize d before its binary16 conversion: otherwise the product and
    // the conversion fold into one mixed-precision FMA with a +0 addend, which
    // turns the -0 scale of an all-zero block into +0.
    asm volatile("" : "+v"(d));
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    int nib[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) nib[j] = min(15, (int)(x[j] * id + 8.5f));
    uint16_t* dst = (uint16_t*)(w4 + idx * 18);
    dst[0] = __half_as_ushort(__float2half_rn(d));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t b0 = (uint32_t)(nib[2 * k] | (nib[2 * k + 16] << 4));
        const uint32_t b1 = (uint32_t)(nib[2 * k + 1] | (nib[2 * k + 17] << 4));
        dst[1 + k] = (uint16_t)(b0 | (b1 << 8));
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_repack_q8_0(const uint8_t* w, uint8_t* packed, int64_t rows, int64_t cols, hipStream_t st) {
    const int64_t G = groups_of(rows), C = chunks_of(cols);
    const int64_t total = G * C * kChunkBlocks * kGroupRows;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_repack_q8, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, w, packed, rows,
                       (int32_t)(cols / 32), (int32_t)C, total);
    return hipGetLastError();
}

template <int N>
static void gemv_q8_n(const MatDesc& m, int64_t n_gsets, hipStream_t st) {
    hipLaunchKernelGGL(k_gemv_q8<N>, dim3((unsigned)n_gsets), dim3(kThreads), 0, st, m);
}

hipError_t launch_gemv_q8_0(const MatDesc& m, int n, int64_t n_gsets, hipStream_t st) {
    if (n_gsets == 0 || n == 0) return hipSuccess;
    if (n == 1 && m.ks == 1) {
        hipLaunchKernelGGL(k_gemv_q8_split<false>, dim3((unsigned)m.G), dim3(64 * kSplitWavesQ8), 0, st, m);
        return hipGetLastError();
    }
    switch (n) {
        case 1: gemv_q8_n<1>(m, n_gsets, st); break;
        case 2: gemv_q8_n<2>(m, n_gsets, st); break;
        case 3: gemv_q8_n<3>(m, n_gsets, st); break;
        case 4: gemv_q8_n<4>(m, n_gsets, st); break;
        case 5: gemv_q8_n<5>(m, n_gsets, st); break;
        case 6: gemv_q8_n<6>(m, n_gsets, st); break;
        case 7: gemv_q8_n<7>(m, n_gsets, st); break;
        case 8: gemv_q8_n<8>(m, n_gsets, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_q8_0_fused(const MatDesc& m, hipStream_t st) {
    if (m.G == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gemv_q8_split<true>, dim3((unsigned)m.G), dim3(64 * kSplitWavesQ8), 0, st, m);
    return hipGetLastError();
}

template <int N>
static void sums_q8_n(const MatDesc& m, int32_t* s, hipStream_t st) {
    hipLaunchKernelGGL(k_block_sums_q8<N>, dim3((unsigned)((m.G + kWaves - 1) / kWaves)), dim3(kThreads), 0, st,
                       m, s);
}

hipError_t launch_block_sums_q8_0(const MatDesc& m, int n, int32_t* s, hipStream_t st) {
    if (m.G == 0 || n == 0 || m.nb == 0) return hipSuccess;
    switch (n) {
        case 1: sums_q8_n<1>(m, s, st); break;
        case 2: sums_q8_n<2>(m, s, st); break;
        case 3: sums_q8_n<3>(m, s, st); break;
        case 4: sums_q8_n<4>(m, s, st); break;
        case 5: sums_q8_n<5>(m, s, st); break;
        case 6: sums_q8_n<6>(m, s, st); break;
        case 7: sums_q8_n<7>(m, s, st); break;
        case 8: sums_q8_n<8>(m, s, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant_q8_0_to_q4_0(const uint8_t* w8, uint8_t* w4, int64_t n_blocks, hipStream_t st) {
    if (n_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_requant_q8_q4, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, st, w8, w4,
                       n_blocks);
    return hipGetLastError();
}

}  // namespace q4s
