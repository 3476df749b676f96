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
#include "q4s_lane.h"

namespace q4s {
namespace {

// ---------------------------------------------------------------- timeline
//
// With a trace buffer (q4s_sweep_set_trace), a sweep launch records, per
// workgroup b, the 100 MHz constant clock when it started (word 9b) and when
// each of its waves w finished its work (word 9b + 1 + w).  NULL: nothing.
constexpr int kTraceWords = kSweepTraceWords;

// Traced kernels are separate instantiations (kTrace), so the untraced ones
// keep their code; a traced one reads the clock when it starts and stores
// both marks only when it is done, so that no store precedes the weight loads.
__device__ __forceinline__ uint64_t trace_clock() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ void trace_marks(uint64_t* trace, uint64_t start) {
    if ((threadIdx.x & 63) == 0) {
        auto* t = gwr<uint64_t>(trace) + (size_t)blockIdx.x * kTraceWords;
        if (threadIdx.x == 0) t[0] = start;
        t[1 + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime();
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
// 4*lg + r: lanes 0-31 run chain A (blocks 0-3), lanes 32-63 chain B (blocks
// 4-7), and the chains are combined per segment exactly as in the 1-row path,
// so each row's result is bit-identical to the 1-row call.  Token slots >= n
// repeat row n-1 and are never stored.
//
// Each chunk's activation is staged through the wave's own LDS slice: two
// coalesced 16-byte loads per lane bring the 8 tokens x 256 bytes, which are
// written in A-operand order; the d_x and d_w scales are converted to fp32
// once per chunk on the way in.

// q: the slice's 16-byte A-operand slots; dx: its d_x/16 [token][block] fp32
__device__ __forceinline__ void stage_act_to(const ActRaw& a, u32x4* q, float* dx) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, b = j >> 1, e = j & 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int t = (lane >> 4) + 4 * k;
        const u32x4 v = k ? a.q1 : a.q0;
        u32x2* s0 = (u32x2*)&q[(t * 8 + b) * 2 + 0];
        u32x2* s1 = (u32x2*)&q[(t * 8 + b) * 2 + 1];
        s0[e] = (u32x2){v[0], v[1]};
        s1[e] = (u32x2){v[2], v[3]};
    }
    dx[lane] = __half2float(__ushort_as_half((uint16_t)a.dxh)) * 0.0625f;
}

__device__ __forceinline__ void stage_act(const ActRaw& a, WaveLds& L) { stage_act_to(a, L.q, (float*)L.dx); }

template <int N>
__device__ __forceinline__ void chunk_mfma(Chunk& ch, const ActRaw& ar, float (&part)[16], WaveLds& L) {
    const int lane = threadIdx.x & 63;
    const int lg = lane >> 4, j = lane & 15, h = lane >> 5;
    // stage: the activation, and the lane's own row scales as fp32
    stage_act(ar, L);
    {
        f32x4 lo = {half_lo(ch.scale[0]), half_hi(ch.scale[0]), half_lo(ch.scale[1]), half_hi(ch.scale[1])};
        f32x4 hi = {half_lo(ch.scale[2]), half_hi(ch.scale[2]), half_lo(ch.scale[3]), half_hi(ch.scale[3])};
        L.dw[2 * lane] = lo;
        L.dw[2 * lane + 1] = hi;
    }
    // the lane's scales: d_w of rows 16*mt + j and d_x/16 of token slots
    // 4*(lg&1) + r, both for its blocks 4h .. 4h+3
    f32x4 dw[4], dx[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dw[mt] = L.dw[2 * (16 * mt + j) + h];
#pragma unroll
    for (int r = 0; r < 4; ++r) dx[r] = L.dx[2 * (4 * (lg & 1) + r) + h];
    const bool active = h == (j >> 3);
    const int abase = active ? ((j & 7) * 8 + 4 * h) * 2 + (lg & 1) : kZeroSlot;
    const int astep = active ? 2 : 0;
#pragma unroll
    for (int p = 0; p < kChunkBlocks / 2; ++p) {
        // B operands: lane (g, j) gets dwords 2(g&1), 2(g&1)+1 of block p + 4(g>>1)
        // of row 16*mt + j, for the 4 row tiles mt
        uint32_t e[4] = {ch.nib[p][0], ch.nib[p][2], ch.nib[p + 4][0], ch.nib[p + 4][2]};
        uint32_t o[4] = {ch.nib[p][1], ch.nib[p][3], ch.nib[p + 4][1], ch.nib[p + 4][3]};
        xpose4x4(e);
        xpose4x4(o);
        const i32x4 aop = (i32x4)L.q[abase + p * astep];
        const i32x4 zero = {0, 0, 0, 0};
        i32x4 d[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const i32x4 bop = {(int)((e[mt] << 4) & 0xF0F0F0F0u), (int)((o[mt] << 4) & 0xF0F0F0F0u),
                               (int)(e[mt] & 0xF0F0F0F0u), (int)(o[mt] & 0xF0F0F0F0u)};
            d[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, zero, 0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[mt * 4 + r] = fmaf(dw[mt][p] * dx[r][p], (float)d[mt][r], part[mt * 4 + r]);
    }
}

// acc[mt*4 + r] = y[token 4*(lg&1) + r][row g*64 + 16*mt + j] (lanes 0-31; lanes
// 32-63 hold the same values)
template <int N, bool kTemporal = false>
__device__ __forceinline__ void wave_task_mfma(const MatDesc& m, int g, int c0, int c1, float (&acc)[16],
                                               WaveLds& L) {
    const int lane = threadIdx.x & 63;
    float part[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = part[k] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    if (lane == 0) L.q[kZeroSlot] = (u32x4){0u, 0u, 0u, 0u};
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kChunkBytes + lane * kBlockNibBytes;
    auto seg_end = [&](int c) {  // after chunk c: close the segment if it ends here
        if (c + 1 == c1 || (c + 1 - c0) % kSegChunks == 0) {
            // chain A lives in lanes 0-31, chain B in lanes 32-63
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[k]), __float_as_uint(part[k]),
                                                           false, false);
                acc[k] += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                part[k] = 0.0f;
            }
        }
    };
    // unconditional prefetch in the steady state, as in the 1-row path
    Chunk wa, wb;
    ActRaw aa, ab;
    load_chunk<kTemporal>(wa, wp);
    load_act<N>(aa, m, c0);
    int c = c0;
    for (; c + 2 < c1; c += 2, wp += 2 * kChunkBytes) {
        load_chunk<kTemporal>(wb, wp + kChunkBytes);
        load_act<N>(ab, m, c + 1);
        chunk_mfma<N>(wa, aa, part, L);
        seg_end(c);
        load_chunk<kTemporal>(wa, wp + 2 * kChunkBytes);
        load_act<N>(aa, m, c + 2);
        chunk_mfma<N>(wb, ab, part, L);
        seg_end(c + 1);
    }
    if (c + 1 < c1) {
        load_chunk<kTemporal>(wb, wp + kChunkBytes);
        load_act<N>(ab, m, c + 1);
        chunk_mfma<N>(wa, aa, part, L);
        seg_end(c);
        chunk_mfma<N>(wb, ab, part, L);
        seg_end(c + 1);
    } else {
        chunk_mfma<N>(wa, aa, part, L);
        seg_end(c);
    }
}

template <int N, bool kTemporal = false>
__device__ __forceinline__ void run_tile_mfma(const MatDesc& m, int64_t gset, float* red, WaveLds* wl) {
    run_tile_mfma_with<N>(m, gset, red, wl, [&](int g, int c0, int c1, float (&acc)[16], WaveLds& L) {
        wave_task_mfma<N, kTemporal>(m, g, c0, c1, acc, L);
    });
}

template <int N>
__device__ __forceinline__ void run_tile(const MatDesc& m, int64_t gset, float* red) {
    run_tile_with<N>(m, gset, red, [&](int g, int c0, int c1, float (&acc)[N]) {
        ActGlobal act{m};
        wave_task<N>(m, g, c0, c1, acc, act);
    });
}

template <int N>
__device__ __forceinline__ void run_any(const MatDesc& m, int64_t gset, TileLds<N>& l) {
    if constexpr (N == 1)
        run_tile<1>(m, gset, l.red);
    else
        run_tile_mfma<N>(m, gset, l.red, l.wl);
}

// The MFMA kernels (n >= 2) are held to 2 waves per SIMD (<= 256 registers).
template <int N>
__global__ __launch_bounds__(kThreads, N == 1 ? 1 : 2) void k_gemv(MatDesc m) {
    __shared__ TileLds<N> l;
    run_any<N>(m, blockIdx.x, l);
}

// The sweep: workgroup i takes tile i = (matrix, group set) of a table sorted
// by tile size, largest first, so the hardware dispatcher's in-order
// assignment to free slots is a longest-first list schedule.
template <int N, bool kTrace>
__global__ __launch_bounds__(kThreads, N == 1 ? 1 : 2) void k_sweep(const MatDesc* __restrict__ mats,
                                                    const uint32_t* __restrict__ tiles,
                                                    uint64_t* __restrict__ trace) {
    __shared__ TileLds<N> l;
    const uint64_t t_start = kTrace ? trace_clock() : 0;
    const uint32_t mi = tiles[2 * (size_t)blockIdx.x];
    const uint32_t gs = tiles[2 * (size_t)blockIdx.x + 1];
    const MatDesc m = mats[mi];
    run_any<N>(m, gs, l);
    if constexpr (kTrace) trace_marks(trace, t_start);
}

// ---------------------------------------------------------------- tiled steps (9..24 rows)
//
// A step of n > 8 rows as token tiles of 8 on separate workgroups, each
// running the 8-row kernel on its rows (so every row is bit-identical to the
// 1-row result).  The tiles of one unit (group set, or sweep table entry) get
// block indices 8 apart: the dispatcher deals workgroups to the 8 XCDs in
// turn, so they land on the same XCD at about the same time and the later
// tiles read the weights from its L2 (the tiled kernels load them without the
// non-temporal hint) instead of HBM.
__device__ __forceinline__ bool tiled_unit(int tt, int64_t n_units, int64_t& unit, int& tile) {
    const int64_t i = blockIdx.x, x = i & 7, s = i >> 3;
    unit = (s / tt) * 8 + x;
    tile = (int)(s % tt);
    return unit < n_units;
}

__device__ __forceinline__ MatDesc token_tile(const MatDesc& m, int tile) {
    MatDesc t = m;
    const int t0 = kTokTile * tile;
    t.xq = m.xq + (int64_t)t0 * m.cols;
    t.xd = m.xd + (int64_t)t0 * m.dstride;
    t.y = m.y + (int64_t)t0 * m.rows;
    t.n = min(kTokTile, m.n - t0);
    return t;
}

__global__ __launch_bounds__(kThreads, 2) void k_gemv_tiled(MatDesc m, int tt, int64_t n_gsets) {
    __shared__ TileLds<kTokTile> l;
    int64_t gset;
    int tile;
    if (!tiled_unit(tt, n_gsets, gset, tile)) return;
    run_tile_mfma<kTokTile, true>(token_tile(m, tile), gset, l.red, l.wl);
}

__global__ __launch_bounds__(kThreads, 2) void k_sweep_tiled(const MatDesc* __restrict__ mats,
                                                            const uint32_t* __restrict__ tiles, int tt,
                                                            int64_t n_entries) {
    __shared__ TileLds<kTokTile> l;
    int64_t e;
    int tile;
    if (!tiled_unit(tt, n_entries, e, tile)) return;
    const uint32_t mi = tiles[2 * (size_t)e];
    const uint32_t gs = tiles[2 * (size_t)e + 1];
    run_tile_mfma<kTokTile, true>(token_tile(mats[mi], tile), gs, l.red, l.wl);
}

// grid of a tiled launch: 8 * tt * ceil(units / 8)
inline unsigned tiled_grid(int tt, int64_t units) { return (unsigned)(8 * tt * ((units + 7) / 8)); }

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

// One block per 8 lanes; `valid` is uniform over the 8 lanes of a block.
// With kNt the codes and scales go out with non-temporal stores: a step of up
// to 8 rows writes its 4.3 MB of Q8_0 bytes just ahead of the weight stream
// (8-row 1.5B step 165 -> 163.5 us), while past 8 rows every token tile
// reads them back and they are better left in L2 (16 rows 236 -> 242 us
// with the hint).
template <bool kNt>
__device__ __forceinline__ void quant_block8(const float* x, int8_t* q, uint16_t* d, bool valid) {
    const int o = threadIdx.x & 7;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid) v = *gp<f32x4>(x + 4 * o);
    const float a = quant8_amax(v);
    if (!valid) return;
    uint32_t packed;
    uint16_t h;
    quant8_codes(v, a, packed, h);
    if constexpr (kNt) {
        __builtin_nontemporal_store(packed, gwr<uint32_t>(q + 4 * o));
        if (o == 0) __builtin_nontemporal_store(h, gwr<uint16_t>(d));
    } else {
        *gwr<uint32_t>(q + 4 * o) = packed;
        if (o == 0) *gwr<uint16_t>(d) = h;
    }
}

// Block lb (row-major over [n][nb]) of one activation; the lanes of a row's
// last block also zero the row's padding entries of d_x.
template <bool kNt>
__device__ __forceinline__ void quant_local(const QuantDesc& qd, int64_t lb, bool valid) {
    const int nb = qd.cols / 32;
    const int64_t t = valid ? lb / nb : 0;
    const int64_t b = valid ? lb - t * nb : 0;
    const int64_t off = t * qd.cols + b * 32;
    quant_block8<kNt>(qd.x + off, qd.q + off, qd.d + t * qd.dstride + b, valid);
    const int o = threadIdx.x & 7;
    if (valid && b == nb - 1 && o < qd.dstride - nb) gwr<uint16_t>(qd.d)[t * qd.dstride + nb + o] = 0;
}

// Standalone quantization: 32 blocks per 256-thread workgroup.
template <bool kNt>
__global__ __launch_bounds__(256) void k_quantize(QuantDesc qd, int64_t total_blocks) {
    const int64_t lb = (int64_t)blockIdx.x * kQuantTileBlocks + (threadIdx.x >> 3);
    quant_local<kNt>(qd, lb, lb < total_blocks);
}

// Batched quantization for the sweep: workgroup i takes tile i = (activation,
// first block) of a host-built table and quantizes up to kQuantTileBlocks
// consecutive blocks of that activation, one block per 8 lanes.
template <bool kNt>
__global__ __launch_bounds__(256) void k_quantize_batch(const QuantDesc* __restrict__ descs,
                                                        const uint32_t* __restrict__ tiles) {
    const uint32_t di = tiles[2 * (size_t)blockIdx.x];
    const uint32_t b0 = tiles[2 * (size_t)blockIdx.x + 1];
    const QuantDesc qd = descs[di];
    const int64_t total = (int64_t)qd.n * (qd.cols / 32);
    const int64_t lb = (int64_t)b0 + (threadIdx.x >> 3);
    quant_local<kNt>(qd, lb, lb < total);
}

// ---------------------------------------------------------------- 1-row split tiles
//
// A 1-row GEMV or sweep whose matrices all have one K split (C <= 8 chunks):
// each row group (a table entry: matrix, row group) gets its own workgroup of
// kSplitWaves waves.  Wave w takes chunks [ceil(wC/W), ceil((w+1)C/W)) -- one
// chunk at most with 8 waves -- issues its loads at once, and leaves in LDS
// each block's exact integer sum (int16: |s| <= 32512) and the fp32 product
// (d_w / 16) * d_x, formed as wave_task forms it.  Waves 0 and 1 then read
// all of their factors at once and run chains A (blocks 0-3) and B (blocks
// 4-7) over all chunks in order with wave_task's fmaf, and wave 0 adds
// 0 + (A + B): bit-identical to a wave task over the whole row, with every
// weight load of the row group in flight from the start.  (Reading d_x inside
// the chain cost the GEMV over quantized codes a global load per chunk: the
// lone head 22.3 -> 21.8 us with the products formed by the chunk's wave.)  (A lone output head, 2374 row groups of 6 chunks, is too
// small for waves that stream their chunks two at a time: one wave per row
// group took 22.7 us as a plain GEMV and 23.1 us quantizing on the fly, 8 waves
// take 22.6 and 22.2 us; 2 and 4 waves were slower.)
constexpr int kSplitWaves = 8;
struct SplitLds {
    float a[kChunkBlocks * kChunkBlocks * 64];      // [chunk][block][lane]: (d_w / 16) * d_x, fp32
    uint32_t s[kChunkBlocks * kChunkBlocks / 2 * 64]; // [chunk][block pair][lane]: the two exact sums, int16 each
    float chain_b[64];
};

template <bool kFused, int kW>
__device__ __forceinline__ void split_group(const MatDesc& m, int g, SplitLds& l) {
    static_assert(kW >= 2 && kW <= 8, "2 to 8 waves per row group");
    constexpr int kPer = (kChunkBlocks + kW - 1) / kW;  // chunks per wave at most (C <= 8)
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int C = m.C;
    const int i0 = (wave * C + kW - 1) / kW, i1 = ((wave + 1) * C + kW - 1) / kW;
    if (i0 < i1) {
        const uint8_t* wp = m.w + ((size_t)g * C + i0) * kChunkBytes + lane * kBlockNibBytes;
        Chunk ch[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (i0 + k < i1) load_chunk(ch[k], wp + k * kChunkBytes);
        ActQuantN<kPer> aq{m, g == 0, {}};
        if constexpr (kFused) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                if (i0 + k < i1) aq.load(k, i0 + k);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int c = i0 + k;
            if (c >= i1) break;
            int s16[kChunkBlocks];
            float dx[kChunkBlocks];
            if constexpr (kFused) {
                const auto pr = aq.prepare(k, c);
                uint32_t y[4];
                rows4(pr.packed, y);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Unpacked u[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) u[x] = unpack(ch[k].nib[4 * h + x]);
                    int sh[4];
                    quad_dot16_rows(u, y[2 * h], y[2 * h + 1], sh);
#pragma unroll
                    for (int x = 0; x < 4; ++x) s16[4 * h + x] = sh[x];
                }
#pragma unroll
                for (int b = 0; b < kChunkBlocks; ++b) dx[b] = aq.d(pr, 0, 0, b);
            } else {
#pragma unroll
                for (int b = 0; b < kChunkBlocks; ++b) {
                    // padding blocks of the last chunk have zero nibbles; read a valid block
                    const int blk = min(c * kChunkBlocks + b, m.nb - 1);
                    s16[b] = block_dot16(unpack(ch[k].nib[b]), act_q(m.xq, (int64_t)blk * 32));
                    dx[b] = act_d(m.xd, blk);
                }
            }
            // the chain's factors, formed here with the chain's own fp32 operations
#pragma unroll
            for (int b = 0; b < kChunkBlocks; ++b) {
                const uint32_t sw = ch[k].scale[b >> 1];
                const float dw16 = ((b & 1) ? half_hi(sw) : half_lo(sw)) * 0.0625f;
                l.a[(c * kChunkBlocks + b) * 64 + lane] = dw16 * dx[b];
            }
#pragma unroll
            for (int b = 0; b < kChunkBlocks; b += 2)
                l.s[(c * (kChunkBlocks / 2) + b / 2) * 64 + lane] =
                    (uint32_t)(uint16_t)(int16_t)(s16[b] >> 4) | ((uint32_t)(uint16_t)(int16_t)(s16[b + 1] >> 4) << 16);
        }
    }
    __syncthreads();
    float p = 0.0f;
    if (wave < 2) {
        // every factor of the chain is read before its first fmaf, so the
        // dependent chain does not wait on LDS between chunks
        float av[kChunkBlocks][4];
        uint32_t sv[kChunkBlocks][2];
#pragma unroll
        for (int c = 0; c < kChunkBlocks; ++c) {
            if (c >= C) break;
#pragma unroll
            for (int x = 0; x < 4; ++x) av[c][x] = l.a[(c * kChunkBlocks + 4 * wave + x) * 64 + lane];
#pragma unroll
            for (int y = 0; y < 2; ++y) sv[c][y] = l.s[(c * (kChunkBlocks / 2) + 2 * wave + y) * 64 + lane];
        }
#pragma unroll
        for (int c = 0; c < kChunkBlocks; ++c) {
            if (c >= C) break;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int sb = (int)(int16_t)(uint16_t)(sv[c][x >> 1] >> (16 * (x & 1)));
                p = fmaf(av[c][x], (float)(sb * 16), p);
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

// At most 64 VGPRs, so that 4 workgroups of 8 waves stay resident per CU.
template <bool kFused, int kW, bool kTrace>
__global__ __launch_bounds__(64 * kW, 8) void k_sweep_split(const MatDesc* __restrict__ mats,
                                                          const uint32_t* __restrict__ tiles,
                                                          uint64_t* __restrict__ trace) {
    __shared__ SplitLds l;
    const uint64_t t_start = kTrace ? trace_clock() : 0;
    const MatDesc m = mats[tiles[2 * (size_t)blockIdx.x]];
    split_group<kFused, kW>(m, (int)tiles[2 * (size_t)blockIdx.x + 1], l);
    if constexpr (kTrace) trace_marks(trace, t_start);
}

template <int kW>
__global__ __launch_bounds__(64 * kW, 8) void k_gemv_split(MatDesc m) {
    __shared__ SplitLds l;
    split_group<false, kW>(m, blockIdx.x, l);
}

// ---------------------------------------------------------------- fused 1-row sweep
//
// With one activation row the sweep quantizes inside the GEMV launch (the
// pages' mega kernel quantizes the activation once per step inside its single
// kernel, milestone M15): every wave quantizes the chunks it streams (see
// ActQuant), so the bytes -- and the results -- equal those of a separate
// quantize launch, and the group-0 waves publish them to x_q8.
//
// A tile entry names a row group of a single-split matrix (C <= 8), whose
// chunks spread over the 4 waves as split tiles (split_group: exact block sums
// in LDS, then chains A and B in the fixed order), or a group set of a
// multi-split matrix (the ks waves of a row group stream contiguous chunk
// ranges).  Short tiles matter at the end of the launch: with 4 row groups of 6
// chunks per workgroup every wave streams 6 chunks in turn, and the last
// workgroups leave HBM under-fed while they finish (a replay of this tile plan
// as plain reads took 133 us with a fixed per-chunk delay, 124 us with one row
// group per workgroup).
union FusedLds {
    SplitLds split;
    float red[kWaves * 64];
};

template <bool kFused>
__device__ __forceinline__ void sweep_row1(const MatDesc& m, uint32_t t, FusedLds& l) {
    if (m.ks == 1) {
        split_group<kFused, kWaves>(m, (int)t, l.split);
        return;
    }
    if constexpr (kFused) {
        run_tile_with<1>(m, t, l.red, [&](int g, int c0, int c1, float (&acc)[1]) {
            ActQuant act{m, g == 0, {}};
            wave_task<1>(m, g, c0, c1, acc, act);
        });
    } else {
        run_tile<1>(m, t, l.red);
    }
}

template <bool kTrace>
__global__ __launch_bounds__(kThreads, 1) void k_sweep_fused(const MatDesc* __restrict__ mats,
                                                            const uint32_t* __restrict__ tiles,
                                                            uint64_t* __restrict__ trace) {
    __shared__ FusedLds l;
    const uint64_t t_start = kTrace ? trace_clock() : 0;
    sweep_row1<true>(mats[tiles[2 * (size_t)blockIdx.x]], tiles[2 * (size_t)blockIdx.x + 1], l);
    if constexpr (kTrace) trace_marks(trace, t_start);
}

// The same tiles over activations quantized beforehand.
template <bool kTrace>
__global__ __launch_bounds__(kThreads, 1) void k_sweep_one(const MatDesc* __restrict__ mats,
                                                          const uint32_t* __restrict__ tiles,
                                                          uint64_t* __restrict__ trace) {
    __shared__ FusedLds l;
    const uint64_t t_start = kTrace ? trace_clock() : 0;
    sweep_row1<false>(mats[tiles[2 * (size_t)blockIdx.x]], tiles[2 * (size_t)blockIdx.x + 1], l);
    if constexpr (kTrace) trace_marks(trace, t_start);
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

// The GEMV's read pattern without its arithmetic: wave i of the launch reads
// unit i (unit_kb contiguous KB) with 1 KB wave loads, 9 in flight (one chunk's
// worth), one workgroup of 4 waves per 4 units.
__global__ __launch_bounds__(256) void k_bench_read_units(const u32x4* __restrict__ buf, int64_t n_units,
                                                          int64_t unit_kb, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (u < n_units) {
        const u32x4* p = buf + u * unit_kb * 64 + lane;
        int64_t i = 0;
        for (; i + 9 <= unit_kb; i += 9) {
            u32x4 v[9];
#pragma unroll
            for (int k = 0; k < 9; ++k) v[k] = __builtin_nontemporal_load(p + (i + k) * 64);
#pragma unroll
            for (int k = 0; k < 9; ++k) acc ^= v[k];
        }
        for (; i < unit_kb; ++i) acc ^= __builtin_nontemporal_load(p + i * 64);
    }
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
    const int64_t grid = (total + kQuantTileBlocks - 1) / kQuantTileBlocks;
    if (d.n <= kTokTile)
        hipLaunchKernelGGL(k_quantize<true>, dim3((unsigned)grid), dim3(256), 0, st, d, total);
    else
        hipLaunchKernelGGL(k_quantize<false>, dim3((unsigned)grid), dim3(256), 0, st, d, total);
    return hipGetLastError();
}

hipError_t launch_quantize_batch(const QuantDesc* dev_descs, const uint32_t* dev_tiles, int64_t n_tiles, int n,
                                 hipStream_t st) {
    if (n_tiles == 0) return hipSuccess;
    if (n <= kTokTile)
        hipLaunchKernelGGL(k_quantize_batch<true>, dim3((unsigned)n_tiles), dim3(256), 0, st, dev_descs, dev_tiles);
    else
        hipLaunchKernelGGL(k_quantize_batch<false>, dim3((unsigned)n_tiles), dim3(256), 0, st, dev_descs, dev_tiles);
    return hipGetLastError();
}

template <int N>
static void gemv_n(const MatDesc& m, int64_t n_gsets, hipStream_t st) {
    hipLaunchKernelGGL(k_gemv<N>, dim3((unsigned)n_gsets), dim3(kThreads), 0, st, m);
}

hipError_t launch_gemv(const MatDesc& m, int n, int64_t n_gsets, hipStream_t st) {
    if (n_gsets == 0 || n == 0) return hipSuccess;
    if (n == 1 && m.ks == 1) {
        hipLaunchKernelGGL(k_gemv_split<kSplitWaves>, dim3((unsigned)m.G), dim3(64 * kSplitWaves), 0, st, m);
        return hipGetLastError();
    }
    if (n > kTokTile) {
        const int tt = (n + kTokTile - 1) / kTokTile;
        hipLaunchKernelGGL(k_gemv_tiled, dim3(tiled_grid(tt, n_gsets)), dim3(kThreads), 0, st, m, tt, n_gsets);
        return hipGetLastError();
    }
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
static void sweep_n(const MatDesc* mats, const uint32_t* tiles, int64_t n_tiles, uint64_t* trace, hipStream_t st) {
    if (trace)
        hipLaunchKernelGGL((k_sweep<N, true>), dim3((unsigned)n_tiles), dim3(kThreads), 0, st, mats, tiles, trace);
    else
        hipLaunchKernelGGL((k_sweep<N, false>), dim3((unsigned)n_tiles), dim3(kThreads), 0, st, mats, tiles, trace);
}

hipError_t launch_sweep(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles, int n,
                        uint64_t* trace, hipStream_t st) {
    if (n_tiles == 0 || n == 0) return hipSuccess;
    if (n > kTokTile) {
        const int tt = (n + kTokTile - 1) / kTokTile;
        hipLaunchKernelGGL(k_sweep_tiled, dim3(tiled_grid(tt, n_tiles)), dim3(kThreads), 0, st, dev_mats, dev_tiles,
                           tt, n_tiles);
        return hipGetLastError();
    }
    switch (n) {
        case 1:  // tiles of single-split matrices are row groups (split tiles)
            if (trace)
                hipLaunchKernelGGL(k_sweep_one<true>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, dev_mats,
                                   dev_tiles, trace);
            else
                hipLaunchKernelGGL(k_sweep_one<false>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, dev_mats,
                                   dev_tiles, trace);
            break;
        case 2: sweep_n<2>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 3: sweep_n<3>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 4: sweep_n<4>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 5: sweep_n<5>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 6: sweep_n<6>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 7: sweep_n<7>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        case 8: sweep_n<8>(dev_mats, dev_tiles, n_tiles, trace, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sweep_split(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles, bool fused,
                             uint64_t* trace, hipStream_t st) {
    if (n_tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)n_tiles), block(64 * kSplitWaves);
    if (fused && trace)
        hipLaunchKernelGGL((k_sweep_split<true, kSplitWaves, true>), grid, block, 0, st, dev_mats, dev_tiles, trace);
    else if (fused)
        hipLaunchKernelGGL((k_sweep_split<true, kSplitWaves, false>), grid, block, 0, st, dev_mats, dev_tiles, trace);
    else if (trace)
        hipLaunchKernelGGL((k_sweep_split<false, kSplitWaves, true>), grid, block, 0, st, dev_mats, dev_tiles, trace);
    else
        hipLaunchKernelGGL((k_sweep_split<false, kSplitWaves, false>), grid, block, 0, st, dev_mats, dev_tiles, trace);
    return hipGetLastError();
}

hipError_t launch_sweep_fused(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles,
                              uint64_t* trace, hipStream_t st) {
    if (n_tiles == 0) return hipSuccess;
    if (trace)
        hipLaunchKernelGGL(k_sweep_fused<true>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, dev_mats, dev_tiles,
                           trace);
    else
        hipLaunchKernelGGL(k_sweep_fused<false>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, dev_mats, dev_tiles,
                           trace);
    return hipGetLastError();
}

template <int N>
static void sums_n(const MatDesc& m, int32_t* s, hipStream_t st) {
    const int64_t grid = (m.G + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_block_sums<N>, dim3((unsigned)grid), dim3(kThreads), 0, st, m, s);
}

hipError_t launch_block_sums(const MatDesc& m, int n, int32_t* s, hipStream_t st) {
    if (m.G == 0 || n == 0 || m.nb == 0) return hipSuccess;
    if (n > kTokTile) {  // slices of up to 8 rows
        for (int t0 = 0; t0 < n; t0 += kTokTile) {
            MatDesc ms = m;
            ms.xq = m.xq + (int64_t)t0 * m.cols;
            ms.xd = m.xd + (int64_t)t0 * m.dstride;
            const int k = min(kTokTile, n - t0);
            ms.n = k;
            const hipError_t e = launch_block_sums(ms, k, s + (int64_t)t0 * m.rows * m.nb, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
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

hipError_t launch_bench_read_units(const void* buf, size_t bytes, size_t unit_bytes, uint32_t* sink, hipStream_t st) {
    const int64_t unit_kb = (int64_t)(unit_bytes / 1024);
    const int64_t n_units = unit_kb > 0 ? (int64_t)(bytes / unit_bytes) : 0;  // whole units only
    if (n_units == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bench_read_units, dim3((unsigned)((n_units + 3) / 4)), dim3(256), 0, st, (const u32x4*)buf,
                       n_units, unit_kb, sink);
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
