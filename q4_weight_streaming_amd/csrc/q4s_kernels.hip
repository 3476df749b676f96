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
#include "q4s_device.h"

namespace q4s {
namespace {

// ---------------------------------------------------------------- loads

// The 9 x 16 bytes a lane reads per chunk: 8 blocks of nibbles, then its row's
// 8 binary16 scales.
struct Chunk {
    u32x4 nib[kChunkBlocks];
    u32x4 scale;
};

// Weights are streamed with non-temporal loads; the tiled many-row steps
// (kTemporal) keep them in L2 for the other token tiles of the same rows.
template <bool kTemporal = false>
__device__ __forceinline__ void load_chunk(Chunk& ch, const uint8_t* p) {
#pragma unroll
    for (int b = 0; b < kChunkBlocks; ++b) {
        const Q4S_GLOBAL u32x4* a = gp<u32x4>(p + b * (kGroupRows * kBlockNibBytes));
        ch.nib[b] = kTemporal ? *a : __builtin_nontemporal_load(a);
    }
    const Q4S_GLOBAL u32x4* a = gp<u32x4>(p + kChunkNibBytes);
    ch.scale = kTemporal ? *a : __builtin_nontemporal_load(a);
}

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

// Summation order shared by every path.  A wave task streams chunks [c0, c1)
// of one row group.  Within a segment of up to kSegChunks chunks, blocks 0-3
// of every chunk form chain A and blocks 4-7 chain B, each one fmaf per block
// in chunk order; at the end of the segment the task accumulator takes
// acc += (A + B).  The per-block term is fmaf(d_w/16 * d_x, (float)(16 s), .):
// the product of the two scales is exact, so it equals fmaf(d_w * d_x,
// (float)s, .) bit for bit.  The MFMA path forms exactly these chains.

// ---------------------------------------------------------------- Q8_0 quantization

// 8 consecutive lanes quantize one block, 4 values each: d = max|x| / 127
// (correctly rounded fp32 division), q = roundf(x / d) (half away from zero),
// d_x = binary16(d) rounded to nearest even.  All-zero blocks give d = 0, q = 0.
// quant8_amax is called by all 8 lanes of a block (it shuffles among them).
__device__ __forceinline__ float quant8_amax(const f32x4& v) {
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 8));
    return a;
}

// this lane's 4 quantized values (packed) and the block's binary16 d_x
__device__ __forceinline__ void quant8_codes(const f32x4& v, float a, uint32_t& packed, uint16_t& h) {
    const float dd = a / 127.0f;
    packed = 0;
    if (a != 0.0f) {
#pragma unroll
        for (int k = 0; k < 4; ++k) packed |= ((uint32_t)(uint8_t)(int8_t)(int)roundf(v[k] / dd)) << (8 * k);
    }
    h = __half_as_ushort(__float2half_rn(dd));
}

// Where the lane-per-row path gets the Q8_0 activation.  load(slot, c) runs
// when chunk c's weight loads are issued (slot 0 or 1 follows the chunk
// buffer), prepare(slot, c) when chunk c is consumed; q and d then give block
// blk (b within the chunk) as scalar operands.
//
// ActGlobal: the planar buffer in global memory, through scalar loads.
struct ActGlobal {
    const MatDesc& m;
    struct Prep {};
    __device__ __forceinline__ void load(int, int) {}
    __device__ __forceinline__ Prep prepare(int, int) { return {}; }
    __device__ __forceinline__ u32x8 q(const Prep&, int t, int blk, int) const {
        return act_q(m.xq, (int64_t)t * m.cols + (int64_t)blk * 32);
    }
    __device__ __forceinline__ float d(const Prep&, int t, int blk, int) const {
        return act_d(m.xd, (int64_t)t * m.dstride + blk);
    }
};

// ActQuant (the fused 1-row sweep): the wave quantizes the 256 fp32 values of
// the chunk it is about to consume itself -- lane l holds values 4(l%8) ..
// 4(l%8)+3 of block l/8, 8 lanes per Q8_0 block with the standalone
// quantizer's arithmetic -- and broadcasts codes and scales with v_readlane.
// The activation load travels with the chunk's weight loads, so no barrier or
// prologue stands between the launch and the weight stream.  With `publish`
// (the waves of row group 0) the codes are also written to x_q8.
struct ActQuant {
    const MatDesc& m;
    bool publish;
    f32x4 xs[2];
    struct Prep {
        uint32_t packed;  // this lane's 4 codes
        uint32_t dbits;   // fp32 bits of its block's binary16 d_x
    };
    __device__ __forceinline__ void load(int slot, int c) {
        const int lane = threadIdx.x & 63;
        // clamped, so the load is unconditional; lanes past the row are zeroed in prepare
        const int64_t i = min((int64_t)c * 256 + 4 * lane, (int64_t)m.cols - 4);
        xs[slot] = *gp<f32x4>(m.x + i);
    }
    __device__ __forceinline__ Prep prepare(int slot, int c) {
        const int lane = threadIdx.x & 63;
        const int blk = c * kChunkBlocks + (lane >> 3);
        const bool valid = blk < m.nb;  // uniform over the 8 lanes of a block
        f32x4 v = xs[slot];
        if (!valid) v = (f32x4){0.f, 0.f, 0.f, 0.f};
        const float a = quant8_amax(v);
        uint32_t packed;
        uint16_t h;
        quant8_codes(v, a, packed, h);
        if (publish && valid) {
            const int o = lane & 7;
            *gwr<uint32_t>((void*)(m.xq + (int64_t)c * 256 + 4 * lane)) = packed;
            if (o == 0) *gwr<uint16_t>((void*)(m.xd + blk)) = h;
            if (blk == m.nb - 1 && o < m.dstride - m.nb) gwr<uint16_t>((void*)m.xd)[m.nb + o] = 0;
        }
        return {packed, __float_as_uint(__half2float(__ushort_as_half(h)))};
    }
    __device__ __forceinline__ u32x8 q(const Prep& p, int, int, int b) const {
        u32x8 r;
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = __builtin_amdgcn_readlane(p.packed, 8 * b + k);
        return r;
    }
    __device__ __forceinline__ float d(const Prep& p, int, int, int b) const {
        return __uint_as_float(__builtin_amdgcn_readlane(p.dbits, 8 * b));
    }
};

// Adds chunk `c` (held in ch) of the lane's row into the chains pa / pb.
template <int N, class Act>
__device__ __forceinline__ void chunk_fma(const MatDesc& m, int c, const Chunk& ch, float (&pa)[N],
                                          float (&pb)[N], Act& act, int slot) {
    const auto pr = act.prepare(slot, c);
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
            const u32x8 q = act.q(pr, t, blk, b);
            const int s16 = block_dot16(u, q);
            const float dx = act.d(pr, t, blk, b);
            float& p = (b < kChunkBlocks / 2) ? pa[t] : pb[t];
            p = fmaf(dw16 * dx, (float)s16, p);
        }
    }
}

// One wave streams chunks [c0, c1) of row group g; lane = row.
template <int N, class Act>
__device__ __forceinline__ void wave_task(const MatDesc& m, int g, int c0, int c1, float (&acc)[N], Act& act) {
    const int lane = threadIdx.x & 63;
    float pa[N], pb[N];
#pragma unroll
    for (int t = 0; t < N; ++t) acc[t] = pa[t] = pb[t] = 0.0f;
    if (g >= m.G || c0 >= c1) return;
    const uint8_t* wp = m.w + ((size_t)g * m.C + c0) * kChunkBytes + lane * kBlockNibBytes;
    auto seg_end = [&](int c) {  // after chunk c: close the segment if it ends here
        if (c + 1 == c1 || (c + 1 - c0) % kSegChunks == 0) {
#pragma unroll
            for (int t = 0; t < N; ++t) {
                acc[t] += pa[t] + pb[t];
                pa[t] = pb[t] = 0.0f;
            }
        }
    };
    // The steady-state body prefetches unconditionally so that every path
    // reaching a chunk's use has the same loads outstanding (a conditional
    // prefetch makes the compiler wait for all loads, the prefetch included).
    Chunk a, b;
    load_chunk(a, wp);
    act.load(0, c0);
    int c = c0;
    for (; c + 2 < c1; c += 2, wp += 2 * kChunkBytes) {
        load_chunk(b, wp + kChunkBytes);
        act.load(1, c + 1);
        chunk_fma<N>(m, c, a, pa, pb, act, 0);
        seg_end(c);
        load_chunk(a, wp + 2 * kChunkBytes);
        act.load(0, c + 2);
        chunk_fma<N>(m, c + 1, b, pa, pb, act, 1);
        seg_end(c + 1);
    }
    if (c + 1 < c1) {  // two chunks left
        load_chunk(b, wp + kChunkBytes);
        act.load(1, c + 1);
        chunk_fma<N>(m, c, a, pa, pb, act, 0);
        seg_end(c);
        chunk_fma<N>(m, c + 1, b, pa, pb, act, 1);
        seg_end(c + 1);
    } else {           // one chunk left
        chunk_fma<N>(m, c, a, pa, pb, act, 0);
        seg_end(c);
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
template <int N>
__global__ __launch_bounds__(kThreads, N == 1 ? 1 : 2) void k_sweep(const MatDesc* __restrict__ mats,
                                                    const uint32_t* __restrict__ tiles) {
    __shared__ TileLds<N> l;
    const uint32_t mi = tiles[2 * (size_t)blockIdx.x];
    const uint32_t gs = tiles[2 * (size_t)blockIdx.x + 1];
    const MatDesc m = mats[mi];
    run_any<N>(m, gs, l);
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
__device__ __forceinline__ void quant_block8(const float* x, int8_t* q, uint16_t* d, bool valid) {
    const int o = threadIdx.x & 7;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid) v = *gp<f32x4>(x + 4 * o);
    const float a = quant8_amax(v);
    if (!valid) return;
    uint32_t packed;
    uint16_t h;
    quant8_codes(v, a, packed, h);
    *gwr<uint32_t>(q + 4 * o) = packed;
    if (o == 0) *gwr<uint16_t>(d) = h;
}

// Block lb (row-major over [n][nb]) of one activation; the lanes of a row's
// last block also zero the row's padding entries of d_x.
__device__ __forceinline__ void quant_local(const QuantDesc& qd, int64_t lb, bool valid) {
    const int nb = qd.cols / 32;
    const int64_t t = valid ? lb / nb : 0;
    const int64_t b = valid ? lb - t * nb : 0;
    const int64_t off = t * qd.cols + b * 32;
    quant_block8(qd.x + off, qd.q + off, qd.d + t * qd.dstride + b, valid);
    const int o = threadIdx.x & 7;
    if (valid && b == nb - 1 && o < qd.dstride - nb) gwr<uint16_t>(qd.d)[t * qd.dstride + nb + o] = 0;
}

// Standalone quantization: 32 blocks per 256-thread workgroup.
__global__ __launch_bounds__(256) void k_quantize(QuantDesc qd, int64_t total_blocks) {
    const int64_t lb = (int64_t)blockIdx.x * kQuantTileBlocks + (threadIdx.x >> 3);
    quant_local(qd, lb, lb < total_blocks);
}

// Batched quantization for the sweep: workgroup i takes tile i = (activation,
// first block) of a host-built table and quantizes up to kQuantTileBlocks
// consecutive blocks of that activation, one block per 8 lanes.
__global__ __launch_bounds__(256) void k_quantize_batch(const QuantDesc* __restrict__ descs,
                                                        const uint32_t* __restrict__ tiles) {
    const uint32_t di = tiles[2 * (size_t)blockIdx.x];
    const uint32_t b0 = tiles[2 * (size_t)blockIdx.x + 1];
    const QuantDesc qd = descs[di];
    const int64_t total = (int64_t)qd.n * (qd.cols / 32);
    const int64_t lb = (int64_t)b0 + (threadIdx.x >> 3);
    quant_local(qd, lb, lb < total);
}

// ---------------------------------------------------------------- fused 1-row sweep
//
// With one activation row the sweep quantizes inside the GEMV launch (the
// pages' mega kernel quantizes the activation once per step inside its single
// kernel, milestone M15): every wave quantizes the chunks it streams (see
// ActQuant), so the bytes -- and the results -- equal those of a separate
// quantize launch, and the group-0 waves publish them to x_q8.
__global__ __launch_bounds__(kThreads, 1) void k_sweep_fused(const MatDesc* __restrict__ mats,
                                                            const uint32_t* __restrict__ tiles) {
    __shared__ float red[kWaves * 64];
    const uint32_t mi = tiles[2 * (size_t)blockIdx.x];
    const uint32_t gs = tiles[2 * (size_t)blockIdx.x + 1];
    const MatDesc m = mats[mi];
    run_tile_with<1>(m, gs, red, [&](int g, int c0, int c1, float (&acc)[1]) {
        ActQuant act{m, g == 0, {}};
        wave_task<1>(m, g, c0, c1, acc, act);
    });
}

// ---------------------------------------------------------------- chained step
//
// One decode step's layers as dependent phases in one persistent cooperative
// launch, as the pages' mega kernel runs a token ("How it works", src/mega.cu
// bullet; milestones M15 and M19): per layer the q/k/v GEMVs share one Q8_0
// activation of the normalized layer input, the output projection reads q,
// gate and up share one activation of the normalized residual stream, and down
// reads their product; the residual adds ride in the output projections'
// epilogues.  The norm (RMS, no learned weight, fixed-order sum of squares)
// and the quantization run in every wave's prologue on the activation blocks
// it streams, so a phase starts with its weight loads in flight.
//
// A wave's GEMV is the lane-per-row task of the sweep (same chains, segments
// and K splits), so every output is bit-identical to the standalone GEMV of
// the same Q8_0 activation.  Workgroups take the tiles of a phase round-robin,
// starting where the previous phase's tiles ended, so phase p+1's tiles land
// on workgroups that had none in phase p.
//
// Activations that cross phases are tagged words (fp32 bits | step tag << 32).
// Phases are separated by
//  * kChainCounter: milestone M19's monotonic arrival counter -- one
//    device-scope release add per workgroup, polls, one acquire fence;
//  * kChainTree: a combining tree of such counters (16 sub-counters, the last
//    arrival of each adds to a top counter whose last arrival releases);
//  * kChainTagged: no barrier -- outputs are stored as relaxed device-scope
//    atomic words and every reader polls the words it needs until they carry
//    this step's tag.  Each word is its own flag, so no fence is needed; this
//    avoids the per-workgroup L2 write-back and invalidate that device-scope
//    release and acquire cost on the multi-XCD chip.
// Every wait is bounded: past the limit the error word is set, every other
// wait then gives up within ~1000 polls, and the launch runs to its end with
// whatever values it has.

constexpr int64_t kChainSpin = 1 << 20;

__device__ __forceinline__ uint64_t tag_word(float v, uint32_t gen) {
    return ((uint64_t)gen << 32) | (uint64_t)__float_as_uint(v);
}

template <int kSync>
__device__ __forceinline__ uint64_t chain_ld(const uint64_t* p) {
    if constexpr (kSync == kChainTagged)
        return __hip_atomic_load((const Q4S_GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *gp<uint64_t>(p);
}

template <int kSync>
__device__ __forceinline__ void chain_st(uint64_t* p, uint64_t w) {
    if constexpr (kSync == kChainTagged)
        __hip_atomic_store((Q4S_GLOBAL uint64_t*)p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *gwr<uint64_t>(p) = w;
}

__device__ __forceinline__ bool chain_failed(const uint32_t* err) {
    return __hip_atomic_load((const Q4S_GLOBAL uint32_t*)err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ void chain_fail(uint32_t* err) {
    __hip_atomic_fetch_or((Q4S_GLOBAL uint32_t*)err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The value of word w (read from p): with tagged phases, poll p until it
// carries this step's tag; after a barrier the tag is only checked.
template <int kSync>
__device__ __forceinline__ float chain_value(const uint64_t* p, uint64_t w, uint32_t gen, uint32_t* err) {
    if constexpr (kSync == kChainTagged) {
        int64_t spins = 0;
        while ((uint32_t)(w >> 32) != gen) {
            // give up past the limit, or at once once any other wait has given up
            if (++spins > kChainSpin || ((spins & 1023) == 0 && chain_failed(err))) {
                chain_fail(err);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            w = chain_ld<kSync>(p);
        }
    } else if ((uint32_t)(w >> 32) != gen) {
        chain_fail(err);
    }
    return __uint_as_float((uint32_t)w);
}

constexpr int kChainMaxChunks = 32;  // chunks of one wave's K range (its LDS slice)
constexpr int kChainBatch = 6;       // chunks per prologue load batch (a 1536-wide vector in one)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define Q4S_LDS __attribute__((address_space(3)))

// Lane's words of chunks [b0, b0 + cnt) (cnt <= kChainBatch) of a tagged
// activation, element 256c + 4 lane + k clamped to the vector; with tagged
// phases every word is re-read until all carry this step's tag.
template <int kSync>
__device__ __forceinline__ void chain_batch(const uint64_t* x, int n, int b0, int cnt, uint32_t gen, uint32_t* err,
                                            uint64_t (&w)[kChainBatch][4]) {
    const int lane = threadIdx.x & 63;
    auto load_all = [&]() {
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
                const int i = min((b0 + cc) * 256 + 4 * lane, n - 4);
#pragma unroll
                for (int k = 0; k < 4; ++k) w[cc][k] = chain_ld<kSync>(x + i + k);
            }
    };
    auto all_tagged = [&]() {
        bool ok = true;
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
#pragma unroll
                for (int k = 0; k < 4; ++k) ok = ok && (uint32_t)(w[cc][k] >> 32) == gen;
            }
        return ok;
    };
    if constexpr (kSync == kChainTagged) {
        int64_t spins = 0;
        for (;;) {
            load_all();
            if (all_tagged()) break;
            if (++spins > kChainSpin || ((spins & 1023) == 0 && chain_failed(err))) {
                chain_fail(err);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    } else {
        load_all();
        if (!all_tagged()) chain_fail(err);
    }
}

// Values of chunks [b0, b0 + cnt): x (fp32 or tagged), times x2 when given.
// What the prologue reads: the activation (fp32 or tagged), the optional second
// factor, and the vector length.
struct ChainSrc {
    const void* x;
    const uint64_t* x2;
    int x_plain, n;
};

template <int kSync>
__device__ __forceinline__ void chain_values(const ChainSrc& cm, int b0, int cnt, uint32_t gen, uint32_t* err,
                                             float (&v)[kChainBatch][4]) {
    const int lane = threadIdx.x & 63;
    const int n = cm.n;
    if (cm.x_plain) {
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
                const f32x4 f = *gp<f32x4>((const float*)cm.x + min((b0 + cc) * 256 + 4 * lane, n - 4));
#pragma unroll
                for (int k = 0; k < 4; ++k) v[cc][k] = f[k];
            }
    } else {
        uint64_t w[kChainBatch][4];
        chain_batch<kSync>((const uint64_t*)cm.x, n, b0, cnt, gen, err, w);
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
#pragma unroll
            for (int k = 0; k < 4; ++k) v[cc][k] = __uint_as_float((uint32_t)w[cc][k]);
    }
    if (cm.x2) {
        uint64_t w[kChainBatch][4];
        chain_batch<kSync>(cm.x2, n, b0, cnt, gen, err, w);
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
#pragma unroll
            for (int k = 0; k < 4; ++k) v[cc][k] = v[cc][k] * __uint_as_float((uint32_t)w[cc][k]);
    }
}

// Quantizes chunk c (the lane's 4 values) into the wave's LDS slice entry.
__device__ __forceinline__ void chain_quant(f32x4 v, int c, int nb, Q4S_LDS u32x2* dst) {
    const int lane = threadIdx.x & 63;
    if (c * kChunkBlocks + (lane >> 3) >= nb) v = (f32x4){0.f, 0.f, 0.f, 0.f};  // past the row
    const float a = quant8_amax(v);
    uint32_t packed;
    uint16_t h;
    quant8_codes(v, a, packed, h);
    dst[lane] = (u32x2){packed, __float_as_uint(__half2float(__ushort_as_half(h)))};
}

// Prologue of a chained-step wave that streams chunks [c0, c1): waits for the
// activation, takes the RMS norm of the whole vector when asked, and leaves
// the Q8_0 codes and scales of its chunks in its LDS slice ([chunk][lane]).
// The norm divisor is sqrt(ss / n + 1e-6) with ss from 64 lane partials
// (fmaf chains over elements 256c + 4 lane + k, chunk by chunk) and the xor
// butterfly 32, 16, ..., 1 -- every lane ends with the same ss, since each
// step adds the same two values on both lanes.
template <int kSync>
__device__ __noinline__ void chain_stage(const void* x, const uint64_t* x2, int x_plain, int norm, int n, int c0,
                                         int c1, uint32_t gen, uint32_t* err, Q4S_LDS u32x2* slice) {
    const int lane = threadIdx.x & 63;
    const ChainSrc cm{x, x2, x_plain, n};
    const int nb = n / 32;
    const int nc = (nb + kChunkBlocks - 1) / kChunkBlocks;
    float v[kChainBatch][4];
    float s = 1.0f;
    if (norm) {
        float p = 0.0f;
        for (int b0 = 0; b0 < nc; b0 += kChainBatch) {
            const int cnt = min(kChainBatch, nc - b0);
            chain_values<kSync>(cm, b0, cnt, gen, err, v);
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (cc < cnt && (b0 + cc) * 256 + 4 * lane + k < n) p = fmaf(v[cc][k], v[cc][k], p);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) p = p + __shfl_xor(p, d);
        s = sqrtf(p / (float)n + 1e-6f);
        if (nc <= kChainBatch && c0 == 0 && c1 == nc) {  // the last batch was the whole range: reuse it
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
                if (cc < nc)
                    chain_quant((f32x4){v[cc][0] / s, v[cc][1] / s, v[cc][2] / s, v[cc][3] / s}, cc, nb,
                                slice + cc * 64);
            return;
        }
    }
    for (int b0 = c0; b0 < c1; b0 += kChainBatch) {
        const int cnt = min(kChainBatch, c1 - b0);
        chain_values<kSync>(cm, b0, cnt, gen, err, v);
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
                f32x4 f = (f32x4){v[cc][0], v[cc][1], v[cc][2], v[cc][3]};
                if (norm) f = (f32x4){f[0] / s, f[1] / s, f[2] / s, f[3] / s};
                chain_quant(f, b0 + cc, nb, slice + (b0 + cc - c0) * 64);
            }
    }
}

// The activation source of a chained-step wave (see ActQuant): on first use
// the prologue stages the wave's whole range, after the first two chunks'
// weight loads are already in flight; every chunk then reads its codes and
// scales from LDS.
template <int kSync>
struct ActStaged {
    const ChainMat& cm;
    int64_t g;
    int c0, c1;
    uint32_t gen;
    uint32_t* err;
    Q4S_LDS u32x2* slice;
    bool staged;
    uint64_t* mark;  // NULL, or where to record when the first tile of the phase had its activation
    struct Prep {
        uint32_t packed;
        uint32_t dbits;
    };
    __device__ __forceinline__ void load(int, int) {}
    __device__ __forceinline__ Prep prepare(int, int c) {
        if (!staged) {
            // With tagged phases the wave usually waits here for the activation: touch the
            // weight chunks after the two already in flight (one dword per 128-byte line) so
            // that their loads after the wait hit this XCD's L2.  (After a barrier there is
            // no wait to hide the touches behind, and they only delay the first loads.)
            uint32_t touch = 0;
            if constexpr (kSync == kChainTagged) {
                const int lane = threadIdx.x & 63;
                const uint8_t* w0 = cm.m.w + ((size_t)g * cm.m.C + c0 + 2) * kChunkBytes;
                const int lines = max(c1 - c0 - 2, 0) * (kChunkBytes / 128);
                for (int i = lane; i < lines; i += 64) touch ^= *gp<uint32_t>(w0 + (size_t)i * 128);
            }
            chain_stage<kSync>(cm.x, cm.x2, cm.x_plain, cm.norm, cm.m.cols, c0, c1, gen, err, slice);
            if (gen == 0) err[2] = touch;  // never taken (tags start at 1); keeps the touches
            staged = true;
            if (mark && threadIdx.x == 0) gwr<uint64_t>(mark)[0] = __builtin_amdgcn_s_memrealtime();
        }
        const u32x2 e = slice[(c - c0) * 64 + (threadIdx.x & 63)];
        return {e[0], e[1]};
    }
    __device__ __forceinline__ u32x8 q(const Prep& p, int, int, int b) const {
        u32x8 r;
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = __builtin_amdgcn_readlane(p.packed, 8 * b + k);
        return r;
    }
    __device__ __forceinline__ float d(const Prep& p, int, int, int b) const {
        return __uint_as_float(__builtin_amdgcn_readlane(p.dbits, 8 * b));
    }
};

// One tile (group set) of a chained-step matrix: the GEMV as in run_tile_with,
// then the epilogue stores (tagged output, residual sum, plain logits).
template <int kSync>
__device__ __forceinline__ void chain_tile(const ChainMat& cm, int64_t gset, float* red, Q4S_LDS u32x2* stage,
                                           uint32_t gen, uint32_t* err, uint64_t* mark_start, uint64_t* mark_ready) {
    if (mark_start && threadIdx.x == 0) gwr<uint64_t>(mark_start)[0] = __builtin_amdgcn_s_memrealtime();
    const MatDesc& m = cm.m;
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ks = m.ks;
    const int gpw = kWaves / ks;
    const int64_t g = gset * gpw + wave / ks;
    const int sp = wave % ks;
    const int c0 = (int)((int64_t)sp * m.C / ks);
    const int c1 = (int)((int64_t)(sp + 1) * m.C / ks);
    float acc[1];
    // the residual word of the lane's row goes out now, long before the epilogue needs it
    const int64_t row = g * kGroupRows + lane;
    const int64_t rrow = min(row, (int64_t)m.rows - 1);
    uint64_t rword = 0;
    if (cm.res && !cm.res_plain && sp == 0 && g < m.G) rword = chain_ld<kSync>((const uint64_t*)cm.res + rrow);
    ActStaged<kSync> act{cm, g, c0, c1, gen, err, stage + wave * (kChainMaxChunks * 64), false, mark_ready};
    wave_task<1>(m, (int)g, c0, c1, acc, act);
    float v = acc[0];
    if (ks > 1) {
        red[wave * 64 + lane] = v;
        __syncthreads();
        if (sp != 0) return;
        v = red[wave * 64 + lane];
        for (int j = 1; j < ks; ++j) v += red[(wave + j) * 64 + lane];
    }
    if (g >= m.G || row >= m.rows) return;
    if (cm.y) chain_st<kSync>(cm.y + row, tag_word(v, gen));
    if (cm.yf) gwr<float>(cm.yf)[row] = v;
    if (cm.res) {
        const float r = cm.res_plain ? ((const float*)cm.res)[row]
                                     : chain_value<kSync>((const uint64_t*)cm.res + row, rword, gen, err);
        chain_st<kSync>(cm.y2 + row, tag_word(r + v, gen));
    }
}

// Phase barrier number k (1-based) of a launch; sync: [0] error word,
// [32] top counter, [64 + 32 i] sub-counter i.  Counters start at 0 per launch.
template <int kSync>
__device__ __forceinline__ void chain_barrier(uint32_t* sync, uint32_t k) {
    __syncthreads();
    if (threadIdx.x == 0) {
        Q4S_GLOBAL uint32_t* err = (Q4S_GLOBAL uint32_t*)sync;
        Q4S_GLOBAL uint32_t* top = (Q4S_GLOBAL uint32_t*)sync + 32;
        const uint32_t n = gridDim.x;
        Q4S_GLOBAL uint32_t* watch;
        uint32_t target;
        if constexpr (kSync == kChainCounter) {
            __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            watch = top;
            target = k * n;
        } else {
            const uint32_t fan = n < 16 ? n : 16;
            const uint32_t sub = blockIdx.x % fan;
            const uint32_t size = (n - sub + fan - 1) / fan;  // workgroups b < n with b mod fan == sub
            Q4S_GLOBAL uint32_t* mine = (Q4S_GLOBAL uint32_t*)sync + 64 + 32 * sub;
            const uint32_t old = __hip_atomic_fetch_add(mine, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == k * size) {
                const uint32_t t = __hip_atomic_fetch_add(top, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                if (t + 1 == k * fan)
                    __hip_atomic_store(err + 1, k, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);  // release word
            }
            watch = err + 1;
            target = k;
        }
        int64_t spins = 0;
        while (__hip_atomic_load(watch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > kChainSpin || ((spins & 1023) == 0 && chain_failed(sync))) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

template <int kSync>
__global__ __launch_bounds__(kThreads, 1) void k_chain(ChainParams P) {
    __shared__ float red[kWaves * 64];
    __shared__ u32x2 stage[kWaves * kChainMaxChunks * 64];
    const uint32_t nwg = gridDim.x, b = blockIdx.x;
    if (P.trace && threadIdx.x == 0)  // when this workgroup started, after the phase-end plane
        gwr<uint64_t>(P.trace)[(size_t)P.n_phases * nwg + b] = __builtin_amdgcn_s_memrealtime();
    uint32_t begin = 0;
    for (int p = 0; p < P.n_phases; ++p) {
        const uint32_t end = P.phase_end[p];
        const uint32_t j0 = (b + nwg - begin % nwg) % nwg;  // phase tiles start on workgroup begin mod nwg
        for (uint32_t j = j0; begin + j < end; j += nwg) {
            const uint32_t t = begin + j;
            const ChainMat cm = P.mats[P.tiles[2 * (size_t)t]];
            // timeline marks of the workgroup's first tile of the phase
            const size_t slot = (size_t)p * nwg + b, plane = (size_t)P.n_phases * nwg;
            uint64_t* ms = P.trace && j == j0 ? P.trace + plane + nwg + slot : nullptr;
            uint64_t* mr = P.trace && j == j0 ? P.trace + 2 * plane + nwg + slot : nullptr;
            chain_tile<kSync>(cm, P.tiles[2 * (size_t)t + 1], red, (Q4S_LDS u32x2*)stage, P.gen, P.sync, ms, mr);
            __syncthreads();
        }
        if (P.trace && threadIdx.x == 0)  // when this workgroup is done with the phase
            gwr<uint64_t>(P.trace)[(size_t)p * nwg + b] = __builtin_amdgcn_s_memrealtime();
        if constexpr (kSync != kChainTagged)
            if (p + 1 < P.n_phases) chain_barrier<kSync>(P.sync, (uint32_t)p + 1);
        begin = end;
    }
}

__global__ __launch_bounds__(256) void k_zero_words(uint32_t* w, int n) {
    for (int i = threadIdx.x; i < n; i += 256) w[i] = 0;
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
    const int64_t grid = (total + kQuantTileBlocks - 1) / kQuantTileBlocks;
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
static void sweep_n(const MatDesc* mats, const uint32_t* tiles, int64_t n_tiles, hipStream_t st) {
    hipLaunchKernelGGL(k_sweep<N>, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, mats, tiles);
}

hipError_t launch_sweep(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles, int n,
                        hipStream_t st) {
    if (n_tiles == 0 || n == 0) return hipSuccess;
    if (n > kTokTile) {
        const int tt = (n + kTokTile - 1) / kTokTile;
        hipLaunchKernelGGL(k_sweep_tiled, dim3(tiled_grid(tt, n_tiles)), dim3(kThreads), 0, st, dev_mats, dev_tiles,
                           tt, n_tiles);
        return hipGetLastError();
    }
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

hipError_t launch_sweep_fused(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles,
                              hipStream_t st) {
    if (n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sweep_fused, dim3((unsigned)n_tiles), dim3(kThreads), 0, st, dev_mats, dev_tiles);
    return hipGetLastError();
}

hipError_t launch_chain(int sync_mode, const ChainParams& p, int workgroups, hipStream_t st) {
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, st, p.sync, kChainSyncWords);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ChainParams a = p;
    void* args[] = {&a};
    const void* fn = sync_mode == kChainCounter ? (const void*)k_chain<kChainCounter>
                     : sync_mode == kChainTree  ? (const void*)k_chain<kChainTree>
                                                : (const void*)k_chain<kChainTagged>;
    return hipLaunchCooperativeKernel(fn, dim3(workgroups), dim3(kThreads), args, 0, st);
}

hipError_t chain_max_workgroups(int sync_mode, int* n) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const void* fn = sync_mode == kChainCounter ? (const void*)k_chain<kChainCounter>
                     : sync_mode == kChainTree  ? (const void*)k_chain<kChainTree>
                                                : (const void*)k_chain<kChainTagged>;
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0);
    *n = e == hipSuccess ? cus * per_cu : 0;
    return e;
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

hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const int64_t grid = std::min<int64_t>((n16 + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(k_bench_copy, dim3((unsigned)grid), dim3(256), 0, st, (const u32x4*)src,
                       (u32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace q4s
