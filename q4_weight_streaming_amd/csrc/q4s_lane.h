// The lane-per-row Q4_0 x Q8_0 GEMV core shared by the sweep kernels and the
// chained step: the chunk loads, the nibble unpack and per-block integer dot,
// the Q8_0 block quantizer, and the wave task that streams a row group's
// chunks in the fixed fp32 order (see the "GEMV core" note below).
#pragma once

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

// Codes held one dword per lane: where a wave quantizes a chunk itself, lane l
// holds code dword l of the chunk (block l/8, values 4(l%8) .. 4(l%8)+3).
// rows4 copies row j (lanes 16j .. 16j+15) of that register into every row of
// y[j] with the lane-swap instructions: a 32-lane swap of the register with
// itself gives [R0 R1 R0 R1] and [R2 R3 R2 R3], a 16-lane swap of each with
// itself gives [R0 R0 R0 R0], [R1 R1 R1 R1] and so on.  A DPP row_newbcast:n
// operand of y[j] then hands dword 16j + n to every lane, so block b's 8
// dwords are y[b/2] at n = 8(b%2) .. 8(b%2)+7.
__device__ __forceinline__ void rows4(uint32_t x, uint32_t (&y)[4]) {
    const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const auto a = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    y[0] = a[0];
    y[1] = a[1];
    y[2] = b[0];
    y[3] = b[1];
}

// block_dot16 for the four blocks 4h .. 4h+3 of a chunk, their codes taken
// from ya = rows4 register 2h (blocks 4h, 4h+1) and yb = register 2h+1 (blocks
// 4h+2, 4h+3) by row_newbcast operands; s[X] is block 4h+X's sum.  The compiler
// does not fold a DPP move into v_dot4c, so the 32 dots are written out.  A DPP
// instruction reads all of its VGPR operands two wait states after a VALU
// write becomes visible, the accumulator included: the four blocks' dots take
// turns, so each accumulator is read again three instructions after it was
// written, and the leading s_nop covers the operands the compiler wrote just
// before (five wait states, which also covers a VALU write of EXEC).  Integer
// sums, so the order of the dots does not change them.  The wait states are
// counted by hand, so only end-to-end results show a miscount; each user has a
// bit-exact test against the two-launch form or the fixed-order oracle:
//   the fused 1-row sweep's group sets and split tiles (test_gpu_sweep.py:
//     test_sweep_fused_quantize_equals_two_launches, test_qwen15_n1_full_parity;
//     test_gpu_fixed_order.py: test_single_split_sweep_equals_fixed_order_oracle),
//   the lone head's 8-wave split tiles (test_lm_head_fused_sweep_full_parity),
//   the Q8_0 head quantizing in the same launch (test_gpu_q8w.py:
//     test_gemv_q8_from_f32_equals_two_launches, test_gemv_q8_from_f32_lm_head_full),
//   the chained step's GEMVs (test_gpu_chain.py: test_chain_small_bit_exact,
//     test_chain_small_against_definition).
#define Q4S_DOT_BCAST(acc, y, w, n) \
    "v_dot4c_i32_i8_dpp %" #acc ", %" #y ", %" #w " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
#define Q4S_DOT_ROUND(wa, wb, wc, wd, n, n8) \
    Q4S_DOT_BCAST(0, 4, wa, n) Q4S_DOT_BCAST(1, 4, wb, n8) Q4S_DOT_BCAST(2, 5, wc, n) Q4S_DOT_BCAST(3, 5, wd, n8)
__device__ __forceinline__ void quad_dot16_rows(const Unpacked (&u)[4], uint32_t ya, uint32_t yb, int (&s)[4]) {
    s[0] = s[1] = s[2] = s[3] = 0;
    asm("s_nop 4\n"
        Q4S_DOT_ROUND(6, 14, 22, 30, 0, 8) Q4S_DOT_ROUND(7, 15, 23, 31, 1, 9)
        Q4S_DOT_ROUND(8, 16, 24, 32, 2, 10) Q4S_DOT_ROUND(9, 17, 25, 33, 3, 11)
        Q4S_DOT_ROUND(10, 18, 26, 34, 4, 12) Q4S_DOT_ROUND(11, 19, 27, 35, 5, 13)
        Q4S_DOT_ROUND(12, 20, 28, 36, 6, 14) Q4S_DOT_ROUND(13, 21, 29, 37, 7, 15)
        : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3])
        : "v"(ya), "v"(yb),
          "v"(u[0].lo[0]), "v"(u[0].lo[1]), "v"(u[0].lo[2]), "v"(u[0].lo[3]),
          "v"(u[0].hi[0]), "v"(u[0].hi[1]), "v"(u[0].hi[2]), "v"(u[0].hi[3]),
          "v"(u[1].lo[0]), "v"(u[1].lo[1]), "v"(u[1].lo[2]), "v"(u[1].lo[3]),
          "v"(u[1].hi[0]), "v"(u[1].hi[1]), "v"(u[1].hi[2]), "v"(u[1].hi[3]),
          "v"(u[2].lo[0]), "v"(u[2].lo[1]), "v"(u[2].lo[2]), "v"(u[2].lo[3]),
          "v"(u[2].hi[0]), "v"(u[2].hi[1]), "v"(u[2].hi[2]), "v"(u[2].hi[3]),
          "v"(u[3].lo[0]), "v"(u[3].lo[1]), "v"(u[3].lo[2]), "v"(u[3].lo[3]),
          "v"(u[3].hi[0]), "v"(u[3].hi[1]), "v"(u[3].hi[2]), "v"(u[3].hi[3]));
}
#undef Q4S_DOT_ROUND
#undef Q4S_DOT_BCAST

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
// Inputs are finite.
//
// quant8_amax is called by all 8 lanes of a block.  The magnitudes are
// compared as integers (for non-negative finite floats the bit patterns order
// as the values do) and move between lanes by DPP: swap neighbours, swap
// pairs, then the mirror within 8 lanes, which pairs each quad with the other.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kCtrl, 0xF, 0xF, true);
}
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i <- lane 7-i within 8
__device__ __forceinline__ float quant8_amax(const f32x4& v) {
    uint32_t a = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) a = max(a, __float_as_uint(v[k]) & 0x7FFFFFFFu);
    a = max(a, dpp_move<kDppQuadSwap1>(a));
    a = max(a, dpp_move<kDppQuadSwap2>(a));
    a = max(a, dpp_move<kDppHalfMirror>(a));
    return __uint_as_float(a);
}

// d = RN(a / 127) without a division: q = RN(a * RN(1/127)) is within one ulp
// of a/127, the residual a - 127 q is exact in one fma, and RN(q + r RN(1/127))
// is then the correctly rounded quotient (Markstein's theorem).  Every step
// scales exactly by powers of two while the operands stay normal, so checking
// every a in [1, 2) covers the guarded range; outside it the division is done.
__device__ __forceinline__ float quant8_scale(float a) {
    if (!(a >= 0x1p-96f && a <= 0x1p96f)) return a / 127.0f;
    constexpr float y = 1.0f / 127.0f;
    const float q = a * y;
    const float r = fmaf(-q, 127.0f, a);
    return fmaf(r, y, q);
}

// this lane's 4 quantized values (packed) and the block's binary16 d_x.
//
// roundf(RN(x / d)) is taken from the exact product x * rcp(d).  With rcp
// within one ulp of 1/d and |x/d| <= 127, the product is within 2^-16 of x/d
// and RN(x/d) within 2^-18 of it, so where the product lies more than 2^-13
// from every half-integer all three round to the same integer n.  One fma
// adds 1.5 * 2^23 to the product and rounds to an integer: the sum is 1.5 *
// 2^23 + n exactly, its low byte is n as a two's-complement byte, and a second
// fma gives the product's distance from n.  Lanes with any value within 2^-13
// of a half-integer, or with d too small or too large for rcp to stay normal,
// redo their values with the correctly rounded division.
__device__ __forceinline__ void quant8_codes(const f32x4& v, float a, uint32_t& packed, uint16_t& h) {
    const float dd = quant8_scale(a);
    packed = 0;
    if (a != 0.0f) {
        constexpr float kMagic = 0x1.8p23f;
        const float rc = __builtin_amdgcn_rcpf(dd);
        bool fast = dd >= 0x1p-125f && dd <= 0x1p125f;
        uint32_t s[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float m = fmaf(v[k], rc, kMagic);
            const float dist = fmaf(v[k], rc, -(m - kMagic));    // m - kMagic is exact
            fast = fast && fabsf(dist) < 0.5f - 0x1p-13f;
            s[k] = __float_as_uint(m);
        }
        packed = __builtin_amdgcn_perm(__builtin_amdgcn_perm(s[3], s[2], 0x0c0c0400u),
                                       __builtin_amdgcn_perm(s[1], s[0], 0x0c0c0400u), 0x05040100u);
        if (!fast) {
            packed = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) packed |= ((uint32_t)(uint8_t)(int8_t)(int)roundf(v[k] / dd)) << (8 * k);
        }
    }
    h = __half_as_ushort(__float2half_rn(dd));
}

// Where the lane-per-row path gets the Q8_0 activation.  load(slot, c) runs
// when chunk c's weight loads are issued (slot 0 or 1 follows the chunk
// buffer), prepare(slot, c) when chunk c is consumed; d gives block blk (b
// within the chunk) a scalar d_x.  Without kLaneCodes, q gives its codes as
// scalar operands; with it, Prep::packed holds the lane's code dword of the
// chunk and the dots take the codes through rows4 and quad_dot16_rows.
//
// ActGlobal: the planar buffer in global memory, through scalar loads.
struct ActGlobal {
    static constexpr bool kLaneCodes = false;
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
// quantizer's arithmetic -- and broadcasts the codes by lane swaps and DPP
// operands (rows4, quad_dot16_rows) and the scales with v_readlane.
// The activation load travels with the chunk's weight loads, so no barrier or
// prologue stands between the launch and the weight stream.  With `publish`
// (the waves of row group 0) the codes are also written to x_q8.
template <int kSlots>
struct ActQuantN {
    static constexpr bool kLaneCodes = true;   // Prep::packed is the lane's code dword
    const MatDesc& m;
    bool publish;
    f32x4 xs[kSlots];
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
    __device__ __forceinline__ float d(const Prep& p, int, int, int b) const {
        return __uint_as_float(__builtin_amdgcn_readlane(p.dbits, 8 * b));
    }
};
using ActQuant = ActQuantN<2>;

// Adds chunk `c` (held in ch) of the lane's row into the chains pa / pb.
template <int N, class Act>
__device__ __forceinline__ void chunk_fma(const MatDesc& m, int c, const Chunk& ch, float (&pa)[N],
                                          float (&pb)[N], Act& act, int slot) {
    const auto pr = act.prepare(slot, c);
    if constexpr (Act::kLaneCodes) {
        static_assert(N == 1, "lane-held codes carry one activation row");
        uint32_t y[4];
        rows4(pr.packed, y);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            Unpacked u[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) u[x] = unpack(ch.nib[4 * h + x]);
            int s16[4];
            quad_dot16_rows(u, y[2 * h], y[2 * h + 1], s16);
            float& p = h == 0 ? pa[0] : pb[0];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int b = 4 * h + x;
                const uint32_t sw = ch.scale[b >> 1];
                const float dw16 = ((b & 1) ? half_hi(sw) : half_lo(sw)) * 0.0625f;
                p = fmaf(dw16 * act.d(pr, 0, 0, b), (float)s16[x], p);
            }
        }
    } else {
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

}  // namespace
}  // namespace q4s
