// gfx950 kernel of libq4stream's chained decode step: a token's layers as
// dependent phases of one persistent cooperative launch (see below), on the
// lane-per-row GEMV core of the sweep.
#include "q4s_chain.h"
#include "q4s_lane.h"

namespace q4s {
namespace {

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
// Every wait is bounded: past the limit (2^20 polls unless the caller sets
// another) the error word is set, every other wait then gives up within ~1000
// polls, and the launch runs to its end with whatever values it has.

// The poll limit of this launch: sync word 3, written by the clearing launch
// before it (q4s_chain_set_wait_limit; 2^20 polls unless set).
__device__ __forceinline__ int64_t chain_spin_limit(const uint32_t* sync) {
    return (int64_t)*gp<uint32_t>(sync + 3);
}

__device__ __forceinline__ uint64_t tag_bits(uint32_t bits, uint32_t gen) {
    return ((uint64_t)gen << 32) | (uint64_t)bits;
}

__device__ __forceinline__ uint64_t tag_word(float v, uint32_t gen) { return tag_bits(__float_as_uint(v), gen); }

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
        const int64_t limit = chain_spin_limit(err);
        int64_t spins = 0;
        while ((uint32_t)(w >> 32) != gen) {
            // give up past the limit, or at once once any other wait has given up
            if (++spins > limit || ((spins & 1023) == 0 && chain_failed(err))) {
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

// A norm phase's input vector, read from global memory once per workgroup: the
// first wave of the workgroup to stage it in a phase claims it (an LDS max on
// the phase number), loads and polls it as every wave otherwise would, leaves
// it here as fp32 and publishes the phase number; the workgroup's other waves
// wait for that and take the vector from LDS.  (The waves of a workgroup are
// always in the same tile, so no later phase overwrites the copy while one of
// them reads it.)  With tagged phases only: there every wave otherwise polls
// the vector at device scope, past the L2 (after a barrier the L2 serves the
// other waves' reads).  Vectors longer than kChainNormShare are read by every wave.
constexpr int kChainNormShare = 4096;
__shared__ f32x4 chain_xs[kChainNormShare / 4];
__shared__ int chain_xs_claim, chain_xs_ready;  // the phase last claimed / published
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define Q4S_LDS __attribute__((address_space(3)))

// Lane's words of chunks [b0, b0 + cnt) (cnt <= kB) of a tagged activation x,
// and of x2 when given (both in one round of loads), element 256c + 4 lane + k
// clamped to the vector; with tagged phases every word is re-read until all
// carry this step's tag.  With `light`, a single word per lane is polled first
// (the lane's last word of the batch: one load per lane and round instead of
// the whole batch, so waiting waves do not crowd the producers' memory
// channels); a stage's later batches skip it, since their words were most
// likely written by the time its first batch was.
template <int kSync, int kB>
__device__ __forceinline__ void chain_batch(const uint64_t* x, const uint64_t* x2, int n, int b0, int cnt,
                                            uint32_t gen, uint32_t* err, bool light, uint64_t (&w)[kB][4],
                                            uint64_t (&w2)[kB][4]) {
    const int lane = threadIdx.x & 63;
    auto load_all = [&]() {
#pragma unroll
        for (int cc = 0; cc < kB; ++cc)
            if (cc < cnt) {
                const int i = min((b0 + cc) * 256 + 4 * lane, n - 4);
#pragma unroll
                for (int k = 0; k < 4; ++k) w[cc][k] = chain_ld<kSync>(x + i + k);
                if (x2) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) w2[cc][k] = chain_ld<kSync>(x2 + i + k);
                }
            }
    };
    auto all_tagged = [&]() {
        bool ok = true;
#pragma unroll
        for (int cc = 0; cc < kB; ++cc)
            if (cc < cnt) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ok = ok && (uint32_t)(w[cc][k] >> 32) == gen;
                    if (x2) ok = ok && (uint32_t)(w2[cc][k] >> 32) == gen;
                }
            }
        return ok;
    };
    if constexpr (kSync == kChainTagged) {
        const int64_t limit = chain_spin_limit(err);
        int64_t spins = 0;
        if (light) {
            const uint64_t* last = x2 ? x2 : x;
            const int i = min((b0 + cnt - 1) * 256 + 4 * lane, n - 4) + 3;
            while ((uint32_t)(chain_ld<kSync>(last + i) >> 32) != gen) {
                if (++spins > limit || ((spins & 1023) == 0 && chain_failed(err))) break;
                __builtin_amdgcn_s_sleep(2);
            }
        }
        for (;;) {
            load_all();
            if (all_tagged()) break;
            if (++spins > limit || ((spins & 1023) == 0 && chain_failed(err))) {
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

template <int kSync, int kB>
__device__ __forceinline__ void chain_values(const ChainSrc& cm, int b0, int cnt, uint32_t gen, uint32_t* err,
                                             bool light, float (&v)[kB][4]) {
    const int lane = threadIdx.x & 63;
    const int n = cm.n;
    if (cm.x_plain) {
#pragma unroll
        for (int cc = 0; cc < kB; ++cc)
            if (cc < cnt) {
                const f32x4 f = *gp<f32x4>((const float*)cm.x + min((b0 + cc) * 256 + 4 * lane, n - 4));
#pragma unroll
                for (int k = 0; k < 4; ++k) v[cc][k] = f[k];
            }
        return;
    }
    uint64_t w[kB][4], w2[kB][4];
    chain_batch<kSync, kB>((const uint64_t*)cm.x, cm.x2, n, b0, cnt, gen, err, light, w, w2);
#pragma unroll
    for (int cc = 0; cc < kB; ++cc)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[cc][k] = __uint_as_float((uint32_t)w[cc][k]);
            if (cm.x2) v[cc][k] = v[cc][k] * __uint_as_float((uint32_t)w2[cc][k]);
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

// The Q8_0 codes and scales of chunks [c0, c1) of an activation given as a
// paired matrix's tagged Q8_0 words (see ChainMat), polled like chain_batch,
// into the wave's LDS slice: lane l of chunk c takes code word 64c + l (its
// 4 values) and the d_x word of block 8c + l/8; lanes past the row take zeros,
// as the quantizer gives them.
template <int kSync>
__device__ __forceinline__ void chain_stage_q8(const uint64_t* xq, int n, int c0, int c1, uint32_t gen,
                                               uint32_t* err, Q4S_LDS u32x2* slice) {
    const int lane = threadIdx.x & 63;
    const int nb = n / 32;
    for (int b0 = c0; b0 < c1; b0 += kChainBatch) {
        const int cnt = min(kChainBatch, c1 - b0);
        uint64_t wq[kChainBatch], wd[kChainBatch];
        auto blk_of = [&](int cc) { return min((b0 + cc) * kChunkBlocks + (lane >> 3), nb - 1); };
        auto load_all = [&]() {
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
                if (cc < cnt) {
                    const int blk = blk_of(cc);
                    wq[cc] = chain_ld<kSync>(xq + blk * 8 + (lane & 7));
                    wd[cc] = chain_ld<kSync>(xq + n / 4 + blk);
                }
        };
        auto all_tagged = [&]() {
            bool ok = true;
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
                if (cc < cnt) ok = ok && (uint32_t)(wq[cc] >> 32) == gen && (uint32_t)(wd[cc] >> 32) == gen;
            return ok;
        };
        if constexpr (kSync == kChainTagged) {
            const int64_t limit = chain_spin_limit(err);
            int64_t spins = 0;
            if (b0 == c0) {  // light poll: the lane's last code word of the batch
                const uint64_t* last = xq + blk_of(cnt - 1) * 8 + (lane & 7);
                while ((uint32_t)(chain_ld<kSync>(last) >> 32) != gen) {
                    if (++spins > limit || ((spins & 1023) == 0 && chain_failed(err))) break;
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            for (;;) {
                load_all();
                if (all_tagged()) break;
                if (++spins > limit || ((spins & 1023) == 0 && chain_failed(err))) {
                    chain_fail(err);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        } else {
            load_all();
            if (!all_tagged()) chain_fail(err);
        }
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
                const bool valid = (b0 + cc) * kChunkBlocks + (lane >> 3) < nb;
                slice[(b0 + cc - c0) * 64 + lane] =
                    valid ? (u32x2){(uint32_t)wq[cc], (uint32_t)wd[cc]} : (u32x2){0u, 0u};
            }
    }
}

// Rows g*64 .. g*64+63 (lane = row) of a tile's output -- a paired tile's
// product y * y_b, or the output itself (q, read by o) -- as tagged Q8_0
// words: two 32-row blocks, each quantized as the block quantizer
// does (quant8_amax, quant8_scale, quant8_codes), one value per lane -- the
// block maximum over its 32 lanes, d = RN(max/127), the code from p * rcp(d)
// rounded through 1.5 * 2^23 where that is exact, else the correctly rounded
// division -- then four lanes' codes per word.  Called by a whole wave.
constexpr int kDppRowMirror = 0x140;  // row_mirror: lane i <- lane 15-i within 16
template <int kSync>
__device__ __forceinline__ void chain_store_q8(uint64_t* yq, int64_t rows, int64_t g, float p, uint32_t gen) {
    const int lane = threadIdx.x & 63;
    const int64_t row = g * kGroupRows + lane;
    const bool valid = row < rows;  // rows is a multiple of 32: uniform over each block
    if (!valid) p = 0.0f;
    uint32_t ab = __float_as_uint(p) & 0x7FFFFFFFu;
    ab = max(ab, dpp_move<kDppQuadSwap1>(ab));
    ab = max(ab, dpp_move<kDppQuadSwap2>(ab));
    ab = max(ab, dpp_move<kDppHalfMirror>(ab));
    ab = max(ab, dpp_move<kDppRowMirror>(ab));
    {   // 16-lane rows 2k and 2k+1 meet: the max of each 32-lane block
        const auto sw = __builtin_amdgcn_permlane16_swap(ab, ab, false, false);
        ab = max((uint32_t)sw[0], (uint32_t)sw[1]);
    }
    const float a = __uint_as_float(ab);
    const float dd = quant8_scale(a);
    uint32_t code = 0;
    if (a != 0.0f) {
        constexpr float kMagic = 0x1.8p23f;
        const float rc = __builtin_amdgcn_rcpf(dd);
        const float mg = fmaf(p, rc, kMagic);
        const float dist = fmaf(p, rc, -(mg - kMagic));
        if (dd >= 0x1p-125f && dd <= 0x1p125f && fabsf(dist) < 0.5f - 0x1p-13f)
            code = __float_as_uint(mg) & 0xFFu;
        else
            code = (uint32_t)(uint8_t)(int8_t)(int)roundf(p / dd);
    }
    // lane 4k gathers the codes of lanes 4k+1 .. 4k+3 (quad_perm broadcasts, no LDS permutes)
    const uint32_t word = code | (dpp_move<0x55>(code) << 8) | (dpp_move<0xAA>(code) << 16) |
                          (dpp_move<0xFF>(code) << 24);
    const uint32_t dbits = __float_as_uint(__half2float(__float2half_rn(dd)));
    if (valid && (lane & 3) == 0) chain_st<kSync>(yq + row / 4, tag_bits(word, gen));
    if (valid && (lane & 31) == 0) chain_st<kSync>(yq + rows / 4 + row / 32, tag_bits(dbits, gen));
}

// Row group vg of a tile's matrix: for a paired matrix group vg/2 of its first
// (vg even) or second (vg odd) matrix, else group vg.
__device__ __forceinline__ MatDesc chain_group(const ChainMat& cm, int64_t vg, int64_t& g, int& half) {
    MatDesc m = cm.m;
    if (cm.w2) {
        half = (int)(vg & 1);
        g = vg >> 1;
        if (half) m.w = cm.w2;
    } else {
        half = 0;
        g = vg;
    }
    return m;
}

// p + (p of lane ^ d) for d = 32, 16, 8, 4, 2, 1 in turn: the xor butterfly
// of __shfl_xor, every lane ending with the same sum (each step adds the same
// two values on both lanes of a pair), by lane swaps and DPP moves instead of
// LDS permutes, which a lone wave waits out one after another.  Called by a
// whole wave.
constexpr int kDppRowShl4 = 0x104;  // row_shl:4: lane i <- lane i + 4 within 16
constexpr int kDppRowShr4 = 0x114;  // row_shr:4: lane i <- lane i - 4 within 16
constexpr int kDppRowRor8 = 0x128;  // row_ror:8: lane i <- lane i ^ 8 within 16
__device__ __forceinline__ float wave_sum_xor(float p) {
    const int lane = threadIdx.x & 63;
    uint32_t v = __float_as_uint(p);
    auto step = [&](uint32_t a, uint32_t b) { v = __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); };
    auto sw32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // {own, lane ^ 32}
    step(sw32[0], sw32[1]);
    auto sw16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // {own, lane ^ 16}
    step(sw16[0], sw16[1]);
    step(v, dpp_move<kDppRowRor8>(v));
    const uint32_t up = dpp_move<kDppRowShl4>(v), down = dpp_move<kDppRowShr4>(v);
    step(v, (lane & 4) ? down : up);
    step(v, dpp_move<kDppQuadSwap2>(v));
    step(v, dpp_move<kDppQuadSwap1>(v));
    return __uint_as_float(v);
}

// The workgroup's copy of a norm phase's vector (nc chunks, nc * 256 <=
// kChainNormShare) in chain_xs: loaded by the wave that claims it, waited for
// by the others.  Called by a whole wave.
template <int kSync>
__device__ __forceinline__ void chain_norm_shared(const ChainSrc& cm, int nc, int phase, uint32_t gen,
                                                  uint32_t* err) {
    const int lane = threadIdx.x & 63;
    int prev = 0;
    if (lane == 0) prev = atomicMax(&chain_xs_claim, phase);
    if (__builtin_amdgcn_readfirstlane(prev) < phase) {  // the first wave here in this phase
        float v[kChainBatch][4];
        for (int b0 = 0; b0 < nc; b0 += kChainBatch) {
            const int cnt = min(kChainBatch, nc - b0);
            chain_values<kSync, kChainBatch>(cm, b0, cnt, gen, err, b0 == 0, v);
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
                if (cc < cnt) chain_xs[(b0 + cc) * 64 + lane] = (f32x4){v[cc][0], v[cc][1], v[cc][2], v[cc][3]};
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (lane == 0) __hip_atomic_store(&chain_xs_ready, phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        const int64_t limit = chain_spin_limit(err);
        int64_t spins = 0;
        while (__hip_atomic_load(&chain_xs_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < phase) {
            if (++spins > limit) {  // the loading wave's own waits are bounded, so this is not reached
                chain_fail(err);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
}

// The norm prologue from the workgroup's copy of the vector: the same sum of
// squares (lane partials over elements 256c + 4 lane + k, chunk by chunk, then
// the xor butterfly), divisor and quantization as the per-wave path in
// chain_stage.  Inlined into the tile code rather than added to chain_stage:
// as part of that called function it would push its register use past what a
// call may clobber, and every call would save registers to scratch memory.
template <int kSync>
__device__ __forceinline__ void chain_stage_norm_shared(ChainSrc cm, int nc, int c0, int c1, int phase,
                                                     uint32_t gen, uint32_t* err, Q4S_LDS u32x2* slice) {
    const int lane = threadIdx.x & 63;
    const int n = cm.n, nb = n / 32;
    chain_norm_shared<kSync>(cm, nc, phase, gen, err);
    float p = 0.0f;
    for (int cb = 0; cb < nc; cb += 2) {  // two chunks' reads issued before their fmafs
        f32x4 f[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) f[j] = chain_xs[min(cb + j, nc - 1) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (cb + j < nc && (cb + j) * 256 + 4 * lane < n) {
#pragma unroll
                for (int k = 0; k < 4; ++k) p = fmaf(f[j][k], f[j][k], p);
            }
    }
    p = wave_sum_xor(p);
    const float sn = sqrtf(p / (float)n + 1e-6f);
    for (int c = c0; c < c1; ++c) {
        const f32x4 f = chain_xs[c * 64 + lane];
        chain_quant((f32x4){f[0] / sn, f[1] / sn, f[2] / sn, f[3] / sn}, c, nb, slice + (c - c0) * 64);
    }
}

// Prologue of a chained-step wave that streams chunks [c0, c1): waits for the
// activation, takes the RMS norm of the whole vector when asked, and leaves
// the Q8_0 codes and scales of its chunks in its LDS slice ([chunk][lane]).
// The norm divisor is sqrt(ss / n + 1e-6) with ss from 64 lane partials
// (fmaf chains over elements 256c + 4 lane + k, chunk by chunk) and the xor
// butterfly 32, 16, ..., 1 -- every lane ends with the same ss, since each
// step adds the same two values on both lanes.
template <int kSync>
__device__ __noinline__ void chain_stage(const void* x, const uint64_t* x2, const uint64_t* xq, int x_plain, int norm,
                                         int n, int c0, int c1, uint32_t gen, uint32_t* err, Q4S_LDS u32x2* slice) {
    if (xq) {  // already quantized by the producing tiles
        chain_stage_q8<kSync>(xq, n, c0, c1, gen, err, slice);
        return;
    }
    const int lane = threadIdx.x & 63;
    const ChainSrc cm{x, x2, x_plain, n};
    const int nb = n / 32;
    const int nc = (nb + kChunkBlocks - 1) / kChunkBlocks;
    if (x2) {  // an elementwise product (no norm): both factors in batches of half the size
        constexpr int kB = kChainBatch / 2;
        float v[kB][4];
        for (int b0 = c0; b0 < c1; b0 += kB) {
            const int cnt = min(kB, c1 - b0);
            chain_values<kSync, kB>(cm, b0, cnt, gen, err, b0 == c0, v);
#pragma unroll
            for (int cc = 0; cc < kB; ++cc)
                if (cc < cnt) chain_quant((f32x4){v[cc][0], v[cc][1], v[cc][2], v[cc][3]}, b0 + cc, nb,
                                          slice + (b0 + cc - c0) * 64);
        }
        return;
    }
    float v[kChainBatch][4];
    float s = 1.0f;
    if (norm) {
        float p = 0.0f;
        for (int b0 = 0; b0 < nc; b0 += kChainBatch) {
            const int cnt = min(kChainBatch, nc - b0);
            chain_values<kSync, kChainBatch>(cm, b0, cnt, gen, err, b0 == 0, v);
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (cc < cnt && (b0 + cc) * 256 + 4 * lane + k < n) p = fmaf(v[cc][k], v[cc][k], p);
        }
        s = sqrtf(wave_sum_xor(p) / (float)n + 1e-6f);
        if (nc <= kChainBatch) {  // the one batch was the whole vector: quantize this wave's chunks from it
#pragma unroll
            for (int cc = 0; cc < kChainBatch; ++cc)
                if (cc >= c0 && cc < c1)
                    chain_quant((f32x4){v[cc][0] / s, v[cc][1] / s, v[cc][2] / s, v[cc][3] / s}, cc, nb,
                                slice + (cc - c0) * 64);
            return;
        }
    }
    for (int b0 = c0; b0 < c1; b0 += kChainBatch) {
        const int cnt = min(kChainBatch, c1 - b0);
        // after a norm pass every word has been seen tagged: no light poll
        chain_values<kSync, kChainBatch>(cm, b0, cnt, gen, err, !norm && b0 == c0, v);
#pragma unroll
        for (int cc = 0; cc < kChainBatch; ++cc)
            if (cc < cnt) {
                f32x4 f = (f32x4){v[cc][0], v[cc][1], v[cc][2], v[cc][3]};
                if (norm) f = (f32x4){f[0] / s, f[1] / s, f[2] / s, f[3] / s};
                chain_quant(f, b0 + cc, nb, slice + (b0 + cc - c0) * 64);
            }
    }
}

// What a wave's LDS slice holds: the Q8_0 codes of chunks [c0, c1) of phase
// `phase`'s activation (the matrices of a phase share one activation), so a
// workgroup's later tiles of a phase skip the prologue the first one ran.
struct StageKey {
    int phase, c0, c1;
};

// The activation source of a chained-step wave (see ActQuant): on first use
// the prologue stages the wave's whole range, after the first two chunks'
// weight loads are already in flight; every chunk then reads its codes and
// scales from LDS.
template <int kSync>
struct ActStaged {
    static constexpr bool kLaneCodes = true;   // Prep::packed is the lane's code dword
    const ChainMat& cm;
    const uint8_t* w;  // the row group's matrix (the second one of a paired matrix's odd groups)
    int64_t g;
    int c0, c1;
    uint32_t gen;
    uint32_t* err;
    Q4S_LDS u32x2* slice;
    StageKey& key;   // what the slice holds
    int phase;
    bool staged;
    uint64_t* mark;  // NULL, or where to record when the first tile of the phase had its activation
    uint64_t* dump;  // NULL, or where the phase's staged codes are copied ([chunk][lane] words)
    struct Prep {
        uint32_t packed;
        uint32_t dbits;
    };
    __device__ __forceinline__ void load(int, int) {}
    __device__ __forceinline__ Prep prepare(int, int c) {
        if (!staged && key.phase == phase && key.c0 == c0 && key.c1 == c1) staged = true;
        if (!staged) {
            // With tagged phases the wave usually waits here for the activation: touch the
            // weight chunks after the two already in flight (one dword per 128-byte line) so
            // that their loads after the wait hit this XCD's L2.  (After a barrier there is
            // no wait to hide the touches behind, and they only delay the first loads.)
            uint32_t touch = 0;
            if constexpr (kSync == kChainTagged) {
                const int lane = threadIdx.x & 63;
                const uint8_t* w0 = w + ((size_t)g * cm.m.C + c0 + 2) * kChunkBytes;
                const int lines = max(c1 - c0 - 2, 0) * (kChunkBytes / 128);
                for (int i = lane; i < lines; i += 64) touch ^= *gp<uint32_t>(w0 + (size_t)i * 128);
            }
            const int n = cm.m.cols, nc = (n / 32 + kChunkBlocks - 1) / kChunkBlocks;
            if (kSync == kChainTagged && cm.norm && !cm.xq && !cm.x2 && nc * 256 <= kChainNormShare)
                chain_stage_norm_shared<kSync>(ChainSrc{cm.x, nullptr, cm.x_plain, n}, nc, c0, c1, phase, gen, err,
                                               slice);  // from the workgroup's copy of the vector
            else
                chain_stage<kSync>(cm.x, cm.x2, cm.xq, cm.x_plain, cm.norm, n, c0, c1, gen, err, slice);
            if (gen == 0) err[2] = touch;  // never taken (tags start at 1); keeps the touches
            staged = true;
            key = {phase, c0, c1};
            if (dump) {  // test hook: the lane's code word and d_x bits of every staged chunk
                const int lane = threadIdx.x & 63;
                for (int cc = 0; cc < c1 - c0; ++cc) {
                    const u32x2 e = slice[cc * 64 + lane];
                    gwr<uint64_t>(dump)[(size_t)(c0 + cc) * 64 + lane] = ((uint64_t)e[1] << 32) | e[0];
                }
            }
            if (mark && threadIdx.x == 0) gwr<uint64_t>(mark)[0] = __builtin_amdgcn_s_memrealtime();
        }
        const u32x2 e = slice[(c - c0) * 64 + (threadIdx.x & 63)];
        return {e[0], e[1]};
    }
    __device__ __forceinline__ float d(const Prep& p, int, int, int b) const {
        return __uint_as_float(__builtin_amdgcn_readlane(p.dbits, 8 * b));
    }
};

// One tile (group set) of a chained-step matrix: the GEMV as in run_tile_with,
// then the epilogue stores (tagged output, residual sum, plain logits).
template <int kSync>
__device__ __forceinline__ void chain_tile(const ChainMat& cm, int64_t gset, float* red, Q4S_LDS u32x2* stage,
                                           StageKey& key, int phase, uint32_t gen, uint32_t* err,
                                           uint64_t* mark_start, uint64_t* mark_ready, uint64_t* dump) {
    if (mark_start && threadIdx.x == 0) gwr<uint64_t>(mark_start)[0] = __builtin_amdgcn_s_memrealtime();
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ks = cm.m.ks;
    const int gpw = kWaves / ks;
    int64_t g;
    int half;
    const MatDesc m = chain_group(cm, gset * gpw + wave / ks, g, half);
    const int sp = wave % ks;
    const int c0 = (int)((int64_t)sp * m.C / ks);
    const int c1 = (int)((int64_t)(sp + 1) * m.C / ks);
    float acc[1];
    // the residual word of the lane's row goes out now, long before the epilogue needs it
    const int64_t row = g * kGroupRows + lane;
    const int64_t rrow = min(row, (int64_t)m.rows - 1);
    uint64_t rword = 0;
    if (cm.res && !cm.res_plain && sp == 0 && g < m.G) rword = chain_ld<kSync>((const uint64_t*)cm.res + rrow);
    ActStaged<kSync> act{cm, m.w, g, c0, c1, gen, err, stage + wave * (kChainMaxChunks * 64), key, phase, false,
                         mark_ready, dump};
    wave_task<1>(m, (int)g, c0, c1, acc, act);
    float v = acc[0];
    if (ks > 1 || cm.w2) {
        red[wave * 64 + lane] = v;
        __syncthreads();
        if (sp != 0) return;
        // a row group's K ranges added in order; a pair's first half also forms its partner's
        auto total = [&](int w0) {
            float t = red[w0 * 64 + lane];
            for (int j = 1; j < ks; ++j) t += red[(w0 + j) * 64 + lane];
            return t;
        };
        v = total(wave);
        if (cm.w2 && half == 0 && g < m.G) chain_store_q8<kSync>(cm.yq, m.rows, g, v * total(wave + ks), gen);
    }
    if (cm.yq && !cm.w2 && g < m.G) chain_store_q8<kSync>(cm.yq, m.rows, g, v, gen);  // the output itself
    if (g >= m.G || row >= m.rows) return;
    uint64_t* y = half ? cm.y_b : cm.y;
    if (y) chain_st<kSync>(y + row, tag_word(v, gen));
    if (cm.yf) gwr<float>(cm.yf)[row] = v;
    if (cm.res) {
        const float r = cm.res_plain ? ((const float*)cm.res)[row]
                                     : chain_value<kSync>((const uint64_t*)cm.res + row, rword, gen, err);
        chain_st<kSync>(cm.y2 + row, tag_word(r + v, gen));
    }
}

// Row groups of a matrix with one or two K splits (at most 16 chunks) in a
// phase small enough to give each row group 4 waves (wpg = 4: one group per
// tile) or, for at most 8 chunks, 2 waves (wpg = 2: two groups per tile).  Wave lw of a group stages
// and multiplies chunks [ceil(lw C/wpg), ceil((lw+1) C/wpg)) and leaves each
// block's exact integer sum (as int16: |s| <= 32512) and its binary16 d_w in
// the group's term table, and its blocks' d_x in the d_x table; then K range r
// of the group runs on its waves 2r (chain A, blocks 0-3 of every chunk) and
// 2r + 1 (chain B, blocks 4-7) -- wave_task's chains, in its order, each term
// fmaf(d_w * d_x, s, p), the bits of wave_task's fmaf(d_w/16 * d_x, 16 s, p)
// -- and the ranges' 0 + (A + B) are added in order.  So the result is
// bit-identical to the one-wave-per-range tile, with 1/wpg of the integer work
// per wave.
constexpr int kChainSplitChunks = 16;  // chunks of a matrix with ks <= 2
constexpr int kChainTermWords = kChainSplitChunks * kChunkBlocks * 64;  // one group's term table
// the workgroup's term table: a split tile's group(s), or a K-range tile's range
constexpr int kChainTableWords =
    (kChainRangeChunks > kChainSplitChunks ? kChainRangeChunks : kChainSplitChunks) * kChunkBlocks * 64;
static_assert(kChainRangeChunks <= 4 * kSegChunks, "a K-range tile's segments fit the hand-off buffer");

template <int kWpg>
__device__ __forceinline__ int split_first(int w, int C) { return (w * C + kWpg - 1) / kWpg; }

// The fixed-order chains read each chunk's exact block sums and binary16 d_w
// (the term table) and its blocks' d_x (the d_x table, 8 floats per chunk,
// written by the wave that staged the chunk).  They read them kChainFold
// chunks at a time, every read of a batch issued before the first fmaf (read
// one after another, each read's latency adds up along the chain); a chunk
// past the range adds fmaf(0, s, p) == p (p is never -0), an exact no-op.
constexpr int kChainFold = 4;

// Table entries of blocks 4 hb .. 4 hb + 3 of chunks cb .. cb + kChainFold - 1
// (entry c - tbase; a chunk from c_end on reads chunk c_end - 1's, which the
// fold then leaves out).
__device__ __forceinline__ void chain_fetch(int cb, int c_end, int tbase, int hb, const Q4S_LDS uint32_t* terms,
                                            const Q4S_LDS f32x4* dx, uint32_t (&t)[kChainFold][4],
                                            f32x4 (&d)[kChainFold]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kChainFold; ++k) {
        const int e = min(cb + k, c_end - 1) - tbase;
#pragma unroll
        for (int x = 0; x < 4; ++x) t[k][x] = terms[(e * kChunkBlocks + 4 * hb + x) * 64 + lane];
        d[k] = dx[2 * e + hb];
    }
}

// p through the batch's first n chunks in order, one fmaf per block: the
// GEMV's fmaf(d_w/16 * d_x, 16 s, p) taken as fmaf(d_w * d_x, s, p).  Both
// scales have binary16 significands (11 bits), so d_w * d_x is exact in fp32,
// and so is its product with 1/16; the two fmafs see the same exact product
// and give the same bits, with fewer instructions on this serial path.
__device__ __forceinline__ void chain_fold(const uint32_t (&t)[kChainFold][4], const f32x4 (&d)[kChainFold], int n,
                                           float& p) {
#pragma unroll
    for (int k = 0; k < kChainFold; ++k)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const float m = half_hi(t[k][x]) * d[k][x];
            const float sv = (float)(int16_t)(t[k][x] & 0xffffu);
            p = fmaf(k < n ? m : 0.0f, sv, p);
        }
}

// A split tile's K range (at most 8 chunks) as one batch of exactly its
// chunks: every read issued before the first fmaf, no padding entries read or
// added (in batches of kChainFold the 1.5B step took 683 us and the 7B-shaped
// one 1.377 ms, in one exact batch 670 us and 1.370 ms; exact batches for the
// K-range tiles as well measured slower, 684 us and 1.403 ms).
template <int K>
__device__ __forceinline__ void chain_exact(int c0, int hb, const Q4S_LDS uint32_t* terms, const Q4S_LDS f32x4* dx,
                                            float& p) {
    const int lane = threadIdx.x & 63;
    uint32_t t[K][4];
    f32x4 d[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int x = 0; x < 4; ++x) t[k][x] = terms[((c0 + k) * kChunkBlocks + 4 * hb + x) * 64 + lane];
        d[k] = dx[2 * (c0 + k) + hb];
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const float m = half_hi(t[k][x]) * d[k][x];
            const float sv = (float)(int16_t)(t[k][x] & 0xffffu);
            p = fmaf(m, sv, p);
        }
}

// p through chunks c0 .. c0 + n - 1 (1 <= n <= 8) of the term table, in order
__device__ __forceinline__ void chain_range(int c0, int n, int hb, const Q4S_LDS uint32_t* terms,
                                            const Q4S_LDS f32x4* dx, float& p) {
    switch (n) {
        case 1: chain_exact<1>(c0, hb, terms, dx, p); break;
        case 2: chain_exact<2>(c0, hb, terms, dx, p); break;
        case 3: chain_exact<3>(c0, hb, terms, dx, p); break;
        case 4: chain_exact<4>(c0, hb, terms, dx, p); break;
        case 5: chain_exact<5>(c0, hb, terms, dx, p); break;
        case 6: chain_exact<6>(c0, hb, terms, dx, p); break;
        case 7: chain_exact<7>(c0, hb, terms, dx, p); break;
        default: chain_exact<8>(c0, hb, terms, dx, p); break;
    }
}

// Chunk c's exact block sums and binary16 d_w into entry tc of the term table,
// its blocks' d_x into entry tc of the d_x table.
template <int kSync>
__device__ __forceinline__ void chunk_terms(int c, int tc, const Chunk& ch, ActStaged<kSync>& act,
                                            Q4S_LDS uint32_t* terms, Q4S_LDS float* dx) {
    const int lane = threadIdx.x & 63;
    const auto pr = act.prepare(0, c);
    if ((lane & 7) == 0) dx[tc * kChunkBlocks + (lane >> 3)] = __uint_as_float(pr.dbits);  // lane 8 b: block b's d_x
    uint32_t y[4];
    rows4(pr.packed, y);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        Unpacked u[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) u[x] = unpack(ch.nib[4 * h + x]);
        int s16[4];
        quad_dot16_rows(u, y[2 * h], y[2 * h + 1], s16);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int b = 4 * h + x;
            const uint32_t sw = ch.scale[b >> 1];
            const uint32_t dw_bits = (b & 1) ? (sw >> 16) : (sw & 0xffffu);
            terms[(tc * kChunkBlocks + b) * 64 + lane] = (uint32_t)(uint16_t)(int16_t)(s16[x] >> 4) | (dw_bits << 16);
        }
    }
}

template <int kSync, int kWpg>
__device__ __forceinline__ void chain_tile_split(const ChainMat& cm, int64_t tile, float* red,
                                                 Q4S_LDS u32x2* stage, Q4S_LDS uint32_t* terms, Q4S_LDS float* dxt,
                                                 StageKey& key, int phase, uint32_t gen, uint32_t* err,
                                                 uint64_t* mark_start, uint64_t* mark_ready, uint64_t* dump) {
    if (mark_start && threadIdx.x == 0) gwr<uint64_t>(mark_start)[0] = __builtin_amdgcn_s_memrealtime();
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int gi = wave / kWpg, lw = wave % kWpg;  // the wave's group within the tile, its place in the group
    int64_t g;
    int half;
    const MatDesc m = chain_group(cm, tile * (kWaves / kWpg) + gi, g, half);
    const int C = m.C, ks = m.ks;
    const bool live = g < m.G;
    // one group's table takes all kChainTermWords (<= 16 chunks); two groups (<= 8 chunks each) halve it
    Q4S_LDS uint32_t* gterms = terms + gi * (kChainTermWords / 2);
    Q4S_LDS float* gdx = dxt + gi * (kChainSplitChunks * kChunkBlocks / 2);
    const int64_t row = g * kGroupRows + lane;
    const int64_t rrow = min(row, (int64_t)m.rows - 1);
    uint64_t rword = 0;
    if (cm.res && !cm.res_plain && lw == 0 && live) rword = chain_ld<kSync>((const uint64_t*)cm.res + rrow);
    // integer work of this wave's chunks
    const int i0 = split_first<kWpg>(lw, C), i1 = split_first<kWpg>(lw + 1, C);
    if (live && i0 < i1) {
        Q4S_LDS u32x2* slice = stage + wave * (kChainMaxChunks * 64);
        ActStaged<kSync> act{cm, m.w, g, i0, i1, gen, err, slice, key, phase, false, wave == 0 ? mark_ready : nullptr,
                             dump};
        const uint8_t* wp = m.w + ((size_t)g * m.C + i0) * kChunkBytes + lane * kBlockNibBytes;
        Chunk a, b;
        load_chunk(a, wp);
        if (i0 + 1 < i1) load_chunk(b, wp + kChunkBytes);
        for (int c = i0; c < i1; c += 2) {
            chunk_terms<kSync>(c, c, a, act, gterms, gdx);
            if (c + 2 < i1) load_chunk(a, wp + (size_t)(c + 2 - i0) * kChunkBytes);
            if (c + 1 < i1) {
                chunk_terms<kSync>(c + 1, c + 1, b, act, gterms, gdx);
                if (c + 3 < i1) load_chunk(b, wp + (size_t)(c + 3 - i0) * kChunkBytes);
            }
        }
    }
    __syncthreads();
    // the fixed-order fp32 chains: K range r of a group on its waves 2r (chain A, blocks 0-3 of
    // every chunk) and 2r + 1 (chain B, blocks 4-7); a range of <= 8 chunks is one segment
    const int r = lw >> 1, hb = lw & 1;
    if (live && r < ks) {
        const int c0 = (int)((int64_t)r * C / ks), c1 = (int)((int64_t)(r + 1) * C / ks);
        float p = 0.0f;
        if (c1 - c0 <= 8) {  // always, for ks <= 2 and C <= 16
            chain_range(c0, __builtin_amdgcn_readfirstlane(c1 - c0), hb, gterms, (const Q4S_LDS f32x4*)gdx, p);
        } else {
            for (int cb = c0; cb < c1; cb += kChainFold) {
                uint32_t t[kChainFold][4];
                f32x4 d[kChainFold];
                chain_fetch(cb, c1, 0, hb, gterms, (const Q4S_LDS f32x4*)gdx, t, d);
                chain_fold(t, d, c1 - cb, p);
            }
        }
        red[wave * 64 + lane] = p;
    }
    __syncthreads();
    if (!live || lw != 0) return;
    // a row group's K ranges added in order, each 0 + (A + B); a pair's first half also forms
    // its partner's
    auto total = [&](int w0) {
        float t = 0.0f;
        for (int j = 0; j < ks; ++j) {
            float a = 0.0f;
            a += red[(w0 + 2 * j) * 64 + lane] + red[(w0 + 2 * j + 1) * 64 + lane];
            t = j == 0 ? a : t + a;
        }
        return t;
    };
    const float v = total(wave);
    if (cm.w2 && half == 0) chain_store_q8<kSync>(cm.yq, m.rows, g, v * total(wave + kWpg), gen);
    if (cm.yq && !cm.w2) chain_store_q8<kSync>(cm.yq, m.rows, g, v, gen);  // the output itself
    if (row >= m.rows) return;
    uint64_t* y = half ? cm.y_b : cm.y;
    if (y) chain_st<kSync>(y + row, tag_word(v, gen));
    if (cm.yf) gwr<float>(cm.yf)[row] = v;
    if (cm.res) {
        const float r = cm.res_plain ? ((const float*)cm.res)[row]
                                     : chain_value<kSync>((const uint64_t*)cm.res + row, rword, gen, err);
        chain_st<kSync>(cm.y2 + row, tag_word(r + v, gen));
    }
}

// One K range of one row group of a matrix with four K splits (ranges of at most
// kChainRangeChunks chunks) on its own workgroup, with tagged phases: the
// range's chunks are spread over the 4 waves as in chain_tile_split (exact
// block sums and d_w in the term table), waves 0 and 1 run the range's
// fixed-order chains A and B, and wave 0 adds each segment's A + B into the
// range's accumulator (segments of kSegChunks chunks), as the
// one-wave-per-range tile does.  Ranges 1..3 store that value as tagged words in kpart; range 0, whose
// tiles come last in the phase's table (so a workgroup never waits on a tile it
// has yet to run), polls them and adds the ranges in order -- ((r0 + r1) + r2)
// + r3, the group set's order -- then runs the epilogue.  So the result is
// bit-identical to the group-set tile, with the row group's chunks on 16 waves
// instead of 4.
template <int kSync>
__device__ __forceinline__ void chain_tile_range(const ChainMat& cm, int64_t idx, float* red, Q4S_LDS u32x2* stage,
                                                 Q4S_LDS uint32_t* terms, Q4S_LDS float* dxt, StageKey& key,
                                                 int phase, uint32_t gen, uint32_t* err, uint64_t* mark_start,
                                                 uint64_t* mark_ready, uint64_t* dump) {
    if (mark_start && threadIdx.x == 0) gwr<uint64_t>(mark_start)[0] = __builtin_amdgcn_s_memrealtime();
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const MatDesc& m = cm.m;
    const int64_t G = m.G;
    const int64_t g = idx % G;
    const int sp = (int)(idx / G);
    const int ks = m.ks;
    const int c0 = (int)((int64_t)sp * m.C / ks), c1 = (int)((int64_t)(sp + 1) * m.C / ks);
    const int n = c1 - c0;
    const int64_t row = g * kGroupRows + lane;
    const int64_t rrow = min(row, (int64_t)m.rows - 1);
    uint64_t rword = 0;
    if (cm.res && !cm.res_plain && sp == 0 && wave == 0) rword = chain_ld<kSync>((const uint64_t*)cm.res + rrow);
    // integer work of this wave's chunks of the range
    const int i0 = c0 + split_first<4>(wave, n), i1 = c0 + split_first<4>(wave + 1, n);
    if (i0 < i1) {
        Q4S_LDS u32x2* slice = stage + wave * (kChainMaxChunks * 64);
        ActStaged<kSync> act{cm, m.w, g, i0, i1, gen, err, slice, key, phase, false, wave == 0 ? mark_ready : nullptr,
                             dump};
        const uint8_t* wp = m.w + ((size_t)g * m.C + i0) * kChunkBytes + lane * kBlockNibBytes;
        Chunk a, b;
        load_chunk(a, wp);
        if (i0 + 1 < i1) load_chunk(b, wp + kChunkBytes);
        for (int c = i0; c < i1; c += 2) {
            chunk_terms<kSync>(c, c - c0, a, act, terms, dxt);
            if (c + 2 < i1) load_chunk(a, wp + (size_t)(c + 2 - i0) * kChunkBytes);
            if (c + 1 < i1) {
                chunk_terms<kSync>(c + 1, c + 1 - c0, b, act, terms, dxt);
                if (c + 3 < i1) load_chunk(b, wp + (size_t)(c + 3 - i0) * kChunkBytes);
            }
        }
    }
    __syncthreads();
    // the range's fixed-order fp32 chains: wave 0 chain A (blocks 0-3 of each chunk), wave 1
    // chain B (blocks 4-7), each closed at every segment end; wave 1 leaves its segment values
    // in red, wave 0 keeps its own
    constexpr int kMaxSeg = (kChainRangeChunks + kSegChunks - 1) / kSegChunks;
    float pseg[kMaxSeg];
#pragma unroll
    for (int k = 0; k < kMaxSeg; ++k) pseg[k] = 0.0f;
    if (wave < 2) {
        float p = 0.0f;
        int seg = 0;
        for (int cb = c0; cb < c1; cb += kChainFold) {
            uint32_t t[kChainFold][4];
            f32x4 d[kChainFold];
            chain_fetch(cb, c1, c0, wave, terms, (const Q4S_LDS f32x4*)dxt, t, d);
            chain_fold(t, d, c1 - cb, p);
            // segments are kSegChunks (a multiple of kChainFold) chunks from c0, the last one to c1
            if (cb + kChainFold >= c1 || (cb + kChainFold - c0) % kSegChunks == 0) {
                if (wave == 1) red[seg * 64 + lane] = p;
#pragma unroll
                for (int k = 0; k < kMaxSeg; ++k)
                    if (k == seg) pseg[k] = p;
                p = 0.0f;
                ++seg;
            }
        }
    }
    __syncthreads();
    if (wave != 0) return;
    float acc = 0.0f;
    const int nseg = (n + kSegChunks - 1) / kSegChunks;
#pragma unroll
    for (int k = 0; k < kMaxSeg; ++k)
        if (k < nseg) acc += pseg[k] + red[k * 64 + lane];
    if (sp != 0) {
        chain_st<kSync>(cm.kpart + ((int64_t)(sp - 1) * G + g) * 64 + lane, tag_word(acc, gen));
        return;
    }
    float v = acc;
    for (int j = 1; j < ks; ++j) {
        const uint64_t* pw = cm.kpart + ((int64_t)(j - 1) * G + g) * 64 + lane;
        v += chain_value<kSync>(pw, chain_ld<kSync>(pw), gen, err);
    }
    if (cm.yq) chain_store_q8<kSync>(cm.yq, m.rows, g, v, gen);
    if (row >= m.rows) return;
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
        const int64_t limit = chain_spin_limit(sync);
        int64_t spins = 0;
        while (__hip_atomic_load(watch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > limit || ((spins & 1023) == 0 && chain_failed(sync))) {
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
    __shared__ uint32_t terms[kChainTableWords];
    __shared__ f32x4 dxt[kChainTableWords / 64 / 4];  // the d_x table: 8 floats per chunk of the term table
    const uint32_t nwg = gridDim.x, b = blockIdx.x;
    if (P.trace && threadIdx.x == 0)  // when this workgroup started, after the phase-end plane
        gwr<uint64_t>(P.trace)[(size_t)P.n_phases * nwg + b] = __builtin_amdgcn_s_memrealtime();
    uint32_t begin = 0;
    StageKey key{-1, 0, 0};  // this wave's LDS slice holds nothing yet
    if (threadIdx.x == 0) chain_xs_claim = chain_xs_ready = -1;  // no phase's vector yet
    __syncthreads();
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
            const uint32_t tw = P.tiles[2 * (size_t)t + 1];
            uint64_t* dp = P.dump ? P.dump + (size_t)p * P.dump_chunks * 64 : nullptr;
            if (tw & kChainSplit4)  // one row group, its chunks spread over the 4 waves
                chain_tile_split<kSync, 4>(cm, tw & kChainTileIndex, red, (Q4S_LDS u32x2*)stage,
                                           (Q4S_LDS uint32_t*)terms, (Q4S_LDS float*)dxt, key, p, P.gen, P.sync,
                                           ms, mr, dp);
            else if (tw & kChainSplit2)  // two row groups, two waves each
                chain_tile_split<kSync, 2>(cm, tw & kChainTileIndex, red, (Q4S_LDS u32x2*)stage,
                                           (Q4S_LDS uint32_t*)terms, (Q4S_LDS float*)dxt, key, p, P.gen, P.sync,
                                           ms, mr, dp);
            else if (kSync == kChainTagged && (tw & kChainRange))  // one K range of a row group
                chain_tile_range<kSync>(cm, tw & kChainTileIndex, red, (Q4S_LDS u32x2*)stage,
                                        (Q4S_LDS uint32_t*)terms, (Q4S_LDS float*)dxt, key, p, P.gen, P.sync, ms,
                                        mr, dp);
            else  // a group set: one wave per row group (or K range)
                chain_tile<kSync>(cm, tw, red, (Q4S_LDS u32x2*)stage, key, p, P.gen, P.sync, ms, mr, dp);
            __syncthreads();
        }
        if (P.trace && threadIdx.x == 0)  // when this workgroup is done with the phase
            gwr<uint64_t>(P.trace)[(size_t)p * nwg + b] = __builtin_amdgcn_s_memrealtime();
        if constexpr (kSync != kChainTagged)
            if (p + 1 < P.n_phases) chain_barrier<kSync>(P.sync, (uint32_t)p + 1);
        begin = end;
    }
}

// Clears the sync words before a launch and sets its poll limit (word 3).
__global__ __launch_bounds__(256) void k_chain_reset(uint32_t* w, int n, uint32_t spin_limit) {
    for (int i = threadIdx.x; i < n; i += 256) w[i] = i == 3 ? spin_limit : 0u;
}

}  // namespace

hipError_t launch_chain(int sync_mode, const ChainParams& p, int workgroups, uint32_t spin_limit, bool cooperative,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_chain_reset, dim3(1), dim3(256), 0, st, p.sync, kChainSyncWords, spin_limit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ChainParams a = p;
    void* args[] = {&a};
    const void* fn = sync_mode == kChainCounter ? (const void*)k_chain<kChainCounter>
                     : sync_mode == kChainTree  ? (const void*)k_chain<kChainTree>
                                                : (const void*)k_chain<kChainTagged>;
    // (the workgroup count never exceeds what can be resident, so a plain launch on an otherwise
    // idle GPU also starts them all; its waits are bounded either way)
    if (!cooperative) return hipLaunchKernel(fn, dim3(workgroups), dim3(kThreads), args, 0, st);
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

}  // namespace q4s
