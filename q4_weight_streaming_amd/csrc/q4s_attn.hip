// gfx950 kernels for decode attention over a KV cache: split-KV partials and
// their combine (the attn_partial / attn_combine kernels of the "minfer"
// README, nano-inference page, milestone M12), grouped so one read of a
// key/value head serves every query head of its group (milestone M15).
//
// Layout (one 32 KB block per (kv head, 64 positions) for keys and values):
// keys blocked and transposed, K [n_kv][l_cap/64][128][64] (position c of
// block b, dimension d at ((g*NB + b)*128 + d)*64 + c), so a thread reads 4
// consecutive positions of a dimension and no dot product crosses lanes;
// values head-major, V [n_kv][l_cap][128].
//
// A workgroup of 8 waves takes one (kv head, 64-position split) and issues
// all of its loads up front.  Wave w forms the partial dots over head
// dimensions 16w .. 16w+15 for all G query heads of the group: a thread holds
// 4 dimensions x 4 positions of the keys, and the 4 lanes of a lane quad are
// added by two DPP moves.  The 8 waves' partials are added in order through
// LDS, then a local softmax per head (one wave per head: maximum, exp, sum by
// wave reduction), then the weighted sum of the split's values: a thread
// holds 4 dimensions x 4 positions, lane quads are added by DPP, and the 4
// groups of 16 positions are added in order.  The combine rescales each split
// by exp(m_s - M) and adds the splits in a fixed order, so results are
// deterministic.
#include "q4s_device.h"

#include <mutex>
#include <type_traits>

namespace q4s {
namespace {

constexpr int kHd = kAttnHeadDim;     // 128
constexpr int kSplit = kAttnSplit;    // 64 positions per split

// op(v, v of lane ^ D), the same value in both lanes of each pair (op is
// commutative: max or +), by lane swaps (D = 32, 16) and DPP moves (D = 8, 4, 2,
// 1) instead of LDS permutes.  Called by a whole wave.
template <int D, class Op>
__device__ __forceinline__ float xor_combine(float v, Op op) {
    const uint32_t x = __float_as_uint(v);
    auto dpp = [](uint32_t y, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)y, decltype(ctrl)::value, 0xF, 0xF, true);
    };
    if constexpr (D == 32 || D == 16) {
        const auto sw = D == 32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                                : __builtin_amdgcn_permlane16_swap(x, x, false, false);  // {own, partner}
        return op(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    } else {
        uint32_t y;
        if constexpr (D == 8) {
            y = dpp(x, std::integral_constant<int, 0x128>{});  // row_ror:8
        } else if constexpr (D == 4) {  // row_shl:4 (lane i + 4) or row_shr:4 (lane i - 4) by lane bit 2
            const uint32_t up = dpp(x, std::integral_constant<int, 0x104>{});
            const uint32_t down = dpp(x, std::integral_constant<int, 0x114>{});
            y = (threadIdx.x & 4) ? down : up;
        } else if constexpr (D == 2) {
            y = dpp(x, std::integral_constant<int, 0x4E>{});  // quad_perm [2,3,0,1]
        } else {
            y = dpp(x, std::integral_constant<int, 0xB1>{});  // quad_perm [1,0,3,2]
        }
        return op(v, __uint_as_float(y));
    }
}
constexpr auto kMax = [](float a, float b) { return fmaxf(a, b); };
constexpr auto kAdd = [](float a, float b) { return a + b; };

// The wave's maximum / sum by the xor butterfly 32, 16, 8, 4, 2, 1.
__device__ __forceinline__ float wave_max(float v) {
    v = xor_combine<32>(v, kMax);
    v = xor_combine<16>(v, kMax);
    v = xor_combine<8>(v, kMax);
    v = xor_combine<4>(v, kMax);
    v = xor_combine<2>(v, kMax);
    return xor_combine<1>(v, kMax);
}
__device__ __forceinline__ float wave_sum(float v) {
    v = xor_combine<32>(v, kAdd);
    v = xor_combine<16>(v, kAdd);
    v = xor_combine<8>(v, kAdd);
    v = xor_combine<4>(v, kAdd);
    v = xor_combine<2>(v, kAdd);
    return xor_combine<1>(v, kAdd);
}
// Over the lanes 4, 8, 16 and 32 apart (the combine's 16 slices of a wave), in that order.
template <class Op>
__device__ __forceinline__ float slices_combine(float v, Op op) {
    v = xor_combine<4>(v, op);
    v = xor_combine<8>(v, op);
    v = xor_combine<16>(v, op);
    return xor_combine<32>(v, op);
}

// workspace (S * attn_split_floats(n_q) floats), head-major so that the combine reads
// each head's splits contiguously: unnormalized outputs [n_q][S][128], then maxima m
// [n_q][S], then sums l [n_q][S]
struct AttnParams {
    const float* q;      // [n_q][128]
    const float* kb;     // [n_kv][l_cap/64][128][64]
    const float* v;      // [n_kv][l_cap][128]
    float* o;            // [n_q][128]
    float* ws;           // [S][attn_split_floats(n_q)]
    int64_t L, l_cap;
    int n_q, n_kv, S;
    float scale;
};

// Sum of v over the 4 lanes of a lane quad (xor 1, then xor 2: a fixed order), by DPP moves.
__device__ __forceinline__ float quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    return v;
}

constexpr int kPartThreads = 512;  // 8 waves per (kv head, split)

template <int G>
__global__ __launch_bounds__(kPartThreads) void k_attn_partial(AttnParams a) {
    __shared__ f32x4 qs[G][kHd / 4];
    __shared__ float pr[G][kSplit];
    // the partial dots are dead once the scores are formed; the value sums reuse their space
    __shared__ union {
        f32x4 part[8][G][kSplit / 4];  // [wave: 16 dimensions][head][position quad]
        f32x4 vred[4][G][kHd / 4];     // [16-position group][head][dimension quad]
    } u;
    auto& part = u.part;
    auto& vred = u.vred;
    const int s = blockIdx.x, g = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, ql = lane & 3;
    const int64_t j0 = (int64_t)s * kSplit;
    const int nk = (int)min((int64_t)kSplit, a.L - j0);
    // Every load of the split is issued up front (queries, keys, values), as
    // 16-byte non-temporal loads; positions past L are masked below.
    f32x4 qv = {0.f, 0.f, 0.f, 0.f};
    if (t < G * kHd / 4) qv = gp<f32x4>(a.q + (int64_t)(g * G) * kHd)[t];
    // keys: thread (dimension group dg = 4w + ql: dimensions 4dg .. 4dg+3, position quad pq = lane/4);
    // each wave load reads 4 rows of 256 contiguous bytes of the split's 32 KB key block
    const int pq = lane >> 2, dg = 4 * w + ql;
    f32x4 kv[4];
    {
        const float* kp = a.kb + (((int64_t)g * (a.l_cap / kSplit) + s) * kHd + 4 * dg) * kSplit + 4 * pq;
#pragma unroll
        for (int d = 0; d < 4; ++d) kv[d] = __builtin_nontemporal_load(gp<f32x4>(kp + d * kSplit));
    }
    // values: thread (dimension quad dq = 16 (w&1) + lane/4, positions 16 (w>>1) + 4 ql .. +3)
    const int dq = 16 * (w & 1) + (lane >> 2), pg = w >> 1;
    f32x4 vv[4];
    {
        const float* vp = a.v + ((int64_t)g * a.l_cap + j0) * kHd + 4 * dq;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vv[e] = __builtin_nontemporal_load(gp<f32x4>(vp + (int64_t)min(16 * pg + 4 * ql + e, nk - 1) * kHd));
    }
    if (t < G * kHd / 4) qs[t / (kHd / 4)][t % (kHd / 4)] = qv;
    __syncthreads();
    // partial dots over the thread's 4 dimensions for its 4 positions, then over the
    // quad's 16 dimensions
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const f32x4 q0 = qs[h][dg];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            acc[0] = fmaf(q0[d], kv[d][0], acc[0]);
            acc[1] = fmaf(q0[d], kv[d][1], acc[1]);
            acc[2] = fmaf(q0[d], kv[d][2], acc[2]);
            acc[3] = fmaf(q0[d], kv[d][3], acc[3]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = quad_sum(acc[c]);
        if (ql == 0) part[w][h][pq] = acc;
    }
    __syncthreads();
    // scores (the 8 waves' dimension groups added in order) and the split's softmax:
    // wave w takes head w; lane = position
    for (int h = w; h < G; h += 8) {
        float sc = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sc += ((const float*)part[k][h])[lane];
        sc = lane < nk ? sc * a.scale : -INFINITY;
        const float m = wave_max(sc);
        const float p = lane < nk ? expf(sc - m) : 0.0f;
        const float l = wave_sum(p);
        pr[h][lane] = p;
        if (lane == 0) {
            float* wsm = a.ws + (int64_t)a.n_q * a.S * kHd + (int64_t)(g * G + h) * a.S + s;
            gwr<float>(wsm)[0] = m;
            gwr<float>(wsm)[(int64_t)a.n_q * a.S] = l;
        }
    }
    __syncthreads();
    // weighted values over the thread's 4 positions, then over the quad's 16 positions,
    // then the 4 position groups in order
#pragma unroll
    for (int h = 0; h < G; ++h) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = pr[h][16 * pg + 4 * ql + e];  // 0 past the split's last position
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(p, vv[e][c], acc[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = quad_sum(acc[c]);
        if (ql == 0) vred[pg][h][dq] = acc;
    }
    __syncthreads();
    if (t < G * kHd / 4) {
        const int h = t / (kHd / 4), d4 = t % (kHd / 4);
        f32x4 o = vred[0][h][d4];
#pragma unroll
        for (int k = 1; k < 4; ++k) o += vred[k][h][d4];
        float* wso = a.ws + ((int64_t)(g * G + h) * a.S + s) * kHd;
        gwr<f32x4>(wso)[d4] = o;
    }
}

// Workgroup (query head h, 16-dimension block), 256 threads: thread (split
// slice k, dimension quad) takes splits [k*S/64, (k+1)*S/64) in order, one
// 16-byte load of its 4 dimensions per split, all of a batch's loads issued
// together.  The 64 slices are reduced in a fixed tree: the 16 slices of a wave
// by an xor butterfly over lanes 4, 8, 16 and 32 apart, then the 4 waves in
// order through LDS.
constexpr int kCombSlices = 64;
constexpr int kCombQuads = 4;                                // dimension quads per workgroup
constexpr int kCombDims = 4 * kCombQuads;                    // 16
constexpr int kCombWaves = kCombSlices * kCombQuads / 64;    // 4
constexpr int kCombBatch = 8;  // splits per slice whose loads are in flight together

__global__ __launch_bounds__(kCombSlices * kCombQuads) void k_attn_combine(AttnParams a) {
    __shared__ float mred[kCombWaves];
    __shared__ f32x4 num[kCombWaves][kCombQuads];
    __shared__ float den[kCombWaves];
    const int h = blockIdx.x, d0 = blockIdx.y * kCombDims;
    const int t = threadIdx.x, dq = t % kCombQuads, k = t / kCombQuads, wv = t >> 6, lane = t & 63;
    const float* om = a.ws + (int64_t)a.n_q * a.S * kHd + (int64_t)h * a.S;  // m of head h; l follows n_q*S later
    const float* ol = om + (int64_t)a.n_q * a.S;
    const float* oo = a.ws + (int64_t)h * a.S * kHd + d0 + 4 * dq;
    const int s0 = (int)((int64_t)k * a.S / kCombSlices), s1 = (int)((int64_t)(k + 1) * a.S / kCombSlices);
    // the first batch of the slice (all of it up to 512 splits) loaded at once
    float mm[kCombBatch], ll[kCombBatch];
    f32x4 ov[kCombBatch];
    auto load_batch = [&](int b) {
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            const int sp = max(min(b + i, s1 - 1), 0);
            mm[i] = om[sp];
            ll[i] = ol[sp];
            ov[i] = gp<f32x4>(oo + (int64_t)sp * kHd)[0];
        }
    };
    load_batch(s0);
    float mk = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i)
        if (s0 + i < s1) mk = fmaxf(mk, mm[i]);
    for (int b = s0 + kCombBatch; b < s1; ++b) mk = fmaxf(mk, om[b]);
    static_assert(kCombQuads == 4, "the slices of a wave sit 4, 8, 16 and 32 lanes apart");
    mk = slices_combine(mk, kMax);
    if (lane == 0) mred[wv] = mk;
    __syncthreads();
    float M = mred[0];
#pragma unroll
    for (int i = 1; i < kCombWaves; ++i) M = fmaxf(M, mred[i]);
    f32x4 nu = {0.f, 0.f, 0.f, 0.f};
    float de = 0.0f;
    for (int b = s0; b < s1; b += kCombBatch) {
        if (b != s0) load_batch(b);
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            if (b + i >= s1) break;
            const float f = expf(mm[i] - M);
            de = fmaf(f, ll[i], de);
#pragma unroll
            for (int c = 0; c < 4; ++c) nu[c] = fmaf(f, ov[i][c], nu[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) nu[c] = slices_combine(nu[c], kAdd);
    de = slices_combine(de, kAdd);
    if (lane < kCombQuads) num[wv][dq] = nu;
    if (lane == 0) den[wv] = de;
    __syncthreads();
    if (t < kCombQuads) {
        f32x4 n = num[0][dq];
        float d = den[0];
#pragma unroll
        for (int i = 1; i < kCombWaves; ++i) {
            n += num[i][dq];
            d += den[i];
        }
        f32x4 r;
#pragma unroll
        for (int c = 0; c < 4; ++c) r[c] = n[c] / d;
        gwr<f32x4>(a.o + (int64_t)h * kHd + d0)[dq] = r;
    }
}

}  // namespace

hipError_t launch_attn_decode(const float* q, const float* kb, const float* v, float* o, float* ws, int n_q,
                              int n_kv, int64_t L, int64_t l_cap, float scale, hipStream_t st) {
    AttnParams a{q, kb, v, o, ws, L, l_cap, n_q, n_kv, (int)((L + kSplit - 1) / kSplit), scale};
    const dim3 grid((unsigned)a.S, (unsigned)n_kv);
    switch (n_q / n_kv) {
        case 1: hipLaunchKernelGGL(k_attn_partial<1>, grid, dim3(kPartThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_attn_partial<2>, grid, dim3(kPartThreads), 0, st, a); break;
        case 3: hipLaunchKernelGGL(k_attn_partial<3>, grid, dim3(kPartThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL(k_attn_partial<4>, grid, dim3(kPartThreads), 0, st, a); break;
        case 5: hipLaunchKernelGGL(k_attn_partial<5>, grid, dim3(kPartThreads), 0, st, a); break;
        case 6: hipLaunchKernelGGL(k_attn_partial<6>, grid, dim3(kPartThreads), 0, st, a); break;
        case 7: hipLaunchKernelGGL(k_attn_partial<7>, grid, dim3(kPartThreads), 0, st, a); break;
        case 8: hipLaunchKernelGGL(k_attn_partial<8>, grid, dim3(kPartThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)n_q, kHd / kCombDims), dim3(kCombSlices * kCombQuads), 0, st,
                       a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- static scratch
//
// The split partials of q4s_attn_decode_noalloc live in this fixed array, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops).  Every GPU the library runs on holds its own copy, from the
// first use until the process ends.  On the host the array's name only stands
// for the symbol: its device address on the current device comes from
// hipGetSymbolAddress, taken once per device and kept, and only that address is
// ever handed to a kernel.
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

constexpr int kScratchDevices = 64;

hipError_t attn_scratch(float** out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* ptr[kScratchDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = (float*)ptr[dev];
    return hipSuccess;
}

}  // namespace q4s
