// C ABI of libq4stream (include/q4s.h): argument validation, the sweep plan
// (tile table), and kernel launches.  Every check runs before any HIP call.
#include "q4s.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "q4s_chain.h"
#include "q4s_internal.h"

using namespace q4s;

namespace {

thread_local char g_err[512] = "";

q4s_status fail(q4s_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

// prepend "matrix i: " to the current error text
q4s_status prefix_matrix(q4s_status s, int i) {
    char tmp[sizeof g_err];
    memcpy(tmp, g_err, sizeof tmp);
    return fail(s, "matrix %d: %s", i, tmp);
}

q4s_status ok() {
    g_err[0] = '\0';
    return Q4S_OK;
}

q4s_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(Q4S_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

q4s_status check_shape(int64_t rows, int64_t cols, int n, int max_n = Q4S_MAX_N) {
    if (rows < 0 || rows >= kMaxDim) return fail(Q4S_ERR_SHAPE, "rows=%lld out of [0, 2^31)", (long long)rows);
    if (cols < 0 || cols >= kMaxDim || cols % 32 != 0)
        return fail(Q4S_ERR_SHAPE, "cols=%lld must be a multiple of 32 in [0, 2^31)", (long long)cols);
    if (n < 0 || n > max_n) return fail(Q4S_ERR_SHAPE, "n=%d out of [0, %d]", n, max_n);
    return Q4S_OK;
}

// pointer p naming `bytes` bytes: may be NULL only when bytes == 0; must be a-aligned
q4s_status check_ptr(const void* p, size_t bytes, uintptr_t a, const char* name) {
    if (p == nullptr) {
        if (bytes == 0) return Q4S_OK;
        return fail(Q4S_ERR_NULL, "%s is NULL", name);
    }
    if (!aligned(p, a)) return fail(Q4S_ERR_ALIGN, "%s must be %u-byte aligned", name, (unsigned)a);
    return Q4S_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

size_t packed_bytes(int64_t rows, int64_t cols) {
    return (size_t)(groups_of(rows) * chunks_of(cols)) * kChunkBytes;
}
size_t packed_q8_bytes(int64_t rows, int64_t cols) {
    return (size_t)(groups_of(rows) * chunks_of(cols)) * kQ8ChunkBytes;
}
// planar Q8_0: q [n][cols], then d_x [n][dstride] (rows padded to 8 entries)
size_t q8_bytes(int n, int64_t cols) {
    return (size_t)n * (size_t)cols + (size_t)n * (size_t)dstride_of(cols) * 2;
}

MatDesc make_desc(const void* w, const void* xq8, float* y, int64_t rows, int64_t cols, int n) {
    MatDesc m;
    m.w = (const uint8_t*)w;
    m.xq = (const int8_t*)xq8;
    m.xd = (const uint16_t*)((const uint8_t*)xq8 + (size_t)n * (size_t)cols);
    m.y = y;
    m.rows = (int32_t)rows;
    m.cols = (int32_t)cols;
    m.nb = (int32_t)(cols / 32);
    m.G = (int32_t)groups_of(rows);
    m.C = (int32_t)chunks_of(cols);
    m.ks = choose_ksplit(m.C);
    m.dstride = (int32_t)dstride_of(cols);
    m.n = n;
    m.x = nullptr;
    return m;
}

// validation shared by the GEMVs and each sweep matrix
q4s_status check_gemv(const void* w, const void* xq8, const float* y, int64_t rows, int64_t cols,
                      int n, bool q8w = false) {
    q4s_status s = check_shape(rows, cols, n, q8w ? Q4S_MAX_N_Q8 : Q4S_MAX_N);
    if (s) return s;
    const bool live = rows > 0 && n > 0;
    const size_t wb = live ? (q8w ? packed_q8_bytes(rows, cols) : packed_bytes(rows, cols)) : 0;
    const size_t xb = live ? q8_bytes(n, cols) : 0;
    const size_t yb = live ? (size_t)n * rows * 4 : 0;
    if ((s = check_ptr(w, wb, 16, "w_packed"))) return s;
    if ((s = check_ptr(xq8, xb, 16, "x_q8"))) return s;
    if ((s = check_ptr(y, yb, 4, "y"))) return s;
    if (overlap(y, yb, w, wb) || overlap(y, yb, xq8, xb))
        return fail(Q4S_ERR_ALIAS, "y overlaps an input");
    return Q4S_OK;
}

}  // namespace

// ====================================================================== ABI

extern "C" {

int q4s_abi_version(void) { return Q4S_ABI_VERSION; }

const char* q4s_status_string(int s) {
    switch (s) {
        case Q4S_OK: return "ok";
        case Q4S_ERR_NULL: return "null pointer";
        case Q4S_ERR_SHAPE: return "invalid shape";
        case Q4S_ERR_ALIGN: return "misaligned pointer";
        case Q4S_ERR_ALIAS: return "output overlaps input";
        case Q4S_ERR_PLAN: return "invalid plan";
        case Q4S_ERR_HIP: return "HIP runtime error";
        case Q4S_ERR_WAIT: return "a bounded wait gave up";
        default: return "unknown status";
    }
}

const char* q4s_last_error(void) { return g_err; }

size_t q4s_q4_0_bytes(int64_t rows, int64_t cols) {
    if (check_shape(rows, cols, 1) != Q4S_OK) return 0;
    return (size_t)rows * (size_t)(cols / 32) * 18;
}

size_t q4s_packed_bytes(int64_t rows, int64_t cols) {
    if (check_shape(rows, cols, 1) != Q4S_OK) return 0;
    return packed_bytes(rows, cols);
}

size_t q4s_q8_bytes(int n, int64_t cols) {
    if (check_shape(0, cols, n) != Q4S_OK) return 0;
    return q8_bytes(n, cols);
}

q4s_status q4s_repack_q4_0(const void* w_q4_0, void* w_packed, int64_t rows, int64_t cols, void* stream) {
    q4s_status s = check_shape(rows, cols, 1);
    if (s) return s;
    const size_t cb = (size_t)rows * (size_t)(cols / 32) * 18;
    const size_t pb = packed_bytes(rows, cols);
    if ((s = check_ptr(w_q4_0, cb, 2, "w_q4_0"))) return s;
    if ((s = check_ptr(w_packed, pb, 16, "w_packed"))) return s;
    if (overlap(w_q4_0, cb, w_packed, pb)) return fail(Q4S_ERR_ALIAS, "w_packed overlaps w_q4_0");
    if (pb == 0) return ok();
    return hip_status(launch_repack((const uint8_t*)w_q4_0, (uint8_t*)w_packed, rows, cols,
                                    (hipStream_t)stream), "repack launch");
}

q4s_status q4s_quantize_q8_0(const float* x, void* x_q8, int n, int64_t cols, void* stream) {
    q4s_status s = check_shape(0, cols, n);
    if (s) return s;
    const size_t xb = (size_t)n * (size_t)cols * 4;
    const size_t qb = (n > 0 && cols > 0) ? q8_bytes(n, cols) : 0;
    if ((s = check_ptr(x, xb, 16, "x"))) return s;
    if ((s = check_ptr(x_q8, qb, 16, "x_q8"))) return s;
    if (overlap(x, xb, x_q8, qb)) return fail(Q4S_ERR_ALIAS, "x_q8 overlaps x");
    if (qb == 0) return ok();
    QuantDesc d;
    d.x = x;
    d.q = (int8_t*)x_q8;
    d.d = (uint16_t*)((uint8_t*)x_q8 + (size_t)n * (size_t)cols);
    d.blk0 = 0;
    d.n = n;
    d.cols = (int32_t)cols;
    d.dstride = (int32_t)dstride_of(cols);
    d.pad_ = 0;
    return hip_status(launch_quantize(d, (hipStream_t)stream), "quantize launch");
}

q4s_status q4s_gemv_q4_0(const void* w_packed, const void* x_q8, float* y, int64_t rows, int64_t cols,
                         int n, void* stream) {
    q4s_status s = check_gemv(w_packed, x_q8, y, rows, cols, n);
    if (s) return s;
    if (rows == 0 || n == 0) return ok();
    const MatDesc m = make_desc(w_packed, x_q8, y, rows, cols, n);
    return hip_status(launch_gemv(m, n, gsets_of(m.G, m.ks), (hipStream_t)stream), "gemv launch");
}

}  // extern "C"

namespace {

q4s_status block_sums_any(const void* w_packed, const void* x_q8, int32_t* sums, int64_t rows, int64_t cols,
                          int n, void* stream, bool q8w) {
    q4s_status s = check_shape(rows, cols, n, q8w ? Q4S_MAX_N_Q8 : Q4S_MAX_N);
    if (s) return s;
    const bool live = rows > 0 && n > 0 && cols > 0;
    const size_t wb = live ? (q8w ? packed_q8_bytes(rows, cols) : packed_bytes(rows, cols)) : 0;
    const size_t xb = live ? q8_bytes(n, cols) : 0;
    const size_t sb = live ? (size_t)n * rows * (cols / 32) * 4 : 0;
    if ((s = check_ptr(w_packed, wb, 16, "w_packed"))) return s;
    if ((s = check_ptr(x_q8, xb, 16, "x_q8"))) return s;
    if ((s = check_ptr(sums, sb, 4, "s"))) return s;
    if (overlap(sums, sb, w_packed, wb) || overlap(sums, sb, x_q8, xb))
        return fail(Q4S_ERR_ALIAS, "s overlaps an input");
    if (!live) return ok();
    const MatDesc m = make_desc(w_packed, x_q8, nullptr, rows, cols, n);
    return hip_status(q8w ? launch_block_sums_q8_0(m, n, sums, (hipStream_t)stream)
                          : launch_block_sums(m, n, sums, (hipStream_t)stream),
                      "block_sums launch");
}

}  // namespace

extern "C" {

q4s_status q4s_block_sums(const void* w_packed, const void* x_q8, int32_t* sums, int64_t rows,
                          int64_t cols, int n, void* stream) {
    return block_sums_any(w_packed, x_q8, sums, rows, cols, n, stream, false);
}

// ============================================================= Q8_0 weights

size_t q4s_q8_0_bytes(int64_t rows, int64_t cols) {
    if (check_shape(rows, cols, 1) != Q4S_OK) return 0;
    return (size_t)rows * (size_t)(cols / 32) * 34;
}

size_t q4s_packed_q8_0_bytes(int64_t rows, int64_t cols) {
    if (check_shape(rows, cols, 1) != Q4S_OK) return 0;
    return packed_q8_bytes(rows, cols);
}

q4s_status q4s_repack_q8_0(const void* w_q8_0, void* w_packed, int64_t rows, int64_t cols, void* stream) {
    q4s_status s = check_shape(rows, cols, 1);
    if (s) return s;
    const size_t cb = (size_t)rows * (size_t)(cols / 32) * 34;
    const size_t pb = packed_q8_bytes(rows, cols);
    if ((s = check_ptr(w_q8_0, cb, 2, "w_q8_0"))) return s;
    if ((s = check_ptr(w_packed, pb, 16, "w_packed"))) return s;
    if (overlap(w_q8_0, cb, w_packed, pb)) return fail(Q4S_ERR_ALIAS, "w_packed overlaps w_q8_0");
    if (pb == 0) return ok();
    return hip_status(launch_repack_q8_0((const uint8_t*)w_q8_0, (uint8_t*)w_packed, rows, cols,
                                         (hipStream_t)stream), "repack launch");
}

q4s_status q4s_gemv_q8_0(const void* w_packed, const void* x_q8, float* y, int64_t rows, int64_t cols,
                         int n, void* stream) {
    q4s_status s = check_gemv(w_packed, x_q8, y, rows, cols, n, true);
    if (s) return s;
    if (rows == 0 || n == 0) return ok();
    const MatDesc m = make_desc(w_packed, x_q8, y, rows, cols, n);
    return hip_status(launch_gemv_q8_0(m, n, gsets_of(m.G, m.ks), (hipStream_t)stream), "gemv launch");
}

q4s_status q4s_gemv_q8_0_f32(const void* w_packed, const float* x, void* x_q8, float* y, int64_t rows,
                             int64_t cols, void* stream) {
    q4s_status s = check_gemv(w_packed, x_q8, y, rows, cols, 1, true);
    if (s) return s;
    const size_t xb = rows > 0 ? (size_t)cols * 4 : 0;
    if ((s = check_ptr(x, xb, 16, "x"))) return s;
    const size_t qb = rows > 0 ? q8_bytes(1, cols) : 0;
    if (overlap(x, xb, x_q8, qb) || overlap(x, xb, y, (size_t)rows * 4) ||
        overlap(x, xb, w_packed, packed_q8_bytes(rows, cols)) || overlap(x_q8, qb, w_packed, packed_q8_bytes(rows, cols)))
        return fail(Q4S_ERR_ALIAS, "x, x_q8, y and w_packed must not overlap");
    if (rows == 0) return ok();
    MatDesc m = make_desc(w_packed, x_q8, y, rows, cols, 1);
    if (m.ks == 1) {  // one launch: the waves quantize the chunks they stream
        m.x = x;
        return hip_status(launch_gemv_q8_0_fused(m, (hipStream_t)stream), "gemv launch");
    }
    if ((s = q4s_quantize_q8_0(x, x_q8, 1, cols, stream))) return s;
    return hip_status(launch_gemv_q8_0(m, 1, gsets_of(m.G, m.ks), (hipStream_t)stream), "gemv launch");
}

q4s_status q4s_block_sums_q8_0(const void* w_packed, const void* x_q8, int32_t* sums, int64_t rows,
                               int64_t cols, int n, void* stream) {
    return block_sums_any(w_packed, x_q8, sums, rows, cols, n, stream, true);
}

q4s_status q4s_requant_q8_0_to_q4_0(const void* w_q8_0, void* w_q4_0, int64_t rows, int64_t cols,
                                    void* stream) {
    q4s_status s = check_shape(rows, cols, 1);
    if (s) return s;
    const int64_t nblk = rows * (cols / 32);
    const size_t b8 = (size_t)nblk * 34, b4 = (size_t)nblk * 18;
    if ((s = check_ptr(w_q8_0, b8, 2, "w_q8_0"))) return s;
    if ((s = check_ptr(w_q4_0, b4, 2, "w_q4_0"))) return s;
    if (overlap(w_q8_0, b8, w_q4_0, b4)) return fail(Q4S_ERR_ALIAS, "w_q4_0 overlaps w_q8_0");
    if (nblk == 0) return ok();
    return hip_status(launch_requant_q8_0_to_q4_0((const uint8_t*)w_q8_0, (uint8_t*)w_q4_0, nblk,
                                                  (hipStream_t)stream), "requant launch");
}

// ========================================================== attention

size_t q4s_attn_workspace_bytes(int n_q, int64_t L) {
    if (n_q < 1 || n_q > 4096 || L < 1 || L >= kMaxDim) return 0;
    return (size_t)attn_splits(L) * (size_t)attn_split_floats(n_q) * 4;
}

namespace {

// shapes and buffers of a decode-attention call, except the workspace
q4s_status check_attn(const float* q, const float* k_blk, const float* v, const float* o, int n_q, int n_kv,
                      int64_t L, int64_t l_cap) {
    if (n_q < 1 || n_q > 4096 || n_kv < 1 || n_q % n_kv != 0 || n_q / n_kv > 8)
        return fail(Q4S_ERR_SHAPE, "n_q=%d, n_kv=%d: n_kv must divide n_q with a group of 1..8", n_q, n_kv);
    if (L < 1 || l_cap < L || l_cap >= kMaxDim || l_cap % kAttnSplit != 0)
        return fail(Q4S_ERR_SHAPE, "need 1 <= L (%lld) <= l_cap (%lld) < 2^31 with l_cap %% 64 == 0",
                    (long long)L, (long long)l_cap);
    const size_t qb = (size_t)n_q * kAttnHeadDim * 4;
    const size_t kvb = (size_t)l_cap * n_kv * kAttnHeadDim * 4;
    q4s_status s;
    if ((s = check_ptr(q, qb, 16, "q"))) return s;
    if ((s = check_ptr(k_blk, kvb, 16, "k_blk"))) return s;
    if ((s = check_ptr(v, kvb, 16, "v"))) return s;
    if ((s = check_ptr(o, qb, 4, "o"))) return s;
    if (overlap(o, qb, q, qb) || overlap(o, qb, k_blk, kvb) || overlap(o, qb, v, kvb))
        return fail(Q4S_ERR_ALIAS, "o overlaps an input");
    return Q4S_OK;
}

}  // namespace

q4s_status q4s_attn_decode(const float* q, const float* k_blk, const float* v, float* o, int n_q, int n_kv,
                           int64_t L, int64_t l_cap, void* workspace, size_t workspace_bytes, void* stream) {
    q4s_status s;
    if ((s = check_attn(q, k_blk, v, o, n_q, n_kv, L, l_cap))) return s;
    const size_t qb = (size_t)n_q * kAttnHeadDim * 4;
    const size_t kvb = (size_t)l_cap * n_kv * kAttnHeadDim * 4;
    const size_t wsb = q4s_attn_workspace_bytes(n_q, L);
    if ((s = check_ptr(workspace, wsb, 16, "workspace"))) return s;
    if (workspace_bytes < wsb)
        return fail(Q4S_ERR_SHAPE, "workspace holds %zu bytes, needs %zu", workspace_bytes, wsb);
    if (overlap(o, qb, workspace, wsb)) return fail(Q4S_ERR_ALIAS, "o overlaps the workspace");
    if (overlap(workspace, wsb, q, qb) || overlap(workspace, wsb, k_blk, kvb) || overlap(workspace, wsb, v, kvb))
        return fail(Q4S_ERR_ALIAS, "workspace overlaps an input");
    return hip_status(launch_attn_decode(q, k_blk, v, o, (float*)workspace, n_q, n_kv, L, l_cap,
                                         (float)(1.0 / std::sqrt((double)kAttnHeadDim)), (hipStream_t)stream),
                      "attention launch");
}

q4s_status q4s_attn_decode_noalloc(const float* q, const float* k_blk, const float* v, float* o, int n_q, int n_kv,
                                   int64_t L, int64_t l_cap, void* stream) {
    static_assert(Q4S_ATTN_SCRATCH_BYTES == kAttnScratchBytes, "header and library agree on the scratch size");
    q4s_status s;
    if ((s = check_attn(q, k_blk, v, o, n_q, n_kv, L, l_cap))) return s;
    const size_t wsb = q4s_attn_workspace_bytes(n_q, L);
    if (wsb > kAttnScratchBytes)
        return fail(Q4S_ERR_SHAPE, "n_q=%d, L=%lld needs %zu bytes of split partials; the static scratch holds %zu",
                    n_q, (long long)L, wsb, (size_t)kAttnScratchBytes);
    float* ws = nullptr;
    const hipError_t e = attn_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "attention scratch lookup");
    return hip_status(launch_attn_decode(q, k_blk, v, o, ws, n_q, n_kv, L, l_cap,
                                         (float)(1.0 / std::sqrt((double)kAttnHeadDim)), (hipStream_t)stream),
                      "attention launch");
}

// ==================================================================== sweep

struct q4s_plan {
    int n = 0;
    std::vector<MatDesc> mats;
    std::vector<uint32_t> tiles;     // (matrix, group set) pairs, largest tiles first
    std::vector<QuantDesc> quant;    // matrices with an fp32 activation to quantize
    std::vector<uint32_t> qtiles;    // (activation, first block) pairs, kQuantTileBlocks blocks each
    int64_t quant_blocks = 0;
    bool fused = false;              // n == 1, every matrix quantized by the GEMV launch itself
    bool split_tiles = false;        // n == 1, one K split everywhere: one workgroup per (matrix, row group)
    q4s_plan_info info{};
    // device image: [MatDesc x n_mats][QuantDesc x n_quant][tiles][quantize tiles], 16-byte aligned parts
    size_t off_mats = 0, off_quant = 0, off_tiles = 0, off_qtiles = 0, dev_bytes = 0;
    std::vector<uint8_t> image;
    uint8_t* dev = nullptr;
    uint64_t* trace = nullptr;       // the GEMV launch's timeline, or NULL
};

q4s_status q4s_sweep_plan_create(const q4s_mat* mats, int n_mats, int n, size_t* dev_bytes_needed,
                                 q4s_plan** out) {
    if (!out || !dev_bytes_needed) return fail(Q4S_ERR_NULL, "out and dev_bytes_needed are required");
    *out = nullptr;
    if (n < 1 || n > Q4S_MAX_N) return fail(Q4S_ERR_SHAPE, "n=%d out of [1, %d]", n, Q4S_MAX_N);
    if (n_mats < 0 || (n_mats > 0 && !mats)) return fail(Q4S_ERR_PLAN, "invalid matrix table");
    q4s_status s;
    // per-matrix checks, then the hazards between the two phases of a run:
    // quantize reads x and writes x_q8; the GEMV reads w_packed and x_q8 and writes y
    struct Region { const void* p; size_t b; };
    std::vector<Region> xs, q8s, ws, ys;
    for (int i = 0; i < n_mats; ++i) {
        const q4s_mat& a = mats[i];
        if ((s = check_gemv(a.w_packed, a.x_q8, a.y, a.rows, a.cols, n))) return prefix_matrix(s, i);
        const bool live = a.rows > 0;
        size_t xb = live && a.cols > 0 ? q8_bytes(n, a.cols) : 0;
        if (a.x) {
            // x is quantized into x_q8 even when rows == 0
            const size_t fb = (size_t)n * a.cols * 4;
            xb = a.cols > 0 ? q8_bytes(n, a.cols) : 0;
            if ((s = check_ptr(a.x, fb, 16, "x"))) return prefix_matrix(s, i);
            if ((s = check_ptr(a.x_q8, xb, 16, "x_q8"))) return prefix_matrix(s, i);
            xs.push_back({a.x, fb});
        }
        q8s.push_back({a.x_q8, xb});
        ws.push_back({a.w_packed, live ? packed_bytes(a.rows, a.cols) : 0});
        ys.push_back({a.y, live ? (size_t)n * a.rows * 4 : 0});
    }
    auto any_overlap = [](const std::vector<Region>& A, const std::vector<Region>& B) {
        for (const Region& a : A)
            for (const Region& b : B)
                if (overlap(a.p, a.b, b.p, b.b)) return true;
        return false;
    };
    if (any_overlap(q8s, xs)) return fail(Q4S_ERR_ALIAS, "an x_q8 of the sweep overlaps an x");
    if (any_overlap(ys, ws) || any_overlap(ys, q8s) || any_overlap(ys, xs))
        return fail(Q4S_ERR_ALIAS, "a y of the sweep overlaps an input");

    q4s_plan* p = new (std::nothrow) q4s_plan;
    if (!p) return fail(Q4S_ERR_PLAN, "out of host memory");
    p->n = n;
    // One activation row, every matrix live and given as fp32: the GEMV waves
    // quantize the activation themselves (no separate quantize launch).  With 2..8
    // rows the quantization stays a launch of its own: the many-row dots leave the
    // waves no spare VALU issue (quantizing inside them took the 8-row step of the
    // Qwen2.5-1.5B sweep from 172 to 231 us).
    p->fused = n == 1 && n_mats > 0;
    for (int i = 0; i < n_mats && p->fused; ++i) {
        const q4s_mat& a = mats[i];
        if (!a.x || a.rows == 0 || a.cols == 0) p->fused = false;
    }
    struct Tile { uint32_t mat, gset; int64_t bytes; };
    std::vector<Tile> tiles;
    // one row, no matrix with more than 8 chunks (one K split): no wave needs another, so
    // the GEMV launch runs one workgroup per (matrix, row group), its chunks over 8 waves, instead of 4-group tiles
    p->split_tiles = n == 1;
    for (int i = 0; i < n_mats && p->split_tiles; ++i)
        if (mats[i].rows > 0 && choose_ksplit(chunks_of(mats[i].cols)) != 1) p->split_tiles = false;
    for (int i = 0; i < n_mats; ++i) {
        const q4s_mat& a = mats[i];
        MatDesc m = make_desc(a.w_packed, a.x_q8, a.y, a.rows, a.cols, n);
        if (p->fused) m.x = a.x;
        p->mats.push_back(m);
        p->info.weight_bytes += a.rows * (a.cols / 32) * 18;
        if (p->fused) {
            p->info.n_quant_blocks += a.cols / 32;
        } else if (a.x && a.cols > 0) {
            QuantDesc q;
            q.x = a.x;
            q.q = (int8_t*)a.x_q8;
            q.d = (uint16_t*)((uint8_t*)a.x_q8 + (size_t)n * a.cols);
            q.blk0 = p->quant_blocks;
            q.n = n;
            q.cols = (int32_t)a.cols;
            q.dstride = (int32_t)dstride_of(a.cols);
            q.pad_ = 0;
            const int64_t nblk = (int64_t)n * (a.cols / 32);
            for (int64_t b = 0; b < nblk; b += kQuantTileBlocks) {
                p->qtiles.push_back((uint32_t)p->quant.size());
                p->qtiles.push_back((uint32_t)b);
            }
            p->quant.push_back(q);
            p->quant_blocks += nblk;
        }
        if (a.rows == 0) continue;
        p->info.packed_bytes += (int64_t)packed_bytes(a.rows, a.cols);
        p->info.act_bytes += (int64_t)n * a.cols / 32 * 34;
        p->info.out_bytes += (int64_t)n * a.rows * 4;
        // one workgroup per row group: the split kernels, and the single-split matrices of other 1-row sweeps
        if (p->split_tiles || (n == 1 && m.ks == 1)) {
            for (int64_t gr = 0; gr < m.G; ++gr) tiles.push_back({(uint32_t)i, (uint32_t)gr, m.C * kChunkBytes});
            continue;
        }
        const int gpw = kWaves / m.ks;
        const int64_t ng = gsets_of(m.G, m.ks);
        for (int64_t gs = 0; gs < ng; ++gs) {
            const int64_t groups = std::min<int64_t>(gpw, m.G - gs * gpw);
            tiles.push_back({(uint32_t)i, (uint32_t)gs, groups * m.C * kChunkBytes});
        }
    }
    std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& a, const Tile& b) { return a.bytes > b.bytes; });
    for (const Tile& t : tiles) {
        p->tiles.push_back(t.mat);
        p->tiles.push_back(t.gset);
    }
    auto up16 = [](size_t v) { return (v + 15) & ~(size_t)15; };
    p->off_mats = 0;
    p->off_quant = up16(p->mats.size() * sizeof(MatDesc));
    p->off_tiles = p->off_quant + up16(p->quant.size() * sizeof(QuantDesc));
    p->off_qtiles = p->off_tiles + up16(p->tiles.size() * sizeof(uint32_t));
    p->dev_bytes = std::max<size_t>(16, p->off_qtiles + up16(p->qtiles.size() * sizeof(uint32_t)));
    p->image.assign(p->dev_bytes, 0);
    if (!p->mats.empty()) memcpy(p->image.data() + p->off_mats, p->mats.data(), p->mats.size() * sizeof(MatDesc));
    if (!p->quant.empty()) memcpy(p->image.data() + p->off_quant, p->quant.data(), p->quant.size() * sizeof(QuantDesc));
    if (!p->tiles.empty()) memcpy(p->image.data() + p->off_tiles, p->tiles.data(), p->tiles.size() * sizeof(uint32_t));
    if (!p->qtiles.empty())
        memcpy(p->image.data() + p->off_qtiles, p->qtiles.data(), p->qtiles.size() * sizeof(uint32_t));
    p->info.n_mats = n_mats;
    p->info.n_tiles = (int64_t)tiles.size();
    if (!p->fused) p->info.n_quant_blocks = p->quant_blocks;
    p->info.fused_quantize = p->fused ? 1 : 0;
    p->info.dev_bytes = (int64_t)p->dev_bytes;
    *dev_bytes_needed = p->dev_bytes;
    *out = p;
    return ok();
}

q4s_status q4s_sweep_plan_upload(q4s_plan* p, void* dev_mem, size_t dev_bytes, void* stream) {
    if (!p) return fail(Q4S_ERR_NULL, "plan is NULL");
    if (!dev_mem) return fail(Q4S_ERR_NULL, "dev_mem is NULL");
    if (!aligned(dev_mem, 16)) return fail(Q4S_ERR_ALIGN, "dev_mem must be 16-byte aligned");
    if (dev_bytes < p->dev_bytes)
        return fail(Q4S_ERR_PLAN, "dev_mem holds %zu bytes, plan needs %zu", dev_bytes, p->dev_bytes);
    // the quantize descriptors' block offsets and the tables are position independent;
    // only the base of the image changes
    hipError_t e = hipMemcpyAsync(dev_mem, p->image.data(), p->dev_bytes, hipMemcpyHostToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "plan upload");
    p->dev = (uint8_t*)dev_mem;
    return ok();
}

q4s_status q4s_sweep_run(const q4s_plan* p, void* stream) {
    if (!p) return fail(Q4S_ERR_NULL, "plan is NULL");
    if (!p->dev) return fail(Q4S_ERR_PLAN, "plan was not uploaded");
    hipStream_t st = (hipStream_t)stream;
    const MatDesc* mats = (const MatDesc*)(p->dev + p->off_mats);
    const uint32_t* tiles = (const uint32_t*)(p->dev + p->off_tiles);
    const int64_t n_tiles = (int64_t)p->tiles.size() / 2;
    if (p->split_tiles && p->fused)
        return hip_status(launch_sweep_split(mats, tiles, n_tiles, true, p->trace, st), "sweep launch");
    if (p->fused) return hip_status(launch_sweep_fused(mats, tiles, n_tiles, p->trace, st), "sweep launch");
    if (!p->quant.empty()) {
        hipError_t e = launch_quantize_batch((const QuantDesc*)(p->dev + p->off_quant),
                                             (const uint32_t*)(p->dev + p->off_qtiles),
                                             (int64_t)p->qtiles.size() / 2, p->n, st);
        if (e != hipSuccess) return hip_status(e, "sweep quantize launch");
    }
    if (p->split_tiles)
        return hip_status(launch_sweep_split(mats, tiles, n_tiles, false, p->trace, st), "sweep launch");
    // the tiled many-row kernels are not traced
    return hip_status(launch_sweep(mats, tiles, n_tiles, p->n, p->n <= kTokTile ? p->trace : nullptr, st),
                      "sweep launch");
}

size_t q4s_sweep_trace_bytes(const q4s_plan* p) {
    if (!p) return 0;
    return p->tiles.size() / 2 * kSweepTraceWords * 8;
}

q4s_status q4s_sweep_set_trace(q4s_plan* p, uint64_t* trace, size_t trace_bytes) {
    if (!p) return fail(Q4S_ERR_NULL, "plan is NULL");
    if (trace) {
        q4s_status s;
        const size_t need = q4s_sweep_trace_bytes(p);
        if ((s = check_ptr(trace, need, 8, "trace"))) return s;
        if (trace_bytes < need) return fail(Q4S_ERR_SHAPE, "trace holds %zu bytes, needs %zu", trace_bytes, need);
        if (p->n > kTokTile) return fail(Q4S_ERR_PLAN, "the timeline covers steps of at most 8 rows");
    }
    p->trace = trace;
    return ok();
}

q4s_status q4s_sweep_plan_info(const q4s_plan* p, q4s_plan_info* info) {
    if (!p || !info) return fail(Q4S_ERR_NULL, "plan and info are required");
    *info = p->info;
    return ok();
}

void q4s_sweep_plan_destroy(q4s_plan* p) { delete p; }

// ============================================================ chained step

struct q4s_chain {
    q4s_chain_shape shape{};
    int mode = 0;
    int workgroups_req = 0;
    int workgroups = 0;
    uint64_t* acts = nullptr;
    int64_t act_words = 0;
    std::vector<ChainMat> mats;
    std::vector<std::vector<uint32_t>> phases;  // the matrices of each phase
    int layout_wg = 0;                // the workgroup count the tile table was laid out for
    std::vector<uint32_t> tiles;      // (matrix, tile word), phase by phase, largest first within a phase
    std::vector<uint32_t> phase_end;  // cumulative tile count per phase
    q4s_chain_info info{};
    // per matrix: byte offset of its tagged Q8_0 product words (paired gate/up: written; down: read)
    // within the Q8_0 area, or -1
    std::vector<int64_t> q8_out, q8_in;
    size_t q8_bytes = 0;
    // per matrix: byte offset of its K-range words (see ChainMat::kpart) within that area, or -1
    std::vector<int64_t> kp_off;
    size_t kp_bytes = 0;
    // device image: [ChainMat x n][tiles][phase_end][sync words][Q8_0 words][K-range words], 16-byte aligned
    size_t off_tiles = 0, off_phase = 0, off_sync = 0, off_q8 = 0, off_kp = 0, dev_bytes = 0;
    std::vector<uint8_t> image;
    uint8_t* dev = nullptr;
    uint32_t gen = 0;
    int64_t steps = 0;
    bool cooperative = true;
    uint64_t* trace = nullptr;
    uint64_t* dump = nullptr;
    uint32_t spin_limit = kChainDefaultSpin;
};

// The tile table for `wg` persistent workgroups.  Per phase, the finest layout
// whose tile count fits the workgroups: one row group per tile with its chunks
// spread over the 4 waves (matrices with one or two K splits), or two row
// groups per tile with two waves each (one K split); else a group set per tile
// (one wave per row group, or per K range).  With tagged phases a phase whose
// one matrix has K-range words (four K splits of <= 32 chunks: down) runs one
// tile per (K range, row group) instead, ranges 1..3 first and range 0 last,
// whatever the workgroup count.  The device image keeps room for the largest
// table (one tile per row group, or per K range and row group).
static void chain_layout(q4s_chain* p, int wg) {
    struct Tile { uint32_t mat, word; int64_t bytes; };
    p->tiles.clear();
    p->phase_end.clear();
    int64_t max_tiles = 0;
    // a paired matrix (see ChainMat) has twice its row groups, and its tiles hold an even number
    auto groups_of_mat = [&](uint32_t i) { return p->mats[i].m.G * (p->mats[i].w2 ? 2 : 1); };
    for (const std::vector<uint32_t>& members : p->phases) {
        int64_t groups = 0;
        bool splittable = true, narrow = true, paired = false;
        for (uint32_t i : members) {
            groups += groups_of_mat(i);
            splittable = splittable && p->mats[i].m.ks <= 2;  // <= 16 chunks
            narrow = narrow && p->mats[i].m.ks == 1;          // <= 8 chunks
            paired = paired || p->mats[i].w2 != nullptr;      // only with ks <= 2
        }
        if (members.size() == 1 && p->kp_off[members[0]] >= 0) {
            const uint32_t i = members[0];
            const MatDesc& m = p->mats[i].m;
            max_tiles += m.G * m.ks;
            for (int sp = 1; sp <= m.ks; ++sp) {
                const int r = sp % m.ks;  // ranges 1 .. ks-1, then 0
                for (int64_t g = 0; g < m.G; ++g) {
                    p->tiles.push_back(i);
                    p->tiles.push_back((uint32_t)(r * m.G + g) | kChainRange);
                }
            }
            p->phase_end.push_back((uint32_t)(p->tiles.size() / 2));
            continue;
        }
        max_tiles += groups;
        const uint32_t mode = !splittable                               ? 0u
                              : groups <= wg && !paired                 ? kChainSplit4
                              : narrow && (groups + 1) / 2 <= wg        ? kChainSplit2
                                                                        : 0u;
        std::vector<Tile> phase;
        for (uint32_t i : members) {
            const MatDesc& m = p->mats[i].m;
            const int64_t G = groups_of_mat(i);
            const int gpt = mode == kChainSplit4 ? 1 : (mode == kChainSplit2 ? 2 : kWaves / m.ks);
            for (int64_t t = 0; t * gpt < G; ++t) {
                const int64_t n = std::min<int64_t>(gpt, G - t * gpt);
                phase.push_back({i, (uint32_t)t | mode, n * m.C * kChunkBytes});
            }
        }
        std::stable_sort(phase.begin(), phase.end(), [](const Tile& a, const Tile& b) { return a.bytes > b.bytes; });
        for (const Tile& t : phase) {
            p->tiles.push_back(t.mat);
            p->tiles.push_back(t.word);
        }
        p->phase_end.push_back((uint32_t)(p->tiles.size() / 2));
    }
    auto up16 = [](size_t v) { return (v + 15) & ~(size_t)15; };
    p->off_tiles = up16(p->mats.size() * sizeof(ChainMat));
    p->off_phase = p->off_tiles + up16((size_t)max_tiles * 2 * sizeof(uint32_t));
    p->off_sync = p->off_phase + up16(p->phase_end.size() * sizeof(uint32_t));
    p->off_q8 = p->off_sync + up16(kChainSyncWords * sizeof(uint32_t));
    p->off_kp = p->off_q8 + up16(p->q8_bytes);
    p->dev_bytes = p->off_kp + up16(p->kp_bytes);
    p->image.assign(p->dev_bytes, 0);
    memcpy(p->image.data(), p->mats.data(), p->mats.size() * sizeof(ChainMat));
    memcpy(p->image.data() + p->off_tiles, p->tiles.data(), p->tiles.size() * sizeof(uint32_t));
    memcpy(p->image.data() + p->off_phase, p->phase_end.data(), p->phase_end.size() * sizeof(uint32_t));
    p->info.n_tiles = (int64_t)p->tiles.size() / 2;
    p->info.dev_bytes = (int64_t)p->dev_bytes;
    p->layout_wg = wg;
}

static bool chain_shape_ok(const q4s_chain_shape* s) {
    // hidden and ff <= 32768 keep every wave's K range within its 32-chunk LDS slice
    return s && s->layers >= 0 && s->layers <= (1 << 16) && s->hidden >= 32 && s->hidden % 32 == 0 &&
           s->hidden <= 32768 && s->ff >= 32 && s->ff % 32 == 0 && s->ff <= 32768 && s->kv_dim >= 1 &&
           s->kv_dim <= (1 << 20) && s->vocab >= 1 && s->vocab <= (1 << 24);
}

static int64_t chain_layer_words(const q4s_chain_shape* s) {
    return 5 * (int64_t)s->hidden + 2 * (int64_t)s->kv_dim + 2 * (int64_t)s->ff;
}

int64_t q4s_chain_act_words(const q4s_chain_shape* s) {
    if (!chain_shape_ok(s)) return 0;
    return (int64_t)s->layers * chain_layer_words(s);
}

q4s_status q4s_chain_create(const q4s_chain_shape* shape, const void* const* w_packed, const float* h0,
                            uint64_t* acts, float* logits, int sync_mode, int workgroups,
                            size_t* dev_bytes_needed, q4s_chain** out) {
    if (!out || !dev_bytes_needed || !shape || !w_packed) return fail(Q4S_ERR_NULL, "shape, w_packed, dev_bytes_needed and out are required");
    *out = nullptr;
    if (!chain_shape_ok(shape))
        return fail(Q4S_ERR_SHAPE,
                    "chain shape needs layers >= 0, hidden and ff multiples of 32 up to 32768, kv_dim and vocab >= 1");
    if (sync_mode < Q4S_CHAIN_COUNTER || sync_mode > Q4S_CHAIN_TAGGED)
        return fail(Q4S_ERR_SHAPE, "sync_mode=%d is not a chain sync mode", sync_mode);
    if (workgroups < 0 || workgroups > (1 << 16)) return fail(Q4S_ERR_SHAPE, "workgroups=%d out of range", workgroups);
    const int64_t L = shape->layers, E = shape->hidden, D = shape->kv_dim, F = shape->ff, V = shape->vocab;
    const int64_t n_mats = 7 * L + 1;
    const int64_t words = L * chain_layer_words(shape);
    q4s_status s;
    if ((s = check_ptr(h0, (size_t)E * 4, 16, "h0"))) return s;
    if ((s = check_ptr(acts, (size_t)words * 8, 16, "acts"))) return s;
    if ((s = check_ptr(logits, (size_t)V * 4, 4, "logits"))) return s;
    const int64_t dims[7][2] = {{E, E}, {D, E}, {D, E}, {E, E}, {F, E}, {F, E}, {E, F}};
    std::vector<std::pair<const void*, size_t>> ins = {{h0, (size_t)E * 4}};
    for (int64_t i = 0; i < n_mats; ++i) {
        const int64_t r = i == 7 * L ? V : dims[i % 7][0], c = i == 7 * L ? E : dims[i % 7][1];
        if ((s = check_ptr(w_packed[i], packed_bytes(r, c), 16, "w_packed"))) return prefix_matrix(s, (int)i);
        ins.push_back({w_packed[i], packed_bytes(r, c)});
    }
    for (const auto& in : ins)
        if (overlap(acts, (size_t)words * 8, in.first, in.second) || overlap(logits, (size_t)V * 4, in.first, in.second))
            return fail(Q4S_ERR_ALIAS, "an output of the chain overlaps an input");
    if (overlap(acts, (size_t)words * 8, logits, (size_t)V * 4)) return fail(Q4S_ERR_ALIAS, "acts overlaps logits");

    q4s_chain* p = new (std::nothrow) q4s_chain;
    if (!p) return fail(Q4S_ERR_PLAN, "out of host memory");
    p->shape = *shape;
    p->mode = sync_mode;
    p->workgroups_req = workgroups;
    p->acts = acts;
    p->act_words = words;
    const int64_t per = chain_layer_words(shape);
    auto word = [&](int64_t l, int64_t off) { return acts + l * per + off; };
    const int64_t oq = 0, ok_ = E, ov = E + D, oo = E + 2 * D, oh1 = 2 * E + 2 * D, og = 3 * E + 2 * D,
                  ou = 3 * E + 2 * D + F, odn = 3 * E + 2 * D + 2 * F, oh2 = 4 * E + 2 * D + 2 * F;
    auto base = [&](const void* w, int64_t r, int64_t c) {
        ChainMat cm{};
        cm.m = make_desc(w, nullptr, nullptr, r, c, 1);
        cm.m.xd = nullptr;
        p->info.packed_bytes += (int64_t)packed_bytes(r, c);
        return cm;
    };
    std::vector<uint32_t> members;  // matrices of the phase being built
    auto add = [&](const ChainMat& cm) {
        members.push_back((uint32_t)p->mats.size());
        p->mats.push_back(cm);
        p->q8_out.push_back(-1);
        p->q8_in.push_back(-1);
        p->kp_off.push_back(-1);
    };
    auto close = [&]() {
        p->phases.push_back(members);
        members.clear();
    };
    for (int64_t l = 0; l < L; ++l) {
        const void* const* lw = w_packed + 7 * l;
        const void* h = l == 0 ? (const void*)h0 : (const void*)word(l - 1, oh2);
        const int hp = l == 0 ? 1 : 0;
        // q, k, v: one activation of norm(h)
        const int64_t qkv_rows[3] = {E, D, D}, qkv_off[3] = {oq, ok_, ov};
        const int64_t q_q8 = (int64_t)p->q8_bytes;  // q's tiles also leave q quantized for o
        p->q8_bytes += (size_t)(E / 4 + E / 32) * 8;
        for (int j = 0; j < 3; ++j) {
            ChainMat cm = base(lw[j], qkv_rows[j], E);
            cm.x = h, cm.x_plain = hp, cm.norm = 1, cm.y = word(l, qkv_off[j]);
            add(cm);
            if (j == 0) p->q8_out.back() = q_q8;
        }
        close();
        {   // o = Wo Q8(q); h1 = h + o
            ChainMat cm = base(lw[3], E, E);
            cm.y = word(l, oo), cm.res = h, cm.res_plain = hp, cm.y2 = word(l, oh1);
            add(cm);
            p->q8_in.back() = q_q8;
        }
        close();
        // gate, up: one activation of norm(h1).  With at most two K splits they run as one
        // paired matrix whose tiles also leave g * u quantized for down (see ChainMat)
        const bool pair = choose_ksplit(chunks_of(E)) <= 2;
        const int64_t q8_at = (int64_t)p->q8_bytes;
        if (pair) {
            ChainMat cm = base(lw[4], F, E);
            cm.w2 = (const uint8_t*)lw[5];
            p->info.packed_bytes += (int64_t)packed_bytes(F, E);
            cm.x = word(l, oh1), cm.norm = 1, cm.y = word(l, og), cm.y_b = word(l, ou);
            add(cm);
            p->q8_out.back() = q8_at;
            p->q8_bytes += (size_t)(F / 4 + F / 32) * 8;
        } else {
            for (int j = 0; j < 2; ++j) {
                ChainMat cm = base(lw[4 + j], F, E);
                cm.x = word(l, oh1), cm.norm = 1, cm.y = word(l, j == 0 ? og : ou);
                add(cm);
            }
        }
        close();
        {   // dn = Wd Q8(g * u); h2 = h1 + dn
            ChainMat cm = base(lw[6], E, F);
            if (!pair) cm.x = word(l, og), cm.x2 = word(l, ou);
            cm.y = word(l, odn), cm.res = word(l, oh1), cm.y2 = word(l, oh2);
            add(cm);
            if (pair) p->q8_in.back() = q8_at;
            // with tagged phases, four K splits of <= 32 chunks each run as K-range tiles
            if (sync_mode == Q4S_CHAIN_TAGGED && cm.m.ks == 4 && cm.m.C <= 4 * kChainRangeChunks) {
                p->kp_off.back() = (int64_t)p->kp_bytes;
                p->kp_bytes += (size_t)(cm.m.ks - 1) * (size_t)cm.m.G * 64 * 8;
            }
        }
        close();
    }
    {
        ChainMat cm = base(w_packed[7 * L], V, E);
        cm.x = L == 0 ? (const void*)h0 : (const void*)word(L - 1, oh2), cm.x_plain = L == 0 ? 1 : 0, cm.norm = 1,
        cm.yf = logits;
        add(cm);
        close();
    }
    // laid out for the requested workgroups (256 when left to the upload, which lays it out
    // again for the count it resolves); dev_bytes does not depend on the count
    chain_layout(p, workgroups ? workgroups : 256);
    p->info.n_mats = n_mats;
    p->info.n_phases = (int64_t)p->phase_end.size();
    p->info.act_words = words;
    *dev_bytes_needed = p->dev_bytes;
    *out = p;
    return ok();
}

q4s_status q4s_chain_upload(q4s_chain* p, void* dev_mem, size_t dev_bytes, void* stream) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    if (!dev_mem) return fail(Q4S_ERR_NULL, "dev_mem is NULL");
    if (!aligned(dev_mem, 16)) return fail(Q4S_ERR_ALIGN, "dev_mem must be 16-byte aligned");
    if (dev_bytes < p->dev_bytes)
        return fail(Q4S_ERR_PLAN, "dev_mem holds %zu bytes, the chain needs %zu", dev_bytes, p->dev_bytes);
    int max_wg = 0;
    hipError_t e = chain_max_workgroups(p->mode, &max_wg);
    if (e != hipSuccess) return hip_status(e, "occupancy query");
    int cus = 0, dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_status(e, "hipGetDevice");
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return hip_status(e, "device attribute");
    const int wg = p->workgroups_req ? p->workgroups_req : std::min(cus, max_wg);
    if (wg < 1 || wg > max_wg)
        return fail(Q4S_ERR_SHAPE, "workgroups=%d out of [1, %d] (all must be resident at once)", wg, max_wg);
    if (wg != p->layout_wg) chain_layout(p, wg);
    // the Q8_0 product words and the K-range words live in dev_mem: point the matrices' copies in
    // the image at them (the areas themselves are uploaded as zeros: tag 0, never written)
    for (size_t i = 0; i < p->mats.size(); ++i) {
        ChainMat* cm = (ChainMat*)p->image.data() + i;
        if (p->q8_out[i] >= 0) cm->yq = (uint64_t*)((uint8_t*)dev_mem + p->off_q8 + p->q8_out[i]);
        if (p->q8_in[i] >= 0) cm->xq = (const uint64_t*)((uint8_t*)dev_mem + p->off_q8 + p->q8_in[i]);
        if (p->kp_off[i] >= 0) cm->kpart = (uint64_t*)((uint8_t*)dev_mem + p->off_kp + p->kp_off[i]);
    }
    hipStream_t st = (hipStream_t)stream;
    if ((e = hipMemcpyAsync(dev_mem, p->image.data(), p->dev_bytes, hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_status(e, "chain upload");
    if (p->act_words > 0 && (e = hipMemsetAsync(p->acts, 0, (size_t)p->act_words * 8, st)) != hipSuccess)
        return hip_status(e, "acts clear");
    p->dev = (uint8_t*)dev_mem;
    p->workgroups = wg;
    p->info.workgroups = wg;
    p->gen = 0;
    p->steps = 0;
    return ok();
}

// chunks per phase in the staged-input dump: those of the widest activation (E or F)
static int64_t chain_dump_chunks(const q4s_chain* p) {
    return std::max(chunks_of(p->shape.hidden), chunks_of(p->shape.ff));
}

q4s_status q4s_chain_run(q4s_chain* p, void* stream) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    if (!p->dev) return fail(Q4S_ERR_PLAN, "chain was not uploaded");
    if (++p->gen == 0) p->gen = 1;  // tag 0 marks words never written
    ChainParams cp;
    cp.mats = (const ChainMat*)p->dev;
    cp.tiles = (const uint32_t*)(p->dev + p->off_tiles);
    cp.phase_end = (const uint32_t*)(p->dev + p->off_phase);
    cp.sync = (uint32_t*)(p->dev + p->off_sync);
    cp.n_phases = (int32_t)p->phase_end.size();
    cp.gen = p->gen;
    cp.trace = p->trace;
    cp.dump = p->dump;
    cp.dump_chunks = (int32_t)chain_dump_chunks(p);
    q4s_status s =
        hip_status(launch_chain(p->mode, cp, p->workgroups, p->spin_limit, p->cooperative, (hipStream_t)stream),
                   "chain launch");
    if (s == Q4S_OK) ++p->steps;
    return s;
}

q4s_status q4s_chain_check(const q4s_chain* p, void* stream) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    if (!p->dev) return fail(Q4S_ERR_PLAN, "chain was not uploaded");
    uint32_t err = 0;
    hipError_t e = hipMemcpyAsync(&err, p->dev + p->off_sync, 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "chain check");
    if (err) return fail(Q4S_ERR_WAIT, "a bounded wait of the chained step gave up");
    return ok();
}

size_t q4s_chain_trace_bytes(const q4s_chain* p) {
    if (!p || !p->dev) return 0;
    return (3 * (size_t)p->phase_end.size() + 1) * (size_t)p->workgroups * 8;
}

q4s_status q4s_chain_set_trace(q4s_chain* p, uint64_t* trace, size_t trace_bytes) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    if (!p->dev) return fail(Q4S_ERR_PLAN, "chain was not uploaded");
    if (trace) {
        q4s_status s;
        const size_t need = q4s_chain_trace_bytes(p);
        if ((s = check_ptr(trace, need, 8, "trace"))) return s;
        if (trace_bytes < need) return fail(Q4S_ERR_SHAPE, "trace holds %zu bytes, needs %zu", trace_bytes, need);
    }
    p->trace = trace;
    return ok();
}

size_t q4s_chain_stage_dump_bytes(const q4s_chain* p) {
    if (!p) return 0;
    return (size_t)p->phase_end.size() * (size_t)chain_dump_chunks(p) * 64 * 8;
}

q4s_status q4s_chain_set_stage_dump(q4s_chain* p, uint64_t* dump, size_t dump_bytes) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    if (dump) {
        q4s_status s;
        const size_t need = q4s_chain_stage_dump_bytes(p);
        if ((s = check_ptr(dump, need, 8, "dump"))) return s;
        if (dump_bytes < need) return fail(Q4S_ERR_SHAPE, "dump holds %zu bytes, needs %zu", dump_bytes, need);
    }
    p->dump = dump;
    return ok();
}

q4s_status q4s_chain_set_wait_limit(q4s_chain* p, uint32_t polls) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    p->spin_limit = polls;
    return ok();
}

q4s_status q4s_chain_set_cooperative(q4s_chain* p, int cooperative) {
    if (!p) return fail(Q4S_ERR_NULL, "chain is NULL");
    p->cooperative = cooperative != 0;
    return ok();
}

q4s_status q4s_chain_get_info(const q4s_chain* p, q4s_chain_info* info) {
    if (!p || !info) return fail(Q4S_ERR_NULL, "chain and info are required");
    *info = p->info;
    info->steps = p->steps;
    return ok();
}

void q4s_chain_destroy(q4s_chain* p) { delete p; }

// ============================================================= measurement

q4s_status q4s_bench_read(const void* buf, size_t bytes, int loads_in_flight, int n_blocks, uint32_t* sink,
                          void* stream) {
    if (bytes % 16) return fail(Q4S_ERR_SHAPE, "bytes must be a multiple of 16");
    if (loads_in_flight != 1 && loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8)
        return fail(Q4S_ERR_SHAPE, "loads_in_flight must be 1, 2, 4 or 8");
    if (n_blocks < 0 || n_blocks > (1 << 20)) return fail(Q4S_ERR_SHAPE, "n_blocks out of range");
    q4s_status s;
    if ((s = check_ptr(buf, bytes, 16, "buf"))) return s;
    if ((s = check_ptr(sink, bytes ? 4 : 0, 4, "sink"))) return s;
    return hip_status(launch_bench_read(buf, bytes, loads_in_flight, n_blocks, sink, (hipStream_t)stream),
                      "bench_read launch");
}

q4s_status q4s_bench_read_units(const void* buf, size_t bytes, size_t unit_bytes, uint32_t* sink, void* stream) {
    if (unit_bytes == 0 || unit_bytes % 1024 || unit_bytes > ((size_t)1 << 30))
        return fail(Q4S_ERR_SHAPE, "unit_bytes must be a positive multiple of 1024, at most 1 GiB");
    if (bytes / unit_bytes > ((size_t)1 << 33)) return fail(Q4S_ERR_SHAPE, "too many units");
    q4s_status s;
    if ((s = check_ptr(buf, bytes, 16, "buf"))) return s;
    if ((s = check_ptr(sink, bytes ? 4 : 0, 4, "sink"))) return s;
    return hip_status(launch_bench_read_units(buf, bytes, unit_bytes, sink, (hipStream_t)stream),
                      "bench_read_units launch");
}

size_t q4s_bench_grid_barrier_scratch_bytes(int n_workgroups) {
    if (n_workgroups < 1 || n_workgroups > (1 << 20)) return 0;
    return grid_barrier_scratch_words(n_workgroups) * 4;
}

q4s_status q4s_bench_grid_barrier(int kind, int n_workgroups, int phases, uint32_t* scratch, size_t scratch_bytes,
                                  void* stream) {
    if (kind < 0 || kind > 9) return fail(Q4S_ERR_SHAPE, "kind must be 0..9");
    if (phases < 1 || phases > (1 << 20)) return fail(Q4S_ERR_SHAPE, "phases must be in 1..2^20");
    int max_wg = 0;
    hipError_t e = grid_barrier_max_workgroups(&max_wg);
    if (e != hipSuccess) return hip_status(e, "occupancy query");
    if (n_workgroups < 1 || n_workgroups > max_wg)
        return fail(Q4S_ERR_SHAPE, "n_workgroups=%d out of [1, %d] (all must be resident at once)", n_workgroups,
                    max_wg);
    const size_t need = q4s_bench_grid_barrier_scratch_bytes(n_workgroups);
    q4s_status s;
    if ((s = check_ptr(scratch, need, 4, "scratch"))) return s;
    if (scratch_bytes < need) return fail(Q4S_ERR_SHAPE, "scratch holds %zu bytes, needs %zu", scratch_bytes, need);
    return hip_status(launch_grid_barrier(kind, n_workgroups, phases, scratch, (hipStream_t)stream),
                      "barrier launch");
}

int q4s_bench_grid_barrier_max_workgroups(void) {
    int n = 0;
    return grid_barrier_max_workgroups(&n) == hipSuccess ? n : 0;
}

q4s_status q4s_bench_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16) return fail(Q4S_ERR_SHAPE, "bytes must be a multiple of 16");
    q4s_status s;
    if ((s = check_ptr(src, bytes, 16, "src"))) return s;
    if ((s = check_ptr(dst, bytes, 16, "dst"))) return s;
    if (overlap(src, bytes, dst, bytes)) return fail(Q4S_ERR_ALIAS, "dst overlaps src");
    return hip_status(launch_bench_copy(src, dst, bytes, (hipStream_t)stream), "bench_copy launch");
}

}  // extern "C"
