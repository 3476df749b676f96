/*
 * q4s.h -- C ABI of libq4stream: Q4_0-weight x Q8_0-activation weight-streaming
 * GEMV / skinny GEMM (1 to 8 activation rows) for AMD Instinct MI355X (gfx950).
 *
 * The operation (the "minfer" README on the nano-inference page):
 *   - weights stay quantized in GPU memory as Q4_0 ("How it works", the
 *     cuda_infer bullet) and are repacked once at load time into 32-row groups
 *     so a warp reads one contiguous span ("How it works", the mega.cu bullet;
 *     milestone M15);
 *   - the activation is quantized to int8 once per product (milestones M3.5
 *     and M15) in the Q8_0 block format (34-byte blocks, milestone M14);
 *   - each output is a sum over 32-wide blocks of an exact integer dot
 *     s = sum_j (nibble_j - 8) * q_j (milestone M9), scaled by d_w * d_x and
 *     accumulated in fp32 ("How it works", mega.cu bullet; milestone M16);
 *   - a step carries up to 8 activation rows that share one pass over the
 *     weights (mega.cu bullet; milestone M16), with every row's result
 *     bit-identical to the same row computed alone; here up to 24 rows share a
 *     pass (prefill chunks and longer verifies, milestones M7 and M17);
 *   - a whole decode step's projections stream in one launch instead of one
 *     launch per matrix (Results paragraph on the roofline; milestone M15).
 *
 * Conventions for every entry point:
 *   - Buffers are device memory owned by the caller.  Nothing here allocates,
 *     frees or synchronizes device memory, except q4s_sweep_plan_upload, which
 *     copies the plan's tables into caller-provided device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it; buffers must stay alive until it completes.
 *   - Arguments are validated before any HIP call; a failed check returns a
 *     status other than Q4S_OK and enqueues nothing.  q4s_last_error() then
 *     describes the failure (thread-local).  No C++ exception crosses the ABI.
 *   - A launch failure reported by the HIP runtime returns Q4S_ERR_HIP; faults
 *     inside a kernel surface at the caller's next stream synchronization.
 *   - A pointer may be NULL only when the buffer it names has 0 bytes.
 *   - Shapes: rows >= 0, cols >= 0 with cols % 32 == 0, n in 0..24 (Q4_0
 *     weights; 0..8 for Q8_0 weights), and
 *     rows, cols < 2^31.  rows == 0 or n == 0 is a no-op; cols == 0 writes
 *     y = 0 (the empty sum).
 *
 * Layouts:
 *   Canonical Q4_0 (GGUF): [rows][cols/32] blocks of 18 bytes: binary16 scale
 *     d_w (little-endian), then 16 bytes qs; element j < 16 is qs[j] & 0xF,
 *     element j >= 16 is qs[j-16] >> 4; weight = (nibble - 8) * d_w.
 *   Packed Q4_0 (this library, produced by q4s_repack_q4_0): rows padded to a
 *     multiple of 64 (G = ceil(rows/64) groups), blocks padded to a multiple of
 *     8 (C = ceil(cols/256) chunks).  Group g, chunk c occupies 9216 bytes at
 *     offset (g*C + c) * 9216:
 *       bytes [0, 8192)   : nibbles, [8 blocks][64 rows][16 bytes]; each byte is
 *                           the canonical qs byte XOR 0x88, i.e. both nibbles
 *                           hold (nibble - 8) in 4-bit two's complement;
 *       bytes [8192, 9216): scales, [64 rows][8 blocks] binary16 d_w.
 *     Padding rows and blocks hold zero bytes (weight 0, scale 0).
 *   Q8_0 activation (planar): for n rows of cols values, with
 *   D = cols/32 rounded up to a multiple of 8,
 *       bytes [0, n*cols)             : q, int8 [n][cols];
 *       bytes [n*cols, n*cols + 2*n*D): d_x, binary16 [n][D] (entries past
 *                                       cols/32 are padding, never read);
 *     at cols % 256 == 0 this is the dense n*cols*34/32 bytes.
 *     Per 32-block: d = max|x| / 127 (fp32, correctly rounded); q =
 *     round-half-away-from-zero(x / d) with the fp32 d as divisor; stored
 *     d_x = binary16(d) (round to nearest even, subnormals kept).  An
 *     all-zero block stores d_x = +0, q = 0.  Inputs must be finite with
 *     |x| < 8e6 (so d_x stays finite); a block whose max|x| is nonzero but
 *     below 127 * 2^-150 (d rounds to 0) gets unspecified q.
 *   Output y: fp32 [n][rows], row-major.
 *
 * Numerics: per block the kernel forms the exact integer s and the term
 *   fmaf(d_w * d_x, (float)s, chain) (d_w * d_x is exact in fp32).  A wave
 *   streams a contiguous range of 256-column chunks of 64 rows; within each
 *   segment of up to 16 chunks, blocks 0-3 of every chunk form chain A and
 *   blocks 4-7 chain B (in chunk order), and the row accumulator takes
 *   acc += (A + B) at the end of the segment.  Rows longer than 2048 columns
 *   are split over 2 or 4 waves of a workgroup, whose accumulators are added
 *   in split order.  The partition depends only on (rows, cols), so results
 *   are deterministic, identical for every n (row t of an n-row call equals
 *   the 1-row call bit for bit), and identical between q4s_gemv_q4_0 and
 *   q4s_sweep_run.  The rounding error is at most
 *   (64 + ceil(c/16) + 4) * 2^-24 * sum_b |d_w d_x s|, c = chunks per wave,
 *   i.e. below 1e-5 * sum_b |d_w d_x s| for rows up to 2^20 columns.
 */
#ifndef Q4S_H
#define Q4S_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4S_ABI_VERSION 4
#define Q4S_MAX_N 24   /* activation rows per Q4_0 product (one weight pass) */
#define Q4S_MAX_N_Q8 8 /* activation rows per Q8_0-weight product */

typedef enum {
    Q4S_OK = 0,
    Q4S_ERR_NULL = 1,      /* a required pointer is NULL                    */
    Q4S_ERR_SHAPE = 2,     /* rows / cols / n out of range                  */
    Q4S_ERR_ALIGN = 3,     /* pointer misaligned for its layout             */
    Q4S_ERR_ALIAS = 4,     /* an output buffer overlaps an input buffer     */
    Q4S_ERR_PLAN = 5,      /* invalid plan, plan memory or matrix table     */
    Q4S_ERR_HIP = 6,       /* the HIP runtime reported an error             */
    Q4S_ERR_WAIT = 7       /* a bounded wait of a chained step gave up      */
} q4s_status;

/* ---------------------------------------------------------------- general */

/* Q4S_ABI_VERSION of the loaded library. */
int q4s_abi_version(void);

/* Static text for a status code (never NULL). */
const char* q4s_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* q4s_last_error(void);

/* --------------------------------------------------------------- sizes */

/* Canonical Q4_0 bytes: rows * cols/32 * 18.  0 for invalid shapes. */
size_t q4s_q4_0_bytes(int64_t rows, int64_t cols);

/* Packed Q4_0 bytes: ceil(rows/64) * ceil(cols/256) * 9216.  0 if invalid. */
size_t q4s_packed_bytes(int64_t rows, int64_t cols);

/* Planar Q8_0 bytes for n rows: n*cols + 2*n*D, D = ceil(cols/256)*8 (the d_x
 * rows are padded to 8 entries so every 8-block chunk of scales is one aligned
 * 16-byte load).  0 if invalid. */
size_t q4s_q8_bytes(int n, int64_t cols);

/* ----------------------------------------------------------- operations */

/*
 * Weight repack (load time).  w_q4_0: canonical Q4_0 [rows][cols/32] x 18 B
 * (2-byte aligned); w_packed: q4s_packed_bytes(rows, cols) bytes (16-byte
 * aligned), fully overwritten, padding included.  Lossless: the canonical
 * bytes are recoverable from the packed ones (layout above).
 * Source: mega.cu bullet of "How it works" and milestone M15 (row-group
 * packing at load).
 */
q4s_status q4s_repack_q4_0(const void* w_q4_0, void* w_packed, int64_t rows, int64_t cols,
                           void* stream);

/*
 * Q8_0 activation quantization.  x: fp32 [n][cols] (16-byte aligned);
 * x_q8: q4s_q8_bytes(n, cols) bytes (16-byte aligned), planar layout above.
 * Source: milestones M3.5 and M15 (int8 activations, quantized once), M14
 * (34-byte Q8_0 blocks).
 */
q4s_status q4s_quantize_q8_0(const float* x, void* x_q8, int n, int64_t cols, void* stream);

/*
 * y[t][r] = sum_b d_w[r][b] * d_x[t][b] * s[t][r][b] for t < n, r < rows.
 * w_packed: packed Q4_0 (16-byte aligned); x_q8: planar Q8_0 of n rows
 * (16-byte aligned); y: fp32 [n][rows] (4-byte aligned), must not overlap
 * either input.  n in 0..24: every row shares one pass over the weights (n = 1
 * on v_dot4, 2..8 in one MFMA token tile, 9..24 in two or three); longer
 * prefill chunks are split by the caller.  Needs no workspace.
 * Source: cuda_infer and mega.cu bullets of "How it works"; milestones M9,
 * M15, M16.
 */
q4s_status q4s_gemv_q4_0(const void* w_packed, const void* x_q8, float* y, int64_t rows,
                         int64_t cols, int n, void* stream);

/*
 * Test hook: the exact per-block integer sums s[t][r][b] = sum_j
 * (nibble_{r,b,j} - 8) * q_{t,b,j}, int32 [n][rows][cols/32], computed by the
 * same device code as the GEMV.  Source: milestone M9.
 */
q4s_status q4s_block_sums(const void* w_packed, const void* x_q8, int32_t* s, int64_t rows,
                          int64_t cols, int n, void* stream);

/* ------------------------------------------------------ Q8_0 weights */

/*
 * The 8-bit output head (milestone M6 of the "minfer" README: Q8_0 weights in
 * a linear layout for a coalesced int8 GEMV, the gemv_q8_dp4a bullet of "How
 * it works"), and its load-time requantization to Q4_0 (milestones M14, M18).
 *
 * Canonical Q8_0 weights (GGUF): [rows][cols/32] blocks of 34 bytes: binary16
 *   scale d_w (little-endian), then 32 int8 values w_j; weight = w_j * d_w.
 * Packed Q8_0 (produced by q4s_repack_q8_0): the Q4_0 groups and chunks
 *   (G = ceil(rows/64), C = ceil(cols/256)); group g, chunk c occupies 17408
 *   bytes at offset (g*C + c) * 17408, as two pieces of 8704 bytes (blocks
 *   0-3, then 4-7 of the chunk), each:
 *     bytes [0, 8192)   : int8 values, [4 blocks][2 halves][64 rows][16 bytes]
 *                         (half h holds elements 16h .. 16h+15);
 *     bytes [8192, 8704): scales, [64 rows][4 blocks] binary16 d_w.
 *   Padding rows and blocks hold zero bytes.
 * Numerics as for Q4_0 with s = sum_j w_j * q_j, except that chain A takes
 *   the even blocks of each chunk and chain B the odd ones; the same
 *   determinism, n-invariance and error bound hold.
 */

/* Canonical Q8_0 bytes: rows * cols/32 * 34.  0 for invalid shapes. */
size_t q4s_q8_0_bytes(int64_t rows, int64_t cols);

/* Packed Q8_0 bytes: ceil(rows/64) * ceil(cols/256) * 17408.  0 if invalid. */
size_t q4s_packed_q8_0_bytes(int64_t rows, int64_t cols);

/*
 * Weight repack (load time).  w_q8_0: canonical Q8_0 (2-byte aligned);
 * w_packed: q4s_packed_q8_0_bytes(rows, cols) bytes (16-byte aligned), fully
 * overwritten, padding included.  Lossless.  Source: milestone M6 (linear
 * layout for coalescing) and M15 (row-group packing at load).
 */
q4s_status q4s_repack_q8_0(const void* w_q8_0, void* w_packed, int64_t rows, int64_t cols,
                           void* stream);

/*
 * y[t][r] = sum_b d_w[r][b] * d_x[t][b] * sum_j w_{r,b,j} q_{t,b,j} for t < n,
 * r < rows.  w_packed: packed Q8_0 (16-byte aligned); x_q8: planar Q8_0
 * activation of n rows (16-byte aligned); y: fp32 [n][rows], must not overlap
 * either input.  n in 0..8 (Q4S_MAX_N_Q8).  Needs no workspace.  Source: milestone M6 and the
 * gemv_q8_dp4a bullet of "How it works".
 */
q4s_status q4s_gemv_q8_0(const void* w_packed, const void* x_q8, float* y, int64_t rows,
                         int64_t cols, int n, void* stream);

/*
 * The 1-row Q8_0-weight GEMV from an fp32 activation: x (fp32 [cols], 16-byte
 * aligned) is quantized into x_q8 (planar Q8_0 of one row, 16-byte aligned,
 * receives exactly what q4s_quantize_q8_0 writes) and y = q4s_gemv_q8_0 of it
 * (bit-identical).  When cols <= 2048 (one K split) both happen in one launch,
 * each wave quantizing the activation of the chunk it streams (the mega
 * kernel of milestone M15 quantizes inside its one kernel); wider matrices
 * take a quantize launch and the GEMV.  x, x_q8 and y must not overlap each
 * other or w_packed.  rows == 0 writes nothing.  Needs no workspace.  Source: as q4s_gemv_q8_0, and the
 * activation quantization of M3.5 / M14.
 */
q4s_status q4s_gemv_q8_0_f32(const void* w_packed, const float* x, void* x_q8, float* y, int64_t rows,
                             int64_t cols, void* stream);

/*
 * Test hook: exact per-block sums s[t][r][b] = sum_j w_{r,b,j} * q_{t,b,j},
 * int32 [n][rows][cols/32], from the same device code as q4s_gemv_q8_0.
 */
q4s_status q4s_block_sums_q8_0(const void* w_packed, const void* x_q8, int32_t* s, int64_t rows,
                               int64_t cols, int n, void* stream);

/*
 * Load-time requantization of canonical Q8_0 weights to canonical Q4_0 (then
 * q4s_repack_q4_0).  w_q8_0: rows * cols/32 blocks of 34 bytes (2-byte
 * aligned); w_q4_0: q4s_q4_0_bytes(rows, cols) bytes (2-byte aligned), must
 * not overlap the input.  Per block, in fp32 (the pages name the conversion,
 * not its rounding; this is the GGUF reference rule for Q4_0):
 * x_j = w_j * d_w; vmax = the x_j of largest magnitude, the first on ties;
 * d = vmax / -8; id = 1/d (0 when d == 0); nibble_j = min(15,
 * trunc(x_j * id + 8.5)); stored scale binary16(d), nearest even (a zero
 * block stores -0).  Blocks with a non-finite scale give unspecified bytes.
 * Source: milestones M14 and M18.
 */
q4s_status q4s_requant_q8_0_to_q4_0(const void* w_q8_0, void* w_q4_0, int64_t rows, int64_t cols,
                                    void* stream);

/* ---------------------------------------------------- decode attention */

/*
 * One decode step's attention over a KV cache, for every query head: the
 * split-KV attn_partial / attn_combine pair of milestone M12 of the "minfer"
 * README, with one read of a key/value head serving all query heads of its
 * group (milestone M15; Qwen2.5-1.5B: 12 query heads over 2 kv heads).
 *   s_hj = scale * q_h . k_{j,g}, g = h / (n_q / n_kv), scale = 1/sqrt(128)
 *   o_h  = sum_j softmax_j(s_hj) v_{j,g}, over positions j < L
 * Head dimension 128 (Q4S_ATTN_HEAD_DIM); n_q / n_kv (the group) in 1..8.
 * Cache layouts (one contiguous 32 KB block per kv head and 64 positions):
 * k_blk: keys blocked and transposed, fp32 [n_kv][l_cap/64][128][64]
 * (position j, dimension d of kv head g at ((g*l_cap/64 + j/64)*128 + d)*64
 * + j%64); v: fp32 [n_kv][l_cap][128].  q: fp32 [n_q][128]; o: fp32
 * [n_q][128].  q, k_blk and v 16-byte aligned; o 4-byte aligned and it
 * must not overlap the inputs or the workspace.  1 <= L <= l_cap < 2^31,
 * l_cap a multiple of 64.
 * workspace: q4s_attn_workspace_bytes(n_q, L) bytes of caller device memory
 * (16-byte aligned) for the per-split partials (max, sum, weighted values);
 * fully overwritten.  Accumulation is fp32 with expf, in a fixed order
 * (deterministic).  Two launches on `stream`.
 */
#define Q4S_ATTN_HEAD_DIM 128
size_t q4s_attn_workspace_bytes(int n_q, int64_t L);
q4s_status q4s_attn_decode(const float* q, const float* k_blk, const float* v, float* o, int n_q, int n_kv,
                           int64_t L, int64_t l_cap, void* workspace, size_t workspace_bytes, void* stream);

/*
 * q4s_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The per-split partials go to a static
 * array of Q4S_ATTN_SCRATCH_BYTES bytes in device memory, one per GPU: it is
 * held from the first call on that GPU until the process ends, and the
 * library takes its address once per GPU (the calling thread's current
 * device, which must be the device of `stream`).  Everything else -- the
 * arguments, their checks, the kernels and the results, bit for bit -- is as
 * for q4s_attn_decode.  A call whose partials, q4s_attn_workspace_bytes(n_q,
 * L), exceed Q4S_ATTN_SCRATCH_BYTES returns Q4S_ERR_SHAPE and enqueues
 * nothing (12 query heads: L up to 86016).  Nothing is allocated or freed,
 * by the library or anything it calls.  All calls on one GPU share its
 * array, which keeps the last call's partials (every call overwrites all it
 * reads, so nothing needs clearing): calls that may overlap in time on one
 * GPU (other streams, other threads) race and give undefined results.
 */
#define Q4S_ATTN_SCRATCH_BYTES ((size_t)8 << 20)
q4s_status q4s_attn_decode_noalloc(const float* q, const float* k_blk, const float* v, float* o, int n_q,
                                   int n_kv, int64_t L, int64_t l_cap, void* stream);

/* ---------------------------------------------------- layer-stack sweep */

/*
 * One matrix of a sweep.  When x is non-NULL, q4s_sweep_run first quantizes
 * x (fp32 [n][cols], 16-byte aligned) into x_q8; otherwise x_q8 must already
 * hold the planar Q8_0 activation.  y: fp32 [n][rows].
 */
typedef struct {
    const void* w_packed;
    const float* x;
    void* x_q8;
    float* y;
    int64_t rows;
    int64_t cols;
} q4s_mat;

typedef struct q4s_plan q4s_plan; /* opaque; host memory only */

typedef struct {
    int64_t n_mats;
    int64_t n_tiles;          /* workgroups of the GEMV launch                */
    int64_t n_quant_blocks;   /* Q8_0 blocks quantized per run (0: none)      */
    int64_t fused_quantize;   /* 1: quantized inside the GEMV launch          */
    int64_t weight_bytes;     /* canonical Q4_0 bytes of all matrices         */
    int64_t packed_bytes;     /* packed bytes read by one run                 */
    int64_t act_bytes;        /* Q8_0 activation bytes read by one run        */
    int64_t out_bytes;        /* y bytes written by one run                   */
    int64_t dev_bytes;        /* device memory the plan needs                 */
} q4s_plan_info;

/*
 * Build a plan for n activation rows (1..24) over n_mats matrices (the table is
 * copied; the buffers it names must stay valid for every run).  Every matrix
 * is checked as in q4s_gemv_q4_0 (a matrix with x is quantized even when
 * rows == 0).  No y may overlap any w_packed, x_q8 or x of the sweep, and no
 * x_q8 may overlap any x; several matrices may read one x_q8.  *dev_bytes_needed receives the device memory size
 * q4s_sweep_plan_upload needs.  Source: Results paragraph on the roofline and
 * milestone M15 (one persistent launch for every projection of a step).
 */
q4s_status q4s_sweep_plan_create(const q4s_mat* mats, int n_mats, int n,
                                 size_t* dev_bytes_needed, q4s_plan** out);

/*
 * Copy the plan's tables into dev_mem (16-byte aligned, >= dev_bytes_needed
 * bytes, owned by the caller and kept alive while the plan is used).  The copy
 * is enqueued on `stream` from host memory held by the plan.
 */
q4s_status q4s_sweep_plan_upload(q4s_plan* plan, void* dev_mem, size_t dev_bytes, void* stream);
/* (Destroy the plan only after `stream` has completed the upload.) */

/*
 * One sweep: if any matrix has x, one launch quantizes all of them; then one
 * launch streams every matrix's weights once and writes every y.  When n == 1
 * and every matrix has x and rows > 0, there is a single launch instead (the
 * mega kernel of milestone M15 quantizes the activation inside its one kernel):
 * each wave quantizes the activation blocks of the chunks it streams, x_q8
 * still receives the Q8_0 bytes, and the results are bit-identical to the
 * two-launch form.  When n == 1 and no matrix has more than 8 chunks (a
 * single K split), the GEMV launch runs one 8-wave workgroup per (matrix, row
 * group), the row's chunks spread over its waves, instead of tiles of 4 row
 * groups (same results), which keeps every weight load of a plan of few
 * large matrices in flight early.  Calls on one plan must not overlap in
 * time (they share the plan's device tables only for reading, but write the
 * same y and x_q8 buffers).
 */
q4s_status q4s_sweep_run(const q4s_plan* plan, void* stream);

q4s_status q4s_sweep_plan_info(const q4s_plan* plan, q4s_plan_info* info);

/*
 * Timeline of later runs' GEMV launch (the pages' clock-delta profiling of the
 * decode step, milestone M19): with a trace buffer set, for workgroup b of the
 * launch (b < n_tiles of q4s_sweep_plan_info), word 9b receives the GPU's
 * 100 MHz constant clock when b started and word 9b + 1 + w when its wave w
 * finished (4 waves, or 8 for the 1-row plans whose matrices all have at most
 * 8 chunks); other words are left untouched.  trace: q4s_sweep_trace_bytes
 * bytes of device memory (8-byte aligned); NULL turns it off.  Plans of more
 * than 8 rows cannot be traced (Q4S_ERR_PLAN).
 */
size_t q4s_sweep_trace_bytes(const q4s_plan* plan);
q4s_status q4s_sweep_set_trace(q4s_plan* plan, uint64_t* trace, size_t trace_bytes);

void q4s_sweep_plan_destroy(q4s_plan* plan);

/* ------------------------------------------------------ chained step */

/*
 * One decode step for one token with its layers as dependent phases inside a
 * single persistent launch (the pages' mega kernel: "How it works",
 * src/mega.cu bullet; milestones M15 and M19).  A Qwen2-shaped stack of
 * `layers` layers, hidden size E, k/v size D, MLP size F, vocabulary V.  Per
 * layer, with h the layer input (h_0 given):
 *   q = Wq Q8(norm h),  k = Wk Q8(norm h),  v = Wv Q8(norm h)
 *   o = Wo Q8(q),       h1 = h + o
 *   g = Wg Q8(norm h1), u = Wu Q8(norm h1)
 *   dn = Wd Q8(g * u),  h2 = h1 + dn          (the next layer's h)
 * then logits = Wout Q8(norm h_L).  norm(x) = x / sqrt(mean(x^2) + 1e-6)
 * (RMS norm without a learned weight; the sum of squares in a fixed order);
 * Q8 is the Q8_0 quantization of q4s_quantize_q8_0; every GEMV is the
 * q4s_gemv_q4_0 product of that activation, bit for bit; + and * are single
 * fp32 operations.  RoPE, attention and the SiLU are not part of the chain:
 * q feeds the output projection where attention's result would, and the MLP
 * product is g * u.
 *
 * Phase synchronisation (sync_mode):
 *   Q4S_CHAIN_COUNTER  M19's monotonic arrival counter: one device-scope
 *                      release add per workgroup and phase, one acquire fence;
 *   Q4S_CHAIN_TREE     a combining tree of such counters (16 + 1);
 *   Q4S_CHAIN_TAGGED   no barrier: every activation word carries the step's tag
 *                      and readers poll the words they need (relaxed
 *                      device-scope atomics, no fences).
 * The three modes give identical results.
 */
typedef struct {
    int32_t layers; /* >= 0 (0: the head alone)            */
    int32_t hidden; /* E, a multiple of 32, <= 32768        */
    int32_t kv_dim; /* D >= 1 (rows of Wk and Wv)           */
    int32_t ff;     /* F, a multiple of 32, <= 32768        */
    int32_t vocab;  /* V >= 1                               */
} q4s_chain_shape;

#define Q4S_CHAIN_COUNTER 0
#define Q4S_CHAIN_TREE 1
#define Q4S_CHAIN_TAGGED 2

typedef struct q4s_chain q4s_chain; /* opaque; host memory only */

typedef struct {
    int64_t n_mats;       /* 7 * layers + 1                              */
    int64_t n_phases;     /* 4 * layers + 1                              */
    int64_t n_tiles;      /* GEMV workgroup tiles over all phases        */
    int64_t workgroups;   /* persistent workgroups (after upload)        */
    int64_t act_words;    /* 64-bit words of the activation buffer       */
    int64_t packed_bytes; /* packed weight bytes read by one step        */
    int64_t dev_bytes;    /* device memory the chain's tables need       */
    int64_t steps;        /* steps run since the upload                  */
} q4s_chain_info;

/*
 * 64-bit words of the activation buffer: per layer [q E | k D | v D | o E |
 * h1 E | g F | u F | dn E | h2 E], layers one after another.  Word = fp32
 * bits in the low 32 bits, the step's tag in the high 32 bits.  0 on a bad shape.
 */
int64_t q4s_chain_act_words(const q4s_chain_shape* shape);

/*
 * Build a chained step.  w_packed: 7 * layers + 1 packed Q4_0 matrices
 * (q4s_repack_q4_0 output, 16-byte aligned): per layer q [E x E], k, v
 * [D x E], o [E x E], gate, up [F x E], down [E x F], then the head [V x E].
 * h0: fp32 [E] (16-byte aligned), read by every step.  acts: the activation
 * buffer (q4s_chain_act_words words, 16-byte aligned), written by every step.
 * logits: fp32 [V].  Outputs may not overlap inputs or each other.
 * workgroups: 0 for one per compute unit, else the count (at most the number
 * resident at once, checked at upload).  *dev_bytes_needed receives the
 * device memory q4s_chain_upload needs.  The buffers must stay valid while
 * the chain is used.
 */
q4s_status q4s_chain_create(const q4s_chain_shape* shape, const void* const* w_packed, const float* h0,
                            uint64_t* acts, float* logits, int sync_mode, int workgroups,
                            size_t* dev_bytes_needed, q4s_chain** out);

/*
 * Copy the chain's tables into dev_mem (16-byte aligned, caller-owned, kept
 * alive while the chain is used) and zero `acts`, both on `stream`.  dev_mem
 * also holds, past the tables, the step's quantized g * u and q words (written
 * by the gate/up and q tiles, read by down and o; gate and up pair when they
 * have at most two K splits, i.e. E <= 4096) and, with Q4S_CHAIN_TAGGED, the
 * words through which down's K ranges meet when each runs on its own
 * workgroup (four K splits of at most 32 chunks, i.e. 4128 <= F <= 32768);
 * the upload zeroes both.  Needs the GPU: resolves and checks the workgroup
 * count.
 */
q4s_status q4s_chain_upload(q4s_chain* chain, void* dev_mem, size_t dev_bytes, void* stream);

/*
 * One step: a small clearing launch, then one cooperative launch of the
 * persistent workgroups on `stream`.  Each step gets a new tag.  Steps on one
 * chain must not overlap in time.  Waits inside the launch are bounded; when
 * one gives up the step's results are invalid and q4s_chain_check reports it.
 */
q4s_status q4s_chain_run(q4s_chain* chain, void* stream);

/* Synchronize `stream`; Q4S_ERR_WAIT if a wait of the last step gave up. */
q4s_status q4s_chain_check(const q4s_chain* chain, void* stream);

/*
 * Polls a wait of later steps may spend before it gives up (default 2^20,
 * about a second; 0: give up at the first read that is not ready yet).  A
 * step whose wait gave up still runs to its end; its results are invalid and
 * q4s_chain_check reports Q4S_ERR_WAIT.  The next step starts afresh.
 */
q4s_status q4s_chain_set_wait_limit(q4s_chain* chain, uint32_t polls);

/*
 * How later steps launch the persistent workgroups: cooperative != 0 (the
 * default) through the cooperative-launch call, which guarantees that all of
 * them are resident at once; 0 through a plain launch, for tools that do not
 * handle cooperative launches (the profiler).  The workgroup count never
 * exceeds what the GPU can hold at once, so on an otherwise idle GPU a plain
 * launch also starts them all; where it cannot (other work holding the GPU),
 * the bounded waits give up and q4s_chain_check reports Q4S_ERR_WAIT.
 * Results are the same either way.
 */
q4s_status q4s_chain_set_cooperative(q4s_chain* chain, int cooperative);

q4s_status q4s_chain_get_info(const q4s_chain* chain, q4s_chain_info* info);

/*
 * Phase timeline of later steps (the clock-delta profiling of milestone M19):
 * with a trace buffer set, every step records, with P = n_phases and
 * W = workgroups, slot s = p * W + b for phase p and workgroup b:
 *   trace[s]              when workgroup b finished phase p;
 *   trace[P * W + b]      when workgroup b started;
 *   trace[P * W + W + s]  when b started its first tile of phase p;
 *   trace[2 P W + W + s]  when that tile's activation prologue was done (its
 *                         input had arrived, been normalized and quantized).
 * The tile entries are left untouched for workgroups without a tile in a phase,
 * so the caller zeroes the buffer before setting it.  Times are the GPU's 100 MHz
 * constant clock.  trace: q4s_chain_trace_bytes bytes of device memory
 * (8-byte aligned; 0 before upload); NULL turns tracing off.  One thread per
 * workgroup stores the marks.
 */
size_t q4s_chain_trace_bytes(const q4s_chain* chain);
q4s_status q4s_chain_set_trace(q4s_chain* chain, uint64_t* trace, size_t trace_bytes);

/*
 * Test hook: the Q8_0 input each phase's GEMVs read, as staged by the step
 * (after the wait, the RMS norm where the phase has one, the quantization;
 * or, for o and down, the codes their producers wrote).  With a dump buffer
 * set, every later step writes, for phase p (4 per layer: q/k/v, o, gate/up,
 * down; then the head) and chunk c of the phase's activation (256 values),
 * at word (p * C + c) * 64 + l, C = max(ceil(E/256), ceil(F/256)): the code
 * dword l of the chunk (int8 values 256c + 4l .. 256c + 4l + 3, low byte
 * first; zero past the vector) in the low half and the fp32 bits of the
 * binary16 d_x of its block (8c + l/8) in the high half.  Words of chunks a
 * phase does not have are left untouched.  dump:
 * q4s_chain_stage_dump_bytes bytes of device memory (8-byte aligned); NULL
 * turns it off.  Source: the pages validate every GPU kernel of the decode
 * step against the CPU reference ("How it works", src/cpu_infer.cpp bullet;
 * milestones M15, M19).
 */
size_t q4s_chain_stage_dump_bytes(const q4s_chain* chain);
q4s_status q4s_chain_set_stage_dump(q4s_chain* chain, uint64_t* dump, size_t dump_bytes);

void q4s_chain_destroy(q4s_chain* chain);

/* -------------------------------------------------- measurement helpers */

/*
 * Streaming-read microbenchmark (the roofline kernel of milestone M15): reads
 * `bytes` (a multiple of 16) from `buf` (16-byte aligned) with 16-byte loads,
 * `loads_in_flight` (1, 2, 4 or 8) per thread per iteration, using `n_blocks`
 * workgroups of 256 threads (0: 2048); writes one word to `sink` (device,
 * 4 bytes) only if a practically impossible checksum occurs.
 */
q4s_status q4s_bench_read(const void* buf, size_t bytes, int loads_in_flight, int n_blocks,
                          uint32_t* sink, void* stream);

/*
 * Streaming read in the GEMV's own pattern: wave i of the launch reads unit i,
 * `unit_bytes` contiguous bytes (a positive multiple of 1024, at most 1 GiB),
 * with 1 KB wave-wide loads (16 bytes per lane), nine in flight, one
 * workgroup of 4 waves per 4 units; the floor(bytes / unit_bytes) whole units
 * of `buf` (16-byte aligned) are read, a tail shorter than a unit is not.
 * This is the achievable-bandwidth reference for the weight stream (the
 * grid-stride q4s_bench_read puts its loads in flight at power-of-two
 * strides, which some grid sizes serve far more slowly).  `sink` as for
 * q4s_bench_read.
 */
q4s_status q4s_bench_read_units(const void* buf, size_t bytes, size_t unit_bytes, uint32_t* sink, void* stream);

/*
 * Grid-barrier microbenchmark (the phase barriers of a chained decode step):
 * one persistent cooperative launch of n_workgroups x 256 threads (1..the
 * number resident at once, see below) that passes `phases` grid barriers.
 * kind 0: milestone M19's monotonic arrival counter (one device-scope atomic
 * add per arrival on one word, everyone polls it with acquire loads);
 * kind 1: each workgroup stores its phase number into its own 128-byte line,
 * workgroup 0 polls them all and stores a release word; kind 2: a combining
 * tree of monotonic counters (16 sub-counters, then a top counter whose last
 * arrival stores the release word; relaxed polls and one acquire fence);
 * kind 3: kind 0 with relaxed polls and one acquire fence; kinds 4, 5, 6:
 * kind 2 with every sub-counter in its own 1 KB, 4 KB or 64 KB slot that also
 * holds a copy of the release word, polled by that sub-counter's workgroups;
 * kinds 7, 8: kind 2 with relaxed arrivals and an acquire fence, or with no
 * fence; kind 9: kind 0 with no fence (fence-cost measurements only: they
 * order no data).
 * scratch:
 * q4s_bench_grid_barrier_scratch_bytes bytes of device memory (4-byte
 * aligned), zeroed by the call; word 1 becomes nonzero if a workgroup gave up
 * waiting (a bounded poll: the launch always
 * ends).  The caller times the launch.
 */
size_t q4s_bench_grid_barrier_scratch_bytes(int n_workgroups);
q4s_status q4s_bench_grid_barrier(int kind, int n_workgroups, int phases, uint32_t* scratch,
                                  size_t scratch_bytes, void* stream);

/* Workgroups of q4s_bench_grid_barrier that fit on the device at once (0 on error). */
int q4s_bench_grid_barrier_max_workgroups(void);

/* Plain 16-byte copy of `bytes` (a multiple of 16) from src to dst. */
q4s_status q4s_bench_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4S_H */
