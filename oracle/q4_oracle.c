/*
 * q4_oracle.c -- plain CPU oracle for the Q4_0-weight x Q8_0-activation product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or constant with the GPU path.
 *
 * Sources (the "minfer" README, "nano-inference" page):
 *   - "How it works", src/gguf.h bullet: weights are Q4_0 GGUF tensors.
 *   - Milestone log M3.5: int8 activations and integer MACs per block.
 *   - Milestone log M9: Q4_0 element value is (nibble - 8) times the block
 *     scale; the product is an integer sum per block, scaled afterwards.
 *   - Milestone log M14: block byte sizes (Q4_0 lm_head 131 MB and Q8_0
 *     lm_head 248 MB at 151936 x 1536), which fix 18 B and 34 B blocks.
 *   - "How it works", src/mega.cu bullet and M16: per-block integer sums,
 *     accumulated through one float expression.
 *   - Milestones M6 and M14, and the gemv_q8_dp4a bullet of "How it works":
 *     the lm_head stored as Q8_0 weights (34 B blocks of 32 int8 values and a
 *     binary16 scale), multiplied by the same int8 activations.
 *   - Milestones M14 and M18: 8-bit heads requantized to Q4_0 at load.
 *   - Milestones M5, M12 and M15, and the model details (12 query heads over
 *     2 key/value heads of dimension 128): decode attention over a KV cache.
 *   - Milestone M16 ("every float operation explicitly rounded", logits
 *     independent of the step size): the GEMV in one fixed fp32 order.
 *   - "How it works", src/mega.cu bullet, and milestones M15 and M19: a
 *     token's layers run as dependent phases (norm prologue, activation
 *     quantize, GEMV, residual) inside one kernel -- the chained step.
 *
 * Block formats (GGUF convention, where the pages leave the byte order open):
 *   Q4_0 (18 B / 32 weights): fp16 scale d (little-endian), then 16 bytes qs.
 *        element j < 16 is qs[j] & 0xF, element j >= 16 is qs[j-16] >> 4;
 *        weight value = (nibble - 8) * d.
 *   Q8_0 (34 B / 32 values): fp16 scale d (little-endian), then 32 int8 q.
 *        d = max|x| / 127 (fp32, correctly rounded), q = round-half-away(x / d)
 *        with the fp32 d as the divisor; stored d = fp16(d), round to nearest
 *        even, subnormals kept.  An all-zero block stores d = +0 and q = 0.
 *
 * Q8_0-weight GEMV: as below with s = sum_j w_j * q_j (int8 weights, no offset).
 *
 * GEMV definition (exact up to the final rounding):
 *   s[n][r][b] = sum_j (nibble_{r,b,j} - 8) * q_{n,b,j}          (int32, literal)
 *   t          = (d_w[r][b] * d_x[n][b]) * s                      (exact in fp64)
 *   y[n][r]    = fp32( sum_b t )                                  (fp64 sum)
 *   S[n][r]    = sum_b |t|                                        (tolerance scale)
 *
 * Every function here is written for clarity, not speed: one output row at a
 * time, one element at a time.  The only parallelism is OpenMP over
 * independent output rows, which changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32
#define Q4_BLOCK_BYTES 18
#define Q8_BLOCK_BYTES 34

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition. */
/* ------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float q4o_fp16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 (zero when m == 0) */
    } else if (e == 31) {
        if (m == 0)
            v = INFINITY;
        else
            return sign ? -NAN : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v); /* exact: every binary16 value is a binary32 value */
}

/* Nearest binary16 value, ties to even fraction, overflow to infinity. */
uint16_t q4o_f32_to_fp16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00);
    double a = fabs((double)f);
    if (isinf(f))
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    /* spacing of the binary16 grid around a */
    int e2;
    frexp(a, &e2);            /* a = fr * 2^e2, fr in [0.5, 1): 2^(e2-1) <= a < 2^e2 */
    int e = e2 - 1;           /* 2^e <= a < 2^(e+1) */
    if (e < -14)
        e = -14;              /* subnormal range shares the spacing of the lowest binade */
    double spacing = ldexp(1.0, e - 10);
    double k = a / spacing;   /* exact: power-of-two division of a 24-bit value */
    double r = nearbyint(k);  /* default rounding mode: nearest, ties to even */
    double v = r * spacing;   /* the rounded magnitude */
    if (v >= 65536.0)
        return (uint16_t)(sign | 0x7c00); /* above the largest finite 65504 */
    if (v < ldexp(1.0, -14))
        return (uint16_t)(sign | (uint16_t)r); /* subnormal: fraction = r */
    int ev2;
    frexp(v, &ev2);
    int ev = ev2 - 1; /* 2^ev <= v < 2^(ev+1) */
    uint32_t frac = (uint32_t)(v / ldexp(1.0, ev - 10)) - 1024u;
    return (uint16_t)(sign | (uint16_t)((ev + 15) << 10) | (uint16_t)frac);
}

void q4o_fp16_to_f32_array(const uint16_t* h, float* f, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        f[i] = q4o_fp16_to_f32(h[i]);
}

void q4o_f32_to_fp16_array(const float* f, uint16_t* h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = q4o_f32_to_fp16(f[i]);
}

static uint16_t load_u16_le(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void store_u16_le(uint8_t* p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------ */
/* Q8_0 quantization of one 32-value block.                             */
/* ------------------------------------------------------------------ */

void q4o_quantize_q8_0_block(const float* x, uint8_t* out /* 34 B */)
{
    float amax = 0.0f;
    for (int j = 0; j < QK; ++j) {
        float a = fabsf(x[j]);
        if (a > amax)
            amax = a;
    }
    float d = amax / 127.0f; /* fp32, correctly rounded */
    store_u16_le(out, q4o_f32_to_fp16(d));
    int8_t* q = (int8_t*)(out + 2);
    for (int j = 0; j < QK; ++j) {
        if (amax == 0.0f) {
            q[j] = 0;
            continue;
        }
        float v = x[j] / d;   /* fp32, correctly rounded */
        float r = roundf(v);  /* half away from zero */
        q[j] = (int8_t)(int)r;
    }
}

/* x: n_elems fp32 values (n_elems % 32 == 0) -> n_elems/32 blocks of 34 B. */
void q4o_quantize_q8_0(const float* x, uint8_t* blocks, int64_t n_elems)
{
    int64_t nb = n_elems / QK;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b)
        q4o_quantize_q8_0_block(x + b * QK, blocks + b * Q8_BLOCK_BYTES);
}

/* ------------------------------------------------------------------ */
/* Q4_0 decode and the per-block integer dot.                           */
/* ------------------------------------------------------------------ */

/* nibble value of element j (0..31) of a Q4_0 block */
static int q4_nibble(const uint8_t* blk, int j)
{
    const uint8_t* qs = blk + 2;
    return j < 16 ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);
}

/* blocks -> d (fp32) and the 32 nibbles (0..15) of each block */
void q4o_decode_q4_0(const uint8_t* blocks, float* d, uint8_t* nibbles, int64_t n_blocks)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t* blk = blocks + b * Q4_BLOCK_BYTES;
        d[b] = q4o_fp16_to_f32(load_u16_le(blk));
        for (int j = 0; j < QK; ++j)
            nibbles[b * QK + j] = (uint8_t)q4_nibble(blk, j);
    }
}

/* s = sum_j (nibble_j - 8) * q_j, summed literally (no offset folding). */
int32_t q4o_block_dot(const uint8_t* q4_block, const uint8_t* q8_block)
{
    const int8_t* q = (const int8_t*)(q8_block + 2);
    int32_t s = 0;
    for (int j = 0; j < QK; ++j)
        s += (q4_nibble(q4_block, j) - 8) * (int32_t)q[j];
    return s;
}

/*
 * w   : [rows][cols/32] Q4_0 blocks, row-major (K contiguous)
 * xq8 : [n][cols/32] Q8_0 blocks
 * s   : [n][rows][cols/32] int32
 */
void q4o_block_sums(const uint8_t* w, const uint8_t* xq8, int64_t rows, int64_t cols, int n,
                    int32_t* s)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int t = 0; t < n; ++t)
            for (int64_t b = 0; b < nb; ++b)
                s[((int64_t)t * rows + r) * nb + b] =
                    q4o_block_dot(w + (r * nb + b) * Q4_BLOCK_BYTES,
                                  xq8 + ((int64_t)t * nb + b) * Q8_BLOCK_BYTES);
}

/* One output element: y (fp32), its fp64 value and S = sum |t|. */
static void gemv_one(const uint8_t* wrow, const uint8_t* xrow, int64_t nb, float* y, double* y64,
                     double* scale)
{
    double acc = 0.0, sabs = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* wb = wrow + b * Q4_BLOCK_BYTES;
        const uint8_t* xb = xrow + b * Q8_BLOCK_BYTES;
        double dw = (double)q4o_fp16_to_f32(load_u16_le(wb));
        double dx = (double)q4o_fp16_to_f32(load_u16_le(xb));
        double p = dw * dx;                 /* exact: two 11-bit significands */
        double t = p * (double)q4o_block_dot(wb, xb); /* exact: <= 38 significant bits */
        acc += t;
        sabs += fabs(t);
    }
    if (y)
        *y = (float)acc;
    if (y64)
        *y64 = acc;
    if (scale)
        *scale = sabs;
}

/*
 * y, scale, y64 : [n][rows] (scale and y64 may be NULL)
 */
void q4o_gemv(const uint8_t* w, const uint8_t* xq8, int64_t rows, int64_t cols, int n, float* y,
              double* scale, double* y64)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int t = 0; t < n; ++t) {
            int64_t o = (int64_t)t * rows + r;
            gemv_one(w + r * nb * Q4_BLOCK_BYTES, xq8 + (int64_t)t * nb * Q8_BLOCK_BYTES, nb,
                     y ? y + o : 0, y64 ? y64 + o : 0, scale ? scale + o : 0);
        }
}

/*
 * Selected rows only: row_idx[i] indexes the full matrix w ([rows][cols/32]);
 * y, scale : [n][n_idx].
 */
void q4o_gemv_rows(const uint8_t* w, const uint8_t* xq8, int64_t cols, int n,
                   const int64_t* row_idx, int64_t n_idx, float* y, double* scale)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_idx; ++i)
        for (int t = 0; t < n; ++t) {
            int64_t o = (int64_t)t * n_idx + i;
            gemv_one(w + row_idx[i] * nb * Q4_BLOCK_BYTES, xq8 + (int64_t)t * nb * Q8_BLOCK_BYTES,
                     nb, y ? y + o : 0, 0, scale ? scale + o : 0);
        }
}

/* ------------------------------------------------------------------ */
/* The GEMV in one fixed fp32 order.                                    */
/* ------------------------------------------------------------------ */

/*
 * Milestone M16 makes every float operation of a token explicitly rounded so
 * that its result does not depend on how many tokens share the step; that
 * fixes one expression per block and one accumulation order.  The pages leave
 * the order itself open; the one taken (the GPU path's) is:
 *   - the blocks of a row are cut into chunks of 8, nc = ceil(nb / 8) chunks;
 *   - the chunks are split into ks contiguous ranges, ks = 1 if nc <= 8,
 *     2 if nc <= 16, else 4; range s is [floor(s*nc/ks), floor((s+1)*nc/ks));
 *   - within a range, blocks 0-3 of every chunk feed chain A and blocks 4-7
 *     chain B, one fmaf(d_w * d_x, (float)s, chain) per block in chunk order
 *     (d_w * d_x, two binary16 values, is exact in fp32);
 *   - after the 16th, 32nd, ... chunk of a range and after its last chunk:
 *     total = total + (A + B), and both chains restart at 0;
 *   - y = ((total_0 + total_1) + total_2) + total_3, left to right.
 * Missing blocks of a last, partial chunk add nothing.
 */
static float gemv_one_f32(const uint8_t* wrow, const uint8_t* xrow, int64_t nb)
{
    const int64_t nc = (nb + 7) / 8;
    const int64_t ks = nc <= 8 ? 1 : (nc <= 16 ? 2 : 4);
    float y = 0.0f;
    for (int64_t s = 0; s < ks; ++s) {
        const int64_t c0 = s * nc / ks, c1 = (s + 1) * nc / ks;
        float total = 0.0f, chain_a = 0.0f, chain_b = 0.0f;
        for (int64_t c = c0; c < c1; ++c) {
            for (int64_t k = 0; k < 8 && c * 8 + k < nb; ++k) {
                const uint8_t* wb = wrow + (c * 8 + k) * Q4_BLOCK_BYTES;
                const uint8_t* xb = xrow + (c * 8 + k) * Q8_BLOCK_BYTES;
                const float scale = q4o_fp16_to_f32(load_u16_le(wb)) * q4o_fp16_to_f32(load_u16_le(xb));
                const float sum = (float)q4o_block_dot(wb, xb);
                if (k < 4)
                    chain_a = fmaf(scale, sum, chain_a);
                else
                    chain_b = fmaf(scale, sum, chain_b);
            }
            if (c + 1 == c1 || (c + 1 - c0) % 16 == 0) {
                total = total + (chain_a + chain_b);
                chain_a = 0.0f;
                chain_b = 0.0f;
            }
        }
        y = s == 0 ? total : y + total;
    }
    return y;
}

/* y : [n][rows], every element in the order above */
void q4o_gemv_f32(const uint8_t* w, const uint8_t* xq8, int64_t rows, int64_t cols, int n, float* y)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int t = 0; t < n; ++t)
            y[(int64_t)t * rows + r] =
                gemv_one_f32(w + r * nb * Q4_BLOCK_BYTES, xq8 + (int64_t)t * nb * Q8_BLOCK_BYTES, nb);
}

/* selected rows of the full matrix: y : [n][n_idx] */
void q4o_gemv_f32_rows(const uint8_t* w, const uint8_t* xq8, int64_t cols, int n, const int64_t* row_idx,
                       int64_t n_idx, float* y)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_idx; ++i)
        for (int t = 0; t < n; ++t)
            y[(int64_t)t * n_idx + i] =
                gemv_one_f32(w + row_idx[i] * nb * Q4_BLOCK_BYTES, xq8 + (int64_t)t * nb * Q8_BLOCK_BYTES, nb);
}

/* ------------------------------------------------------------------ */
/* RMS normalization and the chained token step.                        */
/* ------------------------------------------------------------------ */

/*
 * out_i = x_i / sqrt(ss / n + 1e-6), all fp32, sqrt and division correctly
 * rounded, with no learned weight (the synthetic model's norm weights are 1).
 * Qwen2.5's RMS norm with its epsilon of 1e-6; the pages name "norm
 * prologues" (M19) without a formula.  The sum of squares ss is taken in a
 * fixed order: 64 partial sums, p_l an fmaf chain over the elements
 * 256c + 4l + k (k = 0..3) of every 256-element chunk c in turn (those below
 * n), then for d = 32, 16, 8, 4, 2, 1 every p_l becomes p_l + p_{l xor d}
 * (all at once); ss = p_0.  Returns ss.
 */
float q4o_rmsnorm(const float* x, int64_t n, float* out)
{
    float p[64], q[64];
    for (int l = 0; l < 64; ++l) {
        p[l] = 0.0f;
        for (int64_t c = 0; c * 256 < n; ++c)
            for (int k = 0; k < 4; ++k) {
                const int64_t i = c * 256 + 4 * l + k;
                if (i < n)
                    p[l] = fmaf(x[i], x[i], p[l]);
            }
    }
    for (int d = 32; d >= 1; d /= 2) {
        for (int l = 0; l < 64; ++l)
            q[l] = p[l] + p[l ^ d];
        memcpy(p, q, sizeof p);
    }
    const float ss = p[0];
    const float s = sqrtf(ss / (float)n + 1e-6f);
    for (int64_t i = 0; i < n; ++i)
        out[i] = x[i] / s;
    return ss;
}

/* y = W * Q8(x) for one token, in the fixed fp32 order (scratch: cols/32 Q8_0 blocks) */
static void chain_gemv(const uint8_t* w, int64_t rows, int64_t cols, const float* x, uint8_t* scratch, float* y)
{
    q4o_quantize_q8_0(x, scratch, cols);
    q4o_gemv_f32(w, scratch, rows, cols, 1, y);
}

/*
 * One chained decode step for one token.  The pages' mega kernel runs a
 * token's layers as dependent phases (norm prologue, activation quantize,
 * GEMV, residual; "How it works", src/mega.cu bullet, M15, M19).  The chain
 * keeps the projections and the glue between them; RoPE, attention and the
 * SiLU are outside it (q goes straight to the output projection, where
 * attention's result would enter, and the MLP product is g * u).  Per layer,
 * with h the layer input (h_0 given):
 *   q = Wq Q8(norm h),  k = Wk Q8(norm h),  v = Wv Q8(norm h)
 *   o = Wo Q8(q),       h1 = h + o
 *   g = Wg Q8(norm h1), u = Wu Q8(norm h1)
 *   dn = Wd Q8(g * u),  h2 = h1 + dn          (the next layer's h)
 * and the logits z = Wout Q8(norm h_L).  + and * are single fp32 operations.
 *
 * w    : 7 * layers + 1 canonical Q4_0 matrices: per layer q [E x E], k, v
 *        [D x E], o [E x E], gate, up [F x E], down [E x F]; then the head [V x E]
 * acts : per layer [q E | k D | v D | o E | h1 E | g F | u F | dn E | h2 E]
 */
void q4o_chain_step(const uint8_t* const* w, int layers, int64_t E, int64_t D, int64_t F, int64_t V,
                    const float* h0, float* acts, float* logits)
{
    const int64_t big = E > F ? E : F;
    float* nrm = (float*)malloc((size_t)big * sizeof(float));
    float* prod = (float*)malloc((size_t)F * sizeof(float));
    uint8_t* xq = (uint8_t*)malloc((size_t)(big / QK) * Q8_BLOCK_BYTES);
    const int64_t per_layer = 5 * E + 2 * D + 2 * F;
    const float* h = h0;
    for (int l = 0; l < layers; ++l) {
        const uint8_t* const* lw = w + 7 * l;
        float* a = acts + l * per_layer;
        float *q = a, *k = q + E, *v = k + D, *o = v + D, *h1 = o + E, *g = h1 + E, *u = g + F, *dn = u + F,
              *h2 = dn + E;
        q4o_rmsnorm(h, E, nrm);
        chain_gemv(lw[0], E, E, nrm, xq, q);
        chain_gemv(lw[1], D, E, nrm, xq, k);
        chain_gemv(lw[2], D, E, nrm, xq, v);
        chain_gemv(lw[3], E, E, q, xq, o);
        for (int64_t i = 0; i < E; ++i)
            h1[i] = h[i] + o[i];
        q4o_rmsnorm(h1, E, nrm);
        chain_gemv(lw[4], F, E, nrm, xq, g);
        chain_gemv(lw[5], F, E, nrm, xq, u);
        for (int64_t i = 0; i < F; ++i)
            prod[i] = g[i] * u[i];
        chain_gemv(lw[6], E, F, prod, xq, dn);
        for (int64_t i = 0; i < E; ++i)
            h2[i] = h1[i] + dn[i];
        h = h2;
    }
    q4o_rmsnorm(h, E, nrm);
    chain_gemv(w[7 * layers], V, E, nrm, xq, logits);
    free(nrm);
    free(prod);
    free(xq);
}

/* ------------------------------------------------------------------ */
/* Q8_0 weights (the 8-bit lm_head of milestones M6 and M14).           */
/* ------------------------------------------------------------------ */

/* s = sum_j w_j * q_j over two Q8_0 blocks (weight block, activation block). */
int32_t q4o_q8w_block_dot(const uint8_t* w_block, const uint8_t* x_block)
{
    const int8_t* w = (const int8_t*)(w_block + 2);
    const int8_t* q = (const int8_t*)(x_block + 2);
    int32_t s = 0;
    for (int j = 0; j < QK; ++j)
        s += (int32_t)w[j] * (int32_t)q[j];
    return s;
}

/* w: [rows][cols/32] Q8_0 weight blocks; xq8: [n][cols/32] Q8_0 blocks; s: [n][rows][cols/32] */
void q4o_q8w_block_sums(const uint8_t* w, const uint8_t* xq8, int64_t rows, int64_t cols, int n,
                        int32_t* s)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int t = 0; t < n; ++t)
            for (int64_t b = 0; b < nb; ++b)
                s[((int64_t)t * rows + r) * nb + b] =
                    q4o_q8w_block_dot(w + (r * nb + b) * Q8_BLOCK_BYTES,
                                      xq8 + ((int64_t)t * nb + b) * Q8_BLOCK_BYTES);
}

/* y, scale, y64: [n][rows]; y = fp32(sum_b (d_w d_x) s), summed in fp64 */
void q4o_q8w_gemv(const uint8_t* w, const uint8_t* xq8, int64_t rows, int64_t cols, int n, float* y,
                  double* scale, double* y64)
{
    int64_t nb = cols / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int t = 0; t < n; ++t) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* wb = w + (r * nb + b) * Q8_BLOCK_BYTES;
                const uint8_t* xb = xq8 + ((int64_t)t * nb + b) * Q8_BLOCK_BYTES;
                double p = (double)q4o_fp16_to_f32(load_u16_le(wb)) *
                           (double)q4o_fp16_to_f32(load_u16_le(xb));
                double tv = p * (double)q4o_q8w_block_dot(wb, xb); /* exact: <= 42 bits */
                acc += tv;
                sabs += fabs(tv);
            }
            int64_t o = (int64_t)t * rows + r;
            if (y)
                y[o] = (float)acc;
            if (y64)
                y64[o] = acc;
            if (scale)
                scale[o] = sabs;
        }
}

/* ------------------------------------------------------------------ */
/* Q8_0 -> Q4_0 requantization at load (milestones M14 and M18).        */
/* The pages name the conversion but not the Q4_0 rounding rule; this   */
/* takes the GGUF reference rule for the format: the element of largest */
/* magnitude (first one on ties) maps to nibble 0, d = that value / -8, */
/* nibble = min(15, trunc(x / d + 8.5)) with x / d formed as x * (1/d), */
/* all in fp32, and the stored scale is fp16(d).                        */
/* ------------------------------------------------------------------ */

void q4o_requant_block_q8_0_to_q4_0(const uint8_t* q8_block, uint8_t* q4_block)
{
    float d8 = q4o_fp16_to_f32(load_u16_le(q8_block));
    const int8_t* q = (const int8_t*)(q8_block + 2);
    float x[QK];
    for (int j = 0; j < QK; ++j)
        x[j] = (float)q[j] * d8; /* exact: 8-bit times 11-bit significand */
    float amax = 0.0f, vmax = 0.0f;
    for (int j = 0; j < QK; ++j) {
        if (fabsf(x[j]) > amax) {
            amax = fabsf(x[j]);
            vmax = x[j];
        }
    }
    float d = vmax / -8.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    store_u16_le(q4_block, q4o_f32_to_fp16(d));
    int nib[QK];
    for (int j = 0; j < QK; ++j) {
        float v = x[j] * id + 8.5f; /* two roundings: the product, then the sum */
        int n = (int)v;             /* truncation toward zero; v >= 0 here */
        nib[j] = n > 15 ? 15 : n;
    }
    for (int j = 0; j < 16; ++j)
        q4_block[2 + j] = (uint8_t)(nib[j] | (nib[j + 16] << 4));
}

/* w_q8: [rows][cols/32] Q8_0 blocks -> w_q4: [rows][cols/32] Q4_0 blocks */
void q4o_requant_q8_0_to_q4_0(const uint8_t* w_q8, uint8_t* w_q4, int64_t n_blocks)
{
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < n_blocks; ++b)
        q4o_requant_block_q8_0_to_q4_0(w_q8 + b * Q8_BLOCK_BYTES, w_q4 + b * Q4_BLOCK_BYTES);
}

/* ------------------------------------------------------------------ */
/* Decode attention over a KV cache (milestones M5, M12, M15; model     */
/* details: 12 query heads share 2 key/value heads, head dim 128).      */
/* One new query per head attends to all L cached positions:            */
/*   s_hj = scale * sum_i q[h][i] * k[j][g][i],  g = h / (n_q / n_kv)  */
/*   p_hj = exp(s_hj - max_j s_hj) / sum_j exp(s_hj - max_j s_hj)      */
/*   o[h][i] = sum_j p_hj * v[j][g][i]                                  */
/* all in fp64; o_abs[h][i] = sum_j p_hj * |v[j][g][i]| (tolerance).    */
/* k, v: fp32 [L][n_kv][hd] (token-major); q, o: [n_q][hd].            */
/* ------------------------------------------------------------------ */

void q4o_attn_decode(const float* q, const float* k, const float* v, int64_t L, int n_q, int n_kv, int hd,
                     double scale, double* o, double* o_abs)
{
    int group = n_q / n_kv;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < n_q; ++h) {
        int g = h / group;
        double smax = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
            double dot = 0.0;
            for (int i = 0; i < hd; ++i)
                dot += (double)q[h * hd + i] * (double)k[(j * n_kv + g) * hd + i];
            double sc = scale * dot;
            if (sc > smax)
                smax = sc;
        }
        double denom = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double dot = 0.0;
            for (int i = 0; i < hd; ++i)
                dot += (double)q[h * hd + i] * (double)k[(j * n_kv + g) * hd + i];
            denom += exp(scale * dot - smax);
        }
        for (int i = 0; i < hd; ++i) {
            o[h * hd + i] = 0.0;
            if (o_abs)
                o_abs[h * hd + i] = 0.0;
        }
        for (int64_t j = 0; j < L; ++j) {
            double dot = 0.0;
            for (int i = 0; i < hd; ++i)
                dot += (double)q[h * hd + i] * (double)k[(j * n_kv + g) * hd + i];
            double p = exp(scale * dot - smax) / denom;
            for (int i = 0; i < hd; ++i) {
                double vv = (double)v[(j * n_kv + g) * hd + i];
                o[h * hd + i] += p * vv;
                if (o_abs)
                    o_abs[h * hd + i] += p * fabs(vv);
            }
        }
    }
}

void q4o_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int q4o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
