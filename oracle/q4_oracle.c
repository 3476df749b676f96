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
