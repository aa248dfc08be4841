/*
 * oracle.c -- plain CPU oracle for the Hadamard-rotated W4A4 prompt GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; it is written from the pages' description of the method:
 *
 *   [H32]  "509 tokens a second of prompt: the Hadamard route ships",
 *          sections "Why prompts are a matrix-unit problem" and "The rotation".
 *   [27B]  "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit
 *          activations with a Hadamard rotation", section "Prompt processing:
 *          4-bit activations, rotated first".
 *   [MOE]  "Where the engine is going: HRX and the NPU", section "4-bit
 *          activations reach the MoE experts".
 *
 * What the pages fix, and the readings taken where they are silent:
 *   - activations are rotated per 32-value block by a 32-point Walsh-Hadamard
 *     transform and rounded in blocks of 32 that share one scale [H32 "The
 *     rotation"];
 *   - the transform is Sylvester (natural) order, H[i][j] = (-1)^popcount(i&j),
 *     computed as 5 butterfly stages h = 1,2,4,8,16 in fp32, lower index gets
 *     a+b and upper gets a-b, each a single fp32 rounding, then every value is
 *     multiplied by fp32(1/sqrt(32)) (reading: the pages only say "orthogonal");
 *   - scale d = amax/7 (IEEE fp32 division), code q = clamp(rint(v/d), -8, 7)
 *     with round-half-to-even; a block whose scale is 0 (all-zero, or so small
 *     that amax/7 underflows) has codes 0, which is what every code of it
 *     dequantizes to (reading: the pages give no formula).  The 8-bit route uses amax/127 and
 *     clamps to +-127 (reading: "exact 8-bit activations" is named, not given);
 *   - a Q4_0 weight code u means u-8 [H32 "Why prompts are a matrix-unit
 *     problem"]; a Q4_0 block is an fp16 scale followed by 16 bytes, byte j
 *     holding element j in its low nibble and element j+16 in its high nibble
 *     (reading: the block layout is not printed; an 18-byte block matches a
 *     4.5-bit file);
 *   - each 32-block dot product is an exact int32 sum; the output
 *     y = sum_b da*dw*S is accumulated in fp64, b ascending.
 *
 * Compiled with -O2 -ffp-contract=off and without fast-math, on x86-64 where
 * float arithmetic is IEEE single precision (SSE), so every fp32 operation
 * below is one correctly rounded operation.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32 /* values per block */

/* ------------------------------------------------------------------ */
/* fp16 <-> fp64, written from the IEEE 754 binary16 definition        */
/* (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).       */
/* ------------------------------------------------------------------ */

double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 15 - 10);
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a == 0.0)
        return sign;
    int E;
    frexp(a, &E);      /* a = f * 2^E, f in [0.5, 1) */
    int ex = E - 1;    /* a = g * 2^ex, g in [1, 2) */
    if (ex < -14) {
        /* subnormal range: quantum 2^-24; m == 1024 lands on the smallest
           normal, whose encoding is exactly 0x0400 */
        double m = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    double m = rint(ldexp(a, 10 - ex)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        ex += 1;
    }
    if (ex > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | ((ex + 15) << 10) | ((int)m - 1024));
}

/* ------------------------------------------------------------------ */
/* The rotation [H32 "The rotation"].                                  */
/* ------------------------------------------------------------------ */

/* fp32(1/sqrt(32)): sqrt(2)/8 in double is correctly rounded (the division
   by 8 is exact), then rounded once more to fp32. */
static float inv_sqrt32_f32(void) { return (float)(sqrt(2.0) / 8.0); }
static double inv_sqrt32_f64(void) { return sqrt(2.0) / 8.0; }

float orc_inv_sqrt32_f32(void) { return inv_sqrt32_f32(); }

/* Unnormalised Walsh-Hadamard butterflies in fp32, stages h = 1,2,4,8,16. */
static void wht32_butterflies_f32(float v[QK])
{
    for (int h = 1; h < QK; h <<= 1)
        for (int j = 0; j < QK; j++)
            if ((j & h) == 0) {
                float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

static void wht32_butterflies_f64(double v[QK])
{
    for (int h = 1; h < QK; h <<= 1)
        for (int j = 0; j < QK; j++)
            if ((j & h) == 0) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

/* Rotate nblk blocks of 32 fp32 values: v = fp32(H x) * fp32(1/sqrt 32). */
void orc_rotate_f32(const float *x, float *v, int64_t nblk)
{
    const float c = inv_sqrt32_f32();
    for (int64_t t = 0; t < nblk; t++) {
        float w[QK];
        memcpy(w, x + t * QK, sizeof w);
        wht32_butterflies_f32(w);
        for (int i = 0; i < QK; i++)
            v[t * QK + i] = w[i] * c;
    }
}

/* Same rotation in fp64 (weights, offline; and the unquantized reference). */
void orc_rotate_f64(const double *x, double *v, int64_t nblk)
{
    const double c = inv_sqrt32_f64();
    for (int64_t t = 0; t < nblk; t++) {
        double w[QK];
        memcpy(w, x + t * QK, sizeof w);
        wht32_butterflies_f64(w);
        for (int i = 0; i < QK; i++)
            v[t * QK + i] = w[i] * c;
    }
}

/* ------------------------------------------------------------------ */
/* Activation quantizer [H32 "The rotation"; 27B "Prompt processing"].  */
/* ------------------------------------------------------------------ */

static float load_act(const void *x, int dtype, int64_t idx)
{
    if (dtype == 0)
        return ((const float *)x)[idx];
    /* bf16 is the top half of an fp32; widening is exact */
    uint32_t bits = (uint32_t)((const uint16_t *)x)[idx] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/*
 * Quantize one block of 32 already-rotated values.  Writes 32 codes and the
 * scale; returns how many of the 32 quotients v/d fell exactly on .5.
 */
static int quantize_block(const float v[QK], int bits, int8_t *q, float *d_out)
{
    const float qmaxf = bits == 4 ? 7.0f : 127.0f;
    const float lo = bits == 4 ? -8.0f : -127.0f;
    const float hi = qmaxf;
    float amax = 0.0f;
    for (int i = 0; i < QK; i++) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    int ties = 0;
    float d = amax / qmaxf;
    *d_out = d;
    if (d == 0.0f) {
        for (int i = 0; i < QK; i++)
            q[i] = 0;
        return 0;
    }
    for (int i = 0; i < QK; i++) {
        float r = v[i] / d;
        if (r - floorf(r) == 0.5f)
            ties++;
        float k = rintf(r); /* current rounding mode: nearest, ties to even */
        if (k < lo)
            k = lo;
        if (k > hi)
            k = hi;
        q[i] = (int8_t)k;
    }
    return ties;
}

/*
 * x: [m][ldx] fp32 (dtype 0) or bf16 bits (dtype 1); k a multiple of 32.
 * q: [m][k] code values in natural element order; d: [m][k/32] fp32.
 * rotate = 0 skips the transform (the unrotated 4-bit route).
 * Returns the number of exact .5 quotients met (all rounded to even).
 */
int64_t orc_quantize(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                     int bits, int rotate, int8_t *q, float *d)
{
    const int64_t nb = k / QK;
    int64_t ties = 0;
#pragma omp parallel for reduction(+ : ties) schedule(static)
    for (int64_t r = 0; r < m; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float xin[QK], v[QK];
            for (int i = 0; i < QK; i++)
                xin[i] = load_act(x, dtype, r * ldx + b * QK + i);
            if (rotate)
                orc_rotate_f32(xin, v, 1);
            else
                memcpy(v, xin, sizeof v);
            ties += quantize_block(v, bits, q + r * k + b * QK, d + r * nb + b);
        }
    }
    return ties;
}

/* Storage of 4-bit codes: per block, byte j = (q[j] & 15) | (q[j+16] & 15) << 4. */
void orc_pack_int4(const int8_t *q, int64_t m, int64_t k, uint8_t *codes)
{
    const int64_t nb = k / QK;
    for (int64_t r = 0; r < m; r++)
        for (int64_t b = 0; b < nb; b++) {
            const int8_t *s = q + r * k + b * QK;
            uint8_t *o = codes + r * (k / 2) + b * 16;
            for (int j = 0; j < 16; j++)
                o[j] = (uint8_t)(((uint8_t)s[j] & 0x0f) | (((uint8_t)s[j + 16] & 0x0f) << 4));
        }
}

/* ------------------------------------------------------------------ */
/* Q4_0 weights [H32 "Why prompts are a matrix-unit problem"].          */
/* ------------------------------------------------------------------ */

/*
 * blocks: [rows][k/32] canonical 18-byte blocks (fp16 scale little-endian,
 * then 16 nibble bytes).  w: [rows][k] values u-8; dw: [rows][k/32] scales.
 */
void orc_q4_0_decode(const uint8_t *blocks, int64_t rows, int64_t k, int8_t *w, double *dw)
{
    const int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = blocks + (r * nb + b) * 18;
            uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
            dw[r * nb + b] = orc_f16_to_f64(h);
            for (int j = 0; j < 16; j++) {
                int u_lo = blk[2 + j] & 0x0f;
                int u_hi = blk[2 + j] >> 4;
                w[r * k + b * QK + j] = (int8_t)(u_lo - 8);
                w[r * k + b * QK + j + 16] = (int8_t)(u_hi - 8);
            }
        }
}

/*
 * Offline path for float weights: each 32-block of each row is rotated in
 * fp64 (same butterfly order, times 1/sqrt 32), then quantized to Q4_0:
 * dw = fp16(amax/7), u = clamp(rint(w'/dw), -8, 7) + 8 with the fp16-rounded
 * dw.  (Reading: the pages quantize with an imatrix, which is not modelled.)
 * w: [n][k] fp32 (dtype 0) or bf16 bits (dtype 1).  rotate = 0 quantizes
 * without the transform.  blocks: [n][k/32] x 18 bytes.
 */
/* Q4_0 block of 32 (already rotated) fp64 values. */
static void q4_0_block(const double v[QK], uint8_t blk[18])
{
    double amax = 0.0;
    for (int i = 0; i < QK; i++)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    uint16_t hbits = orc_f64_to_f16(amax / 7.0);
    double dwv = orc_f16_to_f64(hbits);
    blk[0] = (uint8_t)(hbits & 0xff);
    blk[1] = (uint8_t)(hbits >> 8);
    int u[QK];
    for (int i = 0; i < QK; i++) {
        double kq = dwv == 0.0 ? 0.0 : rint(v[i] / dwv);
        if (kq < -8.0)
            kq = -8.0;
        if (kq > 7.0)
            kq = 7.0;
        u[i] = (int)kq + 8;
    }
    for (int j = 0; j < 16; j++)
        blk[2 + j] = (uint8_t)(u[j] | (u[j + 16] << 4));
}

void orc_quantize_weights_q4_0(const void *w, int dtype, int64_t n, int64_t k, int rotate,
                               uint8_t *blocks)
{
    const int64_t nb = k / QK;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nb; b++) {
            double in[QK], v[QK];
            for (int i = 0; i < QK; i++)
                in[i] = (double)load_act(w, dtype, r * k + b * QK + i);
            if (rotate)
                orc_rotate_f64(in, v, 1);
            else
                memcpy(v, in, sizeof v);
            q4_0_block(v, blocks + (r * nb + b) * 18);
        }
}

/* ------------------------------------------------------------------ */
/* Rotations longer than 32 [27B "What's next": rotations larger than   */
/* 32 spread outliers further].  Reading: the Sylvester-order H_n over  */
/* each span of n = 64 or 128 consecutive values (n = 32 is the route's */
/* rotation), butterflies h = 1 .. n/2 in the stage order and sign      */
/* convention of the 32-point one, then times fp32(1/sqrt n); the       */
/* 32-value quantization blocks and their scales are unchanged.         */
/* ------------------------------------------------------------------ */

#define MAXROT 128

/* 1/sqrt(n) for n = 32, 64, 128: sqrt(2)/8, 1/8, sqrt(2)/16 (the divisions
   by powers of two are exact). */
static double inv_sqrt_n_f64(int n)
{
    return n == 64 ? 0.125 : (n == 128 ? sqrt(2.0) / 16.0 : sqrt(2.0) / 8.0);
}

static void wht_butterflies_f32(float *v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int j = 0; j < n; j++)
            if ((j & h) == 0) {
                float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

static void wht_butterflies_f64(double *v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int j = 0; j < n; j++)
            if ((j & h) == 0) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

/* v = fp32(H_n x) * fp32(1/sqrt n) for nspan spans of n values. */
void orc_rotate_n_f32(const float *x, float *v, int64_t nspan, int n)
{
    const float c = (float)inv_sqrt_n_f64(n);
    for (int64_t t = 0; t < nspan; t++) {
        float w[MAXROT];
        memcpy(w, x + t * n, sizeof(float) * n);
        wht_butterflies_f32(w, n);
        for (int i = 0; i < n; i++)
            v[t * n + i] = w[i] * c;
    }
}

void orc_rotate_n_f64(const double *x, double *v, int64_t nspan, int n)
{
    const double c = inv_sqrt_n_f64(n);
    for (int64_t t = 0; t < nspan; t++) {
        double w[MAXROT];
        memcpy(w, x + t * n, sizeof(double) * n);
        wht_butterflies_f64(w, n);
        for (int i = 0; i < n; i++)
            v[t * n + i] = w[i] * c;
    }
}

/*
 * Activation codes with rotation rot (0: none, or 32, 64, 128; k a multiple
 * of rot): every span of rot values is rotated in fp32, then every 32-block
 * is quantized as orc_quantize does.  Returns the number of .5 quotients.
 */
int64_t orc_quantize_rot(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx, int bits,
                         int rot, int8_t *q, float *d)
{
    const int span = rot == 0 ? QK : rot;
    const int64_t nb = k / QK, ns = k / span;
    int64_t ties = 0;
#pragma omp parallel for reduction(+ : ties) schedule(static)
    for (int64_t r = 0; r < m; r++) {
        for (int64_t s = 0; s < ns; s++) {
            float xin[MAXROT], v[MAXROT];
            for (int i = 0; i < span; i++)
                xin[i] = load_act(x, dtype, r * ldx + s * span + i);
            if (rot)
                orc_rotate_n_f32(xin, v, 1, span);
            else
                memcpy(v, xin, sizeof(float) * span);
            for (int b = 0; b < span / QK; b++) {
                const int64_t blk = s * (span / QK) + b;
                ties += quantize_block(v + b * QK, bits, q + r * k + blk * QK, d + r * nb + blk);
            }
        }
    }
    return ties;
}

/* Q4_0 weights with rotation rot (0, 32, 64 or 128), rotated in fp64. */
void orc_quantize_weights_q4_0_rot(const void *w, int dtype, int64_t n, int64_t k, int rot,
                                   uint8_t *blocks)
{
    const int span = rot == 0 ? QK : rot;
    const int64_t nb = k / QK, ns = k / span;
    for (int64_t r = 0; r < n; r++)
        for (int64_t s = 0; s < ns; s++) {
            double in[MAXROT], v[MAXROT];
            for (int i = 0; i < span; i++)
                in[i] = (double)load_act(w, dtype, r * k + s * span + i);
            if (rot)
                orc_rotate_n_f64(in, v, 1, span);
            else
                memcpy(v, in, sizeof(double) * span);
            for (int b = 0; b < span / QK; b++)
                q4_0_block(v + b * QK, blocks + (r * nb + s * (span / QK) + b) * 18);
        }
}

/* ------------------------------------------------------------------ */
/* Block sums and the output.                                          */
/* ------------------------------------------------------------------ */

static int32_t block_dot(const int8_t *a, const int8_t *w)
{
    int32_t s = 0;
    for (int i = 0; i < QK; i++)
        s += (int32_t)a[i] * (int32_t)w[i];
    return s;
}

/*
 * S[(r-m0)][(c-n0)][b] = sum_i q[r][32b+i] * w[c][32b+i] for r in [m0,m1),
 * c in [n0,n1).  q: [*][k] activation codes; w: [*][k] weight values u-8.
 */
void orc_block_sums(const int8_t *q, const int8_t *w, int64_t k, int64_t m0, int64_t m1,
                    int64_t n0, int64_t n1, int32_t *S)
{
    const int64_t nb = k / QK, nn = n1 - n0;
#pragma omp parallel for schedule(static)
    for (int64_t r = m0; r < m1; r++)
        for (int64_t c = n0; c < n1; c++)
            for (int64_t b = 0; b < nb; b++)
                S[((r - m0) * nn + (c - n0)) * nb + b] =
                    block_dot(q + r * k + b * QK, w + c * k + b * QK);
}

/* y[r][c] = sum_b fp64(da[r][b]) * dw[c][b] * S[r][c][b], b ascending. */
static double out_one(const int8_t *q, const float *da, const int8_t *w, const double *dw,
                      int64_t k, int64_t r, int64_t c)
{
    const int64_t nb = k / QK;
    double y = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        int32_t s = block_dot(q + r * k + b * QK, w + c * k + b * QK);
        y += (double)da[r * nb + b] * dw[c * nb + b] * (double)s;
    }
    return y;
}

void orc_gemm_rect(const int8_t *q, const float *da, const int8_t *w, const double *dw,
                   int64_t k, int64_t m0, int64_t m1, int64_t n0, int64_t n1, double *y)
{
    const int64_t nn = n1 - n0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = m0; r < m1; r++)
        for (int64_t c = n0; c < n1; c++)
            y[(r - m0) * nn + (c - n0)] = out_one(q, da, w, dw, k, r, c);
}

/*
 * a[r][c] = sum_b |fp64(da[r][b]) * dw[c][b] * S[r][c][b]|: the sum of the
 * magnitudes of the terms whose sum is y[r][c].  Every fp32 evaluation of
 * that sum (two-sided block scaling of exact block sums, accumulated in any
 * order) is within a small multiple of 2^-24 * a of the exact y, so a is the
 * scale of an element-wise error bound.
 */
static double out_abs_one(const int8_t *q, const float *da, const int8_t *w, const double *dw,
                          int64_t k, int64_t r, int64_t c)
{
    const int64_t nb = k / QK;
    double a = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        int32_t s = block_dot(q + r * k + b * QK, w + c * k + b * QK);
        a += fabs((double)da[r * nb + b] * dw[c * nb + b] * (double)s);
    }
    return a;
}

void orc_gemm_abs_rect(const int8_t *q, const float *da, const int8_t *w, const double *dw,
                       int64_t k, int64_t m0, int64_t m1, int64_t n0, int64_t n1, double *a)
{
    const int64_t nn = n1 - n0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = m0; r < m1; r++)
        for (int64_t c = n0; c < n1; c++)
            a[(r - m0) * nn + (c - n0)] = out_abs_one(q, da, w, dw, k, r, c);
}

void orc_gemm_points(const int8_t *q, const float *da, const int8_t *w, const double *dw,
                     int64_t k, const int64_t *ri, const int64_t *ci, int64_t npts, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; p++)
        y[p] = out_one(q, da, w, dw, k, ri[p], ci[p]);
}

/*
 * Grouped (MoE) output [MOE]: rows are sorted by expert; expert e owns rows
 * [off[e], off[e+1]).  Weights for expert e start at w + e*n*k and
 * dw + e*n*(k/32).  Rows outside [0, off[E]) get NAN.
 */
void orc_grouped_points(const int8_t *q, const float *da, const int32_t *off, int64_t E,
                        const int8_t *w, const double *dw, int64_t n, int64_t k,
                        const int64_t *ri, const int64_t *ci, int64_t npts, double *y)
{
    const int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; p++) {
        int64_t r = ri[p], e = -1;
        for (int64_t t = 0; t < E; t++)
            if (r >= off[t] && r < off[t + 1]) {
                e = t;
                break;
            }
        if (e < 0) {
            y[p] = NAN;
            continue;
        }
        y[p] = out_one(q, da, w + e * n * k, dw + e * n * nb, k, r, ci[p]);
    }
}

/* As orc_grouped_points, with the magnitude sum of out_abs_one (NAN outside). */
void orc_grouped_abs_points(const int8_t *q, const float *da, const int32_t *off, int64_t E,
                            const int8_t *w, const double *dw, int64_t n, int64_t k,
                            const int64_t *ri, const int64_t *ci, int64_t npts, double *a)
{
    const int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; p++) {
        int64_t r = ri[p], e = -1;
        for (int64_t t = 0; t < E; t++)
            if (r >= off[t] && r < off[t + 1]) {
                e = t;
                break;
            }
        a[p] = e < 0 ? NAN : out_abs_one(q, da, w + e * n * k, dw + e * n * nb, k, r, ci[p]);
    }
}

/*
 * Unquantized reference in fp64: y = sum_b sum_i (H x_b / sqrt 32)[i] *
 * dw[c][b] * w[c][32b+i], with the transform in fp64.  Because H/sqrt(32) is
 * orthogonal and symmetric this equals x . (H w_rot / sqrt 32), the product
 * with the unrotated weights [H32 "The rotation"].
 */
void orc_ref_points(const void *x, int dtype, int64_t ldx, const int8_t *w, const double *dw,
                    int64_t k, const int64_t *ri, const int64_t *ci, int64_t npts, double *y)
{
    const int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; p++) {
        int64_t r = ri[p], c = ci[p];
        double acc = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            double in[QK], v[QK];
            for (int i = 0; i < QK; i++)
                in[i] = (double)load_act(x, dtype, r * ldx + b * QK + i);
            orc_rotate_f64(in, v, 1);
            for (int i = 0; i < QK; i++)
                acc += v[i] * (dw[c * nb + b] * (double)w[c * k + b * QK + i]);
        }
        y[p] = acc;
    }
}

/* ------------------------------------------------------------------ */
/* MoE glue around the grouped product [MOE "4-bit activations reach   */
/* the MoE experts": the route covers the expert matmuls].  The pages   */
/* give no detail of the rest of the expert layer; the readings here    */
/* are: h = silu(gate) * up feeds the down projection and is rotated    */
/* and quantized like any activation, and the routed rows are combined  */
/* by their routing weights in a fixed order.                           */
/* ------------------------------------------------------------------ */

/*
 * e^x in fp32, every step one correctly rounded fp32 operation (no FMA):
 * Cody-Waite range reduction n = rint(x log2 e), r = (x - n ln2_hi) - n ln2_lo
 * (ln2_hi has 16 significant bits, so n ln2_hi is exact for |n| <= 128),
 * then the degree-6 Taylor polynomial of e^r in Horner form and a scaling by
 * 2^n.  |r| <= ln2/2, where the truncation error is below 1.4e-7 relative.
 * x is clamped to [-87, 88], which keeps 2^n and the result normal.
 */
float orc_exp_f32(float x)
{
    if (x < -87.0f)
        x = -87.0f;
    if (x > 88.0f)
        x = 88.0f;
    const float log2e = (float)1.4426950408889634;
    const float ln2_hi = 0.693145751953125f;
    const float ln2_lo = (float)(0.6931471805599453 - 0.693145751953125);
    const float n = rintf(x * log2e);
    const float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return ldexpf(p, (int)n);
}

/* silu(g) = g / (1 + e^-g), fp32, IEEE division. */
float orc_silu_f32(float g)
{
    const float e = orc_exp_f32(-g);
    const float den = 1.0f + e;
    return g / den;
}

/*
 * gu: [rows][ld] fp32, the gate projection in columns [0, inter) and the up
 * projection in columns [inter, 2 inter).  h = silu(gate) * up (one fp32
 * multiply), then h is rotated and quantized exactly as orc_quantize does
 * with rotate = 1.  q: [rows][inter] codes, d: [rows][inter/32] scales.
 */
int64_t orc_swiglu_quantize(const float *gu, int64_t rows, int64_t inter, int64_t ld, int bits,
                            int8_t *q, float *d)
{
    const int64_t nb = inter / QK;
    int64_t ties = 0;
#pragma omp parallel for reduction(+ : ties) schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float h[QK], v[QK];
            for (int i = 0; i < QK; i++) {
                const float g = gu[r * ld + b * QK + i];
                const float u = gu[r * ld + inter + b * QK + i];
                h[i] = orc_silu_f32(g) * u;
            }
            orc_rotate_f32(h, v, 1);
            ties += quantize_block(v, bits, q + r * inter + b * QK, d + r * nb + b);
        }
    }
    return ties;
}

/*
 * Weighted combine of the routed rows: out[t][c] = sum_j w[t k + j] *
 * dn[slot[t k + j]][c] for j = 0 .. k-1 in that order, the accumulator
 * starting at 0 and every step one fp32 fma.
 */
void orc_moe_combine(const float *dn, int64_t lddn, const int32_t *slot, const float *w,
                     int64_t tokens, int64_t topk, int64_t hidden, float *out, int64_t ldo)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; t++)
        for (int64_t c = 0; c < hidden; c++) {
            float acc = 0.0f;
            for (int64_t j = 0; j < topk; j++)
                acc = fmaf(w[t * topk + j], dn[(int64_t)slot[t * topk + j] * lddn + c], acc);
            out[t * ldo + c] = acc;
        }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
