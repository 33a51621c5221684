/*
 * CPU oracle for the Q4_0-weight x Q8_0-activation quantized matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Plain, slow, obviously correct loops.  Built with `gcc -O2 -ffp-contract=off`
 * so that every fp32 operation below is one IEEE binary32 operation.
 *
 * Sources (the pages the method is taken from):
 *   [P3-2]  "llama.cpp 深度解读" (luoboask.github.io), section 2
 *           "量化数据结构 — Q4_0 格式详解": the block_q4_0 struct (fp16 d + 16 bytes
 *           of nibbles, 32 weights), how a block is encoded (the scale from the
 *           largest magnitude over 8, each weight rounded against it and offset
 *           by 8) and its decode (value = (nibble - 8) * d, low nibble = even
 *           element).
 *   [P3-3]  same page, section 3 "量化矩阵乘法 — 核心算子": the Q4_0 x Q8_0 dot
 *           product -- per pair of blocks an exact integer dot of the codes,
 *           scaled by the product of the two fp16 scales and summed in fp32.
 *           Activations are Q8_0-quantized so the dot runs in the integer
 *           domain.
 *   [P3-1]  same page, section 1: the table of ggml quantization types, with
 *           Q8_0 (8 bits per weight) beside Q4_0 as a weight format.
 *   [P4]    ggml GPT-2 walkthrough (aicoding.csdn.net): section 3.1 LayerNorm
 *           (gamma * (x - mu) / sqrt(sigma^2 + eps) + beta, after ggml_norm),
 *           section 3.5 (bias add then GELU after c_mlp_fc).
 *   [P3-4]  "llama.cpp 深度解读" section 4: SiLU(x) = x * sigmoid(x) and the
 *           SwiGLU feed-forward SiLU(gate) * up.
 *   [P2-mm] "解锁模型适配能力：Llama.cpp 框架下新架构开发全流程指南" (tahou.com),
 *           section "GGML 的特性与注意事项", item 2: ggml's mul_mat contracts the
 *           innermost dimension of both operands.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   R1 nibble order: byte j = element 2j (low) | element 2j+1 (high), as printed.
 *   R2 the weights are divided by the STORED scale (fp16, widened to fp32).
 *   R3 round() is C roundf: half away from zero.
 *   R4 an all-zero block stores d = 0 and every nibble 8 (Q8_0: every q = 0).
 *   R5 Q8_0: d = fp16(amax / 127), q = clamp(roundf(x / d), -127, 127).
 *   R6 fp32 -> fp16 is IEEE round-to-nearest-even, subnormals kept.
 *   G1 the printed dot loop multiplies the raw nibble; the page itself flags
 *      that real code handles the offset.  The decode formula fixes it: the
 *      dot uses (nibble - 8).
 *   G5 q is clamped to [0, 15] (w = +amax gives round(8) + 8 = 16).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_QK 32            /* weights per block, [P3-2] QK4_0 */
#define ORC_Q4_BYTES 18      /* 2-byte fp16 d + 16 bytes of nibbles, [P3-2] */
#define ORC_Q8_BYTES 34      /* 2-byte fp16 d + 32 int8 (inferred block_q8_0) */

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32 (R6).                                          */
/* ------------------------------------------------------------------------ */

/* m / 2^sh rounded to nearest, ties to even.  sh >= 1. */
static uint32_t orc_shift_rne(uint32_t m, int sh)
{
    uint32_t q = m >> sh;
    uint32_t rem = m & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    return q;
}

uint16_t orc_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) /* inf or nan */
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x0200u : 0u));
    int be = (int)(ax >> 23);          /* biased fp32 exponent */
    if (be < 127 - 25)                 /* |f| < 2^-25: rounds to zero */
        return sign;
    uint32_t m = (ax & 0x7fffffu) | 0x800000u; /* |f| = m * 2^(be - 150) */
    int e = be - 127;                  /* floor(log2 |f|) */
    if (e < -14) {
        /* fp16 subnormal: the result counts units of 2^-24.
         * |f| / 2^-24 = m * 2^(be - 126).  A count of 1024 is the smallest
         * normal number, whose encoding is exactly 0x0400. */
        return (uint16_t)(sign | orc_shift_rne(m, 126 - be));
    }
    uint32_t q = orc_shift_rne(m, 13);   /* 11-bit significand, in [1024, 2048] */
    int e16 = e + 15;
    if (q == 2048u) {
        q = 1024u;
        e16 += 1;
    }
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | ((uint32_t)e16 << 10) | (q - 1024u));
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return (float)(sign ? -v : v);
}

void orc_f32_to_f16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Block codes and scales.                                                   */
/*                                                                           */
/* [P3-2] defines a Q4_0 block as a binary16 scale d followed by 32 four-bit */
/* fields, element j in byte j/2 (low half for even j), whose value is       */
/* (field - 8) * d.  A Q8_0 block is the same scale followed by 32 signed    */
/* bytes, element j worth byte_j * d.  Below, "code" is the signed integer   */
/* that multiplies d: field - 8 in [-8, 7] for Q4_0, the byte in [-127, 127] */
/* for Q8_0.                                                                  */
/* ------------------------------------------------------------------------ */

static float orc_block_d(const uint8_t *blk)
{
    return orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

static int orc_q4_0_code(const uint8_t *blk, int j)
{
    uint8_t byte = blk[2 + j / 2];
    int field = (j % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
    return field - 8;
}

static int orc_q8_0_code(const uint8_t *blk, int j)
{
    return (int)(int8_t)blk[2 + j];
}

/* The scale of 32 values encoded with `top` positive steps (8 for Q4_0, 127
 * for Q8_0): the largest magnitude divided by `top` in fp32, kept as the
 * nearest binary16 (R6).  Returns its bits. */
static uint16_t orc_scale_bits(const float *v, float top)
{
    float amax = 0.0f;
    for (int k = 0; k < ORC_QK; ++k)
        if (fabsf(v[k]) > amax)
            amax = fabsf(v[k]);
    return orc_f32_to_f16(amax / top);
}

/* The code of v against the STORED scale d (R2): v / d in fp32 rounded to the
 * nearest integer, halves away from zero (R3), limited to [lo, hi] (G5 for
 * Q4_0, R5 for Q8_0); 0 when d is 0 (R4). */
static int orc_code(float v, float d, int lo, int hi)
{
    if (d == 0.0f)
        return 0;
    int c = (int)roundf(v / d);
    return c < lo ? lo : (c > hi ? hi : c);
}

static void orc_put_scale(uint16_t dh, uint8_t *blk)
{
    blk[0] = (uint8_t)(dh & 0xffu);
    blk[1] = (uint8_t)(dh >> 8);
}

/* ------------------------------------------------------------------------ */
/* Q4_0 encode / decode, [P3-2].                                            */
/* ------------------------------------------------------------------------ */

/* One block of 32 weights -> 18 bytes: the binary16 scale amax / 8, then the
 * 4-bit fields code + 8 (R1: element j in byte j/2, even j in the low half). */
void orc_q4_0_quantize_block(const float *w, uint8_t *out)
{
    uint16_t dh = orc_scale_bits(w, 8.0f);
    float d = orc_f16_to_f32(dh);
    orc_put_scale(dh, out);
    memset(out + 2, 0, ORC_QK / 2);
    for (int j = 0; j < ORC_QK; ++j) {
        int field = orc_code(w[j], d, -8, 7) + 8;
        out[2 + j / 2] |= (uint8_t)(j % 2 == 0 ? field : field << 4);
    }
}

/* rows x K fp32 (row-major) -> rows x (K/32) blocks of 18 bytes. */
void orc_q4_0_quantize(const float *W, int64_t rows, int64_t K, uint8_t *Wq)
{
    int64_t nb = K / ORC_QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            orc_q4_0_quantize_block(W + r * K + b * ORC_QK,
                                    Wq + (r * nb + b) * ORC_Q4_BYTES);
}

/* Decode: element j of a block is code_j * d. */
void orc_q4_0_dequantize(const uint8_t *Wq, int64_t rows, int64_t K, float *W)
{
    int64_t nb = K / ORC_QK;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = Wq + (r * nb + b) * ORC_Q4_BYTES;
            float d = orc_block_d(blk);
            for (int j = 0; j < ORC_QK; ++j)
                W[r * K + b * ORC_QK + j] = (float)orc_q4_0_code(blk, j) * d;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q8_0 encode (R5): the binary16 scale amax / 127, then the codes.          */
/* ------------------------------------------------------------------------ */

void orc_q8_0_quantize_block(const float *x, uint8_t *out)
{
    uint16_t dh = orc_scale_bits(x, 127.0f);
    float d = orc_f16_to_f32(dh);
    orc_put_scale(dh, out);
    for (int j = 0; j < ORC_QK; ++j)
        out[2 + j] = (uint8_t)(int8_t)orc_code(x[j], d, -127, 127);
}

void orc_q8_0_quantize(const float *X, int64_t N, int64_t K, uint8_t *Xq)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b)
            orc_q8_0_quantize_block(X + n * K + b * ORC_QK,
                                    Xq + (n * nb + b) * ORC_Q8_BYTES);
}

/* ------------------------------------------------------------------------ */
/* Per-block integer dot, [P3-3].  The product of a weight block and an     */
/* activation block is d_w * d_x * (sum over the 32 elements of code_w *     */
/* code_x); with the weights' code being field - 8 by [P3-2]'s decode (G1),  */
/* the sum is an exact integer.                                              */
/* ------------------------------------------------------------------------ */

int32_t orc_block_dot(const uint8_t *wblk, const uint8_t *xblk)
{
    int32_t s = 0;
    for (int j = 0; j < ORC_QK; ++j)
        s += orc_q4_0_code(wblk, j) * orc_q8_0_code(xblk, j);
    return s;
}

/* D[(n * rows + r) * nb + b] = dot of weight block (r, b) with activation
 * block (n, b). */
void orc_block_dots(const uint8_t *Wq, int64_t rows, int64_t K,
                    const uint8_t *Xq, int64_t N, int32_t *D)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b)
                D[(n * rows + r) * nb + b] =
                    orc_block_dot(Wq + (r * nb + b) * ORC_Q4_BYTES,
                                  Xq + (n * nb + b) * ORC_Q8_BYTES);
}

/* ------------------------------------------------------------------------ */
/* The product.  Y is N x rows, rows contiguous ([P2-mm]: the output of       */
/* mul_mat(W[K, rows], X[K, N]) is [rows, N] in ggml's innermost-first order). */
/* ------------------------------------------------------------------------ */

/* Reference: Y[n][r] = sum_b d_w * d_x * s, every term exact in fp64, summed
 * in fp64 in increasing b. */
void orc_mul_mat_ref(const uint8_t *Wq, int64_t rows, int64_t K,
                     const uint8_t *Xq, int64_t N, double *Y)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t r = 0; r < rows; ++r) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *wb = Wq + (r * nb + b) * ORC_Q4_BYTES;
                const uint8_t *xb = Xq + (n * nb + b) * ORC_Q8_BYTES;
                double dw = (double)orc_block_d(wb);
                double dx = (double)orc_block_d(xb);
                acc += dw * dx * (double)orc_block_dot(wb, xb);
            }
            Y[n * rows + r] = acc;
        }
    }
}

/* The same block terms accumulated in binary32, as the page's dot routine
 * does it ([P3-3]): each term is the binary32 product of the two widened
 * scales times the block's integer dot converted to binary32, and the terms
 * are added into a binary32 running sum in increasing block order. */
void orc_mul_mat_pages_f32(const uint8_t *Wq, int64_t rows, int64_t K,
                           const uint8_t *Xq, int64_t N, float *Y)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t r = 0; r < rows; ++r) {
            float acc = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *wb = Wq + (r * nb + b) * ORC_Q4_BYTES;
                const uint8_t *xb = Xq + (n * nb + b) * ORC_Q8_BYTES;
                float scale = orc_block_d(wb) * orc_block_d(xb);
                float term = scale * (float)orc_block_dot(wb, xb);
                acc = acc + term;
            }
            Y[n * rows + r] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q8_0 weights ([P3-1]'s type table lists Q8_0 as a weight type next to     */
/* Q4_0; its block is the block_q8_0 the product takes as activations: fp16  */
/* d + 32 int8).  Weight element j is q_j * d, so the block dot is the plain */
/* integer dot of the two int8 vectors, with no offset.                      */
/* ------------------------------------------------------------------------ */

int32_t orc_block_dot_q8(const uint8_t *wblk, const uint8_t *xblk)
{
    int32_t s = 0;
    for (int j = 0; j < ORC_QK; ++j)
        s += orc_q8_0_code(wblk, j) * orc_q8_0_code(xblk, j);
    return s;
}

void orc_block_dots_q8(const uint8_t *Wq, int64_t rows, int64_t K,
                       const uint8_t *Xq, int64_t N, int32_t *D)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b)
                D[(n * rows + r) * nb + b] =
                    orc_block_dot_q8(Wq + (r * nb + b) * ORC_Q8_BYTES,
                                     Xq + (n * nb + b) * ORC_Q8_BYTES);
}

/* Y[n][r] = sum_b d_w * d_x * s over Q8_0 weight blocks, every term exact in
 * fp64, summed in fp64 in increasing b (the same reference as for Q4_0). */
void orc_mul_mat_q8_ref(const uint8_t *Wq, int64_t rows, int64_t K,
                        const uint8_t *Xq, int64_t N, double *Y)
{
    int64_t nb = K / ORC_QK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t r = 0; r < rows; ++r) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *wb = Wq + (r * nb + b) * ORC_Q8_BYTES;
                const uint8_t *xb = Xq + (n * nb + b) * ORC_Q8_BYTES;
                double dw = (double)orc_block_d(wb);
                double dx = (double)orc_block_d(xb);
                acc += dw * dx * (double)orc_block_dot_q8(wb, xb);
            }
            Y[n * rows + r] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Around the product: LayerNorm before it, bias / activation / gate after   */
/* it ([P4] 3.1 and 3.5, [P3-4]).                                            */
/* ------------------------------------------------------------------------ */

/* LayerNorm of each token (row of X): mu = mean, sigma^2 = mean of (x - mu)^2
 * (the population variance), both in fp64; out = gamma * (x - mu) /
 * sqrt(sigma^2 + eps) + beta evaluated in fp64 and rounded once to fp32.
 * (Reading: the pages give the formula, not its precision; the fp64 statistics
 * make the fp32 result, which decides the Q8_0 codes, independent of the
 * summation order.) */
void orc_layernorm(const float *X, int64_t N, int64_t K, const float *gamma,
                   const float *beta, float eps, float *out)
{
    for (int64_t n = 0; n < N; ++n) {
        const float *x = X + n * K;
        double mu = 0.0;
        for (int64_t k = 0; k < K; ++k)
            mu += (double)x[k];
        mu /= (double)K;
        double var = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double c = (double)x[k] - mu;
            var += c * c;
        }
        var /= (double)K;
        double rstd = 1.0 / sqrt(var + (double)eps);
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = (float)((double)gamma[k] * (((double)x[k] - mu) * rstd) + (double)beta[k]);
    }
}

/* GELU, the tanh form GPT-2 uses (reading: the pages name GELU without a
 * formula): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
double orc_gelu(double x)
{
    const double c = 0.79788456080286535588; /* sqrt(2 / pi) */
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)). */
double orc_silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* Y[n][r] = act(Y[n][r] + bias[r]) * mul[n][r], in place, fp64; bias and mul
 * may be NULL; act 0 = none, 1 = GELU, 2 = SiLU. */
void orc_epilogue(double *Y, int64_t N, int64_t rows, const float *bias, int act,
                  const double *mul)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < rows; ++r) {
            double y = Y[n * rows + r];
            if (bias)
                y += (double)bias[r];
            if (act == 1)
                y = orc_gelu(y);
            else if (act == 2)
                y = orc_silu(y);
            if (mul)
                y *= mul[n * rows + r];
            Y[n * rows + r] = y;
        }
}

/* Whole operator with fp32 activations: quantize X to Q8_0, then the
 * reference product.  Rows are split evenly over `nthreads` threads (the only
 * concession to speed; it changes no arithmetic).  Returns 0, or -1 when the
 * scratch allocation fails. */
struct orc_job {
    const uint8_t *Wq;
    const uint8_t *Xq;
    int64_t rows, K, N, r0, r1;
    double *Y;
};

static void *orc_job_run(void *arg)
{
    struct orc_job *j = (struct orc_job *)arg;
    int64_t nb = j->K / ORC_QK;
    for (int64_t n = 0; n < j->N; ++n) {
        for (int64_t r = j->r0; r < j->r1; ++r) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *wb = j->Wq + (r * nb + b) * ORC_Q4_BYTES;
                const uint8_t *xb = j->Xq + (n * nb + b) * ORC_Q8_BYTES;
                double dw = (double)orc_block_d(wb);
                double dx = (double)orc_block_d(xb);
                acc += dw * dx * (double)orc_block_dot(wb, xb);
            }
            j->Y[n * j->rows + r] = acc;
        }
    }
    return NULL;
}

int orc_mul_mat(const uint8_t *Wq, int64_t rows, int64_t K, const float *X,
                int64_t N, double *Y, int nthreads)
{
    int64_t nb = K / ORC_QK;
    uint8_t *Xq = (uint8_t *)malloc((size_t)(N * nb * ORC_Q8_BYTES) + 1);
    if (!Xq)
        return -1;
    orc_q8_0_quantize(X, N, K, Xq);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t tid[256];
    int running[256];
    struct orc_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].Wq = Wq;
        jobs[t].Xq = Xq;
        jobs[t].rows = rows;
        jobs[t].K = K;
        jobs[t].N = N;
        jobs[t].r0 = rows * t / nthreads;
        jobs[t].r1 = rows * (t + 1) / nthreads;
        jobs[t].Y = Y;
        running[t] = nthreads > 1 &&
                     pthread_create(&tid[t], NULL, orc_job_run, &jobs[t]) == 0;
        if (!running[t])
            orc_job_run(&jobs[t]); /* single thread, or a thread failed to start */
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(tid[t], NULL);
    free(Xq);
    return 0;
}
