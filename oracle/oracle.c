/*
 * Reference oracle for the weight-only 4-bit GEMM  Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the HIP kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the
 * product library never links, calls or falls back to it.  It shares no
 * source, header, table or helper with the GPU code.
 *
 * Plain single-threaded C: no SIMD intrinsics, no threads, no fast-math.
 * Every dequantized weight is formed exactly in binary32 and every product is
 * accumulated in binary64, one accumulator per output, k ascending.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Keep W4A16 zero-points packed at 4 bits instead of expanding to 2 bytes"
 *       (ROCm/vllm pull request 1073) -- sections Problem, Change, Testing.
 *  [P4] "Add BF16xFP4 MoE GEMM stage1 kernel" (ROCm/FlyDSL pull request 424)
 *       -- summary, Technical Details.
 *  [P3] "qsa_prompt_attn: Q4_0 KV on tensor cores (mode 4)" (strata pull
 *       request 452) -- section What (offset-8 codes).
 *  [P4] also names the stage-1 activation (silu); its gate/up split of W1 is
 *       read here as gate = first half of the rows, up = second half.
 *  Outside definitions: IEEE 754-2008 binary16; the bfloat16 format (top 16
 *  bits of binary32); OCP Microscaling Formats (MX) v1.0, E2M1 element and
 *  E8M0 scale.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - packed weight words hold 8 codes along K, code k%8 in bits 4*(k%8), the
 *    same nibble rule [P1] Change states for the zero-points;
 *  - zero-point words are arranged [N/8][K/g] (packed along N, [P1] Problem);
 *  - packed words are read as unsigned 32-bit (logical shifts);
 *  - scales share the activation dtype; a missing zero-point tensor means the
 *    symmetric code offset 8 (as the offset-8 codes of [P3] What);
 *  - MXFP4 bytes hold the even-k element in the low nibble;
 *  - an expert id outside [0, E) yields an all-zero output row;
 *  - the stage-1 activation is silu(gate) * up, silu(v) = v / (1 + e^-v),
 *    with gate the first N/2 outputs of a row and up the last N/2;
 *  - stage 2 (not defined on the pages) is the down projection of the
 *    stage-1 activation rows with each expert's W2, weighted by the routing
 *    weight and summed over the token's slots.
 *
 * Parity pins (tests/test_oracle_*.py): brute-force integer matmul, nibble
 * pack/unpack round trip with hand words, dense fp64/fp32 GEMM on the oracle's
 * own dequantized matrix, the page's byte counts, E8M0/E2M1 closed forms, and
 * exhaustive codec checks against numpy.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define DT_F16 0
#define DT_BF16 1

/* ------------------------------------------------------------------------- */
/* Codecs, written from the format definitions.                              */
/* ------------------------------------------------------------------------- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32 word. */
static double bf16_value(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double act_value(const uint16_t *p, int dtype, size_t i)
{
    return dtype == DT_F16 ? f16_value(p[i]) : bf16_value(p[i]);
}

/* Round-to-nearest-even of a non-negative integer-valued double q + fraction. */
static double round_half_even(double q)
{
    double fl = floor(q);
    double r = q - fl; /* exact: q has far fewer than 52 integer bits here */
    if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    return fl;
}

/*
 * Encode a binary64 value to a binary format with `frac` fraction bits,
 * exponent bias `bias` and all-ones exponent field `emax_field`, rounding to
 * nearest even.  Used for binary16 (10, 15, 31) and bfloat16 (7, 127, 255).
 */
static uint16_t encode_rne(double v, int frac, int bias, int emax_field)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0; /* bit 15 in both formats */
    if (isnan(v))
        return (uint16_t)(sign | ((unsigned)emax_field << frac) | (1u << (frac - 1)));
    double a = fabs(v);
    uint16_t inf = (uint16_t)(sign | ((unsigned)emax_field << frac));
    if (isinf(a))
        return inf;
    int emin = 1 - bias; /* exponent of the smallest normal */
    if (a < ldexp(1.0, emin)) {
        /* subnormal range: units of 2^(emin - frac) */
        double q = round_half_even(ldexp(a, frac - emin));
        return (uint16_t)(sign | (uint16_t)q); /* q == 2^frac becomes the smallest normal */
    }
    int E;
    (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;      /* a in [2^e, 2^(e+1)) */
    if (e + bias >= emax_field)
        return inf;
    double q = round_half_even(ldexp(a, frac - e)); /* in [2^frac, 2^(frac+1)] */
    unsigned bits = ((unsigned)(e + bias) << frac) + (unsigned)q - (1u << frac);
    if ((bits >> frac) >= (unsigned)emax_field)
        return inf;
    return (uint16_t)(sign | bits);
}

static uint16_t f16_encode(double v) { return encode_rne(v, 10, 15, 31); }
static uint16_t bf16_encode(double v) { return encode_rne(v, 7, 127, 255); }

/* OCP MX E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit. */
static double e2m1_value(unsigned c)
{
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(b-127); the all-ones byte is NaN. */
static double e8m0_value(unsigned b)
{
    if (b == 255)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Exported codec entry points (for the exhaustive codec pins). */
void oracle_f16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_value(in[i]);
}
void oracle_bf16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_value(in[i]);
}
void oracle_f16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_encode(in[i]);
}
void oracle_bf16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_encode(in[i]);
}
void oracle_e2m1_decode(const uint8_t *codes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e2m1_value(codes[i] & 0xf);
}
void oracle_e8m0_decode(const uint8_t *bytes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e8m0_value(bytes[i]);
}

/* ------------------------------------------------------------------------- */
/* W4A16 layout and dequantization.                                           */
/* ------------------------------------------------------------------------- */

/* Weight code q(n, k): word k/8 of row n, nibble k%8 (bits 4*(k%8)). */
static unsigned w4_code(const int32_t *qweight, int64_t K, int64_t n, int64_t k)
{
    uint32_t word = (uint32_t)qweight[n * (K / 8) + k / 8];
    return (word >> (4 * (k % 8))) & 0xfu;
}

/* Zero-point z(n, j) for group j: word [n/8][j], nibble n%8 ([P1] Change). */
static unsigned w4_zero(const int32_t *qzeros, int64_t G, int64_t n, int64_t j)
{
    if (!qzeros)
        return 8u; /* symmetric: codes are offset by 8 */
    uint32_t word = (uint32_t)qzeros[(n / 8) * G + j];
    return (word >> (4 * (n % 8))) & 0xfu;
}

void oracle_w4a16_unpack_codes(const int32_t *qweight, int64_t N, int64_t K, uint8_t *codes)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)w4_code(qweight, K, n, k);
}

void oracle_w4a16_unpack_zeros(const int32_t *qzeros, int64_t N, int64_t G, uint8_t *zeros)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < G; ++j)
            zeros[n * G + j] = (uint8_t)w4_zero(qzeros, G, n, j);
}

/*
 * Dequantize row n into w32[0..K): w = (q - z) * s with the group's scale
 * and zero-point.  |q - z| <= 15 and s has at most 11 significant bits, so the
 * binary32 product is exact.
 */
static void w4a16_dequant_row(const int32_t *qweight, const uint16_t *scales, int sdtype,
                              const int32_t *qzeros, int64_t K, int64_t g, int64_t n, float *w32)
{
    int64_t G = K / g;
    for (int64_t k = 0; k < K; ++k) {
        int64_t j = k / g;
        int d = (int)w4_code(qweight, K, n, k) - (int)w4_zero(qzeros, G, n, j);
        float s = (float)act_value(scales, sdtype, (size_t)(n * G + j));
        w32[k] = (float)d * s;
    }
}

void oracle_w4a16_dequant(const int32_t *qweight, const uint16_t *scales, int sdtype,
                          const int32_t *qzeros, int64_t N, int64_t K, int64_t g, float *w32)
{
    for (int64_t n = 0; n < N; ++n)
        w4a16_dequant_row(qweight, scales, sdtype, qzeros, K, g, n, w32 + n * K);
}

/* Dequantized weights rounded to the activation dtype (the MFMA operand form). */
void oracle_w4a16_dequant_act(const int32_t *qweight, const uint16_t *scales, int sdtype,
                              const int32_t *qzeros, int64_t N, int64_t K, int64_t g,
                              float *row_scratch, uint16_t *out)
{
    for (int64_t n = 0; n < N; ++n) {
        w4a16_dequant_row(qweight, scales, sdtype, qzeros, K, g, n, row_scratch);
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = sdtype == DT_F16 ? f16_encode(row_scratch[k]) : bf16_encode(row_scratch[k]);
    }
}

static double dot_row(const uint16_t *x, int xdtype, int64_t m, int64_t K, const float *w32)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += act_value(x, xdtype, (size_t)(m * K + k)) * (double)w32[k];
    return acc;
}

/*
 * y[m][n] = sum_k x[m][k] * w32[n][k]   (fp64 accumulate, k ascending)
 * x[M][K] and scales[N][K/g] in dtype xdtype; qweight[N][K/8]; qzeros[N/8][K/g]
 * or NULL.  w_row is caller scratch of K floats.
 */
void oracle_w4a16_gemm(const uint16_t *x, int xdtype, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, int64_t M, int64_t N, int64_t K, int64_t g,
                       float *w_row, double *y)
{
    for (int64_t n = 0; n < N; ++n) {
        w4a16_dequant_row(qweight, scales, xdtype, qzeros, K, g, n, w_row);
        for (int64_t m = 0; m < M; ++m)
            y[m * N + n] = dot_row(x, xdtype, m, K, w_row);
    }
}

/* The same definition evaluated only at the (ms[i], ns[i]) output positions. */
void oracle_w4a16_gemm_sampled(const uint16_t *x, int xdtype, const int32_t *qweight,
                               const uint16_t *scales, const int32_t *qzeros, int64_t K, int64_t g,
                               const int64_t *ms, const int64_t *ns, int64_t count, float *w_row,
                               double *out)
{
    int64_t last_n = -1;
    for (int64_t i = 0; i < count; ++i) {
        if (ns[i] != last_n) {
            w4a16_dequant_row(qweight, scales, xdtype, qzeros, K, g, ns[i], w_row);
            last_n = ns[i];
        }
        out[i] = dot_row(x, xdtype, ms[i], K, w_row);
    }
}

/*
 * Ragged grouped form: group e owns rows [off[e], off[e+1]) of x and y and uses
 * its own packed weights qweight[e], scales[e], qzeros[e].
 */
void oracle_w4a16_gemm_grouped(const uint16_t *x, int xdtype, const int64_t *m_offsets,
                               int64_t num_groups, const int32_t *qweight, const uint16_t *scales,
                               const int32_t *qzeros, int64_t N, int64_t K, int64_t g, float *w_row,
                               double *y)
{
    int64_t G = K / g;
    for (int64_t e = 0; e < num_groups; ++e) {
        const int32_t *qw = qweight + e * N * (K / 8);
        const uint16_t *sc = scales + e * N * G;
        const int32_t *qz = qzeros ? qzeros + e * (N / 8) * G : NULL;
        for (int64_t n = 0; n < N; ++n) {
            w4a16_dequant_row(qw, sc, xdtype, qz, K, g, n, w_row);
            for (int64_t m = m_offsets[e]; m < m_offsets[e + 1]; ++m)
                y[m * N + n] = dot_row(x, xdtype, m, K, w_row);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* MXFP4 (E2M1 elements, E8M0 scale per 32 along K) and MoE stage 1.          */
/* ------------------------------------------------------------------------- */

/* Row n of one expert: w[k] = e2m1(code(n,k)) * 2^(scale(n,k/32) - 127), exact. */
static void mxfp4_dequant_row(const uint8_t *w_fp4, const uint8_t *w_scale, int64_t K, int64_t n,
                              float *w32)
{
    for (int64_t k = 0; k < K; ++k) {
        uint8_t byte = w_fp4[n * (K / 2) + k / 2];
        unsigned c = (k % 2 == 0) ? (byte & 0xfu) : (byte >> 4);
        double s = e8m0_value(w_scale[n * (K / 32) + k / 32]);
        w32[k] = (float)(e2m1_value(c) * s);
    }
}

void oracle_mxfp4_dequant(const uint8_t *w_fp4, const uint8_t *w_scale, int64_t N, int64_t K,
                          float *w32)
{
    for (int64_t n = 0; n < N; ++n)
        mxfp4_dequant_row(w_fp4, w_scale, K, n, w32 + n * K);
}

/*
 * MoE stage 1 (up to the activation): for token t and routing slot s with
 * expert e = ids[t][s], y[t][s][n] = sum_k x[t][k] * w_e[n][k]; rows whose
 * expert id is outside [0, E) are zero.  x is bfloat16 [T][K];
 * w_fp4[E][N][K/2], w_scale[E][N][K/32].  w_row is caller scratch of K floats.
 */
void oracle_mxfp4_moe_gemm(const uint16_t *x, const int32_t *ids, const uint8_t *w_fp4,
                           const uint8_t *w_scale, int64_t T, int64_t topk, int64_t E, int64_t N,
                           int64_t K, float *w_row, double *y)
{
    for (int64_t i = 0; i < T * topk * N; ++i)
        y[i] = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        const uint8_t *we = w_fp4 + e * N * (K / 2);
        const uint8_t *se = w_scale + e * N * (K / 32);
        for (int64_t n = 0; n < N; ++n) {
            mxfp4_dequant_row(we, se, K, n, w_row);
            for (int64_t t = 0; t < T; ++t)
                for (int64_t s = 0; s < topk; ++s)
                    if (ids[t * topk + s] == e)
                        y[(t * topk + s) * N + n] = dot_row(x, DT_BF16, t, K, w_row);
        }
    }
}

/* The same definition evaluated at (ts[i], slots[i], ns[i]). */
void oracle_mxfp4_moe_gemm_sampled(const uint16_t *x, const int32_t *ids, const uint8_t *w_fp4,
                                   const uint8_t *w_scale, int64_t topk, int64_t E, int64_t N,
                                   int64_t K, const int64_t *ts, const int64_t *slots,
                                   const int64_t *ns, int64_t count, float *w_row, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        int32_t e = ids[ts[i] * topk + slots[i]];
        if (e < 0 || e >= E) {
            out[i] = 0.0;
            continue;
        }
        mxfp4_dequant_row(w_fp4 + (int64_t)e * N * (K / 2), w_scale + (int64_t)e * N * (K / 32), K,
                          ns[i], w_row);
        out[i] = dot_row(x, DT_BF16, ts[i], K, w_row);
    }
}

/*
 * MoE stage-1 activation on pre-activation rows ypre[rows][N]: the first N/2
 * values of a row are the gate half, the last N/2 the up half, and
 * out[r][n] = silu(gate[n]) * up[n] with silu(v) = v / (1 + e^-v), evaluated
 * in binary64.
 */
void oracle_silu_mul(const double *ypre, int64_t rows, int64_t N, double *out)
{
    int64_t I = N / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t n = 0; n < I; ++n) {
            double g = ypre[r * N + n];
            double u = ypre[r * N + I + n];
            out[r * I + n] = g / (1.0 + exp(-g)) * u;
        }
}

/*
 * MoE stage 2 (reading; the stage-1 page names its kernel "stage1" and W1's
 * gate / up halves but does not define the second stage): the down
 * projection of each routed row of the stage-1 activation output, weighted by
 * its routing weight and summed over the token's slots,
 *   y[t][h] = sum over s < topk with e = ids[t][s] in [0, E) of
 *             w[t][s] * sum_i a[t][s][i] * w2_e[h][i]
 * a [T][topk][I] bfloat16; w [T][topk] binary32 routing weights;
 * w2_fp4 [E][H][I/2] and w2_scale [E][H][I/32] as in stage 1 (MXFP4).
 * Slots whose id lies outside [0, E) contribute nothing.  Each slot's dot
 * product is accumulated in binary64 (i ascending), then the weighted slots
 * are summed in slot order.  pre is caller scratch of T*topk*H doubles.
 */
void oracle_mxfp4_moe_stage2(const uint16_t *a, const int32_t *ids, const float *w,
                             const uint8_t *w2_fp4, const uint8_t *w2_scale, int64_t T,
                             int64_t topk, int64_t E, int64_t H, int64_t I, float *w_row,
                             double *pre, double *y)
{
    int64_t P = T * topk;
    for (int64_t i = 0; i < P * H; ++i)
        pre[i] = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        const uint8_t *we = w2_fp4 + e * H * (I / 2);
        const uint8_t *se = w2_scale + e * H * (I / 32);
        for (int64_t h = 0; h < H; ++h) {
            mxfp4_dequant_row(we, se, I, h, w_row);
            for (int64_t p = 0; p < P; ++p)
                if (ids[p] == e)
                    pre[p * H + h] = dot_row(a, DT_BF16, p, I, w_row);
        }
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t s = 0; s < topk; ++s) {
                int32_t e = ids[t * topk + s];
                if (e >= 0 && e < E)
                    acc += (double)w[t * topk + s] * pre[(t * topk + s) * H + h];
            }
            y[t * H + h] = acc;
        }
}

/* The same definition evaluated at (ts[i], hs[i]). */
void oracle_mxfp4_moe_stage2_sampled(const uint16_t *a, const int32_t *ids, const float *w,
                                     const uint8_t *w2_fp4, const uint8_t *w2_scale, int64_t topk,
                                     int64_t E, int64_t H, int64_t I, const int64_t *ts,
                                     const int64_t *hs, int64_t count, float *w_row, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t s = 0; s < topk; ++s) {
            int64_t p = ts[i] * topk + s;
            int32_t e = ids[p];
            if (e < 0 || e >= E)
                continue;
            mxfp4_dequant_row(w2_fp4 + (int64_t)e * H * (I / 2), w2_scale + (int64_t)e * H * (I / 32),
                              I, hs[i], w_row);
            acc += (double)w[p] * dot_row(a, DT_BF16, p, I, w_row);
        }
        out[i] = acc;
    }
}
