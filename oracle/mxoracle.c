/*
 * mxoracle.c -- plain, slow, CPU reference for the MXFP8 block-scaled GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; nothing here is built into
 * or called by the product path.
 *
 * Everything is computed from the definitions, in fp64 where a real number is
 * involved, with no blocking, fusion or reordering beyond what the definition
 * states.  Sources ("pages") are the vLLM API documentation pages for
 *   [mxfp8]  vllm.models.deepseek_v41.nvidia.specialized_decode.attention.mxfp8
 *   [step]   vllm.models.deepseek_v41.nvidia.specialized_decode.attention.step
 *   [cute]   vllm.models.deepseek_v41.nvidia.ops.cute_dsl
 *   [o_proj] vllm.models.deepseek_v41.nvidia.ops.o_proj
 * plus the OCP 8-bit floating point / MX formats that those pages name
 * (float8_e4m3fn elements, Float8E8M0FNU scales, one scale per 32 elements).
 *
 * Readings of points the pages leave open are listed where they are used.
 * Parity unpinned: fidelity to the real model's rotary convention, scale rule
 * and RMSNorm rounding (the pages show no outputs to compare against); each
 * function is pinned to what its own definition fixes by the CPU tests.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* E4M3 "FN" element ([mxfp8] compile_low_latency: Float8E4M3FN operands;
 * _zeros: torch.float8_e4m3fn).  Sign bit, 4-bit exponent with bias 7, 3-bit
 * mantissa; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no
 * infinities. */
double orc_e4m3_value(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    double mag;
    if (E == 15 && m == 7)
        return NAN;
    if (E == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, E - 7);
    return s ? -mag : mag;
}

/* UE8M0 scale ([mxfp8] compile_low_latency: Float8E8M0FNU scale pointers):
 * the value 2^(c-127); 0xFF is NaN; there is no zero. */
double orc_e8m0_value(uint8_t c)
{
    if (c == 0xFF)
        return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* Nearest E4M3 code to v, ties to the even code (mantissa LSB 0).
 * Reading (the pages are silent): magnitudes >= 448 saturate to 448 (the
 * format has no infinity, and NaN would poison the GEMM); the sign is kept, so
 * -0 and tiny negatives give 0x80. */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    /* codes 0..126 are the non-negative finite values in increasing order:
     * find the largest code whose value is <= a, by bisection. */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int best = lo;
    if (lo < 126) {
        double below = orc_e4m3_value((uint8_t)lo);
        double above = orc_e4m3_value((uint8_t)(lo + 1));
        double dlo = a - below, dhi = above - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0))
            best = lo + 1;
    }
    return sign | (uint8_t)best;
}

/* BF16 (the activations' original dtype, [mxfp8] wide_mm requires a BF16 out)
 * bit pattern -> its exact value. */
double orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Nearest BF16 value to v, ties to even, returned as bits.  Normal range:
 * 8 significant bits; below 2^-126 the quantum is fixed at 2^-133. */
uint16_t orc_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);          /* a = f * 2^ex with f in [0.5, 1) */
    int p = ex - 1;         /* floor(log2 a) */
    if (p < -126)
        p = -126;
    double quantum = ldexp(1.0, p - 7);
    double r = nearbyint(a / quantum) * quantum;  /* default mode: ties-to-even */
    float f = (float)r;     /* r is a BF16 value, so this is exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------- quantizer */

/* Block scale exponent e of one 32-element block with absolute maximum amax.
 * Rule (the benchmark definition; the pages do not print it): the scale is
 * 2^(floor(log2 amax) - 8), 8 being E4M3's largest exponent (448 = 1.75*2^8),
 * clamped to the E8M0 range.  amax = 0 gives the smallest scale, byte 0, as
 * the pages' zero input does ([mxfp8] _zeros: zero codes and zero scale
 * bytes).  floor(log2) is taken exactly from frexp, never from log2(). */
int orc_block_exponent(double amax)
{
    if (amax == 0.0)
        return -127;
    int ex;
    frexp(amax, &ex);
    int e = (ex - 1) - 8;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* BF16 -> MXFP8 quantize ([mxfp8] pinned_mm / wide_mm: mxfp8_e4m3_quantize of
 * a BF16 input; [cute] AllReduceMHC: mxfp8_out receives the layer input as
 * MXFP8).  x: BF16 [M, K] with row stride ldx (elements); q: codes [M, K];
 * s: scale bytes [M, K/32], both row-major.  Returns 0, or -1 if K % 32 != 0
 * or an input is not finite (NaN/Inf input is outside the contract). */
int orc_quantize(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                 uint8_t *q, uint8_t *s)
{
    if (K % 32 != 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < K / 32; ++b) {
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                double v = orc_bf16_value(x[m * ldx + b * 32 + j]);
                if (!isfinite(v))
                    return -1;
                if (fabs(v) > amax)
                    amax = fabs(v);
            }
            int e = orc_block_exponent(amax);
            s[m * (K / 32) + b] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; ++j) {
                double v = orc_bf16_value(x[m * ldx + b * 32 + j]);
                q[m * K + b * 32 + j] = orc_e4m3_encode(ldexp(v, -e));
            }
        }
    }
    return 0;
}

/* Element k of row r of an MXFP8 tensor: code value times its block's scale. */
static double dequant(const uint8_t *q, const uint8_t *s, int64_t K, int64_t r,
                      int64_t k)
{
    return orc_e4m3_value(q[r * K + k]) * orc_e8m0_value(s[r * (K / 32) + k / 32]);
}

/* --------------------------------------------------------------- GEMM */

/* out = dequant(a) . dequant(w)^T ([mxfp8] launch_low_latency: out = a
 * (rows x K) times the [K, N] weight, one scale per 32 K elements
 * (sf_vec_size=32) on both operands, FP32 accumulation, BF16 output without
 * scale or bias).  The oracle sums in fp64 over k in order.
 *   a_q [M, K], a_s [M, K/32], w_q [N, K], w_s [N, K/32]
 *   ref [M, N]: the fp64 sum (unrounded); absref [M, N]: sum of |a_k * w_k|
 *   out [M, N]: BF16 bits, round-to-nearest-even of ref.
 * Any of ref/absref/out may be NULL.  Rows of w are split over threads. */
int orc_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a_q,
             const uint8_t *a_s, const uint8_t *w_q, const uint8_t *w_s,
             double *ref, double *absref, uint16_t *out)
{
    if (K % 32 != 0)
        return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!a)
        return -2;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            a[m * K + k] = dequant(a_q, a_s, K, m, k);
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!w) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (!w)
                continue;
            for (int64_t k = 0; k < K; ++k)
                w[k] = dequant(w_q, w_s, K, n, k);
            for (int64_t m = 0; m < M; ++m) {
                double sum = 0.0, sabs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = a[m * K + k] * w[k];
                    sum += p;
                    sabs += fabs(p);
                }
                if (ref)
                    ref[m * N + n] = sum;
                if (absref)
                    absref[m * N + n] = sabs;
                if (out)
                    out[m * N + n] = orc_bf16_round(sum);
            }
        }
        free(w);
    }
    free(a);
    return err;
}

/* ---------------------------------------------------------------- RoPE */

/* Rotary embedding of the last rope_dim dims of each head ([o_proj]
 * dsv41_o_proj: the fused WO-A kernel takes positions and the layer's
 * cos_sin_cache; _can_fuse_wo_a: nope/rope head dims 448/64).
 * Readings (the pages print neither convention nor precision):
 *   - cos_sin is FP32 [max_pos, rope_dim]: the first rope_dim/2 entries of a
 *     row are cos(theta_i), the last rope_dim/2 are sin(theta_i);
 *   - dims (nope + 2i, nope + 2i + 1) form pair i (adjacent pairs) and are
 *     rotated forward: y1 = x1*c - x2*s, y2 = x2*c + x1*s;
 *   - the arithmetic is FP32, each product and sum rounded separately (no
 *     fused multiply-add), and the result is rounded to BF16, the dtype the
 *     unfused path materialises.
 * o: BF16 [M, H, D] with strides ld_row, ld_head (elements), D contiguous;
 * y: BF16 [M, H, D] contiguous.  Nope dims are copied. */
int orc_rope(const uint16_t *o, int64_t M, int64_t H, int64_t D, int64_t ld_row,
             int64_t ld_head, int64_t nope, const int64_t *positions,
             const float *cos_sin, int64_t max_pos, uint16_t *y)
{
    int64_t rope = D - nope;
    if (rope <= 0 || rope % 2 != 0)
        return -1;
    int64_t half = rope / 2;
    for (int64_t m = 0; m < M; ++m) {
        int64_t pos = positions[m];
        if (pos < 0 || pos >= max_pos)
            return -1;
        const float *cs = cos_sin + pos * rope;
        for (int64_t h = 0; h < H; ++h) {
            const uint16_t *src = o + m * ld_row + h * ld_head;
            uint16_t *dst = y + (m * H + h) * D;
            for (int64_t d = 0; d < nope; ++d)
                dst[d] = src[d];
            for (int64_t i = 0; i < half; ++i) {
                volatile float x1 = (float)orc_bf16_value(src[nope + 2 * i]);
                volatile float x2 = (float)orc_bf16_value(src[nope + 2 * i + 1]);
                volatile float c = cs[i], sn = cs[half + i];
                volatile float p1 = x1 * c, p2 = x2 * sn, p3 = x2 * c, p4 = x1 * sn;
                volatile float y1 = p1 - p2, y2 = p3 + p4;
                dst[nope + 2 * i] = orc_bf16_round((double)y1);
                dst[nope + 2 * i + 1] = orc_bf16_round((double)y2);
            }
        }
    }
    return 0;
}

/* RMSNorm of BF16 rows, unrounded ([step] AttentionStep.run normalises the
 * leading columns of fused_wqa_wkv's output in _split_qkv_and_norm before they
 * are requantized for wq_b; [cute] AllReduceMHC normalises its collapse with a
 * BF16 norm_weight and norm_eps and can write the result as MXFP8):
 *   y[m][j] = x[m][j] * w[j] / sqrt(mean_k x[m][k]^2 + eps),
 * the root-mean-square normalisation with a per-column gain.  Reading (the
 * pages print no formula): the mean runs over the K normalised columns, eps
 * is added inside the square root, and the exact real value (here fp64) is
 * what the product path rounds once to BF16 before its MXFP8 quantize.
 * x: BF16 [M, >= K] with row stride ldx; w: BF16 [K]; y: fp64 [M, K]. */
int orc_rmsnorm(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint16_t *w,
                double eps, double *y)
{
    if (K < 1 || ldx < K || !(eps >= 0.0))
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * ldx;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = orc_bf16_value(row[k]);
            if (!isfinite(v))
                return -1;
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            y[m * K + k] = orc_bf16_value(row[k]) * orc_bf16_value(w[k]) * r;
    }
    return 0;
}

/* Thread count for the parallel loop of orc_gemm: set it, and read back the
 * number a parallel region actually runs with. */
void orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
