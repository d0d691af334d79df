/*
 * oracle.c -- plain, slow, single-threaded fp64 reference of the MXFP4
 * mixture-of-experts MLP layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only tests/, the smoke check in __graft_entry__.py and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant generator with the HIP library under mxfp4_quantized_mixture_amd/.
 *
 * Every step is written the way the pages define it, in plain loops, with
 * fp64 arithmetic and libm.  There is no blocking, fusion or reordering beyond
 * what the definitions state.
 *
 * Sources (page titles; sections):
 *  [TRICKS]  "Tricks from OpenAI gpt-oss you can use with transformers"
 *            (pogovet.com summary), section 6 "MXFP4 format and memory
 *            savings" and section 8 "MXFP4 kernel distribution".
 *  [WELCOME] "Welcome GPT OSS, the new open-source model family from OpenAI!"
 *            (pogovet.com summary), section 4 "MoE, quantization, context".
 *  [TALK]    aitrends.kr talk summary, sections "Architecture details: MoE
 *            and attention" (the hyper-parameter block) and "Hardware
 *            optimisation: Triton and Metal kernels".
 *  [REVIEW]  "MXFP4 기반 MoE (Mixture-of-Experts) 기술 리뷰", section 1
 *            (MXFP4 is the OCP Microscaling E2M1 format) and section 4
 *            (block-level outliers).
 *  [JA]      "Transformers 4.40 のパフォーマンス向上（OpenAI GPT-OSS 向け）",
 *            section "MXFP4 とは" (E2M1 bit split, 32-element blocks).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *  - E2M1: exponent bias 1, exponent field 0 is subnormal (0 or 0.5): the OCP
 *    MX reading, since [REVIEW] s.1 names OCP MX as the standard.
 *  - The shared scale is an E8M0 byte b meaning 2^(b-127); b = 255 (NaN) is
 *    never produced.
 *  - Scale rule 0: s = floor(log2(amax / 6)); rule 1 (OCP MX v1.0):
 *    s = floor(log2(amax)) - 2; rule 2: s = ceil(log2(amax / 6)), the
 *    smallest scale at which no element exceeds 6 (so stochastic rounding
 *    never saturates).  s is clamped to [-127, 127]; amax = 0 gives s = -127.
 *  - Element encode: round to nearest E2M1 value, ties to the even code,
 *    saturate at +-6, keep the sign bit (so -0 and negatives that round to
 *    zero give code 0x8).
 *  - Stochastic rounding (the training recipe "MXFP4 기반 MoE 기술 리뷰"
 *    section 2 cites, with no details): between the neighbouring E2M1 values
 *    lo <= |y| < hi, hi is taken with probability (|y| - lo) / (hi - lo), so
 *    the expected value is |y|.  The draw for element i = row * K + col is
 *    output i + 1 of a SplitMix64 generator whose state starts at the seed,
 *    its top 24 bits as an integer u; hi is taken when u < 2^24 (|y| - lo) /
 *    (hi - lo).
 *  - Packing: byte i of a row holds element 2i in its low nibble and element
 *    2i+1 in its high nibble; blocks run along the contraction dimension.
 *  - Router: logits = x . Wr^T + b (a linear layer with bias).
 *  - Top-k order: logit descending, ties to the lower expert id.
 *  - Expert MLP: textbook SwiGLU, h = silu(g) * u with silu(z) = z / (1 + e^-z),
 *    no expert biases, no clamp; W13 stacks the F gate rows over the F up rows.
 *  - Combine: out[t] = sum over slots j = 0..k-1, in slot order, of
 *    w[t,j] * y[t,j].
 *  - Stable permutation: pairs p = t*k + j sorted by (expert, p).
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalars                                                                   */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> double.  bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 code (4 bits: sign, 2 exponent bits, 1 mantissa bit) -> value.
 * [TRICKS] s.6 and [JA] "MXFP4 とは" give the 1/2/1 bit split; bias and the
 * subnormal exponent field follow OCP MX ([REVIEW] s.1). */
double oracle_e2m1_value(int code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * m;                       /* subnormal: m * 2^(1-1) / 2 */
    else
        mag = ldexp(1.0 + 0.5 * m, e - 1);   /* normal: (1 + m/2) * 2^(e-1) */
    return sign ? -mag : mag;
}

/* E8M0 byte -> the power of two it stands for. */
double oracle_e8m0_value(int byte)
{
    if (byte == 255)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/* Largest integer s with c * 2^s <= amax (= floor(log2(amax / c))), exactly:
 * the libm guess is corrected by exact power-of-two comparisons, since
 * amax / c can round onto a power of two. */
static int floor_log2_ratio(double amax, double c)
{
    int s = (int)floor(log2(amax / c));
    while (ldexp(c, s + 1) <= amax)
        ++s;
    while (ldexp(c, s) > amax)
        --s;
    return s;
}

/* Smallest integer s with amax <= c * 2^s (= ceil(log2(amax / c))), exactly. */
static int ceil_log2_ratio(double amax, double c)
{
    int s = (int)ceil(log2(amax / c));
    while (ldexp(c, s - 1) >= amax)
        --s;
    while (ldexp(c, s) < amax)
        ++s;
    return s;
}

/* Shared block exponent s from the block's largest magnitude.
 * rule 0: s = floor(log2(amax / 6)); rule 1 (OCP MX): floor(log2 amax) - 2;
 * rule 2: s = ceil(log2(amax / 6)). */
int oracle_scale_exponent(double amax, int rule)
{
    int s;
    if (amax == 0.0)
        return -127;
    if (rule == 0)
        s = floor_log2_ratio(amax, 6.0);
    else if (rule == 1)
        s = floor_log2_ratio(amax, 1.0) - 2;
    else
        s = ceil_log2_ratio(amax, 6.0);
    if (s < -127)
        s = -127;
    if (s > 127)
        s = 127;
    return s;
}

/* The 8 non-negative E2M1 values, by magnitude code. */
static void e2m1_grid(double grid[8])
{
    for (int c = 0; c < 8; ++c)
        grid[c] = oracle_e2m1_value(c);
}

/* Magnitude code (0..7) of the E2M1 value nearest to a >= 0; ties go to the
 * code whose mantissa bit is 0 (round half to even); values beyond 6 take
 * the largest code (saturation, E2M1 has no infinity). */
static int e2m1_nearest_magnitude(double a, const double grid[8])
{
    if (a >= grid[7])
        return 7;   /* at or beyond the largest value: saturate (checked first,
                       since for huge a the fp64 distances below all round equal) */
    int best = 0;
    double best_err = fabs(a - grid[0]);
    for (int c = 1; c < 8; ++c) {
        double err = fabs(a - grid[c]);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return best;
}

static int e2m1_encode_grid(double y, const double grid[8])
{
    int sign = signbit(y) ? 1 : 0;
    return (sign << 3) | e2m1_nearest_magnitude(fabs(y), grid);
}

/* E2M1 code of an already-scaled value y (sign kept, including -0). */
int oracle_e2m1_encode(double y)
{
    double grid[8];
    e2m1_grid(grid);
    return e2m1_encode_grid(y, grid);
}

/* SplitMix64, output n >= 1 of the generator whose state starts at `seed`:
 * the state advances by the golden-ratio increment 0x9E3779B97F4A7C15 and
 * each output is the state through the mixing function of the JDK's
 * java.util.SplittableRandom (mix64; the same constants as S. Vigna's
 * public-domain splitmix64.c). */
uint64_t oracle_splitmix64(uint64_t seed, uint64_t n)
{
    uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Stochastic rounding of an already-scaled y with the draw u in [0, 2^24):
 * between the neighbouring values grid[c] <= |y| < grid[c + 1], the upper one
 * is taken when u < 2^24 (|y| - grid[c]) / (grid[c + 1] - grid[c]) (every
 * quantity here is exact in fp64); |y| >= 6 saturates; sign kept. */
static int e2m1_encode_stochastic(double y, uint32_t u, const double grid[8])
{
    int sign = signbit(y) ? 1 : 0;
    double a = fabs(y);
    int c = 7;
    if (a < grid[7]) {
        c = 0;
        while (grid[c + 1] <= a)
            ++c;
        double frac = (a - grid[c]) / (grid[c + 1] - grid[c]);
        if ((double)u < ldexp(frac, 24))
            ++c;
    }
    return (sign << 3) | c;
}

int oracle_e2m1_encode_stochastic(double y, uint32_t u)
{
    double grid[8];
    e2m1_grid(grid);
    return e2m1_encode_stochastic(y, u, grid);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 quantize / dequantize                                               */
/* ------------------------------------------------------------------------ */

/* w: bf16 bits [rows, K]; q: [rows, K/2] packed codes; s: [rows, K/32] E8M0.
 * rounding 0: nearest even; 1: stochastic with the given seed.
 * Returns 0, or -1 if K is not a multiple of 32 or the rule or rounding is
 * unknown. */
int oracle_quantize_ex(const uint16_t *w, int64_t rows, int64_t K, int rule,
                       int rounding, uint64_t seed, uint8_t *q, uint8_t *s)
{
    if (K % 32 != 0 || rule < 0 || rule > 2 || rounding < 0 || rounding > 1)
        return -1;
    int64_t nblk = K / 32;
    double grid[8];
    e2m1_grid(grid);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            const uint16_t *blk = w + r * K + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                double a = fabs(oracle_bf16_to_double(blk[i]));
                if (a > amax)
                    amax = a;
            }
            int se = oracle_scale_exponent(amax, rule);
            s[r * nblk + b] = (uint8_t)(se + 127);
            double inv_scale = ldexp(1.0, -se);   /* 2^-s: products are exact */
            int codes[32];
            for (int i = 0; i < 32; ++i) {
                double y = oracle_bf16_to_double(blk[i]) * inv_scale;
                if (rounding == 0) {
                    codes[i] = e2m1_encode_grid(y, grid);
                } else {
                    uint64_t idx = (uint64_t)(r * K + b * 32 + i);
                    uint32_t u = (uint32_t)(oracle_splitmix64(seed, idx + 1) >> 40);
                    codes[i] = e2m1_encode_stochastic(y, u, grid);
                }
            }
            uint8_t *qb = q + r * (K / 2) + b * 16;
            for (int i = 0; i < 16; ++i)
                qb[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
    return 0;
}

int oracle_quantize(const uint16_t *w, int64_t rows, int64_t K, int rule,
                    uint8_t *q, uint8_t *s)
{
    return oracle_quantize_ex(w, rows, K, rule, 0, 0, q, s);
}

/* Element (r, c) of a packed MXFP4 matrix with K columns, as a double. */
double oracle_mxfp4_element(const uint8_t *q, const uint8_t *s, int64_t K,
                            int64_t r, int64_t c)
{
    uint8_t byte = q[r * (K / 2) + c / 2];
    int code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e8m0_value(s[r * (K / 32) + c / 32]);
}

void oracle_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                       int64_t K, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < K; ++c)
            out[r * K + c] = oracle_mxfp4_element(q, s, K, r, c);
}

/* ------------------------------------------------------------------------ */
/* Router: logits, top-k, softmax-after-topk, histogram, permutation          */
/* ------------------------------------------------------------------------ */

/* x: bf16 [T, D]; wr: fp32 [E, D]; b: fp32 [E] or NULL (zero bias).
 * Outputs (all caller-allocated):
 *   logits [T, E] fp64, ids [T, k], w [T, k] fp64, gap [T] fp64,
 *   counts [E], offsets [E+1], sorted [T*k], pos [T*k].
 * gap[t] is the smallest difference between consecutive entries of the
 * token's min(k+1, E) largest logits (+inf when there is only one): when it
 * is tiny, the selected set or its order depends on rounding.
 * Token-choice routing with softmax over the selected experts only:
 * [WELCOME] s.4; k of E experts: [TALK] architecture block. */
int oracle_route(const uint16_t *x, const float *wr, const float *b,
                 int T, int D, int E, int k,
                 double *logits, int32_t *ids, double *w, double *gap,
                 int32_t *counts, int32_t *offsets, int32_t *sorted,
                 int32_t *pos)
{
    if (k < 1 || k > E || E > 256)
        return -1;
    int *taken = (int *)malloc(sizeof(int) * (size_t)E);
    if (!taken)
        return -2;

    for (int t = 0; t < T; ++t) {
        double *L = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += oracle_bf16_to_double(x[(int64_t)t * D + d]) *
                       (double)wr[(int64_t)e * D + d];
            L[e] = acc + (b ? (double)b[e] : 0.0);
        }

        /* Selection: repeatedly take the largest remaining logit, lower id
         * first on equal logits.  Rank min(k+1, E) of them for the gap. */
        int nrank = (k + 1 < E) ? k + 1 : E;
        double ranked[257];
        for (int e = 0; e < E; ++e)
            taken[e] = 0;
        for (int j = 0; j < nrank; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || L[e] > L[best]))
                    best = e;
            taken[best] = 1;
            ranked[j] = L[best];
            if (j < k)
                ids[(int64_t)t * k + j] = best;
        }
        double g = INFINITY;
        for (int j = 0; j + 1 < nrank; ++j)
            if (ranked[j] - ranked[j + 1] < g)
                g = ranked[j] - ranked[j + 1];
        gap[t] = g;

        /* softmax over the k selected logits */
        double mx = L[ids[(int64_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j)
            den += exp(L[ids[(int64_t)t * k + j]] - mx);
        for (int j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = exp(L[ids[(int64_t)t * k + j]] - mx) / den;
    }
    free(taken);

    int64_t P = (int64_t)T * k;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        counts[ids[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    /* stable counting sort: within an expert, pairs keep increasing p */
    int64_t cursor = 0;
    for (int e = 0; e < E; ++e)
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e)
                sorted[cursor++] = (int32_t)p;
    for (int64_t i = 0; i < P; ++i)
        pos[sorted[i]] = (int32_t)i;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert MLP and combine                                                    */
/* ------------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert on widened (fp64) weights, applied to a list of tokens:
 *   y[i, :] = W2 h,  h = silu(Wg x_t) * (Wu x_t),  t = toks[i], i < n.
 *   x    bf16 [T, D] (only the listed rows are read)
 *   w13  fp64 [2F, D]: gate rows 0..F-1, up rows F..2F-1;  w2 fp64 [D, F]
 *   y    fp64 [n, D]
 * SwiGLU experts: [WELCOME] s.4.  Each token is a plain loop. */
static int expert_mlp_dense(const uint16_t *x, int D, int F, const double *w13,
                            const double *w2, const int32_t *toks, int n, double *y)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)D);
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    if (!xd || !h) {
        free(xd); free(h);
        return -2;
    }
    for (int i = 0; i < n; ++i) {
        int t = toks[i];
        for (int d = 0; d < D; ++d)
            xd[d] = oracle_bf16_to_double(x[(int64_t)t * D + d]);
        for (int f = 0; f < F; ++f) {
            double g = 0.0, u = 0.0;
            for (int d = 0; d < D; ++d) {
                g += w13[(int64_t)f * D + d] * xd[d];
                u += w13[(int64_t)(F + f) * D + d] * xd[d];
            }
            h[f] = silu(g) * u;
        }
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int f = 0; f < F; ++f)
                acc += w2[(int64_t)d * F + f] * h[f];
            y[(int64_t)i * D + d] = acc;
        }
    }
    free(xd); free(h);
    return 0;
}

/* One expert on MXFP4 weights:
 *   q13  [2F, D/2], s13 [2F, D/32]: gate rows 0..F-1, up rows F..2F-1
 *   q2   [D, F/2],  s2  [D, F/32]
 * other arguments as expert_mlp_dense.  The weights stay in MXFP4 and are
 * widened only for the arithmetic ([TALK] hardware section, [TRICKS] s.8):
 * here once per call, to fp64. */
int oracle_expert_mlp(const uint16_t *x, int D, int F, const uint8_t *q13,
                      const uint8_t *s13, const uint8_t *q2, const uint8_t *s2,
                      const int32_t *toks, int n, double *y)
{
    if (D % 32 != 0 || F % 32 != 0)
        return -1;
    double *w13 = (double *)malloc(sizeof(double) * (size_t)2 * F * D);
    double *w2 = (double *)malloc(sizeof(double) * (size_t)D * F);
    if (!w13 || !w2) {
        free(w13); free(w2);
        return -2;
    }
    oracle_dequantize(q13, s13, 2 * F, D, w13);
    oracle_dequantize(q2, s2, D, F, w2);
    int rc = expert_mlp_dense(x, D, F, w13, w2, toks, n, y);
    free(w13); free(w2);
    return rc;
}

/* One expert on bf16 weights (the bf16 fallback the pages compare MXFP4 with,
 * [TRICKS] s.7): w13 bf16 [2F, D], w2 bf16 [D, F], widened to fp64 exactly;
 * other arguments as expert_mlp_dense. */
int oracle_expert_mlp_bf16(const uint16_t *x, int D, int F, const uint16_t *w13b,
                           const uint16_t *w2b, const int32_t *toks, int n, double *y)
{
    if (D < 1 || F < 1)
        return -1;
    double *w13 = (double *)malloc(sizeof(double) * (size_t)2 * F * D);
    double *w2 = (double *)malloc(sizeof(double) * (size_t)D * F);
    if (!w13 || !w2) {
        free(w13); free(w2);
        return -2;
    }
    for (int64_t i = 0; i < (int64_t)2 * F * D; ++i)
        w13[i] = oracle_bf16_to_double(w13b[i]);
    for (int64_t i = 0; i < (int64_t)D * F; ++i)
        w2[i] = oracle_bf16_to_double(w2b[i]);
    int rc = expert_mlp_dense(x, D, F, w13, w2, toks, n, y);
    free(w13); free(w2);
    return rc;
}

/* The whole layer for the tokens listed in toks[0..ntok) (all T tokens in
 * order when toks is NULL):
 *   x    bf16 [T, D]
 *   q13  [E, 2F, D/2], s13 [E, 2F, D/32];  q2 [E, D, F/2], s2 [E, D, F/32]
 *   ids  [T, k], w [T, k] (fp64 routing weights)
 *   out  fp64 [ntok, D]
 * out[t] = sum over slots j = 0..k-1, in slot order, of w[t, j] * y(t, j),
 * y(t, j) = expert ids[t, j] applied to x_t (no shared expert: [TALK] Q&A).
 * Experts are visited one at a time only to bound memory. */
int oracle_moe(const uint16_t *x, const uint8_t *q13, const uint8_t *s13,
               const uint8_t *q2, const uint8_t *s2, const int32_t *ids,
               const double *w, int T, int D, int F, int E, int k,
               const int32_t *toks, int ntok, double *out)
{
    if (D % 32 != 0 || F % 32 != 0)
        return -1;
    if (!toks)
        ntok = T;
    double *y = (double *)malloc(sizeof(double) * (size_t)ntok * k * D);
    int32_t *list_tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)ntok * k);
    int32_t *list_slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)ntok * k);
    double *ye = (double *)malloc(sizeof(double) * (size_t)ntok * k * D);
    if (!y || !list_tok || !list_slot || !ye) {
        free(y); free(list_tok); free(list_slot); free(ye);
        return -2;
    }
    for (int e = 0; e < E; ++e) {
        int n = 0;
        for (int i = 0; i < ntok; ++i) {
            int t = toks ? toks[i] : i;
            for (int j = 0; j < k; ++j)
                if (ids[(int64_t)t * k + j] == e) {
                    list_tok[n] = t;
                    list_slot[n] = i * k + j;
                    ++n;
                }
        }
        if (n == 0)
            continue;
        int rc = oracle_expert_mlp(x, D, F, q13 + (int64_t)e * 2 * F * (D / 2),
                                   s13 + (int64_t)e * 2 * F * (D / 32),
                                   q2 + (int64_t)e * D * (F / 2),
                                   s2 + (int64_t)e * D * (F / 32), list_tok, n, ye);
        if (rc != 0) {
            free(y); free(list_tok); free(list_slot); free(ye);
            return rc;
        }
        for (int r = 0; r < n; ++r)
            memcpy(y + (int64_t)list_slot[r] * D, ye + (int64_t)r * D, sizeof(double) * (size_t)D);
    }
    for (int i = 0; i < ntok; ++i) {
        int t = toks ? toks[i] : i;
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(int64_t)t * k + j] * y[((int64_t)i * k + j) * D + d];
            out[(int64_t)i * D + d] = acc;
        }
    }
    free(y); free(list_tok); free(list_slot); free(ye);
    return 0;
}
