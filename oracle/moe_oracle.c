/*
 * moe_oracle.c -- plain, slow CPU oracle for the INT4 group-quantized
 * routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, load
 * or call this file.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table
 * or helper with the HIP path; the two meet only at the documented byte
 * format of their inputs.
 *
 * Sources (the web pages this method is described on):
 *   [VO]  "Running 125B MoE on Three 3090s - vLLM Optimization Edition",
 *         section 3.3 (small GEMVs), sub-section "MoE block (decode-05)";
 *         sub-section "Hyper-connection (decode-04)" for the pack-quantized
 *         word layout.
 *   [VE]  "Running 125B MoE on Three 3090s - vLLM Edition", section 1
 *         (shape of the model) and section 2 (bit allocation).
 *   [MC]  Model card "Qwen3.8-Flash-Next-INT4-Mixed-AutoRound", table
 *         "What is quantized".
 *
 * Everything is computed straight from its definition, in double precision,
 * one output at a time.  Weights are dequantized on the fly as
 * code * scale for every multiply; nothing is blocked, fused or reordered.
 * The only concession to run time is OpenMP loops over independent tokens
 * or (token, expert) pairs, which do not change any arithmetic.
 *
 * Readings where the pages leave a step open (each listed with its reason
 * in the design notes of the repository):
 *   - INT4 words hold 8 codes, element k of a row in nibble k%8 of word
 *     k/8, least significant nibble first, stored as code+8 (by analogy
 *     with the INT8 layout of [VO] decode-04: least significant byte
 *     first, stored as value+128).
 *   - Scales are bf16, one per (output row, 128 consecutive inputs),
 *     symmetric, no zero point ([MC], group A).
 *   - Logits are accumulated exactly enough in fp64 and then rounded once to
 *     fp32; expert selection is made on those fp32 values (the GPU kernel's
 *     precision).  Ties select the lower expert id ([VO] decode-05).
 *   - Fused gate/up: rows [0, I) are the gate (SiLU applied), rows [I, 2I)
 *     the up projection.
 *   - INT6 (shared expert): 32 codes packed tightly in six 32-bit words,
 *     code i in bits [6i, 6i+6) of the little-endian 192-bit block, stored
 *     as code+32; group 64 ([VO] decode-05, [MC] group B).
 *   - The shared expert is added as sigmoid(gate logit) * shared output,
 *     the gate logit being one extra bf16 router row ([VO] decode-05).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE-754 binary32; widening is exact. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------------
 * Unpacking ([VO] decode-04 layout by analogy; [MC] group A)
 * ------------------------------------------------------------------- */

/* Signed INT4 code of element k of one packed row. */
int oracle_int4_code(const int32_t *row_words, int64_t k)
{
    uint32_t word = (uint32_t)row_words[k / 8];
    int nibble = (int)((word >> (4 * (k % 8))) & 0xFu);
    return nibble - 8;
}

/* Signed INT6 code of element k of one packed row (32 codes per 6 words). */
int oracle_int6_code(const int32_t *row_words, int64_t k)
{
    const uint32_t *block = (const uint32_t *)row_words + (k / 32) * 6;
    int i = (int)(k % 32);
    int bit = 6 * i;                 /* first bit inside the 192-bit block */
    int value = 0;
    for (int b = 0; b < 6; ++b) {    /* gather the six bits one at a time */
        int pos = bit + b;
        uint32_t w = block[pos / 32];
        value |= (int)((w >> (pos % 32)) & 1u) << b;
    }
    return value - 32;
}

/* Dequantized weight W[n][k] = code * scale[n][k / group]. */
static double int4_weight(const int32_t *packed, const uint16_t *scales,
                          int64_t n, int64_t K, int64_t group, int64_t k)
{
    const int32_t *row = packed + n * (K / 8);
    double scale = bf16_to_double(scales[n * (K / group) + k / group]);
    return (double)oracle_int4_code(row, k) * scale;
}

static double int6_weight(const int32_t *packed, const uint16_t *scales,
                          int64_t n, int64_t K, int64_t group, int64_t k)
{
    const int32_t *row = packed + n * (K / 32 * 6);
    double scale = bf16_to_double(scales[n * (K / group) + k / group]);
    return (double)oracle_int6_code(row, k) * scale;
}

/* Whole-matrix dequantization (used by the self-tests). W is [rows][K]. */
void oracle_dequant_int4(const int32_t *packed, const uint16_t *scales,
                         int64_t rows, int64_t K, int64_t group, double *W)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = int4_weight(packed, scales, n, K, group, k);
}

void oracle_dequant_int6(const int32_t *packed, const uint16_t *scales,
                         int64_t rows, int64_t K, int64_t group, double *W)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = int6_weight(packed, scales, n, K, group, k);
}

/* ---------------------------------------------------------------------
 * Router ([VE] section 2 and [MC]: the router stays bf16)
 * ------------------------------------------------------------------- */

/* logits[t][e] = sum_h x[t][h] * Wr[e][h], summed in fp64, then rounded
 * once to fp32 (the precision the selection is made in). */
void oracle_router_logits(const uint16_t *x, const uint16_t *router_w,
                          int64_t T, int64_t H, int64_t E, float *logits)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h)
                acc += bf16_to_double(x[t * H + h]) *
                       bf16_to_double(router_w[e * H + h]);
            logits[t * E + e] = (float)acc;
        }
}

/* ---------------------------------------------------------------------
 * Top-k selection and renormalised softmax ([VO] decode-05)
 * ------------------------------------------------------------------- */

/* Strict order on experts: larger logit first, equal logits by lower id. */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la != lb)
        return la > lb;
    return a < b;
}

/* For each token: ids[t][0..k) are the k highest logits, in descending
 * order (ties to the lower id), found by brute force: an expert is chosen
 * iff fewer than k experts rank before it; its position is that count.
 * weights[t][j] = softmax over all E experts, renormalised over the chosen
 * k (the page notes this equals a softmax over only the chosen logits). */
void oracle_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t k,
                         int32_t *ids, double *weights)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t t = 0; t < T; ++t) {
        double *p = (double *)malloc((size_t)E * sizeof(double));
        const float *l = logits + t * E;

        for (int64_t e = 0; e < E; ++e) {
            int64_t before = 0;
            for (int64_t o = 0; o < E; ++o)
                if (o != e && ranks_before(l[o], (int)o, l[e], (int)e))
                    ++before;
            if (before < k)
                ids[t * k + before] = (int32_t)e;
        }

        double lmax = -INFINITY;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > lmax)
                lmax = (double)l[e];
        double denom = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - lmax);
            denom += p[e];
        }
        for (int64_t e = 0; e < E; ++e)
            p[e] /= denom;

        double chosen = 0.0;
        for (int64_t j = 0; j < k; ++j)
            chosen += p[ids[t * k + j]];
        for (int64_t j = 0; j < k; ++j)
            weights[t * k + j] = p[ids[t * k + j]] / chosen;
        free(p);
    }
}

/* ---------------------------------------------------------------------
 * Expert histogram, offsets and stable permutation ([VO] decode-05: the
 * block-alignment step groups token slots by expert)
 * ------------------------------------------------------------------- */

/* slot s = t*k + j.  counts[e] = #slots routed to e; offsets = exclusive
 * prefix sum (offsets[E] = T*k); sorted_slots lists, expert by expert, the
 * slots routed to it in increasing slot order. */
void oracle_permutation(const int32_t *ids, int64_t T, int64_t k, int64_t E,
                        int32_t *counts, int32_t *offsets,
                        int32_t *sorted_slots)
{
    int64_t S = T * k;
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t s = 0; s < S; ++s)
        counts[ids[s]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t e = 0; e < E; ++e) {
        int64_t pos = offsets[e];
        for (int64_t s = 0; s < S; ++s)
            if (ids[s] == e)
                sorted_slots[pos++] = (int32_t)s;
    }
}

/* ---------------------------------------------------------------------
 * SwiGLU experts ([VO] decode-05; [VE] section 1 for the shapes)
 * ------------------------------------------------------------------- */

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* One SwiGLU expert applied to one token, INT4 weights.
 *   g[i] = sum_h W13[i][h] x[h],   u[i] = sum_h W13[I+i][h] x[h]
 *   a[i] = silu(g[i]) * u[i]
 *   y[r] = sum_i W2[r][i] a[i]
 * w13 is [2I][H], w2 is [H][I], both packed, group `group` along inputs. */
static void expert_int4(const uint16_t *xt, const int32_t *w13p,
                        const uint16_t *w13s, const int32_t *w2p,
                        const uint16_t *w2s, int64_t H, int64_t I,
                        int64_t group, double *act, double *y)
{
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double xv = bf16_to_double(xt[h]);
            g += int4_weight(w13p, w13s, i, H, group, h) * xv;
            u += int4_weight(w13p, w13s, I + i, H, group, h) * xv;
        }
        act[i] = silu(g) * u;
    }
    for (int64_t r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i)
            acc += int4_weight(w2p, w2s, r, I, group, i) * act[i];
        y[r] = acc;
    }
}

/* Same expert with INT6 weights (the shared expert). */
static void expert_int6(const uint16_t *xt, const int32_t *w13p,
                        const uint16_t *w13s, const int32_t *w2p,
                        const uint16_t *w2s, int64_t H, int64_t I,
                        int64_t group, double *act, double *y)
{
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double xv = bf16_to_double(xt[h]);
            g += int6_weight(w13p, w13s, i, H, group, h) * xv;
            u += int6_weight(w13p, w13s, I + i, H, group, h) * xv;
        }
        act[i] = silu(g) * u;
    }
    for (int64_t r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i)
            acc += int6_weight(w2p, w2s, r, I, group, i) * act[i];
        y[r] = acc;
    }
}

/* Routed experts combined for a chosen subset of tokens:
 *   out[s][r] = sum_j weights[t][j] * expert_{ids[t][j]}(x[t])[r],
 * t = tokens[s].  Expert e's weights start at e * (rows * words per row).
 * `nthreads` <= 0 uses the OpenMP default. */
void oracle_experts(const uint16_t *x, const int32_t *ids,
                    const double *weights, const int32_t *w13_packed,
                    const uint16_t *w13_scales, const int32_t *w2_packed,
                    const uint16_t *w2_scales, int64_t H, int64_t I,
                    int64_t k, int64_t group, int64_t n_sel,
                    const int32_t *tokens, double *out, int nthreads)
{
    int64_t pairs = n_sel * k;
    double *y = (double *)malloc((size_t)(pairs * H) * sizeof(double));
    int64_t w13_words = 2 * I * (H / 8), w13_nsc = 2 * I * (H / group);
    int64_t w2_words = H * (I / 8), w2_nsc = H * (I / group);
#ifdef _OPENMP
    /* a clause, not omp_set_num_threads: the thread count applies to this
     * call only and later calls keep the OpenMP default */
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
#endif
    {
        double *act = (double *)malloc((size_t)I * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t p = 0; p < pairs; ++p) {
            int64_t t = tokens[p / k];
            int64_t e = ids[t * k + p % k];
            expert_int4(x + t * H, w13_packed + e * w13_words,
                        w13_scales + e * w13_nsc, w2_packed + e * w2_words,
                        w2_scales + e * w2_nsc, H, I, group, act, y + p * H);
        }
        free(act);
    }
    for (int64_t s = 0; s < n_sel; ++s) {
        int64_t t = tokens[s];
        for (int64_t r = 0; r < H; ++r) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += weights[t * k + j] * y[(s * k + j) * H + r];
            out[s * H + r] = acc;
        }
    }
    free(y);
}

/* Shared expert for a subset of tokens: ys[s][r] = expert_int6(x[t])[r] and
 * its gate logit glogit[s] = sum_h x[t][h] gate_w[h] (fp64). */
void oracle_shared_int6(const uint16_t *x, const uint16_t *gate_w,
                        const int32_t *w13_packed, const uint16_t *w13_scales,
                        const int32_t *w2_packed, const uint16_t *w2_scales,
                        int64_t H, int64_t I, int64_t group, int64_t n_sel,
                        const int32_t *tokens, double *ys, double *glogit,
                        int nthreads)
{
#ifdef _OPENMP
    /* a clause, not omp_set_num_threads: the thread count applies to this
     * call only and later calls keep the OpenMP default */
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
#endif
    {
        double *act = (double *)malloc((size_t)I * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t s = 0; s < n_sel; ++s) {
            int64_t t = tokens[s];
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h)
                acc += bf16_to_double(x[t * H + h]) * bf16_to_double(gate_w[h]);
            glogit[s] = acc;
            expert_int6(x + t * H, w13_packed, w13_scales, w2_packed,
                        w2_scales, H, I, group, act, ys + s * H);
        }
        free(act);
    }
}

/* The whole layer for a subset of tokens (routing is computed for all T
 * tokens, since it is cheap, and returned in full).
 *   out[s] = sum_j w[t][j] expert_{id}(x[t])  (+ sigmoid(glogit) * shared)
 * The shared-expert arguments may all be NULL. */
void oracle_forward(const uint16_t *x, const uint16_t *router_w,
                    const int32_t *w13_packed, const uint16_t *w13_scales,
                    const int32_t *w2_packed, const uint16_t *w2_scales,
                    int64_t T, int64_t H, int64_t E, int64_t I, int64_t k,
                    int64_t group, const uint16_t *shared_gate_w,
                    const int32_t *sh_w13_packed, const uint16_t *sh_w13_scales,
                    const int32_t *sh_w2_packed, const uint16_t *sh_w2_scales,
                    int64_t sh_inter, int64_t sh_group, int64_t n_sel,
                    const int32_t *tokens, float *logits, int32_t *ids,
                    double *weights, double *out, int nthreads)
{
    oracle_router_logits(x, router_w, T, H, E, logits);
    oracle_topk_softmax(logits, T, E, k, ids, weights);
    oracle_experts(x, ids, weights, w13_packed, w13_scales, w2_packed,
                   w2_scales, H, I, k, group, n_sel, tokens, out, nthreads);
    if (shared_gate_w != NULL) {
        double *ys = (double *)malloc((size_t)(n_sel * H) * sizeof(double));
        double *gl = (double *)malloc((size_t)n_sel * sizeof(double));
        oracle_shared_int6(x, shared_gate_w, sh_w13_packed, sh_w13_scales,
                           sh_w2_packed, sh_w2_scales, H, sh_inter, sh_group,
                           n_sel, tokens, ys, gl, nthreads);
        for (int64_t s = 0; s < n_sel; ++s) {
            double gate = 1.0 / (1.0 + exp(-gl[s]));
            for (int64_t r = 0; r < H; ++r)
                out[s * H + r] += gate * ys[s * H + r];
        }
        free(ys);
        free(gl);
    }
}

/* ---------------------------------------------------------------------
 * Load-time INT4 quantizer ([VO] section 7: the draft head's experts are
 * made symmetric INT4 in groups of 128 by rounding to nearest, each group
 * taking the clipping range whose squared error is least).
 *
 * Readings (the page names the method only):
 *   - candidate clips: twenty ratios c_j = 1 - j/40, j = 0..19 (1 down to
 *     0.525) of the group's largest magnitude; the scale of candidate j is
 *     bf16(fp32(amax * k_j)) with k_j = fp32(c_j / 7), so the clipped
 *     magnitude maps to the largest positive code 7 (codes span [-8, 7]);
 *   - codes: the nearest integer to w / s, ties to even, clamped to [-8, 7];
 *   - the error of a candidate is sum_i (w_i - q_i s)^2 accumulated in fp32
 *     in index order (each term rounded to fp32, then added): the choice
 *     between candidates is an integer decision, taken in the precision of
 *     the GPU kernel, which makes the same operations in the same order;
 *   - the first candidate with the smallest error wins; candidates whose
 *     scale is below the smallest normal fp32 (2^-126) are skipped, and a
 *     group with none left (all zeros) gets scale 0 and codes 0.
 * Output layout is the path's own: element k of a row is nibble k%8 of
 * word k/8, stored as code+8; scales bf16 [rows][K/group].
 * ------------------------------------------------------------------- */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define ORACLE_QCLIPS 20

/* One group of n values: writes codes (in [-8, 7]) and the bf16 scale, and
 * the errors of the best and second-best candidates (for near-tie checks). */
void oracle_quantize_group(const uint16_t *w, int64_t n, int8_t *codes,
                           uint16_t *scale, float *best_err, float *second_err)
{
    float amax = 0.f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(bf16_bits_to_float(w[i]));
        if (a > amax) amax = a;
    }
    int best = -1;
    float e_best = INFINITY, e_second = INFINITY;
    uint16_t s_best = 0;
    for (int j = 0; j < ORACLE_QCLIPS; ++j) {
        const float kj = (float)((1.0 - j / 40.0) / 7.0);
        const float t = amax * kj;
        const uint16_t sb = float_to_bf16_rne(t);
        const float s = bf16_bits_to_float(sb);
        if (!(s >= 1.17549435e-38f)) continue;   /* below 2^-126: skipped */
        float err = 0.f;
        for (int64_t i = 0; i < n; ++i) {
            const float x = bf16_bits_to_float(w[i]);
            double q = rint((double)x / (double)s);
            if (q < -8.0) q = -8.0;
            if (q > 7.0) q = 7.0;
            const float d = x - (float)q * s;        /* exact */
            const float d2 = d * d;
            err = err + d2;
        }
        if (err < e_best) {
            e_second = e_best;
            e_best = err;
            best = j;
            s_best = sb;
        } else if (err < e_second) {
            e_second = err;
        }
    }
    if (best < 0) {   /* all-zero (or subnormal-only) group */
        for (int64_t i = 0; i < n; ++i) codes[i] = 0;
        *scale = 0;
        if (best_err) *best_err = 0.f;
        if (second_err) *second_err = INFINITY;
        return;
    }
    const float s = bf16_bits_to_float(s_best);
    for (int64_t i = 0; i < n; ++i) {
        double q = rint((double)bf16_bits_to_float(w[i]) / (double)s);
        if (q < -8.0) q = -8.0;
        if (q > 7.0) q = 7.0;
        codes[i] = (int8_t)q;
    }
    *scale = s_best;
    if (best_err) *best_err = e_best;
    if (second_err) *second_err = e_second;
}

/* W bf16 [rows][K] -> packed int32 [rows][K/8], scales bf16 [rows][K/group],
 * and per group the best and second-best candidate errors (may be NULL). */
void oracle_quantize_int4(const uint16_t *w, int64_t rows, int64_t K, int64_t group,
                          int32_t *packed, uint16_t *scales, float *best_err,
                          float *second_err)
{
    const int64_t ng = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int8_t *codes = (int8_t *)malloc((size_t)group);
        for (int64_t g = 0; g < ng; ++g) {
            const int64_t gi = r * ng + g;
            oracle_quantize_group(w + r * K + g * group, group, codes, scales + gi,
                                  best_err ? best_err + gi : NULL,
                                  second_err ? second_err + gi : NULL);
            for (int64_t i = 0; i < group; i += 8) {
                uint32_t word = 0;
                for (int b = 0; b < 8; ++b)
                    word |= (uint32_t)(codes[i + b] + 8) << (4 * b);
                packed[r * (K / 8) + (g * group + i) / 8] = (int32_t)word;
            }
        }
        free(codes);
    }
}

/* ---------------------------------------------------------------------
 * INT8 W8A16 linear layer ([VO] decode-04: four codes per 32-bit word,
 * least significant byte first, each stored as value + 128; [MC] groups C
 * and D: symmetric, group 64 for the hyper-connection mixers, group 128 for
 * lm_head and the embeddings)
 * ------------------------------------------------------------------- */

/* Signed INT8 code of element k of one packed row. */
int oracle_int8_code(const int32_t *row_words, int64_t k)
{
    uint32_t word = (uint32_t)row_words[k / 4];
    int byte = (int)((word >> (8 * (k % 4))) & 0xFFu);
    return byte - 128;
}

/* y[t][n] = sum_k x[t][k] * code[n][k] * scale[n][k / group], in fp64, one
 * output at a time (x bf16 [T][K], packed [N][K/4], scales bf16
 * [N][K/group]).  Not rounded: the comparison is made against the exact
 * value. */
void oracle_int8_linear(const uint16_t *x, const int32_t *packed, const uint16_t *scales,
                        int64_t T, int64_t N, int64_t K, int64_t group, double *y)
{
    int64_t tn;
#pragma omp parallel for schedule(static)
    for (tn = 0; tn < T * N; ++tn) {
        int64_t t = tn / N, n = tn % N;
        const int32_t *row = packed + n * (K / 4);
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)oracle_int8_code(row, k) * bf16_to_double(scales[n * (K / group) + k / group]);
            acc += bf16_to_double(x[t * K + k]) * w;
        }
        y[t * N + n] = acc;
    }
}

/* Threads the OpenMP runtime will use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
