/*
 * fwref.c -- CPU oracle for the routed mixture-of-experts FFN layer run on GGUF
 * Q8_0 / Q4_0 / Q4_K / Q6_K / MXFP4 expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library shares no
 * code, header, table or helper with it, and the GPU path never calls it.
 *
 * It is the plain definition of what the layer computes, written for a reader
 * to check by eye: straight loops, no blocking, no fusion, no reordering.
 * Dequantised Q8_0 / Q4_0 weights are exact in fp32 (an fp16 scale times a code
 * of at most 8 significant bits fits in 24 bits); a Q4_K weight is formed
 * exactly in fp64 and rounded once to fp32 (a Q6_K weight, d * scale * code
 * with an fp16 d, an int8 scale and a six-bit code, is exact in fp32 too);
 * every sum is accumulated in fp64 in
 * ascending index order and rounded to fp32 only where the layer's interface
 * hands a value over (logits, gate weights, output).
 *
 * What is computed, and where the pages describe it:
 *  - the layer itself: "sparse MoE execution" with grouped routed-expert
 *    kernels per format (Flyweight 0.2.0 wheel METADATA, "Features" and
 *    "Quantization"; Flyweight 0.5.1, "Models and formats");
 *  - Q8_0 and Q4_0 as expert formats (Flyweight 0.5.1, "Models and formats";
 *    Gemma 4's routed experts must be Q4_0, Flyweight 0.2.0 "Current
 *    limitations"); the byte layout is GGUF's, which the pages do not print;
 *  - Q4_K, the K-quant the pages name as the smallest a MoE checkpoint packs
 *    to and one of BailingMoE3's two grouped expert formats (Flyweight 0.2.0,
 *    "Quantization" and "Current limitations"; Flyweight 0.5.1, "Models and
 *    formats").  Its layout is again GGUF's and not printed by the pages:
 *    PARITY UNPINNED against an outside encoder (none is available here);
 *    the tests pin it by round trips, by the cases that reduce to Q4_0 and by
 *    brute force over code positions;
 *  - Q6_K, the other of BailingMoE3's two grouped expert formats and one of
 *    the K-quants the newer page lists grouped kernels for (Flyweight 0.2.0,
 *    "Current limitations"; Flyweight 0.5.1, "Models and formats").  GGUF's
 *    layout again, PARITY UNPINNED against an outside encoder; pinned the
 *    same way as Q4_K;
 *  - MXFP4 (group 32), the expert-only format of vOOM's lossy artifacts (vOOM,
 *    the Qwen3.6-35B-A3B side-quest notes: routed expert matrices only, MLX
 *    weight/scale pairs, --mode mxfp4 --group-size 32).  MLX's packing: a
 *    matrix of R rows is its E2M1 codes, R x K/2 bytes (element j of a row in
 *    nibble j % 2 of byte j / 2, low nibble first), followed by its E8M0
 *    scales, R x K/32 bytes; value = E2M1(code) * 2^(scale - 127), exact in
 *    fp32 below 2^128 (from scale 253 on the larger values are infinite);
 *    scale 255 is NaN.  PARITY UNPINNED against an outside encoder;
 *  - MXFP8 expert activations beside MXFP4 experts (vOOM, the lossy artifact
 *    notes: the MXFP8 control and MX formats with group size 32; an option,
 *    fwref_forward_mx8).  OCP MX quantisation of a 32-element block V:
 *    shared scale X = 2^(floor(log2(max |V_i|)) - 8), 8 being E4M3's largest
 *    exponent, stored as the E8M0 byte floor(log2 amax) - 8 + 127 clamped to
 *    0..254 (an all-zero block: byte 0, codes 0); elements E4M3 (OCP E4M3FN:
 *    bias 7, 3 mantissa bits, largest 448) of V_i / X, nearest with ties to
 *    the even code, magnitudes above 448 clamped to 448.  The quantiser's
 *    input is the fp32 value (x as handed in; the SwiGLU output rounded to
 *    fp32), so that both sides of a comparison take each code decision on
 *    the same number.  PARITY UNPINNED against an outside encoder; pinned by
 *    hand-decoded blocks and a brute-force nearest-code search;
 *  - int8 expert activations beside Q8_0 / Q4_0 experts, the pages' MMQ
 *    path: prompt processing's routed experts on block-table MMQ kernels
 *    (Flyweight 0.2.0, "Runtime controls", --routed-moe), activations
 *    quantised to int8 for them (Flyweight 0.2.0, "Image generation", the
 *    `fast` precision) and Q8 activations in the dp4a kernels (Flyweight
 *    0.2.0, "Quantization"); an option, fwref_forward_q8a.  The pages print
 *    no activation format; the reading taken is GGUF's Q8_1-style block of
 *    32: d = max |V_i| / 127 (fp32 division), codes round(V_i / d) (fp32
 *    division, ties away from zero, at most 127 in magnitude), d kept in
 *    fp32 (an all-zero block: d = 0, codes 0).  The value a code stands for
 *    is d * code, exact in fp64.  As for MXFP8 the quantiser's input is the
 *    fp32 value (x as handed in; the SwiGLU output rounded to fp32).  PARITY
 *    UNPINNED against an outside encoder; pinned by hand-computed blocks and
 *    the round-trip bound;
 *  - SwiGLU expert FFNs (vOOM, module layout: layer_runner's block math);
 *  - top-k routing with k a tunable (vOOM notes: the request-local top-2
 *    expert schedule) and DeepSeek-shaped sigmoid routing with an always-on
 *    shared expert (Flyweight 0.2.0, served-families table, K2-Horizon);
 *  - a fixed-order, deterministic expert combine (vOOM notes: the rejected
 *    gathered/fused expert prototype that changed the token stream).
 * Where the pages are silent the plainest reading is taken: selection on the
 * (biased) logits, descending, ties to the lower expert index, slot order =
 * selection order; renormalisation divides each selected score by the sum of
 * the selected scores; the shared expert is added with weight 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_F32 = 0, REF_BF16 = 1 };
enum { REF_Q8_0 = 0, REF_Q4_0 = 1, REF_Q4_K = 2, REF_Q6_K = 3, REF_MXFP4 = 4 };
enum { REF_SOFTMAX = 0, REF_SIGMOID = 1 };

/* IEEE 754 binary16 -> value: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits; exponent 0 is the subnormal range m * 2^-24. */
float fwref_half_to_float(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 31, m = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)m, -24);
    else if (ex == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), ex - 25);
    return (float)(sign ? -v : v);
}

/* bfloat16 is the top half of a binary32. */
float fwref_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Bytes of a row of n elements: 32-element blocks of 34 (Q8_0) or 18 (Q4_0)
 * bytes, 256-element super-blocks of 144 (Q4_K) or 210 (Q6_K) bytes; MXFP4
 * rows hold their n / 2 code bytes here (the scales sit after the matrix). */
static size_t row_bytes(int qtype, int n)
{
    switch (qtype) {
        case REF_Q8_0: return (size_t)n / 32 * 34;
        case REF_Q4_0: return (size_t)n / 32 * 18;
        case REF_Q4_K: return (size_t)n / 256 * 144;
        case REF_Q6_K: return (size_t)n / 256 * 210;
        default: return (size_t)n / 2;
    }
}

/* OCP MX E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; the
 * exponent-0 codes are the subnormals 0 and 0.5. */
static double e2m1_value(int code)
{
    int ex = (code >> 1) & 3, m = code & 1;
    double v = ex == 0 ? 0.5 * m : (1.0 + 0.5 * m) * (double)(1 << (ex - 1));
    return code & 8 ? -v : v;
}

/* Row r (of R) of an MXFP4 matrix of n-element rows starting at base. */
static void mxfp4_row(const uint8_t *base, size_t R, size_t r, int n, float *out)
{
    const uint8_t *codes = base + r * (size_t)(n / 2);
    const uint8_t *scales = base + R * (size_t)(n / 2) + r * (size_t)(n / 32);
    for (int b = 0; b < n / 32; ++b) {
        int s = scales[b];
        double x = ldexp(1.0, s - 127);   /* the block's scale 2^(s - 127), exact */
        for (int j = 32 * b; j < 32 * b + 32; ++j) {
            int code = j % 2 ? codes[j / 2] >> 4 : codes[j / 2] & 15;
            out[j] = s == 255 ? NAN : (float)(e2m1_value(code) * x);
        }
    }
}

void fwref_dequant_row(int qtype, const uint8_t *row, int n, float *out);

/* Row r of a matrix of R rows of n elements in format qtype at base. */
static void matrix_row(int qtype, const uint8_t *base, size_t R, size_t r, int n, float *out)
{
    if (qtype == REF_MXFP4)
        mxfp4_row(base, R, r, n, out);
    else
        fwref_dequant_row(qtype, base + r * row_bytes(qtype, n), n, out);
}

/* Q4_K sub-block j's 6-bit scale and min from the 12 packed bytes: j < 4 keep
 * them in the low 6 bits of bytes j and j + 4; j >= 4 take their low 4 bits
 * from byte j + 4 (scale: low nibble, min: high nibble) and their top 2 bits
 * from the top 2 bits of bytes j - 4 (scale) and j (min). */
static void q4k_scale_min(const uint8_t *sc, int j, int *scale, int *min)
{
    if (j < 4) {
        *scale = sc[j] & 63;
        *min = sc[j + 4] & 63;
    } else {
        *scale = (sc[j + 4] & 15) | (sc[j - 4] >> 6) << 4;
        *min = (sc[j + 4] >> 4) | (sc[j] >> 6) << 4;
    }
}

/* Dequantise one row of n elements (n a multiple of 32; of 256 for Q4_K).
 * Q8_0 block: [fp16 d][32 int8 q], value_i = d * q_i.
 * Q4_0 block: [fp16 d][16 bytes], byte i = q_i | q_{i+16} << 4,
 *             value_i = d * (q_i - 8).
 * Q4_K super-block of 256 elements, 144 bytes: [fp16 d][fp16 dmin]
 *             [12 bytes: eight 6-bit (scale, min) pairs][128 bytes of codes];
 *             group c (0..3) of 64 elements reads code bytes 32c .. 32c + 31:
 *             element 64c + l is the low nibble of byte 32c + l (sub-block
 *             2c), element 64c + 32 + l its high nibble (sub-block 2c + 1);
 *             value = d * scale_j * q - dmin * min_j for sub-block j.
 * Q6_K super-block of 256 elements, 210 bytes: [128 bytes ql][64 bytes qh]
 *             [16 int8 scales][fp16 d].  Each half (128 elements, h = 0, 1)
 *             uses ql bytes 64h .. 64h + 63 and qh bytes 32h .. 32h + 31;
 *             its element 32k + l (k = 0..3, l = 0..31) takes its low four
 *             bits from ql byte 64h + 32 (k % 2) + l (low nibble for k < 2,
 *             high for k >= 2) and its top two bits from bits 2k, 2k + 1 of
 *             qh byte 32h + l: a six-bit code q.  Sub-block j = e / 16 of 16
 *             elements has scale byte j; value = d * scale_j * (q - 32).
 * MXFP4: the row's n / 2 code bytes followed by its n / 32 E8M0 scales. */
void fwref_dequant_row(int qtype, const uint8_t *row, int n, float *out)
{
    if (qtype == REF_MXFP4) {   /* a one-row matrix: n / 2 code bytes, n / 32 scales */
        mxfp4_row(row, 1, 0, n, out);
        return;
    }
    if (qtype == REF_Q6_K) {
        for (int b = 0; b < n / 256; ++b) {
            const uint8_t *blk = row + (size_t)b * 210;
            const uint8_t *ql = blk, *qh = blk + 128;
            const int8_t *sc = (const int8_t *)(blk + 192);
            double d = fwref_half_to_float((uint16_t)(blk[208] | blk[209] << 8));
            for (int e = 0; e < 256; ++e) {
                int h = e / 128, k = (e % 128) / 32, l = e % 32;
                int lo = ql[64 * h + 32 * (k % 2) + l];
                lo = k < 2 ? lo & 15 : lo >> 4;
                int hi = (qh[32 * h + l] >> (2 * k)) & 3;
                int q = lo | hi << 4;
                out[256 * b + e] = (float)(d * sc[e / 16] * (q - 32));
            }
        }
        return;
    }
    if (qtype == REF_Q4_K) {
        for (int b = 0; b < n / 256; ++b) {
            const uint8_t *blk = row + (size_t)b * 144;
            double d = fwref_half_to_float((uint16_t)(blk[0] | blk[1] << 8));
            double dmin = fwref_half_to_float((uint16_t)(blk[2] | blk[3] << 8));
            const uint8_t *sc = blk + 4, *qs = blk + 16;
            for (int e = 0; e < 256; ++e) {
                int c = e / 64, l = e % 32, high = (e % 64) >= 32;
                int j = 2 * c + high, scale, min;
                q4k_scale_min(sc, j, &scale, &min);
                int q = high ? qs[32 * c + l] >> 4 : qs[32 * c + l] & 15;
                out[256 * b + e] = (float)(d * scale * q - dmin * min);
            }
        }
        return;
    }
    for (int b = 0; b < n / 32; ++b) {
        const uint8_t *blk = row + (size_t)b * (qtype == REF_Q8_0 ? 34 : 18);
        float d = fwref_half_to_float((uint16_t)(blk[0] | blk[1] << 8));
        if (qtype == REF_Q8_0) {
            for (int i = 0; i < 32; ++i)
                out[32 * b + i] = d * (float)(int8_t)blk[2 + i];
        } else {
            for (int i = 0; i < 16; ++i) {
                out[32 * b + i] = d * (float)((blk[2 + i] & 15) - 8);
                out[32 * b + i + 16] = d * (float)((blk[2 + i] >> 4) - 8);
            }
        }
    }
}

static float act_value(int dtype, const void *base, size_t i)
{
    if (dtype == REF_F32)
        return ((const float *)base)[i];
    return fwref_bf16_to_float(((const uint16_t *)base)[i]);
}

/* The router's work for token t (formulas at fwref_route). */
static void route_token(int H, int E, int k, int act_dtype, int router_dtype, int score,
                        const void *x, const void *router_w, const float *bias,
                        const float *logits_in, int t, float *logits, int32_t *ids, float *w)
{
    float *l = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e) {
        if (logits_in) {
            l[e] = logits_in[(size_t)t * E + e];
            continue;
        }
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += (double)act_value(act_dtype, x, (size_t)t * H + h) *
                   (double)act_value(router_dtype, router_w, (size_t)e * H + h);
        if (bias)
            acc += (double)bias[e];
        l[e] = (float)acc;
    }
    /* k rounds of "largest remaining logit"; scanning e upwards with a
     * strict comparison keeps the lower index on a tie. */
    char *taken = calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || l[e] > l[best]))
                best = e;
        taken[best] = 1;
        ids[(size_t)t * k + j] = best;
    }
    free(taken);

    double *p = malloc(sizeof(double) * (size_t)E);
    if (score == REF_SOFTMAX) {
        double mx = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > mx)
                mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp((double)l[e] - mx);
        for (int e = 0; e < E; ++e)
            p[e] = exp((double)l[e] - mx) / z;
    } else {
        for (int e = 0; e < E; ++e)
            p[e] = 1.0 / (1.0 + exp(-(double)l[e]));
    }
    double sel = 0.0;
    for (int j = 0; j < k; ++j)
        sel += p[ids[(size_t)t * k + j]];
    for (int j = 0; j < k; ++j)
        w[(size_t)t * k + j] = (float)(p[ids[(size_t)t * k + j]] / sel);
    free(p);
}

/* Router: logits, scoring, top-k selection and renormalised gate weights.
 *   l[t][e] = fp32( sum_h x[t][h] * W_r[e][h] + b_e )
 *   ids[t][0..k-1]: experts in descending order of l, ties to the lower index
 *   softmax: p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l)   (all E)
 *   sigmoid: p_e = 1 / (1 + exp(-l_e))
 *   w[t][j] = p_{ids[t][j]} / sum_{i<k} p_{ids[t][i]}
 * If logits_in is given it replaces the first line (it already holds the bias).
 * Tokens are independent and spread over OpenMP threads.
 * Returns 0, or -1 on a bad argument. */
int fwref_route(int T, int H, int E, int k, int act_dtype, int router_dtype, int score,
                const void *x, const void *router_w, const float *bias,
                const float *logits_in, float *logits, int32_t *ids, float *w)
{
    if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E)
        return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int t = 0; t < T; ++t)
        route_token(H, E, k, act_dtype, router_dtype, score, x, router_w, bias, logits_in, t,
                    logits, ids, w);
    return 0;
}

/* Token -> expert permutation, as a counting sort of the T*k (token, slot)
 * pairs by expert, stable in pair order q = t*k + j:
 *   offsets[e] = number of pairs routed to experts below e   (offsets[E] = T*k)
 *   sorted[offsets[e] ..]  = the pairs routed to e, in ascending q
 *   inv[q] = position of pair q in sorted
 * Returns 0, or -1 if an id lies outside [0, E). */
int fwref_permute(int T, int E, int k, const int32_t *ids, int32_t *offsets,
                  int32_t *sorted, int32_t *inv)
{
    long P = (long)T * k;
    int32_t *cursor = calloc((size_t)E + 1, sizeof(int32_t));
    for (long q = 0; q < P; ++q) {
        if (ids[q] < 0 || ids[q] >= E) {
            free(cursor);
            return -1;
        }
        cursor[ids[q]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + cursor[e];
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (long q = 0; q < P; ++q) {
        int e = ids[q];
        sorted[cursor[e]] = (int32_t)q;
        inv[q] = cursor[e];
        cursor[e]++;
    }
    free(cursor);
    return 0;
}

/* E4M3 (OCP E4M3FN) value of a code: sign bit 7, exponent bits 6..3 (bias
 * 7), mantissa bits 2..0; exponent 0 is subnormal (m / 8 * 2^-6); 0x7F and
 * 0xFF are NaN. */
double fwref_e4m3_value(int code)
{
    int sgn = code & 0x80, e = (code >> 3) & 15, m = code & 7;
    if ((code & 0x7F) == 0x7F)
        return NAN;
    double v = e == 0 ? ldexp(m, -9) : ldexp(8 + m, e - 10);
    return sgn ? -v : v;
}

/* E4M3 code of the nearest value to y (|y| <= 448 after the clamp), ties to
 * the even code: the step at |y|'s binade (2^(E - 3), E = max(floor(log2 |y|),
 * -6)) divides |y| exactly, rint rounds half to even, and the multiple of the
 * step that results is an E4M3 value (possibly the next binade's first). */
static int e4m3_code(float y)
{
    int sgn = signbit(y) ? 0x80 : 0;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sgn | 0x7E;
    if (a == 0.0)
        return sgn;
    int E = ilogb(a);
    if (E < -6)
        E = -6;
    double q = rint(ldexp(a, 3 - E));       /* units of the step 2^(E - 3) */
    if (q == 16.0) {                        /* rounded up into the next binade */
        E += 1;
        q = 8.0;
    }
    if (q < 8.0)                            /* subnormal (E = -6) */
        return sgn | (int)q;
    return sgn | ((E + 7) << 3) | ((int)q - 8);
}

/* OCP MX quantisation of n (a multiple of 32) fp32 values to MXFP8: E4M3
 * codes[n] and one E8M0 scale per 32-element block, scales[n / 32]. */
void fwref_mxfp8_quantize(const float *v, int n, uint8_t *codes, uint8_t *scales)
{
    for (int b = 0; b < n / 32; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i)
            if (fabsf(v[32 * b + i]) > amax)
                amax = fabsf(v[32 * b + i]);
        if (amax == 0.0f) {
            scales[b] = 0;
            for (int i = 0; i < 32; ++i)
                codes[32 * b + i] = signbit(v[32 * b + i]) ? 0x80 : 0;
            continue;
        }
        int e = ilogbf(amax) - 8;
        if (e < -127)
            e = -127;
        if (e > 127)
            e = 127;
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i)
            codes[32 * b + i] = (uint8_t)e4m3_code(ldexpf(v[32 * b + i], -e));
    }
}

/* The values an MXFP8 round trip gives: out = E4M3(code) * 2^(scale - 127). */
static void mxfp8_round_trip(const float *v, int n, float *out, uint8_t *codes,
                             uint8_t *scales)
{
    fwref_mxfp8_quantize(v, n, codes, scales);
    for (int i = 0; i < n; ++i)
        out[i] = (float)ldexp(fwref_e4m3_value(codes[i]), scales[i / 32] - 127);
}

/* int8 (Q8_1-style) quantisation of n (a multiple of 32) fp32 values:
 * codes[n] and one fp32 scale per 32-element block, scales[n / 32]. */
void fwref_q8a_quantize(const float *v, int n, int8_t *codes, float *scales)
{
    for (int b = 0; b < n / 32; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i)
            if (fabsf(v[32 * b + i]) > amax)
                amax = fabsf(v[32 * b + i]);
        float d = amax / 127.0f;
        scales[b] = d;
        for (int i = 0; i < 32; ++i) {
            float q = d == 0.0f ? 0.0f : roundf(v[32 * b + i] / d);
            if (q > 127.0f)
                q = 127.0f;
            if (q < -127.0f)
                q = -127.0f;
            codes[32 * b + i] = (int8_t)q;
        }
    }
}

/* The values an int8 round trip stands for, in fp64: out = d * code. */
static void q8a_round_trip(const float *v, int n, double *out, int8_t *codes, float *scales)
{
    fwref_q8a_quantize(v, n, codes, scales);
    for (int i = 0; i < n; ++i)
        out[i] = (double)scales[i / 32] * (double)codes[i];
}

enum { AQ_NONE = 0, AQ_MXFP8 = 1, AQ_Q8A = 2 };

/* One SwiGLU expert on one token:
 *   g_f = sum_h Wg[f][h] x_h,  u_f = sum_h Wu[f][h] x_h
 *   a_f = g_f * sigmoid(g_f) * u_f          (SiLU(gate) * up)
 *   y_o = sum_f Wd[o][f] a_f
 * Wg, Wu: rows r0gu .. r0gu + F - 1 of matrices of Rgu rows of H elements;
 * Wd: rows r0d .. r0d + H - 1 of a matrix of Rd rows of F elements; blocked
 * along the row (the reduction dimension). */
static void expert_ffn(int qtype, int F, int H, const uint8_t *wg, const uint8_t *wu,
                       const uint8_t *wd, size_t Rgu, size_t Rd, size_t r0gu, size_t r0d,
                       const double *x, double *y, float *row, double *a, int aq,
                       float *hq, uint8_t *qc, uint8_t *qs, float *qd)
{
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        matrix_row(qtype, wg, Rgu, r0gu + f, H, row);
        for (int h = 0; h < H; ++h)
            g += (double)row[h] * (double)x[h];
        matrix_row(qtype, wu, Rgu, r0gu + f, H, row);
        for (int h = 0; h < H; ++h)
            u += (double)row[h] * (double)x[h];
        a[f] = g / (1.0 + exp(-g)) * u;
    }
    if (aq == AQ_MXFP8) {   /* the down projection's input is MXFP8(fp32(a)) */
        for (int f = 0; f < F; ++f)
            hq[f] = (float)a[f];
        mxfp8_round_trip(hq, F, hq, qc, qs);
        for (int f = 0; f < F; ++f)
            a[f] = hq[f];
    } else if (aq == AQ_Q8A) {   /* ... or the int8 round trip of fp32(a) */
        for (int f = 0; f < F; ++f)
            hq[f] = (float)a[f];
        q8a_round_trip(hq, F, a, (int8_t *)qc, qd);
    }
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        matrix_row(qtype, wd, Rd, r0d + o, F, row);
        for (int f = 0; f < F; ++f)
            acc += (double)row[f] * a[f];
        y[o] = acc;
    }
}

/* The layer's output for T tokens:
 *   out[t] = fp32( sum_{j<k} w[t][j] * FFN_{ids[t][j]}(x_t)  +  FFN_shared(x_t) )
 * with the slot sum in order j = 0..k-1 and the shared expert (Fs > 0) last.
 * Expert e's rows are rows e * F .. (gate, up: E * F rows of H elements) and
 * e * H .. (down: E * H rows of F elements) of the routed matrices.  Tokens are independent, so they are spread over
 * n_threads OpenMP threads (0: the runtime's default).
 * Returns 0, or -1 on a bad argument or id. */
static int forward_impl(int T, int H, int E, int k, int F, int qtype, int Fs, int qtype_s,
                        int act_dtype, const void *x, const uint8_t *wg, const uint8_t *wu,
                        const uint8_t *wd, const uint8_t *sg, const uint8_t *su,
                        const uint8_t *sd, const int32_t *ids, const float *w, float *out,
                        int n_threads, int aq)
{
    if (T < 0 || H <= 0 || H % 32 || F <= 0 || F % 32 || k < 1 || k > E || Fs < 0 ||
        Fs % 32)
        return -1;
    /* K-quant rows are whole 256-element super-blocks */
    if ((qtype >= REF_Q4_K && (H % 256 || F % 256)) ||
        (Fs > 0 && qtype_s >= REF_Q4_K && (H % 256 || Fs % 256)))
        return -1;
    if (qtype < REF_Q8_0 || qtype > REF_MXFP4 || (Fs > 0 && (qtype_s < REF_Q8_0 || qtype_s > REF_MXFP4)))
        return -1;
    for (long q = 0; q < (long)T * k; ++q)
        if (ids[q] < 0 || ids[q] >= E)
            return -1;
    int maxf = F > Fs ? F : Fs;
    int maxr = H > maxf ? H : maxf;
#ifdef _OPENMP
    /* a per-region thread count: a request here does not change later calls */
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        float *xf = malloc(sizeof(float) * (size_t)H);
        double *xd = malloc(sizeof(double) * (size_t)H);
        float *qd = malloc(sizeof(float) * ((size_t)maxr / 32 + 1));
        float *row = malloc(sizeof(float) * (size_t)maxr);
        double *a = malloc(sizeof(double) * (size_t)maxf);
        double *y = malloc(sizeof(double) * (size_t)H);
        double *acc = malloc(sizeof(double) * (size_t)H);
        float *hq = malloc(sizeof(float) * (size_t)maxr);
        uint8_t *qc = malloc((size_t)maxr);
        uint8_t *qs = malloc((size_t)maxr / 32 + 1);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < H; ++h) {
                xf[h] = act_value(act_dtype, x, (size_t)t * H + h);
                acc[h] = 0.0;
            }
            /* the experts' input: x, or its MXFP8 or int8 round trip */
            if (aq == AQ_MXFP8)
                mxfp8_round_trip(xf, H, xf, qc, qs);
            if (aq == AQ_Q8A) {
                q8a_round_trip(xf, H, xd, (int8_t *)qc, qd);
            } else {
                for (int h = 0; h < H; ++h)
                    xd[h] = xf[h];
            }
            for (int j = 0; j < k; ++j) {
                int e = ids[(size_t)t * k + j];
                expert_ffn(qtype, F, H, wg, wu, wd, (size_t)E * F, (size_t)E * H,
                           (size_t)e * F, (size_t)e * H, xd, y, row, a, aq, hq, qc, qs, qd);
                for (int h = 0; h < H; ++h)
                    acc[h] += (double)w[(size_t)t * k + j] * y[h];
            }
            if (Fs > 0) {
                expert_ffn(qtype_s, Fs, H, sg, su, sd, (size_t)Fs, (size_t)H, 0, 0, xd, y,
                           row, a, aq, hq, qc, qs, qd);
                for (int h = 0; h < H; ++h)
                    acc[h] += y[h];
            }
            for (int h = 0; h < H; ++h)
                out[(size_t)t * H + h] = (float)acc[h];
        }
        free(xf);
        free(xd);
        free(qd);
        free(row);
        free(a);
        free(y);
        free(acc);
        free(hq);
        free(qc);
        free(qs);
    }
    return 0;
}

int fwref_forward(int T, int H, int E, int k, int F, int qtype, int Fs, int qtype_s,
                  int act_dtype, const void *x, const uint8_t *wg, const uint8_t *wu,
                  const uint8_t *wd, const uint8_t *sg, const uint8_t *su,
                  const uint8_t *sd, const int32_t *ids, const float *w, float *out,
                  int n_threads)
{
    return forward_impl(T, H, E, k, F, qtype, Fs, qtype_s, act_dtype, x, wg, wu, wd, sg, su,
                        sd, ids, w, out, n_threads, AQ_NONE);
}

/* fwref_forward with MXFP8 expert activations: each expert's input is the
 * MXFP8 round trip of the token's fp32 x (blocks of 32 along H) and its down
 * projection's input the MXFP8 round trip of the SwiGLU output rounded to
 * fp32 (blocks of 32 along F); routing and everything else as in
 * fwref_forward.  Only for MXFP4 experts (and an MXFP4 shared expert). */
int fwref_forward_mx8(int T, int H, int E, int k, int F, int qtype, int Fs, int qtype_s,
                      int act_dtype, const void *x, const uint8_t *wg, const uint8_t *wu,
                      const uint8_t *wd, const uint8_t *sg, const uint8_t *su,
                      const uint8_t *sd, const int32_t *ids, const float *w, float *out,
                      int n_threads)
{
    if (qtype != REF_MXFP4 || (Fs > 0 && qtype_s != REF_MXFP4))
        return -1;
    return forward_impl(T, H, E, k, F, qtype, Fs, qtype_s, act_dtype, x, wg, wu, wd, sg, su,
                        sd, ids, w, out, n_threads, AQ_MXFP8);
}

/* fwref_forward with int8 expert activations: each expert's input is the
 * int8 round trip of the token's fp32 x (blocks of 32 along H) and its down
 * projection's input the int8 round trip of the SwiGLU output rounded to fp32
 * (blocks of 32 along F); routing and everything else as in fwref_forward.
 * Only for Q8_0 / Q4_0 experts (and a Q8_0 / Q4_0 shared expert). */
int fwref_forward_q8a(int T, int H, int E, int k, int F, int qtype, int Fs, int qtype_s,
                      int act_dtype, const void *x, const uint8_t *wg, const uint8_t *wu,
                      const uint8_t *wd, const uint8_t *sg, const uint8_t *su,
                      const uint8_t *sd, const int32_t *ids, const float *w, float *out,
                      int n_threads)
{
    if (qtype > REF_Q4_0 || (Fs > 0 && qtype_s > REF_Q4_0))
        return -1;
    return forward_impl(T, H, E, k, F, qtype, Fs, qtype_s, act_dtype, x, wg, wu, wd, sg, su,
                        sd, ids, w, out, n_threads, AQ_Q8A);
}

/* Threads an OpenMP region would use with n_threads (0: default). */
int fwref_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0)
        return n_threads;
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}
