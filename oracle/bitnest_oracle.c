/*
 * CPU oracle for the bit-nested W4/W8 quantized linear.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the HIP library it checks.
 *
 * What it computes, and where each step is defined:
 *
 *  - Weight planes: model card "BitNest-Llama-3-8B", section "Files", entry
 *    planes.safetensors. Each decoder Linear stores two uint8 [N, K/2] planes
 *    `.hi` and `.lo` of unsigned nibbles (u = q + 8). Byte j of a row carries
 *    column 2j in its low nibble and column 2j+1 in its high nibble. One fp16
 *    scale per row and per 128 input columns: `.scale` is fp16 [N, K/128].
 *  - Dequantisation (same entry): the draft weight is (hi - 8) * scale, the
 *    target weight is (16 * (hi - 8) + (lo - 8)) * scale / 16.
 *  - Group size 128: same model card, recipe table, row "Weights".
 *  - Activations: same recipe table, row "Activations": symmetric int8 per
 *    token, and per 128-column group for o_proj. The pages fix neither the
 *    scale formula nor the rounding; the reading used here is
 *        amax = max |x| over the token (or its 128-column group),
 *        s    = amax / 127            (IEEE fp32 division),
 *        q    = 0 if s == 0, else clamp(round_half_even(x / s), -127, 127)
 *    with x / s an IEEE fp32 division. Both sides take this integer decision
 *    in fp32.
 *  - The linear itself is the plain definition: dequantise, then multiply,
 *        y[m, n] = sum_k (q[m, k] * s_a) * W[n, k]
 *    in fp64, k ascending, with s_a the token's (or the token-group's) scale
 *    and W the draft or target weight above.
 *  - The per-group integer partials are the plain definition
 *        P[m, n, g] = sum_{k in group g} q[m, k] * (u[n, k] - 8)
 *    accumulated in int64, with the target's combined partial
 *        P8 = 16 * P_hi + P_lo
 *    (the integer part of the target formula before the scale / 16).
 *
 *  - Online rotation of the down_proj input: same recipe table, row
 *    "Rotation" (an online Hadamard, R4, on the down_proj inputs; the R4
 *    matrices ship in aux.safetensors, entry of section "Files", which is not
 *    available, and the pages do not say how they are built). The reading
 *    used here: R4 is block-diagonal, every block the normalised
 *    Sylvester-Hadamard matrix H_b / sqrt(b) of order b (a power of two
 *    dividing K; 512 for the Llama-3-8B down_proj, K = 14336 = 28 x 512),
 *    applied to each token before its per-token quantisation:
 *        y[m, blk] = (H_b x[m, blk]) * r_b,   r_b = the fp32 value nearest 1/sqrt(b),
 *    with H_b x computed in fp32 by the iterative fast Walsh-Hadamard
 *    transform, stages h = 1, 2, 4, ..., b/2 in that order, each stage
 *    replacing every pair (a, c) = (z[i], z[i + h]) whose index i has bit h
 *    clear by (a + c, a - c), then one fp32 multiply by r_b per element.
 *    Fixing the stage order and the single multiply defines the rotated fp32
 *    values, and therefore their int8 codes, to the bit.
 *  - Offline nested packing of fp32 weights: model card introduction (the
 *    high nibble is a GPTQ-W4 model fitted first, the low nibble the
 *    closed-form residual back to W8) and the planes.safetensors entry (the
 *    format both nibbles must land in). GPTQ itself needs calibration data;
 *    the reading here is its symmetric round-to-nearest quantiser (15 steps,
 *    zero point 8) per (row, 128-column group), with the stored fp16 scale:
 *        amax = max |W| over the group,
 *        s    = fp16(amax / 7.5)   (fp32 division, then round to nearest
 *                                   even in binary16),
 *        c_hi = clamp(rne(W / s), -8, 7),            hi = c_hi + 8,
 *        R    = W - c_hi * s                          (fp32),
 *        c_lo = clamp(rne(R / (s / 16)), -8, 7),     lo = c_lo + 8,
 *    every division an IEEE fp32 division; s == 0 gives c_hi = c_lo = 0.
 *    Then W4 = c_hi * s and W8 = (16 c_hi + c_lo) * s / 16 per the model
 *    card's formulas, and |W8 - W| <= s / 32 wherever neither code clamps.
 *  - Greedy verification of a speculative round: model card introduction
 *    (every draft token is verified with the target, so the output is
 *    exactly the W8A8 target's greedy output). Reading: the target scores
 *    the gamma + 1 verify positions (row r: the position after the prefix
 *    extended by the first r draft tokens); t_r = argmax_v logits[r, v],
 *    ties to the smallest index; the accepted count n is the length of the
 *    longest prefix with draft[r] == t_r; the round emits draft[0 .. n-1]
 *    and then t_n (the target's own token at the first mismatch, or the
 *    bonus token when all gamma drafts are accepted).
 *  - Decode attention over the nested KV cache: recipe table row "KV cache"
 *    (nested at runtime: the draft reads KV4, the target KV8) and the
 *    abstract (the progressive-precision design extends to the KV cache).
 *    The layout, scale granularity and rotation sit in meta.json, which is
 *    not available. Reading: every (token, KV head) K or V vector of 128
 *    values is packed like one 128-column group of a weight row (the packing
 *    above): planes uint8 [T, Hkv, 64], fp16 scale [T, Hkv]; KV4 = (hi - 8)
 *    * s and KV8 = (16 (hi - 8) + (lo - 8)) * s / 16, the weight formulas.
 *    The M query tokens are the last M positions of the sequence (the verify
 *    batch): token i sees positions t <= T - M + i. Query head h reads KV
 *    head h / (Hq / Hkv) (grouped-query attention). Scores q . k / sqrt(128),
 *    softmax over the visible positions, output sum_t p_t v_t, in fp64.
 *
 * Built with -O2 -ffp-contract=off and no fast-math, so every fp32 and fp64
 * operation is the IEEE operation written.
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 128

enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ERANGE = 2 };

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Nibble of column k in a plane row (model card, "Files", planes.safetensors):
 * byte k/2, low nibble for even k, high nibble for odd k. */
static int nibble_at(const uint8_t *plane_row, int k)
{
    uint8_t b = plane_row[k / 2];
    return (k % 2 == 0) ? (b & 0x0F) : (b >> 4);
}

/* Unpack a whole plane [N, K/2] into unsigned nibbles u [N, K]. */
int oracle_unpack_plane(const uint8_t *plane, int N, int K, uint8_t *u)
{
    if (!plane || !u || N < 0 || K < 0 || K % 2) return ORACLE_EINVAL;
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = plane + (size_t)n * (K / 2);
        for (int k = 0; k < K; ++k) u[(size_t)n * K + k] = (uint8_t)nibble_at(row, k);
    }
    return ORACLE_OK;
}

/* Activation quantisation, one token (act_group 0) or one token-group
 * (act_group 128) at a time, following the reading stated at the top. */
int oracle_quant_act(const float *x, int M, int K, int act_group, int8_t *q, float *s)
{
    if (!x || !q || !s || M < 0 || K <= 0) return ORACLE_EINVAL;
    if (act_group != 0 && act_group != ORACLE_GROUP) return ORACLE_EINVAL;
    if (act_group == ORACLE_GROUP && K % ORACLE_GROUP) return ORACLE_EINVAL;
    if (fegetround() != FE_TONEAREST) return ORACLE_EINVAL;
    const int R = act_group ? act_group : K;        /* columns sharing one scale */
    const int S = K / R;                            /* scales per token */
    for (int m = 0; m < M; ++m) {
        for (int r = 0; r < S; ++r) {
            const float *xr = x + (size_t)m * K + (size_t)r * R;
            int8_t *qr = q + (size_t)m * K + (size_t)r * R;
            float amax = 0.0f;
            for (int k = 0; k < R; ++k) {
                float a = fabsf(xr[k]);
                if (a > amax) amax = a;
            }
            float sc = amax / 127.0f;
            s[(size_t)m * S + r] = sc;
            for (int k = 0; k < R; ++k) {
                int code = 0;
                if (sc != 0.0f) {
                    float t = xr[k] / sc;               /* fp32 division */
                    float rt = nearbyintf(t);           /* ties to even */
                    if (rt > 127.0f) rt = 127.0f;
                    if (rt < -127.0f) rt = -127.0f;
                    code = (int)rt;
                }
                qr[k] = (int8_t)code;
            }
        }
    }
    return ORACLE_OK;
}

/* Per-group integer partials of one plane: P[m, n, g] = sum_{k in g} q[m,k] * (u[n,k] - 8). */
static int partials_one_plane(const int8_t *q, const uint8_t *plane, int M, int N, int K,
                              int32_t *P, int nthreads)
{
    const int G = K / ORACLE_GROUP;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(|:bad)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = plane + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            for (int g = 0; g < G; ++g) {
                int64_t acc = 0;
                for (int k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k)
                    acc += (int64_t)q[(size_t)m * K + k] * (int64_t)(nibble_at(row, k) - 8);
                if (acc > INT32_MAX || acc < INT32_MIN) bad = 1;
                P[((size_t)m * N + n) * G + g] = (int32_t)acc;
            }
        }
    }
    return bad ? ORACLE_ERANGE : ORACLE_OK;
}

/* Integer partials, layout int32 [M, N, K/128]. lo, p_lo and p8 may be NULL
 * (draft); if lo is given, p_lo and p8 receive P_lo and 16 * P_hi + P_lo. */
int oracle_partials(const int8_t *q, const uint8_t *hi, const uint8_t *lo,
                    int M, int N, int K, int32_t *p_hi, int32_t *p_lo, int32_t *p8,
                    int nthreads)
{
    if (!q || !hi || !p_hi || M < 0 || N < 0 || K <= 0 || K % ORACLE_GROUP) return ORACLE_EINVAL;
    if (lo && (!p_lo || !p8)) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = 1;
    int rc = partials_one_plane(q, hi, M, N, K, p_hi, nthreads);
    if (rc || !lo) return rc;
    rc = partials_one_plane(q, lo, M, N, K, p_lo, nthreads);
    if (rc) return rc;
    const size_t total = (size_t)M * N * (K / ORACLE_GROUP);
    for (size_t i = 0; i < total; ++i) {
        int64_t v = 16 * (int64_t)p_hi[i] + (int64_t)p_lo[i];
        if (v > INT32_MAX || v < INT32_MIN) return ORACLE_ERANGE;
        p8[i] = (int32_t)v;
    }
    return ORACLE_OK;
}

/* Dequantised weight of one element (model card, "Files", planes.safetensors):
 * mode 0 (draft):  (hi - 8) * scale
 * mode 1 (target): (16 * (hi - 8) + (lo - 8)) * scale / 16 */
static double weight_at(int mode, const uint8_t *hi_row, const uint8_t *lo_row,
                        const uint16_t *scale_row, int k)
{
    double sc = oracle_half_to_double(scale_row[k / ORACLE_GROUP]);
    int h = nibble_at(hi_row, k) - 8;
    if (mode == 0) return (double)h * sc;
    int l = nibble_at(lo_row, k) - 8;
    return (double)(16 * h + l) * sc / 16.0;
}

/* Dense dequantised weight matrix W [N, K] in fp64 (small shapes, tests). */
int oracle_dequant(int mode, const uint8_t *hi, const uint8_t *lo, const uint16_t *scale,
                   int N, int K, double *W)
{
    if (!hi || !scale || !W || N < 0 || K <= 0 || K % ORACLE_GROUP) return ORACLE_EINVAL;
    if (mode != 0 && mode != 1) return ORACLE_EINVAL;
    if (mode == 1 && !lo) return ORACLE_EINVAL;
    const int G = K / ORACLE_GROUP;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            W[(size_t)n * K + k] = weight_at(mode, hi + (size_t)n * (K / 2),
                                             lo ? lo + (size_t)n * (K / 2) : NULL,
                                             scale + (size_t)n * G, k);
    return ORACLE_OK;
}

/* The linear, dequantise-then-multiply in fp64:
 * y64[m, n] = sum_{k ascending} (q[m,k] * s_a[m(,g)]) * W[n,k].
 * s_a is xs[m] (act_group 0) or xs[m * K/128 + k/128] (act_group 128). */
int oracle_linear(int mode, const int8_t *q, const float *xs, int act_group,
                  const uint8_t *hi, const uint8_t *lo, const uint16_t *scale,
                  int M, int N, int K, double *y64, int nthreads)
{
    if (!q || !xs || !hi || !scale || !y64) return ORACLE_EINVAL;
    if (M < 0 || N < 0 || K <= 0 || K % ORACLE_GROUP) return ORACLE_EINVAL;
    if (mode != 0 && mode != 1) return ORACLE_EINVAL;
    if (mode == 1 && !lo) return ORACLE_EINVAL;
    if (act_group != 0 && act_group != ORACLE_GROUP) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = 1;
    const int G = K / ORACLE_GROUP;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int n = 0; n < N; ++n) {
        const uint8_t *hr = hi + (size_t)n * (K / 2);
        const uint8_t *lr = lo ? lo + (size_t)n * (K / 2) : NULL;
        const uint16_t *sr = scale + (size_t)n * G;
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double sa = act_group ? (double)xs[(size_t)m * G + k / ORACLE_GROUP]
                                      : (double)xs[m];
                double xhat = (double)q[(size_t)m * K + k] * sa;
                acc += xhat * weight_at(mode, hr, lr, sr, k);
            }
            y64[(size_t)m * N + n] = acc;
        }
    }
    return ORACLE_OK;
}

/* The R4 rotation reading stated at the top: every token's K columns in
 * blocks of `block` (a power of two, 2 <= block <= K, K % block == 0). */
int oracle_hadamard_rotate(const float *x, int M, int K, int block, float *y)
{
    if (!x || !y || M < 0 || K <= 0 || block < 2 || block > K || K % block) return ORACLE_EINVAL;
    if (block & (block - 1)) return ORACLE_EINVAL;
    if (fegetround() != FE_TONEAREST) return ORACLE_EINVAL;
    const float rb = (float)(1.0 / sqrt((double)block));
    for (int m = 0; m < M; ++m) {
        for (int b0 = 0; b0 < K; b0 += block) {
            float *z = y + (size_t)m * K + b0;
            const float *xr = x + (size_t)m * K + b0;
            for (int i = 0; i < block; ++i) z[i] = xr[i];
            for (int h = 1; h < block; h *= 2) {
                for (int i = 0; i < block; ++i) {
                    if (i & h) continue;
                    float a = z[i], c = z[i + h];
                    z[i] = a + c;
                    z[i + h] = a - c;
                }
            }
            for (int i = 0; i < block; ++i) z[i] = z[i] * rb;
        }
    }
    return ORACLE_OK;
}

/* IEEE binary32 -> binary16, round to nearest even, from the two formats'
 * definitions (finite inputs; overflow gives infinity). */
uint16_t oracle_float_to_half(float f)
{
    union { float f; uint32_t u; } v = { f };
    uint32_t sign = (v.u >> 16) & 0x8000u;
    float a = fabsf(f);
    if (a != a) return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0f) return (uint16_t)(sign | 0x7C00u);        /* rounds past the largest finite */
    if (a < 0x1p-14f) {
        /* subnormal result: a multiple of 2^-24, rounded to nearest even */
        float q = nearbyintf(a * 0x1p24f);                        /* exact scaling, then RNE */
        return (uint16_t)(sign | (uint32_t)q);
    }
    int e;
    float m = frexpf(a, &e);                                      /* a = m * 2^e, 0.5 <= m < 1 */
    /* 11 significant bits: mantissa as an integer in [1024, 2048] after RNE */
    float q = nearbyintf(ldexpf(m, 11));
    if (q == 2048.0f) { q = 1024.0f; e += 1; }
    uint32_t exp16 = (uint32_t)(e - 1 + 15);
    if (exp16 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (exp16 << 10) | ((uint32_t)q - 1024u));
}

static int rne_clamp(float t, int lo, int hi)
{
    float r = nearbyintf(t);
    if (r < (float)lo) r = (float)lo;
    if (r > (float)hi) r = (float)hi;
    return (int)r;
}

/* The packing reading stated at the top: W fp32 [N, K] -> planes hi, lo
 * uint8 [N, K/2] and scale fp16 bits [N, K/128]. */
int oracle_pack_nested(const float *W, int N, int K, uint8_t *hi, uint8_t *lo, uint16_t *scale)
{
    if (!W || !hi || !lo || !scale || N < 0 || K <= 0 || K % ORACLE_GROUP) return ORACLE_EINVAL;
    if (fegetround() != FE_TONEAREST) return ORACLE_EINVAL;
    const int G = K / ORACLE_GROUP;
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            const float *w = W + (size_t)n * K + (size_t)g * ORACLE_GROUP;
            float amax = 0.0f;
            for (int k = 0; k < ORACLE_GROUP; ++k)
                if (fabsf(w[k]) > amax) amax = fabsf(w[k]);
            uint16_t sb = oracle_float_to_half(amax / 7.5f);
            scale[(size_t)n * G + g] = sb;
            float s = (float)oracle_half_to_double(sb);            /* exact */
            float s16th = s / 16.0f;                                /* exact: power of two */
            for (int k = 0; k < ORACLE_GROUP; ++k) {
                int ch = 0, cl = 0;
                if (s != 0.0f) {
                    ch = rne_clamp(w[k] / s, -8, 7);
                    float r = w[k] - (float)ch * s;
                    cl = rne_clamp(r / s16th, -8, 7);
                }
                size_t byte = (size_t)n * (K / 2) + (size_t)(g * ORACLE_GROUP + k) / 2;
                int shift = (k % 2 == 0) ? 0 : 4;                     /* column 2j low nibble, 2j+1 high */
                if (shift == 0) { hi[byte] = 0; lo[byte] = 0; }
                hi[byte] |= (uint8_t)((ch + 8) << shift);
                lo[byte] |= (uint8_t)((cl + 8) << shift);
            }
        }
    }
    return ORACLE_OK;
}

/* Greedy verification, the reading stated at the top. logits fp32 [R, V]
 * (R = gamma + 1), draft int32 [R - 1]; writes targ int32 [R] (t_r), *n_acc
 * and *next (t_n). */
int oracle_greedy_accept(const float *logits, int R, int V, const int32_t *draft,
                         int32_t *targ, int32_t *n_acc, int32_t *next)
{
    if (!logits || !targ || !n_acc || !next || R < 1 || V < 1 || (R > 1 && !draft)) return ORACLE_EINVAL;
    for (int r = 0; r < R; ++r) {
        const float *row = logits + (size_t)r * V;
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (row[v] > row[best]) best = v;          /* strict: the first maximum wins */
        targ[r] = best;
    }
    int n = 0;
    while (n < R - 1 && draft[n] == targ[n]) ++n;
    *n_acc = n;
    *next = targ[n];
    return ORACLE_OK;
}

#define ORACLE_HEAD_DIM 128

/* One KV value (token t, KV head h, dimension j) of a nested cache:
 * hi / lo planes [T, Hkv, 64], scale [T, Hkv]; lo == NULL reads KV4. */
static double kv_value(const uint8_t *hi, const uint8_t *lo, const uint16_t *scale, int Hkv,
                       int t, int h, int j)
{
    const size_t row = (size_t)t * Hkv + h;
    const uint8_t *hr = hi + row * (ORACLE_HEAD_DIM / 2);
    double s = oracle_half_to_double(scale[row]);
    int ch = nibble_at(hr, j) - 8;
    if (!lo) return (double)ch * s;
    int cl = nibble_at(lo + row * (ORACLE_HEAD_DIM / 2), j) - 8;
    return (double)(16 * ch + cl) * s / 16.0;
}

/* The attention reading stated at the top. q fp32 [M, Hq, 128]; out fp64
 * [M, Hq, 128]. k_lo and v_lo both NULL (KV4) or both given (KV8). */
int oracle_kv_attention(const float *q, int M, int Hq, int Hkv, int T,
                        const uint8_t *k_hi, const uint8_t *k_lo, const uint16_t *k_scale,
                        const uint8_t *v_hi, const uint8_t *v_lo, const uint16_t *v_scale,
                        double *out, int nthreads)
{
    if (!q || !k_hi || !k_scale || !v_hi || !v_scale || !out) return ORACLE_EINVAL;
    if (M < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || T < M) return ORACLE_EINVAL;
    if ((k_lo == NULL) != (v_lo == NULL)) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = 1;
    const int G = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)ORACLE_HEAD_DIM);
#pragma omp parallel for schedule(static) num_threads(nthreads) collapse(2)
    for (int i = 0; i < M; ++i) {
        for (int h = 0; h < Hq; ++h) {
            const int hk = h / G;
            const int visible = T - M + i + 1;          /* positions 0 .. T - M + i */
            const float *qv = q + ((size_t)i * Hq + h) * ORACLE_HEAD_DIM;
            double *o = out + ((size_t)i * Hq + h) * ORACLE_HEAD_DIM;
            double mx = -INFINITY;
            for (int t = 0; t < visible; ++t) {
                double sc = 0.0;
                for (int j = 0; j < ORACLE_HEAD_DIM; ++j)
                    sc += (double)qv[j] * kv_value(k_hi, k_lo, k_scale, Hkv, t, hk, j);
                sc *= inv_sqrt_d;
                if (sc > mx) mx = sc;
            }
            double den = 0.0;
            for (int j = 0; j < ORACLE_HEAD_DIM; ++j) o[j] = 0.0;
            for (int t = 0; t < visible; ++t) {
                double sc = 0.0;
                for (int j = 0; j < ORACLE_HEAD_DIM; ++j)
                    sc += (double)qv[j] * kv_value(k_hi, k_lo, k_scale, Hkv, t, hk, j);
                double p = exp(sc * inv_sqrt_d - mx);
                den += p;
                for (int j = 0; j < ORACLE_HEAD_DIM; ++j)
                    o[j] += p * kv_value(v_hi, v_lo, v_scale, Hkv, t, hk, j);
            }
            for (int j = 0; j < ORACLE_HEAD_DIM; ++j) o[j] /= den;
        }
    }
    return ORACLE_OK;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
