/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of the fused activation-quantisation
 * step of an MoE expert: SwiGLU on a packed [gate | up] bf16 row, optional
 * clamp with a clamp counter, scaling by the token's top-k routing weight,
 * an abs-max per token or per column group, and the cast to FP8 E4M3 or
 * FP4 E2M1 codes with an fp32 or UE8M0 (power-of-two) scale; the same cast
 * on its own; the deterministic top-k gating that produces the routing
 * weights; the map from each token's top-k slots to its expert rows; and the
 * weighted top-k reduce of the experts' output rows.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The GPU library never calls it, and the two share no
 * code, headers, tables or constants.
 *
 * Sources (pages on DeepSeek's TileKernels library):
 *  [Tutorial]  "【DeepSeek】TileKernels从入门到精通" (zhichai.net/topic/177618752)
 *              ch.2 "解剖麻雀（SwiGLU与Quant的单次Kernel融合）": sections
 *              "内存的“连体双胞胎”：布局的艺术" (packed gate|up row),
 *              "算子融合的“三重境界”" (sigmoid(x_L)*x_L, then * x_R, then the
 *              top-k weight, then abs-max -> scale factor -> FP8), and
 *              "守门员 Clamp" (clamp of the left value and its counter);
 *              ch.5 "越过性能红线" (the unfused reference: swiglu_forward then
 *              cast).
 *  [Summary]   "TileKernels from Beginner to Master: DeepSeek's
 *              TileLang-Powered GPU Kernel Guide" (zhichai.net/en/topic/
 *              177618752), "Chapter 2: Anatomy of SwiGLU + Quant
 *              Single-Kernel Fusion".
 *  [Overview]  "TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式"
 *              (zhichai.net/topic/177618740), "3. Quantization" table
 *              (FP8 E4M3 per-token/per-block, FP4 E2M1, UE8M0 scales) and
 *              the per-block vs per-token note under it.
 *  [Essay]     "TileLang在DeepSeek-V4中的工业实战" (yunpan.plus/t/24864-1-1),
 *              third point on precision and bitwise alignment (no fast-math,
 *              IEEE operations, FMA fusion changes bits).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - sigma(g) is the correctly rounded fp32 value of 1/(1+e^-g); it is
 *    evaluated here in binary128 and rounded once to fp32.
 *  - a = RN(g*sigma), b = RN(a*u), y = RN(b*w): three fp32 products in the
 *    order the Tutorial lists them, no fused multiply-add, y kept in fp32.
 *  - clamp: gate g <- min(g, L) (counted when g > L), up u <- clamp(u,-L,L).
 *  - fp32 scale s = RN(amax/fmt_max); codes from q = RN(y * inv) with
 *    inv = min(RN(fmt_max/amax), FLT_MAX).
 *  - UE8M0: smallest k with fmt_max*2^k >= amax (clamped to [-127,127]),
 *    stored as the byte k+127; inv = 2^-k.
 *  - casts round to nearest, ties to even, saturate at +-fmt_max and keep
 *    the sign of zero; FP4 element 2i goes to the low nibble of byte i.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared oracle.c -lquadmath -lm
 * (no -ffast-math, no FMA contraction: every fp32 operation is one IEEE
 * operation rounded to nearest-even).
 */
#include <float.h>
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FP8 8
#define ORACLE_FP4 4
#define ORACLE_SCALE_FP32 0
#define ORACLE_SCALE_UE8M0 1

/* bf16 is the upper half of an fp32: widening is exact. */
static float bf16_to_float(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* sigma(g) = 1 / (1 + e^-g), correctly rounded to fp32.
 * Binary128 keeps about 112 bits, far more than the closest approach of any
 * bf16 gate's sigmoid to an fp32 rounding midpoint, so the single final
 * rounding is the correct one. */
float oracle_sigmoid(float g)
{
    __float128 e = expq(-(__float128)g);
    __float128 s = 1 / (1 + e);
    return (float)s;
}

/* FP8 E4M3 (OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF are NaN and
 * never produced).  Normal codes: 2^(e-7) * (1 + m/8), e in 1..15;
 * subnormals: 2^-6 * m/8.  Largest finite value 448.
 * Round to nearest, ties to the even code, saturate, keep the sign. */
uint8_t oracle_e4m3(float q)
{
    uint8_t sign = signbit(q) ? 0x80 : 0x00;
    double a = fabs((double)q);
    int code;
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < 0x1p-6) {
        /* subnormal range, step 2^-9; n == 8 is the smallest normal */
        code = (int)nearbyint(a * 0x1p9);
    } else {
        int e;
        frexp(a, &e);
        e -= 1; /* a = 1.f * 2^e, e in [-6, 8] */
        /* a / 2^(e-3) lies in [8, 16); 16 carries into the next binade */
        code = ((e + 7) << 3) + (int)nearbyint(ldexp(a, 3 - e)) - 8;
    }
    if (code > 0x7E)
        code = 0x7E;
    return sign | (uint8_t)code;
}

/* FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Normal codes:
 * 2^(e-1) * (1 + m/2), e in 1..3; subnormal: 0.5 * m.
 * Round to nearest, ties to the even code, saturate, keep the sign. */
uint8_t oracle_e2m1(float q)
{
    uint8_t sign = signbit(q) ? 0x8 : 0x0;
    double a = fabs((double)q);
    int code;
    if (a >= 6.0)
        return sign | 0x7;
    if (a < 1.0) {
        code = (int)nearbyint(a * 2.0); /* step 0.5; 2 is the value 1.0 */
    } else {
        int e;
        frexp(a, &e);
        e -= 1; /* e in {0, 1, 2} */
        code = ((e + 1) << 1) + (int)nearbyint(ldexp(a, 1 - e)) - 2;
    }
    if (code > 7)
        code = 7;
    return sign | (uint8_t)code;
}

/* UE8M0: the smallest k in [-127, 127] with fmt_max * 2^k >= amax, found by
 * counting up with exact double comparisons; returns k. */
int oracle_ue8m0_exponent(float amax, float fmt_max)
{
    int k = -127;
    while (k < 127 && ldexp((double)fmt_max, k) < (double)amax)
        ++k;
    return k;
}

static float fmt_max_of(int fmt) { return fmt == ORACLE_FP8 ? 448.0f : 6.0f; }

/* The per-group tail: amax -> scale (+ inverse) -> codes.
 * y[0..len) are one group's fp32 values; codes are written as one byte per
 * element (the caller packs FP4 nibbles). */
static void quantize_group(const float* y, int64_t len, int fmt, int scale_fmt,
                           uint8_t* code_out, float* scale_f32, uint8_t* scale_u8)
{
    const float fmt_max = fmt_max_of(fmt);
    float amax = 0.0f;
    for (int64_t j = 0; j < len; ++j) {
        float m = fabsf(y[j]);
        if (m > amax)
            amax = m;
    }
    float inv;
    if (scale_fmt == ORACLE_SCALE_FP32) {
        *scale_f32 = amax / fmt_max;
        inv = fmt_max / amax; /* +inf when amax == 0 */
        if (inv > FLT_MAX)
            inv = FLT_MAX;
    } else {
        int k = oracle_ue8m0_exponent(amax, fmt_max);
        *scale_u8 = (uint8_t)(k + 127);
        inv = ldexpf(1.0f, -k);
    }
    for (int64_t j = 0; j < len; ++j) {
        float q = y[j] * inv;
        code_out[j] = fmt == ORACLE_FP8 ? oracle_e4m3(q) : oracle_e2m1(q);
    }
}

static int check_args(int64_t n, int64_t hidden, int64_t group_size, int fmt, int scale_fmt)
{
    if (n < 0 || hidden <= 0 || group_size < 0)
        return 1;
    if (group_size != 0 && hidden % group_size != 0)
        return 1;
    if (fmt != ORACLE_FP8 && fmt != ORACLE_FP4)
        return 1;
    if (fmt == ORACLE_FP4 && hidden % 2 != 0)
        return 1;
    if (scale_fmt != ORACLE_SCALE_FP32 && scale_fmt != ORACLE_SCALE_UE8M0)
        return 1;
    return 0;
}

/* Stage 1 of the unfused reference (Tutorial ch.5 "越过性能红线"):
 * y[r, j] = RN(RN(RN(g*sigma(g)) * u) * w[r]) with g = x[r, j],
 * u = x[r, hidden + j] (Tutorial ch.2 layout section), after the optional
 * clamp (Tutorial ch.2 "守门员 Clamp").  clamp_limit = +inf means no clamp.
 * w == NULL means no weight.  *clamped_count (if given) is increased by the
 * number of gate values strictly above the limit. */
int oracle_swiglu_forward(const uint16_t* x, const float* w, int64_t n, int64_t hidden,
                          float clamp_limit, float* y, int64_t* clamped_count)
{
    if (n < 0 || hidden <= 0)
        return 1;
    int64_t count = 0;
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t* row = x + r * 2 * hidden;
        const float wr = w ? w[r] : 1.0f;
        for (int64_t j = 0; j < hidden; ++j) {
            float g = bf16_to_float(row[j]);
            float u = bf16_to_float(row[hidden + j]);
            if (g > clamp_limit) {
                g = clamp_limit;
                ++count;
            }
            if (u > clamp_limit)
                u = clamp_limit;
            if (u < -clamp_limit)
                u = -clamp_limit;
            float sig = oracle_sigmoid(g);
            float a = g * sig;
            float b = a * u;
            float yv = w ? b * wr : b;
            y[r * hidden + j] = yv;
        }
    }
    if (clamped_count)
        *clamped_count += count;
    return 0;
}

/* Stage 2 of the unfused reference: cast fp32 rows y[n, hidden] to codes and
 * scales.  group_size 0 means one group per row (per-token).  FP8 codes are
 * [n, hidden] bytes; FP4 codes are [n, hidden/2] bytes with element 2i in the
 * low nibble.  Scales are [n, hidden/G] (fp32 or UE8M0 bytes), row-major. */
int oracle_cast(const float* y, int64_t n, int64_t hidden, int64_t group_size, int fmt,
                int scale_fmt, uint8_t* codes, void* scales)
{
    if (check_args(n, hidden, group_size, fmt, scale_fmt))
        return 1;
    const int64_t G = group_size ? group_size : hidden;
    const int64_t groups = hidden / G;
    uint8_t* tmp = (uint8_t*)malloc((size_t)hidden);
    if (!tmp)
        return 2;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t k = 0; k < groups; ++k) {
            float* sf = (float*)scales + r * groups + k;
            uint8_t* su = (uint8_t*)scales + r * groups + k;
            quantize_group(y + r * hidden + k * G, G, fmt, scale_fmt, tmp + k * G, sf, su);
        }
        if (fmt == ORACLE_FP8) {
            memcpy(codes + r * hidden, tmp, (size_t)hidden);
        } else {
            for (int64_t i = 0; i < hidden / 2; ++i)
                codes[r * (hidden / 2) + i] = (uint8_t)(tmp[2 * i] | (tmp[2 * i + 1] << 4));
        }
    }
    free(tmp);
    return 0;
}

/* UE8M0 exponent from the binary exponents and significands of amax and
 * fmt_max (a closed form, independent of oracle_ue8m0_exponent's search):
 * with amax = ma*2^ea and fmt_max = mf*2^ef, ma and mf in [0.5, 1), the
 * smallest k with fmt_max*2^k >= amax is ea - ef, plus 1 when ma > mf;
 * clamped to [-127, 127]; amax == 0 gives -127. */
static int ue8m0_exponent_closed_form(float amax, float fmt_max)
{
    if (amax == 0.0f)
        return -127;
    int ea, ef;
    const double ma = frexp((double)amax, &ea);
    const double mf = frexp((double)fmt_max, &ef);
    int k = ea - ef + (ma > mf ? 1 : 0);
    if (k < -127)
        k = -127;
    if (k > 127)
        k = 127;
    return k;
}

/* The fused form (Tutorial ch.2 "算子融合的“三重境界”"; Summary ch.2): one row
 * at a time and, within it, one column group at a time.  Each value of the
 * group goes from the bf16 pair through the clamp, sigma and the three
 * products into a buffer of one group, its magnitude into the running
 * abs-max; then the group's scale, then its codes, written straight into the
 * output row (FP4: element 2i into the low nibble of byte i, 2i+1 into the
 * high nibble).  It calls neither stage function of the unfused form, so the
 * two agree only if both follow the same statement of the step. */
int oracle_swiglu_cast(const uint16_t* x, const float* w, int64_t n, int64_t hidden,
                       int64_t group_size, float clamp_limit, int fmt, int scale_fmt,
                       uint8_t* codes, void* scales, int64_t* clamped_count)
{
    if (check_args(n, hidden, group_size, fmt, scale_fmt))
        return 1;
    const int64_t G = group_size ? group_size : hidden;
    const int64_t groups = hidden / G;
    const float fmt_max = fmt == ORACLE_FP8 ? 448.0f : 6.0f;
    float* vals = (float*)malloc((size_t)G * sizeof(float));
    if (!vals)
        return 2;
    int64_t clamped = 0;
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t* gate_row = x + r * 2 * hidden;
        const uint16_t* up_row = gate_row + hidden;
        uint8_t* out_row = codes + (fmt == ORACLE_FP8 ? r * hidden : r * (hidden / 2));
        for (int64_t k = 0; k < groups; ++k) {
            float group_amax = 0.0f;
            for (int64_t j = 0; j < G; ++j) {
                const int64_t col = k * G + j;
                float gv = bf16_to_float(gate_row[col]);
                float uv = bf16_to_float(up_row[col]);
                if (clamp_limit < INFINITY) {
                    if (gv > clamp_limit) {
                        ++clamped;
                        gv = clamp_limit;
                    }
                    if (uv < -clamp_limit)
                        uv = -clamp_limit;
                    else if (uv > clamp_limit)
                        uv = clamp_limit;
                }
                const float act = gv * oracle_sigmoid(gv);
                const float prod = act * uv;
                const float v = w != NULL ? prod * w[r] : prod;
                vals[j] = v;
                const float mag = v < 0.0f ? -v : v;
                if (mag > group_amax)
                    group_amax = mag;
            }
            float mult;
            if (scale_fmt == ORACLE_SCALE_FP32) {
                ((float*)scales)[r * groups + k] = group_amax / fmt_max;
                mult = group_amax > 0.0f ? fmt_max / group_amax : FLT_MAX;
                if (mult > FLT_MAX)
                    mult = FLT_MAX;
            } else {
                const int e = ue8m0_exponent_closed_form(group_amax, fmt_max);
                ((uint8_t*)scales)[r * groups + k] = (uint8_t)(e + 127);
                mult = ldexpf(1.0f, -e);
            }
            for (int64_t j = 0; j < G; ++j) {
                const int64_t col = k * G + j;
                const float q = vals[j] * mult;
                if (fmt == ORACLE_FP8) {
                    out_row[col] = oracle_e4m3(q);
                } else if (col % 2 == 0) {
                    out_row[col / 2] = oracle_e2m1(q);
                } else {
                    out_row[col / 2] = (uint8_t)(out_row[col / 2] | (oracle_e2m1(q) << 4));
                }
            }
        }
    }
    free(vals);
    if (clamped_count)
        *clamped_count += clamped;
    return 0;
}

/* Element-wise cast of fp32 values to codes (one byte per value), for codec
 * sweeps: fmt 8 -> oracle_e4m3, fmt 4 -> oracle_e2m1. */
int oracle_encode(int fmt, const float* q, int64_t n, uint8_t* out)
{
    if (fmt != ORACLE_FP8 && fmt != ORACLE_FP4)
        return 1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = fmt == ORACLE_FP8 ? oracle_e4m3(q[i]) : oracle_e2m1(q[i]);
    return 0;
}

/* The stand-alone cast of bf16 rows ("per_token_cast" in Tutorial ch.1
 * "透视底层" / "闭环": bf16 in, FP8/FP4 codes and scales out, the same abs-max ->
 * scale -> cast tail as the fused step).  Each bf16 value is widened exactly to
 * fp32, then oracle_cast applies. */
int oracle_cast_bf16(const uint16_t* x, int64_t n, int64_t hidden, int64_t group_size, int fmt,
                     int scale_fmt, uint8_t* codes, void* scales)
{
    if (n < 0 || hidden <= 0)
        return 1;
    float* row = (float*)malloc((size_t)hidden * sizeof(float));
    if (!row)
        return 2;
    const int64_t groups = hidden / (group_size ? group_size : hidden);
    const int64_t code_bytes = fmt == ORACLE_FP8 ? hidden : hidden / 2;
    const size_t scale_bytes = scale_fmt == ORACLE_SCALE_FP32 ? sizeof(float) : 1;
    int rc = 0;
    for (int64_t r = 0; r < n && rc == 0; ++r) {
        for (int64_t j = 0; j < hidden; ++j)
            row[j] = bf16_to_float(x[r * hidden + j]);
        rc = oracle_cast(row, 1, hidden, group_size, fmt, scale_fmt, codes + r * code_bytes,
                         (uint8_t*)scales + (size_t)(r * groups) * scale_bytes);
    }
    free(row);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Top-k expert gating ("TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式"
 * "1. Gating": pick each token's top-k experts from [num_tokens, num_experts]
 * scores, equal scores going to the smaller index; "【DeepSeek】TileKernels从入门
 * 到精通" ch.3 "导诊台的“工号制度”": take the best, label it, take the next; the
 * group step compares the sums of each group's two best scores, equal sums
 * going to the smaller group index).
 *
 * Readings: "a beats b" means score_a > score_b, or score_a == score_b (as
 * numbers, so -0 == +0) and a < b.  With n_group > 1 the experts form n_group
 * consecutive groups; a group's score is RN(best + second best) of its members,
 * and a score that is NaN (best +inf, second best -inf) counts as -inf, so that
 * groups are totally ordered (the pages do not say how such a group ranks);
 * the topk_group best groups (same tie rule on group index) are kept and the k
 * experts are chosen among their members only.  Output order: best first.
 * Weights are the chosen scores, or, when normalise is set, each chosen score
 * divided by the fp32 sum of the chosen scores added best first (a zero sum
 * leaves the chosen scores as they are).
 * ------------------------------------------------------------------------- */
static int beats(float sa, int64_t a, float sb, int64_t b) { return sa > sb || (sa == sb && a < b); }

int oracle_topk_gate(const float* scores, int64_t tokens, int64_t experts, int64_t k, int64_t n_group,
                     int64_t topk_group, int normalise, int32_t* idx_out, float* w_out)
{
    if (tokens < 0 || experts <= 0 || k <= 0 || n_group <= 0 || experts % n_group != 0)
        return 1;
    const int64_t per = experts / n_group;
    if (topk_group <= 0 || topk_group > n_group || k > topk_group * per || (n_group > 1 && per < 2))
        return 1;
    unsigned char* allowed = (unsigned char*)malloc((size_t)experts);
    unsigned char* taken = (unsigned char*)malloc((size_t)(experts > n_group ? experts : n_group));
    float* gscore = (float*)malloc((size_t)n_group * sizeof(float));
    if (!allowed || !taken || !gscore) {
        free(allowed); free(taken); free(gscore);
        return 2;
    }
    for (int64_t t = 0; t < tokens; ++t) {
        const float* s = scores + t * experts;
        /* groups: best two members' sum, then the topk_group best groups */
        if (n_group > 1) {
            for (int64_t g = 0; g < n_group; ++g) {
                int64_t b1 = -1, b2 = -1;
                for (int64_t e = g * per; e < (g + 1) * per; ++e) {
                    if (b1 < 0 || beats(s[e], e, s[b1], b1)) {
                        b2 = b1;
                        b1 = e;
                    } else if (b2 < 0 || beats(s[e], e, s[b2], b2)) {
                        b2 = e;
                    }
                }
                gscore[g] = s[b1] + s[b2];
                if (gscore[g] != gscore[g]) /* +inf + -inf: ranks as -inf */
                    gscore[g] = -INFINITY;
            }
            memset(taken, 0, (size_t)n_group);
            memset(allowed, 0, (size_t)experts);
            for (int64_t j = 0; j < topk_group; ++j) {
                int64_t best = -1;
                for (int64_t g = 0; g < n_group; ++g)
                    if (!taken[g] && (best < 0 || beats(gscore[g], g, gscore[best], best)))
                        best = g;
                taken[best] = 1;
                memset(allowed + best * per, 1, (size_t)per);
            }
        } else {
            memset(allowed, 1, (size_t)experts);
        }
        /* experts: the best allowed one, k times */
        memset(taken, 0, (size_t)experts);
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < experts; ++e)
                if (allowed[e] && !taken[e] && (best < 0 || beats(s[e], e, s[best], best)))
                    best = e;
            taken[best] = 1;
            idx_out[t * k + j] = (int32_t)best;
            w_out[t * k + j] = s[best];
        }
        if (normalise) {
            float sum = 0.0f;
            for (int64_t j = 0; j < k; ++j)
                sum += w_out[t * k + j];
            if (sum != 0.0f)
                for (int64_t j = 0; j < k; ++j)
                    w_out[t * k + j] = w_out[t * k + j] / sum;
        }
    }
    free(allowed);
    free(taken);
    free(gscore);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Fused MoE reduce ("【DeepSeek】TileKernels从入门到精通" ch.3 "结算中心的“减法
 * 工程”": each token's top-k expert outputs are weighted and summed in one pass,
 * the routing weights, the quantisation scale factors and a global scale
 * applied on the way; "动态寻址": a token/top-k -> position map says where each
 * expert output row lies).
 *
 * Readings: x holds the experts' output rows (bf16 [n_rows, hidden]); pos[t,j]
 * is the row of token t's j-th expert output; an entry outside [0, n_rows)
 * (negative: a dropped slot) contributes nothing.  row_scale (nullable) is a
 * per-row dequantisation factor.  Per token t and column c, over the present
 * slots in order j = 0..k-1:
 *   f = RN(w[t,j] * row_scale[p]) (or w[t,j]),  acc = RN(acc + RN(f * x[p,c]))
 * from acc = +0; out = RN(acc * global_scale), then rounded to the nearest
 * bf16 (ties to even) when out_bf16 is set, else kept as fp32.
 * ------------------------------------------------------------------------- */

/* nearest bf16 to a finite fp32 value, ties to the even code; a value at or
   past the midpoint between the largest bf16 and 2^128 becomes infinity */
static uint16_t float_to_bf16_rne(float v)
{
    uint32_t b;
    memcpy(&b, &v, 4);
    const uint32_t lo_b = b & 0xFFFF0000u; /* v truncated toward zero */
    float lo;
    memcpy(&lo, &lo_b, 4);
    /* the next bf16 away from zero, as an exact double (2^128 past the top) */
    const double ulp = ldexp(1.0, ((int)((lo_b >> 23) & 0xFFu) > 0 ? (int)((lo_b >> 23) & 0xFFu) - 127 - 7 : -126 - 7));
    const double dlo = fabs((double)v - (double)lo);
    const double dhi = ulp - dlo;
    int up;
    if (dlo < dhi)
        up = 0;
    else if (dhi < dlo)
        up = 1;
    else
        up = (int)((lo_b >> 16) & 1u); /* tie: go to the even code */
    return (uint16_t)((lo_b >> 16) + (uint32_t)up);
}

int oracle_moe_reduce(const uint16_t* x, const float* row_scale, const int32_t* pos, const float* w,
                      float global_scale, int64_t tokens, int64_t k, int64_t hidden, int64_t n_rows,
                      int out_bf16, void* out)
{
    if (tokens < 0 || k <= 0 || hidden <= 0 || n_rows < 0)
        return 1;
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t c = 0; c < hidden; ++c) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; ++j) {
                const int64_t p = pos[t * k + j];
                if (p < 0 || p >= n_rows)
                    continue;
                const float f = row_scale ? w[t * k + j] * row_scale[p] : w[t * k + j];
                const float term = f * bf16_to_float(x[p * hidden + c]);
                acc = acc + term;
            }
            const float o = acc * global_scale;
            if (out_bf16)
                ((uint16_t*)out)[t * hidden + c] = float_to_bf16_rne(o);
            else
                ((float*)out)[t * hidden + c] = o;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * The token/top-k -> position map of "【DeepSeek】TileKernels从入门到精通" ch.3,
 * section "动态寻址": the table that tells the reduce where each token's j-th
 * expert output sits.  The pages do not fix the layout of the expanded rows;
 * the reading here is the plainest one a grouped expert GEMM consumes: the
 * rows of expert 0 first, then expert 1, ..., and within an expert in token
 * order.
 *   Slot (t, j) is present when 0 <= e = idx[t,j] < experts and no earlier
 *   slot of the same token names e; other slots get pos = -1.
 *   offsets[e] = number of present slots naming an expert below e
 *   (offsets[experts] = all present slots);
 *   pos[t,j] = offsets[e] + number of tokens t' < t with a present slot
 *   naming e.
 * ------------------------------------------------------------------------- */
int oracle_topk_to_pos(const int32_t* idx, int64_t tokens, int64_t k, int64_t experts, int32_t* pos,
                       int32_t* offsets)
{
    if (tokens < 0 || k <= 0 || experts <= 0)
        return 1;
    int64_t* count = (int64_t*)calloc((size_t)experts, sizeof(int64_t));
    if (!count)
        return 2;
    /* which slots are present: a valid expert not named earlier in its token */
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            const int32_t e = idx[t * k + j];
            int present = e >= 0 && e < experts;
            for (int64_t i = 0; present && i < j; ++i)
                if (idx[t * k + i] == e)
                    present = 0;
            pos[t * k + j] = present ? 0 : -1;
            if (present)
                count[e] += 1;
        }
    }
    /* expert e's rows start after every row of the experts below it */
    int64_t run = 0;
    for (int64_t e = 0; e < experts; ++e) {
        offsets[e] = (int32_t)run;
        run += count[e];
    }
    offsets[experts] = (int32_t)run;
    /* then the tokens in order: each takes the next row of each of its experts */
    for (int64_t e = 0; e < experts; ++e)
        count[e] = 0;
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            if (pos[t * k + j] < 0)
                continue;
            const int32_t e = idx[t * k + j];
            pos[t * k + j] = (int32_t)(offsets[e] + count[e]);
            count[e] += 1;
        }
    }
    free(count);
    return 0;
}
