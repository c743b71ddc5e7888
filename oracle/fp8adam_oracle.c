/*
 * fp8adam_oracle.c -- slow, scalar CPU oracle for the FP8-moment Adam/AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * cpu_baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the GPU library and never calls it.
 *
 * What it computes, and where that is stated:
 *
 *  [P1] "daoxuan.cc explainer of arXiv 2409.12517" (blog.daoxuan.cc/posts/32114),
 *       section "Why Adam stores the first moment in E4M3 and the second in E5M2":
 *         - "The two FP8 formats" table: E4M3 = 4 exponent / 3 mantissa bits,
 *           E5M2 = 5 exponent / 2 mantissa bits;
 *         - "Adam's update makes the needs asymmetric": m is a moving average of
 *           the gradient that enters the update linearly (numerator, times the
 *           learning rate); v is a moving average of the squared gradient that
 *           enters under a square root in the denominator;
 *         - "A numerical example": the E4M3 smallest normal is 2^-6, and the
 *           epsilon is added after the square root (sqrt(0) = 0 gives 1/(0+eps)).
 *  [P2] "Scaling FP8 training to trillion-token LLMs" (shd-paper.top summary of
 *       arXiv 2409.12517v2), "Method details" and abstract: both Adam moments
 *       are quantized to FP8; the quantization method itself is not given.
 *  [P3] "FP8 training stability: mixed E5M2/E4M3 precision" (zyxy.net/?p=24419):
 *         - "FP8 formats": sign/exponent/mantissa bit splits;
 *         - "Mixed-precision strategy": master weights kept in FP32/FP16;
 *         - "Strategies": dynamic range set by tracking the max-abs value and
 *           adjusting the exponent offset (read here as a power-of-two scale);
 *           round-to-nearest is the standard rounding;
 *         - "Code example": the optimizer is AdamW (decoupled weight decay).
 *
 * Readings where the pages are silent:
 *  - Formats are the OCP ones: E4M3FN (bias 7, max 448, no infinities, NaN =
 *    S.1111.111) and E5M2 (bias 15, max 57344, IEEE infinities and NaNs).
 *    Subnormals are kept.  Encoding rounds to nearest, ties to even, and
 *    saturates magnitudes above the format maximum (including infinities) to
 *    the maximum.  NaN input encodes to S.1111111 (outside the contract).
 *  - real value = scale * fp8 value; quantization multiplies by inv_scale.
 *  - POW2 scale (default): the smallest power of two s with amax/s <= FMAX,
 *    exponent clamped to [-126, 126]; amax = 0 or non-finite gives s = 1.
 *    AMAX scale (alternative): s = amax/FMAX, inv_s = FMAX/amax, both fp32;
 *    s below the smallest fp32 normal is raised to it (inv_s = 2^126).
 *  - The scale is chosen just-in-time from the new moments of this step, over
 *    the whole tensor or over each run of `block` consecutive elements.
 *  - The moment update is evaluated in fp32, the precision in which the GPU
 *    takes the quantization decision:  m' = fma(b1, m, (1-b1)*g),
 *    v' = fma(b2, v, (1-b2)*(g*g)).
 *  - Bias correction 1 - beta^t with the caller's 1-based t; weight decay is
 *    decoupled (AdamW) and applied to the old p; p is updated from the fresh
 *    (unquantized) m', v'.
 *  - Delayed scaling (history_len > 0, per-tensor scales): the scale of step t
 *    comes from the largest amax recorded over the previous H steps (times
 *    2^margin) instead of this step's amax; values beyond the format maximum
 *    saturate.  [P3 "Strategies" (track the max-abs value) and the code
 *    example's delayed-scaling recipe: history of 16, margin 0, interval 1,
 *    MAX of the history.]  Steps t < delayed_from are just in time, so the
 *    first step has a history to start from.
 *  - Stochastic rounding (stochastic = 1): each moment code rounds up or down
 *    with probability given by the distance to its two FP8 neighbours, using
 *    16 bits of a Philox4x32-10 word per element and moment (ref_encode_sr).
 *  - Coupled-L2 variant (l2_coupled): the L2 term of an L2-regularised loss
 *    enters the gradient instead, g_eff = fma(wd, p, g) in fp32 with the old
 *    p, and there is no decoupled decay.  [P1] "Why the SwiGLU weights align",
 *    Theorem 1 set-up: the training objective (Eq. 1) is the loss plus an L2
 *    penalty on the weights.  The parameter update is evaluated in fp64 and
 *    rounded once to the master dtype (fp32, or bf16 round-to-nearest-even).
 *
 * Build: plain C11, no SIMD intrinsics, -ffp-contract=off.
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <math.h>
#include <fenv.h>

/* ------------------------------------------------------------------ formats */

/* [P1 "The two FP8 formats"; P3 "FP8 formats"]: bit splits.  Bias, maximum
 * code and NaN/Inf encodings are the OCP FP8 definitions. */
typedef struct {
    int ebits;        /* exponent bits */
    int mbits;        /* mantissa bits */
    int bias;         /* exponent bias */
    uint8_t max_code; /* largest finite magnitude code */
    int has_inf;      /* 1: IEEE-style Inf/NaN in the top exponent; 0: E4M3FN */
} ref_format;

static const ref_format REF_FORMATS[2] = {
    {4, 3, 7, 0x7E, 0},  /* 0: E4M3 (OCP E4M3FN), max 448   */
    {5, 2, 15, 0x7B, 1}, /* 1: E5M2 (OCP E5M2),   max 57344 */
};

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* Decode one FP8 code to fp32, exactly, by assembling the fp32 bit fields. */
float ref_decode(int fmt, uint8_t code)
{
    const ref_format *F = &REF_FORMATS[fmt];
    uint32_t sign = (uint32_t)(code >> 7) << 31;
    uint32_t emax = (1u << F->ebits) - 1;
    uint32_t e = (code >> F->mbits) & emax;
    uint32_t m = code & ((1u << F->mbits) - 1);

    if (F->has_inf) {
        if (e == emax) return u2f(sign | (m == 0 ? 0x7F800000u : 0x7FC00000u));
    } else {
        if (e == emax && m == (1u << F->mbits) - 1) return u2f(sign | 0x7FC00000u);
    }
    if (e == 0) {
        if (m == 0) return u2f(sign); /* signed zero */
        /* subnormal: m * 2^(1 - bias - mbits); normalise so the leading 1 of m
         * becomes the implicit bit of the fp32 result */
        int len = 0;
        while ((m >> len) != 0) len++;           /* bit length of m, 1..mbits */
        int exp = (len - 1) + (1 - F->bias - F->mbits);
        uint32_t frac = (m - (1u << (len - 1))) << (23 - (len - 1));
        return u2f(sign | ((uint32_t)(exp + 127) << 23) | frac);
    }
    /* normal: (1 + m/2^mbits) * 2^(e - bias) */
    return u2f(sign | ((e - (uint32_t)F->bias + 127u) << 23) | (m << (23 - F->mbits)));
}

float ref_format_max(int fmt) { return ref_decode(fmt, REF_FORMATS[fmt].max_code); }

/* Encode fp32 -> FP8 code: round to nearest, ties to even, saturating. */
uint8_t ref_encode(int fmt, float x)
{
    const ref_format *F = &REF_FORMATS[fmt];
    uint32_t u = f2u(x);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    uint32_t a = u & 0x7FFFFFFFu;

    if (a > 0x7F800000u) return sign | 0x7F;                 /* NaN */
    if (a > f2u(ref_format_max(fmt))) return sign | F->max_code; /* saturate (incl. Inf) */
    if (a == 0) return sign;

    /* a = sig * 2^(ue - 23) with sig the 24-bit significand (no implicit bit
     * for fp32 subnormals). */
    int e32 = (int)(a >> 23);
    uint32_t sig = a & 0x7FFFFFu;
    int ue;
    if (e32 == 0) {
        ue = -126;
    } else {
        ue = e32 - 127;
        sig |= 0x800000u;
    }
    /* The FP8 binade that holds a: below the smallest normal exponent the
     * spacing stays that of the subnormal range. */
    int emin = 1 - F->bias;
    int eq = ue > emin ? ue : emin;
    /* Express a in units of the FP8 spacing 2^(eq - mbits). */
    int r = 23 + (eq - F->mbits) - ue; /* >= 23 - mbits >= 20 */
    if (r >= 25) return sign;          /* sig < 2^24 <= half a unit: rounds to zero */
    uint32_t q = sig >> r;
    uint32_t rem = sig & ((1u << r) - 1);
    uint32_t half = 1u << (r - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    /* Codes are ordered like magnitudes: binade offset plus units.  A carry out
     * of the mantissa moves into the exponent field by itself. */
    uint32_t code = ((uint32_t)(eq - emin) << F->mbits) + q;
    return sign | (uint8_t)code;
}

void ref_encode_array(int fmt, const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = ref_encode(fmt, x[i]);
}

void ref_decode_array(int fmt, const uint8_t *c, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = ref_decode(fmt, c[i]);
}

/* Encode every fp32 bit pattern in [start, start+count) (count may reach 2^32
 * when start = 0); used to compare against an exhaustive device sweep. */
void ref_encode_bits_range(int fmt, uint32_t start, int64_t count, uint8_t *out)
{
    for (int64_t i = 0; i < count; i++) out[i] = ref_encode(fmt, u2f(start + (uint32_t)i));
}

/* -------------------------------------------------------- stochastic rounding */

/* [P3 "Strategies": stochastic rounding, to cut the rounding error that
 * accumulates over many updates]  Round x to one of its two FP8 neighbours
 * lo <= |x| < hi, up with probability equal to its distance from lo, resolved
 * with 16 random bits: with f = (|x| - lo) / (hi - lo) in [0, 1), round up iff
 * floor(f * 2^16) + r16 >= 2^16.  Values at or beyond FMAX saturate as in
 * round-to-nearest; zeros, NaN and exact FP8 values are unchanged. */
uint8_t ref_encode_sr(int fmt, float x, uint32_t r16)
{
    const ref_format *F = &REF_FORMATS[fmt];
    double a = fabs((double)x);
    if (isnan(x) || a == 0.0 || a >= (double)ref_format_max(fmt)) return ref_encode(fmt, x);
    int e;
    (void)frexp(a, &e);                    /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    int emin = 1 - F->bias;                /* exponent of the smallest normal */
    if (ex < emin) ex = emin;              /* subnormal range: one fixed spacing */
    double spacing = ldexp(1.0, ex - F->mbits);
    double units = a / spacing;            /* exact: division by a power of two */
    double lo = floor(units);
    uint32_t d = (uint32_t)floor((units - lo) * 65536.0);
    double mag = (d + (r16 & 0xFFFFu) >= 65536u ? lo + 1.0 : lo) * spacing;
    return ref_encode(fmt, (float)copysign(mag, (double)x)); /* an FP8 value: exact */
}

/* Stochastic-rounding encode of n values, each with its own 16 random bits. */
void ref_encode_sr_array(int fmt, const float *x, const uint16_t *r16, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = ref_encode_sr(fmt, x[i], r16[i]);
}

/* Stochastic-rounding encode of every fp32 bit pattern in [start, start+count) with one
 * fixed r16; used to compare against a device sweep. */
void ref_encode_sr_bits_range(int fmt, uint32_t start, int64_t count, uint32_t r16, uint8_t *out)
{
    for (int64_t i = 0; i < count; i++) out[i] = ref_encode_sr(fmt, u2f(start + (uint32_t)i), r16);
}

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 multiplies with the
 * round constants below, the key bumped by the Weyl constants between rounds. */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; r++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The random word of element i of tensor `tensor` at step t: word i mod 4 of
 * Philox4x32-10 with counter (i/4 low, i/4 high, t, tensor) and the 64-bit
 * seed as key.  The first moment takes its low 16 bits, the second its high
 * 16 bits. */
uint32_t ref_sr_word(uint64_t seed, uint32_t tensor, int64_t t, int64_t i)
{
    uint64_t grp = (uint64_t)i >> 2;
    uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)(grp >> 32), (uint32_t)t, tensor};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ref_philox4x32_10(ctr, key, out);
    return out[i & 3];
}

/* --------------------------------------------------------------- bf16 helpers */

static float bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

/* Round a double to bf16 (8 significant bits, fp32 exponent range, subnormals
 * down to 2^-133), round-to-nearest-even, via frexp/ldexp/nearbyint. */
uint16_t ref_double_to_bf16(double d)
{
    if (isnan(d)) return (uint16_t)((signbit(d) ? 0x8000u : 0) | 0x7FC0u);
    if (d == 0.0 || isinf(d)) return (uint16_t)(f2u((float)d) >> 16);
    int e;
    (void)frexp(d, &e);                 /* |d| in [2^(e-1), 2^e) */
    int qexp = e - 8;                   /* spacing of an 8-bit significand */
    if (qexp < -133) qexp = -133;       /* bf16 subnormal spacing */
    double r = ldexp(nearbyint(ldexp(d, -qexp)), qexp); /* RNE in the default mode */
    return (uint16_t)(f2u((float)r) >> 16); /* exact; overflow becomes Inf */
}

uint16_t ref_f32_to_bf16(float x) { return ref_double_to_bf16((double)x); }

/* -------------------------------------------------------------------- scales */

enum { REF_SCALE_POW2 = 0, REF_SCALE_AMAX = 1 };

/* [P3 "Strategies": dynamic range from the tracked max-abs, exponent offset
 * adjustment]  Scale for a block whose largest magnitude is amax.
 * Writes s and inv_s (real = s * fp8 value; quantize with x * inv_s). */
void ref_choose_scale(int fmt, int mode, float amax, float *s, float *inv_s)
{
    float fmax = ref_format_max(fmt);
    if (!(amax > 0.0f) || !isfinite(amax)) { *s = 1.0f; *inv_s = 1.0f; return; }
    if (mode == REF_SCALE_POW2) {
        /* smallest k with amax / 2^k <= fmax */
        int e;
        float f = frexpf(amax, &e);     /* amax = f * 2^e, f in [0.5, 1) */
        int ef;
        float ff = frexpf(fmax, &ef);   /* fmax = 0.875 * 2^ef for both formats */
        int k = e - ef + (f > ff ? 1 : 0);
        if (k < -126) k = -126;
        if (k > 126) k = 126;
        *s = ldexpf(1.0f, k);
        *inv_s = ldexpf(1.0f, -k);
    } else {
        float sc = amax / fmax;
        if (sc < 0x1p-126f) { *s = 0x1p-126f; *inv_s = 0x1p126f; return; }
        *s = sc;
        *inv_s = fmax / amax;
    }
}

/* ---------------------------------------------------------------------- step */

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;     /* t >= 1 */
    int m_fmt, v_fmt; /* 0 = E4M3, 1 = E5M2 */
    int block;        /* 0: one scale per tensor; else block length (128) */
    int scale_mode;   /* REF_SCALE_POW2 / REF_SCALE_AMAX */
    int master_bf16;  /* 0: p is fp32; 1: p is bf16 bits */
    int l2_coupled;   /* 0: decoupled decay (AdamW); 1: wd * p added to the gradient */
    int history_len;  /* 0: just-in-time scales; H >= 1: delayed scaling over an amax history of H steps */
    int margin;       /* delayed: the scale is chosen for amax_ref * 2^margin (0..64) */
    int64_t delayed_from; /* delayed: steps t < delayed_from choose the scale just in time */
    float grad_factor;    /* every bf16 gradient is multiplied by this first (1: none; loss-scale
                             unscaling and norm clipping otherwise) */
    int64_t sched_step;   /* the step number compared with delayed_from (0: step) */
    int stochastic;       /* 0: round to nearest even; 1: stochastic rounding of both moments */
    uint32_t tensor_index;/* stochastic: the tensor's position in its list (part of the counter) */
    uint64_t seed;        /* stochastic: the generator's key */
    int update_from_codes;/* 0 (the contract): p is updated from the fresh fp32 m', v'.  1 (the
                             other reading of the update order, for study only): from the new
                             codes dequantized with the new scales */
} ref_config;

typedef struct {
    int64_t underflow_m, underflow_v;  /* nonzero moment whose code is +-0 */
    int64_t saturated_m, saturated_v;  /* |x * inv_s| > FMAX before clamping */
    int64_t nonfinite;                 /* elements with a non-finite m' or v' */
    float amax_m, amax_v;              /* max over the tensor of |m'| and v' */
    float scale_m, scale_v;            /* new scale (block mode: largest block scale) */
} ref_stats;

/* Constants shared by every element of a step, from the hyperparameters
 * (fp32 values, widened exactly). */
typedef struct {
    float b1, b2, omb1, omb2;     /* fp32, for the moment update */
    float l2;                     /* coupled-L2 coefficient (0 when decoupled) */
    double decay, step_size, bc2, eps;
} ref_consts;

static ref_consts make_consts(const ref_config *c)
{
    ref_consts k;
    k.b1 = c->beta1;
    k.b2 = c->beta2;
    k.omb1 = 1.0f - c->beta1;
    k.omb2 = 1.0f - c->beta2;
    double bc1 = 1.0 - pow((double)c->beta1, (double)c->step);
    k.bc2 = 1.0 - pow((double)c->beta2, (double)c->step);
    k.l2 = c->l2_coupled ? c->weight_decay : 0.0f;
    k.decay = c->l2_coupled ? 1.0 : 1.0 - (double)c->lr * (double)c->weight_decay;
    k.step_size = (double)c->lr / bc1;
    k.eps = (double)c->eps;
    return k;
}

/* [P1 "Adam's update makes the needs asymmetric", "A numerical example";
 *  P3 "Code example" (AdamW)]  New parameter from the old one and the fresh
 * moments:  p * (1 - lr*wd) - (lr/bc1) * m' / (sqrt(v'/bc2) + eps), in fp64. */
static double param_update(const ref_consts *k, double p, float m1, float v1)
{
    double mhat_num = (double)m1;
    double denom = sqrt((double)v1 / k->bc2) + k->eps;
    return p * k->decay - k->step_size * mhat_num / denom;
}

/* Gradient seen by the moments: g itself, or g + wd * p in the coupled-L2
 * variant (one fp32 rounding). */
static float effective_grad(const ref_consts *k, float g, float p)
{
    return k->l2 != 0.0f ? fmaf(k->l2, p, g) : g;
}

/* [P1 "Adam's update makes the needs asymmetric"]  m moving average of g,
 * v moving average of g^2, in fp32 (see the header for the op order). */
static void moment_update(const ref_consts *k, float g, float m, float v, float *m1, float *v1)
{
    *m1 = fmaf(k->b1, m, k->omb1 * g);
    *v1 = fmaf(k->b2, v, k->omb2 * (g * g));
}

static float amax_update(float acc, float x)
{
    float a = fabsf(x);
    if (isnan(a)) return a;          /* NaN sticks */
    if (isnan(acc)) return acc;
    return a > acc ? a : acc;
}

/* [P3 "Strategies"; code example: delayed scaling with an amax history,
 * margin 0, interval 1, the MAX of the history]  The reference amax of a
 * delayed step: the largest entry of the history (a non-finite entry makes it
 * non-finite, which gives scale 1), times 2^margin. */
static float history_reference(const float *h, int H, int margin)
{
    float r = 0.0f;
    for (int j = 0; j < H; j++) r = amax_update(r, h[j]);
    return ldexpf(r, margin);
}

/*
 * One optimizer step for one tensor, in place on host arrays.
 *   p     : n fp32 (or n bf16 bit patterns when master_bf16)
 *   g     : n bf16 bit patterns
 *   cm,cv : n FP8 codes of m and v
 *   sm,sv : scales (1 per tensor, or ceil(n/block) per block), replaced by the new ones
 *   hist  : delayed scaling only (history_len = H > 0, per-tensor scales): 2H
 *           floats, the amax history of m then of v.  A delayed step (t >=
 *           delayed_from) quantizes with the scale of history_reference() and
 *           saturates what no longer fits; every step (just-in-time ones too)
 *           then records its amax of m' and v' in slot (t-1) mod H, so the
 *           history always holds the last H steps.  NULL when H = 0.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int ref_step_hist(const ref_config *c, int64_t n, void *p, const uint16_t *g,
                  uint8_t *cm, uint8_t *cv, float *sm, float *sv, float *hist, ref_stats *st)
{
    if (!c || n < 0 || c->step < 1 || c->m_fmt < 0 || c->m_fmt > 1 || c->v_fmt < 0 ||
        c->v_fmt > 1 || c->block < 0 || c->history_len < 0)
        return -1;
    const int H = c->history_len;
    if (H > 0 && (c->block > 0 || !hist || c->margin < 0 || c->margin > 64)) return -1;
    const int delayed = H > 0 && (c->sched_step > 0 ? c->sched_step : c->step) >= c->delayed_from;
    ref_consts k = make_consts(c);
    float fmax_m = ref_format_max(c->m_fmt), fmax_v = ref_format_max(c->v_fmt);
    int64_t blen = c->block > 0 ? c->block : (n > 0 ? n : 1);
    /* an empty tensor has no blocks: its scales (and history) stay as they are */
    int64_t nblocks = n > 0 ? (n + blen - 1) / blen : 0;

    float *m1 = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    float *v1 = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!m1 || !v1) { free(m1); free(v1); return -1; }

    ref_stats s;
    memset(&s, 0, sizeof s);
    s.scale_m = s.scale_v = (c->block > 0) ? 0.0f : 1.0f;

    for (int64_t b = 0; b < nblocks; b++) {
        int64_t lo = b * blen, hi = lo + blen < n ? lo + blen : n;
        int64_t si = c->block > 0 ? b : 0;
        float old_sm = sm[si], old_sv = sv[si];

        /* 1. dequantize and update the moments; track the block's amax */
        float am = 0.0f, av = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            float pi = c->master_bf16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
            float gi = effective_grad(&k, bf16_to_f32(g[i]) * c->grad_factor, pi);
            float mi = ref_decode(c->m_fmt, cm[i]) * old_sm;
            float vi = ref_decode(c->v_fmt, cv[i]) * old_sv;
            moment_update(&k, gi, mi, vi, &m1[i], &v1[i]);
            am = amax_update(am, m1[i]);
            av = amax_update(av, v1[i]);
        }

        /* 2. new scales: from the amax of the new moments (just in time), or
         *    from the history of earlier steps (delayed) */
        float nsm, nism, nsv, nisv;
        float ref_m = delayed ? history_reference(hist, H, c->margin) : am;
        float ref_v = delayed ? history_reference(hist + H, H, c->margin) : av;
        ref_choose_scale(c->m_fmt, c->scale_mode, ref_m, &nsm, &nism);
        ref_choose_scale(c->v_fmt, c->scale_mode, ref_v, &nsv, &nisv);

        /* 3. requantize the moments and update the parameters */
        for (int64_t i = lo; i < hi; i++) {
            float qm = m1[i] * nism, qv = v1[i] * nisv;
            if (c->stochastic) {
                uint32_t r = ref_sr_word(c->seed, c->tensor_index, c->step, i);
                cm[i] = ref_encode_sr(c->m_fmt, qm, r & 0xFFFFu);
                cv[i] = ref_encode_sr(c->v_fmt, qv, r >> 16);
            } else {
                cm[i] = ref_encode(c->m_fmt, qm);
                cv[i] = ref_encode(c->v_fmt, qv);
            }
            if (m1[i] != 0.0f && (cm[i] & 0x7F) == 0) s.underflow_m++;
            if (v1[i] != 0.0f && (cv[i] & 0x7F) == 0) s.underflow_v++;
            if (fabsf(qm) > fmax_m) s.saturated_m++;
            if (fabsf(qv) > fmax_v) s.saturated_v++;
            if (!isfinite(m1[i]) || !isfinite(v1[i])) s.nonfinite++;

            float um = m1[i], uv = v1[i];
            if (c->update_from_codes) {
                um = ref_decode(c->m_fmt, cm[i]) * nsm;
                uv = ref_decode(c->v_fmt, cv[i]) * nsv;
            }
            if (c->master_bf16) {
                uint16_t *pb = (uint16_t *)p;
                double np = param_update(&k, (double)bf16_to_f32(pb[i]), um, uv);
                pb[i] = ref_double_to_bf16(np);
            } else {
                float *pf = (float *)p;
                pf[i] = (float)param_update(&k, (double)pf[i], um, uv);
            }
        }

        sm[si] = nsm;
        sv[si] = nsv;
        if (H > 0) {
            int slot = (int)((c->step - 1) % H);
            hist[slot] = am;
            hist[H + slot] = av;
        }
        s.amax_m = amax_update(s.amax_m, am);
        s.amax_v = amax_update(s.amax_v, av);
        if (c->block > 0) {
            if (nsm > s.scale_m) s.scale_m = nsm;
            if (nsv > s.scale_v) s.scale_v = nsv;
        } else {
            s.scale_m = nsm;
            s.scale_v = nsv;
        }
    }
    free(m1);
    free(v1);
    if (st) *st = s;
    return 0;
}

/* Just-in-time step (no history). */
int ref_step(const ref_config *c, int64_t n, void *p, const uint16_t *g,
             uint8_t *cm, uint8_t *cv, float *sm, float *sv, ref_stats *st)
{
    if (!c || c->history_len != 0) return -1;
    return ref_step_hist(c, n, p, g, cm, cv, sm, sv, NULL, st);
}

/*
 * Plain AdamW with the moments kept in fp32 (no FP8 storage): the same moment
 * and parameter arithmetic as ref_step with the codec taken out.  Used to pin
 * the step against closed forms and a library AdamW.
 *   p : n fp32;  g : n bf16 bits;  m, v : n fp32, updated in place.
 */
int ref_step_fp32_moments(const ref_config *c, int64_t n, float *p, const uint16_t *g,
                          float *m, float *v)
{
    if (!c || n < 0 || c->step < 1) return -1;
    ref_consts k = make_consts(c);
    for (int64_t i = 0; i < n; i++) {
        float m1, v1;
        moment_update(&k, effective_grad(&k, bf16_to_f32(g[i]) * c->grad_factor, p[i]), m[i], v[i], &m1, &v1);
        p[i] = (float)param_update(&k, (double)p[i], m1, v1);
        m[i] = m1;
        v[i] = v1;
    }
    return 0;
}

/* The library is meant to run in the default rounding mode. */
int ref_rounding_is_nearest(void) { return fegetround() == FE_TONEAREST; }

/* ------------------------------------------------- loss scaling and clipping
 *
 * [P3 "Strategies": gradient (loss) scaling that grows the scale after a run of
 * overflow-free iterations and shrinks it on overflow; gradient clipping.
 * P3 code example: the gradients are unscaled, clipped to a global norm of
 * max_norm = 1.0, and the optimizer step is skipped when they overflowed.]
 * Readings (the page gives the calls, not the arithmetic; these are the
 * definitions of the library calls it names):
 *   - unscale: g / S with inv_S = 1/S rounded to fp32;
 *   - non-finite: any Inf/NaN gradient element skips the whole step (nothing
 *     changes but the loss scale), S *= backoff and the growth count restarts;
 *     otherwise the count grows, and reaching growth_interval multiplies S by
 *     growth (if that stays finite) and restarts it;
 *   - norm: ||g / S|| over every tensor, from the EXACT sum of squares;
 *   - clip coefficient c = min(1, max_norm / (norm + 1e-6)) rounded to fp32
 *     (c = 1 without clipping); every gradient is then multiplied by the one
 *     fp32 factor c * inv_S (one rounding per element);
 *   - a skipped step does not count: the Adam step t is the number of steps
 *     taken, kept with the scaler.
 */

/* Exact sum of squares of bf16 values, kept per binary exponent: a finite
 * bf16 value is M * 2^(E - 134) with M = 128 + mantissa for E >= 1 and
 * M = mantissa (E taken as 1) for subnormals, so its square is
 * M^2 * 2^(2E - 268) with M^2 < 2^16; acc[E] sums M^2 exactly. */
void ref_grad_sumsq(const uint16_t *g, int64_t n, uint64_t acc[256], int64_t *nonfinite)
{
    for (int64_t i = 0; i < n; i++) {
        uint32_t b = g[i];
        uint32_t e = (b >> 7) & 0xFFu, mant = b & 0x7Fu;
        if (e == 0xFFu) { (*nonfinite)++; continue; }
        uint32_t m = e ? (0x80u | mant) : mant;
        if (!e) e = 1;
        acc[e] += (uint64_t)m * m;
    }
}

/* sum_E acc[E] * 2^(2E - 268), exact in a 704-bit integer (bit 0 = 2^-266),
 * then rounded once to double (round to nearest even). */
double ref_sumsq_total(const uint64_t acc[256])
{
    enum { L = 11 };
    uint64_t big[L];
    memset(big, 0, sizeof big);
    for (int e = 1; e < 255; e++) {
        if (!acc[e]) continue;
        int sh = 2 * e - 2;                       /* 2E - 268 - (-266) */
        int w = sh / 64, b = sh % 64;
        uint64_t lo = acc[e] << b, hi = b ? acc[e] >> (64 - b) : 0;
        unsigned __int128 carry = 0;
        for (int k = w; k < L; k++) {
            unsigned __int128 add = (k == w ? lo : (k == w + 1 ? hi : 0));
            unsigned __int128 sum = (unsigned __int128)big[k] + add + carry;
            big[k] = (uint64_t)sum;
            carry = sum >> 64;
            if (k > w + 1 && !carry) break;
        }
    }
    int top = -1;
    for (int k = L - 1; k >= 0 && top < 0; k--)
        if (big[k]) top = 64 * k + 63 - __builtin_clzll(big[k]);
    if (top < 0) return 0.0;
    /* the 64 bits top..top-63 (zeros below bit 0), and whether anything lies below them */
    uint64_t hi64 = 0;
    int sticky = 0;
    for (int j = 0; j < 64; j++) {
        int bit = top - j;
        uint64_t v = bit >= 0 ? (big[bit / 64] >> (bit % 64)) & 1u : 0u;
        hi64 = (hi64 << 1) | v;
    }
    for (int bit = top - 64; bit >= 0 && !sticky; bit--)
        if ((big[bit / 64] >> (bit % 64)) & 1u) sticky = 1;
    uint64_t keep = hi64 >> 11, rem = hi64 & 0x7FFu;
    if (rem > 0x400u || (rem == 0x400u && (sticky || (keep & 1u)))) keep++;
    return ldexp((double)keep, top - 52 - 266);
}

typedef struct {
    float max_norm;         /* <= 0: no clipping */
    float growth_factor, backoff_factor;
    int32_t growth_interval;
} ref_amp_config;

typedef struct {
    float scale;
    int32_t growth_tracker;
    int64_t step;           /* Adam steps taken */
    int32_t found_inf;
    float grad_norm, clip_coef, grad_factor;
} ref_amp_state;

/* One scaler decision from the sums of every tensor's gradients (acc and
 * nonfinite summed over the list).  Updates st; on success st->step is the t
 * of the step to run and st->grad_factor the factor for ref_step. */
void ref_amp_control(const uint64_t acc[256], int64_t nonfinite, const ref_amp_config *cfg,
                     ref_amp_state *st)
{
    float inv = (float)(1.0 / (double)st->scale);
    if (nonfinite > 0) {
        st->found_inf = 1;
        st->grad_norm = NAN;
        st->clip_coef = 1.0f;
        st->grad_factor = 0.0f;
        st->scale = st->scale * cfg->backoff_factor;
        st->growth_tracker = 0;
        return;
    }
    double norm = sqrt(ref_sumsq_total(acc)) * (double)inv;
    double c = 1.0;
    if (cfg->max_norm > 0.0f) {
        c = (double)cfg->max_norm / (norm + 1e-6);
        if (c > 1.0) c = 1.0;
    }
    st->found_inf = 0;
    st->grad_norm = (float)norm;
    st->clip_coef = (float)c;
    st->grad_factor = st->clip_coef * inv;
    st->step += 1;
    int32_t next = st->growth_tracker + 1;
    if (next == cfg->growth_interval) {
        float grown = st->scale * cfg->growth_factor;
        if (isfinite(grown)) st->scale = grown;
        st->growth_tracker = 0;
    } else {
        st->growth_tracker = next;
    }
}
