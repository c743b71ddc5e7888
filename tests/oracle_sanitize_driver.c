/*
 * Drives every entry point of the CPU oracle (oracle/fp8adam_oracle.c, compiled
 * into this program) over small ragged tensors in every mode, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer can check the oracle's
 * own memory accesses and integer/float conversions.  Host code only.
 * Exit status 0 and no sanitizer report on stderr is the pass condition.
 */
#include "../oracle/fp8adam_oracle.c"

#include <stdio.h>
#include <stdlib.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    /* xorshift64*: a test input generator, nothing of the method */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static float uniform(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }

/* bf16 gradient bits: sign, a wide spread of magnitudes, some zeros */
static uint16_t random_grad_bits(void)
{
    const uint32_t r = next_u32();
    if ((r & 31u) == 0u) return (uint16_t)((r & 32u) ? 0x8000u : 0u);
    const float x = (uniform() * 2.0f - 1.0f) * powf(10.0f, -7.0f + 8.0f * uniform());
    return ref_f32_to_bf16(x);
}

static int run_case(int64_t n, int m_fmt, int v_fmt, int block, int mode, int bf16, int l2, int hist_len,
                    int stochastic)
{
    const int64_t nb = block ? (n + block - 1) / block : 1;
    void *p = malloc((size_t)(n ? n : 1) * (bf16 ? 2 : 4));
    uint16_t *g = malloc((size_t)(n ? n : 1) * 2);
    uint8_t *cm = calloc((size_t)(n ? n : 1), 1), *cv = calloc((size_t)(n ? n : 1), 1);
    float *sm = malloc((size_t)nb * 4), *sv = malloc((size_t)nb * 4);
    float *hist = hist_len ? calloc((size_t)(2 * hist_len), 4) : NULL;
    if (!p || !g || !cm || !cv || !sm || !sv || (hist_len && !hist)) return -1;
    for (int64_t i = 0; i < nb; i++) sm[i] = sv[i] = 1.0f;
    for (int64_t i = 0; i < n; i++) {
        const float x = (uniform() - 0.5f) * 0.04f;
        if (bf16) ((uint16_t *)p)[i] = ref_f32_to_bf16(x);
        else ((float *)p)[i] = x;
    }
    int rc = 0;
    for (int t = 1; t <= 4 && rc == 0; t++) {
        for (int64_t i = 0; i < n; i++) g[i] = random_grad_bits();
        ref_config c;
        memset(&c, 0, sizeof c);
        c.lr = 1e-3f; c.beta1 = 0.9f; c.beta2 = 0.95f; c.eps = 1e-8f; c.weight_decay = 0.1f;
        c.step = t; c.m_fmt = m_fmt; c.v_fmt = v_fmt; c.block = block; c.scale_mode = mode;
        c.master_bf16 = bf16; c.l2_coupled = l2; c.history_len = hist_len; c.margin = hist_len ? 1 : 0;
        c.delayed_from = 2; c.grad_factor = 1.0f; c.stochastic = stochastic; c.tensor_index = 3;
        c.seed = 1234; c.update_from_codes = (t == 4);
        ref_stats st;
        rc = hist_len ? ref_step_hist(&c, n, p, g, cm, cv, sm, sv, hist, &st)
                      : ref_step(&c, n, p, g, cm, cv, sm, sv, &st);
    }
    free(p); free(g); free(cm); free(cv); free(sm); free(sv); free(hist);
    return rc;
}

int main(void)
{
    int failures = 0;
    /* codec: every code, a stride over all fp32 patterns, stochastic rounding */
    for (int fmt = 0; fmt < 2; fmt++) {
        for (int c = 0; c < 256; c++) (void)ref_decode(fmt, (uint8_t)c);
        uint8_t out[4096];
        for (uint64_t start = 0; start < (1ull << 32); start += 4096ull * 1021ull)
            ref_encode_bits_range(fmt, (uint32_t)start, 4096, out);
        ref_encode_sr_bits_range(fmt, 0x3F800000u, 4096, 0x8000u, out);
        float x[64];
        uint16_t r16[64];
        for (int i = 0; i < 64; i++) { x[i] = (uniform() - 0.5f) * 1000.0f; r16[i] = (uint16_t)next_u32(); }
        ref_encode_sr_array(fmt, x, r16, 64, out);
        ref_encode_array(fmt, x, out, 64);
        float s, inv;
        ref_choose_scale(fmt, 0, 0.0f, &s, &inv);
        ref_choose_scale(fmt, 0, 3.0e38f, &s, &inv);
        ref_choose_scale(fmt, 1, 1e-40f, &s, &inv);
        ref_choose_scale(fmt, 1, INFINITY, &s, &inv);
    }
    /* steps: ragged sizes over every option */
    const int64_t sizes[] = {0, 1, 3, 4, 5, 127, 128, 129, 255, 1025};
    for (size_t k = 0; k < sizeof sizes / sizeof sizes[0]; k++)
        for (int fmts = 0; fmts < 4; fmts++)
            for (int block = 0; block <= 128; block += 128)
                for (int mode = 0; mode < 2; mode++)
                    for (int opt = 0; opt < 5; opt++) {
                        const int bf16 = opt == 1, l2 = opt == 2, hist = (opt == 3 && !block) ? 4 : 0,
                                  sr = opt == 4;
                        if (run_case(sizes[k], fmts >> 1, fmts & 1, block, mode, bf16, l2, hist, sr) != 0) {
                            fprintf(stderr, "case failed: n=%lld fmts=%d block=%d mode=%d opt=%d\n",
                                    (long long)sizes[k], fmts, block, mode, opt);
                            failures++;
                        }
                    }
    /* fp32-moment mode, gradient sums and the loss-scaler decision */
    {
        enum { N = 777 };
        float p[N], m[N], v[N];
        uint16_t g[N];
        for (int i = 0; i < N; i++) { p[i] = uniform(); m[i] = 0.0f; v[i] = 0.0f; g[i] = random_grad_bits(); }
        ref_config c;
        memset(&c, 0, sizeof c);
        c.lr = 1e-3f; c.beta1 = 0.9f; c.beta2 = 0.999f; c.eps = 1e-8f; c.step = 1; c.grad_factor = 1.0f;
        if (ref_step_fp32_moments(&c, N, p, g, m, v) != 0) failures++;
        uint64_t acc[256] = {0};
        int64_t nonfinite = 0;
        g[5] = 0x7F80u; /* +Inf */
        ref_grad_sumsq(g, N, acc, &nonfinite);
        (void)ref_sumsq_total(acc);
        ref_amp_config ac = {1.0f, 2.0f, 0.5f, 3};
        ref_amp_state as;
        memset(&as, 0, sizeof as);
        as.scale = 65536.0f;
        ref_amp_control(acc, nonfinite, &ac, &as);
        ref_amp_control(acc, 0, &ac, &as);
        uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
        ref_philox4x32_10(ctr, key, out);
        (void)ref_sr_word(99, 7, 3, 123456789);
    }
    if (failures) fprintf(stderr, "%d cases failed\n", failures);
    printf("oracle driver done\n");
    return failures ? 1 : 0;
}
