/* A plain C11 caller of the FP8-moment Adam library: no torch, no Python.  It
 * allocates two tensors' buffers with hipMalloc (the moments and scales left
 * uninitialized: the context writes the fresh state, zero_state), runs two
 * AdamW steps with deterministic gradients, and writes the inputs and the
 * results to a file for the test to replay through the oracle.
 *
 * Output, little-endian, per tensor: int64 n; float p0[n]; uint16 g1[n];
 * uint16 g2[n]; float p[n]; uint8 m[n]; uint8 v[n]; float m_scale; float v_scale.
 * Usage: c_abi_demo OUT_FILE; exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8adam.h"

#define NT 2
static const int64_t SIZES[NT] = {1000, 4097};

static uint32_t next31(uint64_t *s) {
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(*s >> 33);
}

static double uniform(uint64_t *s) { return (next31(s) + 0.5) / 2147483648.0; }

static uint16_t to_bf16(float x) {  /* round to nearest even (finite inputs) */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(e) do { hipError_t r_ = (e); if (r_ != hipSuccess) { \
    fprintf(stderr, "%s: %s\n", #e, hipGetErrorString(r_)); return 1; } } while (0)
#define CHECK_LIB(e) do { int r_ = (e); if (r_ != 0) { \
    fprintf(stderr, "%s: %d %s\n", #e, r_, fp8adam_last_error()); return 1; } } while (0)

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    uint64_t seed = 2409;
    float *p0[NT], *p_out[NT], *d_p[NT], *d_ms[NT], *d_vs[NT], ms[NT], vs[NT];
    uint16_t *g[NT][2], *d_g[NT];
    uint8_t *d_m[NT], *d_v[NT], *m_out[NT], *v_out[NT];
    fp8adam_tensor tens[NT];
    memset(tens, 0, sizeof tens);
    for (int t = 0; t < NT; t++) {
        const int64_t n = SIZES[t];
        p0[t] = malloc(sizeof(float) * n);
        p_out[t] = malloc(sizeof(float) * n);
        m_out[t] = malloc(n);
        v_out[t] = malloc(n);
        const double gscale = t == 0 ? 1e-3 : 3e-5;
        for (int s = 0; s < 2; s++) {
            g[t][s] = malloc(sizeof(uint16_t) * n);
            for (int64_t i = 0; i < n; i++) g[t][s][i] = to_bf16((float)((uniform(&seed) - 0.5) * gscale));
        }
        for (int64_t i = 0; i < n; i++) p0[t][i] = (float)((uniform(&seed) - 0.5) * 0.04);
        CHECK_HIP(hipMalloc((void **)&d_p[t], sizeof(float) * n));
        CHECK_HIP(hipMalloc((void **)&d_g[t], sizeof(uint16_t) * n));
        CHECK_HIP(hipMalloc((void **)&d_m[t], n));
        CHECK_HIP(hipMalloc((void **)&d_v[t], n));
        CHECK_HIP(hipMalloc((void **)&d_ms[t], sizeof(float)));
        CHECK_HIP(hipMalloc((void **)&d_vs[t], sizeof(float)));
        CHECK_HIP(hipMemcpy(d_p[t], p0[t], sizeof(float) * n, hipMemcpyHostToDevice));
        tens[t].param = d_p[t];
        tens[t].grad = d_g[t];
        tens[t].m = d_m[t];
        tens[t].v = d_v[t];
        tens[t].m_scale = d_ms[t];
        tens[t].v_scale = d_vs[t];
        tens[t].numel = n;
    }
    fp8adam_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.m_format = FP8ADAM_E4M3;
    cfg.v_format = FP8ADAM_E5M2;
    cfg.granularity = FP8ADAM_SCALE_TENSOR;
    cfg.scale_mode = FP8ADAM_SCALE_POW2;
    cfg.master = FP8ADAM_MASTER_FP32;
    cfg.schedule = FP8ADAM_SCHEDULE_TWO_PASS;
    cfg.zero_state = 1;
    fp8adam_ctx *ctx = NULL;
    CHECK_LIB(fp8adam_init(&ctx, tens, NT, &cfg, NULL));
    for (int s = 0; s < 2; s++) {
        for (int t = 0; t < NT; t++)
            CHECK_HIP(hipMemcpy(d_g[t], g[t][s], sizeof(uint16_t) * SIZES[t], hipMemcpyHostToDevice));
        fp8adam_hparams hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, s + 1};
        CHECK_LIB(fp8adam_step(ctx, &hp, NULL));
        CHECK_HIP(hipDeviceSynchronize());
    }
    fp8adam_stats_t st[NT];
    CHECK_LIB(fp8adam_stats(ctx, st, NT, NULL));
    fp8adam_destroy(ctx);
    FILE *f = fopen(argv[1], "wb");
    if (!f) return 1;
    for (int t = 0; t < NT; t++) {
        const int64_t n = SIZES[t];
        CHECK_HIP(hipMemcpy(p_out[t], d_p[t], sizeof(float) * n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(m_out[t], d_m[t], n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(v_out[t], d_v[t], n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(&ms[t], d_ms[t], sizeof(float), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(&vs[t], d_vs[t], sizeof(float), hipMemcpyDeviceToHost));
        if (st[t].scale_m != ms[t] || st[t].scale_v != vs[t]) {
            fprintf(stderr, "stats disagree with the scales of tensor %d\n", t);
            return 1;
        }
        fwrite(&n, sizeof n, 1, f);
        fwrite(p0[t], sizeof(float), n, f);
        fwrite(g[t][0], sizeof(uint16_t), n, f);
        fwrite(g[t][1], sizeof(uint16_t), n, f);
        fwrite(p_out[t], sizeof(float), n, f);
        fwrite(m_out[t], 1, n, f);
        fwrite(v_out[t], 1, n, f);
        fwrite(&ms[t], sizeof(float), 1, f);
        fwrite(&vs[t], sizeof(float), 1, f);
        hipFree(d_p[t]); hipFree(d_g[t]); hipFree(d_m[t]); hipFree(d_v[t]); hipFree(d_ms[t]); hipFree(d_vs[t]);
    }
    fclose(f);
    printf("c abi demo: %d tensors, 2 steps\n", NT);
    return 0;
}
