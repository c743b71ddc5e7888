/* A plain C11 caller of fp8adam_step_noalloc, the step for callers that cannot
 * allocate device memory, inside a HIP graph: no torch, no Python.  Three
 * ragged tensors get two copies of the same state (A and B) and one shared
 * set of gradients.  One eager call on a third copy sets up the library's
 * scratch address on the device; then a step on A is captured into a graph
 * (capture records the launches without running them, so A must be
 * unchanged) and the graph is replayed three times, each replay followed by
 * the same step called eagerly on B and a device-to-host copy of both: A and
 * B must agree bit for bit (weights, codes, scales) after every replay.
 * Usage: c_noalloc_graph_demo; exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8adam.h"

#define NT 3
#define NSETS 3 /* 0: captured (A), 1: eager (B), 2: the set-up call's copy */
static const int64_t SIZES[NT] = {70001, 4096, 33};

static uint32_t next31(uint64_t *s) {
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(*s >> 33);
}

static double uniform(uint64_t *s) { return (next31(s) + 0.5) / 2147483648.0; }

static uint16_t to_bf16(float x) { /* round to nearest even (finite inputs) */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(e) do { hipError_t r_ = (e); if (r_ != hipSuccess) { \
    fprintf(stderr, "%s: %s\n", #e, hipGetErrorString(r_)); return 1; } } while (0)
#define CHECK_LIB(e) do { int r_ = (e); if (r_ != 0) { \
    fprintf(stderr, "%s: %d %s\n", #e, r_, fp8adam_last_error()); return 1; } } while (0)

struct host_state { float *p; uint8_t *m, *v; float ms, vs; };

/* Copies one tensor's device state to the host. */
static int fetch(fp8adam_tensor *T, int64_t n, struct host_state *h) {
    CHECK_HIP(hipMemcpy(h->p, T->param, sizeof(float) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h->m, T->m, n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h->v, T->v, n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&h->ms, T->m_scale, sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&h->vs, T->v_scale, sizeof(float), hipMemcpyDeviceToHost));
    return 0;
}

static int same(const struct host_state *a, const struct host_state *b, int64_t n) {
    return memcmp(a->p, b->p, sizeof(float) * n) == 0 && memcmp(a->m, b->m, n) == 0 &&
           memcmp(a->v, b->v, n) == 0 && memcmp(&a->ms, &b->ms, sizeof(float)) == 0 &&
           memcmp(&a->vs, &b->vs, sizeof(float)) == 0;
}

int main(void) {
    uint64_t seed = 95;
    fp8adam_tensor tens[NSETS][NT];
    memset(tens, 0, sizeof tens);
    struct host_state init[NT], ha[NT], hb[NT];
    for (int t = 0; t < NT; t++) {
        const int64_t n = SIZES[t];
        float *p0 = malloc(sizeof(float) * n);
        uint16_t *g = malloc(sizeof(uint16_t) * n);
        uint8_t *m0 = malloc(n), *v0 = malloc(n);
        if (!p0 || !g || !m0 || !v0) return 1;
        for (int64_t i = 0; i < n; i++) {
            p0[i] = (float)((uniform(&seed) - 0.5) * 0.04);
            g[i] = to_bf16((float)((uniform(&seed) - 0.5) * (t == 1 ? 3e-5 : 1e-3)));
            m0[i] = (uint8_t)(next31(&seed) & 0xF7u); /* finite E4M3 codes, both signs */
            v0[i] = (uint8_t)(next31(&seed) & 0x77u); /* finite non-negative E5M2 codes */
        }
        const float ms0 = 0.0078125f, vs0 = 9.5367431640625e-07f; /* 2^-7, 2^-20 */
        void *d_g;
        CHECK_HIP(hipMalloc(&d_g, sizeof(uint16_t) * n));
        CHECK_HIP(hipMemcpy(d_g, g, sizeof(uint16_t) * n, hipMemcpyHostToDevice));
        for (int k = 0; k < NSETS; k++) {
            fp8adam_tensor *T = &tens[k][t];
            CHECK_HIP(hipMalloc(&T->param, sizeof(float) * n));
            CHECK_HIP(hipMalloc((void **)&T->m, n));
            CHECK_HIP(hipMalloc((void **)&T->v, n));
            CHECK_HIP(hipMalloc((void **)&T->m_scale, sizeof(float)));
            CHECK_HIP(hipMalloc((void **)&T->v_scale, sizeof(float)));
            CHECK_HIP(hipMemcpy(T->param, p0, sizeof(float) * n, hipMemcpyHostToDevice));
            CHECK_HIP(hipMemcpy(T->m, m0, n, hipMemcpyHostToDevice));
            CHECK_HIP(hipMemcpy(T->v, v0, n, hipMemcpyHostToDevice));
            CHECK_HIP(hipMemcpy(T->m_scale, &ms0, sizeof(float), hipMemcpyHostToDevice));
            CHECK_HIP(hipMemcpy(T->v_scale, &vs0, sizeof(float), hipMemcpyHostToDevice));
            T->grad = d_g;
            T->numel = n;
        }
        init[t].p = p0;
        init[t].m = m0;
        init[t].v = v0;
        ha[t].p = malloc(sizeof(float) * n);
        ha[t].m = malloc(n);
        ha[t].v = malloc(n);
        hb[t].p = malloc(sizeof(float) * n);
        hb[t].m = malloc(n);
        hb[t].v = malloc(n);
        if (!ha[t].p || !ha[t].m || !ha[t].v || !hb[t].p || !hb[t].m || !hb[t].v) return 1;
        free(g);
    }
    fp8adam_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.m_format = FP8ADAM_E4M3;
    cfg.v_format = FP8ADAM_E5M2;
    cfg.granularity = FP8ADAM_SCALE_TENSOR;
    cfg.scale_mode = FP8ADAM_SCALE_POW2;
    cfg.master = FP8ADAM_MASTER_FP32;
    cfg.schedule = FP8ADAM_SCHEDULE_TWO_PASS;
    const fp8adam_hparams hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 3};
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    CHECK_LIB(fp8adam_step_noalloc(tens[2], NT, &cfg, &hp, s)); /* sets up the scratch address */
    CHECK_HIP(hipStreamSynchronize(s));

    hipGraph_t graph;
    hipGraphExec_t exec;
    CHECK_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    CHECK_LIB(fp8adam_step_noalloc(tens[0], NT, &cfg, &hp, s));
    CHECK_HIP(hipStreamEndCapture(s, &graph));
    CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
    for (int t = 0; t < NT; t++) {
        if (fetch(&tens[0][t], SIZES[t], &ha[t])) return 1;
        init[t].ms = 0.0078125f;
        init[t].vs = 9.5367431640625e-07f;
        if (!same(&ha[t], &init[t], SIZES[t])) {
            fprintf(stderr, "capture changed tensor %d\n", t);
            return 1;
        }
    }
    for (int r = 0; r < 3; r++) {
        CHECK_HIP(hipGraphLaunch(exec, s));
        CHECK_HIP(hipStreamSynchronize(s));
        CHECK_LIB(fp8adam_step_noalloc(tens[1], NT, &cfg, &hp, s));
        CHECK_HIP(hipStreamSynchronize(s));
        for (int t = 0; t < NT; t++) {
            if (fetch(&tens[0][t], SIZES[t], &ha[t]) || fetch(&tens[1][t], SIZES[t], &hb[t])) return 1;
            if (!same(&ha[t], &hb[t], SIZES[t])) {
                fprintf(stderr, "replay %d: tensor %d differs from the eager step\n", r + 1, t);
                return 1;
            }
            if (same(&ha[t], &init[t], SIZES[t])) {
                fprintf(stderr, "replay %d: tensor %d did not change\n", r + 1, t);
                return 1;
            }
        }
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));
    CHECK_HIP(hipStreamDestroy(s));
    printf("c noalloc graph demo: %d tensors, 3 replays equal to eager steps\n", NT);
    return 0;
}
