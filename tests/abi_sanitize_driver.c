/* Calls every argument-checking path of the C ABI that returns before any
 * device work (null and misaligned pointers, bad enums and option
 * combinations, bad hyperparameters, contexts past the launch limit, bad
 * codec-probe arguments), for a build of the library whose host code carries
 * AddressSanitizer.  No GPU is needed.  Exit status 0 and no sanitizer report
 * is the pass condition; a wrong return code prints the case and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8adam.h"

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: returned %d, expected %d (%s)\n", what, got, want, fp8adam_last_error());
        failures++;
    }
    (void)strlen(fp8adam_last_error());  /* the message is a valid string */
}

static fp8adam_tensor tensor(uintptr_t base, int64_t numel) {
    fp8adam_tensor t;
    memset(&t, 0, sizeof t);
    t.param = (void *)(base + 0);
    t.grad = (const void *)(base + 16);
    t.m = (uint8_t *)(base + 32);
    t.v = (uint8_t *)(base + 48);
    t.m_scale = (float *)(base + 64);
    t.v_scale = (float *)(base + 80);
    t.numel = numel;
    return t;
}

int main(void) {
    fp8adam_ctx *h = NULL;
    fp8adam_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.m_format = FP8ADAM_E4M3;
    cfg.v_format = FP8ADAM_E5M2;
    fp8adam_tensor one = tensor(0x1000, 10);

    expect(fp8adam_init(NULL, &one, 1, &cfg, NULL), FP8ADAM_EINVAL, "null out");
    expect(fp8adam_init(&h, NULL, 1, &cfg, NULL), FP8ADAM_EINVAL, "null tensors");
    expect(fp8adam_init(&h, &one, 0, &cfg, NULL), FP8ADAM_EINVAL, "n = 0");
    expect(fp8adam_init(&h, &one, 1, NULL, NULL), FP8ADAM_EINVAL, "null cfg");
    fp8adam_config bad = cfg;
    bad.m_format = 7;
    expect(fp8adam_init(&h, &one, 1, &bad, NULL), FP8ADAM_EINVAL, "bad format");
    bad = cfg;
    bad.schedule = FP8ADAM_SCHEDULE_SPECULATIVE;
    expect(fp8adam_init(&h, &one, 1, &bad, NULL), FP8ADAM_EINVAL, "speculative without m_alt");
    bad.granularity = FP8ADAM_SCALE_BLOCK128;
    expect(fp8adam_init(&h, &one, 1, &bad, NULL), FP8ADAM_EINVAL, "speculative with block scales");
    bad = cfg;
    bad.scaling = FP8ADAM_SCALING_DELAYED;
    expect(fp8adam_init(&h, &one, 1, &bad, NULL), FP8ADAM_EINVAL, "delayed without a history");
    bad.amax_history_len = 5000;
    expect(fp8adam_init(&h, &one, 1, &bad, NULL), FP8ADAM_EINVAL, "history too long");
    fp8adam_tensor odd = tensor(0x1004, 10);
    expect(fp8adam_init(&h, &odd, 1, &cfg, NULL), FP8ADAM_EALIGN, "misaligned param");
    fp8adam_tensor neg = tensor(0x1000, -1);
    expect(fp8adam_init(&h, &neg, 1, &cfg, NULL), FP8ADAM_EINVAL, "negative numel");
    fp8adam_tensor huge = tensor(0x1000, (int64_t)1 << 62);
    expect(fp8adam_init(&h, &huge, 1, &cfg, NULL), FP8ADAM_EINVAL, "too many elements");
    /* a list that only overflows once each tensor is rounded up to whole chunks */
    const int32_t n_many = 524272;
    fp8adam_tensor *many = malloc(sizeof(fp8adam_tensor) * (size_t)n_many);
    if (!many) return 2;
    for (int32_t i = 0; i < n_many; i++) many[i] = tensor(0x1000, 32769);
    expect(fp8adam_init(&h, many, n_many, &cfg, NULL), FP8ADAM_EINVAL, "too many chunks");
    free(many);
    if (h != NULL) { fprintf(stderr, "handle set on failure\n"); failures++; }

    fp8adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1};
    expect(fp8adam_step(NULL, &hp, NULL), FP8ADAM_EINVAL, "step without a context");
    fp8adam_amp_config amp = {1.0f, 2.0f, 0.5f, 2000};
    expect(fp8adam_step_amp(NULL, &hp, &amp, (void *)64, NULL), FP8ADAM_EINVAL, "amp without a context");
    fp8adam_stats_t st;
    expect(fp8adam_stats(NULL, &st, 1, NULL), FP8ADAM_EINVAL, "stats without a context");
    fp8adam_destroy(NULL);
    expect(fp8adam_encode(3, NULL, NULL, 10, NULL), FP8ADAM_EINVAL, "encode: bad format");
    expect(fp8adam_decode(0, NULL, NULL, 10, NULL), FP8ADAM_EINVAL, "decode: null pointers");
    expect(fp8adam_encode_bits_range(0, 10, (int64_t)1 << 32, NULL, NULL), FP8ADAM_EINVAL, "bits range: too long");
    expect(fp8adam_encode_sr(0, NULL, NULL, NULL, -1, NULL), FP8ADAM_EINVAL, "encode_sr: negative n");
    expect(fp8adam_encode_sr(1, NULL, NULL, NULL, 0, NULL), 0, "encode_sr: empty");
    expect(fp8adam_stream_copy(NULL, NULL, 24, NULL), FP8ADAM_EINVAL, "copy: not a multiple of 16");
    expect(fp8adam_stream_copy((const void *)8, (void *)16, 32, NULL), FP8ADAM_EALIGN, "copy: misaligned");
    expect(fp8adam_stream_copy(NULL, NULL, 0, NULL), 0, "copy: empty");
    expect((int)fp8adam_num_chunks(NULL), -1, "num_chunks without a context");
    expect(fp8adam_current_buffer(NULL), -1, "current_buffer without a context");
    expect(fp8adam_set_timing(NULL, 1), FP8ADAM_EINVAL, "set_timing without a context");
    double ms[4];
    int32_t cnt[4];
    expect(fp8adam_kernel_times(NULL, ms, cnt, 4), FP8ADAM_EINVAL, "kernel_times without a context");
    expect(fp8adam_runtime_version(NULL), FP8ADAM_EINVAL, "runtime_version: null");

    printf("abi driver done, %d failures\n", failures);
    return failures ? 1 : 0;
}
