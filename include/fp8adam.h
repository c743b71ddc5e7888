/*
 * fp8adam.h -- C ABI of the FP8-moment Adam/AdamW step for AMD MI355X (gfx950).
 *
 * The step is Adam/AdamW whose two moments are stored as FP8 codes with a
 * scale: the first moment m in E4M3, the second moment v in E5M2 by default.
 * Sources (the three pages the method is taken from):
 *   - daoxuan.cc explainer of arXiv 2409.12517 (blog.daoxuan.cc/posts/32114),
 *     section on why Adam keeps m in E4M3 and v in E5M2: the format table,
 *     the asymmetry of the update (m in the numerator times the learning rate,
 *     v under a square root in the denominator), and the numerical example
 *     (epsilon added after the square root; E4M3 smallest normal 2^-6).
 *   - shd-paper.top summary of arXiv 2409.12517v2 ("Scaling FP8 training to
 *     trillion-token LLMs"), method details and abstract: both Adam moments
 *     are quantized to FP8.
 *   - zyxy.net/?p=24419 (FP8 mixed-precision article), sections on FP8
 *     formats, mixed-precision strategy (FP32 master weights), strategies
 *     (dynamic range by max-abs tracking, exponent-offset adjustment,
 *     round-to-nearest) and the code example (AdamW).
 *
 * Arithmetic, per element (fp32):
 *   m  = decode(c_m) * s_m            v  = decode(c_v) * s_v
 *   m' = fma(b1, m, (1-b1)*g)         v' = fma(b2, v, (1-b2)*(g*g))
 *   p' = p*(1 - lr*wd) - lr/(1-b1^t) * m' / (sqrt(v'/(1-b2^t)) + eps)
 *   (decay_mode L2: g is replaced by fma(wd, p, g) and the factor (1 - lr*wd) by 1)
 *   s_m', s_v' chosen from max|m'| and max v' over the tensor (or over each
 *   128-element block);  c_m' = encode(m' / s_m'),  c_v' = encode(v' / s_v')
 * Encoding is OCP E4M3FN / E5M2, round-to-nearest-even, saturating at the
 * format maximum (448 / 57344).  The FP8 codes and scales are bit-exact
 * functions of the inputs; p' is within 1e-6 relative of the exact update
 * (fast sqrt / reciprocal on the device).
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative FP8ADAM_E* code; fp8adam_last_error()
 *     then gives a message (thread-local, valid until the next call on that
 *     thread).  Nothing aborts and no C++ exception crosses the ABI.
 *   - Pointers named "device" are HIP device memory of the current device;
 *     pointers named "host" are ordinary host memory.
 *   - Work is enqueued on the given stream (0 = the null stream) and runs
 *     asynchronously unless stated otherwise.
 */
#ifndef FP8ADAM_H
#define FP8ADAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8ADAM_OK 0
#define FP8ADAM_EINVAL (-1) /* bad argument (null, n <= 0, numel < 0, t < 1, beta outside [0,1), eps < 0, bad enum) */
#define FP8ADAM_EALIGN (-2) /* a device pointer is not 16-byte aligned */
#define FP8ADAM_ENOMEM (-3) /* host or device allocation failed */
#define FP8ADAM_EHIP (-4)   /* a HIP runtime call failed; the message holds hipGetErrorString */

/* FP8 storage formats (OCP): E4M3FN (bias 7, max 448, no Inf) and E5M2 (bias 15, max 57344). */
typedef enum { FP8ADAM_E4M3 = 0, FP8ADAM_E5M2 = 1 } fp8adam_format;
/* One scale per tensor, or one per contiguous run of 128 elements of the flattened tensor. */
typedef enum { FP8ADAM_SCALE_TENSOR = 0, FP8ADAM_SCALE_BLOCK128 = 1 } fp8adam_granularity;
/* POW2: smallest power of two s with amax/s <= FMAX (exponent clamped to [-126,126]).
 * AMAX: s = amax/FMAX and inv_s = FMAX/amax (s raised to 2^-126 if smaller).
 * amax = 0 or non-finite gives s = 1 in both modes. */
typedef enum { FP8ADAM_SCALE_POW2 = 0, FP8ADAM_SCALE_AMAX = 1 } fp8adam_scale_mode;
/* Master weights: fp32, or bf16 (the update is rounded to nearest-even bf16). */
typedef enum { FP8ADAM_MASTER_FP32 = 0, FP8ADAM_MASTER_BF16 = 1 } fp8adam_master;
/* How a per-tensor-scaled step is scheduled on the device.  Both give bit-identical results.
 * TWO_PASS: an amax pass over (g, m, v), then the update pass (18 bytes per fp32 parameter).
 * SPECULATIVE: one update pass that quantizes with a predicted power-of-two scale and
 *   writes the codes into the other of two code buffers (m/v and m_alt/v_alt, alternating
 *   every step); a per-tensor check then brings only the moments whose true scale differs to
 *   it: most codes just have their exponent field moved (2 bytes per element and moment), the
 *   few that cannot be moved exactly are recomputed from the gradient and the old codes (3
 *   more).  14 bytes per fp32 parameter plus that.  The prediction (see fp8adam_predictor): a
 *   probe before the pass computes the exact new amax over the parts of each tensor that held
 *   values near its amax at the step before (about 1% of the elements, 4 bytes each) and takes
 *   its scale; a tensor with too many such parts (more than 1/32 of them) takes the previous
 *   amax times its expected growth.  Needs per-tensor POW2 scales, decoupled decay (a recomputed moment is
 *   formed after p is overwritten, and coupled L2 would need the old p) and m_alt/v_alt.
 *   Steps with t < speculate_from_step - 1 run TWO_PASS in place on the current buffer; step
 *   speculate_from_step - 1 runs the amax pass and then the speculative pass with the true
 *   scales (nothing to fix up; its check lists the probe's first candidates). */
typedef enum { FP8ADAM_SCHEDULE_TWO_PASS = 0, FP8ADAM_SCHEDULE_SPECULATIVE = 1 } fp8adam_schedule;
/* How the SPECULATIVE schedule predicts a tensor's scale (results are bit-identical every
 * way; only the share of moments the fix-up moves, and the time, differ).
 * AUTO (the default): PROBE for a list of at least 2^28 elements, GROWTH for a smaller one
 *   (whose step is short enough that the probe's two extra launches cost more than they save).
 * PROBE: from the probe's exact amax over the tensor's candidate parts.
 * GROWTH: always from the previous amax times its expected growth (no probe, no list). */
typedef enum {
    FP8ADAM_PREDICT_AUTO = 0,
    FP8ADAM_PREDICT_PROBE = 1,
    FP8ADAM_PREDICT_GROWTH = 2
} fp8adam_predictor;
/* How weight_decay enters the step.
 * DECOUPLED (AdamW, the zyxy.net code example): p' = p*(1 - lr*wd) - (Adam update).
 * L2 (Adam on an L2-regularised loss: the training objective in the set-up of Theorem 1,
 *   daoxuan.cc explainer, section on why the two SwiGLU weight vectors align): the
 *   moments see g_eff = fma(wd, p, g) in fp32 with the old p, and p is not decayed
 *   separately.  With wd = 0 both are plain Adam. */
typedef enum { FP8ADAM_DECAY_DECOUPLED = 0, FP8ADAM_DECAY_L2 = 1 } fp8adam_decay_mode;
/* When the scale is chosen (per-tensor granularity).
 * JUST_IN_TIME: from this step's amax of m' and v' (codes never saturate under POW2).
 * DELAYED: delayed scaling as in the zyxy.net article (strategies: track the max-abs value;
 *   code example: a history of 16 amaxes, margin 0, interval 1, MAX of the history).  Step t
 *   quantizes with the scale of max(history) * 2^margin, saturating what no longer fits
 *   (counted as saturated), in one pass over the data (14 bytes per fp32 parameter); each step
 *   then records its amax of m' and v' in slot (t-1) mod H of the tensor's amax_history.
 *   Steps with t < delayed_from_step are just in time (two passes) and also record their amax,
 *   so the history is seeded.  Needs per-tensor scales and the TWO_PASS schedule value. */
typedef enum { FP8ADAM_SCALING_JUST_IN_TIME = 0, FP8ADAM_SCALING_DELAYED = 1 } fp8adam_scaling;
/* How the moments are rounded to FP8.
 * NEAREST: round to nearest, ties to even (the zyxy.net article's strategies: the standard).
 * STOCHASTIC: stochastic rounding (same section: against the error that accumulates over many
 *   updates).  A moment value x with FP8 neighbours lo <= |x| < hi and f = (|x| - lo)/(hi - lo)
 *   rounds up iff floor(f * 2^16) + r >= 2^16, r = 16 random bits; saturation as for NEAREST.
 *   The bits come from Philox4x32-10 (Salmon et al., SC 2011) with key = seed and counter
 *   (i/4 low 32 bits, i/4 high 32 bits, t, tensor index) for element i of a tensor: word i mod 4,
 *   low 16 bits for m, high 16 bits for v.  Deterministic for a given seed and t; every
 *   schedule gives the same codes. */
typedef enum { FP8ADAM_ROUND_NEAREST = 0, FP8ADAM_ROUND_STOCHASTIC = 1 } fp8adam_rounding;

typedef struct {
    int32_t m_format;      /* fp8adam_format of the first moment (default E4M3) */
    int32_t v_format;      /* fp8adam_format of the second moment (default E5M2) */
    int32_t granularity;   /* fp8adam_granularity */
    int32_t scale_mode;    /* fp8adam_scale_mode */
    int32_t master;        /* fp8adam_master */
    int32_t collect_stats; /* nonzero: count underflow / saturation / non-finite per tensor */
    int32_t schedule;      /* fp8adam_schedule (block granularity is always one pass) */
    int32_t speculate_from_step; /* first t of the speculative schedule; <= 0 means 4 */
    int32_t decay_mode;    /* fp8adam_decay_mode */
    int32_t scaling;       /* fp8adam_scaling */
    int32_t amax_history_len;  /* DELAYED: H in [1, 1024]; <= 0 means 16 */
    int32_t margin;            /* DELAYED: scale chosen for max(history) * 2^margin, margin in [0, 64] */
    int32_t delayed_from_step; /* DELAYED: first t quantized with the delayed scale; <= 0 means 2 */
    int32_t rounding;          /* fp8adam_rounding */
    uint64_t seed;             /* STOCHASTIC: the generator's key */
    int32_t zero_state;        /* nonzero: fp8adam_init writes a fresh optimizer state into the
                                  caller's buffers (m, v codes 0; every scale 1.0; the amax
                                  history 0), so they may start with any content; 0: the caller
                                  provides the state (fresh, or restored from a checkpoint) */
    int32_t predictor;         /* SPECULATIVE: fp8adam_predictor (ignored otherwise) */
} fp8adam_config;

/* One parameter tensor.  All pointers are device pointers owned by the caller,
 * 16-byte aligned, and must stay valid and unchanged until fp8adam_destroy.
 *   param   : numel fp32 (or bf16) master weights, updated in place
 *   grad    : numel bf16 gradients, read only
 *   m, v    : numel FP8 codes of the moments, updated in place
 *   m_scale : 1 float (tensor granularity) or ceil(numel/128) floats (block), in place
 *   v_scale : same as m_scale, for v
 *   m_alt, v_alt : numel bytes each, the second code buffers of the speculative
 *             schedule (ignored, may be NULL, otherwise); fp8adam_current_buffer
 *             tells which pair holds the moments after a step
 *   amax_history : DELAYED scaling only (else ignored, may be NULL): 2*H floats, 4-byte
 *             aligned, the amax history of m (first H) then of v; read and updated by
 *             every step.  Part of the optimizer state (checkpoint it with the codes).
 * The state before the first step is all-zero codes with scales 1.0 (and a zero history);
 * fp8adam_config.zero_state asks fp8adam_init to write it.  An empty tensor (numel 0) needs
 * no pointers; with zero_state and tensor granularity its m_scale / v_scale, if not NULL,
 * still receive 1.0. */
typedef struct {
    void *param;
    const void *grad;
    uint8_t *m;
    uint8_t *v;
    float *m_scale;
    float *v_scale;
    int64_t numel;
    uint8_t *m_alt;
    uint8_t *v_alt;
    float *amax_history;
} fp8adam_tensor;

/* Hyperparameters of one step: the quantities of Adam as the daoxuan.cc explainer describes
 * it (section on why Adam keeps m in E4M3 and v in E5M2, subsection on the asymmetry of the
 * update: m and v moving averages of g and g^2, m in the numerator times the learning rate,
 * the square root of v in the denominator; subsection with the numerical example: eps added
 * after the square root) and the decoupled weight decay of the AdamW call in the zyxy.net
 * article's code example.  step is the 1-based t used for bias correction (1 - beta^t);
 * lr and weight_decay finite; beta1, beta2 in [0, 1); eps >= 0. */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} fp8adam_hparams;

/* Per-tensor diagnostics of the most recent step: the max-abs tracking and the
 * underflow / overflow monitoring of the zyxy.net article's strategies section (dynamic
 * range from the tracked max-abs value; small values lost to zero, large ones saturating),
 * and the daoxuan.cc explainer's numerical example (a small v stored as zero in E4M3).
 * In block mode amax_* is the max over the tensor's blocks and scale_* the largest
 * block scale; both need collect_stats in block mode (else 0). */
typedef struct {
    float amax_m, amax_v;   /* max |m'| and max v' over the tensor */
    float scale_m, scale_v; /* new scales */
    int64_t underflow_m, underflow_v; /* nonzero moment stored as a +-0 code */
    int64_t saturated_m, saturated_v; /* |x * inv_s| > FMAX before clamping */
    int64_t nonfinite;                /* elements with a non-finite m' or v' */
    int64_t requantized;              /* speculative schedule: (element, moment) pairs brought to the
                                         true scale because the predicted one was off: numel per
                                         mispredicted moment (0, numel or 2 numel); else 0 */
    int64_t probed;                   /* speculative schedule: elements whose gradient and codes the
                                         scale probe read before the pass (the parts that held values
                                         near the tensor's amax at the step before); else 0 */
} fp8adam_stats_t;

typedef struct fp8adam_ctx fp8adam_ctx;

/* Quantizing the Adam moments of every tensor of a model (shd-paper.top summary, method
 * details: both moments in FP8) as one multi-tensor step.
 * Build a context over n tensors: validates them (EINVAL / EALIGN), builds the
 * multi-tensor chunk table and the per-tensor descriptors on the device
 * (allocates; ENOMEM / EHIP), and synchronizes `stream` before returning.
 * *out receives the handle (NULL on failure).  The device is the current one.
 * A context holds at most 16,777,208 * 1024 (about 1.7e10) elements, each tensor
 * counted in whole chunks, so that every launch fits one grid dimension; a
 * larger list is split over several contexts (EINVAL otherwise). */
int fp8adam_init(fp8adam_ctx **out, const fp8adam_tensor *tensors, int32_t n,
                 const fp8adam_config *cfg, hipStream_t stream);

/* The per-element arithmetic at the top of this header (dequantize, Adam/AdamW update from
 * the daoxuan.cc explainer's statement of the update, new amax, requantize with saturation).
 * One optimizer step over every tensor of the context, enqueued on `stream`
 * and returning at once.  Validates hp (EINVAL).  Allocates nothing.  After the
 * stream reaches the end of the step each tensor's (codes, scale) pair is
 * consistent.  Steps of one context must not overlap.  `stream` must belong to the
 * context's device (EINVAL otherwise; the same holds for fp8adam_step_amp and
 * fp8adam_stats). */
int fp8adam_step(fp8adam_ctx *ctx, const fp8adam_hparams *hp, hipStream_t stream);

/* ---- loss scaling, non-finite skip and global-norm clipping, fused ----
 * The zyxy.net article's strategies section scales the loss, grows the scale after a
 * run of overflow-free steps and shrinks it on overflow, and clips gradients; its code
 * example unscales the gradients, clips them to a global norm of 1.0 and skips the
 * optimizer step when they overflowed.  fp8adam_step_amp does all of it on the device,
 * with no host synchronization:
 *   1. one read of every gradient (2 bytes per parameter): the sum of squares in fp64 and
 *      the count of Inf/NaN elements, over every tensor of the context;
 *   2. one work-group takes the decision, like torch.amp.GradScaler with a fused optimizer:
 *      any Inf/NaN -> the step is skipped (parameters, codes, scales and history unchanged),
 *      scale *= backoff_factor, growth_tracker = 0; otherwise norm = ||g|| / scale,
 *      clip_coef = min(1, max_norm / (norm + 1e-6)) in fp32 (1 if max_norm <= 0),
 *      grad_factor = clip_coef * fp32(1/scale), step += 1 and the growth rule (after
 *      growth_interval taken steps, scale *= growth_factor if that stays finite);
 *   3. the step as fp8adam_step, with every bf16 gradient multiplied by grad_factor and the
 *      bias corrections of t = state.step (skipped steps are not counted); with delayed
 *      scaling this t also picks the history slot, (t-1) mod H.
 * The sum of squares is deterministic (fixed reduction order). */
typedef struct {
    float scale;             /* in/out: loss scale S (the gradients are those of loss * S) */
    int32_t growth_tracker;  /* in/out: taken steps since the scale last changed */
    int64_t step;            /* in/out: Adam steps taken so far (start at 0) */
    int32_t found_inf;       /* out: 1 if the last call found an Inf/NaN gradient and skipped */
    float grad_norm;         /* out: ||g|| / S over every tensor (NaN when skipped) */
    float clip_coef;         /* out: the clip coefficient (1: not clipped) */
    float grad_factor;       /* out: clip_coef / S, the factor applied to every gradient */
} fp8adam_amp_state;         /* device memory, caller-owned, 8-byte aligned, 32 bytes */

typedef struct {
    float max_norm;          /* > 0: clip the global norm to it; <= 0: no clipping */
    float growth_factor;     /* > 1 (torch's default 2) */
    float backoff_factor;    /* in (0, 1) (default 0.5) */
    int32_t growth_interval; /* >= 1 (default 2000) */
} fp8adam_amp_config;

/* One step with loss scaling and clipping, enqueued on `stream`; state is device memory
 * read and written by the step.  hp->step is the caller's call count and only chooses the
 * schedule (speculative / delayed from which call); the bias correction uses state.step.
 * Returns EINVAL for a bad hp, amp or state (null, misaligned) before enqueuing anything. */
int fp8adam_step_amp(fp8adam_ctx *ctx, const fp8adam_hparams *hp, const fp8adam_amp_config *amp,
                     fp8adam_amp_state *state, hipStream_t stream);

/* ---- allocation-free step ----
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  One step over a tensor list without a context: the
 * same kernels, and so the same results bit for bit, as fp8adam_init (zero_state 0) followed
 * by one fp8adam_step, for the TWO_PASS schedule with just-in-time scaling and stats off, in
 * either granularity, scale mode, master dtype, decay mode and rounding.  Arguments as for
 * fp8adam_init and fp8adam_step; the caller provides the state (codes and scales).  Calls
 * nothing that allocates: what the step needs beyond the caller's buffers (descriptors, chunk
 * table, amax partials, staged scales) lives in one file-scope device array of
 * FP8ADAM_NOALLOC_SCRATCH_BYTES bytes, which every GPU the library runs on holds until the
 * process ends; the descriptors reach it through a kernel's arguments (no host-to-device copy).
 * Limits: n <= FP8ADAM_NOALLOC_MAX_TENSORS and the element limit of a context (about 1.7e10);
 * the chunk table holds FP8ADAM_NOALLOC_MAX_CHUNKS chunks, which any such list fits once its
 * chunks grow (up to 2^18 elements; the results do not depend on the chunk size).  Beyond the
 * limits, or for another schedule, scaling, stats or zero_state: EINVAL before anything is
 * enqueued.  The stream must belong to the current device.  Every call on one GPU shares
 * that GPU's array and leaves its contents behind (each call rewrites what it reads), so calls
 * that overlap on one GPU (on different streams, or from several threads) race: order them. */
#define FP8ADAM_NOALLOC_MAX_TENSORS 4096
#define FP8ADAM_NOALLOC_MAX_CHUNKS 131072
#define FP8ADAM_NOALLOC_SCRATCH_BYTES 2015232
int fp8adam_step_noalloc(const fp8adam_tensor *tensors, int32_t n, const fp8adam_config *cfg,
                         const fp8adam_hparams *hp, hipStream_t stream);

/* The diagnostics of fp8adam_stats_t (the zyxy.net article, strategies: tracked max-abs,
 * underflow and overflow).
 * Copy the diagnostics of the last step into out_host[0..n) (n = the context's
 * tensor count; EINVAL otherwise).  Synchronizes `stream`. */
int fp8adam_stats(fp8adam_ctx *ctx, fp8adam_stats_t *out_host, int32_t n, hipStream_t stream);

/* Free the context (device buffers and events).  NULL is ignored.  The caller
 * must make sure no step of this context is still running. */
void fp8adam_destroy(fp8adam_ctx *ctx);

/* Message for the last nonzero return on this thread ("" if none). */
const char *fp8adam_last_error(void);

/* ---- device codec (the same converts the step uses), for verification ---- */

/* out[i] = encode_fmt(x[i]) for i < n.  x, out: device.  RNE, saturating. */
int fp8adam_encode(int32_t fmt, const float *x, uint8_t *out, int64_t n, hipStream_t stream);
/* out[i] = decode_fmt(codes[i]) for i < n.  codes, out: device.  Exact. */
int fp8adam_decode(int32_t fmt, const uint8_t *codes, float *out, int64_t n, hipStream_t stream);
/* out[i] = encode_fmt(fp32 with bit pattern start + i), i < count, count <= 2^32 - start.
 * out: device, count bytes. */
int fp8adam_encode_bits_range(int32_t fmt, uint32_t start, int64_t count, uint8_t *out,
                              hipStream_t stream);

/* out[i] = stochastic-rounding encode of the fp32 with bit pattern start + i, with the 16
 * random bits r16 (< 2^16) for every value: the rounding FP8ADAM_ROUND_STOCHASTIC applies to
 * each moment value.  count <= 2^32 - start; out: device, count bytes. */
int fp8adam_encode_sr_bits_range(int32_t fmt, uint32_t start, int64_t count, uint32_t r16, uint8_t *out,
                                 hipStream_t stream);

/* out[i] = stochastic-rounding encode of x[i] with its own 16 random bits r16[i], i < n:
 * the same rounding as fp8adam_encode_sr_bits_range (rounding up iff
 * floor(f * 2^16) + r16 >= 2^16, f the position of |x| between its FP8 neighbours,
 * saturating at +-FMAX; the zyxy.net FP8 article, strategies section, names stochastic
 * rounding).  x (float), r16 (uint16), out (n bytes): device, owned by the caller.
 * NaN inputs give a NaN code of either sign.  EINVAL for a bad format, n < 0 or a
 * NULL pointer with n > 0. */
int fp8adam_encode_sr(int32_t fmt, const float *x, const uint16_t *r16, uint8_t *out, int64_t n,
                      hipStream_t stream);

/* ---- measurement ---- */

/* dst[0..bytes) = src[0..bytes) on `stream` with the step kernels' access pattern (16-byte
 * non-temporal loads and stores, four in flight per lane, 16 KiB per work-group): a plain
 * streaming copy whose rate is the practical read + write ceiling the step's kernels are
 * compared with.  src, dst: device, 16-byte aligned, not overlapping; bytes a multiple of
 * 16 (EINVAL otherwise, EALIGN for misaligned pointers). */
int fp8adam_stream_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

/* Read read_bytes of src and write write_bytes of dst on `stream` with fp8adam_stream_copy's
 * access pattern: dst[i] = src[i] where both sizes cover byte i, 0 where only write_bytes
 * does.  write_bytes = 0 gives a read-only stream and read_bytes = 0 a write-only one: the
 * two rates that bound any mix of reads and writes (such as the step's).  src, dst: device,
 * 16-byte aligned, not overlapping (either may be NULL where its size is 0); sizes
 * non-negative multiples of 16 (EINVAL otherwise, EALIGN for misaligned pointers). */
int fp8adam_stream_rw(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, hipStream_t stream);

/* The update pass's access pattern with trivial arithmetic, over n elements: reads p (n fp32
 * weights, or bf16 with master FP8ADAM_MASTER_BF16), g (n bf16), m_in and v_in (n bytes each),
 * writes p in place (p += g) and m_out, v_out (n bytes each): 14 bytes per element (10 with a
 * bf16 master), with the pass's buffer instructions, non-temporal cache policy, one-shot
 * work-groups (1024 elements; 2048 with a bf16 master) and XCD order.  Its rate is the
 * practical ceiling of the pass's byte mix (4 read streams, 3 write streams) on the GPU it runs
 * on.  n: a multiple of the work-group's elements (EINVAL otherwise); device pointers, 16-byte
 * aligned (EALIGN), caller-owned; m_out and v_out must not overlap the inputs. */
int fp8adam_stream_mix(int32_t master, void *p, const void *g, const void *m_in, const void *v_in,
                       void *m_out, void *v_out, int64_t n, hipStream_t stream);

/* Enable (1) or disable (0) per-kernel timing of every launch of later steps:
 * each timed kernel is launched with two HIP events (hipExtLaunchKernel), which
 * the runtime stamps with the dispatch's own start and end (creates the
 * events; may allocate).  Timing records at most 4096 launches between two
 * fp8adam_kernel_times calls; launches into a stream under graph capture are
 * not timed. */
int fp8adam_set_timing(fp8adam_ctx *ctx, int32_t enable);

/* As fp8adam_set_timing, for the launches of the kernel kinds whose bit is set in
 * kinds (bit k: kind k, as numbered for fp8adam_kernel_times; 0 disables timing).
 * Each timed launch still adds a gap of a few microseconds to the stream:
 * timing only the kinds of interest keeps a step's time close to its untimed
 * one. */
int fp8adam_set_timing_kinds(fp8adam_ctx *ctx, uint32_t kinds);

/* Per-kernel timing since the last call (or since timing was enabled):
 * for kernel kind k < max (0 = amax pass, 1 = update pass, 2 = scale reduction,
 * 3 = block-scaled single pass, 4 = stats reset, 5 = speculative pass,
 * 6 = speculative scale check, 7 = speculative fix-up, 8 = delayed-scaling pass,
 * 9 = delayed-scaling commit, 10 = gradient-norm pass, 11 = loss-scale decision,
 * 12 = scale preparation of the speculative and delayed passes, 13 = speculative
 * scale probe, 14 = speculative per-chunk fold of the part partials),
 * total_ms[k] and count[k].
 * Host arrays of length max.  Synchronizes the recorded events, then clears. */
int fp8adam_kernel_times(fp8adam_ctx *ctx, double *total_ms, int32_t *count, int32_t max);

/* HIP runtime version the library runs on (hipRuntimeGetVersion), in *version. */
int fp8adam_runtime_version(int32_t *version);

/* Number of chunks (work-groups of the amax pass) of the context; -1 for NULL. */
int64_t fp8adam_num_chunks(const fp8adam_ctx *ctx);

/* Which code buffers hold the moments once the steps enqueued so far have run:
 * 0 = m/v, 1 = m_alt/v_alt (only the speculative schedule alternates); -1 for NULL. */
int32_t fp8adam_current_buffer(const fp8adam_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* FP8ADAM_H */
