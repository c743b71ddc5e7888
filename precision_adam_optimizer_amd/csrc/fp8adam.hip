// fp8adam.hip -- FP8-moment Adam/AdamW step for AMD MI355X (gfx950): the C
// ABI declared in include/fp8adam.h, the loss-scaling kernels (gradient norm
// and the scaler's decision), the fresh-state kernel of zero_state, the
// allocation-free step and its file-scope scratch, the codec probes and the
// bandwidth probes (streaming copy, the update pass's byte mix).  The step
// kernels and their dispatch are in fp8adam_engine.h, instantiated in
// fp8adam_step_*.hip.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/fp8adam.h"
#include "fp8_codec.h"
#include "fp8adam_engine.h"

using namespace fp8adam;
using namespace fp8adam_engine;

namespace fp8adam_engine {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FP8ADAM_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace fp8adam_engine

namespace {

// Speculative schedule: the predicted growth of a tensor's amax from step t-1
// to step t (t >= 2; 1 at t = 1), a weighted geometric mean of two models of a
// moving average with factor beta: its mean under a steady gradient grows as
// (1 - beta^t) / (1 - beta^(t-1)); its spread under independent noise grows as
// the square root of the same ratio taken at beta^2.  Minibatch gradients are
// mostly noise, so the spread model gets weight 3/4: on recorded amax
// trajectories of the 7B, 13B and 100M lists (steps 4-23) the mispredicted
// share of (element, moment) pairs is 6.8 / 7.1 / 7.9% against 7.6 / 7.9 /
// 8.1% with equal weights; on simulated gradients with a per-element mean of
// one and of three noise standard deviations it mispredicts 7.0% and 4.0%
// (equal weights 5.8% and 2.2%, the mean model alone 5.9% and 1.2%).
__host__ __device__ inline float amax_growth(double beta, double t) {
  const double mean_prev = 1.0 - pow(beta, t - 1.0);
  const double var_prev = 1.0 - pow(beta * beta, t - 1.0);
  if (!(mean_prev > 0.0) || !(var_prev > 0.0)) return 1.0f;
  const double mean_growth = (1.0 - pow(beta, t)) / mean_prev;
  const double spread_growth = sqrt((1.0 - pow(beta * beta, t)) / var_prev);
  return (float)(pow(mean_growth, 0.25) * pow(spread_growth, 0.75));
}

// ------------------------------------------- loss scaling and clipping
//
// k_gradnorm: one work-group per chunk reads the bf16 gradients only (2 bytes
// per parameter) and writes the chunk's sum of squares in fp64 (each square is
// exact in fp64) and its count of Inf/NaN elements.  k_gradctl (one
// work-group) sums the partials in a fixed order, so the result is
// deterministic, and takes the scaler's decision: skip the step (non-finite
// gradient; the scale backs off) or run it with the gradient factor
// c / S, c = min(1, max_norm / (||g||/S + 1e-6)), and the bias corrections of
// the device-side step count, which only a taken step advances.

// Work-groups of the gradient-norm pass: a fixed grid that strides over the
// chunks, so the decision kernel sums few partials (and always in one order).
constexpr int kNormGroups = 2048;

__device__ __forceinline__ void sumsq_bf16x2(uint32_t x, double& acc, uint32_t& bad) {
  bad += ((x & 0x7F80u) == 0x7F80u) + ((x & 0x7F800000u) == 0x7F800000u);
  const double a = bf16_lo(x), b = bf16_hi(x);
  acc = __builtin_fma(a, a, acc);
  acc = __builtin_fma(b, b, acc);
}

__global__ __launch_bounds__(kThreads) void k_gradnorm(const TensorDesc* __restrict__ descs,
                                                       const int32_t* __restrict__ chunk_tid,
                                                       double* __restrict__ gpart, int chunk_log2, int64_t nchunks) {
  constexpr int kU = 4;                         // 16-byte loads in flight per lane
  constexpr int kStep = kThreads * 8;           // elements per load of the work-group
  double acc = 0.0;
  uint32_t bad = 0;
  for (int64_t w = blockIdx.x; w < nchunks; w += gridDim.x) {
    const TensorDesc d = descs[chunk_tid[w]];
    const int64_t start = (w - d.chunk0) << chunk_log2;
    const int64_t end = min(start + ((int64_t)1 << chunk_log2), d.numel);
    const int64_t gend = start + ((end - start) & ~(int64_t)7);  // whole groups of 8
    for (int64_t base = start + 8 * threadIdx.x; base < gend; base += (int64_t)kStep * kU) {
      vu4 gg[kU];
#pragma unroll
      for (int u = 0; u < kU; u++) {
        const int64_t i = base + (int64_t)u * kStep;
        if (i < gend) gg[u] = ld_stream<vu4, FP8ADAM_NT_AMAX != 0>(d.g + i);
      }
#pragma unroll
      for (int u = 0; u < kU; u++) {
        const int64_t i = base + (int64_t)u * kStep;
        if (i < gend) {
          sumsq_bf16x2(gg[u].x, acc, bad);
          sumsq_bf16x2(gg[u].y, acc, bad);
          sumsq_bf16x2(gg[u].z, acc, bad);
          sumsq_bf16x2(gg[u].w, acc, bad);
        }
      }
    }
    if (gend + threadIdx.x < end) {  // ragged tail (< 8 elements at the end of a tensor)
      const uint32_t x = ld_global<uint16_t>(d.g + gend + threadIdx.x);
      bad += (x & 0x7F80u) == 0x7F80u;
      const double a = bf16_lo(x);
      acc = __builtin_fma(a, a, acc);
    }
  }
  // fixed-order reduction: butterfly within the wave, then waves in order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    acc += __shfl_xor(acc, o);
    bad += (uint32_t)__shfl_xor((int)bad, o);
  }
  __shared__ double sacc[kThreads / 64];
  __shared__ uint32_t sbad[kThreads / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sacc[wave] = acc;
    sbad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; k++) {
      acc += sacc[k];
      bad += sbad[k];
    }
    st_global<double>(gpart + 2 * blockIdx.x, acc);
    st_global<double>(gpart + 2 * blockIdx.x + 1, (double)bad);
  }
}

__global__ __launch_bounds__(kReduceThreads) void k_gradctl(const double* __restrict__ gpart, int64_t nparts,
                                                           fp8adam_amp_state* __restrict__ st, GradCtl* __restrict__ ctl,
                                                           fp8adam_amp_config cfg, float lr, float beta1, float beta2,
                                                           int hist_len) {
  double acc = 0.0, bad = 0.0;
  for (int64_t k = threadIdx.x; k < nparts; k += kReduceThreads) {
    acc += gpart[2 * k];
    bad += gpart[2 * k + 1];
  }
  __shared__ double sacc[kReduceThreads], sbad[kReduceThreads];
  sacc[threadIdx.x] = acc;
  sbad[threadIdx.x] = bad;
  __syncthreads();
  for (int h = kReduceThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      sacc[threadIdx.x] += sacc[threadIdx.x + h];
      sbad[threadIdx.x] += sbad[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const float scale = st->scale;
  const float inv = __double2float_rn(__ddiv_rn(1.0, (double)scale));
  if (sbad[0] > 0.0) {
    st_global(&st->found_inf, 1);
    st_global(&st->grad_norm, __builtin_nanf(""));
    st_global(&st->clip_coef, 1.0f);
    st_global(&st->grad_factor, 0.0f);
    st_global(&st->scale, __fmul_rn(scale, cfg.backoff_factor));
    st_global(&st->growth_tracker, 0);
    st_global(&ctl->skip, 1);
    return;
  }
  const double norm = __dmul_rn(__dsqrt_rn(sacc[0]), (double)inv);
  double cc = 1.0;
  if (cfg.max_norm > 0.0f) {
    cc = __ddiv_rn((double)cfg.max_norm, __dadd_rn(norm, 1e-6));
    if (cc > 1.0) cc = 1.0;
  }
  const float c32 = __double2float_rn(cc);
  const float gfac = __fmul_rn(c32, inv);
  const int64_t t = st->step + 1;
  st_global(&st->found_inf, 0);
  st_global(&st->grad_norm, __double2float_rn(norm));
  st_global(&st->clip_coef, c32);
  st_global(&st->grad_factor, gfac);
  st_global(&st->step, t);
  const int32_t next = st->growth_tracker + 1;
  if (next == cfg.growth_interval) {
    const float grown = __fmul_rn(scale, cfg.growth_factor);
    if (isfinite(grown)) st_global(&st->scale, grown);
    st_global(&st->growth_tracker, 0);
  } else {
    st_global(&st->growth_tracker, next);
  }
  const double bc1 = 1.0 - pow((double)beta1, (double)t), bc2 = 1.0 - pow((double)beta2, (double)t);
  st_global(&ctl->skip, 0);
  st_global(&ctl->gfac, gfac);
  st_global(&ctl->step_size, (float)((double)lr / bc1));
  st_global(&ctl->inv_bc2, (float)(1.0 / bc2));
  st_global(&ctl->grow_m, amax_growth((double)beta1, (double)t));
  st_global(&ctl->grow_v, amax_growth((double)beta2, (double)t));
  st_global(&ctl->hist_slot, hist_len > 0 ? (int32_t)((t - 1) % hist_len) : 0);
  st_global(&ctl->t, (uint32_t)t);
}

// ------------------------------------------------------------- codec probes

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_encode(const float* __restrict__ x, uint8_t* __restrict__ out,
                                                     int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n && (((uintptr_t)(x + i) | (uintptr_t)(out + i)) & 3) == 0 &&
        ((uintptr_t)(x + i) & 15) == 0) {
      const float4 v = *reinterpret_cast<const float4*>(x + i);
      *reinterpret_cast<uint32_t*>(out + i) = encode4<FMT>(v.x, v.y, v.z, v.w);
    } else {
      for (int64_t k = i; k < n && k < i + 4; k++) out[k] = (uint8_t)encode1<FMT>(x[k]);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_encode_bits(uint32_t start, int64_t count,
                                                          uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < count; i += stride) {
    const uint32_t b = start + (uint32_t)i;
    if (i + 4 <= count && (((uintptr_t)(out + i)) & 3) == 0) {
      *reinterpret_cast<uint32_t*>(out + i) =
          encode4<FMT>(__uint_as_float(b), __uint_as_float(b + 1u), __uint_as_float(b + 2u), __uint_as_float(b + 3u));
    } else {
      for (int64_t k = i; k < count && k < i + 4; k++)
        out[k] = (uint8_t)encode1<FMT>(__uint_as_float(start + (uint32_t)k));
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_encode_sr_bits(uint32_t start, int64_t count, uint32_t r16,
                                                             uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  const uint32_t r[4] = {r16, r16, r16, r16};
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < count; i += stride) {
    const uint32_t b = start + (uint32_t)i;
    if (i + 4 <= count && (((uintptr_t)(out + i)) & 3) == 0) {
      *reinterpret_cast<uint32_t*>(out + i) = encode4_sr<FMT>(__uint_as_float(b), __uint_as_float(b + 1u),
                                                              __uint_as_float(b + 2u), __uint_as_float(b + 3u), r);
    } else {
      for (int64_t k = i; k < count && k < i + 4; k++)
        out[k] = (uint8_t)(encode4_sr<FMT>(__uint_as_float(start + (uint32_t)k), 0.0f, 0.0f, 0.0f, r) & 0xFFu);
    }
  }
}

// Streaming copy with the step kernels' access pattern (16-byte non-temporal
// loads and stores, four per lane in flight, 16 KiB per one-shot work-group):
// the box's practical ceiling for a read + write stream, measured beside the step.
__global__ __launch_bounds__(kThreads) void k_stream_copy(const vu4* __restrict__ src, vu4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * (4 * kThreads) + threadIdx.x;
  vu4 x[4];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n16) x[u] = ld_stream<vu4, true>(src + i);
  }
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n16) st_stream<vu4, true>(dst + i, x[u]);
  }
}

// A read stream and a write stream with k_stream_copy's access pattern:
// work-group b covers 16-byte elements [1024 b, 1024 b + 1024); it reads those
// below n_read and writes those below n_write (src's value where it was read,
// else zero).  With n_write = 0 it is a read-only stream (each loaded value is
// consumed by an empty asm statement, so the loads are neither dropped nor left
// in flight when the wave ends), with n_read = 0 a write-only one: the two rates
// any mix of reads and writes is measured against.  A work-group whose whole
// range lies below a size issues its four accesses per lane unconditionally,
// all loads before the first wait.
__global__ __launch_bounds__(kThreads) void k_stream_rw(const vu4* __restrict__ src, int64_t n_read,
                                                        vu4* __restrict__ dst, int64_t n_write) {
  const int64_t first = (int64_t)blockIdx.x * (4 * kThreads);
  const int64_t base = first + threadIdx.x;
  vu4 x[4];
  if (first + 4 * kThreads <= n_read) {  // uniform
#pragma unroll
    for (int u = 0; u < 4; u++) x[u] = ld_stream<vu4, true>(src + base + (int64_t)u * kThreads);
#pragma unroll
    for (int u = 0; u < 4; u++) asm volatile("" ::"v"(x[u].x), "v"(x[u].y), "v"(x[u].z), "v"(x[u].w));
  } else {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int64_t i = base + (int64_t)u * kThreads;
      x[u] = vu4{0u, 0u, 0u, 0u};
      if (i < n_read) {
        x[u] = ld_stream<vu4, true>(src + i);
        asm volatile("" ::"v"(x[u].x), "v"(x[u].y), "v"(x[u].z), "v"(x[u].w));
      }
    }
  }
  if (first + 4 * kThreads <= n_write) {  // uniform
#pragma unroll
    for (int u = 0; u < 4; u++) st_stream<vu4, true>(dst + base + (int64_t)u * kThreads, x[u]);
  } else {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int64_t i = base + (int64_t)u * kThreads;
      if (i < n_write) st_stream<vu4, true>(dst + i, x[u]);
    }
  }
}

// The update pass's byte stream with trivial arithmetic (p += g, codes xor g):
// per group of four elements it reads the weights (16 bytes fp32 / 8 bf16),
// the gradients (8) and two code words (4 each), writes the weights back in
// place and two code words to other buffers, with the pass's buffer
// instructions, cache policy, one-shot work-group shape and XCD order.  Its
// rate is the practical ceiling for the pass's access pattern on the GPU it
// runs on.
template <bool BF16P>
__global__ __launch_bounds__(kThreads) void k_stream_mix(void* p, const uint16_t* __restrict__ g,
                                                         const uint8_t* __restrict__ m, const uint8_t* __restrict__ v,
                                                         uint8_t* __restrict__ m_out, uint8_t* __restrict__ v_out,
                                                         int64_t nparts) {
  const int64_t w = work_index<kXcdStreams>(nparts);
  if (w < 0) return;
  constexpr int PL = upd_part_log2<BF16P>();
  constexpr int64_t kLen = (int64_t)1 << PL;
  const int64_t start = w << PL;
  const TensorDesc d{p, g, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr};
  const PartBufs B = part_bufs<BF16P>(d, m, v, start, kLen);
  const Rsrc bdm = rsrc(m_out + start, kLen), bdv = rsrc(v_out + start, kLen);
  for (uint32_t o = kGroup * threadIdx.x; o < (uint32_t)kLen; o += kSubTile) {
    Group G;
    load_group_buf<BF16P>(B, o, G, true);
    float x[4];
    unpack_p<BF16P>(G, x);
    x[0] += bf16_lo(G.g.x);
    x[1] += bf16_hi(G.g.x);
    x[2] += bf16_lo(G.g.y);
    x[3] += bf16_hi(G.g.y);
    store_group_buf<BF16P>(B.p, bdm, bdv, o, x, G.cm ^ G.g.x, G.cv ^ G.g.y);
  }
}

// A fresh optimizer state's scales and history (fp8adam_config.zero_state): one
// work-group per tensor writes 1.0 into every scale slot of m and v and zeroes
// the 2H-entry amax history; the codes are cleared with a memset.
__global__ __launch_bounds__(kThreads) void k_fresh_state(const TensorDesc* __restrict__ descs, int block, int hist2) {
  const TensorDesc d = descs[blockIdx.x];
  const int64_t ns = block ? (d.numel + kBlock - 1) / kBlock : 1;
  for (int64_t i = threadIdx.x; i < ns; i += kThreads) {
    if (d.sm) st_global<float>(d.sm + i, 1.0f);
    if (d.sv) st_global<float>(d.sv + i, 1.0f);
  }
  if (d.hist)
    for (int j = threadIdx.x; j < hist2; j += kThreads) st_global<float>(d.hist + j, 0.0f);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_encode_sr(const float* __restrict__ x, const uint16_t* __restrict__ r16,
                                                        uint8_t* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t r[4] = {(uint32_t)r16[i], 0u, 0u, 0u};
    out[i] = (uint8_t)(encode4_sr<FMT>(x[i], 0.0f, 0.0f, 0.0f, r) & 0xFFu);
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_decode(const uint8_t* __restrict__ codes, float* __restrict__ out,
                                                     int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = decode1<FMT>(codes[i]);
}

bool valid_fmt(int32_t f) { return f == FP8ADAM_E4M3 || f == FP8ADAM_E5M2; }

int check_aligned(const void* p, const char* what, int32_t t) {
  if (((uintptr_t)p & 15u) != 0)
    return fail(FP8ADAM_EALIGN, std::string(what) + " of tensor " + std::to_string(t) + " is not 16-byte aligned");
  return 0;
}

// Every launch must fit one grid dimension of at most 2^32 - 1 work-items:
// kMaxGroups work-groups of kThreads (XCD-ordered grids round up to 8), and the
// widest grid has one work-group per 2^min(kPartLog2, kUPartLog2Min) elements of
// every chunk.  That caps one step at about 1.7e10 elements; larger lists are
// split over several contexts.
constexpr int64_t kMaxGroups = ((int64_t)UINT32_MAX / kThreads) & ~(int64_t)7;
constexpr int kNarrowPartLog2 = kPartLog2 < kUPartLog2Min ? kPartLog2 : kUPartLog2Min;
constexpr int64_t kMaxElements = kMaxGroups << kNarrowPartLog2;

// The config's enums and the combinations the step supports (fp8adam_init and
// fp8adam_step_noalloc).
int check_config(const fp8adam_config* cfg) {
  if (!valid_fmt(cfg->m_format) || !valid_fmt(cfg->v_format))
    return fail(FP8ADAM_EINVAL, "m_format / v_format must be FP8ADAM_E4M3 or FP8ADAM_E5M2");
  if (cfg->granularity != FP8ADAM_SCALE_TENSOR && cfg->granularity != FP8ADAM_SCALE_BLOCK128)
    return fail(FP8ADAM_EINVAL, "bad granularity");
  if (cfg->scale_mode != FP8ADAM_SCALE_POW2 && cfg->scale_mode != FP8ADAM_SCALE_AMAX)
    return fail(FP8ADAM_EINVAL, "bad scale_mode");
  if (cfg->master != FP8ADAM_MASTER_FP32 && cfg->master != FP8ADAM_MASTER_BF16)
    return fail(FP8ADAM_EINVAL, "bad master dtype");
  if (cfg->schedule != FP8ADAM_SCHEDULE_TWO_PASS && cfg->schedule != FP8ADAM_SCHEDULE_SPECULATIVE)
    return fail(FP8ADAM_EINVAL, "bad schedule");
  if (cfg->decay_mode != FP8ADAM_DECAY_DECOUPLED && cfg->decay_mode != FP8ADAM_DECAY_L2)
    return fail(FP8ADAM_EINVAL, "bad decay_mode");
  if (cfg->rounding != FP8ADAM_ROUND_NEAREST && cfg->rounding != FP8ADAM_ROUND_STOCHASTIC)
    return fail(FP8ADAM_EINVAL, "bad rounding");
  if (cfg->predictor != FP8ADAM_PREDICT_AUTO && cfg->predictor != FP8ADAM_PREDICT_PROBE &&
      cfg->predictor != FP8ADAM_PREDICT_GROWTH)
    return fail(FP8ADAM_EINVAL, "bad predictor");
  const bool spec = cfg->schedule == FP8ADAM_SCHEDULE_SPECULATIVE;
  if (spec && (cfg->granularity != FP8ADAM_SCALE_TENSOR || cfg->scale_mode != FP8ADAM_SCALE_POW2))
    return fail(FP8ADAM_EINVAL, "the speculative schedule needs per-tensor POW2 scales");
  if (spec && cfg->decay_mode == FP8ADAM_DECAY_L2)
    return fail(FP8ADAM_EINVAL, "the speculative schedule cannot be combined with coupled L2 decay");
  if (cfg->scaling != FP8ADAM_SCALING_JUST_IN_TIME && cfg->scaling != FP8ADAM_SCALING_DELAYED)
    return fail(FP8ADAM_EINVAL, "bad scaling");
  const bool delayed = cfg->scaling == FP8ADAM_SCALING_DELAYED;
  const int hist_len = cfg->amax_history_len > 0 ? cfg->amax_history_len : 16;
  if (delayed) {
    if (cfg->granularity != FP8ADAM_SCALE_TENSOR || spec)
      return fail(FP8ADAM_EINVAL, "delayed scaling needs per-tensor scales and the TWO_PASS schedule value");
    if (hist_len > 1024) return fail(FP8ADAM_EINVAL, "amax_history_len must be at most 1024");
    if (cfg->margin < 0 || cfg->margin > 64) return fail(FP8ADAM_EINVAL, "margin must lie in [0, 64]");
  }
  return 0;
}

// One tensor's pointers and their alignment (nothing to check for an empty tensor).
int check_tensor(const fp8adam_tensor& T, int32_t t, bool delayed, bool spec) {
  if (T.numel < 0) return fail(FP8ADAM_EINVAL, "numel of tensor " + std::to_string(t) + " is negative");
  if (T.numel == 0) return 0;
  if (!T.param || !T.grad || !T.m || !T.v || !T.m_scale || !T.v_scale)
    return fail(FP8ADAM_EINVAL, "null pointer in tensor " + std::to_string(t));
  if (int r = check_aligned(T.param, "param", t)) return r;
  if (int r = check_aligned(T.grad, "grad", t)) return r;
  if (int r = check_aligned(T.m, "m", t)) return r;
  if (int r = check_aligned(T.v, "v", t)) return r;
  if (((uintptr_t)T.m_scale & 3u) || ((uintptr_t)T.v_scale & 3u))
    return fail(FP8ADAM_EALIGN, "scale pointer of tensor " + std::to_string(t) + " is not 4-byte aligned");
  if (delayed) {
    if (!T.amax_history)
      return fail(FP8ADAM_EINVAL, "delayed scaling needs amax_history (tensor " + std::to_string(t) + ")");
    if ((uintptr_t)T.amax_history & 3u)
      return fail(FP8ADAM_EALIGN, "amax_history of tensor " + std::to_string(t) + " is not 4-byte aligned");
  }
  if (spec) {
    if (!T.m_alt || !T.v_alt)
      return fail(FP8ADAM_EINVAL, "the speculative schedule needs m_alt and v_alt (tensor " + std::to_string(t) + ")");
    if (int r = check_aligned(T.m_alt, "m_alt", t)) return r;
    if (int r = check_aligned(T.v_alt, "v_alt", t)) return r;
  }
  return 0;
}

void free_ctx(fp8adam_ctx* c) {
  if (!c) return;
  if (c->d_desc) (void)hipFree(c->d_desc);
  if (c->d_chunk_tid) (void)hipFree(c->d_chunk_tid);
  if (c->d_amax) (void)hipFree(c->d_amax);
  if (c->d_partial) (void)hipFree(c->d_partial);
  if (c->d_part_amax) (void)hipFree(c->d_part_amax);
  if (c->d_flags) (void)hipFree(c->d_flags);
  if (c->d_fix_count) (void)hipFree(c->d_fix_count);
  if (c->d_fix_list) (void)hipFree(c->d_fix_list);
  if (c->d_cand_count) (void)hipFree(c->d_cand_count);
  if (c->d_cand_work) (void)hipFree(c->d_cand_work);
  if (c->d_cand_n) (void)hipFree(c->d_cand_n);
  if (c->d_cand_len) (void)hipFree(c->d_cand_len);
  if (c->d_lb) (void)hipFree(c->d_lb);
  if (c->d_probed) (void)hipFree(c->d_probed);
  if (c->d_old_scale) (void)hipFree(c->d_old_scale);
  if (c->d_counters) (void)hipFree(c->d_counters);
  if (c->d_gpart) (void)hipFree(c->d_gpart);
  if (c->d_gctl) (void)hipFree(c->d_gctl);
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  delete c;
}

int64_t norm_groups(const fp8adam_ctx* c) { return std::min<int64_t>(c->nchunks, kNormGroups); }

void launch_gradnorm(fp8adam_ctx* c, hipStream_t s) {
  launch_k(c, k_gradnorm, dim3((unsigned)norm_groups(c)), dim3(kThreads), s, descs_of(c, c->cur), c->d_chunk_tid,
           c->d_gpart, c->chunk_log2, c->nchunks);
}

void launch_gradctl(fp8adam_ctx* c, const fp8adam_amp_config& amp, fp8adam_amp_state* state,
                    const fp8adam_hparams& hp, hipStream_t s) {
  launch_k(c, k_gradctl, dim3(1), dim3(kReduceThreads), s, c->d_gpart, norm_groups(c), state, c->d_gctl, amp, hp.lr,
           hp.beta1, hp.beta2, c->hist_len);
}

int run_step(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  const int mf = c->cfg.m_format, vf = c->cfg.v_format;
  if (mf == 0 && vf == 1) return run_step_f<0, 1>(c, k, t, s);
  if (mf == 1 && vf == 1) return run_step_f<1, 1>(c, k, t, s);
  if (mf == 1 && vf == 0) return run_step_f<1, 0>(c, k, t, s);
  return run_step_f<0, 0>(c, k, t, s);
}

unsigned probe_grid(int64_t n, int per_thread) {
  const int64_t blocks = (n + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 65536));
}

}  // namespace


// ------------------------------------------------ allocation-free step: scratch
//
// fp8adam_step_noalloc keeps what the two-pass step needs beyond the caller's
// buffers in one file-scope device array, `scratch`: the tensor descriptors,
// the chunk table, the per-chunk amax partials, the per-tensor amax, the staged
// old scales and the flags.  Every call writes each of them before reading it
// (descriptors and chunk table by k_noalloc_setup, partials by the amax pass,
// amax, old scales and flags by the reduction), so nothing is cleared between
// calls.  In host code the array's name is only a host-side stand-in: each
// device's copy has its own address, looked up with hipGetSymbolAddress once
// per device (with that device current), and that address is what the kernels
// receive.

namespace {

constexpr int64_t kNaMaxTensors = FP8ADAM_NOALLOC_MAX_TENSORS;
constexpr int64_t kNaMaxChunks = FP8ADAM_NOALLOC_MAX_CHUNKS;
// Chunks grow (up to 2^18 elements) until the table fits: any list within kMaxElements
// then needs at most kMaxElements / 2^18 + kNaMaxTensors chunks.
constexpr int kNaMaxChunkLog2 = 18;
constexpr int kSetupBatch = 32;      // descriptors per set-up launch, passed by value (2.3 KB)

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr size_t kNaDesc = 0;
constexpr size_t kNaChunkTid = align256(kNaDesc + sizeof(TensorDesc) * kNaMaxTensors);
constexpr size_t kNaPartial = align256(kNaChunkTid + sizeof(int32_t) * kNaMaxChunks);
constexpr size_t kNaAmax = align256(kNaPartial + sizeof(uint2) * kNaMaxChunks);
constexpr size_t kNaOldScale = align256(kNaAmax + sizeof(uint32_t) * 4 * kNaMaxTensors);
constexpr size_t kNaFlags = align256(kNaOldScale + sizeof(float) * 4 * kNaMaxTensors);
constexpr size_t kNaBytes = align256(kNaFlags + sizeof(int32_t) * kNaMaxTensors);
static_assert(kNaBytes == FP8ADAM_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static_assert((kMaxElements >> kNaMaxChunkLog2) + 1 + kNaMaxTensors <= kNaMaxChunks,
              "every list within the element limit fits the chunk table");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNaBytes];

namespace {

constexpr int kNaMaxDevices = 256;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kNaMaxDevices] = {};

// Device address of `scratch` on device dev, which must be the current device.
int scratch_of(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kNaMaxDevices) return fail(FP8ADAM_EINVAL, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(FP8ADAM_EHIP, "hipGetSymbolAddress returned a null address for the scratch array");
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch[dev];
  return 0;
}

// Up to kSetupBatch tensor descriptors, by value in the kernel's arguments.
struct SetupBatch {
  int32_t first, count;
  TensorDesc d[kSetupBatch];
};

// One work-group per tensor of the batch: its descriptor and its entries of
// the chunk table (chunk -> tensor) into the scratch.
__global__ __launch_bounds__(kThreads) void k_noalloc_setup(SetupBatch b, TensorDesc* __restrict__ descs,
                                                            int32_t* __restrict__ chunk_tid, int chunk_log2) {
  const int j = blockIdx.x;
  if (j >= b.count) return;
  const int32_t t = b.first + j;
  const TensorDesc d = b.d[j];
  if (threadIdx.x == 0) descs[t] = d;
  const int64_t nc = (d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
  for (int64_t k = threadIdx.x; k < nc; k += kThreads) chunk_tid[d.chunk0 + k] = t;
}

// Chunks of the list at chunk size 2^chunk_log2 (each tensor rounded up to whole chunks).
int64_t count_chunks(const fp8adam_tensor* tensors, int32_t n, int chunk_log2) {
  int64_t nc = 0;
  for (int32_t t = 0; t < n; t++) nc += (tensors[t].numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
  return nc;
}

}  // namespace

// ================================================================== C ABI

extern "C" {

const char* fp8adam_last_error(void) { return g_last_error.c_str(); }

int fp8adam_runtime_version(int32_t* version) {
  if (!version) return fail(FP8ADAM_EINVAL, "version is null");
  int v = 0;
  HIP_TRY(hipRuntimeGetVersion(&v));
  *version = v;
  return 0;
}

int fp8adam_init(fp8adam_ctx** out, const fp8adam_tensor* tensors, int32_t n, const fp8adam_config* cfg,
                 hipStream_t stream) {
  try {
    if (!out) return fail(FP8ADAM_EINVAL, "out is null");
    *out = nullptr;
    if (!tensors || !cfg) return fail(FP8ADAM_EINVAL, "tensors or cfg is null");
    if (n <= 0) return fail(FP8ADAM_EINVAL, "n must be positive");
    if (int r = check_config(cfg)) return r;
    const bool spec = cfg->schedule == FP8ADAM_SCHEDULE_SPECULATIVE;
    const bool delayed = cfg->scaling == FP8ADAM_SCALING_DELAYED;
    const int hist_len = cfg->amax_history_len > 0 ? cfg->amax_history_len : 16;
    // Chunk size: the largest power of two in [2^kMinChunkLog2, 2^kMaxChunkLog2] that still
    // gives the amax pass at least kMinAmaxGroups work-groups.
    int64_t total = 0;
    for (int32_t t = 0; t < n; t++) {
      total += tensors[t].numel > 0 ? std::min(tensors[t].numel, kMaxElements + 1) : 0;
      if (total > kMaxElements)
        return fail(FP8ADAM_EINVAL, "too many elements for one context (at most " + std::to_string(kMaxElements) +
                                        "); split the tensor list over several contexts");
    }
    int chunk_log2 = kMaxChunkLog2;
    while (chunk_log2 > kMinChunkLog2 && (total >> chunk_log2) < kMinAmaxGroups) chunk_log2--;
    const int64_t chunk = (int64_t)1 << chunk_log2;

    std::vector<TensorDesc> desc(2 * (size_t)n);  // [m/v set][m_alt/v_alt set]
    std::vector<int32_t> chunk_tid;
    int64_t nchunks = 0;
    for (int32_t t = 0; t < n; t++) {
      const fp8adam_tensor& T = tensors[t];
      if (int r = check_tensor(T, t, delayed, spec)) return r;
      const int64_t nc = (T.numel + chunk - 1) / chunk;
      desc[t] = TensorDesc{T.param, static_cast<const uint16_t*>(T.grad), T.m, T.v, T.m_scale, T.v_scale,
                           T.numel, nchunks, delayed ? T.amax_history : nullptr};
      desc[(size_t)n + t] = desc[t];
      if (spec) {
        desc[(size_t)n + t].m = T.m_alt;
        desc[(size_t)n + t].v = T.v_alt;
      }
      if (((nchunks + nc) << (chunk_log2 - kNarrowPartLog2)) > kMaxGroups)
        return fail(FP8ADAM_EINVAL, "too many elements for one context once each tensor is rounded up to whole "
                                    "chunks; split the tensor list over several contexts");
      for (int64_t k = 0; k < nc; k++) chunk_tid.push_back(t);
      nchunks += nc;
    }

    fp8adam_ctx* c = new (std::nothrow) fp8adam_ctx();
    if (!c) return fail(FP8ADAM_ENOMEM, "host allocation failed");
    c->cfg = *cfg;
    c->n = n;
    c->nchunks = nchunks;
    c->chunk_log2 = chunk_log2;
    c->nparts = nchunks << (chunk_log2 - kPartLog2);
    c->nuparts = nchunks << (chunk_log2 - kUPartLog2Min);
    c->speculate_from = cfg->speculate_from_step > 0 ? cfg->speculate_from_step : 4;
    c->hist_len = delayed ? hist_len : 0;
    c->delayed_from = cfg->delayed_from_step > 0 ? cfg->delayed_from_step : 2;
    c->margin_scale = ldexpf(1.0f, delayed ? cfg->margin : 0);
    // the scale probe's work list: room for cand_cap(its update-pass parts) entries per tensor
    // AUTO: the probe on lists of at least kProbeMinElements (its two launches and the fold
    // cost about 15-20 us a step, more than the fix-up it saves on a short step)
    const bool probe = cfg->predictor == FP8ADAM_PREDICT_PROBE ||
                       (cfg->predictor == FP8ADAM_PREDICT_AUTO && total >= kProbeMinElements);
    if (spec && probe) {
      const int pl = cfg->master == FP8ADAM_MASTER_BF16 ? upd_part_log2<true>() : upd_part_log2<false>();
      for (int32_t t = 0; t < n; t++) c->ncand_slots += cand_cap((tensors[t].numel + ((int64_t)1 << pl) - 1) >> pl);
    }
    hipError_t e = hipGetDevice(&c->device);
    const size_t namax = (size_t)n * 4;
    if (e == hipSuccess) e = hipMalloc(&c->d_desc, sizeof(TensorDesc) * 2 * (size_t)n);
    if (e == hipSuccess && (spec || delayed)) e = hipMalloc(&c->d_part_amax, sizeof(uint2) * (size_t)std::max<int64_t>(1, c->nuparts));
    if (e == hipSuccess) e = hipMalloc(&c->d_flags, sizeof(int32_t) * (size_t)n);
    if (e == hipSuccess && spec) e = hipMalloc(&c->d_fix_count, sizeof(uint32_t));
    if (e == hipSuccess && spec) e = hipMalloc(&c->d_fix_list, sizeof(uint32_t) * (size_t)std::max<int64_t>(1, 2 * nchunks));
    if (spec) {
      const size_t ns = (size_t)std::max<int64_t>(1, c->ncand_slots);
      if (e == hipSuccess) e = hipMalloc(&c->d_cand_count, sizeof(uint32_t));
      if (e == hipSuccess) e = hipMalloc(&c->d_cand_work, sizeof(uint2) * ns);
      if (e == hipSuccess) e = hipMalloc(&c->d_cand_n, sizeof(int32_t) * (size_t)n);
      if (e == hipSuccess) e = hipMalloc(&c->d_cand_len, sizeof(int64_t) * (size_t)n);
      if (e == hipSuccess) e = hipMalloc(&c->d_lb, sizeof(uint32_t) * 2 * (size_t)n);
      if (e == hipSuccess) e = hipMalloc(&c->d_probed, sizeof(int64_t) * (size_t)n);
      if (e == hipSuccess) e = hipMemsetAsync(c->d_cand_count, 0, sizeof(uint32_t), stream);
      // the pass never writes the partials of the parts past a tensor's end: k_part_fold reads them as 0
      if (e == hipSuccess)
        e = hipMemsetAsync(c->d_part_amax, 0, sizeof(uint2) * (size_t)std::max<int64_t>(1, c->nuparts), stream);
      if (e == hipSuccess) e = hipMemsetAsync(c->d_cand_n, 0, sizeof(int32_t) * (size_t)n, stream);
      if (e == hipSuccess) e = hipMemsetAsync(c->d_cand_len, 0, sizeof(int64_t) * (size_t)n, stream);
      if (e == hipSuccess) e = hipMemsetAsync(c->d_lb, 0, sizeof(uint32_t) * 2 * (size_t)n, stream);
      if (e == hipSuccess) e = hipMemsetAsync(c->d_probed, 0, sizeof(int64_t) * (size_t)n, stream);
    }
    if (e == hipSuccess) e = hipMalloc(&c->d_chunk_tid, sizeof(int32_t) * (size_t)std::max<int64_t>(1, nchunks));
    if (e == hipSuccess) e = hipMalloc(&c->d_amax, sizeof(uint32_t) * namax);
    if (e == hipSuccess) e = hipMalloc(&c->d_partial, sizeof(uint2) * (size_t)std::max<int64_t>(1, nchunks));
    if (e == hipSuccess) e = hipMalloc(&c->d_old_scale, sizeof(float) * 4 * (size_t)n);
    if (e == hipSuccess) e = hipMalloc(&c->d_counters, sizeof(unsigned long long) * (size_t)n * kStatsPerTensor);
    if (e == hipSuccess)
      e = hipMalloc(&c->d_gpart, 2 * sizeof(double) * (size_t)std::max<int64_t>(1, std::min<int64_t>(nchunks, kNormGroups)));
    if (e == hipSuccess) e = hipMalloc(&c->d_gctl, sizeof(GradCtl));
    if (e == hipSuccess)
      e = hipMemcpyAsync(c->d_desc, desc.data(), sizeof(TensorDesc) * 2 * (size_t)n, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->d_flags, 0, sizeof(int32_t) * (size_t)n, stream);
    if (e == hipSuccess && nchunks > 0)
      e = hipMemcpyAsync(c->d_chunk_tid, chunk_tid.data(), sizeof(int32_t) * (size_t)nchunks, hipMemcpyHostToDevice,
                         stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->d_amax, 0, sizeof(uint32_t) * namax, stream);
    if (cfg->zero_state) {
      for (int32_t t = 0; e == hipSuccess && t < n; t++) {
        if (tensors[t].numel <= 0) continue;
        e = hipMemsetAsync(tensors[t].m, 0, (size_t)tensors[t].numel, stream);
        if (e == hipSuccess) e = hipMemsetAsync(tensors[t].v, 0, (size_t)tensors[t].numel, stream);
      }
      if (e == hipSuccess) {
        hipLaunchKernelGGL(k_fresh_state, dim3((unsigned)n), dim3(kThreads), 0, stream, c->d_desc,
                           cfg->granularity == FP8ADAM_SCALE_BLOCK128 ? 1 : 0, 2 * c->hist_len);
        e = hipGetLastError();
      }
    }
    if (e == hipSuccess)
      e = hipMemsetAsync(c->d_counters, 0, sizeof(unsigned long long) * (size_t)n * kStatsPerTensor, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
      free_ctx(c);
      return e == hipErrorOutOfMemory ? fail(FP8ADAM_ENOMEM, "device allocation failed")
                                      : hip_fail(e, "fp8adam_init");
    }
    *out = c;
    return 0;
  } catch (const std::bad_alloc&) {
    return fail(FP8ADAM_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(FP8ADAM_EINVAL, "unexpected error in fp8adam_init");
  }
}

namespace {

// The context's buffers live on the device it was built on: a stream of
// another device would run the kernels there, against this device's memory.
int check_device(const fp8adam_ctx* ctx, hipStream_t stream) {
  hipDevice_t dev = -1;
  const hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  if (dev != ctx->device)
    return fail(FP8ADAM_EINVAL, "the stream belongs to device " + std::to_string(dev) + ", the context to device " +
                                    std::to_string(ctx->device));
  return 0;
}

// Validate the hyperparameters and fill the per-step constants of step hp->step.
int step_consts(const fp8adam_ctx* ctx, const fp8adam_hparams* hp, StepConsts& k) {
    if (!ctx || !hp) return fail(FP8ADAM_EINVAL, "ctx or hp is null");
    if (hp->step < 1) return fail(FP8ADAM_EINVAL, "step must be >= 1");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
      return fail(FP8ADAM_EINVAL, "beta1 and beta2 must lie in [0, 1)");
    if (!(hp->eps >= 0.0f) || !isfinite(hp->eps)) return fail(FP8ADAM_EINVAL, "eps must be finite and >= 0");
    if (!isfinite(hp->lr) || !isfinite(hp->weight_decay)) return fail(FP8ADAM_EINVAL, "lr and weight_decay must be finite");
    const double bc1 = 1.0 - pow((double)hp->beta1, (double)hp->step);
    const double bc2 = 1.0 - pow((double)hp->beta2, (double)hp->step);
    k.b1 = hp->beta1;
    k.b2 = hp->beta2;
    k.omb1 = 1.0f - hp->beta1;
    k.omb2 = 1.0f - hp->beta2;
    const bool l2 = ctx->cfg.decay_mode == FP8ADAM_DECAY_L2;
    k.decay = l2 ? 1.0f : (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    k.l2 = l2 ? hp->weight_decay : 0.0f;
    k.step_size = (float)((double)hp->lr / bc1);
    k.inv_bc2 = (float)(1.0 / bc2);
    k.eps = hp->eps;
    // the speculative schedule's prediction of how each tensor's amax moves
    k.grow_m = amax_growth((double)hp->beta1, (double)hp->step);
    k.grow_v = amax_growth((double)hp->beta2, (double)hp->step);
    k.margin_scale = ctx->margin_scale;
    k.hist_len = ctx->hist_len;
    k.hist_slot = ctx->hist_len > 0 ? (int)((hp->step - 1) % ctx->hist_len) : 0;
    k.gfac = 1.0f;
    k.seed_lo = (uint32_t)ctx->cfg.seed;
    k.seed_hi = (uint32_t)(ctx->cfg.seed >> 32);
    k.rng_t = (uint32_t)hp->step;
    return 0;
}

}  // namespace

int fp8adam_step(fp8adam_ctx* ctx, const fp8adam_hparams* hp, hipStream_t stream) {
  try {
    StepConsts k;
    if (int r = step_consts(ctx, hp, k)) return r;
    if (int r = check_device(ctx, stream)) return r;
    return run_step(ctx, k, hp->step, stream);
  } catch (...) {
    return fail(FP8ADAM_EINVAL, "unexpected error in fp8adam_step");
  }
}

int fp8adam_step_amp(fp8adam_ctx* ctx, const fp8adam_hparams* hp, const fp8adam_amp_config* amp,
                     fp8adam_amp_state* state, hipStream_t stream) {
  try {
    StepConsts k;
    if (int r = step_consts(ctx, hp, k)) return r;
    if (!amp || !state) return fail(FP8ADAM_EINVAL, "amp or state is null");
    if (int r = check_device(ctx, stream)) return r;
    if ((uintptr_t)state & 7u) return fail(FP8ADAM_EINVAL, "state must be 8-byte aligned");
    if (!(amp->growth_factor > 1.0f) || !isfinite(amp->growth_factor) || !(amp->backoff_factor > 0.0f) ||
        !(amp->backoff_factor < 1.0f) || amp->growth_interval < 1 || !isfinite(amp->max_norm))
      return fail(FP8ADAM_EINVAL, "growth_factor must exceed 1, backoff_factor lie in (0, 1), "
                                  "growth_interval be >= 1 and max_norm be finite");
    fp8adam_ctx* c = ctx;
    hipStream_t s = stream;
    if (c->nchunks > 0) TIMED(10, launch_gradnorm(c, s));
    TIMED(11, (launch_gradctl(c, *amp, state, *hp, s)));
    HIP_TRY(hipGetLastError());
    c->gctl = c->d_gctl;
    const int r = run_step(c, k, hp->step, s);
    c->gctl = nullptr;
    return r;
  } catch (...) {
    if (ctx) ctx->gctl = nullptr;
    return fail(FP8ADAM_EINVAL, "unexpected error in fp8adam_step_amp");
  }
}

int fp8adam_step_noalloc(const fp8adam_tensor* tensors, int32_t n, const fp8adam_config* cfg,
                         const fp8adam_hparams* hp, hipStream_t stream) {
  try {
    if (!tensors || !cfg || !hp) return fail(FP8ADAM_EINVAL, "tensors, cfg or hp is null");
    if (n <= 0 || n > kNaMaxTensors)
      return fail(FP8ADAM_EINVAL, "n must lie in [1, " + std::to_string(kNaMaxTensors) +
                                      "] (FP8ADAM_NOALLOC_MAX_TENSORS)");
    if (int r = check_config(cfg)) return r;
    if (cfg->schedule != FP8ADAM_SCHEDULE_TWO_PASS || cfg->scaling != FP8ADAM_SCALING_JUST_IN_TIME)
      return fail(FP8ADAM_EINVAL, "fp8adam_step_noalloc runs the TWO_PASS schedule with just-in-time scaling");
    if (cfg->collect_stats || cfg->zero_state)
      return fail(FP8ADAM_EINVAL, "fp8adam_step_noalloc takes neither collect_stats nor zero_state");
    int64_t total = 0;
    for (int32_t t = 0; t < n; t++) {
      if (int r = check_tensor(tensors[t], t, false, false)) return r;
      total += std::min(tensors[t].numel, kMaxElements + 1);
      if (total > kMaxElements)
        return fail(FP8ADAM_EINVAL, "too many elements for one step (at most " + std::to_string(kMaxElements) + ")");
    }
    // the chunk size fp8adam_init would take, raised until the chunk table fits the scratch
    int chunk_log2 = kMaxChunkLog2;
    while (chunk_log2 > kMinChunkLog2 && (total >> chunk_log2) < kMinAmaxGroups) chunk_log2--;
    int64_t nchunks = count_chunks(tensors, n, chunk_log2);
    while (nchunks > kNaMaxChunks && chunk_log2 < kNaMaxChunkLog2) nchunks = count_chunks(tensors, n, ++chunk_log2);
    if (nchunks > kNaMaxChunks)
      return fail(FP8ADAM_EINVAL, "the list needs " + std::to_string(nchunks) + " chunks, more than the scratch holds (" +
                                      std::to_string(kNaMaxChunks) + ", FP8ADAM_NOALLOC_MAX_CHUNKS)");
    if ((nchunks << (chunk_log2 - kNarrowPartLog2)) > kMaxGroups)
      return fail(FP8ADAM_EINVAL, "too many elements for one step once each tensor is rounded up to whole chunks");
    fp8adam_ctx c;  // on the stack: every buffer it names lies in the scratch array
    c.cfg = *cfg;
    c.n = n;
    c.nchunks = nchunks;
    c.chunk_log2 = chunk_log2;
    c.nparts = nchunks << (chunk_log2 - kPartLog2);
    c.nuparts = nchunks << (chunk_log2 - kUPartLog2Min);
    StepConsts k;
    if (int r = step_consts(&c, hp, k)) return r;

    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    hipDevice_t sdev = -1;
    HIP_TRY(hipStreamGetDevice(stream, &sdev));
    if (sdev != dev)
      return fail(FP8ADAM_EINVAL, "the stream belongs to device " + std::to_string(sdev) + ", not the current device " +
                                      std::to_string(dev));
    unsigned char* base = nullptr;
    if (int r = scratch_of(dev, &base)) return r;
    c.device = dev;
    c.d_desc = reinterpret_cast<TensorDesc*>(base + kNaDesc);
    c.d_chunk_tid = reinterpret_cast<int32_t*>(base + kNaChunkTid);
    c.d_partial = reinterpret_cast<uint2*>(base + kNaPartial);
    c.d_amax = reinterpret_cast<uint32_t*>(base + kNaAmax);
    c.d_old_scale = reinterpret_cast<float*>(base + kNaOldScale);
    c.d_flags = reinterpret_cast<int32_t*>(base + kNaFlags);

    SetupBatch b{};  // unused slots are zero
    int64_t chunk0 = 0;
    for (int32_t t0 = 0; t0 < n; t0 += kSetupBatch) {
      b.first = t0;
      b.count = std::min<int32_t>(kSetupBatch, n - t0);
      for (int32_t j = 0; j < b.count; j++) {
        const fp8adam_tensor& T = tensors[t0 + j];
        b.d[j] = TensorDesc{T.param, static_cast<const uint16_t*>(T.grad), T.m, T.v, T.m_scale, T.v_scale,
                            T.numel, chunk0, nullptr};
        chunk0 += (T.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
      }
      hipLaunchKernelGGL(k_noalloc_setup, dim3((unsigned)b.count), dim3(kThreads), 0, stream, b, c.d_desc,
                         c.d_chunk_tid, chunk_log2);
      HIP_TRY(hipGetLastError());
    }
    return run_step(&c, k, hp->step, stream);
  } catch (...) {
    return fail(FP8ADAM_EINVAL, "unexpected error in fp8adam_step_noalloc");
  }
}

int fp8adam_stats(fp8adam_ctx* ctx, fp8adam_stats_t* out_host, int32_t n, hipStream_t stream) {
  try {
    if (!ctx || !out_host) return fail(FP8ADAM_EINVAL, "ctx or out is null");
    if (n != ctx->n) return fail(FP8ADAM_EINVAL, "n must equal the context's tensor count");
    if (int r = check_device(ctx, stream)) return r;
    std::vector<uint32_t> amax((size_t)n * 4, 0u);
    std::vector<unsigned long long> cnt((size_t)n * kStatsPerTensor, 0ull);
    std::vector<TensorDesc> desc((size_t)n);
    std::vector<int32_t> flags((size_t)n, 0);
    std::vector<int64_t> probed((size_t)n, 0);
    const bool block = ctx->cfg.granularity == FP8ADAM_SCALE_BLOCK128;
    HIP_TRY(hipMemcpyAsync(flags.data(), ctx->d_flags, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream));
    if (ctx->d_probed && ctx->last_spec)
      HIP_TRY(hipMemcpyAsync(probed.data(), ctx->d_probed, sizeof(int64_t) * (size_t)n, hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipMemcpyAsync(amax.data(), ctx->d_amax,
                           sizeof(uint32_t) * (size_t)n * (block ? 4 : 2), hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipMemcpyAsync(cnt.data(), ctx->d_counters, sizeof(unsigned long long) * cnt.size(),
                           hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipMemcpyAsync(desc.data(), ctx->d_desc, sizeof(TensorDesc) * (size_t)n, hipMemcpyDeviceToHost, stream));
    std::vector<float> sm((size_t)n, 0.0f), sv((size_t)n, 0.0f);
    if (!block) {
      for (int32_t t = 0; t < n; t++) {
        if (desc[t].numel == 0) continue;
        HIP_TRY(hipMemcpyAsync(&sm[t], desc[t].sm, sizeof(float), hipMemcpyDeviceToHost, stream));
        HIP_TRY(hipMemcpyAsync(&sv[t], desc[t].sv, sizeof(float), hipMemcpyDeviceToHost, stream));
      }
    }
    HIP_TRY(hipStreamSynchronize(stream));
    for (int32_t t = 0; t < n; t++) {
      fp8adam_stats_t& o = out_host[t];
      auto f = [](uint32_t b) {
        float x;
        memcpy(&x, &b, 4);
        return x;
      };
      if (block) {
        o.amax_m = f(amax[4 * t]);
        o.amax_v = f(amax[4 * t + 1]);
        o.scale_m = f(amax[4 * t + 2]);
        o.scale_v = f(amax[4 * t + 3]);
      } else {
        o.amax_m = f(amax[2 * t]);
        o.amax_v = f(amax[2 * t + 1]);
        o.scale_m = sm[t];
        o.scale_v = sv[t];
      }
      o.underflow_m = (int64_t)cnt[kStatsPerTensor * t + kUnderM];
      o.underflow_v = (int64_t)cnt[kStatsPerTensor * t + kUnderV];
      o.saturated_m = (int64_t)cnt[kStatsPerTensor * t + kSatM];
      o.saturated_v = (int64_t)cnt[kStatsPerTensor * t + kSatV];
      o.nonfinite = (int64_t)cnt[kStatsPerTensor * t + kNonFinite];
      o.requantized = (int64_t)(((flags[t] & 1) ? 1 : 0) + ((flags[t] & 2) ? 1 : 0)) * desc[t].numel;
      o.probed = probed[t];
    }
    return 0;
  } catch (...) {
    return fail(FP8ADAM_EINVAL, "unexpected error in fp8adam_stats");
  }
}

void fp8adam_destroy(fp8adam_ctx* ctx) { free_ctx(ctx); }

int64_t fp8adam_num_chunks(const fp8adam_ctx* ctx) { return ctx ? ctx->nchunks : -1; }

int32_t fp8adam_current_buffer(const fp8adam_ctx* ctx) { return ctx ? ctx->cur : -1; }

int fp8adam_set_timing_kinds(fp8adam_ctx* ctx, uint32_t kinds) {
  try {
    if (!ctx) return fail(FP8ADAM_EINVAL, "ctx is null");
    if (kinds && ctx->ev.empty()) {
      ctx->ev.resize(2 * kMaxTimed, nullptr);
      ctx->ev_kind.resize(kMaxTimed, 0);
      for (auto& e : ctx->ev) HIP_TRY(hipEventCreate(&e));
    }
    ctx->timing = kinds != 0;
    ctx->timing_kinds = kinds;
    ctx->ev_used = 0;
    return 0;
  } catch (...) {
    return fail(FP8ADAM_ENOMEM, "host allocation failed");
  }
}

int fp8adam_set_timing(fp8adam_ctx* ctx, int32_t enable) {
  try {
    return fp8adam_set_timing_kinds(ctx, enable ? 0xFFFFFFFFu : 0u);
  } catch (...) {
    return fail(FP8ADAM_ENOMEM, "host allocation failed");
  }
}

int fp8adam_kernel_times(fp8adam_ctx* ctx, double* total_ms, int32_t* count, int32_t max) {
  if (!ctx || !total_ms || !count || max <= 0) return fail(FP8ADAM_EINVAL, "bad argument");
  for (int32_t k = 0; k < max; k++) {
    total_ms[k] = 0.0;
    count[k] = 0;
  }
  for (int i = 0; i < ctx->ev_used; i++) {
    HIP_TRY(hipEventSynchronize(ctx->ev[2 * i + 1]));
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, ctx->ev[2 * i], ctx->ev[2 * i + 1]));
    const int kind = ctx->ev_kind[i];
    if (kind < max) {
      total_ms[kind] += ms;
      count[kind] += 1;
    }
  }
  ctx->ev_used = 0;
  return 0;
}

int fp8adam_encode(int32_t fmt, const float* x, uint8_t* out, int64_t n, hipStream_t stream) {
  if (!valid_fmt(fmt) || n < 0 || (n > 0 && (!x || !out))) return fail(FP8ADAM_EINVAL, "bad argument");
  if (n == 0) return 0;
  if (fmt == 0)
    hipLaunchKernelGGL(k_encode<0>, dim3(probe_grid(n, 4)), dim3(kThreads), 0, stream, x, out, n);
  else
    hipLaunchKernelGGL(k_encode<1>, dim3(probe_grid(n, 4)), dim3(kThreads), 0, stream, x, out, n);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_decode(int32_t fmt, const uint8_t* codes, float* out, int64_t n, hipStream_t stream) {
  if (!valid_fmt(fmt) || n < 0 || (n > 0 && (!codes || !out))) return fail(FP8ADAM_EINVAL, "bad argument");
  if (n == 0) return 0;
  if (fmt == 0)
    hipLaunchKernelGGL(k_decode<0>, dim3(probe_grid(n, 1)), dim3(kThreads), 0, stream, codes, out, n);
  else
    hipLaunchKernelGGL(k_decode<1>, dim3(probe_grid(n, 1)), dim3(kThreads), 0, stream, codes, out, n);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_encode_sr_bits_range(int32_t fmt, uint32_t start, int64_t count, uint32_t r16, uint8_t* out,
                                 hipStream_t stream) {
  if (!valid_fmt(fmt) || count < 0 || count > ((int64_t)1 << 32) - (int64_t)start || r16 > 0xFFFFu ||
      (count > 0 && !out))
    return fail(FP8ADAM_EINVAL, "bad argument");
  if (count == 0) return 0;
  if (fmt == 0)
    hipLaunchKernelGGL(k_encode_sr_bits<0>, dim3(probe_grid(count, 4)), dim3(kThreads), 0, stream, start, count, r16,
                       out);
  else
    hipLaunchKernelGGL(k_encode_sr_bits<1>, dim3(probe_grid(count, 4)), dim3(kThreads), 0, stream, start, count, r16,
                       out);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_encode_sr(int32_t fmt, const float* x, const uint16_t* r16, uint8_t* out, int64_t n,
                      hipStream_t stream) {
  if (!valid_fmt(fmt) || n < 0 || (n > 0 && (!x || !r16 || !out))) return fail(FP8ADAM_EINVAL, "bad argument");
  if (n == 0) return 0;
  if (fmt == 0)
    hipLaunchKernelGGL(k_encode_sr<0>, dim3(probe_grid(n, 1)), dim3(kThreads), 0, stream, x, r16, out, n);
  else
    hipLaunchKernelGGL(k_encode_sr<1>, dim3(probe_grid(n, 1)), dim3(kThreads), 0, stream, x, r16, out, n);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || (bytes & 15) || (bytes > 0 && (!src || !dst)))
    return fail(FP8ADAM_EINVAL, "bytes must be a non-negative multiple of 16 with non-null pointers");
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return fail(FP8ADAM_EALIGN, "src and dst must be 16-byte aligned");
  if (bytes == 0) return 0;
  const int64_t n16 = bytes / 16;
  const int64_t groups = (n16 + 4 * kThreads - 1) / (4 * kThreads);
  if (groups > (int64_t)INT32_MAX) return fail(FP8ADAM_EINVAL, "copy too large");
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)groups), dim3(kThreads), 0, stream, static_cast<const vu4*>(src),
                     static_cast<vu4*>(dst), n16);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_stream_rw(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, hipStream_t stream) {
  if (read_bytes < 0 || write_bytes < 0 || ((read_bytes | write_bytes) & 15) || (read_bytes > 0 && !src) ||
      (write_bytes > 0 && !dst))
    return fail(FP8ADAM_EINVAL, "sizes must be non-negative multiples of 16, with a non-null pointer where nonzero");
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return fail(FP8ADAM_EALIGN, "src and dst must be 16-byte aligned");
  const int64_t n_read = read_bytes / 16, n_write = write_bytes / 16;
  const int64_t groups = (std::max(n_read, n_write) + 4 * kThreads - 1) / (4 * kThreads);
  if (groups > (int64_t)INT32_MAX) return fail(FP8ADAM_EINVAL, "stream too large");
  if (groups == 0) return 0;
  hipLaunchKernelGGL(k_stream_rw, dim3((unsigned)groups), dim3(kThreads), 0, stream, static_cast<const vu4*>(src),
                     n_read, static_cast<vu4*>(dst), n_write);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_stream_mix(int32_t master, void* p, const void* g, const void* m_in, const void* v_in, void* m_out,
                       void* v_out, int64_t n, hipStream_t stream) {
  if (master != FP8ADAM_MASTER_FP32 && master != FP8ADAM_MASTER_BF16) return fail(FP8ADAM_EINVAL, "bad master dtype");
  const bool bf16 = master == FP8ADAM_MASTER_BF16;
  const int pl = bf16 ? upd_part_log2<true>() : upd_part_log2<false>();
  if (n < 0 || (n & (((int64_t)1 << pl) - 1)))
    return fail(FP8ADAM_EINVAL, "n must be a non-negative multiple of " + std::to_string(1 << pl));
  if (n > 0 && (!p || !g || !m_in || !v_in || !m_out || !v_out)) return fail(FP8ADAM_EINVAL, "null pointer");
  for (const void* q : {(const void*)p, g, m_in, v_in, (const void*)m_out, (const void*)v_out})
    if ((uintptr_t)q & 15u) return fail(FP8ADAM_EALIGN, "every buffer must be 16-byte aligned");
  const int64_t nparts = n >> pl;
  if (nparts > kMaxGroups) return fail(FP8ADAM_EINVAL, "n too large for one launch");
  if (nparts == 0) return 0;
  const auto* gg = static_cast<const uint16_t*>(g);
  const auto* mi = static_cast<const uint8_t*>(m_in);
  const auto* vi = static_cast<const uint8_t*>(v_in);
  auto* mo = static_cast<uint8_t*>(m_out);
  auto* vo = static_cast<uint8_t*>(v_out);
  if (bf16)
    hipLaunchKernelGGL(k_stream_mix<true>, dim3(grid_for<kXcdStreams>(nparts)), dim3(kThreads), 0, stream, p, gg, mi, vi,
                       mo, vo, nparts);
  else
    hipLaunchKernelGGL(k_stream_mix<false>, dim3(grid_for<kXcdStreams>(nparts)), dim3(kThreads), 0, stream, p, gg, mi,
                       vi, mo, vo, nparts);
  HIP_TRY(hipGetLastError());
  return 0;
}

int fp8adam_encode_bits_range(int32_t fmt, uint32_t start, int64_t count, uint8_t* out, hipStream_t stream) {
  if (!valid_fmt(fmt) || count < 0 || (count > 0 && !out) || count > (int64_t)(1ull << 32) - (int64_t)start)
    return fail(FP8ADAM_EINVAL, "bad argument");
  if (count == 0) return 0;
  if (fmt == 0)
    hipLaunchKernelGGL(k_encode_bits<0>, dim3(probe_grid(count, 4)), dim3(kThreads), 0, stream, start, count, out);
  else
    hipLaunchKernelGGL(k_encode_bits<1>, dim3(probe_grid(count, 4)), dim3(kThreads), 0, stream, start, count, out);
  HIP_TRY(hipGetLastError());
  return 0;
}

}  // extern "C"
