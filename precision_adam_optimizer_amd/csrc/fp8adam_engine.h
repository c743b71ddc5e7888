// fp8adam_engine.h -- the step kernels of the FP8-moment Adam step and their
// dispatch over the template parameters, shared by the translation units that
// instantiate them (one per (m format, v format) pair, built in parallel) and
// by fp8adam.hip, which holds the C ABI.
//
// Method: Adam whose first moment is stored in FP8 E4M3 and second moment in
// FP8 E5M2, each with a scale (daoxuan.cc explainer of arXiv 2409.12517,
// section on why Adam keeps m in E4M3 and v in E5M2; shd-paper.top summary of
// arXiv 2409.12517v2, method details: both Adam moments quantized to FP8).
//
// Device work per step:
//   per-tensor scales, two passes over a chunked multi-tensor list
//     k_amax    : dequantize, update m and v in registers, max|m'| / max v'
//                 per chunk (DPP wave max, then LDS) -> one partial per
//                 chunk, no atomics
//     k_reduce  : one work-group per tensor: max over the tensor's partials,
//                 stage the old scales, write the new scales into the
//                 caller's slots (and clear the tensor's stats counters)
//     k_update  : recompute m', v' with the staged old scales; update p;
//                 requantize m', v' with the new scales and saturation
//   per-tensor scales, speculative schedule (bit-identical results)
//     k_spec_probe : the exact amax of m', v' over each tensor's candidate
//                 parts (those that held values near its amax at the step
//                 before), a lower bound of the new amax
//     k_spec_prepare : per tensor, stage the old scales and the predicted ones
//                 (from the probe's bound, else from the growth model)
//     k_update<kModeSpec> : one pass that quantizes with a predicted scale,
//                 writes the codes into the other code buffer (ping-pong),
//                 updates p and records per-part amax partials
//     k_spec_reduce : per tensor, the true scale; a mispredicted moment is
//                 flagged; the next step's candidate parts are listed
//     k_fixup   : the chunks of flagged tensors only (a work list that
//                 k_spec_reduce appends to): move the codes' exponent fields to
//                 the true scale, recomputing the few that cannot be moved from
//                 the old codes (still intact in the source buffer)
//     the step before the first speculative one: k_amax, k_exact_prepare (the
//                 true scales as the prediction), then the speculative pass
//                 and check (which lists the first candidates)
//   per-tensor delayed scaling (scale from an amax history)
//     k_delayed_prepare (scales from the history), k_update<kModeDelayed>,
//     k_delayed_reduce (commit the scales, record this step's amax)
//   per-128-element scales (one pass)
//     k_block   : 32 lanes own one 128-element block; the block amax is a
//                 5-step DPP/swizzle max, then update and requantize as above
// Options on every pass: coupled L2 (L2), stochastic rounding (SR), and the
// loss-scaling hook (GradCtl: skip the step, or scale the gradients).
// The chunk table (built once at init) cuts every tensor into chunks of
// 2^chunk_log2 elements (4096..32768, chosen per context so that even small
// lists give a few thousand work-groups); an amax-pass work-group owns one
// chunk, an update-pass work-group one part of 2^upd_part_log2 elements, a
// block-pass work-group one kPart-element part.
// Loads and stores are dword-granular per lane and contiguous across the wave
// (fp32 master: 16 B per lane); the amax, update and block passes stream
// through buffer resources based at each work-group's part.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/fp8adam.h"
#include "fp8_codec.h"

namespace fp8adam_engine {

using namespace fp8adam;


// Launch-shape tunables (compile-time; the defaults are the measured best on MI355X).
#ifndef FP8ADAM_MAX_CHUNK_LOG2
#define FP8ADAM_MAX_CHUNK_LOG2 15  // largest chunk = amax-pass work-group (32768 elements)
#endif
// Block pass: one-shot work-groups of 1024 elements (8 blocks, one per
// half-wave); 6.5% faster than 4096-element work-groups (4 blocks per
// half-wave) and 4% faster than 2048, for the same reason as the update pass.
#ifndef FP8ADAM_PART_LOG2
#define FP8ADAM_PART_LOG2 10       // block-pass work-group (1024 elements)
#endif
#ifndef FP8ADAM_BLOCK_J
#define FP8ADAM_BLOCK_J 1          // block pass: 128-element blocks per half-wave per tile
#endif
// Update pass, fp32 master: one-shot work-groups of 1024 elements, one group
// of 4 per lane.  Measured against 2048 (two groups
// per lane) and 4096 (four): the mixed read/write stream runs 7% faster
// (two-pass) / 4% (speculative) with the smallest work-groups, which keep more
// distinct work-groups, and so more independent address streams, in flight
// per CU.
#ifndef FP8ADAM_UPD_PART_LOG2
#define FP8ADAM_UPD_PART_LOG2 10
#endif
// Update pass with a bf16 master (10 bytes per element, so a 1024-element
// work-group moves only 10 KiB): 2048-element work-groups, two groups per
// lane, measured 5-6% faster than 1024 and 3% faster than 4096.
#ifndef FP8ADAM_UPD_PART_LOG2_WIDE
#define FP8ADAM_UPD_PART_LOG2_WIDE 11
#endif
#ifndef FP8ADAM_AMAX_UNROLL
#define FP8ADAM_AMAX_UNROLL 8
#endif
#ifndef FP8ADAM_UPDATE_UNROLL
#define FP8ADAM_UPDATE_UNROLL 1
#endif
// 1: non-temporal global loads of the fix-up and the gradient-norm pass (each
// byte is touched once per pass)
#ifndef FP8ADAM_NT_AMAX
#define FP8ADAM_NT_AMAX 1
#endif
// Cache-policy operand of the streamed buffer loads and stores of the amax,
// update and block passes (gfx950: bit 0 sc0, bit 1 nt, bit 4 sc1); 2 = nt.
#ifndef FP8ADAM_BUF_LOAD_POLICY
#define FP8ADAM_BUF_LOAD_POLICY 2
#endif
#ifndef FP8ADAM_BUF_STORE_POLICY
#define FP8ADAM_BUF_STORE_POLICY 2
#endif
#ifndef FP8ADAM_XCD_ORDER
#define FP8ADAM_XCD_ORDER 1  // update / block passes: each XCD walks its own contiguous eighth
#endif

constexpr int kThreads = 256;                     // 4 waves of 64
constexpr int kGroup = 4;                         // consecutive elements per lane per access
constexpr int kSubTile = kThreads * kGroup;       // 1024 elements per work-group access
constexpr int kAmaxUnroll = FP8ADAM_AMAX_UNROLL;  // accesses in flight per lane, amax pass
constexpr int kUpdUnroll = FP8ADAM_UPDATE_UNROLL; // accesses in flight per lane, update pass
constexpr int kPartLog2 = FP8ADAM_PART_LOG2;
constexpr int64_t kPart = (int64_t)1 << kPartLog2;  // elements per block-pass work-group
// log2 of the elements per update-pass work-group
template <bool BF16P>
constexpr int upd_part_log2() {
  return BF16P ? FP8ADAM_UPD_PART_LOG2_WIDE : FP8ADAM_UPD_PART_LOG2;
}
constexpr int kUPartLog2Min = FP8ADAM_UPD_PART_LOG2 < FP8ADAM_UPD_PART_LOG2_WIDE ? FP8ADAM_UPD_PART_LOG2
                                                                                  : FP8ADAM_UPD_PART_LOG2_WIDE;
constexpr int kUPartLog2Max = FP8ADAM_UPD_PART_LOG2 < FP8ADAM_UPD_PART_LOG2_WIDE ? FP8ADAM_UPD_PART_LOG2_WIDE
                                                                                  : FP8ADAM_UPD_PART_LOG2;
constexpr int kMaxChunkLog2 = FP8ADAM_MAX_CHUNK_LOG2;
constexpr int kMinChunkLog2 = 12;                   // smallest chunk = amax-pass work-group (4096 elements)
constexpr int kMinAmaxGroups = 2048;                // 8 work-groups per CU
constexpr int kBlock = 128;                       // block-scale granularity
constexpr int kBlkJ = FP8ADAM_BLOCK_J;            // a block-pass tile is 8 half-waves x kBlkJ blocks
constexpr int kReduceThreads = 1024;              // one work-group per tensor in k_reduce
constexpr int kStatsPerTensor = 5;
// Speculative schedule, scale probe: a part whose amax of |m'| (or of v') was at
// least kCandTheta times its tensor's becomes a candidate for the next step; a
// tensor lists at most cand_cap(its parts) of them, a 2^-kCandShift share but
// at least kCandMin and at most kCandMax parts (with more, the probe would cost
// more than the fix-up it saves: the tensor falls back to the growth model).
constexpr float kCandTheta = 0.8f;
constexpr int kCandShift = 5;
constexpr int64_t kCandMin = 8;
constexpr int64_t kCandMax = 4096;
constexpr int64_t kProbeMinElements = (int64_t)1 << 28;  // FP8ADAM_PREDICT_AUTO's threshold
__host__ __device__ constexpr int64_t cand_cap(int64_t nparts) {
  return nparts < kCandMin ? nparts
                           : (nparts >> kCandShift) < kCandMin ? kCandMin
                                                               : (nparts >> kCandShift) > kCandMax ? kCandMax
                                                                                                   : (nparts >> kCandShift);
}

static_assert(kMaxChunkLog2 >= kMinChunkLog2 && kMinChunkLog2 >= kPartLog2 && kMinChunkLog2 >= kUPartLog2Max,
              "a chunk holds whole parts");
static_assert(((int64_t)1 << kUPartLog2Min) % (kSubTile * kUpdUnroll) == 0,
              "part must hold whole unrolled update tiles");
static_assert(kPart % (kBlock * 8 * kBlkJ) == 0, "part must hold whole block tiles");

struct TensorDesc {
  void* p;
  const uint16_t* g;
  uint8_t* m;
  uint8_t* v;
  float* sm;
  float* sv;
  int64_t numel;
  int64_t chunk0;  // index of the tensor's first chunk
  float* hist;     // delayed scaling: [2][H] amax history of m, v
};

// Update-pass variants: just-in-time scales known before the pass (two-pass
// schedule), a predicted scale with codes to the other buffer (speculative),
// or the delayed scale from the amax history.
enum UpdateMode { kModeJit = 0, kModeSpec = 1, kModeDelayed = 2 };

// Loss-scaling control of the step in flight, written on the device by
// k_gradctl (library-owned): whether the step is skipped (a non-finite
// gradient), the gradient factor clip_coef / S, and the bias-correction
// constants of the device-side step count.
struct GradCtl {
  int32_t skip;
  float gfac;
  float step_size, inv_bc2, grow_m, grow_v;
  int32_t hist_slot;  // delayed scaling: (t-1) mod H of the device-side t
  uint32_t t;         // the device-side t (stochastic rounding's counter)
};

// With loss scaling, take the step's gradient factor and bias corrections;
// true if the step is skipped (the kernel then changes nothing).
__device__ __forceinline__ bool amp_apply(const GradCtl* gctl, StepConsts& c) {
  if (gctl == nullptr) return false;
  if (gctl->skip) return true;
  c.gfac = gctl->gfac;
  c.step_size = gctl->step_size;
  c.inv_bc2 = gctl->inv_bc2;
  c.grow_m = gctl->grow_m;
  c.grow_v = gctl->grow_v;
  c.hist_slot = gctl->hist_slot;
  c.rng_t = gctl->t;
  return false;
}

// Random words of the group of 4 elements starting at element i of tensor
// tid: Philox4x32-10 with counter (i/4, t, tid) and the seed as key.  Word j
// belongs to element i + j; the first moment uses its low 16 bits, the second
// its high 16 bits.
template <bool SR>
__device__ __forceinline__ void sr_words(const StepConsts& c, int tid, int64_t i, uint32_t (&rw)[4]) {
  if constexpr (SR) {
    const uint64_t grp = (uint64_t)i >> 2;
    philox4x32_10((uint32_t)grp, (uint32_t)(grp >> 32), c.rng_t, (uint32_t)tid, c.seed_lo, c.seed_hi, rw);
  } else {
    rw[0] = rw[1] = rw[2] = rw[3] = 0u;
  }
}

// Quantize four values: round to nearest even, or stochastically with 16
// bits of each word (low half for m, high half for v).
template <int FMT, bool SR, bool HIGH>
__device__ __forceinline__ uint32_t quant4(const float (&q)[4], const uint32_t (&rw)[4]) {
  if constexpr (SR) {
    const uint32_t r[4] = {HIGH ? rw[0] >> 16 : rw[0] & 0xFFFFu, HIGH ? rw[1] >> 16 : rw[1] & 0xFFFFu,
                           HIGH ? rw[2] >> 16 : rw[2] & 0xFFFFu, HIGH ? rw[3] >> 16 : rw[3] & 0xFFFFu};
    return encode4_sr<FMT>(q[0], q[1], q[2], q[3], r);
  } else {
    return encode4<FMT>(q[0], q[1], q[2], q[3]);
  }
}

// The random word of element i of tensor tid alone (the ragged tails; 0 when
// rounding to nearest).
template <bool SR>
__device__ __forceinline__ uint32_t sr_word1(const StepConsts& c, int tid, int64_t i) {
  if constexpr (SR) {
    uint32_t rw[4];
    sr_words<true>(c, tid, i & ~(int64_t)3, rw);
    return rw[i & 3];
  } else {
    return 0u;
  }
}

// One value with its element's random word w (the ragged tails).
template <int FMT, bool SR, bool HIGH>
__device__ __forceinline__ uint32_t quant1(uint32_t w, float q) {
  if constexpr (SR) {
    const uint32_t r[4] = {HIGH ? w >> 16 : w & 0xFFFFu, 0u, 0u, 0u};
    return encode4_sr<FMT>(q, 0.0f, 0.0f, 0.0f, r) & 0xFFu;
  } else {
    return encode1<FMT>(q);
  }
}

enum Counter { kUnderM = 0, kUnderV = 1, kSatM = 2, kSatV = 3, kNonFinite = 4 };

// Wave-wide max / sum, returned to every lane (called with the whole wave
// active): an inclusive scan by DPP moves -- row_shr 1, 2, 4, 8 within each
// row of 16 lanes, then row_bcast 15 and 31 carry a row's last lane into the
// next rows -- leaves the total in lane 63, which readlane broadcasts.  A lane
// with no source in a step reads 0, the identity of both.  Six VALU
// instructions with fused DPP operands, against about thirty for a butterfly
// of ds_bpermute shuffles.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_move<0x111>(x));       // row_shr:1
  x = max(x, dpp_move<0x112>(x));       // row_shr:2
  x = max(x, dpp_move<0x114>(x));       // row_shr:4
  x = max(x, dpp_move<0x118>(x));       // row_shr:8
  x = max(x, dpp_move<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
  x = max(x, dpp_move<0x143, 0xC>(x));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += dpp_move<0x111>(x);
  x += dpp_move<0x112>(x);
  x += dpp_move<0x114>(x);
  x += dpp_move<0x118>(x);
  x += dpp_move<0x142, 0xA>(x);
  x += dpp_move<0x143, 0xC>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Logical work item (chunk or part) of this work-group.  Work-groups are
// dispatched round-robin over the 8 XCDs (work-group b runs on XCD b % 8).
// In XCD order, work-group b takes item (b % 8) * ceil(n/8) + b / 8, so each
// XCD streams through its own contiguous eighth of the list (measured: update
// pass -3%, block pass -5%); the grid is then 8 * ceil(n/8) and a surplus
// work-group gets -1 (returns at once).  The amax pass and the fix-up keep
// the linear order (XCD order measured +4% there, and it would put a flagged
// tensor's chunks on few XCDs).
template <bool XCD>
__device__ __forceinline__ int64_t work_index(int64_t n) {
  if constexpr (XCD) {
    const int64_t per = (n + 7) >> 3;
    const int64_t w = (int64_t)(blockIdx.x & 7u) * per + (int64_t)(blockIdx.x >> 3);
    return w < n ? w : -1;
  } else {
    (void)n;
    return (int64_t)blockIdx.x;
  }
}

template <bool XCD>
inline unsigned grid_for(int64_t n) {
  return XCD ? (unsigned)(((n + 7) >> 3) << 3) : (unsigned)n;
}

constexpr bool kXcdStreams = FP8ADAM_XCD_ORDER != 0;  // update and block passes

// Work-group max of two values over TH threads; result valid in thread 0.
template <int TH = kThreads>
__device__ __forceinline__ void block_max2(uint32_t& a, uint32_t& b) {
  __shared__ uint32_t red[2][TH / 64];
  a = wave_max(a);
  b = wave_max(b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][wave] = a;
    red[1][wave] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < TH / 64; w++) {
      a = max(a, red[0][w]);
      b = max(b, red[1][w]);
    }
  }
}

template <bool STATS>
__device__ __forceinline__ void flush_counters(unsigned long long* counters, int tid,
                                               const uint32_t (&cnt)[kStatsPerTensor]) {
  if constexpr (STATS) {
#pragma unroll
    for (int k = 0; k < kStatsPerTensor; k++) {
      const uint32_t s = wave_sum(cnt[k]);
      if ((threadIdx.x & 63) == 0 && s != 0)
        atomicAdd(&counters[(int64_t)tid * kStatsPerTensor + k], (unsigned long long)s);
    }
  }
}

template <int MF, int VF, bool STATS>
__device__ __forceinline__ void count_element(uint32_t (&cnt)[kStatsPerTensor], float m1, float v1,
                                              float qm, float qv, uint32_t cm, uint32_t cv) {
  if constexpr (STATS) {
    cnt[kUnderM] += (m1 != 0.0f && (cm & 0x7Fu) == 0u);
    cnt[kUnderV] += (v1 != 0.0f && (cv & 0x7Fu) == 0u);
    cnt[kSatM] += (fabsf(qm) > Format<MF>::kMax);
    cnt[kSatV] += (fabsf(qv) > Format<VF>::kMax);
    cnt[kNonFinite] += (!isfinite(m1) || !isfinite(v1));
  }
}

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu2 __attribute__((ext_vector_type(2)));
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));

// Streamed loads and stores (optionally non-temporal: the data is touched once per pass).
// The tensor pointers come from a descriptor in memory, so the compiler cannot
// prove they are global and would emit flat instructions; these helpers cast
// them into the global address space (global_load / global_store).
#define FP8ADAM_GLOBAL __attribute__((address_space(1)))

template <typename T, bool NT>
__device__ __forceinline__ T ld_stream(const void* p) {
  const FP8ADAM_GLOBAL T* g = (const FP8ADAM_GLOBAL T*)(p);
  if constexpr (NT) return __builtin_nontemporal_load(g);
  else return *g;
}

template <typename T, bool NT>
__device__ __forceinline__ void st_stream(void* p, T x) {
  FP8ADAM_GLOBAL T* g = (FP8ADAM_GLOBAL T*)(p);
  if constexpr (NT) __builtin_nontemporal_store(x, g);
  else *g = x;
}

template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
  return *(const FP8ADAM_GLOBAL T*)(p);
}

template <typename T>
__device__ __forceinline__ void st_global(void* p, T x) {
  *(FP8ADAM_GLOBAL T*)(p) = x;
}

// Loads of one group of four consecutive elements.
struct Group {
  vu2 g;         // 4 bf16
  uint32_t cm;   // 4 codes
  uint32_t cv;   // 4 codes
  vf4 p;         // fp32 master (or 4 bf16 in .x/.y)
};

// Buffer instructions for the streamed accesses of the amax, update and block
// passes.  A work-group addresses its own part of a tensor through buffer
// resources based at the part's first element (64-bit base in scalar
// registers, 32-bit offsets within the part).  On the update pass's byte mix
// (read 16 + 8 + 4 + 4, write 16 + 4 + 4 bytes per lane, one-shot 1024-element
// work-groups, non-temporal) buffer loads and stores streamed 6.42-6.49 TB/s
// against 6.02-6.08 TB/s for global ones (three runs each, one box).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
constexpr int kLdPol = FP8ADAM_BUF_LOAD_POLICY;
constexpr int kStPol = FP8ADAM_BUF_STORE_POLICY;

// Resource over [base, base + bytes); bytes < 2^31 (a part or a chunk).
__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// The four input streams of elements [start, start + len) of a tensor (m, v:
// the code buffers read).
struct PartBufs {
  Rsrc p, g, m, v;
};

template <bool BF16P>
__device__ __forceinline__ PartBufs part_bufs(const TensorDesc& d, const uint8_t* m, const uint8_t* v, int64_t start,
                                              int64_t len) {
  constexpr int64_t PB = BF16P ? 2 : 4;
  return PartBufs{rsrc(static_cast<const char*>(d.p) + PB * start, PB * len), rsrc(d.g + start, 2 * len),
                  rsrc(m + start, len), rsrc(v + start, len)};
}

// Loads of the group of four elements at offset o (elements) of the part.
template <bool BF16P>
__device__ __forceinline__ void load_group_buf(const PartBufs& B, uint32_t o, Group& G, bool with_p) {
  G.g = __builtin_amdgcn_raw_buffer_load_b64(B.g, 2 * o, 0, kLdPol);
  G.cm = __builtin_amdgcn_raw_buffer_load_b32(B.m, o, 0, kLdPol);
  G.cv = __builtin_amdgcn_raw_buffer_load_b32(B.v, o, 0, kLdPol);
  if (with_p) {
    if constexpr (BF16P) {
      const vu2 pb = __builtin_amdgcn_raw_buffer_load_b64(B.p, 2 * o, 0, kLdPol);
      G.p = vf4{__uint_as_float(pb.x), __uint_as_float(pb.y), 0.0f, 0.0f};
    } else {
      const vu4 x = __builtin_amdgcn_raw_buffer_load_b128(B.p, 4 * o, 0, kLdPol);
      G.p = vf4{__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
    }
  }
}

// Stores of the group at offset o: the four weights and the two code words.
template <bool BF16P>
__device__ __forceinline__ void store_group_buf(Rsrc bp, Rsrc bm, Rsrc bv, uint32_t o, const float (&p)[4],
                                                uint32_t wm, uint32_t wv) {
  if constexpr (BF16P) {
    __builtin_amdgcn_raw_buffer_store_b64(vu2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])}, bp, 2 * o, 0, kStPol);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(
        vu4{__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3])}, bp, 4 * o, 0,
        kStPol);
  }
  __builtin_amdgcn_raw_buffer_store_b32(wm, bm, o, 0, kStPol);
  __builtin_amdgcn_raw_buffer_store_b32(wv, bv, o, 0, kStPol);
}

// Unpack 4 grads, 4 dequantized moments, and the fresh moments.  p (the
// parameters before the step) is read only with coupled L2.
template <int MF, int VF, bool L2>
__device__ __forceinline__ void fresh_moments(const StepConsts& c, const Group& G, const float (&p)[4], float sm,
                                              float sv, float (&m1)[4], float (&v1)[4]) {
  const float g[4] = {bf16_lo(G.g.x), bf16_hi(G.g.x), bf16_lo(G.g.y), bf16_hi(G.g.y)};
  float m[4], v[4];
  decode4<MF>(G.cm, m);
  decode4<VF>(G.cv, v);
#pragma unroll
  for (int j = 0; j < 4; j++) moment_update(c, grad_in<L2>(c, g[j], p[j]), m[j] * sm, v[j] * sv, m1[j], v1[j]);
}

template <bool BF16P>
__device__ __forceinline__ void unpack_p(const Group& G, float (&p)[4]) {
  if constexpr (BF16P) {
    const uint32_t a = __float_as_uint(G.p.x), b = __float_as_uint(G.p.y);
    p[0] = bf16_lo(a); p[1] = bf16_hi(a); p[2] = bf16_lo(b); p[3] = bf16_hi(b);
  } else {
    p[0] = G.p.x; p[1] = G.p.y; p[2] = G.p.z; p[3] = G.p.w;
  }
}

template <bool BF16P>
__device__ __forceinline__ float load_p1(const TensorDesc& d, int64_t i) {
  if constexpr (BF16P) return __uint_as_float((uint32_t)ld_global<uint16_t>(static_cast<const uint16_t*>(d.p) + i) << 16);
  else return ld_global<float>(static_cast<const float*>(d.p) + i);
}

__device__ __forceinline__ float load_g1(const TensorDesc& d, int64_t i) {
  return __uint_as_float((uint32_t)ld_global<uint16_t>(d.g + i) << 16);
}

template <bool BF16P>
__device__ __forceinline__ void store_p1(const TensorDesc& d, int64_t i, float x) {
  if constexpr (BF16P) st_global<uint16_t>(static_cast<uint16_t*>(d.p) + i, (uint16_t)f32_to_bf16_rne(x));
  else st_global<float>(static_cast<float*>(d.p) + i, x);
}

// Speculative schedule: the predicted scale is the POW2 scale of the previous
// step's amax times the predicted growth of the moving average from step t-1
// to t (StepConsts::grow_m / grow_v).  Without a usable previous amax (zero or
// non-finite) it is the power of two with the exponent of the tensor's current
// scale (1 if that is zero, subnormal, Inf or NaN).  The update pass and the
// check evaluate exactly the same expression, so they agree on the prediction.
__device__ __forceinline__ uint32_t exponent_scale_bits(float s_old) {
  const uint32_t e = (__float_as_uint(s_old) >> 23) & 0xFFu;
  if (e == 0u || e == 255u) return 0x3F800000u;
  return e << 23;
}

template <int FMT>
__device__ __forceinline__ uint32_t predicted_scale_bits(uint32_t amax_prev, float s_old, float growth) {
  if (amax_prev == 0u || (amax_prev >> 23) >= 255u) return exponent_scale_bits(s_old);
  float s, inv;
  choose_scale<FMT, 0>(__float_as_uint(__uint_as_float(amax_prev) * growth) & 0x7FFFFFFFu, s, inv);
  return __float_as_uint(s);
}

__device__ __forceinline__ float inverse_pow2(uint32_t pow2_bits) {
  return __uint_as_float((254u - (pow2_bits >> 23)) << 23);
}

// Delayed scaling: the scale of the largest entry of a tensor's amax history
// (H entries, sign bits ignored; a non-finite entry gives scale 1) times
// 2^margin.  Called by whole waves; every lane gets the same s and inv.
template <int FMT, int SMODE>
__device__ __forceinline__ void delayed_scale(const float* h, const StepConsts& c, float& s, float& inv) {
  uint32_t r = 0;
  for (int j = threadIdx.x & 63; j < c.hist_len; j += 64) r = max(r, abs_bits(ld_global<float>(h + j)));
  r = wave_max(r);
  choose_scale<FMT, SMODE>(abs_bits(__uint_as_float(r) * c.margin_scale), s, inv);
}

// ------------------------------------------------------------------ pass 1

// The amax of |m'| and of v' over the elements [start, end) of tensor d (whole
// groups of 4 through buffer loads, then a ragged tail of < 4 elements at the
// tensor's end), each lane's share folded into am / av.
template <int MF, int VF, bool BF16P, bool L2>
__device__ __forceinline__ void range_amax(const StepConsts& c, const TensorDesc& d, int64_t start, int64_t end,
                                           uint32_t& am, uint32_t& av) {
  const int64_t gend = start + ((end - start) & ~(int64_t)3);  // end of whole groups
  const float sm = ld_global<float>(d.sm), sv = ld_global<float>(d.sv);
  const PartBufs B = part_bufs<BF16P>(d, d.m, d.v, start, end - start);
  for (int64_t base = start + kGroup * threadIdx.x; base < gend; base += (int64_t)kSubTile * kAmaxUnroll) {
    Group G[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; u++) {
      const int64_t i = base + (int64_t)u * kSubTile;
      if (i < gend) load_group_buf<BF16P>(B, (uint32_t)(i - start), G[u], L2);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; u++) {
      const int64_t i = base + (int64_t)u * kSubTile;
      if (i < gend) {
        float m1[4], v1[4], p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (L2) unpack_p<BF16P>(G[u], p);
        fresh_moments<MF, VF, L2>(c, G[u], p, sm, sv, m1, v1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          am = max(am, abs_bits(m1[j]));
          av = max(av, abs_bits(v1[j]));
        }
      }
    }
  }
  if (gend + threadIdx.x < end) {
    const int64_t i = gend + threadIdx.x;
    const float g = grad_in<L2>(c, load_g1(d, i), L2 ? load_p1<BF16P>(d, i) : 0.0f);
    float m1, v1;
    moment_update(c, g, decode1<MF>(ld_global<uint8_t>(d.m + i)) * sm, decode1<VF>(ld_global<uint8_t>(d.v + i)) * sv, m1, v1);
    am = max(am, abs_bits(m1));
    av = max(av, abs_bits(v1));
  }
}

template <int MF, int VF, bool BF16P, bool L2>
__global__ __launch_bounds__(kThreads) void k_amax(const TensorDesc* __restrict__ descs,
                                                   const int32_t* __restrict__ chunk_tid,
                                                   uint2* __restrict__ partial, StepConsts c, int chunk_log2,
                                                   int64_t nwork, const GradCtl* __restrict__ gctl) {
  const int64_t w = work_index<false>(nwork);
  if (w < 0 || amp_apply(gctl, c)) return;
  const int tid = chunk_tid[w];
  const TensorDesc d = descs[tid];
  const int64_t start = (w - d.chunk0) << chunk_log2;
  const int64_t end = min(start + ((int64_t)1 << chunk_log2), d.numel);
  uint32_t am = 0, av = 0;
  range_amax<MF, VF, BF16P, L2>(c, d, start, end, am, av);
  block_max2(am, av);
  if (threadIdx.x == 0) partial[w] = make_uint2(am, av);
}

// ------------------------------------------------------------------ reduce
//
// One work-group per tensor: amax over the tensor's chunk partials (unsigned
// max of fp32 bit patterns of non-negative values: exact and order-free),
// then the old scales are staged for the update pass and the new scales are
// written into the caller's slots.  Non-finite amax (NaN/Inf bit patterns
// are the largest) gives scale 1.

template <int MF, int VF, int SMODE, bool STATS>
__global__ __launch_bounds__(kReduceThreads) void k_reduce(const TensorDesc* __restrict__ descs,
                                                           const uint2* __restrict__ partial,
                                                           uint32_t* __restrict__ amax,
                                                           float* __restrict__ old_scale,
                                                           unsigned long long* __restrict__ counters,
                                                           int chunk_log2, int32_t* __restrict__ flags,
                                                           int hist_len, int hist_slot,
                                                           const GradCtl* __restrict__ gctl) {
  const int t = blockIdx.x;
  if (gctl != nullptr && gctl->skip) {  // skipped step: scales, amax and history stay
    if (threadIdx.x == 0) flags[t] = 0;
    if (STATS && threadIdx.x < kStatsPerTensor) counters[(int64_t)t * kStatsPerTensor + threadIdx.x] = 0ull;
    return;
  }
  if (gctl != nullptr) hist_slot = gctl->hist_slot;
  const TensorDesc d = descs[t];
  const int64_t nc = (d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
  uint32_t am = 0, av = 0;
  for (int64_t k = threadIdx.x; k < nc; k += kReduceThreads) {
    const uint2 pv = partial[d.chunk0 + k];
    am = max(am, pv.x);
    av = max(av, pv.y);
  }
  __shared__ uint32_t red[2][kReduceThreads / 64];
  am = wave_max(am);
  av = wave_max(av);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][wave] = am;
    red[1][wave] = av;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kReduceThreads / 64; w++) {
      am = max(am, red[0][w]);
      av = max(av, red[1][w]);
    }
    amax[2 * t] = am;
    amax[2 * t + 1] = av;
    flags[t] = 0;
    if (d.numel > 0) {
      old_scale[2 * t] = ld_global<float>(d.sm);
      old_scale[2 * t + 1] = ld_global<float>(d.sv);
      float s, inv;
      choose_scale<MF, SMODE>(am, s, inv);
      st_global<float>(d.sm, s);
      choose_scale<VF, SMODE>(av, s, inv);
      st_global<float>(d.sv, s);
      if (hist_len > 0) {  // just-in-time step of delayed scaling: seed the history
        st_global<float>(d.hist + hist_slot, __uint_as_float(am));
        st_global<float>(d.hist + hist_len + hist_slot, __uint_as_float(av));
      }
    }
  }
  if constexpr (STATS) {
    if (threadIdx.x < kStatsPerTensor) counters[(int64_t)t * kStatsPerTensor + threadIdx.x] = 0ull;
  }
}

// ------------------------------------------------------------------ pass 2

// Eight waves per SIMD: the buffer resources raise the stochastic-rounding
// instantiations to 98-101 scalar registers, which leaves room for seven waves;
// held to eight (a few scalar registers spill to vector lanes), the speculative
// stochastic-rounding pass runs within 0.2% of the round-to-nearest one (in one
// process on the same buffers: 15.20 against 15.18 ms on the 7B list, against
// 15.23-15.26 ms at seven waves).
template <int MF, int VF, bool BF16P, bool STATS, int SMODE, int MODE, bool L2, bool SR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_update(const TensorDesc* __restrict__ descs,
                                                     const TensorDesc* __restrict__ dst_descs,
                                                     const int32_t* __restrict__ chunk_tid,
                                                     const uint32_t* __restrict__ amax,
                                                     const float* __restrict__ old_scale, StepConsts c,
                                                     unsigned long long* __restrict__ counters, int chunk_log2,
                                                     uint2* __restrict__ part_amax, int64_t nwork,
                                                     const GradCtl* __restrict__ gctl) {
  constexpr bool SPEC = MODE == kModeSpec;
  constexpr bool PARTS = MODE != kModeJit;  // per-part amax partials for the commit kernel
  const int64_t w = work_index<kXcdStreams>(nwork);
  if (w < 0) return;
  constexpr int PL = upd_part_log2<BF16P>();
  const int split_log2 = chunk_log2 - PL;
  const int64_t chunk = w >> split_log2;
  const int tid = chunk_tid[chunk];
  const TensorDesc d = descs[tid];
  const int64_t start = ((chunk - d.chunk0) << chunk_log2) + ((w & ((1 << split_log2) - 1)) << PL);
  const int64_t end = min(start + ((int64_t)1 << PL), d.numel);
  if (start >= end) return;  // empty part at the end of a tensor (uniform for the work-group)
  const int64_t gend = start + ((end - start) & ~(int64_t)3);
  // codes go back in place (two-pass) or into the other buffer (speculative)
  uint8_t* const dm = SPEC ? dst_descs[tid].m : d.m;
  uint8_t* const dv = SPEC ? dst_descs[tid].v : d.v;
  if (amp_apply(gctl, c)) {  // skipped step
    // the speculative schedule switches buffers regardless: carry the codes over
    if constexpr (SPEC) {
      for (int64_t i = start + kGroup * threadIdx.x; i < gend; i += kSubTile) {
        st_global<uint32_t>(dm + i, ld_global<uint32_t>(d.m + i));
        st_global<uint32_t>(dv + i, ld_global<uint32_t>(d.v + i));
      }
      if (gend + threadIdx.x < end) {
        st_global<uint8_t>(dm + gend + threadIdx.x, ld_global<uint8_t>(d.m + gend + threadIdx.x));
        st_global<uint8_t>(dv + gend + threadIdx.x, ld_global<uint8_t>(d.v + gend + threadIdx.x));
      }
    }
    return;
  }
  float sm, sv, ism, isv;
  if constexpr (SPEC) {
    // prepared per tensor by k_spec_prepare: [old s_m, old s_v, predicted s_m, predicted s_v]
    sm = old_scale[4 * tid];
    sv = old_scale[4 * tid + 1];
    ism = inverse_pow2(__float_as_uint(old_scale[4 * tid + 2]));
    isv = inverse_pow2(__float_as_uint(old_scale[4 * tid + 3]));
  } else if constexpr (MODE == kModeDelayed) {
    // the delayed scales, prepared per tensor by k_delayed_prepare: [s_m, s_v, inv_m, inv_v]
    sm = ld_global<float>(d.sm);
    sv = ld_global<float>(d.sv);
    ism = old_scale[4 * tid + 2];
    isv = old_scale[4 * tid + 3];
  } else {
    float nsm, nsv;
    sm = old_scale[2 * tid];
    sv = old_scale[2 * tid + 1];
    choose_scale<MF, SMODE>(amax[2 * tid], nsm, ism);
    choose_scale<VF, SMODE>(amax[2 * tid + 1], nsv, isv);
  }
  uint32_t am = 0, av = 0;  // speculative / delayed: this part's amax
  uint32_t cnt[kStatsPerTensor] = {0, 0, 0, 0, 0};
  const PartBufs B = part_bufs<BF16P>(d, d.m, d.v, start, end - start);
  const Rsrc bdm = rsrc(dm + start, end - start), bdv = rsrc(dv + start, end - start);

  for (int64_t base = start + kGroup * threadIdx.x; base < gend; base += (int64_t)kSubTile * kUpdUnroll) {
    Group G[kUpdUnroll];
#pragma unroll
    for (int u = 0; u < kUpdUnroll; u++) {
      const int64_t i = base + (int64_t)u * kSubTile;
      if (i < gend) load_group_buf<BF16P>(B, (uint32_t)(i - start), G[u], true);
    }
#pragma unroll
    for (int u = 0; u < kUpdUnroll; u++) {
      const int64_t i = base + (int64_t)u * kSubTile;
      if (i < gend) {
        float m1[4], v1[4], p[4], qm[4], qv[4];
        unpack_p<BF16P>(G[u], p);
        fresh_moments<MF, VF, L2>(c, G[u], p, sm, sv, m1, v1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          p[j] = param_update(c, p[j], m1[j], v1[j]);
          qm[j] = m1[j] * ism;
          qv[j] = v1[j] * isv;
          if constexpr (PARTS) {
            am = max(am, abs_bits(m1[j]));
            av = max(av, abs_bits(v1[j]));
          }
        }
        uint32_t rw[4];
        sr_words<SR>(c, tid, i, rw);
        const uint32_t wm = quant4<MF, SR, false>(qm, rw);
        const uint32_t wv = quant4<VF, SR, true>(qv, rw);
        if constexpr (STATS) {
#pragma unroll
          for (int j = 0; j < 4; j++)
            count_element<MF, VF, STATS>(cnt, m1[j], v1[j], qm[j], qv[j], wm >> (8 * j), wv >> (8 * j));
        }
        store_group_buf<BF16P>(B.p, bdm, bdv, (uint32_t)(i - start), p, wm, wv);
      }
    }
  }
  if (gend + threadIdx.x < end) {
    const int64_t i = gend + threadIdx.x;
    const float p0 = load_p1<BF16P>(d, i);
    const float g = grad_in<L2>(c, load_g1(d, i), p0);
    float m1, v1;
    moment_update(c, g, decode1<MF>(ld_global<uint8_t>(d.m + i)) * sm, decode1<VF>(ld_global<uint8_t>(d.v + i)) * sv, m1, v1);
    const float p = param_update(c, p0, m1, v1);
    const float qm = m1 * ism, qv = v1 * isv;
    const uint32_t w = sr_word1<SR>(c, tid, i);
    const uint32_t cm = quant1<MF, SR, false>(w, qm), cv = quant1<VF, SR, true>(w, qv);
    count_element<MF, VF, STATS>(cnt, m1, v1, qm, qv, cm, cv);
    if constexpr (PARTS) {
      am = max(am, abs_bits(m1));
      av = max(av, abs_bits(v1));
    }
    store_p1<BF16P>(d, i, p);
    st_global<uint8_t>(dm + i, (uint8_t)cm);
    st_global<uint8_t>(dv + i, (uint8_t)cv);
  }
  flush_counters<STATS>(counters, tid, cnt);
  if constexpr (PARTS) {
    block_max2(am, av);
    if (threadIdx.x == 0) part_amax[w] = make_uint2(am, av);
  }
}

// Max over a tensor's per-part amax partials, strided over the work-group's
// kReduceThreads lanes with eight loads in flight per lane (the largest
// tensors have 10^5 parts, so a one-load-at-a-time loop is latency-bound).
__device__ __forceinline__ void parts_max(const uint2* __restrict__ parts, int64_t nparts, uint32_t& am,
                                          uint32_t& av) {
  constexpr int U = 8;
  int64_t k = threadIdx.x;
  for (; k + (U - 1) * kReduceThreads < nparts; k += U * kReduceThreads) {
    uint2 pv[U];
#pragma unroll
    for (int u = 0; u < U; u++) pv[u] = parts[k + u * kReduceThreads];
#pragma unroll
    for (int u = 0; u < U; u++) {
      am = max(am, pv[u].x);
      av = max(av, pv[u].y);
    }
  }
  for (; k < nparts; k += kReduceThreads) {
    const uint2 pv = parts[k];
    am = max(am, pv.x);
    av = max(av, pv.y);
  }
}

// ------------------------------------------------------- delayed: commit
//
// One work-group per tensor, after the delayed pass: the tensor's amax from the
// per-part partials; wave 0 recomputes the delayed scales exactly as the pass
// did (before the history changes), thread 0 commits them and records this
// step's amax in the history slot.

// One wave per tensor, before the delayed pass: the tensor's delayed scales
// from its amax history, into prep[4t..4t+3] = [s_m, s_v, inv_m, inv_v], so
// the pass and the commit read them instead of reducing the history in every
// work-group.
template <int MF, int VF, int SMODE>
__global__ __launch_bounds__(64) void k_delayed_prepare(const TensorDesc* __restrict__ descs, StepConsts c,
                                                        float* __restrict__ prep) {
  const int t = blockIdx.x;
  const TensorDesc d = descs[t];
  if (d.numel == 0) return;  // uniform: the whole wave
  float s_m, s_v, i_m, i_v;
  delayed_scale<MF, SMODE>(d.hist, c, s_m, i_m);
  delayed_scale<VF, SMODE>(d.hist + c.hist_len, c, s_v, i_v);
  if (threadIdx.x == 0) {
    st_global<float>(prep + 4 * t, s_m);
    st_global<float>(prep + 4 * t + 1, s_v);
    st_global<float>(prep + 4 * t + 2, i_m);
    st_global<float>(prep + 4 * t + 3, i_v);
  }
}

template <int MF, int VF, int SMODE>
__global__ __launch_bounds__(kReduceThreads) void k_delayed_reduce(const TensorDesc* __restrict__ descs,
                                                                   const uint2* __restrict__ part_amax,
                                                                   uint32_t* __restrict__ amax, StepConsts c,
                                                                   int chunk_log2, int part_log2,
                                                                   const GradCtl* __restrict__ gctl,
                                                                   const float* __restrict__ prep) {
  if (amp_apply(gctl, c)) return;  // skipped step: scales, amax and history stay
  const int t = blockIdx.x;
  const TensorDesc d = descs[t];
  const int64_t nparts = (d.numel + ((int64_t)1 << part_log2) - 1) >> part_log2;
  const int64_t part0 = d.chunk0 << (chunk_log2 - part_log2);
  uint32_t am = 0, av = 0;
  parts_max(part_amax + part0, nparts, am, av);
  __shared__ uint32_t red[2][kReduceThreads / 64];
  am = wave_max(am);
  av = wave_max(av);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][wave] = am;
    red[1][wave] = av;
  }
  __syncthreads();
  if (wave == 0 && d.numel > 0) {  // uniform: all of wave 0, or none
    const float s_m = prep[4 * t], s_v = prep[4 * t + 1];  // the scales the pass quantized with
    if (lane == 0) {
      for (int w = 1; w < kReduceThreads / 64; w++) {
        am = max(am, red[0][w]);
        av = max(av, red[1][w]);
      }
      st_global<float>(d.sm, s_m);
      st_global<float>(d.sv, s_v);
      st_global<float>(d.hist + c.hist_slot, __uint_as_float(am));
      st_global<float>(d.hist + c.hist_len + c.hist_slot, __uint_as_float(av));
      amax[2 * t] = am;
      amax[2 * t + 1] = av;
    }
  } else if (threadIdx.x == 0) {
    amax[2 * t] = 0u;
    amax[2 * t + 1] = 0u;
  }
}

// ------------------------------------------------- speculative: verify, fix up
//
// After the speculative pass: the max of the per-part amax partials over each
// chunk, into chunk_amax (the amax pass's partials buffer, free in a
// speculative step), so that the check, one work-group per tensor, reads
// 2^(chunk_log2 - PL) times fewer values.  A chunk's partials are contiguous:
// L lanes read them 16 bytes (two parts) each and reduce by shuffles, so a
// wave folds 64 / L chunks.  The partials of parts past a tensor's end are
// never written by the pass and stay 0 from init.
template <int PL>
__global__ __launch_bounds__(kThreads) void k_part_fold(const uint2* __restrict__ part_amax,
                                                        uint2* __restrict__ chunk_amax, int chunk_log2,
                                                        int64_t nchunks, StepConsts c,
                                                        const GradCtl* __restrict__ gctl) {
  if (amp_apply(gctl, c)) return;  // skipped step: the pass wrote no partials
  const int split = chunk_log2 - PL;              // parts per chunk: 2^split, 2..32
  const int lanes = split > 1 ? 1 << (split - 1) : 1;  // lanes per chunk, two parts each
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t chunk = g / lanes;
  const int sub = (int)(g % lanes);
  uint32_t am = 0, av = 0;
  if (chunk < nchunks) {
    const vu4 two = ld_global<vu4>(part_amax + (chunk << split) + 2 * sub);
    am = max(two.x, two.z);
    av = max(two.y, two.w);
  }
  for (int o = lanes >> 1; o > 0; o >>= 1) {  // within the chunk's aligned group of lanes
    am = max(am, (uint32_t)__shfl_xor((int)am, o));
    av = max(av, (uint32_t)__shfl_xor((int)av, o));
  }
  if (chunk < nchunks && sub == 0) chunk_amax[chunk] = make_uint2(am, av);
}

//
// One work-group per tensor: the true amax from the per-part partials, the
// true POW2 scales, and a comparison with the predicted ones.  The old scales
// are staged for the fix-up, the true scales committed; a flagged tensor's
// stats counters are cleared (the fix-up recounts them).

// Speculative schedule, first kernel of the step: the exact amax of |m'| and
// v' over the candidate parts that the last step's k_spec_reduce listed (the
// parts that held values near their tensor's amax), atomically maxed into
// lb[2t], lb[2t+1].  It reads g and the old codes of those parts only (about
// 1% of the list) and bounds this step's amax from below; k_spec_prepare
// predicts the scale from it.  The work list holds *cand_count entries
// (tensor, part index within the tensor), each tensor's entries adjacent.  A
// work-group takes R consecutive entries per round and issues all their loads
// before it computes (8 accesses of 1024 elements in flight), and folds its
// running max into lb only where the tensor changes and at the round's end.
// PL is the update pass's part size (log2).
constexpr int kProbeAccesses = 8;

template <int MF, int VF, int PL>
__global__ __launch_bounds__(kThreads) void k_spec_probe(const TensorDesc* __restrict__ descs, StepConsts c,
                                                         const uint32_t* __restrict__ cand_count,
                                                         const uint2* __restrict__ cand_work,
                                                         uint32_t* __restrict__ lb, const GradCtl* __restrict__ gctl) {
  constexpr int A = (1 << PL) / kSubTile;  // accesses per entry
  constexpr int R = kProbeAccesses / A;    // entries per round
  static_assert(A >= 1 && R >= 1 && (1 << PL) % kSubTile == 0, "whole accesses per part");
  if (amp_apply(gctl, c)) return;  // skipped step: nothing to predict
  const int64_t nwork = ld_global<uint32_t>(cand_count);
  for (int64_t w0 = (int64_t)blockIdx.x * R; w0 < nwork; w0 += (int64_t)gridDim.x * R) {
    uint2 e[R];
    Group G[R][A];
    // every load of the round is issued before any is used: buffer loads bounded
    // by the part's length (past it they read 0, so no lane branches here)
#pragma unroll
    for (int u = 0; u < R; u++) {
      e[u] = w0 + u < nwork ? cand_work[w0 + u] : make_uint2(0xFFFFFFFFu, 0u);
      if (e[u].x == 0xFFFFFFFFu) continue;  // past the list's end (uniform)
      const TensorDesc d = descs[e[u].x];
      const int64_t start = (int64_t)e[u].y << PL;
      const PartBufs B = part_bufs<false>(d, d.m, d.v, start, min((int64_t)1 << PL, d.numel - start));
#pragma unroll
      for (int a = 0; a < A; a++) load_group_buf<false>(B, a * kSubTile + kGroup * threadIdx.x, G[u][a], false);
    }
    uint32_t cur = e[0].x, am = 0, av = 0;
#pragma unroll
    for (int u = 0; u < R; u++) {
      if (e[u].x == 0xFFFFFFFFu) break;  // past the list's end (uniform)
      if (e[u].x != cur) {               // uniform: every lane reads the same entries
        block_max2(am, av);
        if (threadIdx.x == 0) {
          atomicMax(lb + 2 * cur, am);
          atomicMax(lb + 2 * cur + 1, av);
        }
        __syncthreads();  // block_max2's LDS is written again
        cur = e[u].x;
        am = av = 0;
      }
      const TensorDesc d = descs[e[u].x];
      const float sm = ld_global<float>(d.sm), sv = ld_global<float>(d.sv);
      const int64_t end = min(((int64_t)e[u].y + 1) << PL, d.numel);
#pragma unroll
      for (int a = 0; a < A; a++) {
        // elements past the part read as zero codes and gradients: m' = v' = 0
        float m1[4], v1[4];
        const float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        fresh_moments<MF, VF, false>(c, G[u][a], p, sm, sv, m1, v1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          am = max(am, abs_bits(m1[j]));
          av = max(av, abs_bits(v1[j]));
        }
        // the ragged end of a tensor (< 4 elements, in a group the buffer range cuts)
        const int64_t i = ((int64_t)e[u].y << PL) + a * kSubTile + kGroup * threadIdx.x;
        if (i < end && i + kGroup > end) {
          for (int64_t k = i; k < end; k++) {
            float m1s, v1s;
            moment_update(c, load_g1(d, k), decode1<MF>(ld_global<uint8_t>(d.m + k)) * sm,
                          decode1<VF>(ld_global<uint8_t>(d.v + k)) * sv, m1s, v1s);
            am = max(am, abs_bits(m1s));
            av = max(av, abs_bits(v1s));
          }
        }
      }
    }
    block_max2(am, av);
    if (threadIdx.x == 0) {
      atomicMax(lb + 2 * cur, am);
      atomicMax(lb + 2 * cur + 1, av);
    }
    __syncthreads();  // block_max2's LDS is written again in the next round
  }
}

// The POW2 scale of an amax given as fp32 bits (the rule the check applies).
template <int FMT>
__device__ __forceinline__ uint32_t scale_bits_of(uint32_t amax_bits) {
  float s, inv;
  choose_scale<FMT, 0>(amax_bits, s, inv);
  return __float_as_uint(s);
}

// One thread per tensor, after the probe: stage the old scales and the
// predicted ones in prep[4t..4t+3] = [s_m, s_v, pred s_m, pred s_v] (the pass,
// the check and the fix-up all read them from there).  A moment predicts from
// the probe's bound when its tensor listed candidates at the last step and its
// amax there was nonzero (then the part that held it is among them), else from
// the last amax times the growth model.  lb is cleared for the next step, and
// probed[t] records the elements the probe read (for the stats).
template <int MF, int VF>
__global__ __launch_bounds__(64) void k_spec_prepare(const TensorDesc* __restrict__ descs,
                                                     const uint32_t* __restrict__ amax, StepConsts c,
                                                     const GradCtl* __restrict__ gctl, float* __restrict__ prep,
                                                     int32_t n, uint32_t* __restrict__ fix_count,
                                                     const int32_t* __restrict__ cand_n,
                                                     const int64_t* __restrict__ cand_len, uint32_t* __restrict__ lb,
                                                     int64_t* __restrict__ probed, uint32_t* __restrict__ cand_count) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t == 0) st_global<uint32_t>(fix_count, 0u);  // k_spec_reduce appends this step's fix-up work
  if (t >= n) return;
  if (amp_apply(gctl, c)) {  // skipped step: the candidates stay listed for the next one
    probed[t] = 0;
    return;
  }
  if (t == 0) st_global<uint32_t>(cand_count, 0u);  // the probe has read them; k_spec_reduce lists the next
  const TensorDesc d = descs[t];
  const uint32_t lbm = lb[2 * t], lbv = lb[2 * t + 1];
  lb[2 * t] = 0u;
  lb[2 * t + 1] = 0u;
  const bool listed = cand_n != nullptr && cand_n[t] > 0;  // null: the growth model only
  probed[t] = listed ? cand_len[t] : 0;
  if (d.numel == 0) return;
  const float so_m = ld_global<float>(d.sm), so_v = ld_global<float>(d.sv);
  st_global<float>(prep + 4 * t, so_m);
  st_global<float>(prep + 4 * t + 1, so_v);
  st_global<uint32_t>(prep + 4 * t + 2, listed && amax[2 * t] != 0u ? scale_bits_of<MF>(lbm)
                                                                    : predicted_scale_bits<MF>(amax[2 * t], so_m, c.grow_m));
  st_global<uint32_t>(prep + 4 * t + 3, listed && amax[2 * t + 1] != 0u
                                            ? scale_bits_of<VF>(lbv)
                                            : predicted_scale_bits<VF>(amax[2 * t + 1], so_v, c.grow_v));
}

// The step before the first speculative one runs the amax pass first and then
// the speculative pass with the true scales as its "prediction", so that its
// check lists the probe's candidates for the next step and flags nothing.  One
// work-group per tensor: the amax over the chunk partials of the amax pass,
// staged in prep as [s_m, s_v, true s_m, true s_v] (the caller's slots still
// hold the old scales; the check commits the new ones).
template <int MF, int VF>
__global__ __launch_bounds__(kReduceThreads) void k_exact_prepare(const TensorDesc* __restrict__ descs,
                                                                  const uint2* __restrict__ partial, int chunk_log2,
                                                                  StepConsts c, const GradCtl* __restrict__ gctl,
                                                                  float* __restrict__ prep,
                                                                  uint32_t* __restrict__ fix_count,
                                                                  int64_t* __restrict__ probed,
                                                                  uint32_t* __restrict__ cand_count) {
  const int t = blockIdx.x;
  if (t == 0 && threadIdx.x == 0) st_global<uint32_t>(fix_count, 0u);
  if (threadIdx.x == 0) probed[t] = 0;
  if (amp_apply(gctl, c)) return;  // skipped step: the pass carries the codes over, the check keeps the rest
  if (t == 0 && threadIdx.x == 0) st_global<uint32_t>(cand_count, 0u);
  const TensorDesc d = descs[t];
  const int64_t nc = (d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
  uint32_t am = 0, av = 0;
  for (int64_t k = threadIdx.x; k < nc; k += kReduceThreads) {
    const uint2 pv = partial[d.chunk0 + k];
    am = max(am, pv.x);
    av = max(av, pv.y);
  }
  block_max2<kReduceThreads>(am, av);
  if (threadIdx.x == 0 && d.numel > 0) {
    st_global<float>(prep + 4 * t, ld_global<float>(d.sm));
    st_global<float>(prep + 4 * t + 1, ld_global<float>(d.sv));
    st_global<uint32_t>(prep + 4 * t + 2, scale_bits_of<MF>(am));
    st_global<uint32_t>(prep + 4 * t + 3, scale_bits_of<VF>(av));
  }
}

template <int MF, int VF, bool STATS>
__global__ __launch_bounds__(kReduceThreads) void k_spec_reduce(const TensorDesc* __restrict__ descs,
                                                                const uint2* __restrict__ part_amax,
                                                                const uint2* __restrict__ chunk_amax,
                                                                uint32_t* __restrict__ amax,
                                                                float* __restrict__ old_scale,
                                                                int32_t* __restrict__ flags,
                                                                unsigned long long* __restrict__ counters,
                                                                int chunk_log2, int part_log2, StepConsts c,
                                                                const GradCtl* __restrict__ gctl,
                                                                uint32_t* __restrict__ fix_count,
                                                                uint32_t* __restrict__ fix_list,
                                                                int32_t* __restrict__ cand_n,
                                                                int64_t* __restrict__ cand_len,
                                                                uint32_t* __restrict__ cand_count,
                                                                uint2* __restrict__ cand_work) {
  const int t = blockIdx.x;
  if (amp_apply(gctl, c)) {  // skipped step: scales, amax and candidates stay, nothing to fix up
    if (threadIdx.x == 0) flags[t] = 0;
    return;
  }
  const TensorDesc d = descs[t];
  const int64_t nparts = (d.numel + ((int64_t)1 << part_log2) - 1) >> part_log2;
  const int64_t part0 = d.chunk0 << (chunk_log2 - part_log2);
  const int64_t nchunk = (d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
  uint32_t am = 0, av = 0;
  if (chunk_amax != nullptr) parts_max(chunk_amax + d.chunk0, nchunk, am, av);  // k_part_fold's per-chunk maxima
  else parts_max(part_amax + part0, nparts, am, av);                            // (growth model: no fold)
  __shared__ uint32_t red[2][kReduceThreads / 64];
  __shared__ int32_t flag;
  __shared__ uint32_t list_base;
  __shared__ uint32_t tensor_amax[2];
  __shared__ uint32_t ncand, nchunks_q, cand_base;
  __shared__ unsigned long long candlen;
  __shared__ uint32_t cand_parts[kCandMax];
  __shared__ uint32_t cand_chunks[kCandMax];
  am = wave_max(am);
  av = wave_max(av);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][wave] = am;
    red[1][wave] = av;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kReduceThreads / 64; w++) {
      am = max(am, red[0][w]);
      av = max(av, red[1][w]);
    }
    int32_t f = 0;
    if (d.numel > 0) {
      // the prediction the update pass used, as k_spec_prepare left it (old scales stay staged there)
      const uint32_t pm = __float_as_uint(old_scale[4 * t + 2]);
      const uint32_t pv = __float_as_uint(old_scale[4 * t + 3]);
      float s_m, s_v, inv;
      choose_scale<MF, 0>(am, s_m, inv);
      choose_scale<VF, 0>(av, s_v, inv);
      f = (__float_as_uint(s_m) != pm ? 1 : 0) | (__float_as_uint(s_v) != pv ? 2 : 0);
      st_global<float>(d.sm, s_m);
      st_global<float>(d.sv, s_v);
    }
    amax[2 * t] = am;
    amax[2 * t + 1] = av;
    tensor_amax[0] = am;
    tensor_amax[1] = av;
    ncand = 0u;
    nchunks_q = 0u;
    candlen = 0ull;
    flags[t] = f;
    flag = f;
    // room in the fix-up's work list for the tensor's chunks, once per
    // mispredicted moment (the order there does not matter: every chunk and
    // moment is fixed up on its own)
    const uint32_t nc = (uint32_t)((d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2);
    list_base = f ? atomicAdd(fix_count, nc * (uint32_t)__popc(f)) : 0u;
  }
  __syncthreads();
  if (flag) {  // entries: chunk * 2 + moment (0: m, 1: v)
    const int64_t nc = (d.numel + ((int64_t)1 << chunk_log2) - 1) >> chunk_log2;
    int64_t base = list_base;
    for (int b = 0; b < 2; b++) {
      if (!(flag & (1 << b))) continue;  // uniform
      for (int64_t k = threadIdx.x; k < nc; k += kReduceThreads)
        fix_list[base + k] = (uint32_t)(((d.chunk0 + k) << 1) | b);
      base += nc;
    }
  }
  // the next step's probe candidates: the parts within kCandTheta of this
  // step's amax of either moment (their order in the list does not matter),
  // found among the parts of the chunks whose maximum qualifies
  if (cand_work != nullptr) {  // (null: the growth model predicts, nothing to list; else chunk_amax is set)
    const float am_t = __uint_as_float(tensor_amax[0]), av_t = __uint_as_float(tensor_amax[1]);
    const uint32_t thr_m = tensor_amax[0] != 0u ? __float_as_uint(kCandTheta * am_t) : 0xFFFFFFFFu;
    const uint32_t thr_v = tensor_amax[1] != 0u ? __float_as_uint(kCandTheta * av_t) : 0xFFFFFFFFu;
    const int64_t cap = cand_cap(nparts);
    // a chunk with a candidate part qualifies itself, so more than cap chunks means more than cap parts
    for (int64_t k = threadIdx.x; k < nchunk; k += kReduceThreads) {
      const uint2 cv = chunk_amax[d.chunk0 + k];
      if (cv.x >= thr_m || cv.y >= thr_v) {
        const uint32_t j = atomicAdd(&nchunks_q, 1u);
        if (j < cap) cand_chunks[j] = (uint32_t)k;
      }
    }
    __syncthreads();
    const int split = chunk_log2 - part_log2;
    const int64_t nitems = nchunks_q <= cap ? (int64_t)nchunks_q << split : 0;
    for (int64_t j = threadIdx.x; j < nitems; j += kReduceThreads) {
      const int64_t k = ((int64_t)cand_chunks[j >> split] << split) + (j & ((1 << split) - 1));
      if (k >= nparts) continue;  // past the tensor's last part
      const uint2 pv = part_amax[part0 + k];
      if (pv.x >= thr_m || pv.y >= thr_v) {
        const uint32_t i = atomicAdd(&ncand, 1u);
        if (i < cap) cand_parts[i] = (uint32_t)k;
        atomicAdd(&candlen, (unsigned long long)min((int64_t)1 << part_log2, d.numel - (k << part_log2)));
      }
    }
    __syncthreads();
    const bool fits = nchunks_q <= cap && ncand > 0u && ncand <= cap;  // uniform
    if (threadIdx.x == 0) {
      cand_n[t] = fits ? (int32_t)ncand : 0;
      cand_len[t] = fits ? (int64_t)candlen : 0;
      // room in the probe's work list (this step's k_spec_prepare emptied it)
      cand_base = fits ? atomicAdd(cand_count, ncand) : 0u;
    }
    __syncthreads();
    if (fits)
      for (uint32_t j = threadIdx.x; j < ncand; j += kReduceThreads) cand_work[cand_base + j] = make_uint2(t, cand_parts[j]);
  }
  if constexpr (STATS) {
    // the fix-up recounts the underflow / saturation counts of a re-quantized moment
    if (threadIdx.x == 0 && (flag & 1)) {
      counters[(int64_t)t * kStatsPerTensor + kUnderM] = 0ull;
      counters[(int64_t)t * kStatsPerTensor + kSatM] = 0ull;
    }
    if (threadIdx.x == 0 && (flag & 2)) {
      counters[(int64_t)t * kStatsPerTensor + kUnderV] = 0ull;
      counters[(int64_t)t * kStatsPerTensor + kSatV] = 0ull;
    }
  }
}

// The fix-up, per listed chunk (or piece of one) and mispredicted moment of a
// flagged tensor: bring the moment in the destination buffer to the true scale.  Both scales are powers of two, so most codes only need their
// exponent field moved (shift_codes4: 1 byte read and written per element);
// a group of four with a code that cannot be moved exactly (zero, subnormal,
// FMAX) is recomputed from the gradient and the old codes still intact in the
// source buffer and requantized with the true scale.  p is not touched: its
// update does not depend on the scales.
template <int FMT, bool STATS, bool IS_V, bool SR>
__device__ __forceinline__ uint32_t recompute4(const StepConsts& c, int tid, const TensorDesc& d, int64_t i,
                                               float s_old, float inv_new, uint32_t& under, uint32_t& sat) {
  const vu2 gg = ld_global<vu2>(d.g + i);
  const uint32_t cc = ld_global<uint32_t>((IS_V ? d.v : d.m) + i);
  const float g[4] = {bf16_lo(gg.x), bf16_hi(gg.x), bf16_lo(gg.y), bf16_hi(gg.y)};
  float x[4], q[4];
  decode4<FMT>(cc, x);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    float m1, v1;
    // moment_update computes both moments; only the one being fixed is used
    moment_update(c, g[j] * c.gfac, x[j] * s_old, x[j] * s_old, m1, v1);
    x[j] = IS_V ? v1 : m1;
    q[j] = x[j] * inv_new;
  }
  uint32_t rw[4];
  sr_words<SR>(c, tid, i, rw);
  const uint32_t w = quant4<FMT, SR, IS_V>(q, rw);
  if constexpr (STATS) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      under += (x[j] != 0.0f && ((w >> (8 * j)) & 0x7Fu) == 0u);
      sat += (fabsf(q[j]) > Format<FMT>::kMax);
    }
  }
  return w;
}

template <int FMT, bool STATS, bool IS_V, bool SR>
__device__ __forceinline__ void fixup_moment(const StepConsts& c, int tid, const TensorDesc& d, uint8_t* dst,
                                             int64_t start, int64_t end, float s_old, uint32_t pred_bits,
                                             float s_new, float inv_new, uint32_t& under, uint32_t& sat) {
  // exponent difference of the two powers of two; zero codes stay zero when the
  // values shrink, except where a zero must be checked against its value (the
  // underflow count) or may round up stochastically
  const int dexp = (int)(__float_as_uint(s_new) >> 23) - (int)(pred_bits >> 23);
  const bool zero_ok = !SR && !STATS && dexp > 0;
  // 16 codes per lane per access (a byte stream: wide accesses), then groups
  // of 4 and single elements for the last < 16 of the tensor
  constexpr int kWide = 16;
  constexpr int kWideUnroll = 4;
  const int64_t wend = start + ((end - start) & ~(int64_t)(kWide - 1));
  for (int64_t base = start + kWide * threadIdx.x; base < wend; base += (int64_t)kWide * kThreads * kWideUnroll) {
    vu4 cc[kWideUnroll];
#pragma unroll
    for (int u = 0; u < kWideUnroll; u++) {
      const int64_t i = base + (int64_t)u * kWide * kThreads;
      if (i < wend) cc[u] = ld_stream<vu4, FP8ADAM_NT_AMAX != 0>(dst + i);
    }
#pragma unroll
    for (int u = 0; u < kWideUnroll; u++) {
      const int64_t i = base + (int64_t)u * kWide * kThreads;
      if (i < wend) {
        vu4 w;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          uint32_t x;
          if (!shift_codes4<FMT>(cc[u][k], dexp, zero_ok, x))
            x = recompute4<FMT, STATS, IS_V, SR>(c, tid, d, i + 4 * k, s_old, inv_new, under, sat);
          w[k] = x;
        }
        st_global<vu4>(dst + i, w);
      }
    }
  }
  const int64_t gend = wend + ((end - wend) & ~(int64_t)3);
  if (threadIdx.x < kWide / 4 && wend + 4 * (int64_t)threadIdx.x < gend) {
    const int64_t i = wend + 4 * (int64_t)threadIdx.x;
    uint32_t w;
    if (!shift_codes4<FMT>(ld_global<uint32_t>(dst + i), dexp, zero_ok, w))
      w = recompute4<FMT, STATS, IS_V, SR>(c, tid, d, i, s_old, inv_new, under, sat);
    st_global<uint32_t>(dst + i, w);
  }
  if (gend + threadIdx.x < end) {
    const int64_t i = gend + threadIdx.x;
    const float g = load_g1(d, i) * c.gfac;
    const float x0 = decode1<FMT>(ld_global<uint8_t>((IS_V ? d.v : d.m) + i)) * s_old;
    float m1, v1;
    moment_update(c, g, x0, x0, m1, v1);
    const float x = IS_V ? v1 : m1;
    const float q = x * inv_new;
    const uint32_t code = quant1<FMT, SR, IS_V>(sr_word1<SR>(c, tid, i), q);
    if constexpr (STATS) {
      under += (x != 0.0f && (code & 0x7Fu) == 0u);
      sat += (fabsf(q) > Format<FMT>::kMax);
    }
    st_global<uint8_t>(dst + i, (uint8_t)code);
  }
}

// Work-groups of the fix-up: a fixed grid striding over the work list of the
// flagged chunks and moments, which k_spec_reduce builds, so no work-group is
// launched for the (most) chunks whose tensor was predicted right.  Measured on the 7B list
// (steps 4-23, 6.8% of the (element, moment) pairs moved, one box per sweep):
// 1024 work-groups 497 us per fix-up, 2048 459, 4096 395, 8192 369, 16384
// 359, 32768 356, 65536 358; one list item per chunk (32768 elements) against
// halves 379 us and quarters 392 us (always split, more items than work-groups);
// non-temporal stores of the moved codes 366 us against 360 us plain.
#ifndef FP8ADAM_FIX_GROUPS
#define FP8ADAM_FIX_GROUPS 16384
#endif
constexpr int64_t kFixGroups = FP8ADAM_FIX_GROUPS;
// Smallest piece of a chunk the fix-up hands to one work-group: one 16-code
// access per lane.  When the list holds fewer entries than the grid has
// work-groups, each chunk is split into 2^s pieces, the largest s whose pieces
// still fit the grid, so that a short list (a small model, or a step with few
// mispredicted tensors) spreads over the chip instead of leaving a few
// work-groups to walk whole chunks.
constexpr int kFixPieceLog2Min = 12;
static_assert((1 << kFixPieceLog2Min) == 16 * kThreads, "one 16-code access per lane");
static_assert(kMinChunkLog2 >= kFixPieceLog2Min, "a chunk holds at least one piece");
// Work-groups of the scale probe (a fixed grid striding over the list's slots).
constexpr int64_t kProbeGroups = 8192;

template <int MF, int VF, bool STATS, bool SR>
__global__ __launch_bounds__(kThreads) void k_fixup(const TensorDesc* __restrict__ descs,
                                                    const TensorDesc* __restrict__ dst_descs,
                                                    const int32_t* __restrict__ chunk_tid,
                                                    const uint32_t* __restrict__ amax,
                                                    const float* __restrict__ old_scale, StepConsts c,
                                                    unsigned long long* __restrict__ counters, int chunk_log2,
                                                    const uint32_t* __restrict__ fix_count,
                                                    const uint32_t* __restrict__ fix_list,
                                                    const GradCtl* __restrict__ gctl) {
  if (amp_apply(gctl, c)) return;
  const int64_t nlisted = ld_global<uint32_t>(fix_count);
  int split = 0;  // pieces per listed entry: 2^split (the same in every work-group)
  while (split < chunk_log2 - kFixPieceLog2Min && (nlisted << (split + 1)) <= (int64_t)gridDim.x) split++;
  const int piece_log2 = chunk_log2 - split;
  const int64_t nwork = nlisted << split;
  for (int64_t w = blockIdx.x; w < nwork; w += gridDim.x) {
    const uint32_t e = ld_global<uint32_t>(fix_list + (w >> split));
    const int64_t chunk = e >> 1;
    const int tid = chunk_tid[chunk];
    const TensorDesc d = descs[tid];
    const int64_t start = ((chunk - d.chunk0) << chunk_log2) + ((w & (((int64_t)1 << split) - 1)) << piece_log2);
    if (start >= d.numel) continue;  // a piece past the end of the tensor's last chunk
    const int64_t end = min(start + ((int64_t)1 << piece_log2), d.numel);
    uint32_t cnt[kStatsPerTensor] = {0, 0, 0, 0, 0};
    if ((e & 1u) == 0u) {
      float s, inv;
      choose_scale<MF, 0>(amax[2 * tid], s, inv);
      fixup_moment<MF, STATS, false, SR>(c, tid, d, dst_descs[tid].m, start, end, old_scale[4 * tid],
                                         __float_as_uint(old_scale[4 * tid + 2]), s, inv, cnt[kUnderM],
                                         cnt[kSatM]);
    } else {
      float s, inv;
      choose_scale<VF, 0>(amax[2 * tid + 1], s, inv);
      fixup_moment<VF, STATS, true, SR>(c, tid, d, dst_descs[tid].v, start, end, old_scale[4 * tid + 1],
                                        __float_as_uint(old_scale[4 * tid + 3]), s, inv, cnt[kUnderV],
                                        cnt[kSatV]);
    }
    flush_counters<STATS>(counters, tid, cnt);
  }
}

// Zero the stats counters (and, in block mode, the amax used for stats).
static __global__ __launch_bounds__(kThreads) void k_reset(unsigned long long* __restrict__ counters, int64_t ncnt,
                                                    uint32_t* __restrict__ amax, int64_t namax) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ncnt; i += (int64_t)gridDim.x * blockDim.x)
    counters[i] = 0ull;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < namax; i += (int64_t)gridDim.x * blockDim.x)
    amax[i] = 0u;
}

// ------------------------------------------------------------ block-128 mode
//
// 32 lanes own one 128-element block, each lane 4
// consecutive elements per access, so every access of the wave covers two
// whole blocks (a full 128-byte line of codes per block and moment; a layout
// with 8 lanes x 16 elements per block wrote 32-byte pieces of each line and
// ran ~4% slower).  The block amax is a 5-step max over the 32 lanes (DPP
// within 16 lanes, then a swizzle across the two 16-lane rows).

__device__ __forceinline__ uint32_t group32_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F));                          // lane ^ 16
  return x;
}

template <int MF, int VF, bool BF16P, bool STATS, int SMODE, bool L2, bool SR>
__global__ __launch_bounds__(kThreads) void k_block(const TensorDesc* __restrict__ descs,
                                                      const int32_t* __restrict__ chunk_tid, StepConsts c,
                                                      unsigned long long* __restrict__ counters,
                                                      uint32_t* __restrict__ amax, int chunk_log2, int64_t nwork,
                                                      const GradCtl* __restrict__ gctl) {
  const int64_t w = work_index<kXcdStreams>(nwork);
  if (w < 0 || amp_apply(gctl, c)) return;
  const int split_log2 = chunk_log2 - kPartLog2;
  const int64_t chunk = w >> split_log2;
  const int tid = chunk_tid[chunk];
  const TensorDesc d = descs[tid];
  const int64_t start = ((chunk - d.chunk0) << chunk_log2) + ((w & ((1 << split_log2) - 1)) << kPartLog2);
  const int64_t end = min(start + kPart, d.numel);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  uint32_t cnt[kStatsPerTensor] = {0, 0, 0, 0, 0};
  uint32_t tam = 0, tav = 0;
  float tsm = 0.0f, tsv = 0.0f;
  const PartBufs B = part_bufs<BF16P>(d, d.m, d.v, start, end - start);

  for (int64_t tile = start; tile < end; tile += (int64_t)kBlock * 8 * kBlkJ) {
    int64_t b0[kBlkJ];
    bool ex[kBlkJ], full[kBlkJ];
    float sm[kBlkJ], sv[kBlkJ];
    Group G[kBlkJ];
#pragma unroll
    for (int j = 0; j < kBlkJ; j++) {
      b0[j] = tile + (int64_t)(wave * 2 * kBlkJ + 2 * j + half) * kBlock;
      ex[j] = b0[j] < end;
      full[j] = b0[j] + kBlock <= end;
      sm[j] = 1.0f;
      sv[j] = 1.0f;
      if (ex[j]) {
        sm[j] = ld_global<float>(d.sm + b0[j] / kBlock);
        sv[j] = ld_global<float>(d.sv + b0[j] / kBlock);
      }
      if (full[j]) load_group_buf<BF16P>(B, (uint32_t)(b0[j] + 4 * hl - start), G[j], true);
    }
#pragma unroll
    for (int j = 0; j < kBlkJ; j++) {
      float m1[4], v1[4], p[4];
      const int64_t i0 = b0[j] + 4 * hl;
      if (full[j]) {
        unpack_p<BF16P>(G[j], p);
        fresh_moments<MF, VF, L2>(c, G[j], p, sm[j], sv[j], m1, v1);
      } else {
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int64_t i = i0 + r;
          float a = 0.0f, b = 0.0f, q = 0.0f;
          if (ex[j] && i < end) {
            q = load_p1<BF16P>(d, i);
            const float g = grad_in<L2>(c, load_g1(d, i), q);
            moment_update(c, g, decode1<MF>(ld_global<uint8_t>(d.m + i)) * sm[j],
                          decode1<VF>(ld_global<uint8_t>(d.v + i)) * sv[j], a, b);
          }
          m1[r] = a;
          v1[r] = b;
          p[r] = q;
        }
      }
      uint32_t am = 0, av = 0;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        am = max(am, abs_bits(m1[r]));
        av = max(av, abs_bits(v1[r]));
      }
      am = group32_max(am);
      av = group32_max(av);
      float nsm, ism, nsv, isv;
      choose_scale<MF, SMODE>(am, nsm, ism);
      choose_scale<VF, SMODE>(av, nsv, isv);
      if constexpr (STATS) {
        if (ex[j]) {
          tam = max(tam, am);
          tav = max(tav, av);
          tsm = fmaxf(tsm, nsm);
          tsv = fmaxf(tsv, nsv);
        }
      }
      float qm[4], qv[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = param_update(c, p[r], m1[r], v1[r]);
        qm[r] = m1[r] * ism;
        qv[r] = v1[r] * isv;
      }
      if (full[j]) {
        uint32_t rw[4];
        sr_words<SR>(c, tid, i0, rw);
        const uint32_t wm = quant4<MF, SR, false>(qm, rw);
        const uint32_t wv = quant4<VF, SR, true>(qv, rw);
        if constexpr (STATS) {
#pragma unroll
          for (int r = 0; r < 4; r++)
            count_element<MF, VF, STATS>(cnt, m1[r], v1[r], qm[r], qv[r], wm >> (8 * r), wv >> (8 * r));
        }
        store_group_buf<BF16P>(B.p, B.m, B.v, (uint32_t)(i0 - start), p, wm, wv);
      } else if (ex[j]) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int64_t i = i0 + r;
          if (i < end) {
            const uint32_t w = sr_word1<SR>(c, tid, i);
            const uint32_t cm = quant1<MF, SR, false>(w, qm[r]), cv = quant1<VF, SR, true>(w, qv[r]);
            count_element<MF, VF, STATS>(cnt, m1[r], v1[r], qm[r], qv[r], cm, cv);
            store_p1<BF16P>(d, i, p[r]);
            st_global<uint8_t>(d.m + i, (uint8_t)cm);
            st_global<uint8_t>(d.v + i, (uint8_t)cv);
          }
        }
      }
      if (ex[j] && hl == 0) {
        st_global<float>(d.sm + b0[j] / kBlock, nsm);
        st_global<float>(d.sv + b0[j] / kBlock, nsv);
      }
    }
  }
  if constexpr (STATS) {
    flush_counters<STATS>(counters, tid, cnt);
    uint32_t sa = __float_as_uint(tsm), sb = __float_as_uint(tsv);
    uint32_t a = wave_max(tam), b = wave_max(tav);
    sa = wave_max(sa);
    sb = wave_max(sb);
    if (lane == 0) {
      if (a) atomicMax(&amax[4 * tid], a);
      if (b) atomicMax(&amax[4 * tid + 1], b);
      if (sa) atomicMax(&amax[4 * tid + 2], sa);
      if (sb) atomicMax(&amax[4 * tid + 3], sb);
    }
  }
}

// ================================================================== host side

// Error reporting (defined with the C ABI): set the thread's last error and return code.
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);





#define HIP_TRY(expr)                                    \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return hip_fail(e_, #expr);    \
  } while (0)

constexpr int kMaxTimed = 4096;

}  // namespace fp8adam_engine

// The context behind the opaque handle of the C ABI.
struct fp8adam_ctx {
  int device = 0;
  fp8adam_config cfg{};
  int32_t n = 0;
  int64_t nchunks = 0;
  int chunk_log2 = fp8adam_engine::kMaxChunkLog2;  // elements per chunk = 2^chunk_log2
  int speculate_from = 4;          // first step t that runs the speculative schedule
  int hist_len = 0;                // delayed scaling: amax history length H (0: just in time)
  int delayed_from = 2;            // delayed scaling: first step t quantized with the delayed scale
  float margin_scale = 1.0f;       // delayed scaling: 2^margin
  int cur = 0;                     // code buffer holding the moments: 0 = m/v, 1 = m_alt/v_alt
  int64_t nparts = 0;              // block-pass work-groups
  int64_t nuparts = 0;             // update-pass work-groups at the smallest part size
  fp8adam_engine::TensorDesc* d_desc = nullptr;    // [2][n]: descriptors with m/v, then with m_alt/v_alt
  int32_t* d_chunk_tid = nullptr;
  uint32_t* d_amax = nullptr;       // tensor mode: [n][2] amax of the last step; block mode: [n][4] stats
  uint2* d_partial = nullptr;       // tensor mode: [nchunks] per-chunk amax of m', v'
  uint2* d_part_amax = nullptr;     // speculative / delayed: [<= nuparts] per-part amax of m', v'
  float* d_old_scale = nullptr;     // tensor mode: [n][4]: scales before the step (+ prepared ones)
  int32_t* d_flags = nullptr;       // [n]: the last step re-quantized the tensor (speculative)
  uint32_t* d_fix_count = nullptr;  // speculative: entries in the fix-up's work list this step
  uint32_t* d_fix_list = nullptr;   // speculative: [<= 2 nchunks] chunk * 2 + moment of the flagged tensors
  int64_t ncand_slots = 0;          // speculative: room in the probe's work list (the tensors' caps summed)
  uint32_t* d_cand_count = nullptr; // speculative: entries in the probe's work list
  uint2* d_cand_work = nullptr;     // speculative: [ncand_slots] (tensor, part index within the tensor)
  int32_t* d_cand_n = nullptr;      // speculative: [n] parts listed (0: none, the growth model predicts)
  int64_t* d_cand_len = nullptr;    // speculative: [n] elements in the listed parts
  uint32_t* d_lb = nullptr;         // speculative: [n][2] the probe's amax over the candidates
  int64_t* d_probed = nullptr;      // speculative: [n] elements the probe read in the last step
  bool last_spec = false;           // the last step ran the speculative schedule
  unsigned long long* d_counters = nullptr;  // [n][5]
  double* d_gpart = nullptr;        // loss scaling: [norm groups][2] sum of squares and Inf/NaN count of g
  fp8adam_engine::GradCtl* d_gctl = nullptr;       // loss scaling: the decision of the step in flight
  const fp8adam_engine::GradCtl* gctl = nullptr;   // d_gctl during fp8adam_step_amp, else null
  bool timing = false;
  uint32_t timing_kinds = 0xFFFFFFFFu;  // the kinds timed while timing is on (bit k: kind k)
  std::vector<hipEvent_t> ev;  // pairs
  std::vector<int> ev_kind;
  int ev_used = 0;
  int ev_pending = -1;  // the slot whose events the next launch takes (-1: none)
};

namespace fp8adam_engine {

// A timed launch hands its slot's two events to the kernel launch itself
// (launch_k), which stamps them with the dispatch's own start and end: no
// event packets of their own in the stream, so timing adds less to a step and
// the recorded duration is the kernel's.  Launches into a stream under graph
// capture are not timed (a captured kernel runs when the graph is launched).
inline int timed_begin(fp8adam_ctx* c, int kind, hipStream_t s, int* slot) {
  *slot = -1;
  if (!c->timing || !((c->timing_kinds >> kind) & 1u) || c->ev_used >= kMaxTimed) return 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(s, &cs));
  if (cs != hipStreamCaptureStatusNone) return 0;
  *slot = c->ev_used++;
  c->ev_kind[*slot] = kind;
  c->ev_pending = *slot;
  return 0;
}

inline int timed_end(fp8adam_ctx* c, int slot, hipStream_t) {
  if (slot >= 0 && c->ev_pending == slot) {  // nothing was launched: give the slot back
    c->ev_pending = -1;
    c->ev_used--;
  }
  return 0;
}

// Launch a kernel with the argument conversions of hipLaunchKernelGGL; inside a
// timed launch through hipExtLaunchKernel with the pending slot's events.
template <typename... Formals, typename... Actuals>
inline void launch_k(fp8adam_ctx* c, void (*kernel)(Formals...), dim3 grid, dim3 block, hipStream_t s,
                     Actuals... actuals) {
  static_assert(sizeof...(Formals) == sizeof...(Actuals), "kernel argument count");
  std::tuple<Formals...> formals{actuals...};
  void* argv[sizeof...(Formals) > 0 ? sizeof...(Formals) : 1];
  std::apply([&argv](auto&... f) {
    int i = 0;
    ((argv[i++] = static_cast<void*>(&f)), ...);
  }, formals);
  const void* fn = reinterpret_cast<const void*>(kernel);
  if (c->ev_pending >= 0) {
    const int slot = c->ev_pending;
    c->ev_pending = -1;
    (void)hipExtLaunchKernel(fn, grid, block, argv, 0, s, c->ev[2 * slot], c->ev[2 * slot + 1], 0);
  } else {
    (void)hipLaunchKernel(fn, grid, block, argv, 0, s);
  }
}

// ---- kernel dispatch over the template parameters ----

inline const TensorDesc* descs_of(const fp8adam_ctx* c, int which) { return c->d_desc + (size_t)which * c->n; }

template <int MF, int VF, bool BF16P, bool L2>
void launch_amax(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_amax<MF, VF, BF16P && L2, L2>, dim3(grid_for<false>(c->nchunks)), dim3(kThreads), s, descs_of(c, c->cur),
           c->d_chunk_tid, c->d_partial, k, c->chunk_log2, c->nchunks, c->gctl);
}

template <int MF, int VF, int SMODE, bool STATS>
void launch_reduce(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_reduce<MF, VF, SMODE, STATS>, dim3((unsigned)c->n), dim3(kReduceThreads), s,
           descs_of(c, c->cur), c->d_partial, c->d_amax, c->d_old_scale, c->d_counters, c->chunk_log2,
           c->d_flags, k.hist_len, k.hist_slot, c->gctl);
}

template <int MF, int VF, int SMODE>
void launch_delayed_prepare(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_delayed_prepare<MF, VF, SMODE>, dim3((unsigned)c->n), dim3(64), s, descs_of(c, 0), k,
           c->d_old_scale);
}

template <int MF, int VF, int SMODE>
void launch_delayed_reduce(fp8adam_ctx* c, const StepConsts& k, int part_log2, hipStream_t s) {
  launch_k(c, k_delayed_reduce<MF, VF, SMODE>, dim3((unsigned)c->n), dim3(kReduceThreads), s,
           descs_of(c, 0), c->d_part_amax, c->d_amax, k, c->chunk_log2, part_log2, c->gctl,
           c->d_old_scale);
}

template <int MF, int VF, bool BF16P, bool STATS, int SMODE, int MODE, bool L2, bool SR>
void launch_update(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  const int64_t nwork = c->nchunks << (c->chunk_log2 - upd_part_log2<BF16P>());
  launch_k(c, k_update<MF, VF, BF16P, STATS, SMODE, MODE, L2, SR>, dim3(grid_for<kXcdStreams>(nwork)), dim3(kThreads), s,
           descs_of(c, c->cur), descs_of(c, MODE == kModeSpec ? 1 - c->cur : c->cur), c->d_chunk_tid, c->d_amax,
           c->d_old_scale, k, c->d_counters, c->chunk_log2, c->d_part_amax, nwork, c->gctl);
}

template <int MF, int VF, bool BF16P>
void launch_spec_probe(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_spec_probe<MF, VF, upd_part_log2<BF16P>()>,
           dim3((unsigned)std::min<int64_t>(c->ncand_slots, kProbeGroups)), dim3(kThreads), s,
           descs_of(c, c->cur), k, c->d_cand_count, c->d_cand_work, c->d_lb, c->gctl);
}

template <int MF, int VF>
void launch_spec_prepare(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_spec_prepare<MF, VF>, dim3((unsigned)((c->n + 63) / 64)), dim3(64), s, descs_of(c, c->cur),
           c->d_amax, k, c->gctl, c->d_old_scale, c->n, c->d_fix_count,
           c->ncand_slots > 0 ? c->d_cand_n : nullptr, c->d_cand_len, c->d_lb, c->d_probed,
           c->d_cand_count);
}

template <int MF, int VF>
void launch_exact_prepare(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_exact_prepare<MF, VF>, dim3((unsigned)c->n), dim3(kReduceThreads), s, descs_of(c, c->cur),
           c->d_partial, c->chunk_log2, k, c->gctl, c->d_old_scale, c->d_fix_count, c->d_probed,
           c->d_cand_count);
}

template <bool BF16P>
void launch_part_fold(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  const int split = c->chunk_log2 - upd_part_log2<BF16P>();
  const int64_t lanes = split > 1 ? (int64_t)1 << (split - 1) : 1;
  launch_k(c, k_part_fold<upd_part_log2<BF16P>()>, dim3((unsigned)((c->nchunks * lanes + kThreads - 1) / kThreads)),
           dim3(kThreads), s, c->d_part_amax, c->d_partial, c->chunk_log2, c->nchunks, k, c->gctl);
}

template <int MF, int VF, bool STATS>
void launch_spec_reduce(fp8adam_ctx* c, const StepConsts& k, int part_log2, hipStream_t s) {
  launch_k(c, k_spec_reduce<MF, VF, STATS>, dim3((unsigned)c->n), dim3(kReduceThreads), s,
           descs_of(c, c->cur), c->d_part_amax, c->ncand_slots > 0 ? c->d_partial : nullptr, c->d_amax, c->d_old_scale, c->d_flags, c->d_counters,
           c->chunk_log2, part_log2, k, c->gctl, c->d_fix_count, c->d_fix_list, c->d_cand_n,
           c->d_cand_len, c->d_cand_count, c->ncand_slots > 0 ? c->d_cand_work : nullptr);
}

template <int MF, int VF, bool STATS, bool SR>
void launch_fixup(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  // room for every chunk split down to the smallest piece, up to the fixed grid
  const int64_t groups = std::min<int64_t>((2 * c->nchunks) << (c->chunk_log2 - kFixPieceLog2Min), kFixGroups);
  launch_k(c, k_fixup<MF, VF, STATS, SR>, dim3((unsigned)groups),
           dim3(kThreads), s, descs_of(c, c->cur), descs_of(c, 1 - c->cur), c->d_chunk_tid, c->d_amax,
           c->d_old_scale, k, c->d_counters, c->chunk_log2, c->d_fix_count, c->d_fix_list,
           c->gctl);
}

template <int MF, int VF, bool BF16P, bool STATS, int SMODE, bool L2, bool SR>
void launch_block(fp8adam_ctx* c, const StepConsts& k, hipStream_t s) {
  launch_k(c, k_block<MF, VF, BF16P, STATS, SMODE, L2, SR>, dim3(grid_for<kXcdStreams>(c->nparts)), dim3(kThreads), s,
           descs_of(c, 0), c->d_chunk_tid, k, c->d_counters, c->d_amax, c->chunk_log2, c->nparts, c->gctl);
}

// Timing kinds: 0 amax pass, 1 update pass, 2 scale reduce, 3 block pass,
// 4 stats reset, 5 speculative pass, 6 speculative reduce, 7 fix-up,
// 8 delayed pass, 9 delayed commit, 10 gradient-norm pass, 11 loss-scale decision,
// 12 scale preparation (speculative / delayed), 13 speculative scale probe,
// 14 speculative per-chunk fold of the part partials.
#define TIMED(kind, call)                              \
  do {                                                 \
    int slot_;                                         \
    if (int r_ = timed_begin(c, (kind), s, &slot_)) return r_; \
    call;                                              \
    if (int r_ = timed_end(c, slot_, s)) return r_;    \
  } while (0)

inline void launch_reset(fp8adam_ctx* c, int64_t namax, hipStream_t s) {
  launch_k(c, k_reset, dim3(std::max<int64_t>(1, std::min<int64_t>(1024, (5 * (int64_t)c->n + 255) / 256))),
           dim3(kThreads), s, c->d_counters, (int64_t)kStatsPerTensor * c->n, c->d_amax, namax);
}

template <int MF, int VF, bool BF16P, bool STATS, int SMODE, bool L2, bool SR>
int run_step_t(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  bool done = false;
  c->last_spec = false;
  if (c->cfg.granularity == FP8ADAM_SCALE_BLOCK128) {
    if (STATS) TIMED(4, launch_reset(c, 4 * (int64_t)c->n, s));
    if (c->nchunks > 0) TIMED(3, (launch_block<MF, VF, BF16P, STATS, SMODE, L2, SR>(c, k, s)));
    done = true;
  }
  // (fp8adam_init refuses the speculative schedule with coupled L2 or AMAX scales:
  // the fix-up recomputes moments after p has been overwritten, and g_eff needs the old p)
  if constexpr (!L2 && SMODE == 0) {
    // the step before the first speculative one: the amax pass, then the speculative
    // pass with the true scales (its check lists the probe's first candidates)
    if (!done && c->cfg.schedule == FP8ADAM_SCHEDULE_SPECULATIVE && t >= c->speculate_from - 1) {
      if (STATS) TIMED(4, launch_reset(c, 0, s));
      if (t < c->speculate_from) {
        if (c->nchunks > 0) TIMED(0, (launch_amax<MF, VF, BF16P, false>(c, k, s)));
        TIMED(2, (launch_exact_prepare<MF, VF>(c, k, s)));
      } else {
        if (c->ncand_slots > 0) TIMED(13, (launch_spec_probe<MF, VF, BF16P>(c, k, s)));
        TIMED(12, (launch_spec_prepare<MF, VF>(c, k, s)));
      }
      if (c->nchunks > 0) TIMED(5, (launch_update<MF, VF, BF16P, STATS, SMODE, kModeSpec, false, SR>(c, k, s)));
      if (c->nchunks > 0 && c->ncand_slots > 0) TIMED(14, (launch_part_fold<BF16P>(c, k, s)));
      TIMED(6, (launch_spec_reduce<MF, VF, STATS>(c, k, upd_part_log2<BF16P>(), s)));
      if (c->nchunks > 0) TIMED(7, (launch_fixup<MF, VF, STATS, SR>(c, k, s)));
      c->cur = 1 - c->cur;
      c->last_spec = true;
      done = true;
    }
  }
  if (!done && c->hist_len > 0 && t >= c->delayed_from) {
    if (STATS) TIMED(4, launch_reset(c, 0, s));
    TIMED(12, (launch_delayed_prepare<MF, VF, SMODE>(c, k, s)));
    if (c->nchunks > 0) TIMED(8, (launch_update<MF, VF, BF16P, STATS, SMODE, kModeDelayed, L2, SR>(c, k, s)));
    TIMED(9, (launch_delayed_reduce<MF, VF, SMODE>(c, k, upd_part_log2<BF16P>(), s)));
  } else if (!done) {
    if (c->nchunks > 0) TIMED(0, (launch_amax<MF, VF, BF16P, L2>(c, k, s)));
    // the reduce also runs for an all-empty list: it sets amax 0 and clears the counters
    TIMED(2, (launch_reduce<MF, VF, SMODE, STATS>(c, k, s)));
    if (c->nchunks > 0) TIMED(1, (launch_update<MF, VF, BF16P, STATS, SMODE, kModeJit, L2, SR>(c, k, s)));
  }
  HIP_TRY(hipGetLastError());
  return 0;
}

template <int MF, int VF, bool BF16P, bool STATS, int SMODE, bool L2>
int run_step_r(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  return c->cfg.rounding == FP8ADAM_ROUND_STOCHASTIC ? run_step_t<MF, VF, BF16P, STATS, SMODE, L2, true>(c, k, t, s)
                                                     : run_step_t<MF, VF, BF16P, STATS, SMODE, L2, false>(c, k, t, s);
}

// Coupled L2 with weight_decay 0 is plain Adam: it runs the kernels without
// the extra term (which would also turn a -0 gradient into +0).
template <int MF, int VF, bool BF16P, bool STATS, int SMODE>
int run_step_l(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  return k.l2 != 0.0f ? run_step_r<MF, VF, BF16P, STATS, SMODE, true>(c, k, t, s)
                      : run_step_r<MF, VF, BF16P, STATS, SMODE, false>(c, k, t, s);
}

template <int MF, int VF, bool BF16P, bool STATS>
int run_step_s(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  return c->cfg.scale_mode == FP8ADAM_SCALE_POW2 ? run_step_l<MF, VF, BF16P, STATS, 0>(c, k, t, s)
                                                 : run_step_l<MF, VF, BF16P, STATS, 1>(c, k, t, s);
}

template <int MF, int VF, bool BF16P>
int run_step_b(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  return c->cfg.collect_stats ? run_step_s<MF, VF, BF16P, true>(c, k, t, s)
                              : run_step_s<MF, VF, BF16P, false>(c, k, t, s);
}

template <int MF, int VF>
int run_step_f(fp8adam_ctx* c, const StepConsts& k, int64_t t, hipStream_t s) {
  return c->cfg.master == FP8ADAM_MASTER_BF16 ? run_step_b<MF, VF, true>(c, k, t, s)
                                              : run_step_b<MF, VF, false>(c, k, t, s);
}

// One instantiation per (m, v) format pair, each in a translation unit of its own.
extern template int run_step_f<0, 1>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);
extern template int run_step_f<1, 1>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);
extern template int run_step_f<1, 0>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);
extern template int run_step_f<0, 0>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);

}  // namespace fp8adam_engine
