// NVFP4 block-scaled quantization (rtn6 and Four Over Six) for gfx950 -- kernels and C ABI.
//
// The operation is defined in include/nvfp4_amax.h (with the page citations).  This file
// holds the HIP kernels and the host entry points that validate arguments and enqueue them.
//
// Kernels:
//   clear_kernel     amax accumulator <- 0 (a tiny fill kernel rather than a memset, so the
//                    sequence stays capturable in a HIP graph)
//   amax_kernel      streaming 128-bit loads; the max of bf16 magnitudes is an unsigned
//                    16-bit integer max (exact, order-free, NaN/Inf sort above finite
//                    values), reduced per wavefront with DPP row moves and per workgroup in
//                    LDS, then one atomicMax per workgroup on the tensor's float bits
//   quantize_kernel  one lane owns whole 16-element blocks: both candidate scales, the FP4
//                    rounding, the error reduction and the selection stay in VGPRs; codes
//                    and scale bytes (or bf16 fake-quant values) leave in streaming stores
//   alpha_kernel     alpha[e] <- amax[e] / (6*M) once every block is done
//   (the diagnostics variant of quantize_kernel also reduces per-tensor error statistics
//   in binary64: each workgroup leaves its partial sums in a slot of the caller's
//   workspace, and the last to arrive sums the slots in a fixed order)
//   fused_kernel     single-read dynamic quantization for tensors that fit on chip: loads
//                    and keeps each lane's blocks (VGPRs + LDS), reduces amax, waits for
//                    every workgroup of the tensor (per-workgroup slots read by one
//                    collector, or a two-level counter), then runs the
//                    block pass on the blocks it holds; workgroups of 256, 512 or 1024
//                    threads by tier; a batch larger than the chip runs as teams of
//                    workgroups that take its tensors in turn
//   dequant_kernel   packed codes + scale bytes + alpha -> bf16, one block per lane
//
// All floating-point steps of the encoding are IEEE binary32 with round-to-nearest-even, no
// contraction (-ffp-contract=off) and no denormal flushing; fp32 division and reciprocal are
// the correctly rounded HIP defaults.  (Only the diagnostics' error sums are binary64.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "nvfp4_amax.h"

#define NVFP4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kThreads = 256;          // 4 wavefronts of 64
constexpr float kC6x448 = 2688.0f;     // 6 * 448: standard NVFP4
constexpr float kC6x256 = 1536.0f;     // 6 * 256: Four Over Six

// ----------------------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> E4M3FN byte for s >= 0: round to nearest even on the E4M3 grid, saturating
// at 448.  Below 2^-6 the grid is the subnormal k * 2^-9, so scaling by 2^9 (exact) and
// rounding to an integer gives k.  Above it, the 23-bit mantissa is rounded to 3 bits in
// place; a carry moves into the exponent, and the exponent is rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_from_f32(float s) {
  s = fminf(s, 448.0f);
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  uint32_t u = __float_as_uint(s);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);
}

// E4M3FN byte (0x00..0x7E) -> exact binary32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Magnitude a >= 0 -> E2M1 magnitude code 0..7 by counting the rounding thresholds it
// passes.  The thresholds are the midpoints of {0, .5, 1, 1.5, 2, 3, 4, 6}; at a midpoint
// the even code wins, which is ">" where the lower neighbour is even, ">=" where it is odd.
__device__ __forceinline__ uint32_t e2m1_code_of(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// E2M1 magnitude code -> value: 0 and 0.5 (subnormal), else 2^(e-1) * (1 + m/2), which
// as binary32 bits is ((code + 252) << 22).
__device__ __forceinline__ float e2m1_value_of(uint32_t m) {
  return m < 2 ? 0.5f * (float)m : __uint_as_float((m + 252u) << 22);
}

// ----------------------------------------------------------------------------- kernels
__global__ void clear_kernel(uint32_t* __restrict__ acc, uint32_t* __restrict__ acc2, int64_t E,
                             uint32_t* __restrict__ acc3, int64_t n3, uint32_t* __restrict__ acc4,
                             int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) {
    acc[i] = 0u;
    if (acc2) acc2[i] = 0u;
  }
  if (acc3 && i < n3) acc3[i] = 0u;
  if (acc4 && i < n4) acc4[i] = 0u;
}

// Max of two packed unsigned 16-bit lanes (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  const us2 r = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t mag_max8(uint32_t m, uint4 v) {
  m = pk_max_u16(m, v.x & 0x7FFF7FFFu);
  m = pk_max_u16(m, v.y & 0x7FFF7FFFu);
  m = pk_max_u16(m, v.z & 0x7FFF7FFFu);
  return pk_max_u16(m, v.w & 0x7FFF7FFFu);
}

// Wavefront max: DPP row shifts reduce each row of 16 lanes, then the four row results
// are read with readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  // lane 15 of each row now holds the row max
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(r0, r1), max(r2, r3));
}

// Grid: x = workgroups per tensor, y = tensor.  Few, large workgroups (one atomic each:
// same-address atomics serialize, so their count is kept near the CU count).  Each lane
// reads C 16-byte chunks per step, the workgroups striding over the tensor: C = 8 (64 bf16
// values) when that still gives every tensor its share of the workgroups, else C = 1 so that
// small tensors spread over more CUs.  The C chunks are consecutive (128 bytes per lane), or
// with COAL 1024 chunks apart, so that each load instruction of a wave reads 1 KB contiguous.
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxWGs = 256;
template <int C, bool COAL>
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint4* __restrict__ in,
                                                            int64_t chunks,
                                                            uint32_t* __restrict__ acc) {
  const uint4* p = in + (int64_t)blockIdx.y * chunks;
  uint32_t m = 0;
  if (COAL) {     // a workgroup's step is C * 1024 consecutive chunks, 1 KB per load instruction
    const int64_t span = (int64_t)kAmaxThreads * C;
    const int64_t stride = (int64_t)gridDim.x * span;
    int64_t b = (int64_t)blockIdx.x * span;
    for (; b + span <= chunks; b += stride) {
      uint4 v[C];
#pragma unroll
      for (int k = 0; k < C; ++k) v[k] = p[b + k * kAmaxThreads + threadIdx.x];
#pragma unroll
      for (int k = 0; k < C; ++k) m = mag_max8(m, v[k]);
    }
    if (b < chunks)                                // the one span that runs past the end
      for (int k = 0; k < C; ++k) {
        const int64_t j = b + k * kAmaxThreads + threadIdx.x;
        if (j < chunks) m = mag_max8(m, p[j]);
      }
  } else {
    const int64_t stride = (int64_t)gridDim.x * kAmaxThreads * C;
    int64_t i = ((int64_t)blockIdx.x * kAmaxThreads + threadIdx.x) * C;
    for (; i + C <= chunks; i += stride) {
      uint4 v[C];
#pragma unroll
      for (int k = 0; k < C; ++k) v[k] = p[i + k];
#pragma unroll
      for (int k = 0; k < C; ++k) m = mag_max8(m, v[k]);
    }
    if (C > 1)
      for (; i < chunks; ++i) m = mag_max8(m, p[i]);   // the one lane whose chunks run past the end
  }
  // the larger of the two 16-bit magnitudes, as the bits of a binary32 value
  m = max(m & 0xFFFFu, m >> 16) << 16;
  m = wave_max_u32(m);
  __shared__ uint32_t part[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (int w = 1; w < kAmaxThreads / 64; ++w) r = max(r, part[w]);
    atomicMax(acc + blockIdx.y, r);
  }
}

// Blocks scaled to 4 per tensor, counted from the per-block choice bytes (4 or 6; 0 for a
// poisoned tensor): count4[t] += the bytes equal to 4 in qstar[t * nblk, (t + 1) * nblk).
// Grid: x = workgroups per tensor, y = tensor.  The 16-byte-aligned middle of the range is read
// in 16-byte chunks, the at most 15 bytes before and after it one by one; one atomic per
// workgroup.
__global__ __launch_bounds__(kThreads) void count4_kernel(const uint8_t* __restrict__ qstar,
                                                          int64_t nblk,
                                                          uint32_t* __restrict__ count4) {
  const int64_t t = blockIdx.y;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(qstar) + (uintptr_t)(t * nblk);
  const uintptr_t hi = lo + (uintptr_t)nblk;
  const uintptr_t a = std::min((lo + 15) & ~(uintptr_t)15, hi);
  const uintptr_t b = std::max(a, hi & ~(uintptr_t)15);
  const uint4* q = reinterpret_cast<const uint4*>(a);
  const int64_t chunks = (int64_t)((b - a) >> 4);
  uint32_t c = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 v = q[i];   // a byte is 4 when its bit 2 is set and its bit 1 clear
    c += __popc(v.x & ~(v.x << 1) & 0x04040404u) + __popc(v.y & ~(v.y << 1) & 0x04040404u) +
         __popc(v.z & ~(v.z << 1) & 0x04040404u) + __popc(v.w & ~(v.w << 1) & 0x04040404u);
  }
  if (blockIdx.x == 0 && threadIdx.x < 32) {
    const uintptr_t j = threadIdx.x < 16 ? lo + threadIdx.x : b + (threadIdx.x - 16);
    if (j < (threadIdx.x < 16 ? a : hi) && *reinterpret_cast<const uint8_t*>(j) == 4) ++c;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  __shared__ uint32_t wsum[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot += wsum[w];
    if (tot) atomicAdd(count4 + t, tot);
  }
}

__global__ void alpha_kernel(const uint32_t* amax_bits, float* alpha,
                             int64_t E, float C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E) return;
  const uint32_t a = amax_bits[i] & 0x7FFFFFFFu;
  alpha[i] = a >= 0x7F800000u ? __uint_as_float(0x7FC00000u) : __uint_as_float(a) / C;
}

// ----------------------------------------------------------------------------- block pass
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#ifndef NVFP4_WAVES_PER_EU
#define NVFP4_WAVES_PER_EU 4         // occupancy floor: caps the block pass at 128 VGPRs
#endif
// Grid of the block pass (grid-stride loop, the next block's loads issued before the current
// block's arithmetic).  Measured on 67 MB to 1.3 GB inputs, same box, A/B:
//   - rtn6 and fake-quant are light per block and run fastest with one block per lane and as
//     many waves as fit: 5-17 % faster than a fixed 1024 workgroups.
//   - Four Over Six into packed output (two trials per block) needs its own loads in flight
//     across its arithmetic.  Below 2^23 blocks (268 MB of input) a fixed grid (1024
//     workgroups, 14 blocks per lane for the 4096x14336 weight) beat 4 blocks per lane by 3-5 %;
//     from 2^23 blocks on, 4 blocks per lane beat 1024 or 768 workgroups by 4-12 % (MoE 10 %),
//     and 3 blocks per lane beat 4 in four same-box A/B runs on three boxes: the 64-expert MoE
//     batch 293.7-298.4 against 299.6-304.0 us, the 16384x14336 tensor 107.5-109.1 against
//     109.5-110.3 us.  (2 per lane: faster than 3 on the 16384x14336 tensor in one run and
//     slower on the MoE batch in another; 6 and 8: 4-10 % slower.)
//   - The diagnostics variant ends with one or two same-address atomics per workgroup (the
//     count of blocks scaled to 4, the statistics counter): 1024 workgroups in all with
//     statistics (one workspace slot each); without, the block pass's 768 (same-box A/B: the
//     8192x4096 activation 37.64 against 39.67 us, the 4096x14336 weight 52.76 against 53.37).
//   With paced waves (see the block-pass loop) the choices were measured again: 768, 1536 or
//   2048 workgroups, 8 or 16 blocks per lane, 2048 or 4096 workgroups for long launches, and
//   1024-4096 workgroups for rtn6 and fake-quant were all slower or equal.  With the first loads issued
//   at the kernel's start, 768, 1536 and 2048 workgroups measured 1-7 % slower than 1024 on
//   the 4096x14336 weight.  With the outputs stored one step late, 768 workgroups (3 per CU)
//   overtook 1024 (4 per CU) below 2^23 blocks in three same-box A/B runs: the 4096x14336
//   weight 28.51 against 29.00 us (MSE) and 28.42 against 29.12 (MAE), 28.41 against 29.04 on
//   another box, the 8192x4096 activation packed 17.31 against 17.40; 512 and 896 workgroups
//   were slower than both (30.10 and 30.16 us on the weight).
constexpr int64_t kLongLaunchBlocks = INT64_C(1) << 23;
constexpr int64_t kShortLaunchWGs = 768;
constexpr int64_t kLaneBlocksLong = 3;
constexpr int64_t kDiagLaunchWGs = 1024;
constexpr uint32_t kPacedSteps = 8;      // grid-stride steps per lane from which waves pace themselves
constexpr int kDiagCtrWords = 32;        // statistics workspace: one 128-byte counter line per tensor
constexpr int kDiagSlot = NVFP4_NSTATS;  // and six binary64 partials per workgroup
static_assert(NVFP4_DIAG_WS_WORDS(1) == kDiagCtrWords + 2 * kDiagSlot * kDiagLaunchWGs &&
                  NVFP4_DIAG_WS_WORDS(2048) == 2048 * (kDiagCtrWords + 2 * kDiagSlot),
              "statistics workspace size");
using u64 = unsigned long long;

// Reference path for one candidate, straight from the definition, one binary32 step at a
// time (correctly rounded division and reciprocal, threshold-count FP4 rounding).  The
// table-driven path below covers every block except three rare kinds, which come here:
// a block max below 2^-126, a tensor alpha below 2^-118, and a block scaled to 4 whose
// scaled values may pass 5 (so that the cap at FP4 value 4 bites).  The loop is kept
// rolled and re-reads the block's values (cache-resident) so that this path adds almost
// no registers to the kernel: the hot loop's occupancy is set by the fast path alone.
template <int RULE>
__device__ __forceinline__ float ref_candidate(const uint16_t* __restrict__ xb, float bmax,
                                               float alpha, float cq, uint32_t cap,
                                               uint32_t& scale, float& d_out, uint32_t& w0,
                                               uint32_t& w1) {
  const float sigma = alpha == 0.0f ? 0.0f : bmax / cq;
  scale = e4m3_from_f32(sigma);
  const float d = e4m3_to_f32(scale) * alpha;
  d_out = d;
  const float r = d == 0.0f ? 0.0f : 1.0f / d;
  const bool r_finite = r != __builtin_inff();   // 1/d overflows only for tiny alpha
  float acc = 0.0f;
  uint32_t lo = 0u, hi = 0u;
#pragma unroll 1
  for (int i = 0; i < 16; ++i) {
    const float x = __uint_as_float((uint32_t)xb[i] << 16);
    const float v = r_finite ? x * r : x / d;
    const uint32_t m = min(e2m1_code_of(fabsf(v)), cap);
    const uint32_t sgn = __float_as_uint(x) & 0x80000000u;
    const float xhat = __uint_as_float(__float_as_uint(e2m1_value_of(m) * d) | sgn);
    const float e = x - xhat;
    if (RULE == NVFP4_RULE_MSE)      acc = __builtin_fmaf(e, e, acc);
    else if (RULE == NVFP4_RULE_MAE) acc = acc + fabsf(e);
    else                             acc = fmaxf(acc, fabsf(e));
    const uint32_t code = ((sgn >> 28) | m) << (4 * (i & 7));
    if (i < 8) lo |= code;
    else       hi |= code;
  }
  w0 = lo;
  w1 = hi;
  return acc;
}

struct RefOut {
  uint32_t s, w0, w1;
  float d;
  bool four;   // the block was scaled to 4
};

// Returned by value (in registers): outputs passed by reference would make the caller
// keep them in scratch memory on every step of the hot loop.
template <int MODE, int RULE>
__device__ __noinline__ RefOut ref_block(const uint16_t* __restrict__ xb, float bmax,
                                         float alpha) {
  RefOut o;
  o.four = false;
  const float err6 = ref_candidate<RULE>(xb, bmax, alpha, 6.0f * alpha, 7u, o.s, o.d, o.w0, o.w1);
  if (MODE == NVFP4_FOUR_OVER_SIX) {
    uint32_t s4, a4, b4;
    float d4;
    const float err4 = ref_candidate<RULE>(xb, bmax, alpha, 4.0f * alpha, 6u, s4, d4, a4, b4);
    if (err4 < err6) { o.s = s4; o.d = d4; o.w0 = a4; o.w1 = b4; o.four = true; }   // ties keep 6
  }
  return o;
}

// max(acc, |a|, |b|) in one v_max3_f32.  fmaxf on values built from integer bits makes
// the compiler canonicalize each operand first (three instructions per pair); no NaN
// reaches this code (non-finite tensors are poisoned before), so the plain max is exact.
__device__ __forceinline__ float max3_abs(float acc, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(acc), "v"(a), "v"(b));
  return r;
}

// One pair of elements of one candidate: v = x*r, FP4 round (hardware, round to nearest
// even, saturating at 6, sign kept), decode, xhat = val*d, error into the running sum.
// SEL (0..3) is the byte of the code word the pair lands in.  The two errors are also
// returned (the statistics of the diagnostics variant use them; elsewhere they are dead).
template <int RULE, int SEL>
__device__ __forceinline__ void fp4_pair(float xa, float xb, float r, float d, uint32_t& word,
                                         float& acc, float& ea, float& eb) {
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, xa * r, xb * r, 1.0f, SEL);
  const f32x2 val = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
  ea = xa - val.x * d;
  eb = xb - val.y * d;
  if (RULE == NVFP4_RULE_MSE) {
    acc = __builtin_fmaf(ea, ea, acc);
    acc = __builtin_fmaf(eb, eb, acc);
  } else if (RULE == NVFP4_RULE_MAE) {
    acc = acc + fabsf(ea);
    acc = acc + fabsf(eb);
  } else {
    acc = fmaxf(acc, fmaxf(fabsf(ea), fabsf(eb)));
  }
}

// One candidate, table-driven: 8 code bytes in two words, returns the error.  All four bytes
// of each word are written below, so their start values (init0, init1) are irrelevant: the
// caller passes values it no longer needs, so that the words need no register copies.
template <int RULE>
__device__ __forceinline__ float fast_candidate(const float (&x)[16], float r, float d,
                                                uint32_t& w0, uint32_t& w1, uint32_t init0,
                                                uint32_t init1, float (&e)[16]) {
  float acc = 0.0f;
  w0 = init0;
  w1 = init1;
  fp4_pair<RULE, 0>(x[0], x[1], r, d, w0, acc, e[0], e[1]);
  fp4_pair<RULE, 1>(x[2], x[3], r, d, w0, acc, e[2], e[3]);
  fp4_pair<RULE, 2>(x[4], x[5], r, d, w0, acc, e[4], e[5]);
  fp4_pair<RULE, 3>(x[6], x[7], r, d, w0, acc, e[6], e[7]);
  fp4_pair<RULE, 0>(x[8], x[9], r, d, w1, acc, e[8], e[9]);
  fp4_pair<RULE, 1>(x[10], x[11], r, d, w1, acc, e[10], e[11]);
  fp4_pair<RULE, 2>(x[12], x[13], r, d, w1, acc, e[12], e[13]);
  fp4_pair<RULE, 3>(x[14], x[15], r, d, w1, acc, e[14], e[15]);
  return acc;
}


// Per-tensor tables in LDS.
//   D[s] = (d, r): the step d = RN(dec(s) * alpha) of E4M3 byte s and r = RN(1/d) (0 if d = 0)
//   T[k] = (T6, T4): 2^-p_Q * RN((1 + k/128) / m_Q), where Q*alpha = m_Q * 2^p_Q, m_Q in [0.5, 1).
// A normal block max is bmax = (1 + k/128) * 2^(e-127) (bf16: 7 fraction bits), so
// bmax / (Q*alpha) = ((1 + k/128) / m_Q) * 2^(e-127-p_Q).  Rounding to binary32 commutes
// with scaling by a power of two while the result stays normal, so
// RN(bmax / (Q*alpha)) = T_Q[k] * 2^(e-127), and 2^(e-127) is bmax with its fraction bits
// cleared: one exact multiply per candidate.  T_Q[k] itself is normal whenever the block pass
// takes this path (alpha at least 2^-118, and alpha at most FLT_MAX / 1536 because it is
// amax / (6*M) for a finite amax), so its scaling by 2^-p_Q is exact too.  A product below
// 2^-126 is below half the least E4M3 subnormal, as is the exact quotient, so both become
// scale byte 0; one above the binary32 range saturates like the quotient.  This replaces two
// divisions and two reciprocals per block.
struct BlockTables {
  f32x2 D[256];
  f32x2 T[128];
};

template <int MODE>
__device__ __forceinline__ void build_tables(BlockTables& tb, float alpha) {
  const int i = threadIdx.x;
  const float c6 = 6.0f * alpha, c4 = 4.0f * alpha;
  int p6 = 0, p4 = 0;
  const float m6 = frexpf(c6, &p6);
  const float m4 = frexpf(c4, &p4);
  if (i < 256) {
    const float d = e4m3_to_f32((uint32_t)i & 0x7Fu) * alpha;
    tb.D[i] = f32x2{d, d == 0.0f ? 0.0f : 1.0f / d};
  }
  if (i < 128) {
    const float mk = 1.0f + (float)i * 0.0078125f;
    tb.T[i] = f32x2{__builtin_amdgcn_ldexpf(mk / m6, -p6),
                    MODE == NVFP4_FOUR_OVER_SIX ? __builtin_amdgcn_ldexpf(mk / m4, -p4) : 0.0f};
  }
}

// Whole block: bmax, both candidate scales from the tables, both trials, selection.
// Writes the chosen scale byte s, step d and code words; `slow` marks blocks that must be
// redone on the reference path.  For the diagnostics' statistics it also writes the chosen
// candidate's errors e and its binary32 block scale sig = RN(bmax / RN(Q*alpha)) before the
// E4M3 rounding and the clamp (valid for blocks not marked slow, while sig is normal); the
// block pass leaves them unused and the compiler drops them.
template <int MODE, int RULE>
__device__ __forceinline__ void fast_block(const float (&x)[16], const BlockTables& tb,
                                           bool& slow, uint32_t& s, float& d,
                                           uint32_t& w0, uint32_t& w1, float& bmax, bool& four,
                                           float (&e)[16], float& sig) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) m = max3_abs(m, x[i], x[i + 1]);
  bmax = m;
  const uint32_t bb = __float_as_uint(m);
  const f32x2 T = tb.T[(bb >> 16) & 0x7Fu];
  const float pe = __uint_as_float(bb & 0x7F800000u);   // 2^(e-127)
  // The E4M3 conversion turns every value above 448 into byte 0x7E or 0x7F (checked on every
  // input by the hardware-conversion test).  For 4/6 that needs no clamp: the 4-scale is 1.5
  // times the 6-scale, so whenever either passes 448 the 4-scale byte is 0x7E or above, and
  // the range check below sends the block to the reference path.  rtn6 clamps at 448.
  const float raw6 = T.x * pe;
  const float sig6 = MODE == NVFP4_FOUR_OVER_SIX ? raw6 : fminf(raw6, 448.0f);
  const float sig4 = MODE == NVFP4_FOUR_OVER_SIX ? T.y * pe : 0.0f;
  slow = bb < 0x00800000u;   // block max below 2^-126 (or zero)
  // the conversion writes the low 16 bits; the high half keeps bits of pe, which nothing reads
  const uint32_t sp =
      (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sig6, sig4, (int)__float_as_uint(pe), false);
  const uint32_t s6 = sp & 0xFFu;
  const f32x2 D6 = tb.D[s6];
  four = false;
  const float err6 = fast_candidate<RULE>(
      x, D6.y, D6.x, w0, w1, __float_as_uint(sig6),
      __float_as_uint(MODE == NVFP4_FOUR_OVER_SIX ? sig4 : T.x), e);
  s = s6;
  d = D6.x;
  sig = raw6;
  if (MODE == NVFP4_FOUR_OVER_SIX) {
    const uint32_t s4 = (sp >> 8) & 0xFFu;
    const f32x2 D4 = tb.D[s4];
    // Scaled values can pass 5 (so the cap at FP4 value 4 bites) only when the E4M3 scale
    // rounded far down: a subnormal byte, or a scale past 448 (byte 0x7E or 0x7F).  A normal
    // byte below 0x7E is within 1/16 of sigma, so the block max lands at most near 4.27.
    slow = slow || (s4 - 8u) >= 0x76u;
    uint32_t a4, b4;
    float e4[16];
    const float err4 = fast_candidate<RULE>(x, D4.y, D4.x, a4, b4, __float_as_uint(T.x),
                                            __float_as_uint(T.y), e4);
    if (err4 < err6) {                                                       // ties keep 6
      s = s4; d = D4.x; w0 = a4; w1 = b4; four = true; sig = sig4;
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = e4[i];
    }
  }
}

// ----------------------------------------------------------------------------- diagnostics
// Per-tensor error statistics over the chosen candidate of every block (fields in the order
// of NVFP4_STAT_*): sum e^2, sum |e|, max |e|, sum e^2 over the elements above 2/3 of their
// block max, sum e^2 if the chosen candidate kept its binary32 block scale, and the count of
// elements above 2/3 of their block max.  e = x - xhat is exact in binary32, so e^2 is exact
// in binary64; the sums are binary64 (lane, then wavefront, then workgroup, then the
// workgroups' partials summed by the last workgroup), so only their rounding depends on the
// order, and the launch shape fixes that order.
struct LaneStats {
  double sse, sae, near_sse, f32_sse;
  float mx;
  uint32_t near;
};

// The near-max band is 3|x| > 2 bmax.  |x| and bmax are bf16 values, and for those the test
// equals |x| > t with the per-block threshold t = RN(bmax * RN(2/3)) with its low 16 bits
// cleared: 2 bmax / 3 is either a bf16 value, which the product then rounds to exactly, or
// lies at least a third of a bf16 step away from the nearest bf16 values, so that the
// product (within 2^-23 of it, relatively) truncates to the bf16 value just below it.  (A
// test checks the equivalence for every pair of bf16 magnitudes |x| <= bmax.)
__device__ __forceinline__ float near_threshold(float bmax) {
  return __uint_as_float(__float_as_uint(bmax * 0.6666667f) & 0xFFFF0000u);
}

// Statistics of one block from its elements x and the chosen candidate's errors e (exact in
// binary32, so each e^2 is exact in binary64).  Branch-free: the far elements add a zero to
// the near sum.
__device__ __forceinline__ void block_stats(const float (&x)[16], const float (&e)[16],
                                            float tnear, LaneStats& st) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const double da = e[i], db = e[i + 1];
    st.sse = __builtin_fma(da, da, st.sse);
    st.sse = __builtin_fma(db, db, st.sse);
    st.sae = st.sae + __builtin_fabs(da);
    st.sae = st.sae + __builtin_fabs(db);
    st.mx = max3_abs(st.mx, e[i], e[i + 1]);
    const bool na = fabsf(x[i]) > tnear, nb = fabsf(x[i + 1]) > tnear;
    const double na_e = na ? e[i] : 0.0f, nb_e = nb ? e[i + 1] : 0.0f;
    st.near_sse = __builtin_fma(na_e, na_e, st.near_sse);
    st.near_sse = __builtin_fma(nb_e, nb_e, st.near_sse);
    st.near += (uint32_t)na + (uint32_t)nb;
  }
}

// The chosen candidate's errors recomputed from its codes and step d (for the blocks that
// the reference path redid): e = x - val*d, with the signed values the codes decode to.
template <int SEL>
__device__ __forceinline__ void pair_errors(uint32_t w, float xa, float xb, float d, float& ea,
                                            float& eb) {
  const f32x2 val = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  ea = xa - val.x * d;
  eb = xb - val.y * d;
}

__device__ __forceinline__ void chosen_errors(const float (&x)[16], uint32_t w0, uint32_t w1,
                                              float d, float (&e)[16]) {
  pair_errors<0>(w0, x[0], x[1], d, e[0], e[1]);
  pair_errors<1>(w0, x[2], x[3], d, e[2], e[3]);
  pair_errors<2>(w0, x[4], x[5], d, e[4], e[5]);
  pair_errors<3>(w0, x[6], x[7], d, e[6], e[7]);
  pair_errors<0>(w1, x[8], x[9], d, e[8], e[9]);
  pair_errors<1>(w1, x[10], x[11], d, e[10], e[11]);
  pair_errors<2>(w1, x[12], x[13], d, e[12], e[13]);
  pair_errors<3>(w1, x[14], x[15], d, e[14], e[15]);
}

// Sum of e^2 of one block when the chosen candidate (cq = RN(Q*alpha), capv its largest FP4
// value) keeps sigma = RN(bmax / cq) in binary32 as its block scale instead of the E4M3 byte:
// d = RN(sigma * alpha), v = RN(|x| * RN(1/d)), FP4 rounding by the hardware conversion
// (round to nearest even, saturating at 6), value capped at capv, xhat = RN(val * d),
// e = |x| - xhat (the sign of x does not change e^2).
// Blocks whose 1/d overflows (alpha far below 2^-118) divide per element instead, out of line.
__device__ __noinline__ double f32_scale_sse_div(const uint16_t* __restrict__ xb, float d,
                                                 float capv) {
  double acc = 0.0;
#pragma unroll 1
  for (int i = 0; i < 16; ++i) {
    const float x = fabsf(__uint_as_float((uint32_t)xb[i] << 16));
    const float val = fminf(e2m1_value_of(e2m1_code_of(x / d)), capv);
    const double e = (double)(x - val * d);
    acc = __builtin_fma(e, e, acc);
  }
  return acc;
}

// sig_t is the fast path's table product for the chosen candidate; table_ok says it equals
// RN(bmax / cq) (a block the fast path kept, with a normal product), else the quotient is
// formed here.
__device__ __forceinline__ double f32_scale_sse(const float (&x)[16],
                                                const uint16_t* __restrict__ xb, float bmax,
                                                float alpha, float cq, float capv, float sig_t,
                                                bool table_ok) {
  float sigma = sig_t;
  if (!table_ok) sigma = alpha == 0.0f ? 0.0f : bmax / cq;
  const float d = sigma * alpha;
  const float r = d == 0.0f ? 0.0f : 1.0f / d;
  if (r == __builtin_inff()) return f32_scale_sse_div(xb, d, capv);
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 16; k += 2) {
    const float xa = fabsf(x[k]), xc = fabsf(x[k + 1]);
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xa * r, xc * r, 1.0f, 0);
    const f32x2 val = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const double ea = (double)(xa - fminf(val.x, capv) * d);
    const double ec = (double)(xc - fminf(val.y, capv) * d);
    acc = __builtin_fma(ea, ea, acc);
    acc = __builtin_fma(ec, ec, acc);
  }
  return acc;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Outputs are written with non-temporal (streaming) stores: nothing here reads them again,
// and the pass that follows in a dynamic quantization (the next tensor's amax pass) then does
// not meet write-backs of dirty output lines.  Measured against write-back stores: the packed
// block pass 2-4 % faster and an amax + block-pass step 8-10 % faster; the fake-quant pass
// 1-2 % slower but its step 3-7 % faster.
__device__ __forceinline__ void store_packed(char* codesT, uint8_t* scalesT, uint32_t u,
                                             uint32_t w0, uint32_t w1, uint32_t sc) {
  typedef unsigned int u2v __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u2v{w0, w1}, reinterpret_cast<u2v*>(codesT + (u << 3)));
  __builtin_nontemporal_store((uint8_t)sc, scalesT + u);
}

__device__ __forceinline__ void store_fakequant(char* outT, uint32_t u, const uint32_t (&y)[8]) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4v{y[0], y[1], y[2], y[3]}, reinterpret_cast<u4v*>(outT + (u << 5)));
  __builtin_nontemporal_store(u4v{y[4], y[5], y[6], y[7]},
                              reinterpret_cast<u4v*>(outT + (u << 5) + 16));
}

// Fake-quant output with ordinary (write-back) stores.  The fused kernel's rtn6 block pass is
// light enough that its outputs leave as one burst of writes, and there ordinary stores beat
// streaming ones (8192x4096: 35.3 against 46.3 us; 4096x14336: 57.9 against 79.6 us); the
// Four Over Six pass spreads its writes over its arithmetic and keeps streaming stores (they
// measured 2-8 % faster there).
__device__ __forceinline__ void store_fakequant_wb(char* outT, uint32_t u, const uint32_t (&y)[8]) {
  *reinterpret_cast<uint4*>(outT + (u << 5)) = make_uint4(y[0], y[1], y[2], y[3]);
  *reinterpret_cast<uint4*>(outT + (u << 5) + 16) = make_uint4(y[4], y[5], y[6], y[7]);
}
__device__ __forceinline__ void unpack16(const uint4& p0, const uint4& p1, float (&x)[16]) {
  const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16_lo(w[k]);
    x[2 * k + 1] = bf16_hi(w[k]);
  }
}

// Dequantized bf16 of one block from its codes and step: 8 words (two elements each).
__device__ __forceinline__ void dequant_bf16(uint32_t w0, uint32_t w1, float d, uint32_t (&y)[8]) {
#define NVFP4_DQ(J, W, SEL)                                                              \
  {                                                                                      \
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(W, 1.0f, SEL);             \
    const f32x2 q = {v.x * d, v.y * d};                                                  \
    y[J] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, bf16x2));             \
  }
  NVFP4_DQ(0, w0, 0) NVFP4_DQ(1, w0, 1) NVFP4_DQ(2, w0, 2) NVFP4_DQ(3, w0, 3)
  NVFP4_DQ(4, w1, 0) NVFP4_DQ(5, w1, 1) NVFP4_DQ(6, w1, 2) NVFP4_DQ(7, w1, 3)
#undef NVFP4_DQ
}

// The outputs of block u held back by one step (see the block-pass loop): fake-quant, the 8
// bf16 pair words y[0..7]; packed, the code words y[0], y[1], the scale byte y[2] and, for the
// diagnostics, the block maximum it was scaled to, y[3] (qstarT is the tensor's choice array).
template <bool FQ, int DIAG>
__device__ __forceinline__ void store_late(char* outT, char* codesT, uint8_t* scalesT,
                                           uint8_t* qstarT, uint32_t u, const uint32_t (&y)[8]) {
  if (FQ) {
    store_fakequant(outT, u, y);
  } else {
    store_packed(codesT, scalesT, u, y[0], y[1], y[2]);
    if (DIAG) qstarT[u] = (uint8_t)y[3];
  }
}

// Grid: x = workgroups per tensor, y = tensor.  Lane = one 16-element block per step,
// grid-stride over the tensor's blocks; the next step's two 16-byte loads are issued before
// the current step's arithmetic.  Block indices are 32-bit (the host splits tensors of 2^27
// blocks or more into launches below that), so every access is a uniform 64-bit base plus a
// 32-bit lane offset.  DIAG (packed output only) also writes, per block, the block maximum
// it was scaled to (4 or 6) and counts the blocks scaled to 4 per tensor; DIAG == kDiagStats
// also reduces the error statistics (a variant of its own: keeping the chosen candidate's
// errors for them costs registers that the call without statistics should not pay).
constexpr int kDiagPlain = 1, kDiagStats = 2;
template <int MODE, int RULE, bool FQ, int DIAG>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NVFP4_WAVES_PER_EU))) void quantize_kernel(
    const uint4* __restrict__ in, int64_t nblk, const float* __restrict__ amax,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales, uint4* __restrict__ out,
    float* __restrict__ alpha_out, uint8_t* __restrict__ qstar, uint32_t* __restrict__ count4,
    double* __restrict__ stats, uint32_t* __restrict__ stats_ctr, double* __restrict__ stats_slots) {
  __shared__ BlockTables tb;
  const int64_t t = blockIdx.y;
  const uint32_t abits = __float_as_uint(amax[t]) & 0x7FFFFFFFu;
  const bool poison = abits >= 0x7F800000u;
  const float alpha =
      poison ? 0.0f : __uint_as_float(abits) / (MODE == NVFP4_FOUR_OVER_SIX ? kC6x256 : kC6x448);
  // alpha_out (distinct from amax) is written by the first lane of each tensor
  if (alpha_out && blockIdx.x == 0 && threadIdx.x == 0)
    alpha_out[t] = poison ? __uint_as_float(0x7FC00000u) : alpha;

  // this tensor's arrays (uniform) and 32-bit block indices
  const int64_t base = t * nblk;
  const char* inT = reinterpret_cast<const char*>(in + 2 * base);       // 32 bytes per block
  char* codesT = reinterpret_cast<char*>(codes + base);                  // 8 bytes per block
  uint8_t* scalesT = scales + base;
  char* outT = reinterpret_cast<char*>(out + 2 * base);                  // 32 bytes per block
  const uint32_t n = (uint32_t)nblk;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t u_start = u;
  // the first block's loads go out before the tables are built (they do not depend on alpha)
  uint4 nx0 = make_uint4(0u, 0u, 0u, 0u), nx1 = nx0;
  if (u < n) {
    nx0 = *reinterpret_cast<const uint4*>(inT + (u << 5));
    nx1 = *reinterpret_cast<const uint4*>(inT + (u << 5) + 16);
  }

  if (poison) {                                  // non-finite input or amax
    if (DIAG && stats && blockIdx.x == 0 && threadIdx.x == 0)
      for (int k = 0; k < NVFP4_NSTATS; ++k) stats[t * NVFP4_NSTATS + k] = __longlong_as_double(0x7FF8000000000000LL);
    for (; u < n; u += stride) {
      if (FQ) {
        const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
        *reinterpret_cast<uint4*>(outT + (u << 5)) = nan4;
        *reinterpret_cast<uint4*>(outT + (u << 5) + 16) = nan4;
      } else {
        *reinterpret_cast<uint2*>(codesT + (u << 3)) = make_uint2(0u, 0u);
        scalesT[u] = 0x7F;
        if (DIAG) qstar[base + u] = 0;
      }
    }
    return;
  }
  uint32_t n_four = 0;   // DIAG: blocks of this lane scaled to 4
  LaneStats st = {0.0, 0.0, 0.0, 0.0, 0.0f, 0u};
  constexpr bool want_stats = DIAG == kDiagStats;   // stats and its workspaces are then set

  build_tables<MODE>(tb, alpha);
  __syncthreads();
  const bool tiny_alpha = alpha < 0x1p-118f;   // 1/d may overflow below 2^-118

  // Waves that start together on a SIMD do not progress together: issue goes to the oldest
  // ready wave, so in a grid that strides over many blocks per lane some waves finish far
  // ahead of others and the launch ends with few waves in flight.  With 8 or more steps per
  // lane, each wave lowers its issue priority at a quarter, half and three quarters of its
  // steps, so the waves that are behind are issued first.  (Fewer steps: the hardware's
  // dispatch of many workgroups balances the load instead.  The diagnostics variant without
  // statistics measured 6 % slower paced, so it does not pace.)
  const uint32_t u_first = (uint32_t)__builtin_amdgcn_readfirstlane(u);
  const uint32_t steps = u_first < n ? (n - u_first + stride - 1) / stride : 0;  // wave-uniform
  const bool pace = steps >= kPacedSteps && (!DIAG || want_stats);
  const uint32_t q1 = steps / 4, q2 = steps / 2, q3 = (3 * steps) / 4;
  // Each block's outputs are stored one step late, right after the wait for the step's loads.
  // On this chip one counter (vmcnt) tracks loads and stores alike.  With the stores at the
  // end of their own step, the compiler's wait at the top of the next step came out as
  // vmcnt(0) (the loop header joins the entry path and the back edge, and the loop calls the
  // reference path), so the wait for the prefetched block also waited for the stores just
  // issued.  Stored one step late, after the vmcnt(0) that the step needs anyway for its
  // prefetched block, they have a whole step to complete, like the prefetch.  Measured
  // against stores at the end of the step (same box, A/B, two boxes): Four Over Six packed
  // 2-3 % faster (the weight 28.9 against 29.8 us, the large tensor 106.2 against 108.8, the
  // MoE batch 288.3-294.3 against 296.6-299.0); rtn6 and fake-quant equal; the diagnostics
  // call within -3.5 to +0.8 %.
  uint32_t pu = 0;                                     // the block held back, and its outputs:
  uint32_t py[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};   // fake-quant words, or codes, scale, Q*
  if (pace) __builtin_amdgcn_s_setprio(3);
  for (uint32_t step = 0; u < n; pu = u, u += stride, ++step) {
    if (pace) {
      if (step == q1) __builtin_amdgcn_s_setprio(2);
      if (step == q2) __builtin_amdgcn_s_setprio(1);
      if (step == q3) __builtin_amdgcn_s_setprio(0);
    }
    const uint4 c0 = nx0, c1 = nx1;
    float x[16];
    unpack16(c0, c1, x);
    // vmcnt(0) (expcnt 7 and lgkmcnt 15 wait for nothing) ahead of the late stores, so that
    // the wait the step needs anyway does not also cover them
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (step != 0) store_late<FQ, DIAG>(outT, codesT, scalesT, DIAG ? qstar + base : nullptr, pu, py);
    const uint32_t un = min(u + stride, n - 1);   // always in bounds: reloads the last block
    nx0 = *reinterpret_cast<const uint4*>(inT + (un << 5));
    nx1 = *reinterpret_cast<const uint4*>(inT + (un << 5) + 16);

    uint32_t sc, w0, w1;
    float dq, bm, e[16], sg;
    bool slow, four;
    fast_block<MODE, RULE>(x, tb, slow, sc, dq, w0, w1, bm, four, e, sg);
    const bool redo = slow || tiny_alpha;
    if (redo) {                      // rare: redo the block on the reference path
      const RefOut o =
          ref_block<MODE, RULE>(reinterpret_cast<const uint16_t*>(inT + (u << 5)), bm, alpha);
      sc = o.s;
      dq = o.d;
      w0 = o.w0;
      w1 = o.w1;
      four = o.four;
    }
    if (FQ) {
      dequant_bf16(w0, w1, dq, py);
    } else {
      py[0] = w0;
      py[1] = w1;
      py[2] = sc;
      py[3] = four ? 4u : 6u;
      if (DIAG) {
        n_four += four ? 1u : 0u;
        if (want_stats) {
          if (redo) chosen_errors(x, w0, w1, dq, e);
          block_stats(x, e, near_threshold(bm), st);
          st.f32_sse += f32_scale_sse(x, reinterpret_cast<const uint16_t*>(inT + (u << 5)), bm,
                                      alpha, four ? 4.0f * alpha : 6.0f * alpha,
                                      four ? 4.0f : 6.0f, sg, !redo && sg >= 0x1p-126f);
        }
      }
    }
  }
  if (u_start < n) store_late<FQ, DIAG>(outT, codesT, scalesT, DIAG ? qstar + base : nullptr, pu, py);
  if (DIAG && count4) {  // blocks scaled to 4: one integer atomic per workgroup, exact and
                         // order-free (long plain diagnostics launches count qstar afterwards)
    __shared__ uint32_t wsum[kThreads / 64];
    uint32_t v = n_four;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kThreads / 64; ++w) tot += wsum[w];
      if (tot) atomicAdd(count4 + t, tot);
    }
    if (want_stats) {
      __shared__ double wst[kThreads / 64][5];
      __shared__ float wmx[kThreads / 64];
      const double v0 = wave_sum_f64(st.sse), v1 = wave_sum_f64(st.sae);
      const double v3 = wave_sum_f64(st.near_sse), v4 = wave_sum_f64(st.f32_sse);
      uint32_t nn = st.near;
      float mx = st.mx;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        nn += __shfl_xor(nn, off);
        mx = fmaxf(mx, __shfl_xor(mx, off));
      }
      if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        wst[w][0] = v0; wst[w][1] = v1; wst[w][2] = v3; wst[w][3] = v4; wst[w][4] = (double)nn;
        wmx[w] = mx;
      }
      __syncthreads();
      // This workgroup's partial sums go to its own slot (no two workgroups write one
      // address).  Each exchange returns once it is performed at device scope, and the
      // counter increment takes its operand from all six results, so it is issued after them:
      // the workgroup whose increment finds G - 1 earlier arrivals finds every slot written.
      __shared__ int last_sh;
      if (threadIdx.x == 0) {
        double a[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
        float m = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) {
          for (int k = 0; k < 5; ++k) a[k] += wst[w][k];
          m = fmaxf(m, wmx[w]);
        }
        u64* slot = reinterpret_cast<u64*>(stats_slots + ((int64_t)t * gridDim.x + blockIdx.x) * kDiagSlot);
        const u64 r0 = __hip_atomic_exchange(slot + 0, (u64)__double_as_longlong(a[0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u64 r1 = __hip_atomic_exchange(slot + 1, (u64)__double_as_longlong(a[1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u64 r2 = __hip_atomic_exchange(slot + 2, (u64)__double_as_longlong(a[2]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u64 r3 = __hip_atomic_exchange(slot + 3, (u64)__double_as_longlong(a[3]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u64 r4 = __hip_atomic_exchange(slot + 4, (u64)__double_as_longlong(a[4]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u64 r5 = __hip_atomic_exchange(slot + 5, (u64)__double_as_longlong((double)m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t one;
        asm volatile("v_mov_b32 %0, 1" : "=v"(one) : "v"(r0), "v"(r1), "v"(r2), "v"(r3), "v"(r4), "v"(r5));
        last_sh = __hip_atomic_fetch_add(stats_ctr + t * kDiagCtrWords, one, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
      }
      __syncthreads();
      if (last_sh) {      // the last workgroup of the tensor: sum the slots in a fixed order
        const u64* sl = reinterpret_cast<const u64*>(stats_slots + (int64_t)t * gridDim.x * kDiagSlot);
        double a[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
        double m = 0.0;
        for (uint32_t g = threadIdx.x; g < gridDim.x; g += kThreads) {
          for (int k = 0; k < 5; ++k)
            a[k] += __longlong_as_double((long long)__hip_atomic_load(sl + g * kDiagSlot + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          m = fmax(m, __longlong_as_double((long long)__hip_atomic_load(sl + g * kDiagSlot + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
        }
        for (int k = 0; k < 5; ++k) a[k] = wave_sum_f64(a[k]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
        __syncthreads();                             // wst / wmx are reused below
        if ((threadIdx.x & 63) == 0) {
          const int w = threadIdx.x >> 6;
          for (int k = 0; k < 5; ++k) wst[w][k] = a[k];
          wmx[w] = (float)m;                         // m is a binary32 value
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          double tot[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
          float mt = 0.0f;
          for (int w = 0; w < kThreads / 64; ++w) {
            for (int k = 0; k < 5; ++k) tot[k] += wst[w][k];
            mt = fmaxf(mt, wmx[w]);
          }
          // added to what earlier launches over this tensor left (0 before the first)
          double* o = stats + t * NVFP4_NSTATS;
          o[NVFP4_STAT_SSE] += tot[0];
          o[NVFP4_STAT_SAE] += tot[1];
          o[NVFP4_STAT_SSE_NEAR] += tot[2];
          o[NVFP4_STAT_SSE_F32SCALE] += tot[3];
          o[NVFP4_STAT_NEAR_COUNT] += tot[4];
          o[NVFP4_STAT_MAXERR] = fmax(o[NVFP4_STAT_MAXERR], (double)mt);
          // the counter is ready for the next launch over this tensor
          __hip_atomic_store(stats_ctr + t * kDiagCtrWords, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- fused path
// Single-read dynamic quantization.  alpha depends on the whole tensor, so the two-pass path
// reads the input twice (amax pass, block pass).  Here each lane keeps its blocks on chip
// between the two phases: KR blocks in VGPRs and KL in LDS, blocks (k*G + g)*NT + lane for
// k < KR + KL (coalesced per k; NT threads per workgroup).  Phase 1 loads them and reduces the
// magnitude max.  The
// workgroups of a tensor then meet in the caller's workspace (see wait_collector and
// wait_groups), amax is published, and each workgroup runs the block pass on the blocks it holds.
// The host sizes the grid so that every workgroup can be resident at once.  The wait is
// bounded: after `wait_polls` polls or `wait_ticks` ticks of the device's constant-rate wall
// clock, whichever comes first, a workgroup computes the tensor amax itself from the input (the
// same exact value), so every wave exits whatever the scheduling.  The host derives the time
// bound from the work (a small multiple of the launch's expected load time), so that a
// workgroup kept waiting by CUs held elsewhere gives up after a few hundred microseconds.
//
// Workspace of one tensor (kFusedWsWords words, zeroed before the launch).  The collector form
// of the wait keeps one 16-bit slot per workgroup in lines 0-7 and the published amax at the
// start of lines 8-15.  The group form keeps one 128-byte line
// per group so that arrivals and polls spread over many lines.  Workgroup g belongs to group
// g % S, with S = min(16, max(1, G / 8)) groups of at least 8 workgroups (one group for up to
// 16 workgroups).  Line i starts with one 64-bit word that holds the group's max in its low
// half (a 32-bit atomicMax) and its arrival count in its high half (a 64-bit atomicAdd of
// 2^32), followed by the ready flag; the top line holds the same word over the groups.  An
// arrival's add returns the whole word, so the workgroup that completes a group reads the
// group max from that return value, with no further load, and forwards it to the top line;
// the one that completes the top line writes (amax | 1) into every group's flag (amax bits
// have 16 zero low bits), so a poller needs nothing else from memory.  With one group its
// completer publishes directly.  (Max and count in separate words took two more dependent
// round trips per level: each device-scope atomic takes about 0.7 us while the loads of other
// workgroups fill the memory system.  Measured: the 64-expert MoE batch 418.5 against 423.1
// us, 600 tensors of 256x256 35.8 against 38.0 us, the 8192x4096 fake-quant 35.7 against
// 36.5 us.  One word for all workgroups of a tensor, polled by all, measured 1.5x slower.)
//
// All of it is relaxed device-scope atomics: an acquire or release at device scope writes
// back and invalidates the L2 of the XCD, which at a thousand workgroups cost more than
// 100 us.  The one ordering needed, a workgroup's max performed before its count, comes from
// issuing the count only after the returning atomicMax is back (a register dependency on its
// result).  The completer's add is the last add to the word, and every member's max was
// performed before that member's add, so the returned low half holds every member's max;
// the top level works the same way.
constexpr uint32_t kFusedMaxWaitPolls = 1u << 26;   // the poll cap (the default); each poll is
                                                     // a device-scope load and a short sleep
// Time bound of every wait of a launch: kWaitFactor times the launch's expected load time (the
// bytes its resident workgroups load at once, at kWaitLoadRate bytes per microsecond, below the
// device-copy rate measured on MI355X) plus kWaitFloorUs.
constexpr double kWaitFactor = 8.0;
constexpr double kWaitLoadRate = 4.0e6;   // bytes per microsecond: 4 TB/s
constexpr double kWaitFloorUs = 50.0;
// Blocks per lane in team launches: kTeamKR in VGPRs plus kTeamKL in LDS.  20 per lane with
// two workgroups per CU measured best on the 64-expert MoE batch (24: no gain over two passes,
// 16: slower).  18 + 2 leaves the registers that the loop over tensors needs without spilling
// (20 in VGPRs would spill).  On the MoE batch, 4/6-MSE: 12 + 8 454-470 us, 16 + 4 430-445 us,
// 18 + 2 429-437 us (16 + 4 and 18 + 2 equal on the other batches measured).
constexpr int kTeamKR = 18;
constexpr int kTeamKL = 2;
constexpr int64_t kFusedMaxTensorWGs = 512;           // see fused_tier_wgs
// Teams of tensors under kTeamSmallBlocks blocks hold kTeamSmallKR blocks per lane in VGPRs
// and none in LDS, so that more workgroups fit per CU.  4/6-MSE against 12 + 8: 600 tensors of
// 256x256 38.9 against 47.2 us; 128 of 1024x1024 96.1 against 108.8 us (12 per lane: 107.7;
// 8 per lane: 95.7, but rtn6 fake-quant up to 4 % slower than 10).  From 262,144 blocks on,
// the larger team tier measured equal or faster (the 64-expert MoE batch: 452 against 526 us).
constexpr int64_t kTeamSmallBlocks = INT64_C(1) << 18;
constexpr int kTeamSmallKR = 10;
// Four Over Six into packed output (from kTeamSmallBlocks on) runs its teams with wider
// workgroups (at most 128 VGPRs): 512 threads, 2 waves on each SIMD and two workgroups per CU,
// holding kTeamWideKR blocks per lane in VGPRs, or kTeamWideKR - 1 in VGPRs and 4 in LDS; or
// 1024 threads, 4 waves per SIMD, one per CU, kTeamWideKR in VGPRs.  The block pass of a held
// tensor needs about four waves per SIMD to keep the VALU issuing (two per SIMD issue about
// half as fast), and the two workgroups that share a CU (workgroups i and i + #CUs) should
// compute at the same time: with teams of a power-of-two size and at least four teams, the
// odd/even start of the teams gives that (teams y and y + T/2 share CUs); otherwise the
// 1024-thread form keeps every CU in one team.  Same-box A/B (4/6-MSE packed, us per call; 18 +
// 2 at 256 threads / 10 at 512 threads, teams widened to fill every slot / 10 at 1024
// threads): 64x2048x5120 (4 teams of 128 at 512) 418 / 389 / 405; 40x2048x6144 (3 teams of
// 170) 376 / 352 / 366; 24x3072x4096 (3) 224 / 216 / 210; 96x1024x4096 (9 of 56) 279 / 273 /
// 274; 16x2048x8192 (2) 215 / 211 / 176; 12x4096x4096 (2) 165 / 154 / 135.  Then with
// power-of-two teams, 9 + 4 when 10 alone cannot make four of them: 40x2048x6144 293 against
// 349 us, 24x3072x4096 179 against 213 (4 teams of 128, 9 + 4), 96x1024x4096 263 against 265
// (8 of 64), the others unchanged.  rtn6 and fake-quant output keep the 18 + 2 tier: there the
// wide tiers measured equal or slower (rtn6 on the MoE batch 352 / 353 / 384 us, rtn6
// fake-quant 518 / 561 / 528 us, 4/6-MAE fake-quant 547 / 556 / 586 us).  (Those figures were
// taken with the group form of the wait.  With the collector form and Four Over Six loading at
// the highest issue priority, the two workgroups of a CU settle into opposite phases instead,
// one computing while the other loads and waits, and the 512-thread teams ran faster again:
// 64x2048x5120 342 against 378 us, 40x2048x6144 261 against 288, 24x3072x4096 162 against
// 181, 96x1024x4096 218 against 262.)
constexpr int kTeamWideKR = 10;
constexpr int kFusedGroups = 16;
constexpr int kLineWords = 32;                           // 128 bytes
constexpr int64_t kFusedWsWords = (kFusedGroups + 1) * kLineWords;
// The collector form of the wait (see wait_collector): 16-bit slots in lines 0-7, flags at the
// start of lines 8-15.
constexpr uint32_t kFlagLine0 = 8, kFlagLines = 8;
static_assert(2 * kFusedMaxTensorWGs <= 4 * kLineWords * kFlagLine0 &&
                  (kFlagLine0 + kFlagLines) * kLineWords <= kFusedWsWords,
              "fused workspace: one slot per workgroup and the flag lines");
static_assert(kFusedWsWords == NVFP4_FUSED_WS_WORDS, "workspace size of the fused calls");

// Magnitude max of tensor t computed by one workgroup of NT threads alone (the fallback of the
// wait).
template <int NT>
__device__ __noinline__ uint32_t wg_tensor_amax(const uint4* __restrict__ p, int64_t chunks,
                                                uint32_t* part) {
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < chunks; i += NT) m = mag_max8(m, p[i]);
  m = max(m & 0xFFFFu, m >> 16) << 16;
  m = wave_max_u32(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = part[0];
  for (int w = 1; w < NT / 64; ++w) r = max(r, part[w]);
  __syncthreads();   // every wave has read part[] before any reuses it (the next tensor)
  return r;
}

// Block pass of one block held on chip: the same steps and stores as quantize_kernel.
template <int MODE, int RULE, bool FQ>
__device__ __forceinline__ void fused_emit(const uint4& c0, const uint4& c1, uint32_t u,
                                           const char* inT, char* codesT, uint8_t* scalesT,
                                           char* outT, const BlockTables& tb,
                                           float alpha, bool tiny_alpha) {
  float x[16];
  unpack16(c0, c1, x);
  uint32_t sc, w0, w1;
  float dq, bm, e_unused[16], sg_unused;
  bool slow, four;
  fast_block<MODE, RULE>(x, tb, slow, sc, dq, w0, w1, bm, four, e_unused, sg_unused);
  if (slow || tiny_alpha) {
    const RefOut o =
        ref_block<MODE, RULE>(reinterpret_cast<const uint16_t*>(inT + (u << 5)), bm, alpha);
    sc = o.s;
    dq = o.d;
    w0 = o.w0;
    w1 = o.w1;
  }
  if (FQ) {
    uint32_t y[8];
    dequant_bf16(w0, w1, dq, y);
    if (MODE == NVFP4_RTN6) store_fakequant_wb(outT, u, y);
    else                    store_fakequant(outT, u, y);
  } else {
    store_packed(codesT, scalesT, u, w0, w1, sc);
  }
}

template <bool FQ>
__device__ __forceinline__ void fused_poison(uint32_t u, char* codesT, uint8_t* scalesT,
                                             char* outT) {
  if (FQ) {
    const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    *reinterpret_cast<uint4*>(outT + (u << 5)) = nan4;
    *reinterpret_cast<uint4*>(outT + (u << 5) + 16) = nan4;
  } else {
    *reinterpret_cast<uint2*>(codesT + (u << 3)) = make_uint2(0u, 0u);
    scalesT[u] = 0x7F;
  }
}

// The grid-wide wait of the G workgroups of one tensor, in one of two forms, each bounded by
// polls and wall-clock ticks.  Both return the tensor's magnitude max (bf16 magnitude bits
// << 16) in lane 0, or 0xFFFFFFFF when the wait gave up ("compute it here").  wt is the tensor's
// workspace (kFusedWsWords words, zero at the call's start), wgm this workgroup's max.
//
// Collector form (wave 0 of every workgroup).  Each workgroup stores its max with a set top
// bit into its own 16-bit slot (words 0-255: up to 512 slots): the value is its own flag, so
// nothing orders one word against another.  Workgroup 0 alone reads all slots (16 bytes per
// lane) until each is set, then writes max | 1 to kFlagLines flag lines, each of which a
// share of the workgroups polls.  From the last arrival to the release this is a store, one
// read of the slots and a store, about half the chain of the group form.
// Two words at device scope (the coherence of agent-scope atomic loads) from a uniform base
// plus a lane's byte offset (plus 512 bytes when HI), waited for in the same statement.
template <bool HI>
__device__ __forceinline__ uint2 load_slots(const uint32_t* base, uint32_t off) {
  uint2 v;
  if (HI)
    asm volatile("global_load_dwordx2 %0, %1, %2 offset:512 sc1\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(v) : "v"(off), "s"(base) : "memory");
  else
    asm volatile("global_load_dwordx2 %0, %1, %2 sc1\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(v) : "v"(off), "s"(base) : "memory");
  return v;
}

__device__ __forceinline__ void slots_check(uint2 v, uint32_t first, uint32_t G, bool& ok,
                                            uint32_t& mx) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (first + c < G) {
      const uint32_t h = ((c < 2 ? v.x : v.y) >> (16 * (c & 1))) & 0xFFFFu;
      ok = ok && (h & 0x8000u);
      mx = max(mx, h & 0x7FFFu);
    }
}

__device__ __forceinline__ uint32_t wait_collector(uint32_t* wt, uint32_t wgm, uint32_t g,
                                                   uint32_t G, uint32_t lane,
                                                   uint32_t wait_polls, uint64_t wait_ticks) {
  if (lane == 0)
    __hip_atomic_store(reinterpret_cast<uint16_t*>(wt) + g, (uint16_t)(0x8000u | (wgm >> 16)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t0 = wall_clock64();
  if (g == 0) {
    uint32_t polls = 0, mx = 0;
    bool done = false;
    for (;;) {                                     // lane l reads slots 4l.. and 256 + 4l..
      bool ok = true;
      mx = 0;
      if (4 * lane < G) slots_check(load_slots<false>(wt, 8 * lane), 4 * lane, G, ok, mx);
      if (256 + 4 * lane < G) slots_check(load_slots<true>(wt, 8 * lane), 256 + 4 * lane, G, ok, mx);
      if (__all(ok)) { done = true; break; }
      if (polls++ >= wait_polls || wall_clock64() - t0 > wait_ticks) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (done) {
      mx = wave_max_u32(mx);
      if (lane < kFlagLines)
        __hip_atomic_store(wt + (kFlagLine0 + lane) * kLineWords, (mx << 16) | 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  uint32_t flag = 0;
  if (lane == 0) {
    const uint32_t* line = wt + (kFlagLine0 + g % kFlagLines) * kLineWords;
    uint32_t polls = 0;
    while (!((flag = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & 1u)) {
      if (polls++ >= wait_polls || wall_clock64() - t0 > wait_ticks) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return (flag & 1u) ? (flag & ~1u) : 0xFFFFFFFFu;
}

// Group form (lane 0).  Groups of at least 8 workgroups, at most 16 groups, one 128-byte line
// each; one group needs no top level.  Up to 16 workgroups meet on one line (measured 11 %
// faster for the 16-workgroup 256x256 call); 128 workgroups on one line measured 1.5x slower
// than 16 groups of 8.  A line starts with one 64-bit word: the max in its low half and the
// arrival count in its high half; word 2 is the group's ready flag.
__device__ __forceinline__ uint32_t wait_groups(uint32_t* wt, uint32_t wgm, uint32_t g,
                                                uint32_t G, uint32_t lane,
                                                uint32_t wait_polls, uint64_t wait_ticks) {
  if (lane != 0) return 0xFFFFFFFFu;
  const uint32_t S = G <= 16u ? 1u : min((uint32_t)kFusedGroups, max(1u, G / 8u));
  const uint32_t grp = g % S;
  uint32_t* line = wt + grp * kLineWords;     // [0] max, [1] count (one 64-bit word), [2] flag
  uint32_t* top = wt + kFusedGroups * kLineWords;        // [0] max, [1] count
  const uint32_t members = (G - grp + S - 1) / S;
  const uint32_t prev =
      __hip_atomic_fetch_max(line, wgm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t one;
  asm volatile("v_mov_b32 %0, 1" : "=v"(one) : "v"(prev));   // waits for the max to return
  const uint64_t word = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(line),
                                               (uint64_t)one << 32, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(word >> 32) == members - 1) {                // this group is complete
    const uint32_t gm = max((uint32_t)word, wgm);
    if (S == 1) {                                             // the only group: publish
      __hip_atomic_store(line + 2, gm | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const uint32_t prev2 =
          __hip_atomic_fetch_max(top, gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t one2;
      asm volatile("v_mov_b32 %0, 1" : "=v"(one2) : "v"(prev2));
      const uint64_t word2 = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(top),
                                                    (uint64_t)one2 << 32, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(word2 >> 32) == S - 1) {                 // every group is complete
        const uint32_t ready = max((uint32_t)word2, gm) | 1u;
        for (uint32_t i = 0; i < S; ++i)
          __hip_atomic_store(wt + i * kLineWords + 2, ready, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  uint32_t polls = 0, flag;
  const uint64_t t0 = wall_clock64();
  while (!((flag = __hip_atomic_load(line + 2, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT)) & 1u)) {
    if (polls++ >= wait_polls || wall_clock64() - t0 > wait_ticks) break;
    __builtin_amdgcn_s_sleep(2);
  }
  return (flag & 1u) ? (flag & ~1u) : 0xFFFFFFFFu;
}

// One tensor t of a fused launch (x = G workgroups of NT threads per tensor): phase 1, the
// grid-wide wait (the group form when GROUPS, else the collector form), phase 2.
// nblk <= (KR + KL) * G * NT per tensor, G <= kFusedMaxTensorWGs and nblk < 2^27 (the host
// checks all three).
template <int MODE, int RULE, bool FQ, int KR, int KL, int NT, bool GROUPS>
__device__ __forceinline__ void fused_tensor(
    int64_t t, uint32_t tid, const uint4* __restrict__ in, int64_t nblk,
    uint32_t* __restrict__ ws, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    uint4* __restrict__ out, float* __restrict__ alpha_out, uint32_t wait_polls,
    uint64_t wait_ticks, BlockTables& tb,
    uint4 (&held)[KL > 0 ? KL : 1][2][NT], uint32_t* part, uint32_t& amax_sh) {
  const uint32_t G = gridDim.x, g = blockIdx.x;
  const uint32_t n = (uint32_t)nblk;
  const int64_t base = t * nblk;
  const char* inT = reinterpret_cast<const char*>(in + 2 * base);
  char* codesT = reinterpret_cast<char*>(codes + base);
  uint8_t* scalesT = scales + base;
  char* outT = reinterpret_cast<char*>(out + 2 * base);

  // Four Over Six loads at the highest issue priority: a workgroup's loading phase has few
  // VALU instructions, and when the workgroup sharing its CU is in the block pass (two trials
  // per block, VALU-bound), they would otherwise wait behind it and delay the arrival of the
  // whole tensor.  rtn6's block pass is light; there the plain pacing measured faster.
  constexpr bool kLoadFirst = MODE == NVFP4_FOUR_OVER_SIX;
  if (kLoadFirst) __builtin_amdgcn_s_setprio(3);
  // phase 1: load every held block (all loads in flight together), magnitude max.  In
  // workgroups of 512 and 1024 threads the blocks held in LDS are loaded straight into it
  // (global_load_lds_dwordx4: each wave writes 1 KB, 16 bytes per lane in lane order, which is
  // the layout of held[k][half][tid]), so they take no VGPRs on the way; lanes past the end
  // load the last block again, which leaves the magnitude max as it is.  Each wave then reads
  // back only its own lanes' blocks, after its own loads have landed.
  constexpr bool kDma = NT >= 512 && KL > 0;
  uint4 r0[KR], r1[KR], l0[KL > 0 ? KL : 1], l1[KL > 0 ? KL : 1];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const uint32_t u = ((uint32_t)k * G + g) * NT + tid;
    r0[k] = r1[k] = make_uint4(0u, 0u, 0u, 0u);
    if (u < n) {
      r0[k] = *reinterpret_cast<const uint4*>(inT + (u << 5));
      r1[k] = *reinterpret_cast<const uint4*>(inT + (u << 5) + 16);
    }
  }
#pragma unroll
  for (int k = 0; k < KL; ++k) {
    const uint32_t u = ((uint32_t)(KR + k) * G + g) * NT + tid;
    if constexpr (kDma) {
      const uint4* src = reinterpret_cast<const uint4*>(inT + (min(u, n - 1) << 5));
      __builtin_amdgcn_global_load_lds(src, &held[k][0][tid & ~63u], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(src + 1, &held[k][1][tid & ~63u], 16, 0, 0);
    } else {
      l0[k] = l1[k] = make_uint4(0u, 0u, 0u, 0u);
      if (u < n) {
        l0[k] = *reinterpret_cast<const uint4*>(inT + (u << 5));
        l1[k] = *reinterpret_cast<const uint4*>(inT + (u << 5) + 16);
      }
    }
  }
  // Every load is issued before the first use of a loaded register: the compiler waits for
  // all outstanding loads at such a use once LDS-bound loads are among them, so a use
  // scheduled between the loads would hold back the loads after it by a whole round trip.
  if constexpr (kDma) __builtin_amdgcn_sched_barrier(0);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < KR; ++k) m = mag_max8(mag_max8(m, r0[k]), r1[k]);
  if constexpr (kDma) __builtin_amdgcn_s_waitcnt(0);   // this wave's loads have landed
#pragma unroll
  for (int k = 0; k < KL; ++k) {
    if constexpr (kDma) {
      m = mag_max8(mag_max8(m, held[k][0][tid]), held[k][1][tid]);
    } else {
      m = mag_max8(mag_max8(m, l0[k]), l1[k]);
      held[k][0][tid] = l0[k];
      held[k][1][tid] = l1[k];
    }
  }
  m = max(m & 0xFFFFu, m >> 16) << 16;
  m = wave_max_u32(m);
  if ((tid & 63) == 0) part[tid >> 6] = m;
  __syncthreads();

  // arrival and the grid-wide wait (wave 0), bounded
  if (tid < 64) {
    uint32_t wgm = part[0];
    for (int w = 1; w < NT / 64; ++w) wgm = max(wgm, part[w]);
    uint32_t* wt = ws + t * kFusedWsWords;
    const uint32_t a = GROUPS ? wait_groups(wt, wgm, g, G, tid, wait_polls, wait_ticks)
                              : wait_collector(wt, wgm, g, G, tid, wait_polls, wait_ticks);
    if (tid == 0) amax_sh = a;
  }
  __syncthreads();
  uint32_t abits = amax_sh;
  if (abits == 0xFFFFFFFFu)
    abits = wg_tensor_amax<NT>(reinterpret_cast<const uint4*>(inT), nblk * 2, part);

  // phase 2: the block pass on the held blocks
  const bool poison = abits >= 0x7F800000u;
  const float alpha =
      poison ? 0.0f : __uint_as_float(abits) / (MODE == NVFP4_FOUR_OVER_SIX ? kC6x256 : kC6x448);
  if (g == 0 && tid == 0) alpha_out[t] = poison ? __uint_as_float(0x7FC00000u) : alpha;
  if (poison) {
#pragma unroll
    for (int k = 0; k < KR + KL; ++k) {
      const uint32_t u = ((uint32_t)k * G + g) * NT + tid;
      if (u < n) fused_poison<FQ>(u, codesT, scalesT, outT);
    }
    return;
  }
  build_tables<MODE>(tb, alpha);
  __syncthreads();
  const bool tiny_alpha = alpha < 0x1p-118f;   // 1/d may overflow below 2^-118
  // Phase 2 is bound by the VALU and every workgroup starts it at once: the waves pace
  // themselves as in quantize_kernel, lowering their issue priority by quarters of the held
  // blocks (3, 2, 1, 0; for Four Over Six 2, 1, 0, 0, below its loading phase).
  constexpr int K = KR + KL;
  constexpr bool pace = K >= (int)kPacedSteps;
  constexpr int P0 = kLoadFirst ? 2 : 3;
  if (pace) __builtin_amdgcn_s_setprio(P0);
  else if (kLoadFirst) __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (pace && k == K / 4) __builtin_amdgcn_s_setprio(P0 - 1);
    if (pace && k == K / 2) __builtin_amdgcn_s_setprio(P0 - 2 > 0 ? P0 - 2 : 0);
    if (pace && k == (3 * K) / 4) __builtin_amdgcn_s_setprio(0);
    const uint32_t u = ((uint32_t)k * G + g) * NT + tid;
    if (u < n)
      fused_emit<MODE, RULE, FQ>(r0[k], r1[k], u, inT, codesT, scalesT, outT, tb,
                                 alpha, tiny_alpha);
  }
#pragma unroll
  for (int k = 0; k < KL; ++k) {
    if (pace && KR + k == K / 4) __builtin_amdgcn_s_setprio(P0 - 1);
    if (pace && KR + k == K / 2) __builtin_amdgcn_s_setprio(P0 - 2 > 0 ? P0 - 2 : 0);
    if (pace && KR + k == (3 * K) / 4) __builtin_amdgcn_s_setprio(0);
    const uint32_t u = ((uint32_t)(KR + k) * G + g) * NT + tid;
    if (u < n)
      fused_emit<MODE, RULE, FQ>(held[k][0][tid], held[k][1][tid], u, inT, codesT, scalesT,
                                 outT, tb, alpha, tiny_alpha);
  }
}

// Grid: x = G workgroups per tensor, y = tensor (TEAMS false), or y = team (TEAMS true): a team
// of G workgroups takes tensors y, y + gridDim.y, ... in turn.  All workgroups are resident
// together, and teams at different tensors overlap one tensor's loads with another's
// arithmetic.  Between tensors a team needs no barrier of its own: a workgroup's threads reuse
// only their own held blocks, and the shared tables and flags are rewritten only after the next
// tensor's phase-1 barriers, which every thread of the workgroup reaches after its phase 2.
// NT threads per workgroup: 256, or 512 and 1024 for the Four Over Six team tiers below (at
// most 128 VGPRs, so that 4 waves per SIMD fit).
template <int MODE, int RULE, bool FQ, int KR, int KL, bool TEAMS, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT > 256 ? 4 : 2))) void fused_kernel(
    const uint4* __restrict__ in, int64_t nblk, uint32_t* __restrict__ ws,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales, uint4* __restrict__ out,
    float* __restrict__ alpha_out, uint32_t wait_polls, uint64_t wait_ticks, int64_t E) {
  __shared__ BlockTables tb;
  __shared__ uint4 held[KL > 0 ? KL : 1][2][NT];
  __shared__ uint32_t part[NT / 64];
  __shared__ uint32_t amax_sh;
  // The wait's form: groups for the 28-block fake-quant instances (the collector's state does
  // not fit beside their 224 VGPRs of held blocks), the collector for every other instance.
  constexpr bool kGroups = FQ && KR + KL >= 28;
  if (!TEAMS) {
    fused_tensor<MODE, RULE, FQ, KR, KL, NT, kGroups>(blockIdx.y, threadIdx.x, in, nblk, ws, codes,
                                                    scales, out, alpha_out, wait_polls,
                                                    wait_ticks, tb, held, part, amax_sh);
    return;
  }
  // Teams that start together stay in step: all load, then all compute, and memory idles while
  // the VALU works.  Odd teams therefore start when the team before them has published its
  // first amax (that tensor's ready flag), half a cycle later, so that one half of the
  // teams loads while the other computes.  The wait is bounded like the grid-wide one; giving
  // up only costs the overlap.  Measured on the 64-expert MoE batch: 445 against 495 us.
  if ((blockIdx.y & 1) && threadIdx.x == 0) {
    const uint32_t* flag =
        ws + (blockIdx.y - 1) * kFusedWsWords + (kGroups ? 2 : kFlagLine0 * kLineWords);
    const uint64_t t0 = wall_clock64();
    for (uint32_t polls = 0; polls < wait_polls && wall_clock64() - t0 <= wait_ticks &&
         !(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u); ++polls)
      __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
  for (int64_t t = blockIdx.y; t < E; t += gridDim.y) {
    // The block offsets do not depend on t; an opaque copy of the lane id keeps the compiler
    // from hoisting them out of the loop, where they would stay live in registers.
    uint32_t tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(threadIdx.x));
    fused_tensor<MODE, RULE, FQ, KR, KL, NT, kGroups>(t, tid, in, nblk, ws, codes, scales, out,
                                                      alpha_out, wait_polls, wait_ticks, tb,
                                                      held, part, amax_sh);
  }
}

// Dequantize: packed codes + scale bytes + alpha -> bf16, one block per lane per step.
// d = RN(dec(s) * alpha) and y = bf16(RN(val(code) * d)): the values the fake-quant output
// holds for the tensor that was quantized.  A NaN alpha or scale byte gives NaN (0x7FC0).
// Grid and addressing as in quantize_kernel: x = workgroups per tensor, y = tensor, 32-bit
// block indices, grid-stride with the next step's 9 bytes loaded before the current step's
// arithmetic; launched with one block per lane.
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint2* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ alpha,
                                                           int64_t nblk, uint4* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const float al = alpha[t];
  const bool nan_alpha = al != al;
  const int64_t base = t * nblk;
  const char* codesT = reinterpret_cast<const char*>(codes + base);   // 8 bytes per block
  const uint8_t* scalesT = scales + base;
  char* outT = reinterpret_cast<char*>(out + 2 * base);              // 32 bytes per block
  const uint32_t n = (uint32_t)nblk;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  uint2 nc = make_uint2(0u, 0u);
  uint32_t ns = 0u;
  if (u < n) {
    nc = *reinterpret_cast<const uint2*>(codesT + (u << 3));
    ns = scalesT[u];
  }
  for (; u < n; u += stride) {
    const uint2 c = nc;
    const uint32_t sb = ns;
    const uint32_t un = min(u + stride, n - 1);   // always in bounds: reloads the last block
    nc = *reinterpret_cast<const uint2*>(codesT + (un << 3));
    ns = scalesT[un];
    uint32_t y[8];
    if (nan_alpha || (sb & 0x7Fu) == 0x7Fu) {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = 0x7FC07FC0u;
    } else {
      const float dec = e4m3_to_f32(sb & 0x7Fu);
      dequant_bf16(c.x, c.y, (sb & 0x80u ? -dec : dec) * al, y);
    }
    // ordinary stores: streaming ones measured 20 % slower here (a write-only stream)
    *reinterpret_cast<uint4*>(outT + (u << 5)) = make_uint4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<uint4*>(outT + (u << 5) + 16) = make_uint4(y[4], y[5], y[6], y[7]);
  }
}

// ----------------------------------------------------------------------------- host side
struct Shape {
  int64_t E, rows, cols, n, nblk;   // n = elements per tensor, nblk = blocks per tensor
};

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + (uintptr_t)bbytes && pb < pa + (uintptr_t)abytes;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

nvfp4_status check_shape(int64_t E, int64_t rows, int64_t cols, Shape* s) {
  if (E <= 0 || rows <= 0 || cols <= 0 || cols % NVFP4_BLOCK != 0 || E > 65535)
    return NVFP4_ERR_SHAPE;
  // E * rows * cols * 2 bytes must fit in int64 with room for index arithmetic
  const int64_t lim = INT64_C(1) << 60;
  if (rows > lim / cols || E > lim / (rows * cols)) return NVFP4_ERR_SHAPE;
  s->E = E;
  s->rows = rows;
  s->cols = cols;
  s->n = rows * cols;
  s->nblk = s->n / NVFP4_BLOCK;
  if ((s->nblk + kThreads - 1) / kThreads > INT32_MAX) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

nvfp4_status check_common(const uint16_t* in, const Shape& s, int block, int mode, int rule) {
  if (!in) return NVFP4_ERR_NULL;
  if (block != NVFP4_BLOCK) return NVFP4_ERR_BLOCK;
  if ((mode != NVFP4_RTN6 && mode != NVFP4_FOUR_OVER_SIX) ||
      (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAXERR))
    return NVFP4_ERR_ENUM;
  if (!aligned(in, 16)) return NVFP4_ERR_ALIGN;
  (void)s;
  return NVFP4_OK;
}

hipError_t launch_amax(const uint16_t* in, const Shape& s, uint32_t* acc, hipStream_t stream,
                       uint32_t* acc2 = nullptr, uint32_t* acc3 = nullptr, int64_t n3 = 0,
                       uint32_t* acc4 = nullptr, int64_t n4 = 0) {
  const int64_t chunks = s.n / 8;
  const int64_t share = std::max<int64_t>(1, kAmaxWGs / s.E);   // workgroups per tensor
  const int64_t want8 = (chunks + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
  const int64_t want1 = (chunks + kAmaxThreads - 1) / kAmaxThreads;
  const bool wide = want8 >= share;
  // wide: as few workgroups as keep the steps per lane at ceil(want8 / share), so that no
  // workgroup runs a last step that the others do not
  // (4096x14336: 224 workgroups of 4 steps, 23.31 against 23.81 us for 256 of 3.5 steps)
  const int64_t per_tensor =
      wide ? (want8 + (want8 + share - 1) / share - 1) / ((want8 + share - 1) / share)
           : std::max<int64_t>(1, std::min<int64_t>(want1, share));
  const int64_t nclear = std::max({s.E, acc3 ? n3 : 0, acc4 ? n4 : 0});
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclear + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, stream, acc, acc2, s.E, acc3, n3, acc4, n4);
  // A single tensor of at most 8 steps per lane reads coalesced (each load instruction 1 KB
  // contiguous); longer tensors and batches read 128 contiguous bytes per lane.  Same-box A/B,
  // median of 6 rounds: 4096x14336 22.72 against 23.27 us, 8192x4096 15.54 against 16.12, but
  // 16384x14336 (14 steps) 78.93 against 77.10; an earlier A/B found the 64-expert batch
  // 227.4 against 217.4 coalesced.
  const bool coalesced = wide && s.E == 1 && want8 <= 8 * share;
  if (coalesced)
    hipLaunchKernelGGL((amax_kernel<8, true>), dim3((unsigned)per_tensor, (unsigned)s.E), dim3(kAmaxThreads),
                       0, stream, reinterpret_cast<const uint4*>(in), chunks, acc);
  else if (wide)
    hipLaunchKernelGGL((amax_kernel<8, false>), dim3((unsigned)per_tensor, (unsigned)s.E), dim3(kAmaxThreads),
                       0, stream, reinterpret_cast<const uint4*>(in), chunks, acc);
  else
    hipLaunchKernelGGL((amax_kernel<1, false>), dim3((unsigned)per_tensor, (unsigned)s.E), dim3(kAmaxThreads),
                       0, stream, reinterpret_cast<const uint4*>(in), chunks, acc);
  return hipGetLastError();
}

constexpr int64_t kMaxLaunchBlocks = (INT64_C(1) << 27) - 1;   // 32-bit byte offsets in kernels

template <int MODE, int RULE, bool FQ, int DIAG>
void launch_quantize_t(const uint16_t* in, const Shape& s, const float* amax, uint8_t* codes,
                       uint8_t* scales, uint16_t* out, float* alpha_out, uint8_t* qstar,
                       uint32_t* count4, double* stats, uint32_t* stats_ws, hipStream_t stream) {
  // statistics workspace: E counter lines, then the slots (reused by consecutive launches)
  double* const slots = stats_ws ? reinterpret_cast<double*>(stats_ws + s.E * kDiagCtrWords)
                                 : nullptr;
  // The diagnostics count the blocks scaled to 4 with one atomic per workgroup, which keeps
  // their grid at kDiagLaunchWGs workgroups.  A long plain diagnostics call instead takes the
  // block pass's grid and counts the choice bytes afterwards (count4_kernel): the 64-expert MoE
  // batch 538 against 595 us (4/6-MSE) and 522 against 605 (rtn6); short calls measured up to
  // 7 % slower that way (the weight: 58.1 against 55.0 us), so they keep the atomic.
  const bool count_after = DIAG == kDiagPlain && s.E * s.nblk >= kLongLaunchBlocks;
  auto launch = [&](int64_t E, int64_t nblk, int64_t first_tensor, int64_t first_block) {
    const int64_t one_per_lane = (nblk + kThreads - 1) / kThreads;
    int64_t per_tensor = one_per_lane;
    if (DIAG && !count_after)   // the statistics need their kDiagLaunchWGs workspace slots
      per_tensor = std::min(one_per_lane,
                            std::max<int64_t>(1, (DIAG == kDiagPlain ? kShortLaunchWGs
                                                                      : kDiagLaunchWGs) / E));
    else if (MODE == NVFP4_FOUR_OVER_SIX && !FQ)
      per_tensor = E * nblk < kLongLaunchBlocks
                       ? std::min(one_per_lane, std::max<int64_t>(1, kShortLaunchWGs / E))
                       : (nblk + kThreads * kLaneBlocksLong - 1) / (kThreads * kLaneBlocksLong);
    const int64_t b0 = first_tensor * s.nblk + first_block;   // first block of this launch
    hipLaunchKernelGGL((quantize_kernel<MODE, RULE, FQ, DIAG>),
                       dim3((unsigned)per_tensor, (unsigned)E), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(in + b0 * 16), nblk, amax + first_tensor,
                       reinterpret_cast<uint2*>(codes ? codes + b0 * 8 : nullptr),
                       scales ? scales + b0 : nullptr,
                       reinterpret_cast<uint4*>(out ? out + b0 * 16 : nullptr),
                       alpha_out ? alpha_out + first_tensor : nullptr, qstar ? qstar + b0 : nullptr,
                       count4 && !count_after ? count4 + first_tensor : nullptr,
                       stats ? stats + first_tensor * NVFP4_NSTATS : nullptr,
                       stats ? stats_ws + first_tensor * kDiagCtrWords : nullptr,
                       stats ? slots : nullptr);
  };
  if (s.nblk <= kMaxLaunchBlocks) {
    launch(s.E, s.nblk, 0, 0);
  } else {                  // tensors of 2^27 blocks or more: one launch per tensor and chunk
    for (int64_t t = 0; t < s.E; ++t)
      for (int64_t b = 0; b < s.nblk; b += kMaxLaunchBlocks)
        launch(1, std::min(kMaxLaunchBlocks, s.nblk - b), t, b);
  }
  if (count_after) {        // 16-byte chunks per tensor, 16 per lane, up to kDiagLaunchWGs WGs
    const int64_t per_tensor = std::max<int64_t>(
        1, std::min<int64_t>(std::max<int64_t>(1, kDiagLaunchWGs / s.E),
                             (s.nblk + 16 * 16 * kThreads - 1) / (16 * 16 * kThreads)));
    hipLaunchKernelGGL(count4_kernel, dim3((unsigned)per_tensor, (unsigned)s.E), dim3(kThreads),
                       0, stream, qstar, s.nblk, count4);
  }
}

template <bool FQ, int DIAG>
void launch_quantize(int mode, int rule, const uint16_t* in, const Shape& s, const float* amax,
                     uint8_t* codes, uint8_t* scales, uint16_t* out, float* alpha_out,
                     uint8_t* qstar, uint32_t* count4, double* stats, uint32_t* stats_ws,
                     hipStream_t stream) {
  if (mode == NVFP4_RTN6) {
    launch_quantize_t<NVFP4_RTN6, NVFP4_RULE_MSE, FQ, DIAG>(in, s, amax, codes, scales, out,
                                                            alpha_out, qstar, count4, stats, stats_ws, stream);
  } else if (rule == NVFP4_RULE_MSE) {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE, FQ, DIAG>(
        in, s, amax, codes, scales, out, alpha_out, qstar, count4, stats, stats_ws, stream);
  } else if (rule == NVFP4_RULE_MAE) {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAE, FQ, DIAG>(
        in, s, amax, codes, scales, out, alpha_out, qstar, count4, stats, stats_ws, stream);
  } else {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAXERR, FQ, DIAG>(
        in, s, amax, codes, scales, out, alpha_out, qstar, count4, stats, stats_ws, stream);
  }
}

hipError_t launch_alpha(const uint32_t* amax_bits, float* alpha, const Shape& s, int mode,
                        hipStream_t stream) {
  hipLaunchKernelGGL(alpha_kernel, dim3((unsigned)((s.E + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, amax_bits, alpha, s.E,
                     mode == NVFP4_FOUR_OVER_SIX ? kC6x256 : kC6x448);
  return hipGetLastError();
}

// Shared body of every packed / fake-quant entry point.  amax_in == nullptr: dynamic scale
// (out_alpha is the amax accumulator); otherwise the caller's amax.
// Arguments shared by every packed / fake-quant entry point: shape, enums, the outputs of the
// chosen form (packed or fake-quant), alignment and overlaps.
nvfp4_status validate_main(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int block,
                           int mode, int rule, const float* amax_in, const uint8_t* codes,
                           const uint8_t* scales, const uint16_t* out, const float* alpha, bool fq,
                           Shape* sp) {
  Shape& s = *sp;
  nvfp4_status st = check_shape(E, rows, cols, &s);
  if (st != NVFP4_OK) return st;
  st = check_common(in, s, block, mode, rule);
  if (st != NVFP4_OK) return st;
  if (!alpha || (fq ? !out : (!codes || !scales))) return NVFP4_ERR_NULL;
  if (!aligned(alpha, 4) || (amax_in && !aligned(amax_in, 4))) return NVFP4_ERR_ALIGN;
  if (fq ? !aligned(out, 16) : !aligned(codes, 16)) return NVFP4_ERR_ALIGN;
  const int64_t in_bytes = s.E * s.n * 2;
  const int64_t alpha_bytes = s.E * 4;
  if (overlap(alpha, alpha_bytes, in, in_bytes)) return NVFP4_ERR_ALIAS;
  if (amax_in && overlap(alpha, alpha_bytes, amax_in, alpha_bytes) && alpha != amax_in)
    return NVFP4_ERR_ALIAS;
  if (fq) {
    if (out != in && overlap(out, in_bytes, in, in_bytes)) return NVFP4_ERR_ALIAS;
    if (overlap(out, in_bytes, alpha, alpha_bytes)) return NVFP4_ERR_ALIAS;
    if (amax_in && overlap(out, in_bytes, amax_in, alpha_bytes)) return NVFP4_ERR_ALIAS;
  } else {
    const int64_t cb = s.E * s.n / 2, sb = s.E * s.nblk;
    if (overlap(codes, cb, in, in_bytes) || overlap(scales, sb, in, in_bytes) ||
        overlap(codes, cb, scales, sb) || overlap(codes, cb, alpha, alpha_bytes) ||
        overlap(scales, sb, alpha, alpha_bytes))
      return NVFP4_ERR_ALIAS;
    if (amax_in && (overlap(codes, cb, amax_in, alpha_bytes) ||
                    overlap(scales, sb, amax_in, alpha_bytes)))
      return NVFP4_ERR_ALIAS;
  }
  return NVFP4_OK;
}

nvfp4_status run(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int block, int mode,
                 int rule, const float* amax_in, uint8_t* codes, uint8_t* scales, uint16_t* out,
                 float* alpha, bool fq, hipStream_t stream, uint8_t* qstar = nullptr,
                 uint32_t* count4 = nullptr, double* stats = nullptr,
                 uint32_t* stats_ws = nullptr) {
  Shape s;
  nvfp4_status st = validate_main(in, E, rows, cols, block, mode, rule, amax_in, codes, scales,
                                  out, alpha, fq, &s);
  if (st != NVFP4_OK) return st;

  const bool diag = qstar != nullptr;
  if (diag) {
    if (!count4) return NVFP4_ERR_NULL;
    if (!aligned(count4, 4)) return NVFP4_ERR_ALIGN;
    const int64_t qb = s.E * s.nblk, in_bytes2 = s.E * s.n * 2;
    if (overlap(qstar, qb, in, in_bytes2) || overlap(qstar, qb, codes, s.E * s.n / 2) ||
        overlap(qstar, qb, scales, s.E * s.nblk) || overlap(qstar, qb, alpha, s.E * 4) ||
        overlap(qstar, qb, count4, s.E * 4) || overlap(count4, s.E * 4, in, in_bytes2) ||
        overlap(count4, s.E * 4, codes, s.E * s.n / 2) ||
        overlap(count4, s.E * 4, scales, s.E * s.nblk) || overlap(count4, s.E * 4, alpha, s.E * 4))
      return NVFP4_ERR_ALIAS;
    if (stats) {
      if (!aligned(stats, 8)) return NVFP4_ERR_ALIGN;
      const int64_t sb = s.E * NVFP4_NSTATS * 8;
      if (overlap(stats, sb, in, in_bytes2) || overlap(stats, sb, codes, s.E * s.n / 2) ||
          overlap(stats, sb, scales, s.E * s.nblk) || overlap(stats, sb, alpha, s.E * 4) ||
          overlap(stats, sb, qstar, qb) || overlap(stats, sb, count4, s.E * 4))
        return NVFP4_ERR_ALIAS;
      if (!stats_ws) return NVFP4_ERR_NULL;
      if (!aligned(stats_ws, 128)) return NVFP4_ERR_ALIGN;
      const int64_t wb = NVFP4_DIAG_WS_WORDS(s.E) * 4;
      if (overlap(stats_ws, wb, in, in_bytes2) || overlap(stats_ws, wb, codes, s.E * s.n / 2) ||
          overlap(stats_ws, wb, scales, s.E * s.nblk) || overlap(stats_ws, wb, alpha, s.E * 4) ||
          overlap(stats_ws, wb, qstar, qb) || overlap(stats_ws, wb, count4, s.E * 4) ||
          overlap(stats_ws, wb, stats, sb))
        return NVFP4_ERR_ALIAS;
    }
  }

  (void)hipGetLastError();   // clear a stale error so the status below is this call's
  const float* amax = amax_in;
  if (!amax) {
    if (launch_amax(in, s, reinterpret_cast<uint32_t*>(alpha), stream, count4,
                    reinterpret_cast<uint32_t*>(stats), stats ? s.E * NVFP4_NSTATS * 2 : 0,
                    stats ? stats_ws : nullptr, stats ? s.E * kDiagCtrWords : 0) != hipSuccess)
      return NVFP4_ERR_HIP;
    amax = alpha;
  }
  // With a separate amax buffer the quantize kernel writes alpha itself (one launch);
  // when alpha doubles as the amax accumulator a follow-up kernel converts it in place.
  float* alpha_in_kernel = amax == alpha ? nullptr : alpha;
  if (fq)
    launch_quantize<true, 0>(mode, rule, in, s, amax, nullptr, nullptr, out, alpha_in_kernel,
                                 nullptr, nullptr, nullptr, nullptr, stream);
  else if (diag && stats)
    launch_quantize<false, kDiagStats>(mode, rule, in, s, amax, codes, scales, nullptr,
                                       alpha_in_kernel, qstar, count4, stats, stats_ws, stream);
  else if (diag)
    launch_quantize<false, kDiagPlain>(mode, rule, in, s, amax, codes, scales, nullptr,
                                       alpha_in_kernel, qstar, count4, nullptr, nullptr, stream);
  else
    launch_quantize<false, 0>(mode, rule, in, s, amax, codes, scales, nullptr, alpha_in_kernel,
                                  nullptr, nullptr, nullptr, nullptr, stream);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  if (!alpha_in_kernel &&
      launch_alpha(reinterpret_cast<const uint32_t*>(amax), alpha, s, mode, stream) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

// ----------------------------------------------------------------------------- fused (host)
std::atomic<uint32_t> g_wait_polls{kFusedMaxWaitPolls};

// Ticks per microsecond of the device's constant-rate wall clock (the clock the waits read),
// cached per device; 100 (100 MHz) if the attribute is unavailable.
double wall_ticks_per_us() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100.0;
  int khz = cache[dev].load(std::memory_order_relaxed);
  if (khz == 0) {
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
      khz = 100000;
    cache[dev].store(khz, std::memory_order_relaxed);
  }
  return khz / 1000.0;
}

// Time bound of the waits of a fused launch in which `at_once` tensors are loaded together.
uint64_t fused_wait_ticks(const Shape& s, int64_t at_once) {
  const double us = kWaitFactor * (double)at_once * (double)s.n * 2.0 / kWaitLoadRate + kWaitFloorUs;
  return (uint64_t)(us * wall_ticks_per_us());
}

// Workgroups of one fused_kernel instance that fit on the current device at once (occupancy
// per CU times the CU count), cached per device; 0 if unknown.
template <int MODE, int RULE, bool FQ, int KR, int KL, bool TEAMS, int NT>
int64_t fused_resident_wgs() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v != 0) return v > 0 ? v : 0;
  int per_cu = 0, cus = 0;
  const bool ok =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&fused_kernel<MODE, RULE, FQ, KR, KL, TEAMS, NT>),
          NT,
          0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  v = ok ? (int64_t)per_cu * cus : 0;
  cache[dev].store(v > 0 ? v : -1, std::memory_order_relaxed);
  return v > 0 ? v : 0;
}

// Workgroups per tensor G and teams T for one tier: T = E when every tensor fits on chip at
// once (TEAMS false), else (TEAMS true) as many teams as are resident together, when at least
// one is; T = 0 when the tier does not fit.
//   - A tensor takes at most kFusedMaxTensorWGs workgroups: the collector form of the wait has
//     that many slots, and beyond it the 16 counter lines of the group form take more than 32
//     arrivals each.
//     Measured on an 8192x4096 tensor, 4/6-MSE packed: the 4-block tier with 2048 workgroups
//     48.5 us, the 28-block tier with 512 workgroups 34.4 us; rtn6 40.5 against 26.5 us.
//   - The 12- and 28-block tiers spread each tensor over resident / E workgroups (fewer blocks
//     per lane): 2-8 % faster on the tensors and batches measured.
//   - Teams are widened to fill every resident slot: a team holds one tensor with at least G
//     workgroups, and with T teams each gets resident / T (fewer blocks per lane).  Measured
//     against teams of exactly G: 18-20 % faster on batches of 524,288-block tensors (where 4
//     teams of 103 workgroups left 100 of 512 slots idle), 6-9 % on 262,144- and
//     1,048,576-block tensors.
template <int MODE, int RULE, bool FQ, int KR, int KL, bool TEAMS, int NT>
int64_t fused_tier_wgs(const Shape& s, int64_t* teams) {
  constexpr int64_t per_wg = (int64_t)(KR + KL) * NT;
  const int64_t G = (s.nblk + per_wg - 1) / per_wg;
  const int64_t resident = fused_resident_wgs<MODE, RULE, FQ, KR, KL, TEAMS, NT>();
  if (!TEAMS) {
    *teams = (G * s.E <= resident && G <= kFusedMaxTensorWGs) ? s.E : 0;
    return (KR + KL >= 12 || NT > kThreads) && *teams > 0
               ? std::min(kFusedMaxTensorWGs, std::max(G, resident / s.E)) : G;
  }
  // Teams of the kTeamKR + kTeamKL tier round their size up to a power of two when that still
  // fits four teams and adds at most a quarter: then the two workgroups that share a CU (i and
  // i + #CUs) belong to teams y and y + T/2, started in the same phase.  Same-box A/B, us per
  // call (team size as computed / as rounded): 16x1024x4096 (52 / 64) rtn6 50.1 / 46.3,
  // 4/6-MAE fake-quant 75.1 / 66.7, rtn6 fake-quant 68.0 / 61.2; 96x1024x4096 rtn6 235 / 228.
  // Rounded without the quarter bound, teams of 74 and 90 measured up to 3 % slower (rtn6,
  // 32x1472x4096 and 32x1800x4096); with only two teams (154 / 256: 6x3072x4096, 24x3072x4096,
  // 40x2048x6144) up to 13 % slower.  The small-tensor tier keeps its sizes: rounded, rtn6 and
  // 4/6 teams of 128x1024x1024, 256x256x1024 and 32x512x4096 measured 2-12 % slower.
  if constexpr (KR == kTeamKR && KL == kTeamKL) {
    int64_t Gp = 1;
    while (Gp < G) Gp <<= 1;
    if (4 * Gp <= resident && 4 * Gp <= 5 * G) {
      *teams = std::min(s.E, resident / Gp);
      return Gp;
    }
  }
  const int64_t T = G <= kFusedMaxTensorWGs ? std::min(s.E, resident / G) : 0;
  *teams = T;
  return T > 0 ? std::min(kFusedMaxTensorWGs, std::max(G, resident / T)) : G;
}

template <int MODE, int RULE, bool FQ, int KR, int KL, bool TEAMS, int NT>
void fused_launch(int64_t G, int64_t T, const uint16_t* in, const Shape& s, uint32_t* ws,
                  uint8_t* codes, uint8_t* scales, uint16_t* out, float* alpha,
                  hipStream_t stream) {
  const int64_t words = s.E * kFusedWsWords;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((words + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, ws, nullptr, words, nullptr, (int64_t)0, nullptr,
                     (int64_t)0);
  hipLaunchKernelGGL((fused_kernel<MODE, RULE, FQ, KR, KL, TEAMS, NT>), dim3((unsigned)G, (unsigned)T),
                     dim3(NT), 0, stream, reinterpret_cast<const uint4*>(in), s.nblk, ws,
                     reinterpret_cast<uint2*>(codes), scales, reinterpret_cast<uint4*>(out), alpha,
                     g_wait_polls.load(std::memory_order_relaxed), fused_wait_ticks(s, T),
                     s.E);
}

// Four Over Six teams in 512-thread workgroups, KR + KL blocks per lane (the KL in LDS, loaded
// straight into it), in teams of a power-of-two number of workgroups: then the two workgroups
// that share a CU (i and i + #CUs) belong to teams y and y + T/2, and every CU holds the same
// pair of teams.  Taken when at least four such teams fit; returns whether it was (and
// launches when asked).
template <int MODE, int RULE, bool FQ, int KR, int KL>
bool fused_team512(bool launch, const uint16_t* in, const Shape& s, uint32_t* ws,
                   uint8_t* codes, uint8_t* scales, float* alpha, hipStream_t stream) {
  constexpr int64_t per_wg = (int64_t)(KR + KL) * 512;
  const int64_t G = (s.nblk + per_wg - 1) / per_wg;
  int64_t Gp = 1;
  while (Gp < G) Gp <<= 1;
  const int64_t resident = fused_resident_wgs<MODE, RULE, FQ, KR, KL, true, 512>();
  const int64_t T = std::min(s.E, resident / Gp);
  if (resident < 4 * Gp || T < 4) return false;
  if (launch)
    fused_launch<MODE, RULE, FQ, KR, KL, true, 512>(Gp, T, in, s, ws, codes, scales, nullptr,
                                                    alpha, stream);
  return true;
}

// Tiers of blocks held per lane, (KR in VGPRs, KL in LDS) in workgroups of NT threads, tried in
// this order: (1,0) and (4,0) at 256; (10,0) at 1024 (4 waves per SIMD, see kTeamWideKR; up
// to 2,621,440 blocks in all); (12,0) at 256; (10,4) at 1024 (3,670,016 blocks); (20,8) at 256
// (as many, at two waves per SIMD; Four Over Six fake-quant, which does not fit (10,4) in 128
// VGPRs).  The first tier that holds every tensor at once runs (more workgroups for smaller
// tensors).  Same-box A/B of the (10,0) tier against the tier that held the tensor before it:
// an 8192x4096 tensor (against (20,8)): 4/6-MSE packed 28.4 against 33.4 us (then routed to
// two passes), rtn6 packed 21.8 against 25.6, 4/6-MAE fake-quant 32.0 against 35.2, rtn6
// fake-quant 31.0 against 33.6; 4096x4112 and 2048x8192 (against (12,0)): 4/6-MSE packed 19.4
// / 18.0 against 20.8 / 20.2 us, rtn6 packed 15.0 / 14.4 against 19.0 / 18.4, 4/6-MAE
// fake-quant 21.9 / 19.9 against 23.3 / 22.5, rtn6 fake-quant 21.5 / 20.3 against 25.2 / 24.2;
// two 4096x4096 tensors equal.  Before (4,0) it measured equal or up to 6 % slower on tensors
// of 0.26 M blocks and less.  (12,0) is left for batches of many mid-size tensors whose
// workgroups the 1024-thread tier cannot all place.  A batch that no tier holds at once runs in
// teams (kTeamSmallKR + 0, kTeamWideKR + 0 or kTeamKR + kTeamKL per lane) when one tensor
// fits: teams at different tensors overlap loads with arithmetic.  Returns the blocks held per
// lane (1, 4, 10, 12, 14 or 28, or 10 / 13 / 20 for teams), or 0 for the two-pass path, when
// not even one tensor fits.
template <int MODE, int RULE, bool FQ>
int fused_try(bool launch, const uint16_t* in, const Shape& s, uint32_t* ws, uint8_t* codes,
               uint8_t* scales, uint16_t* out, float* alpha, hipStream_t stream) {
  if (s.nblk > kMaxLaunchBlocks) return 0;
  int64_t G, T;
#define NVFP4_FUSED_TIER(KR, KL, TEAMS, NT)                                                     \
  G = fused_tier_wgs<MODE, RULE, FQ, KR, KL, TEAMS, NT>(s, &T);                               \
  if (T > 0) {                                                                                \
    if (launch)                                                                               \
      fused_launch<MODE, RULE, FQ, KR, KL, TEAMS, NT>(G, T, in, s, ws, codes, scales, out,      \
                                                      alpha, stream);                         \
    return KR + KL;                                                                           \
  }
  NVFP4_FUSED_TIER(1, 0, false, kThreads)
  NVFP4_FUSED_TIER(4, 0, false, kThreads)
  NVFP4_FUSED_TIER(kTeamWideKR, 0, false, 1024)
  NVFP4_FUSED_TIER(12, 0, false, kThreads)
  // 10 in VGPRs and 4 in LDS in 1024-thread workgroups (one per CU, 3,670,016 blocks in all: the
  // 4096x14336 weight), before (20,8), which holds as many at two waves per SIMD.  Same-box A/B
  // on the weight: 4/6-MSE packed 44.6 against 50.7 us (then routed to two passes: (20,8) read
  // once was no faster than two passes, 50.2 against 50.5 us), rtn6 packed 33.1 against 38.6,
  // rtn6 fake-quant 53.2 against 55.8; three 4096x4096 tensors 4/6 packed 39.9 against 40.7.
  // Four Over Six fake-quant needs more than 128 VGPRs here and keeps (20,8).
  if constexpr (!(MODE == NVFP4_FOUR_OVER_SIX && FQ)) {
    NVFP4_FUSED_TIER(kTeamWideKR, 4, false, 1024)
  }
  NVFP4_FUSED_TIER(20, 8, false, kThreads)
  if (s.nblk < kTeamSmallBlocks) {
    NVFP4_FUSED_TIER(kTeamSmallKR, 0, true, kThreads)
  }
  if constexpr (MODE == NVFP4_FOUR_OVER_SIX && !FQ) {
    // wide workgroups: 512 threads in aligned teams of 10 or 9 + 4 per lane, else 1024
    if (fused_team512<MODE, RULE, FQ, kTeamWideKR, 0>(launch, in, s, ws, codes, scales, alpha,
                                                      stream))
      return kTeamWideKR;
    if (fused_team512<MODE, RULE, FQ, kTeamWideKR - 1, 4>(launch, in, s, ws, codes, scales,
                                                          alpha, stream))
      return kTeamWideKR + 3;
    NVFP4_FUSED_TIER(kTeamWideKR, 0, true, 1024)
  }
  NVFP4_FUSED_TIER(kTeamKR, kTeamKL, true, kThreads)
#undef NVFP4_FUSED_TIER
  return 0;
}

template <bool FQ>
int fused_dispatch(bool launch, int mode, int rule, const uint16_t* in, const Shape& s,
                    uint32_t* ws, uint8_t* codes, uint8_t* scales, uint16_t* out, float* alpha,
                    hipStream_t stream) {
  if (mode == NVFP4_RTN6)
    return fused_try<NVFP4_RTN6, NVFP4_RULE_MSE, FQ>(launch, in, s, ws, codes, scales, out, alpha,
                                                     stream);
  if (rule == NVFP4_RULE_MSE)
    return fused_try<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE, FQ>(launch, in, s, ws, codes, scales,
                                                              out, alpha, stream);
  if (rule == NVFP4_RULE_MAE)
    return fused_try<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAE, FQ>(launch, in, s, ws, codes, scales,
                                                              out, alpha, stream);
  return fused_try<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAXERR, FQ>(launch, in, s, ws, codes, scales,
                                                               out, alpha, stream);
}

nvfp4_status run_fused(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int block,
                       int mode, int rule, uint8_t* codes, uint8_t* scales, uint16_t* out,
                       float* alpha, uint32_t* ws, bool fq, hipStream_t stream) {
  Shape s;
  nvfp4_status st = validate_main(in, E, rows, cols, block, mode, rule, nullptr, codes, scales,
                                  out, alpha, fq, &s);
  if (st != NVFP4_OK) return st;
  if (!ws) return NVFP4_ERR_NULL;
  if (!aligned(ws, 128)) return NVFP4_ERR_ALIGN;
  const int64_t wb = s.E * kFusedWsWords * 4, in_bytes = s.E * s.n * 2;
  if (overlap(ws, wb, in, in_bytes) || overlap(ws, wb, alpha, s.E * 4) ||
      (fq ? overlap(ws, wb, out, in_bytes)
          : (overlap(ws, wb, codes, s.E * s.n / 2) || overlap(ws, wb, scales, s.E * s.nblk))))
    return NVFP4_ERR_ALIAS;
  (void)hipGetLastError();
  // In-place fake-quant takes the two-pass path: a workgroup that stops waiting re-reads the
  // whole input, which other workgroups may already be overwriting.
  const int fused = fq && out == in ? 0
                  : fq ? fused_dispatch<true>(true, mode, rule, in, s, ws, nullptr, nullptr,
                                               out, alpha, stream)
                        : fused_dispatch<false>(true, mode, rule, in, s, ws, codes, scales,
                                                nullptr, alpha, stream);
  if (!fused)   // too large to hold on chip: the two-pass path (the workspace is not used)
    return run(in, E, rows, cols, block, mode, rule, nullptr, codes, scales, out, alpha, fq,
               stream);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace

// ----------------------------------------------------------------------------- static scratch
// The allocation-free single-read call keeps the grid-wide wait's words here instead of
// in a caller workspace: up to kScratchTensors tensors of NVFP4_FUSED_WS_WORDS words (2176
// bytes each, 2.1 MiB in all).  Each GPU the library runs on holds its own copy until the
// process ends.  In host code the array's name is only a stand-in: its device address on a
// device is taken once with hipGetSymbolAddress, with that device current, and that address
// is what the kernels get.  Every call on a GPU shares the array, so calls that may overlap on
// one GPU (different streams, graph branches) race; the launch clears what it uses first.
constexpr int64_t kScratchTensors = NVFP4_NOALLOC_MAX_TENSORS;
static __device__ __align__(256) uint32_t scratch[kScratchTensors * kFusedWsWords];

namespace {

std::atomic<uintptr_t> g_scratch_ptr[64];   // device address of `scratch` per device, 0 = not yet

nvfp4_status scratch_on_current_device(uint32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return NVFP4_ERR_HIP;
  uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return NVFP4_ERR_HIP;
    p = reinterpret_cast<uintptr_t>(ptr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = reinterpret_cast<uint32_t*>(p);
  return NVFP4_OK;
}

}  // namespace

// ----------------------------------------------------------------------------- C ABI
NVFP4_EXPORT int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

NVFP4_EXPORT const char* nvfp4_status_str(nvfp4_status st) {
  switch (st) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer argument";
    case NVFP4_ERR_SHAPE: return "bad shape (E, rows, cols > 0; cols % 16 == 0; E <= 65535)";
    case NVFP4_ERR_BLOCK: return "block size must be 16";
    case NVFP4_ERR_ENUM: return "mode or rule out of range";
    case NVFP4_ERR_ALIGN: return "misaligned pointer (16 B for tensors and codes, 4 B for alpha/amax)";
    case NVFP4_ERR_ALIAS: return "overlapping arguments";
    case NVFP4_ERR_HIP: return "HIP kernel launch failed";
    case NVFP4_ERR_SCRATCH:
      return "batch too large for the static scratch of the allocation-free call (E > 1024)";
  }
  return "unknown status";
}

NVFP4_EXPORT nvfp4_status nvfp4_amax(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                                     float* out_amax, hipStream_t stream) {
  Shape s;
  nvfp4_status st = check_shape(E, rows, cols, &s);
  if (st != NVFP4_OK) return st;
  if (!in || !out_amax) return NVFP4_ERR_NULL;
  if (!aligned(in, 16) || !aligned(out_amax, 4)) return NVFP4_ERR_ALIGN;
  if (overlap(out_amax, s.E * 4, in, s.E * s.n * 2)) return NVFP4_ERR_ALIAS;
  (void)hipGetLastError();
  return launch_amax(in, s, reinterpret_cast<uint32_t*>(out_amax), stream) == hipSuccess
             ? NVFP4_OK : NVFP4_ERR_HIP;
}

NVFP4_EXPORT nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                                           const float* alpha, int64_t E, int64_t rows,
                                           int64_t cols, uint16_t* out, hipStream_t stream) {
  Shape s;
  nvfp4_status st = check_shape(E, rows, cols, &s);
  if (st != NVFP4_OK) return st;
  if (!codes || !scales || !alpha || !out) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8) || !aligned(alpha, 4) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  const int64_t out_bytes = s.E * s.n * 2;
  if (overlap(out, out_bytes, codes, s.E * s.n / 2) || overlap(out, out_bytes, scales, s.E * s.nblk) ||
      overlap(out, out_bytes, alpha, s.E * 4))
    return NVFP4_ERR_ALIAS;
  (void)hipGetLastError();
  auto launch = [&](int64_t E2, int64_t nblk, int64_t first_tensor, int64_t first_block) {
    // one block per lane (measured 12-30 % faster than 1024 workgroups striding the tensor)
    const int64_t per_tensor = std::max<int64_t>(1, (nblk + kThreads - 1) / kThreads);
    const int64_t b0 = first_tensor * s.nblk + first_block;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)per_tensor, (unsigned)E2), dim3(kThreads), 0,
                       stream, reinterpret_cast<const uint2*>(codes + b0 * 8), scales + b0,
                       alpha + first_tensor, nblk, reinterpret_cast<uint4*>(out + b0 * 16));
  };
  if (s.nblk <= kMaxLaunchBlocks) {
    launch(s.E, s.nblk, 0, 0);
  } else {                  // tensors of 2^27 blocks or more: one launch per tensor and chunk
    for (int64_t t = 0; t < s.E; ++t)
      for (int64_t b = 0; b < s.nblk; b += kMaxLaunchBlocks)
        launch(1, std::min(kMaxLaunchBlocks, s.nblk - b), t, b);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize(const uint16_t* in, int64_t rows, int64_t cols, int block,
                                         nvfp4_mode mode, nvfp4_rule rule, uint8_t* out_codes,
                                         uint8_t* out_scales, float* out_alpha, hipStream_t stream) {
  return run(in, 1, rows, cols, block, mode, rule, nullptr, out_codes, out_scales, nullptr,
             out_alpha, false, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_fakequant(const uint16_t* in, int64_t rows, int64_t cols, int block,
                                          nvfp4_mode mode, nvfp4_rule rule, uint16_t* out,
                                          float* out_alpha, hipStream_t stream) {
  return run(in, 1, rows, cols, block, mode, rule, nullptr, nullptr, nullptr, out, out_alpha,
             true, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_batched(const uint16_t* in, int64_t E, int64_t rows,
                                                 int64_t cols, int block, nvfp4_mode mode,
                                                 nvfp4_rule rule, uint8_t* out_codes,
                                                 uint8_t* out_scales, float* out_alpha,
                                                 hipStream_t stream) {
  return run(in, E, rows, cols, block, mode, rule, nullptr, out_codes, out_scales, nullptr,
             out_alpha, false, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_fakequant_batched(const uint16_t* in, int64_t E, int64_t rows,
                                                  int64_t cols, int block, nvfp4_mode mode,
                                                  nvfp4_rule rule, uint16_t* out,
                                                  float* out_alpha, hipStream_t stream) {
  return run(in, E, rows, cols, block, mode, rule, nullptr, nullptr, nullptr, out, out_alpha,
             true, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_diag(const uint16_t* in, int64_t E, int64_t rows,
                                              int64_t cols, int block, nvfp4_mode mode,
                                              nvfp4_rule rule, uint8_t* out_codes,
                                              uint8_t* out_scales, float* out_alpha,
                                              uint8_t* out_qstar, uint32_t* out_count4,
                                              double* out_stats, uint32_t* stats_workspace,
                                              hipStream_t stream) {
  if (!out_qstar || !out_count4) return NVFP4_ERR_NULL;
  return run(in, E, rows, cols, block, mode, rule, nullptr, out_codes, out_scales, nullptr,
             out_alpha, false, stream, out_qstar, out_count4, out_stats, stats_workspace);
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_from_amax(const uint16_t* in, int64_t E, int64_t rows,
                                                   int64_t cols, int block, nvfp4_mode mode,
                                                   nvfp4_rule rule, const float* amax,
                                                   uint8_t* out_codes, uint8_t* out_scales,
                                                   float* out_alpha, hipStream_t stream) {
  if (!amax) return NVFP4_ERR_NULL;
  return run(in, E, rows, cols, block, mode, rule, amax, out_codes, out_scales, nullptr,
             out_alpha, false, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_fakequant_from_amax(const uint16_t* in, int64_t E, int64_t rows,
                                                    int64_t cols, int block, nvfp4_mode mode,
                                                    nvfp4_rule rule, const float* amax,
                                                    uint16_t* out, float* out_alpha,
                                                    hipStream_t stream) {
  if (!amax) return NVFP4_ERR_NULL;
  return run(in, E, rows, cols, block, mode, rule, amax, nullptr, nullptr, out, out_alpha, true,
             stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_fused(const uint16_t* in, int64_t E, int64_t rows,
                                               int64_t cols, int block, nvfp4_mode mode,
                                               nvfp4_rule rule, uint8_t* out_codes,
                                               uint8_t* out_scales, float* out_alpha,
                                               uint32_t* workspace, hipStream_t stream) {
  return run_fused(in, E, rows, cols, block, mode, rule, out_codes, out_scales, nullptr,
                   out_alpha, workspace, false, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_fakequant_fused(const uint16_t* in, int64_t E, int64_t rows,
                                                int64_t cols, int block, nvfp4_mode mode,
                                                nvfp4_rule rule, uint16_t* out, float* out_alpha,
                                                uint32_t* workspace, hipStream_t stream) {
  return run_fused(in, E, rows, cols, block, mode, rule, nullptr, nullptr, out, out_alpha,
                   workspace, true, stream);
}

NVFP4_EXPORT nvfp4_status nvfp4_quantize_fused_noalloc(const uint16_t* in, int64_t E,
                                                       int64_t rows, int64_t cols, int block,
                                                       nvfp4_mode mode, nvfp4_rule rule,
                                                       uint8_t* out_codes, uint8_t* out_scales,
                                                       float* out_alpha, hipStream_t stream) {
  Shape s;
  const nvfp4_status st = validate_main(in, E, rows, cols, block, mode, rule, nullptr,
                                        out_codes, out_scales, nullptr, out_alpha, false, &s);
  if (st != NVFP4_OK) return st;
  if (s.E > kScratchTensors) return NVFP4_ERR_SCRATCH;
  uint32_t* ws = nullptr;
  const nvfp4_status sst = scratch_on_current_device(&ws);
  if (sst != NVFP4_OK) return sst;
  return run_fused(in, E, rows, cols, block, mode, rule, out_codes, out_scales, nullptr,
                   out_alpha, ws, false, stream);
}

NVFP4_EXPORT int nvfp4_fused_single_read(int64_t E, int64_t rows, int64_t cols,
                                         nvfp4_mode mode, nvfp4_rule rule, int fakequant) {
  Shape s;
  nvfp4_status st = check_shape(E, rows, cols, &s);
  if (st != NVFP4_OK) return -(int)st;
  if ((mode != NVFP4_RTN6 && mode != NVFP4_FOUR_OVER_SIX) ||
      (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAXERR))
    return -(int)NVFP4_ERR_ENUM;
  return fakequant ? fused_dispatch<true>(false, mode, rule, nullptr, s, nullptr, nullptr, nullptr,
                                          nullptr, nullptr, nullptr)
                   : fused_dispatch<false>(false, mode, rule, nullptr, s, nullptr, nullptr,
                                           nullptr, nullptr, nullptr, nullptr);
}

NVFP4_EXPORT void nvfp4_fused_set_wait_limit(int64_t polls) {
  g_wait_polls.store(polls < 0 ? kFusedMaxWaitPolls
                               : (uint32_t)std::min<int64_t>(polls, kFusedMaxWaitPolls),
                     std::memory_order_relaxed);
}
