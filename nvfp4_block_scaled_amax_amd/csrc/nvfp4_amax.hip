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
//                    rounding, the error reduction and the selection stay in VGPRs; codes,
//                    scale bytes (or bf16 fake-quant values) are written with vector stores
//   alpha_kernel     alpha[e] <- amax[e] / (6*M) once every block is done
//
// All floating-point steps are IEEE binary32 with round-to-nearest-even, no contraction
// (-ffp-contract=off) and no denormal flushing; fp32 division and reciprocal are the
// correctly rounded HIP defaults.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

// binary32 (finite) -> bfloat16 bits, round to nearest even.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ----------------------------------------------------------------------------- kernels
__global__ void clear_kernel(uint32_t* __restrict__ acc, int64_t E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) acc[i] = 0u;
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

// Grid: x = workgroups per tensor, y = tensor.  Each workgroup strides over the tensor's
// 16-byte chunks (8 bf16 values), four loads in flight per lane.
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ in,
                                                        int64_t chunks, uint32_t* __restrict__ acc) {
  const uint4* p = in + (int64_t)blockIdx.y * chunks;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  for (; i + 3 * stride < chunks; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    m = mag_max8(m, a);
    m = mag_max8(m, b);
    m = mag_max8(m, c);
    m = mag_max8(m, d);
  }
  for (; i < chunks; i += stride) m = mag_max8(m, p[i]);
  // the larger of the two 16-bit magnitudes, as the bits of a binary32 value
  m = max(m & 0xFFFFu, m >> 16) << 16;
  m = wave_max_u32(m);
  __shared__ uint32_t part[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (int w = 1; w < kThreads / 64; ++w) r = max(r, part[w]);
    atomicMax(acc + blockIdx.y, r);
  }
}

__global__ void alpha_kernel(const uint32_t* amax_bits, float* alpha,
                             int64_t E, float C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E) return;
  const uint32_t a = amax_bits[i] & 0x7FFFFFFFu;
  alpha[i] = a >= 0x7F800000u ? __uint_as_float(0x7FC00000u) : __uint_as_float(a) / C;
}

// One candidate block maximum (Q = 6, or 4 under Four Over Six), all in registers.
// Returns the error under RULE; writes the scale byte, the 16 codes as two packed words
// and (FQ) the 16 dequantized values.
template <int RULE, bool FQ>
__device__ __forceinline__ float run_candidate(const float (&x)[16], float bmax, float alpha,
                                               float cq, uint32_t cap, uint32_t& scale,
                                               uint32_t& w0, uint32_t& w1, float (&xh)[16]) {
  const float sigma = alpha == 0.0f ? 0.0f : bmax / cq;
  scale = e4m3_from_f32(sigma);
  const float d = e4m3_to_f32(scale) * alpha;
  const float r = d == 0.0f ? 0.0f : 1.0f / d;
  const bool r_finite = r != __builtin_inff();
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = x[i] * r;
  if (!r_finite) {                 // 1/d overflows: only when alpha is a binary32 subnormal
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x[i] / d;
  }
  float acc = 0.0f;
  w0 = 0u;
  w1 = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = min(e2m1_code_of(fabsf(v[i])), cap);
    const uint32_t sgn = __float_as_uint(x[i]) & 0x80000000u;
    const float xhat = __uint_as_float(__float_as_uint(e2m1_value_of(m) * d) | sgn);
    const float e = x[i] - xhat;
    if (RULE == NVFP4_RULE_MSE)      acc = __builtin_fmaf(e, e, acc);
    else if (RULE == NVFP4_RULE_MAE) acc = acc + fabsf(e);
    else                             acc = fmaxf(acc, fabsf(e));
    const uint32_t code = (sgn >> 28) | m;
    if (i < 8) w0 |= code << (4 * i);
    else       w1 |= code << (4 * (i - 8));
    if (FQ) xh[i] = xhat;
  }
  return acc;
}

// Grid: x = ceil(blocks per tensor / 256), y = tensor.  Lane = one 16-element block.
template <int MODE, int RULE, bool FQ>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint4* __restrict__ in, int64_t nblk, const float* __restrict__ amax,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales, uint4* __restrict__ out,
    float* __restrict__ alpha_out) {
  const int64_t t = blockIdx.y;
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint32_t abits = __float_as_uint(amax[t]) & 0x7FFFFFFFu;
  // alpha_out (distinct from amax) is written by the first lane of each tensor
  if (alpha_out && b == 0)
    alpha_out[t] = abits >= 0x7F800000u ? __uint_as_float(0x7FC00000u)
                   : __uint_as_float(abits) / (MODE == NVFP4_FOUR_OVER_SIX ? kC6x256 : kC6x448);
  if (b >= nblk) return;
  const int64_t g = t * nblk + b;
  if (abits >= 0x7F800000u) {      // non-finite input or amax: poison the tensor
    if (FQ) {
      const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
      out[2 * g] = nan4;
      out[2 * g + 1] = nan4;
    } else {
      codes[g] = make_uint2(0u, 0u);
      scales[g] = 0x7F;
    }
    return;
  }
  const float alpha = __uint_as_float(abits) / (MODE == NVFP4_FOUR_OVER_SIX ? kC6x256 : kC6x448);
  const uint4 p0 = in[2 * g], p1 = in[2 * g + 1];
  const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16_lo(w[k]);
    x[2 * k + 1] = bf16_hi(w[k]);
  }
  float bmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(x[i]));

  float xh6[16], xh4[16];
  uint32_t s6, a6, b6;
  const float err6 = run_candidate<RULE, FQ>(x, bmax, alpha, 6.0f * alpha, 7u, s6, a6, b6, xh6);
  uint32_t s = s6, c0 = a6, c1 = b6;
  bool four = false;
  if (MODE == NVFP4_FOUR_OVER_SIX) {
    uint32_t s4, a4, b4;
    const float err4 = run_candidate<RULE, FQ>(x, bmax, alpha, 4.0f * alpha, 6u, s4, a4, b4, xh4);
    four = err4 < err6;            // ties keep 6
    if (four) { s = s4; c0 = a4; c1 = b4; }
  }
  if (FQ) {
    uint32_t y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float lo = four ? xh4[2 * k] : xh6[2 * k];
      const float hi = four ? xh4[2 * k + 1] : xh6[2 * k + 1];
      y[k] = bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
    }
    out[2 * g] = make_uint4(y[0], y[1], y[2], y[3]);
    out[2 * g + 1] = make_uint4(y[4], y[5], y[6], y[7]);
  } else {
    codes[g] = make_uint2(c0, c1);
    scales[g] = (uint8_t)s;
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

hipError_t launch_amax(const uint16_t* in, const Shape& s, uint32_t* acc, hipStream_t stream) {
  const int64_t chunks = s.n / 8;
  const int64_t want = (chunks + kThreads * 4 - 1) / (kThreads * 4);
  const int64_t per_tensor = std::max<int64_t>(1, std::min<int64_t>(want, 4096 / s.E + 1));
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((s.E + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, acc, s.E);
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)per_tensor, (unsigned)s.E), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(in), chunks, acc);
  return hipGetLastError();
}

template <int MODE, int RULE, bool FQ>
void launch_quantize_t(const uint16_t* in, const Shape& s, const float* amax, uint8_t* codes,
                       uint8_t* scales, uint16_t* out, float* alpha_out, hipStream_t stream) {
  const dim3 grid((unsigned)((s.nblk + kThreads - 1) / kThreads), (unsigned)s.E);
  hipLaunchKernelGGL((quantize_kernel<MODE, RULE, FQ>), grid, dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(in), s.nblk, amax,
                     reinterpret_cast<uint2*>(codes), scales, reinterpret_cast<uint4*>(out),
                     alpha_out);
}

template <bool FQ>
void launch_quantize(int mode, int rule, const uint16_t* in, const Shape& s, const float* amax,
                     uint8_t* codes, uint8_t* scales, uint16_t* out, float* alpha_out,
                     hipStream_t stream) {
  if (mode == NVFP4_RTN6) {
    launch_quantize_t<NVFP4_RTN6, NVFP4_RULE_MSE, FQ>(in, s, amax, codes, scales, out, alpha_out, stream);
  } else if (rule == NVFP4_RULE_MSE) {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE, FQ>(in, s, amax, codes, scales, out, alpha_out, stream);
  } else if (rule == NVFP4_RULE_MAE) {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAE, FQ>(in, s, amax, codes, scales, out, alpha_out, stream);
  } else {
    launch_quantize_t<NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAXERR, FQ>(in, s, amax, codes, scales, out, alpha_out, stream);
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
nvfp4_status run(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int block, int mode,
                 int rule, const float* amax_in, uint8_t* codes, uint8_t* scales, uint16_t* out,
                 float* alpha, bool fq, hipStream_t stream) {
  Shape s;
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

  (void)hipGetLastError();   // clear a stale error so the status below is this call's
  const float* amax = amax_in;
  if (!amax) {
    if (launch_amax(in, s, reinterpret_cast<uint32_t*>(alpha), stream) != hipSuccess)
      return NVFP4_ERR_HIP;
    amax = alpha;
  }
  // With a separate amax buffer the quantize kernel writes alpha itself (one launch);
  // when alpha doubles as the amax accumulator a follow-up kernel converts it in place.
  float* alpha_in_kernel = amax == alpha ? nullptr : alpha;
  if (fq) launch_quantize<true>(mode, rule, in, s, amax, nullptr, nullptr, out, alpha_in_kernel, stream);
  else    launch_quantize<false>(mode, rule, in, s, amax, codes, scales, nullptr, alpha_in_kernel, stream);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  if (!alpha_in_kernel &&
      launch_alpha(reinterpret_cast<const uint32_t*>(amax), alpha, s, mode, stream) != hipSuccess)
    return NVFP4_ERR_HIP;
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
