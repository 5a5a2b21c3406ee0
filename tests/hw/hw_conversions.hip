// Exhaustive check of the gfx950 conversion instructions that the block pass relies on,
// against their definitions written out in plain integer and float code:
//   - v_cvt_scalef32_pk_fp4_f32 (scale 1): E2M1 round to nearest, ties to the even code,
//     saturating at 6, sign kept; every byte position of the packed word;
//   - v_cvt_scalef32_pk_f32_fp4 (scale 1): the 16 E2M1 codes to their values;
//   - v_cvt_pk_fp8_f32 after a clamp at 448: E4M3 (FN) round to nearest even, subnormals kept;
//   - v_cvt_pk_fp8_f32 without a clamp, above 448 (up to +inf): byte 0x7E or 0x7F in both
//     positions, which is all the Four Over Six scale pair relies on there;
//   - v_cvt_pk_bf16_f32: bf16 round to nearest even.
// Every binary32 bit pattern is tried (NaN inputs excepted; non-negative ones for E4M3, which
// the block pass only feeds non-negative scales).  Test infrastructure: built beside the tests
// and called from tests/test_gpu_hw_conversions.py; it shares no code with the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct Result {
  unsigned long long count;   // mismatches
  unsigned long long checked; // inputs compared
  uint32_t in, hw, sw;        // the first mismatch
};

// One atomic per lane for the number of inputs it compared.
__device__ void tally(Result* r, unsigned long long n) { atomicAdd(&r->checked, n); }

__device__ void record(Result* r, uint32_t in, uint32_t hw, uint32_t sw) {
  if (atomicAdd(&r->count, 1ull) == 0ull) {
    r->in = in;
    r->hw = hw;
    r->sw = sw;
  }
}

// E2M1 magnitude code of a >= 0: the number of rounding thresholds a reaches.  The
// thresholds are the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 of the grid
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}; at a midpoint the even code wins, so a midpoint whose lower
// neighbour has an even code must be passed strictly.
__device__ uint32_t e2m1_code(float a) {
  const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t c = 0;
  for (int k = 0; k < 7; ++k) c += (k % 2 == 0) ? (a > mid[k]) : (a >= mid[k]);
  return c;
}

// E4M3 (FN) byte of s in [0, 448]: below 2^-6 the grid is k * 2^-9; above, 3 mantissa bits.
__device__ uint32_t e4m3_byte(float s) {
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  int e = 0;
  const float m = frexpf(s, &e);                   // s = m * 2^e, m in [0.5, 1)
  float q = __builtin_rintf(m * 16.0f);            // 1.xxx with 3 fraction bits, times 8
  if (q == 16.0f) { q = 8.0f; ++e; }               // rounded up to the next binade
  return (uint32_t)((e + 6) << 3) | ((uint32_t)q - 8u);
}

// bf16 bits of f (finite): keep the top 16 bits, rounding the low 16 to nearest, ties to even.
__device__ uint32_t bf16_bits(uint32_t u) {
  const uint32_t low = u & 0xFFFFu, top = u >> 16;
  return top + ((low > 0x8000u || (low == 0x8000u && (top & 1u))) ? 1u : 0u);
}

__global__ void fp4_encode_all(uint64_t lo, uint64_t hi, Result* r) {
  unsigned long long n = 0;
  for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t u = (uint32_t)i;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) continue;   // NaN
    const float f = __uint_as_float(u);
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f, -f, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, -f, f, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f, f, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, -f, -f, 1.0f, 3);
    const uint32_t m = e2m1_code(fabsf(f));
    const uint32_t s = u >> 31;
    const uint32_t pos = (s << 3) | m, neg = ((s ^ 1u) << 3) | m;
    const uint32_t want = (pos | neg << 4) | (neg | pos << 4) << 8 | (pos | pos << 4) << 16 |
                          (neg | neg << 4) << 24;
    if (w != want) record(r, u, w, want);
    ++n;
  }
  tally(r, n);
}

__global__ void fp4_decode_all(Result* r) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const float val[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const uint32_t b = threadIdx.x;                  // one byte = two codes
  if (b >= 256) return;
  // byte k of the word is b ^ (0x11 * k), so each byte position decodes different codes
  const uint32_t w = b | (b ^ 0x11u) << 8 | (b ^ 0x22u) << 16 | (b ^ 0x33u) << 24;
  const f2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0),
                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1),
                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2),
                   __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)};
  for (int k = 0; k < 4; ++k)
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = ((b ^ (0x11u * k)) >> (4 * h)) & 15u;
      const float want = (c & 8u) ? -val[c & 7u] : val[c & 7u];
      const float got = h ? v[k].y : v[k].x;
      if (__float_as_uint(got) != __float_as_uint(want))
        record(r, c | (uint32_t)k << 8, __float_as_uint(got), __float_as_uint(want));
    }
  tally(r, 8);
}

__global__ void fp8_encode_all(uint64_t lo, uint64_t hi, Result* r) {
  unsigned long long n = 0;
  for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t u = (uint32_t)i;                // non-negative, up to +inf
    const float s = fminf(__uint_as_float(u), 448.0f);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false);
    const uint32_t b = e4m3_byte(s);
    if (hw != (b | b << 8)) record(r, u, hw, b | b << 8);
    ++n;
  }
  tally(r, n);
}

__global__ void fp8_encode_over(uint64_t lo, uint64_t hi, Result* r) {
  unsigned long long n = 0;
  for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t u = (uint32_t)i;                // above 448, up to +inf
    const float s = __uint_as_float(u);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false) & 0xFFFFu;
    const uint32_t b0 = hw & 0xFFu, b1 = hw >> 8;
    if (b0 < 0x7Eu || b0 > 0x7Fu || b1 < 0x7Eu || b1 > 0x7Fu) record(r, u, hw, 0x7E7Eu);
    ++n;
  }
  tally(r, n);
}

__global__ void bf16_encode_all(uint64_t lo, uint64_t hi, Result* r) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  unsigned long long n = 0;
  for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint32_t u = (uint32_t)i;
    if ((u & 0x7F800000u) == 0x7F800000u) continue;                     // inf, NaN
    const float f = __uint_as_float(u);
    const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{f, -f}, b2));
    const uint32_t want = bf16_bits(u) | bf16_bits(u ^ 0x80000000u) << 16;
    if (hw != want) record(r, u, hw, want);
    ++n;
  }
  tally(r, n);
}

}  // namespace

// which: 0 FP4 encode, 1 FP4 decode, 2 E4M3 encode, 3 bf16 encode, 4 E4M3 above 448.  out[0] = mismatches,
// out[1..3] = input, hardware and software results of the first one, out[4] = the number of
// inputs compared.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int hwconv_check(int which,
                                                                   unsigned long long* out) {
  Result* d = nullptr;
  hipError_t e = hipMalloc(&d, sizeof(Result));
  if (e != hipSuccess) return (int)e;
  e = hipMemset(d, 0, sizeof(Result));
  const uint64_t all = UINT64_C(1) << 32;
  if (e == hipSuccess) {
    if (which == 0) hipLaunchKernelGGL(fp4_encode_all, dim3(8192), dim3(256), 0, 0, 0ull, all, d);
    else if (which == 1) hipLaunchKernelGGL(fp4_decode_all, dim3(1), dim3(256), 0, 0, d);
    else if (which == 2)
      hipLaunchKernelGGL(fp8_encode_all, dim3(8192), dim3(256), 0, 0, 0ull, 0x7F800001ull, d);
    else if (which == 4)
      hipLaunchKernelGGL(fp8_encode_over, dim3(8192), dim3(256), 0, 0, 0x43E00001ull, 0x7F800001ull, d);
    else hipLaunchKernelGGL(bf16_encode_all, dim3(8192), dim3(256), 0, 0, 0ull, all, d);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  Result h = {};
  if (e == hipSuccess) e = hipMemcpy(&h, d, sizeof(Result), hipMemcpyDeviceToHost);
  hipFree(d);
  out[0] = h.count;
  out[1] = h.in;
  out[2] = h.hw;
  out[3] = h.sw;
  out[4] = h.checked;
  return (int)e;
}
