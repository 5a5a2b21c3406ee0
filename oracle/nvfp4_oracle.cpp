// CPU oracle for NVFP4 block-scaled quantization (rtn6 and Four Over Six).
//
// TEST INFRASTRUCTURE ONLY -- loaded by the tests, the smoke check and the benchmark's
// CPU-baseline leg, never by the product path.  No code is shared with the HIP library.
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fPIC -shared (no fast-math).
//
// Readings of the pages that this file fixes (the pages are silent on them) are marked
// "reading:".  Everything else states what the pages define.
#include "nvfp4_oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

std::atomic<int64_t> g_inexact{0};
std::atomic<int64_t> g_shadow_inexact{0};   // the exact shadow's own checks (expected 0)

float f32_from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
uint32_t bits_from_f32(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float bf16_value(uint16_t h) { return f32_from_bits(uint32_t(h) << 16); }

// The FP4 (E2M1) value set: 0, 0.5, 1, 1.5, 2, 3, 4, 6 -- steps of 0.5 on [0,2], 1 on
// [2,4] and 2 on [4,6] [4/6, lay section on the problem; "Problem definition"].  Index =
// 3-bit magnitude code e1 e0 m (exponent bias 1, e = 0 is the subnormal 0.5*m).
const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// Nearest E2M1 magnitude by exact distance.  reading: ties go to the even code (IEEE RNE:
// the code whose mantissa bit is 0); values above 6 saturate to 6 (FP4 has no infinity).
int e2m1_round_mag(float a) {
  if (a >= 6.0f) return 7;                       // saturation, an explicit clamp
  const double ad = a;
  int best = 0;
  double bestd = std::fabs(ad - kE2M1Mag[0]);
  for (int c = 1; c < 8; ++c) {
    const double dist = std::fabs(ad - kE2M1Mag[c]);
    // a tie is between neighbours c-1 and c: keep whichever code is even
    if (dist < bestd || (dist == bestd && (c & 1) == 0)) { best = c; bestd = dist; }
  }
  return best;
}

// E4M3FN byte -> exact value: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent
// field 0 is subnormal m * 2^-9; 0x7E = 448 is the largest finite value, 0x7F is NaN.
// The block scale is FP8 E4M3 with largest value 448 [4/6, "Implementation details"].
double e4m3_value(int b) {
  const int e = (b >> 3) & 0xF, m = b & 7;
  const double mag = e == 0 ? std::ldexp(double(m), -9) : std::ldexp(1.0 + m / 8.0, e - 7);
  return (b & 0x80) ? -mag : mag;
}

// Nearest non-negative finite E4M3 value by exact distance.  reading: RNE (ties to the
// even byte), saturating at 448 instead of producing NaN, subnormal scales kept.
int e4m3_encode(float sigma) {
  const double s = sigma > 448.0f ? 448.0 : double(sigma);
  int best = 0;
  double bestd = std::fabs(s - e4m3_value(0));
  for (int b = 1; b <= 0x7E; ++b) {
    const double dist = std::fabs(s - e4m3_value(b));
    if (dist < bestd || (dist == bestd && (b & 1) == 0)) { best = b; bestd = dist; }
  }
  return best;
}

// Value of a bfloat16 pattern (1 sign, 8 exponent bits, bias 127, 7 mantissa bits).  The
// all-ones exponent with a zero mantissa stands for 2^128 here, the value IEEE rounding
// compares against before it overflows to infinity.
double bf16_pattern_value(uint16_t p) {
  const int e = (p >> 7) & 0xFF, m = p & 0x7F;
  const double mag = e == 0 ? std::ldexp(double(m), -133) : std::ldexp(1.0 + m / 128.0, e - 127);
  return (p & 0x8000) ? -mag : mag;
}

// binary32 -> bfloat16 (finite input), nearest by exact distance, ties to the even pattern.
uint16_t bf16_rne(float f) {
  const uint32_t u = bits_from_f32(f);
  const uint16_t lo = uint16_t(u >> 16);         // truncation toward zero
  const uint16_t hi = uint16_t(lo + 1);          // next bfloat16 away from zero
  const double dl = std::fabs(double(f) - bf16_pattern_value(lo));
  const double dh = std::fabs(double(f) - bf16_pattern_value(hi));
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo;
}

float alpha_of(float amax, int mode) {
  // alpha maps the tensor amax to (largest FP4 value 6) x (largest block-scale value M);
  // Four Over Six uses M = 256 instead of 448 so the 1.5x larger scale of blocks scaled
  // to 4 cannot overflow E4M3 [4/6, "Implementation details"].  reading: alpha =
  // amax / (6*M), one binary32 division by the exact constant 2688 or 1536.
  const float C = mode == ORC_FOUR_OVER_SIX ? 1536.0f : 2688.0f;
  return amax / C;
}

struct Candidate {
  uint8_t scale;
  uint8_t mag[16];
  float xhat[16];
  float err;
};

// One candidate target block maximum Q (6, or 4 under Four Over Six): scale the block so
// its max maps to Q, round every value to FP4, dequantize, and measure the error against
// the original values [4/6, "Adaptive block scaling algorithm": quantize twice, compute
// both errors against the original high-precision values].
// e4m3_scale = false is a diagnostic only: the block scale sigma stays in binary32 instead
// of being rounded to E4M3 (scale byte reported as 0), everything else unchanged.
void run_candidate(const float x[16], float bmax, float alpha, int Q, int rule, Candidate* c,
                   bool e4m3_scale = true) {
  // reading: block scale sigma = bmax / RN32(Q*alpha), then E4M3 (RNE, saturating).
  const float cq = float(Q) * alpha;
  const float sigma = alpha == 0.0f ? 0.0f : bmax / cq;
  c->scale = e4m3_scale ? uint8_t(e4m3_encode(sigma)) : uint8_t(0);
  // reading: the block's dequantization step d = RN32(dec(s) * alpha).
  const float d = e4m3_scale ? float(e4m3_value(c->scale)) * alpha : sigma * alpha;
  // A block scaled to 4 lives in [-4, 4] and gives up 5 and 6 [4/6, "core mechanism"]:
  // its magnitude code is capped at 4 (code 6).  Scale 6 keeps the full grid (code 7).
  const int cap = Q == 4 ? 6 : 7;
  // reading: values are scaled by the correctly rounded reciprocal r = RN32(1/d) and
  // v = RN32(x*r); when 1/d overflows binary32 (d <= 2^-128), v = RN32(x/d) instead.
  // A zero step (scale byte 0) quantizes every value to a (signed) zero code.
  const float r = d == 0.0f ? 0.0f : 1.0f / d;
  const bool recip_finite = std::isfinite(r);
  for (int i = 0; i < 16; ++i) {
    int m = 0;
    if (d != 0.0f) {
      const float v = recip_finite ? x[i] * r : x[i] / d;
      m = std::min(e2m1_round_mag(std::fabs(v)), cap);
    }
    c->mag[i] = uint8_t(m);
    const float mag_hat = float(kE2M1Mag[m]) * d;       // RN32(val(m) * d)
    c->xhat[i] = std::signbit(x[i]) ? -mag_hat : mag_hat;
  }
  // reading: errors are sums (the 1/16 of a mean never changes which candidate wins),
  // accumulated sequentially over i = 0..15 in binary32: fma for the squared error, an
  // add for the absolute error, an exact max for the max error.
  float acc = 0.0f;
  for (int i = 0; i < 16; ++i) {
    const float e = x[i] - c->xhat[i];
    if (double(x[i]) - double(c->xhat[i]) != double(e)) g_inexact.fetch_add(1);
    if (rule == ORC_MSE)      acc = std::fma(e, e, acc);
    else if (rule == ORC_MAE) acc = acc + std::fabs(e);
    else                      acc = std::max(acc, std::fabs(e));
  }
  c->err = acc;
}

void quantize_block(const float x[16], float alpha, int mode, int rule, uint8_t codes8[8],
                    uint8_t* scale, uint16_t y16[16], orc_block_debug* dbg,
                    Candidate* chosen = nullptr) {
  if (std::isnan(alpha)) {                        // poisoned tensor (non-finite input)
    std::memset(codes8, 0, 8);
    *scale = 0x7F;
    if (y16) for (int i = 0; i < 16; ++i) y16[i] = 0x7FC0;
    if (dbg) { dbg->qstar = 0; dbg->s6 = dbg->s4 = 0x7F; dbg->err6 = dbg->err4 = NAN; }
    return;
  }
  float bmax = 0.0f;                              // block max |x|, exact
  for (int i = 0; i < 16; ++i) bmax = std::max(bmax, std::fabs(x[i]));

  Candidate c6, c4;
  run_candidate(x, bmax, alpha, 6, rule, &c6);     // standard NVFP4: block max -> 6
  const Candidate* win = &c6;
  if (mode == ORC_FOUR_OVER_SIX) {
    run_candidate(x, bmax, alpha, 4, rule, &c4);   // Four Over Six: also block max -> 4
    // keep the scale with the smaller error; reading: a tie keeps 6
    if (c4.err < c6.err) win = &c4;
  }
  *scale = win->scale;
  for (int j = 0; j < 8; ++j) {
    // reading: code = sign of x (bit 3, also for zero magnitudes) | magnitude; two codes
    // per byte, the even element in the low nibble.
    const int lo = (std::signbit(x[2 * j]) ? 8 : 0) | win->mag[2 * j];
    const int hi = (std::signbit(x[2 * j + 1]) ? 8 : 0) | win->mag[2 * j + 1];
    codes8[j] = uint8_t(lo | (hi << 4));
  }
  // simulated quantization output: the dequantized value rounded to bf16
  if (y16) for (int i = 0; i < 16; ++i) y16[i] = bf16_rne(win->xhat[i]);
  if (chosen) *chosen = *win;
  if (dbg) {
    dbg->qstar = win == &c4 ? 4 : 6;
    dbg->s6 = c6.scale;
    dbg->err6 = c6.err;
    dbg->s4 = mode == ORC_FOUR_OVER_SIX ? c4.scale : 0;
    dbg->err4 = mode == ORC_FOUR_OVER_SIX ? c4.err : NAN;
  }
}

// Error statistics of a quantized tensor (diagnostics; the encoding does not use them).
// The Four Over Six explainer ("Problem definition") reports that, on a real model, the
// error of rounding the block scales to FP8 matters little while rounding the values near
// the block max (66.6 % to 100 % of it, where scale 6 has no FP4 value between 4 and 6)
// drives the loss.  reading: per tensor, over the chosen candidate of every block,
//   sse      = sum e_i^2           sae = sum |e_i|          maxerr = max |e_i|
//   sse_near = sum e_i^2 over elements with |x_i| > (2/3) bmax of their block, near = their
//              count (3|x| > 2 bmax, an exact comparison)
//   sse_f32  = sum e_i^2 when the chosen candidate keeps its binary32 block scale sigma
//              instead of the E4M3 byte (so sse - sse_f32 is what rounding the scales costs)
// e_i = x_i - xhat_i is exact (binary32), so each term e_i^2 is exact in long double; the
// sums are taken in long double in element order.
struct TensorStats {
  long double sse = 0, sae = 0, sse_near = 0, sse_f32 = 0;
  float maxerr = 0.0f;
  int64_t near = 0;
};

void accumulate_block_stats(const float x[16], float alpha, int mode, int rule,
                            TensorStats* st) {
  uint8_t codes8[8], scale;
  orc_block_debug dbg;
  Candidate win, f32;
  quantize_block(x, alpha, mode, rule, codes8, &scale, nullptr, &dbg, &win);
  float bmax = 0.0f;
  for (int i = 0; i < 16; ++i) bmax = std::max(bmax, std::fabs(x[i]));
  run_candidate(x, bmax, alpha, dbg.qstar, rule, &f32, /*e4m3_scale=*/false);
  for (int i = 0; i < 16; ++i) {
    const float e = x[i] - win.xhat[i];
    const long double e2 = (long double)e * (long double)e;
    st->sse += e2;
    st->sae += std::fabs((long double)e);
    st->maxerr = std::max(st->maxerr, std::fabs(e));
    if (3.0 * std::fabs(double(x[i])) > 2.0 * double(bmax)) {
      st->sse_near += e2;
      ++st->near;
    }
    const float eu = x[i] - f32.xhat[i];
    st->sse_f32 += (long double)eu * (long double)eu;
  }
}

// amax over n elements; NaN if any element is NaN or infinite.
float tensor_amax(const uint16_t* in, int64_t n) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    const float x = bf16_value(in[i]);
    if (!std::isfinite(x)) return NAN;
    amax = std::max(amax, std::fabs(x));
  }
  return amax;
}

template <class F>
void parallel_ranges(int64_t n, int nthreads, F&& fn) {
  if (nthreads <= 1 || n < 2) { fn(int64_t(0), n); return; }
  std::vector<std::thread> ts;
  const int64_t chunk = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    ts.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& t : ts) t.join();
}

// ----------------------------------------------------------------------------- exact shadow
// The exact-quotient reading of the same encoding: no step rounds except the encodings
// themselves (E4M3 scale, E2M1 codes, bf16 output), either after the binary32 per-tensor scale
// alpha (an FP32 value of the format) or with alpha = amax / (6*M) taken exactly.  Values live
// in x87 extended precision (64-bit significand):
//   Q*alpha                 2 + 24 significant bits   exact
//   dec(s) * alpha          4 + 24                    exact
//   t * dec(s) * Q * alpha  products of the grids' values (at most 2 bits each) with the above,
//                           at most 32 bits           exact
// (with alpha exact, every value is scaled by 6*M, at most 5 significant bits, and alpha
// becomes the 8-bit amax: fewer bits still)
// so every product below is exact, and every distance that can decide a nearest value or a
// tie (a difference of a bf16 value, 8 bits, and such a product of similar magnitude) is exact
// too.  The error terms e = x - xhat are checked for exactness with an error-free sum, and the
// error sums are taken exactly in a fixed-point integer, so the choice between 6 and 4 is the
// one exact arithmetic makes.
typedef long double xf;

// Exact sum of non-negative terms m * 2^k (m < 2^128): a 768-bit fixed-point integer whose
// least bit weighs 2^-kExactLo.  e is a multiple of 2^-159 (bf16 inputs are multiples of
// 2^-133, and val * dec(s) * alpha of 2^-1 * 2^-9 * 2^-149) and below 2^130, so e^2 and |e|
// and sums of 16 of them fit with room to spare.
constexpr int kExactLo = 330;
constexpr int kExactLimbs = 12;
struct ExactSum {
  uint64_t w[kExactLimbs] = {};
  bool out_of_range = false;
  void add64(uint64_t v, int p) {
    int i = p / 64;
    const int sh = p % 64;
    uint64_t lo = v << sh, hi = sh ? v >> (64 - sh) : 0;
    for (; i < kExactLimbs && (lo | hi); ++i) {
      const uint64_t old = w[i];
      w[i] += lo;
      const uint64_t carry = w[i] < old ? 1 : 0;
      lo = hi + carry;
      hi = (lo < carry) ? 1 : 0;        // hi + carry wrapped only if hi was all ones
    }
    if (lo | hi) out_of_range = true;
  }
  void add(unsigned __int128 m, int k) {
    const int p = k + kExactLo;
    if (p < 0 || p + 128 > 64 * kExactLimbs) { out_of_range = true; return; }
    add64(uint64_t(m), p);
    add64(uint64_t(m >> 64), p + 64);
  }
};

int exact_cmp(const ExactSum& a, const ExactSum& b) {
  for (int i = kExactLimbs - 1; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i] ? -1 : 1;
  return 0;
}

// |v| = m * 2^k with m odd (v != 0 and exact in xf).
void split_exact(xf v, uint64_t* m, int* k) {
  int e = 0;
  const xf f = std::frexp(std::fabs(v), &e);     // [0.5, 1)
  uint64_t mm = uint64_t(std::ldexp(f, 64));      // 64-bit significand, an integer
  int kk = e - 64;
  while ((mm & 1) == 0) { mm >>= 1; ++kk; }
  *m = mm;
  *k = kk;
}

// Nearest E4M3 byte to sigma = bmax / qa (qa = Q*alpha > 0) by exact distance, ties to the
// even byte: |bmax - dec(b)*qa| = |sigma - dec(b)| * qa.  Above 448 the nearest is 448 itself,
// which is the saturation of the binary32 reading too.
int exact_e4m3(xf bmax, xf qa) {
  int best = 0;
  xf bestd = bmax;
  for (int b = 1; b <= 0x7E; ++b) {
    const xf dist = std::fabs(bmax - xf(e4m3_value(b)) * qa);
    if (dist < bestd || (dist == bestd && (b & 1) == 0)) { best = b; bestd = dist; }
  }
  return best;
}

// Nearest E2M1 magnitude code to a / D (D > 0) by exact distance, ties to the even code;
// above 6 the nearest is 6 (saturation).
int exact_e2m1(xf a, xf D) {
  int best = 0;
  xf bestd = a;
  for (int c = 1; c < 8; ++c) {
    const xf dist = std::fabs(a - xf(kE2M1Mag[c]) * D);
    if (dist < bestd || (dist == bestd && (c & 1) == 0)) { best = c; bestd = dist; }
  }
  return best;
}

// Nearest bfloat16 to v / c for an exact v and c in {1, 1536, 2688} (ties to the even
// pattern): the nearest lies next to the truncation of the quotient's binary32 rounding, and
// |v - c * value(p)| compares the candidates exactly (c * value(p) has at most 13 bits).
uint16_t bf16_rne_exact(xf v, xf c) {
  const bool neg = std::signbit(v);
  const xf a = std::fabs(v);
  const uint16_t t = uint16_t(bits_from_f32(float(a / c)) >> 16);
  uint16_t best = t;
  xf bestd = std::fabs(a - c * xf(bf16_pattern_value(t)));
  for (int dlt = -1; dlt <= 1; dlt += 2) {
    const int p = int(t) + dlt;
    if (p < 0 || p > 0x7F80) continue;
    const xf dist = std::fabs(a - c * xf(bf16_pattern_value(uint16_t(p))));
    if (dist < bestd || (dist == bestd && (p & 1) == 0)) { best = uint16_t(p); bestd = dist; }
  }
  return uint16_t(best | (neg ? 0x8000 : 0));
}

struct ExactCand {
  int scale = 0;
  uint8_t mag[16] = {};
  xf xhat[16] = {};
  ExactSum sum;          // MSE: sum of e^2; MAE: sum of |e|
  xf maxerr = 0;         // MAXERR: max |e|
};

// One candidate target block maximum Q under exact arithmetic.  Every value is given scaled
// by a common factor c (x[i] = c * x_i, bmax = c * bmax, a = c * alpha): with c = 1 and a the
// binary32 alpha this is the exact reading after alpha; with c = 6*M and a = amax it is the
// fully exact reading with alpha = amax / (6*M) as a rational.  The scale byte, the codes and
// the choice do not depend on c (every comparison scales with it), and xhat and e come out
// scaled by c.
void exact_candidate(const xf x[16], xf bmax, xf a, int Q, int rule, ExactCand* c,
                     int64_t* inexact) {
  const xf qa = xf(Q) * a;
  c->scale = a == 0 ? 0 : exact_e4m3(bmax, qa);
  const xf D = xf(e4m3_value(c->scale)) * a;
  const int cap = Q == 4 ? 6 : 7;                 // a block scaled to 4 stays within [-4, 4]
  for (int i = 0; i < 16; ++i) {
    const xf xi = x[i];
    const int m = D == 0 ? 0 : std::min(exact_e2m1(std::fabs(xi), D), cap);
    c->mag[i] = uint8_t(m);
    const xf mag_hat = xf(kE2M1Mag[m]) * D;
    c->xhat[i] = std::signbit(xi) ? -mag_hat : mag_hat;
    // e = x - xhat, with Knuth's two-sum error term to confirm the subtraction is exact
    const xf b = -c->xhat[i];
    const xf e = xi + b;
    const xf bb = e - xi;
    const xf err = (xi - (e - bb)) + (b - bb);
    if (err != 0) ++*inexact;
    if (e == 0) continue;
    if (rule == ORC_MAXERR) {
      c->maxerr = std::max(c->maxerr, std::fabs(e));
    } else {
      uint64_t mm;
      int kk;
      split_exact(e, &mm, &kk);
      if (rule == ORC_MSE) c->sum.add((unsigned __int128)mm * mm, 2 * kk);
      else                 c->sum.add(mm, kk);
    }
  }
  if (c->sum.out_of_range) ++*inexact;
}

// One block under the exact reading.  exact_alpha = false: a is the binary32 alpha;
// exact_alpha = true: a is the tensor amax and alpha = amax / (6*M) exactly.
void exact_block(const float xin[16], float a, int mode, int rule, bool exact_alpha,
                 uint8_t codes8[8], uint8_t* scale, uint16_t y16[16], int* qstar, bool* tie,
                 int64_t* inexact) {
  const xf c = exact_alpha ? xf(mode == ORC_FOUR_OVER_SIX ? 1536 : 2688) : xf(1);
  xf x[16];
  xf bmax = 0;
  for (int i = 0; i < 16; ++i) {
    x[i] = c * xf(xin[i]);                        // exact: 8 + 5 significant bits
    bmax = std::max(bmax, std::fabs(x[i]));
  }
  ExactCand c6, c4;
  exact_candidate(x, bmax, xf(a), 6, rule, &c6, inexact);
  const ExactCand* win = &c6;
  *tie = false;
  if (mode == ORC_FOUR_OVER_SIX) {
    exact_candidate(x, bmax, xf(a), 4, rule, &c4, inexact);
    const int cmp = rule == ORC_MAXERR ? (c4.maxerr < c6.maxerr ? -1 : c4.maxerr > c6.maxerr ? 1 : 0)
                                       : exact_cmp(c4.sum, c6.sum);
    if (cmp < 0) win = &c4;                       // a tie keeps 6
    *tie = cmp == 0;
  }
  *scale = uint8_t(win->scale);
  for (int j = 0; j < 8; ++j) {
    const int lo = (std::signbit(xin[2 * j]) ? 8 : 0) | win->mag[2 * j];
    const int hi = (std::signbit(xin[2 * j + 1]) ? 8 : 0) | win->mag[2 * j + 1];
    codes8[j] = uint8_t(lo | (hi << 4));
  }
  if (y16) for (int i = 0; i < 16; ++i) y16[i] = bf16_rne_exact(win->xhat[i], c);
  *qstar = win == &c4 ? 4 : 6;
}

bool bad_args(const void* in, int64_t E, int64_t rows, int64_t cols, int mode, int rule) {
  return !in || E <= 0 || rows <= 0 || cols <= 0 || cols % 16 != 0 ||
         (mode != ORC_RTN6 && mode != ORC_FOUR_OVER_SIX) ||
         (rule != ORC_MSE && rule != ORC_MAE && rule != ORC_MAXERR);
}

}  // namespace

extern "C" {

float orc_e2m1_decode(int code) {
  const float mag = float(kE2M1Mag[code & 7]);
  return (code & 8) ? -mag : mag;
}
int orc_e2m1_round_mag(float a) { return e2m1_round_mag(a); }
void orc_e2m1_round_mag_many(const float* a, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = uint8_t(e2m1_round_mag(a[i]));
}
double orc_e4m3_decode(int byte) { return e4m3_value(byte); }
int orc_e4m3_encode(float sigma) { return e4m3_encode(sigma); }
void orc_e4m3_encode_many(const float* s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = uint8_t(e4m3_encode(s[i]));
}
uint16_t orc_bf16_rne(float f) { return bf16_rne(f); }
void orc_bf16_rne_many(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(f[i]);
}
float orc_alpha(float amax, int mode) { return alpha_of(amax, mode); }

int orc_amax(const uint16_t* in, int64_t E, int64_t n, float* amax_out) {
  if (!in || !amax_out || E <= 0 || n <= 0) return -1;
  for (int64_t t = 0; t < E; ++t) amax_out[t] = tensor_amax(in + t * n, n);
  return 0;
}

void orc_quantize_block(const uint16_t* x16, float alpha, int mode, int rule, uint8_t* codes8,
                        uint8_t* scale, uint16_t* y16, orc_block_debug* dbg) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = bf16_value(x16[i]);
  quantize_block(x, alpha, mode, rule, codes8, scale, y16, dbg);
}

void orc_candidate(const uint16_t* x16, float alpha, int Q, int rule, uint8_t* mag16,
                   uint8_t* scale, float* xhat16, float* err) {
  float x[16], bmax = 0.0f;
  for (int i = 0; i < 16; ++i) { x[i] = bf16_value(x16[i]); bmax = std::max(bmax, std::fabs(x[i])); }
  Candidate c;
  run_candidate(x, bmax, alpha, Q == 4 ? 4 : 6, rule, &c);
  std::memcpy(mag16, c.mag, 16);
  *scale = c.scale;
  std::memcpy(xhat16, c.xhat, sizeof c.xhat);
  *err = c.err;
}

int orc_quantize(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode, int rule,
                 uint8_t* codes, uint8_t* scales, float* alpha, uint16_t* y, uint8_t* qstar,
                 int nthreads) {
  if (bad_args(in, E, rows, cols, mode, rule) || !codes || !scales || !alpha) return -1;
  const int64_t n = rows * cols, nb = n / 16;
  for (int64_t t = 0; t < E; ++t) {
    const uint16_t* x = in + t * n;
    // pass 1: the tensor amax (combined over ranges by max, which is exact)
    std::vector<float> part(std::max(1, nthreads), 0.0f);
    std::atomic<bool> nonfinite{false};
    std::atomic<int> slot{0};
    parallel_ranges(n, nthreads, [&](int64_t lo, int64_t hi) {
      const float a = tensor_amax(x + lo, hi - lo);
      if (std::isnan(a)) nonfinite = true; else part[slot++] = a;
    });
    float amax = 0.0f;
    for (float a : part) amax = std::max(amax, a);
    const float al = nonfinite ? NAN : alpha_of(amax, mode);
    alpha[t] = al;
    // pass 2: every block with the tensor's alpha
    parallel_ranges(nb, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t b = lo; b < hi; ++b) {
        orc_block_debug dbg;
        float xb[16];
        for (int i = 0; i < 16; ++i) xb[i] = bf16_value(x[b * 16 + i]);
        quantize_block(xb, al, mode, rule, codes + (t * nb + b) * 8, scales + t * nb + b,
                       y ? y + (t * nb + b) * 16 : nullptr, &dbg);
        if (qstar) qstar[t * nb + b] = uint8_t(dbg.qstar);
      }
    });
  }
  return 0;
}

int orc_quantize_blocks(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode,
                        int rule, const float* alpha, const int64_t* ids, int64_t nsel,
                        uint8_t* codes, uint8_t* scales, uint16_t* y, uint8_t* qstar) {
  if (bad_args(in, E, rows, cols, mode, rule) || !alpha || !ids || nsel < 0 || !codes ||
      !scales)
    return -1;
  const int64_t nb = rows * cols / 16;
  for (int64_t k = 0; k < nsel; ++k) {
    const int64_t b = ids[k];
    if (b < 0 || b >= E * nb) return -2;
    float xb[16];
    for (int i = 0; i < 16; ++i) xb[i] = bf16_value(in[b * 16 + i]);
    orc_block_debug dbg;
    quantize_block(xb, alpha[b / nb], mode, rule, codes + k * 8, scales + k,
                   y ? y + k * 16 : nullptr, &dbg);
    if (qstar) qstar[k] = uint8_t(dbg.qstar);
  }
  return 0;
}

int orc_dequantize(const uint8_t* codes, const uint8_t* scales, const float* alpha, int64_t E,
                   int64_t rows, int64_t cols, uint16_t* y) {
  if (!codes || !scales || !alpha || !y || E <= 0 || rows <= 0 || cols <= 0 || cols % 16 != 0)
    return -1;
  const int64_t nb = rows * cols / 16;
  for (int64_t t = 0; t < E; ++t) {
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t g = t * nb + b;
      const uint8_t s = scales[g];
      uint16_t* yb = y + g * 16;
      if (std::isnan(alpha[t]) || (s & 0x7F) == 0x7F) {       // poisoned tensor or NaN scale
        for (int i = 0; i < 16; ++i) yb[i] = 0x7FC0;
        continue;
      }
      // the block's step, as in quantization: d = RN32(dec(s) * alpha)
      const float d = float(e4m3_value(s)) * alpha[t];
      for (int i = 0; i < 16; ++i) {
        const int code = (codes[g * 8 + i / 2] >> (4 * (i & 1))) & 0xF;
        const float mag = float(kE2M1Mag[code & 7]) * d;     // RN32(val * d)
        yb[i] = bf16_rne((code & 8) ? -mag : mag);
      }
    }
  }
  return 0;
}

int orc_quantize_stats(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode,
                       int rule, double* stats, int nthreads) {
  if (bad_args(in, E, rows, cols, mode, rule) || !stats) return -1;
  const int64_t n = rows * cols, nb = n / 16;
  const int nt = std::max(1, nthreads);
  for (int64_t t = 0; t < E; ++t) {
    const uint16_t* x = in + t * n;
    double* out = stats + t * ORC_NSTATS;
    const float amax = tensor_amax(x, n);
    if (std::isnan(amax)) {                       // poisoned tensor: no statistics
      for (int k = 0; k < ORC_NSTATS; ++k) out[k] = NAN;
      continue;
    }
    const float al = alpha_of(amax, mode);
    // contiguous block ranges, combined in range order
    const int64_t chunk = (nb + nt - 1) / nt;
    std::vector<TensorStats> parts(nt);
    parallel_ranges(nb, nt, [&](int64_t lo, int64_t hi) {
      TensorStats& p = parts[lo / std::max<int64_t>(1, chunk)];
      for (int64_t b = lo; b < hi; ++b) {
        float xb[16];
        for (int i = 0; i < 16; ++i) xb[i] = bf16_value(x[b * 16 + i]);
        accumulate_block_stats(xb, al, mode, rule, &p);
      }
    });
    TensorStats tot;
    for (const TensorStats& p : parts) {
      tot.sse += p.sse;
      tot.sae += p.sae;
      tot.sse_near += p.sse_near;
      tot.sse_f32 += p.sse_f32;
      tot.maxerr = std::max(tot.maxerr, p.maxerr);
      tot.near += p.near;
    }
    out[ORC_STAT_SSE] = double(tot.sse);
    out[ORC_STAT_SAE] = double(tot.sae);
    out[ORC_STAT_MAXERR] = double(tot.maxerr);
    out[ORC_STAT_SSE_NEAR] = double(tot.sse_near);
    out[ORC_STAT_SSE_F32SCALE] = double(tot.sse_f32);
    out[ORC_STAT_NEAR_COUNT] = double(tot.near);
  }
  return 0;
}

int64_t orc_inexact_subtractions(void) { return g_inexact.load(); }

void orc_shadow_block(const uint16_t* x16, float a, int mode, int rule, int exact_alpha,
                      uint8_t* codes8, uint8_t* scale, uint16_t* y16, int* qstar) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = bf16_value(x16[i]);
  bool tie = false;
  int64_t inexact = 0;
  exact_block(x, a, mode, rule, exact_alpha != 0, codes8, scale, y16, qstar, &tie, &inexact);
  g_shadow_inexact.fetch_add(inexact);
}

int64_t orc_shadow_inexact(void) { return g_shadow_inexact.load(); }

int orc_shadow_compare(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode,
                       int rule, int exact_alpha, orc_shadow_counts* out, int nthreads) {
  if (bad_args(in, E, rows, cols, mode, rule) || !out) return -1;
  const int64_t n = rows * cols, nb = n / 16;
  const int nt = std::max(1, nthreads);
  std::vector<orc_shadow_counts> parts(nt);
  for (auto& p : parts) std::memset(&p, 0, sizeof p);
  for (int64_t t = 0; t < E; ++t) {
    const uint16_t* x = in + t * n;
    const float amax = tensor_amax(x, n);
    if (std::isnan(amax)) continue;               // poisoned tensor: nothing to compare
    const float al = alpha_of(amax, mode);
    const int64_t chunk = (nb + nt - 1) / nt;
    parallel_ranges(nb, nt, [&](int64_t lo, int64_t hi) {
      orc_shadow_counts& c = parts[lo / std::max<int64_t>(1, chunk)];
      for (int64_t b = lo; b < hi; ++b) {
        float xb[16];
        for (int i = 0; i < 16; ++i) xb[i] = bf16_value(x[b * 16 + i]);
        uint8_t c32[8], cx[8], s32, sx;
        uint16_t y32[16], yx[16];
        orc_block_debug dbg;
        quantize_block(xb, al, mode, rule, c32, &s32, y32, &dbg);
        int qx = 0;
        bool tie = false;
        exact_block(xb, exact_alpha ? amax : al, mode, rule, exact_alpha != 0, cx, &sx, yx, &qx,
                    &tie, &c.inexact);
        ++c.blocks;
        int dc = 0, dy = 0;
        for (int i = 0; i < 16; ++i) {
          dc += ((c32[i / 2] >> (4 * (i & 1))) & 0xF) != ((cx[i / 2] >> (4 * (i & 1))) & 0xF);
          dy += y32[i] != yx[i];
        }
        c.code_diff += dc;
        c.y_diff += dy;
        c.scale_diff += s32 != sx;
        c.choice_diff += dbg.qstar != qx;
        c.block_diff += (dc > 0 || s32 != sx);
        c.exact_ties += tie;
      }
    });
  }
  std::memset(out, 0, sizeof *out);
  for (const auto& p : parts) {
    out->blocks += p.blocks;
    out->scale_diff += p.scale_diff;
    out->choice_diff += p.choice_diff;
    out->block_diff += p.block_diff;
    out->code_diff += p.code_diff;
    out->y_diff += p.y_diff;
    out->exact_ties += p.exact_ties;
    out->inexact += p.inexact;
  }
  return 0;
}

}  // extern "C"
