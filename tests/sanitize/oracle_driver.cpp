// Drives every function of the CPU oracle on small inputs, for a build with
// -fsanitize=address,undefined: any out-of-bounds access, use of uninitialised or freed
// memory, signed overflow or bad shift aborts the program with a report.  The checks below
// are consistency checks between the oracle's own entry points (the oracle's pins live in
// the Python tests); the point of this program is that every code path runs under the
// sanitizers.  Inputs are bf16 bit patterns from a fixed linear congruential generator.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "nvfp4_oracle.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return uint32_t(g_state >> 33);
}

// A bf16 pattern: mostly finite values over a wide exponent range, some zeros of both signs,
// some subnormals.
uint16_t random_bf16(int lo_exp, int hi_exp) {
  const uint32_t r = next_u32();
  const uint16_t sign = uint16_t((r & 1) << 15);
  switch ((r >> 1) % 16) {
    case 0: return sign;                                        // +-0
    case 1: return uint16_t(sign | ((r >> 8) % 0x7F + 1));      // subnormal
    default: {
      const int e = lo_exp + int((r >> 8) % uint32_t(hi_exp - lo_exp + 1));
      return uint16_t(sign | (uint16_t(e + 127) << 7) | ((r >> 20) & 0x7F));
    }
  }
}

int g_fail = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s\n", what);
    ++g_fail;
  }
}

void run_shape(int64_t E, int64_t rows, int64_t cols, int lo_exp, int hi_exp, int poison) {
  const int64_t n = rows * cols, nb = n / 16;
  std::vector<uint16_t> x(E * n);
  for (auto& v : x) v = random_bf16(lo_exp, hi_exp);
  if (poison >= 0 && poison < E) x[poison * n + n / 2] = 0x7FC0;   // NaN in tensor `poison`
  for (int mode = 0; mode < 2; ++mode) {
    for (int rule = 0; rule < 3; ++rule) {
      std::vector<uint8_t> codes(E * n / 2), scales(E * nb), qstar(E * nb);
      std::vector<float> alpha(E), amax(E);
      std::vector<uint16_t> y(E * n), y2(E * n);
      check(orc_quantize(x.data(), E, rows, cols, mode, rule, codes.data(), scales.data(),
                         alpha.data(), y.data(), qstar.data(), 3) == 0, "quantize");
      check(orc_amax(x.data(), E, n, amax.data()) == 0, "amax");
      std::vector<float> al(E);
      for (int64_t t = 0; t < E; ++t) al[t] = std::isnan(amax[t]) ? NAN : orc_alpha(amax[t], mode);
      for (int64_t t = 0; t < E; ++t)
        check(std::memcmp(&al[t], &alpha[t], 4) == 0, "alpha from amax");
      std::vector<int64_t> ids(E * nb);
      for (int64_t b = 0; b < E * nb; ++b) ids[b] = E * nb - 1 - b;      // reversed
      std::vector<uint8_t> c2(E * n / 2), s2(E * nb), q2(E * nb);
      std::vector<uint16_t> y3(E * n);
      check(orc_quantize_blocks(x.data(), E, rows, cols, mode, rule, al.data(), ids.data(),
                                E * nb, c2.data(), s2.data(), y3.data(), q2.data()) == 0,
            "quantize_blocks");
      for (int64_t k = 0; k < E * nb; ++k) {
        const int64_t b = ids[k];
        check(std::memcmp(&c2[k * 8], &codes[b * 8], 8) == 0 && s2[k] == scales[b] &&
                  q2[k] == qstar[b] && std::memcmp(&y3[k * 16], &y[b * 16], 32) == 0,
              "sampled blocks equal the whole tensor");
      }
      check(orc_dequantize(codes.data(), scales.data(), alpha.data(), E, rows, cols,
                           y2.data()) == 0, "dequantize");
      check(y == y2, "dequantize equals fake-quant");
      std::vector<double> stats(E * ORC_NSTATS);
      check(orc_quantize_stats(x.data(), E, rows, cols, mode, rule, stats.data(), 2) == 0,
            "stats");
      for (int exact_alpha = 0; exact_alpha < 2; ++exact_alpha) {
        orc_shadow_counts sc;
        check(orc_shadow_compare(x.data(), E, rows, cols, mode, rule, exact_alpha, &sc, 2) == 0,
              "shadow_compare");
        for (int64_t b = 0; b < nb; ++b) {
          uint8_t c8[8], s;
          uint16_t y16[16];
          int q = 0;
          if (!std::isnan(al[0]))
            orc_shadow_block(&x[b * 16], exact_alpha ? amax[0] : al[0], mode, rule, exact_alpha,
                             c8, &s, y16, &q);
        }
      }
      for (int64_t b = 0; b < nb && !std::isnan(al[0]); ++b) {
        uint8_t mag[16], s;
        float xh[16], err;
        orc_candidate(&x[b * 16], al[0], b & 1 ? 4 : 6, rule, mag, &s, xh, &err);
        orc_block_debug dbg;
        uint8_t c8[8];
        uint16_t y16[16];
        orc_quantize_block(&x[b * 16], al[0], mode, rule, c8, &s, y16, &dbg);
      }
    }
  }
}

}  // namespace

int main() {
  // formats over their whole domains
  for (int c = 0; c < 16; ++c) (void)orc_e2m1_decode(c);
  for (int b = 0; b < 256; ++b) if ((b & 0x7F) != 0x7F) (void)orc_e4m3_decode(b);
  std::vector<float> f(4096);
  for (size_t i = 0; i < f.size(); ++i) f[i] = float(i) * 0.01f;
  std::vector<uint8_t> o8(f.size());
  std::vector<uint16_t> o16(f.size());
  orc_e2m1_round_mag_many(f.data(), int64_t(f.size()), o8.data());
  orc_e4m3_encode_many(f.data(), int64_t(f.size()), o8.data());
  orc_bf16_rne_many(f.data(), int64_t(f.size()), o16.data());
  // worked example A of the pins: one block [6, 5, 4.5, 0 x 13] under Four Over Six
  uint16_t a[16] = {0x40C0, 0x40A0, 0x4090};
  uint8_t codes[8], scale;
  uint16_t y[16];
  orc_block_debug dbg;
  orc_quantize_block(a, orc_alpha(6.0f, 1), 1, 0, codes, &scale, y, &dbg);
  check(scale == 0x7C && codes[0] == 0x56 && codes[1] == 0x05 && dbg.qstar == 4, "example A");
  // shapes: single block, ragged thread splits, batches with a poisoned tensor, tiny alpha
  run_shape(1, 1, 16, -10, 10, -1);
  run_shape(3, 5, 48, -20, 20, 1);
  run_shape(2, 7, 32, -130, -110, -1);       // subnormal alpha: division fallback, clamps
  run_shape(2, 3, 64, 100, 127, -1);         // near the bf16 maximum
  run_shape(4, 2, 16, -4, 4, 3);
  // bad arguments are rejected
  check(orc_quantize(nullptr, 1, 1, 16, 0, 0, codes, &scale, nullptr, nullptr, nullptr, 1) < 0,
        "null input rejected");
  check(orc_quantize(a, 1, 1, 15, 0, 0, codes, &scale, nullptr, nullptr, nullptr, 1) < 0,
        "ragged columns rejected");
  std::printf("oracle driver: %s, %lld inexact subtractions, %lld shadow exactness failures\n",
              g_fail ? "FAILED" : "ok", (long long)orc_inexact_subtractions(),
              (long long)orc_shadow_inexact());
  return g_fail ? 1 : 0;
}
