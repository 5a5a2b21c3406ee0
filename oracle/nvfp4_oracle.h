/*
 * CPU oracle for NVFP4 block-scaled quantization (standard "rtn6" and Four Over Six).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call this
 * code: only the tests, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no source, header, table or constant with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [4/6]  "Four Over Six: More Accurate NVFP4 Quantization with Adaptive Block Scaling"
 *          (gist.science explainer): "Problem definition", "Method / core mechanism",
 *          "Adaptive block scaling algorithm", "Implementation details".
 *   [QAD]  "Quantization-Aware Distillation for NVFP4 Inference Accuracy Recovery"
 *          (gist.science explainer), key findings item 3 (NVFP4 block size 16).
 *   [LTN]  Nemotron 3.5 Lightning NVFP4 news page, "two-stage QAD process" (student forward
 *          runs through simulated quantization).
 *
 * Every floating-point step is one IEEE binary32 operation with round-to-nearest-even,
 * no contraction (built with -ffp-contract=off), no flush-to-zero; std::fma only where the
 * spec says fma.  E2M1, E4M3 and bfloat16 rounding are done by brute force: the nearest
 * grid value by exact binary64 distance, ties to the even code.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_RTN6 = 0, ORC_FOUR_OVER_SIX = 1 };
enum { ORC_MSE = 0, ORC_MAE = 1, ORC_MAXERR = 2 };

/* Element and scale formats. */
float    orc_e2m1_decode(int code);              /* 4-bit code s|e1 e0|m -> value */
int      orc_e2m1_round_mag(float a);            /* a >= 0 (not NaN) -> magnitude code 0..7 */
void     orc_e2m1_round_mag_many(const float* a, int64_t n, uint8_t* out);
double   orc_e4m3_decode(int byte);              /* E4M3FN byte (not 0x7F/0xFF) -> value */
int      orc_e4m3_encode(float sigma);           /* sigma >= 0 -> byte 0x00..0x7E (saturating) */
void     orc_e4m3_encode_many(const float* s, int64_t n, uint8_t* out);
uint16_t orc_bf16_rne(float f);                  /* binary32 -> bfloat16, RNE (finite f) */
void     orc_bf16_rne_many(const float* f, int64_t n, uint16_t* out);

/* Per-tensor scale alpha = RN32(amax / (6*M)), M = 448 (rtn6) or 256 (four over six). */
float    orc_alpha(float amax, int mode);

/* Tensor amax of E tensors of n elements each, as binary32; NaN if any element is not finite. */
int      orc_amax(const uint16_t* in, int64_t E, int64_t n, float* amax_out);

/* Quantize one 16-element block given the tensor's alpha.  Outputs: 8 packed code bytes,
 * the chosen scale byte, the 16 dequantized values rounded to bf16 (fake-quant), and
 * debug values: chosen candidate Q (6 or 4), each candidate's scale byte and error (the
 * 4-candidate fields are 0 / NaN in rtn6 mode). */
typedef struct {
  int      qstar;
  uint8_t  s6, s4;
  float    err6, err4;
} orc_block_debug;
void     orc_quantize_block(const uint16_t* x16, float alpha, int mode, int rule,
                            uint8_t* codes8, uint8_t* scale, uint16_t* y16,
                            orc_block_debug* dbg);

/* One candidate alone (Q = 6 or 4) with the given alpha: magnitude codes (16 bytes, 0..7,
 * sign not included), scale byte, dequantized binary32 values and the error under rule. */
void     orc_candidate(const uint16_t* x16, float alpha, int Q, int rule, uint8_t* mag16,
                       uint8_t* scale, float* xhat16, float* err);

/* Whole tensors: in is [E][rows][cols] bf16, cols % 16 == 0.  codes [E][rows][cols/2],
 * scales [E][rows][cols/16], alpha [E]; y (fake-quant bf16, [E][rows][cols]) and qstar
 * ([E][rows][cols/16], 6 or 4) may be NULL.  nthreads >= 1 splits each tensor's blocks
 * into contiguous ranges; the result does not depend on it.  Returns 0 or a negative
 * error for bad arguments. */
int      orc_quantize(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode,
                      int rule, uint8_t* codes, uint8_t* scales, float* alpha, uint16_t* y,
                      uint8_t* qstar, int nthreads);

/* Selected blocks only (for sampled checks at full size): flat block ids over
 * [E][rows][cols/16]; alpha[E] from orc_amax + orc_alpha (NaN = poisoned tensor). */
int      orc_quantize_blocks(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                             int mode, int rule, const float* alpha, const int64_t* ids,
                             int64_t nsel, uint8_t* codes, uint8_t* scales, uint16_t* y,
                             uint8_t* qstar);

/* Dequantize packed NVFP4 to bf16: y = RNbf16(val(code) * RN32(dec(scale) * alpha)), sign
 * from the code.  A NaN alpha or a NaN scale byte (0x7F / 0xFF) gives 0x7FC0 for the block.
 * codes [E][rows][cols/2], scales [E][rows][cols/16], alpha [E], y [E][rows][cols]. */
int      orc_dequantize(const uint8_t* codes, const uint8_t* scales, const float* alpha,
                        int64_t E, int64_t rows, int64_t cols, uint16_t* y);

/* Error statistics per tensor (diagnostics), stats [E][ORC_NSTATS] as double, over the
 * chosen candidate of every block: sum e^2, sum |e|, max |e|, sum e^2 over the elements
 * above two thirds of their block max, the same sum with each block's binary32 scale
 * instead of its E4M3 byte, and the count of elements above two thirds of their block
 * max.  Sums in long double, element order.  A poisoned tensor gets NaN everywhere. */
enum { ORC_STAT_SSE = 0, ORC_STAT_SAE = 1, ORC_STAT_MAXERR = 2, ORC_STAT_SSE_NEAR = 3,
       ORC_STAT_SSE_F32SCALE = 4, ORC_STAT_NEAR_COUNT = 5, ORC_NSTATS = 6 };
int      orc_quantize_stats(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                            int mode, int rule, double* stats, int nthreads);

/* Count of error subtractions e = x - xhat that were not exact (expected 0). */
int64_t  orc_inexact_subtractions(void);

/* Exact-quotient shadow: the same encoding read with exact arithmetic after the per-tensor
 * scale.  Per block and candidate Q: sigma = bmax / (Q*alpha) exactly, s = E4M3 RNE of sigma
 * (saturating at 448), D = dec(s) * alpha exactly, code = E2M1 RNE of |x| / D exactly (capped
 * at 4 for Q = 4), xhat = val(code) * D exactly, e = x - xhat exactly, and the error sums or
 * max exactly; the smaller error wins, ties keep 6 [4/6, "Adaptive block scaling algorithm":
 * both errors against the original high-precision values].  Fake-quant: y = RNbf16(xhat).
 * exact_alpha = 0: `a` is the binary32 alpha (an FP32 value of the format);
 * exact_alpha = 1: `a` is the tensor amax and alpha = amax / (6*M) is taken exactly.
 * A diagnostic of how far the binary32 reading departs from exact arithmetic; not what the
 * GPU path is checked against. */
void     orc_shadow_block(const uint16_t* x16, float a, int mode, int rule, int exact_alpha,
                          uint8_t* codes8, uint8_t* scale, uint16_t* y16, int* qstar);
/* Count of the shadow's exactness checks (error subtractions, exact sums) that failed in
 * orc_shadow_block calls so far (expected 0). */
int64_t  orc_shadow_inexact(void);

/* Both readings over whole tensors ([E][rows][cols], alpha per tensor from the tensor amax as
 * in orc_quantize; poisoned tensors are skipped), with counts of what differs. */
typedef struct {
  int64_t blocks;        /* blocks compared */
  int64_t scale_diff;    /* blocks whose chosen scale byte differs */
  int64_t choice_diff;   /* blocks whose choice between 6 and 4 differs */
  int64_t block_diff;    /* blocks with any code or scale byte that differs */
  int64_t code_diff;     /* 4-bit element codes that differ */
  int64_t y_diff;        /* fake-quant bf16 values that differ */
  int64_t exact_ties;    /* Four Over Six blocks whose two exact errors are equal */
  int64_t inexact;       /* exactness checks of the shadow's own arithmetic that failed (0) */
} orc_shadow_counts;
int      orc_shadow_compare(const uint16_t* in, int64_t E, int64_t rows, int64_t cols, int mode,
                            int rule, int exact_alpha, orc_shadow_counts* out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
