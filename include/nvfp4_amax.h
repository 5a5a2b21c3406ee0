/*
 * nvfp4_amax -- NVFP4 block-scaled quantization of bf16 tensors on AMD Instinct MI355X
 * (gfx950): standard NVFP4 ("rtn6") and Four Over Six ("4/6") adaptive block scaling,
 * as a packed quantizer and as a simulated-quantization (quantize-dequantize) op.
 *
 * What is computed (sources cited by page title and section):
 *   - Elements are FP4 E2M1 codes with values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and a sign
 *     ("Four Over Six: More Accurate NVFP4 Quantization with Adaptive Block Scaling",
 *     gist.science explainer, "Problem definition").
 *   - One FP8 E4M3 scale per block of 16 consecutive elements ("Quantization-Aware
 *     Distillation for NVFP4 Inference Accuracy Recovery", gist.science explainer, key
 *     findings item 3; Four Over Six explainer, "Implementation details").
 *   - One FP32 scale alpha per tensor, from the tensor's absolute maximum amax:
 *     alpha = amax / (6 * 448) for standard NVFP4, amax / (6 * 256) for Four Over Six,
 *     because blocks scaled to 4 need a 1.5x larger E4M3 scale (Four Over Six explainer,
 *     "Implementation details").
 *   - rtn6 scales every block so its max maps to 6.  Four Over Six quantizes each block
 *     twice, with its max mapped to 6 and to 4, measures both errors against the original
 *     values, and keeps the smaller under the chosen rule: MSE, MAE or max error (Four
 *     Over Six explainer, "Method / core mechanism", "Adaptive block scaling algorithm").
 *     Ties keep 6.  A block scaled to 4 never uses FP4 values above 4.
 *   - Simulated quantization returns the dequantized values in bf16, as a QAD student
 *     forward uses them (Nemotron 3.5 Lightning NVFP4 news page, "two-stage QAD").
 *
 * Arithmetic: IEEE binary32 round-to-nearest-even steps, fixed order; the outputs are
 * bit-identical to the CPU oracle that ships with the tests.  In short, per tensor
 * alpha = RN(amax / C); per block, for each candidate Q: s = E4M3(RN(bmax / RN(Q*alpha)))
 * (RNE, saturating at 448), d = RN(dec(s) * alpha), v_i = RN(x_i * RN(1/d)) (RN(x_i / d)
 * when 1/d overflows), code_i = min(E2M1_RNE(|v_i|), Q), xhat_i = RN(val(code_i) * d),
 * error accumulated over i = 0..15 in order (fma for MSE).
 *
 * Layouts (all row-major, blocks run along the last, contiguous dimension):
 *   in        [E][rows][cols]     bf16 bit patterns (uint16), cols % 16 == 0
 *   codes     [E][rows][cols/2]   uint8: element 2j in bits 0-3, element 2j+1 in bits 4-7;
 *                                 code = sign << 3 | magnitude (E2M1: e1 e0 m, bias 1)
 *   scales    [E][rows][cols/16]  uint8 E4M3FN (bias 7; 0x7E = 448; no swizzle)
 *   alpha     [E]                 float32
 *   out       [E][rows][cols]     bf16 (fake-quant)
 * E = 1 for the non-batched calls.
 *
 * Ownership and ordering: every pointer is a device pointer owned by the caller.  The
 * library allocates nothing.  Its only process-wide state is the wait limit of the
 * single-read calls (a test setting) and per-device caches of device figures (occupancy and
 * wall-clock rate) and of the allocation-free call's scratch address, all read
 * and written atomically; calls are reentrant.  All work is
 * enqueued on `stream` (0 = the null stream) and the call returns at once; outputs are
 * defined once the stream passes the call.  During a dynamic-scale call out_alpha holds
 * the running amax, so it must not alias any other argument.  Fake-quant may run in
 * place (out == in); any other overlap between arguments is rejected.
 *
 * Errors: argument errors are returned before anything is enqueued and leave the outputs
 * untouched.  NVFP4_ERR_HIP reports a failed kernel launch.  Device faults surface at the
 * caller's next synchronization.  Non-finite input is not an error: it poisons that
 * tensor's outputs (alpha = NaN 0x7FC00000, every scale 0x7F, every code byte 0x00,
 * every fake-quant value 0x7FC0).
 */
#ifndef NVFP4_AMAX_H
#define NVFP4_AMAX_H

#include <stdint.h>
/* The library targets AMD GPUs only.  A plain C or C++ compiler (not hipcc) including this
 * header gets the AMD platform of the HIP runtime API without having to define it. */
#if !defined(__HIP_PLATFORM_AMD__) && !defined(__HIP_PLATFORM_NVIDIA__)
#define __HIP_PLATFORM_AMD__ 1
#endif
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 5
#define NVFP4_BLOCK 16

typedef enum { NVFP4_RTN6 = 0, NVFP4_FOUR_OVER_SIX = 1 } nvfp4_mode;

/* Four Over Six selection rule (ignored by rtn6 but still validated). */
typedef enum { NVFP4_RULE_MSE = 0, NVFP4_RULE_MAE = 1, NVFP4_RULE_MAXERR = 2 } nvfp4_rule;

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,   /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,  /* E, rows or cols <= 0, cols % 16 != 0, E > 65535, size overflow */
  NVFP4_ERR_BLOCK = 3,  /* block != 16 */
  NVFP4_ERR_ENUM = 4,   /* mode or rule out of range */
  NVFP4_ERR_ALIGN = 5,  /* in/out/codes not 16-byte aligned, alpha/amax not 4-byte */
  NVFP4_ERR_HIP = 6,    /* a kernel launch failed */
  NVFP4_ERR_ALIAS = 7,  /* overlapping arguments (other than in-place fake-quant); added
                           after the first six, so it takes the next free number */
  NVFP4_ERR_SCRATCH = 8 /* nvfp4_quantize_fused_noalloc: E > NVFP4_NOALLOC_MAX_TENSORS */
} nvfp4_status;

/* ABI version (NVFP4_ABI_VERSION) and a static description of a status code. */
int nvfp4_abi_version(void);
const char* nvfp4_status_str(nvfp4_status status);

/* Tensor amax: out_amax[e] = max |x| over tensor e of [E][rows][cols], exact (a max of
 * bf16 magnitudes); +Inf or NaN when the tensor holds one (NaN wins).  The reduction
 * that alpha is computed from (Four Over Six explainer, "Implementation details").
 * Launches: a clear of out_amax, then one streaming pass. */
nvfp4_status nvfp4_amax(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                        float* out_amax, hipStream_t stream);

/* Packed NVFP4 quantization with a dynamic per-tensor scale.  Each block of 16 values gets
 * one E4M3 scale and 16 FP4 codes; under Four Over Six each block is quantized twice, with
 * its max mapped to 6 and to 4, and the candidate with the smaller error (rule: MSE, MAE or
 * max error, against the original values) is kept (Four Over Six explainer, "Method / core
 * mechanism" and "Adaptive block scaling algorithm"; the per-tensor scale with 448 or 256,
 * "Implementation details").  Launches: amax pass, then the block pass (both candidates and
 * the selection in registers), then alpha is written.
 * out_codes [rows][cols/2], out_scales [rows][cols/16], out_alpha [1]. */
nvfp4_status nvfp4_quantize(const uint16_t* in, int64_t rows, int64_t cols, int block,
                            nvfp4_mode mode, nvfp4_rule rule, uint8_t* out_codes,
                            uint8_t* out_scales, float* out_alpha, hipStream_t stream);

/* Simulated quantization: out = bf16(dequantize(quantize(in))), bit-identical to decoding
 * the packed result of nvfp4_quantize.  The QAD student forward runs through this op
 * (Nemotron 3.5 Lightning NVFP4 news page, "two-stage QAD"; the Model Optimizer blog's QAD
 * section); the encoding is the one of nvfp4_quantize.  out may equal in.  out [rows][cols]
 * bf16, out_alpha [1]. */
nvfp4_status nvfp4_fakequant(const uint16_t* in, int64_t rows, int64_t cols, int block,
                             nvfp4_mode mode, nvfp4_rule rule, uint16_t* out,
                             float* out_alpha, hipStream_t stream);

/* E independent tensors [E][rows][cols] in one launch per pass, one alpha per tensor: the
 * per-tensor scale of the Four Over Six explainer ("Implementation details") taken per
 * tensor of the batch, e.g. per expert of a mixture-of-experts layer (the Model Optimizer
 * blog quantizes an MoE model).  Outputs as above with a leading [E]; out_alpha [E]. */
nvfp4_status nvfp4_quantize_batched(const uint16_t* in, int64_t E, int64_t rows,
                                    int64_t cols, int block, nvfp4_mode mode,
                                    nvfp4_rule rule, uint8_t* out_codes,
                                    uint8_t* out_scales, float* out_alpha,
                                    hipStream_t stream);
nvfp4_status nvfp4_fakequant_batched(const uint16_t* in, int64_t E, int64_t rows,
                                     int64_t cols, int block, nvfp4_mode mode,
                                     nvfp4_rule rule, uint16_t* out, float* out_alpha,
                                     hipStream_t stream);

/* Fixed (static) scale: the caller supplies amax[E] (device memory, e.g. from a
 * calibration or from nvfp4_amax) and the amax pass is skipped; alpha is derived from it
 * exactly as in the dynamic calls (the Nemotron 3.5 Lightning NVFP4 news page offers
 * dynamic and fixed scale settings, "workflow" paragraph).  Values beyond the supplied
 * amax saturate: block scales clamp at 448, FP4 values at 6 (4 for blocks scaled to 4).
 * nvfp4_amax followed by these calls is bit-identical to the dynamic calls.
 * A non-finite amax poisons the tensor's outputs. */
nvfp4_status nvfp4_quantize_from_amax(const uint16_t* in, int64_t E, int64_t rows,
                                      int64_t cols, int block, nvfp4_mode mode,
                                      nvfp4_rule rule, const float* amax,
                                      uint8_t* out_codes, uint8_t* out_scales,
                                      float* out_alpha, hipStream_t stream);
nvfp4_status nvfp4_fakequant_from_amax(const uint16_t* in, int64_t E, int64_t rows,
                                       int64_t cols, int block, nvfp4_mode mode,
                                       nvfp4_rule rule, const float* amax, uint16_t* out,
                                       float* out_alpha, hipStream_t stream);

/* Columns of the per-tensor error statistics of nvfp4_quantize_diag (out_stats[E][6]). */
enum {
  NVFP4_STAT_SSE = 0,           /* sum of e^2 over the tensor, e = x - xhat of the chosen code */
  NVFP4_STAT_SAE = 1,           /* sum of |e| */
  NVFP4_STAT_MAXERR = 2,        /* max |e| (exact) */
  NVFP4_STAT_SSE_NEAR = 3,      /* sum of e^2 over the elements with |x| > (2/3) * block max */
  NVFP4_STAT_SSE_F32SCALE = 4,  /* sum of e^2 if each block's chosen candidate kept its
                                   binary32 scale sigma instead of the E4M3 byte */
  NVFP4_STAT_NEAR_COUNT = 5,    /* number of elements with |x| > (2/3) * block max (exact) */
  NVFP4_NSTATS = 6
};

/* Diagnostics of a packed quantization (dynamic scale, E tensors): the outputs of
 * nvfp4_quantize_batched plus
 *   - per block, the block maximum it was scaled to (out_qstar [E][rows][cols/16]: 4 or 6,
 *     always 6 for rtn6, 0 for a poisoned tensor);
 *   - per tensor, the number of blocks scaled to 4 (out_count4 [E], cleared by the call);
 *   - optionally (out_stats may be NULL), per tensor, the error statistics NVFP4_STAT_*
 *     (out_stats [E][6] binary64, 8-byte aligned, cleared by the call; NaN for a poisoned
 *     tensor).  They need stats_workspace: device memory of NVFP4_DIAG_WS_WORDS(E) uint32,
 *     128-byte aligned, owned by the caller, any content (the call clears what it uses),
 *     not shared with a call that may overlap this one; ignored (may be NULL) without
 *     out_stats.  Each workgroup leaves its partial sums there, and the last one of each
 *     tensor adds them up.
 * The Four Over Six explainer expects blocks with large near-max values to pick 4 ("Key
 * contributions and results"), and reports that rounding the block scales to FP8 costs
 * little while rounding the values between 66.6 % and 100 % of the block max drives the
 * error ("Problem definition"): out_count4, NVFP4_STAT_SSE_NEAR and the gap between
 * NVFP4_STAT_SSE and NVFP4_STAT_SSE_F32SCALE measure these on a given tensor.  The maximum
 * and the count are exact; the sums are binary64, within (n - 1) * 2^-53 of the exact sum
 * relative to it (n = elements per tensor), and their summation order is fixed by the shape
 * alone, so repeated calls give the same bits.  Errors as for the other calls, plus
 * NVFP4_ERR_NULL for a null qstar, count4 or (with out_stats) stats_workspace,
 * NVFP4_ERR_ALIGN and NVFP4_ERR_ALIAS for those arrays. */
#define NVFP4_DIAG_WS_WORDS(E) \
  (32 * (int64_t)(E) + 12 * ((int64_t)(E) > 1024 ? (int64_t)(E) : (int64_t)1024))
nvfp4_status nvfp4_quantize_diag(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                                 int block, nvfp4_mode mode, nvfp4_rule rule,
                                 uint8_t* out_codes, uint8_t* out_scales, float* out_alpha,
                                 uint8_t* out_qstar, uint32_t* out_count4, double* out_stats,
                                 uint32_t* stats_workspace, hipStream_t stream);

/* Single-read dynamic quantization: the outputs of nvfp4_quantize_batched /
 * nvfp4_fakequant_batched, bit for bit, reading the input from HBM once instead of twice.
 * Because alpha depends on the whole tensor, the dynamic entry points above read every input
 * twice (the amax pass, then the block pass).  Here each workgroup keeps its blocks on chip
 * (VGPRs and LDS) while the tensor amax is reduced across the grid, then quantizes what it
 * holds; the Four Over Six explainer ("Implementation details") keeps every intermediate value
 * in registers, and this extends that across the amax dependency.
 *   workspace  device memory of E * NVFP4_FUSED_WS_WORDS uint32 (2176 bytes per tensor,
 *              128-byte aligned) owned by the caller; any content (the call clears it first).  Calls
 *              that share a workspace must not overlap (calls on one stream never do).
 * Tensors whose blocks do not fit on chip (see nvfp4_fused_single_read), and in-place
 * fake-quant (out == in), take the two-pass path instead, with the same results; the
 * workspace is then unused.  All workgroups of a
 * single-read launch must be resident together; the grid is sized for that from the
 * device's occupancy.  Their wait for each other is bounded in time by the work: 8 times the
 * launch's expected load time (the bytes loaded at once, at 4 TB/s) plus 50 us, on the
 * device's constant-rate wall clock.  A workgroup that waits longer (for instance while other
 * kernels hold the CUs) computes the tensor amax itself from the input, so the call always
 * completes with the same result, at the cost of that extra read.  Two fused calls that run
 * concurrently (different streams or graph branches) can each leave part of their workgroups
 * unplaced and then take that slow path.  Errors as above, plus
 * NVFP4_ERR_NULL for a null workspace and NVFP4_ERR_ALIAS when it overlaps another argument. */
#define NVFP4_FUSED_WS_WORDS 544   /* workspace words per tensor of the fused calls */
nvfp4_status nvfp4_quantize_fused(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                                  int block, nvfp4_mode mode, nvfp4_rule rule,
                                  uint8_t* out_codes, uint8_t* out_scales, float* out_alpha,
                                  uint32_t* workspace, hipStream_t stream);
nvfp4_status nvfp4_fakequant_fused(const uint16_t* in, int64_t E, int64_t rows, int64_t cols,
                                   int block, nvfp4_mode mode, nvfp4_rule rule, uint16_t* out,
                                   float* out_alpha, uint32_t* workspace, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): nvfp4_quantize_fused without the workspace
 * argument.  The grid-wide wait's counters live in a static device array of the library
 * (NVFP4_NOALLOC_MAX_TENSORS * NVFP4_FUSED_WS_WORDS words, 2.1 MiB, one copy per GPU, held
 * until the process ends); the call allocates nothing, and at its first call on a device it
 * looks up the array's address there.  Every call on one GPU shares that array, so calls that
 * may overlap on one GPU (different streams, graph branches) race and must not be issued;
 * calls in order on one stream are fine (each clears what it uses first).  Results, paths and
 * errors as nvfp4_quantize_fused, plus NVFP4_ERR_SCRATCH for E > NVFP4_NOALLOC_MAX_TENSORS
 * (returned before anything is enqueued). */
#define NVFP4_NOALLOC_MAX_TENSORS 1024
nvfp4_status nvfp4_quantize_fused_noalloc(const uint16_t* in, int64_t E, int64_t rows,
                                          int64_t cols, int block, nvfp4_mode mode,
                                          nvfp4_rule rule, uint8_t* out_codes,
                                          uint8_t* out_scales, float* out_alpha,
                                          hipStream_t stream);

/* For a fused call of this shape, mode, rule and output form on the current device: the
 * most blocks a lane holds on chip (1, 4 or 12 in workgroups of 256 threads, 10 or 14 in
 * workgroups of 1024 threads, or 28; a tensor spread over more workgroups leaves each lane
 * fewer) if it reads its input once, 0 if it takes the two-pass path, or minus a status code
 * for bad arguments.  On MI355X up to 3,670,016 blocks per launch (E * rows * cols / 16; 117 MB
 * of bf16) are held at once, in every mode.  A larger batch whose single tensors fit (up to
 * 2,621,440 blocks each) is read once too, by teams of workgroups that take its tensors in
 * turn: the call then returns 20, or 10 for tensors under 262,144 blocks, or 10 or 13 for
 * Four Over Six into packed output. */
int nvfp4_fused_single_read(int64_t E, int64_t rows, int64_t cols, nvfp4_mode mode,
                            nvfp4_rule rule, int fakequant);

/* Test hook (process-wide, the library's only setting): at most how many times a workgroup
 * of a single-read launch polls for the other workgroups before it computes the tensor amax
 * itself; the time bound above applies as well.  0 = never wait; a negative value restores
 * the default (2^26 polls, so that the time bound governs); larger values are capped at 2^26. */
void nvfp4_fused_set_wait_limit(int64_t polls);

/* Dequantize packed NVFP4 to bf16 (for W4A16-style consumers that store 4-bit weights; the
 * Nemotron 3.5 Lightning NVFP4 news page, "two-stage QAD", quantizes the student to W4A16):
 *   out = bf16(RN(val(code) * RN(dec(scale) * alpha[e])))
 * which is bit-identical to the fake-quant output of the tensor that produced the codes.
 * codes [E][rows][cols/2] (8-byte aligned), scales [E][rows][cols/16], alpha [E] (device),
 * out [E][rows][cols] bf16 (16-byte aligned).  A NaN alpha or a NaN scale byte (0x7F, 0xFF)
 * gives 0x7FC0 for the whole block.  One launch. */
nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* alpha,
                              int64_t E, int64_t rows, int64_t cols, uint16_t* out,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_AMAX_H */
