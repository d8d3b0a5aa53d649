/*
 * fp4bs.h - C ABI of the block-scaled FP4 quantize + GEMM library for MI355X (gfx950).
 *
 * The library implements the data-parallel hot path of FP4 linear layers in LLM
 * pretraining: block-scaled E2M1 quantization of activations, weights and upstream
 * gradients, and the three block-scaled FP4 GEMMs (fprop, dgrad, wgrad) under the
 * probe-matched accumulation model.
 *
 * Sources (page title, section):
 *  [UE5M3]  "UE5M3 FP4 Block Scaling for Stable Language Model Pretraining": approach
 *           (접근 방법) for formats, amax cache, T, rounding, zero-scale rule, 2D weights and
 *           the GEMM model; key contributions (핵심 기여) for the 137x / 30x headroom.
 *  [MXFP4]  "技術概要：MXFP4 による大規模言語モデルの事前学習": method (手法) for the
 *           fprop / dgrad / wgrad GEMMs and the deterministic H16 / H32 Hadamard rotation.
 *  [HOPPER] "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs":
 *           methodology (방법론) for MXFP4 (E2M1, block 32) and fused transposed quantization.
 *  [FUSION] "Format-Aware Fusion for Fast FP4 Pretraining": abstract, for producers that
 *           write the consumer's layout and for fixed-sign 32-value Hadamard wgrad
 *           preconditioning.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are device pointers owned by the caller; the library allocates
 *    and frees nothing and keeps no state between calls.
 *  - Work is enqueued on ``stream`` (a hipStream_t; NULL = the null stream) and ordered on
 *    it; no call synchronises the host or copies device data to the host.
 *  - Arguments are validated before anything is enqueued; an invalid call returns a
 *    non-zero fp4_status, enqueues nothing, and sets a thread-local message readable with
 *    fp4_last_error(). A failed launch returns FP4_EHIP.
 *  - Matrices are row-major. Packed E2M1 payloads store element 2j of a row in the low
 *    nibble and 2j+1 in the high nibble of byte j (sign in bit 3 of each nibble).
 *  - Device pointers must be 16-byte aligned, except amax/g scalars (4-byte).
 *  - Calls are thread-safe; concurrent calls on different streams that write the same
 *    buffers race, as with any stream-ordered API.
 */
#ifndef FP4BS_H
#define FP4BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4BS_ABI_VERSION 3

typedef enum {
  FP4_OK = 0,
  FP4_EINVAL = 1,        /* null pointer, bad size, bad enum value */
  FP4_EUNSUPPORTED = 2,  /* valid but unsupported combination (e.g. E8M0 with block 16) */
  FP4_EALIGN = 3,        /* misaligned pointer or leading dimension */
  FP4_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
  FP4_ERANGE = 5         /* fp4_gemm_check_range: operands outside the GEMM's exact range */
} fp4_status;

/* Block-scale formats [UE5M3 approach; HOPPER methodology]. */
typedef enum {
  FP4_UE5M3 = 0,  /* unsigned E5M3, bias 15, max 61440; block 16 (main recipe) or 32 */
  FP4_E4M3 = 1,   /* E4M3 (bias 7, max 448) with an FP32 tensor scale; block 16 or 32 */
  FP4_E8M0 = 2    /* power-of-two MX scale, block 32, no tensor scale (MXFP4) */
} fp4_scale_fmt;

/* Which operand view a quantization produces. */
typedef enum {
  FP4_VIEW_ROW = 0,    /* x [rows x cols] -> operand [rows x cols], blocks along cols (fprop X, dgrad dY) */
  FP4_VIEW_COL = 1,    /* x [rows x cols] -> operand x^T [cols x rows], blocks along rows = tokens
                          (wgrad operands dY^T and X^T), optional Hadamard along rows */
  FP4_VIEW_TILE2D = 2  /* weight w [rows x cols] -> 16x16-tile scales shared by the forward
                          operand w [rows x cols] and the dgrad operand w^T [cols x rows] */
} fp4_view;

typedef enum { FP4_IN_BF16 = 0, FP4_IN_FP32 = 1 } fp4_in_dtype;

/* How an operand's scale codes map to its (row, K-block) pairs. */
typedef enum {
  FP4_SCALES_1D = 0,    /* s[row * (k/block) + kb] */
  FP4_SCALES_2D = 1,    /* forward weight view: s[(row/16) * (k/16) + kb] */
  FP4_SCALES_2D_T = 2   /* transposed weight view: s[kb * (rows/16) + row/16] */
} fp4_scale_layout;

/* Per-call quantization recipe. */
typedef struct {
  int32_t fmt;         /* fp4_scale_fmt */
  int32_t block;       /* 16 or 32 (E8M0 requires 32; TILE2D requires 16) */
  int32_t view;        /* fp4_view */
  int32_t stochastic;  /* 0: nearest-even payload; 1: stochastic rounding (ROW/COL only;
                          the recipe uses it for the upstream gradient dY only) */
  int32_t hadamard_n;  /* 0, 16 or 32: unnormalised Sylvester FWHT along tokens before
                          quantizing; COL view only [MXFP4 method; FUSION abstract] */
  float T;             /* scale target: the cached amax maps to block-scale value T
                          (448 default, 2048 override); ignored for E8M0 */
  uint64_t seed;       /* stochastic rounding: Philox-4x32-10 key */
  uint64_t offset;     /* stochastic rounding: counter words 2-3 (e.g. step*8 + view id) */
} fp4_quant_cfg;

/* A quantized GEMM operand: K-contiguous payload [rows x k/2] plus scale codes. */
typedef struct {
  const uint8_t* q;    /* device, packed E2M1 [rows x k/2] */
  const uint8_t* s;    /* device, scale codes, layout per scale_layout */
  const float* g;      /* device, tensor decode scale (1 float); NULL means 1.0. With
                          g_stripe > 0: one float per stripe of g_stripe rows */
  int32_t fmt;         /* fp4_scale_fmt */
  int32_t block;       /* 16 or 32 */
  int32_t scale_layout;/* fp4_scale_layout */
  int32_t g_stripe;    /* 0: one tensor scale; 16, 32, 64 or 128: tile-local scales, row r of
                          the operand uses g[r / g_stripe] (fp4_quantize_local; UE5M3/E4M3
                          with 1D scales only) [FUSION abstract: CTA-local NVFP4] */
  int64_t rows;        /* M (or N) */
  int64_t k;           /* contraction length; multiple of 64 */
} fp4_operand;

/* Per-operand sample-and-hold amax cache; both fields live in device memory. */
typedef struct {
  float* amax;         /* cached amax A */
  int32_t* valid;      /* 0 = empty (start or resume: the cache is not checkpointed) */
  int32_t D;           /* sample period (50 delayed, 1 current) */
} fp4_amax_cache;

/*
 * fp4_quantize - block-scaled FP4 quantization of one tensor [UE5M3 approach].
 *
 *   x        device, rows x cols elements of x_dtype, row stride ld (elements, >= cols,
 *            ld*elem_size multiple of 16 bytes)
 *   d_amax   device float: the cached amax A used for the scales (UE5M3/E4M3; may be NULL
 *            for E8M0)
 *   q        ROW/TILE2D: [rows x cols/2] bytes; COL: [cols x rows/2] bytes
 *   s        ROW: [rows x cols/B]; COL: [cols x rows/B]; TILE2D: [rows/16 x cols/16] codes
 *   q_t      TILE2D only: the transposed (dgrad) payload [cols x rows/2]; NULL otherwise
 *   d_g      device float receiving the tensor decode scale g = 1/s_enc (1 for E8M0); may be NULL
 *   d_amax_obs  optional device float receiving the observed max|x| of this tensor (after
 *            the Hadamard rotation when enabled); overwritten. A NaN anywhere in x makes it NaN
 *            (NaN propagates through every maximum the library takes, as in the float maximum)
 *   d_stats  optional device uint32[3], overwritten with the call's health counts [UE5M3 key
 *            contributions: a stale cached amax stays safe while the data grows by less than
 *            61440/T; these counts show when it does not]: [0] blocks whose unrounded scale
 *            amax_b*s_blk exceeds the format maximum (the scale saturates; always 0 for E8M0),
 *            [1] blocks whose scale encodes to zero and becomes one (E8M0: all-zero blocks),
 *            [2] blocks whose maximum is not finite (an Inf or NaN input; out of contract for
 *            the payload). A TILE2D block is a 16x16 tile.
 * Arithmetic (float32, nearest-even): s_enc = 6T/A, s_blk = T/A, g = 1/s_enc (all 1 when A
 * is 0 or not finite or 6T/A overflows); block scale S = enc(amax_b*s_blk) saturating,
 * replaced by 1 if it encodes to 0; payload E2M1(x * (s_enc/S)). E8M0: exponent
 * floor(log2 amax_b) - 2 clamped to [-127, 127], 0 for a zero block; payload E2M1(x * 2^-E).
 * Stochastic rounding draws 16 bits per element from Philox-4x32-10 with counter
 * (i>>3, offset) for logical operand index i, word (i>>1)&3, half i&1.
 * Requires: cols % B == 0 (ROW), rows % B == 0 and rows % hadamard_n == 0 (COL),
 * rows % 16 == 0 and cols % 16 == 0 (TILE2D). Empty tensors are a no-op (g is still written).
 */
fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                        const fp4_quant_cfg* cfg, const float* d_amax,
                        uint8_t* q, uint8_t* s, uint8_t* q_t, float* d_g, float* d_amax_obs,
                        uint32_t* d_stats, void* stream);

/*
 * fp4_quantize_rowcol - the ROW view and the COL view of one tensor from a single read of x
 * [FUSION abstract: the producer writes the layouts its consumers read; HOPPER methodology:
 * fused transposed quantization]. The outputs are byte-identical to two fp4_quantize calls,
 * one with cfg_row (forward operand: q, s, d_g, d_amax_obs_row) and one with cfg_col
 * (saved-for-backward operand x^T: q_t [cols x rows/2], s_t [cols x rows/B], d_g_t,
 * d_amax_obs_col).
 *   cfg_row  view FP4_VIEW_ROW, hadamard_n 0
 *   cfg_col  view FP4_VIEW_COL; same fmt and block as cfg_row; its own T, stochastic flag,
 *            seed/offset and hadamard_n (0, 16, 32)
 *   d_amax_row, d_amax_col  device floats: each view's cached amax (UE5M3/E4M3; may be NULL
 *            for E8M0). With a Hadamard rotation the COL view's amax is that of the rotated
 *            tensor, so the two usually differ.
 *   d_g, d_g_t, d_amax_obs_row, d_amax_obs_col  optional device float outputs, as in
 *            fp4_quantize
 *   d_stats_row, d_stats_col  optional device uint32[3] health counts of each view, as in
 *            fp4_quantize
 * Requires the shape conditions of both views: cols % B == 0, rows % B == 0 and
 * rows % hadamard_n == 0; also ld * elem_size <= 2^24 bytes, rows <= 2^24 and cols <= 2^25
 * (FP4_EUNSUPPORTED otherwise). Empty tensors are a no-op (g values are still written).
 */
fp4_status fp4_quantize_rowcol(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                               const fp4_quant_cfg* cfg_row, const fp4_quant_cfg* cfg_col,
                               const float* d_amax_row, const float* d_amax_col,
                               uint8_t* q, uint8_t* s, float* d_g, float* d_amax_obs_row,
                               uint8_t* q_t, uint8_t* s_t, float* d_g_t, float* d_amax_obs_col,
                               uint32_t* d_stats_row, uint32_t* d_stats_col, void* stream);

/*
 * fp4_fake_quant - inference fake quantization: y = the decoded value of x's FP4 ROW-view
 * quantization, x_hat = E2M1(q) * S * g (g = 1 for E8M0), in one pass [UE5M3 approach,
 * training and inference setup: held-out likelihoods with FP4 fake quantization under a
 * delayed D=50, current D=1 or frozen activation-scale policy; the policy only decides
 * which cached amax d_amax holds for the call].
 *   x, x_dtype, rows, cols, ld   as in fp4_quantize
 *   cfg      view FP4_VIEW_ROW, stochastic 0, hadamard_n 0; fmt, block and T as in
 *            fp4_quantize
 *   d_amax   device float, the cached amax (UE5M3/E4M3; may be NULL for E8M0)
 *   y        device, rows x cols of y_dtype (FP4_IN_FP32 or FP4_IN_BF16), row stride ldy
 *            elements (>= cols, ldy * elem_size a multiple of 16 bytes and <= 2^24)
 * Arithmetic: the codes and scales are exactly those fp4_quantize writes; E2M1(q) * S is
 * exact in float32 and the product with g is one float32 multiply (nearest-even); bfloat16
 * output rounds that float32 to nearest-even. Requires cols % B == 0.
 */
fp4_status fp4_fake_quant(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                          const fp4_quant_cfg* cfg, const float* d_amax, void* y, int32_t y_dtype, int64_t ldy,
                          void* stream);

/*
 * fp4_dequantize - decode a quantized operand (any scale layout) to y [rows x k] of y_dtype
 * (FP4_IN_FP32 or FP4_IN_BF16), row stride ldy: y = E2M1(q) * S * g with the arithmetic of
 * fp4_fake_quant [UE5M3 approach]. For a TILE2D weight, the forward operand gives W and the
 * transposed operand W^T. The operand's g may be NULL (1.0).
 */
fp4_status fp4_dequantize(const fp4_operand* a, void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * fp4_mxfp4_to_fp8 - direct MXFP4 -> FP8 E4M3 conversion with hierarchical scale alignment
 * [HOPPER methodology: FP4 -> FP8 without a BF16 intermediate, block 32 -> block 128 scale
 * alignment, transpose fused with the conversion].
 *   a          MXFP4 operand (E8M0, block 32, FP4_SCALES_1D), rows x k, k % 128 == 0
 *   transpose  0: y is [rows x k] E4M3 bytes; 1: y is [k x rows] (rows % 16 == 0)
 *   y          device, rows * k bytes, 16-byte aligned
 *   s8         device, [rows x k/128] E8M0 chunk scale codes: the chunk's FP8 values times
 *              2^(code - 127) are its real values
 * Arithmetic: chunk code c = e_max - min(6, e_max) over the chunk's four block codes; each
 * element becomes E4M3(E2M1(q) * 2^(e_b - c)), nearest-even with subnormals and the sign
 * kept (|y| <= 384). Exact whenever e_max - e_b <= 14; smaller blocks round on E4M3's
 * subnormal grid. rows, k <= 2^23.
 */
fp4_status fp4_mxfp4_to_fp8(const fp4_operand* a, int32_t transpose, uint8_t* y, uint8_t* s8, void* stream);

/*
 * fp4_quantize_local - ROW-view quantization with tile-local tensor scales [FUSION abstract:
 * cooperative-thread-array-local NVFP4 scale domain]: the rows are cut into stripes of
 * 2^k = stripe rows (16, 32, 64 or 128; the last may be shorter), each spanning all cols; a
 * stripe's tensor scales come from its own amax (current scaling, no cached amax and no
 * global pass) with the fp4_quantize arithmetic and cfg->T; codes and scales are laid out
 * as for FP4_VIEW_ROW.
 *   cfg      view FP4_VIEW_ROW, fmt FP4_UE5M3 or FP4_E4M3, block 16 or 32, hadamard_n 0;
 *            stochastic rounding allowed
 *   q, s     as fp4_quantize ROW
 *   d_g      device float[ceil(rows / stripe)]: each stripe's decode scale g
 *   d_amax_obs  optional device float[ceil(rows / stripe)]: each stripe's amax
 * The GEMMs take the result as an operand with g = d_g and g_stripe = stripe.
 */
fp4_status fp4_quantize_local(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                              const fp4_quant_cfg* cfg, int32_t stripe, uint8_t* q, uint8_t* s, float* d_g,
                              float* d_amax_obs, void* stream);

/* fp4_quantize_sizes - byte sizes of q, s and q_t for a call with these arguments (host only). */
fp4_status fp4_quantize_sizes(int64_t rows, int64_t cols, const fp4_quant_cfg* cfg,
                              size_t* q_bytes, size_t* s_bytes, size_t* qt_bytes);

/*
 * fp4_tensor_amax - d_amax_out = max|x| over rows x cols, after the blockwise FWHT along rows
 * when hadamard_n is 16 or 32 (the amax that a COL-view quantization with that rotation
 * sees). Overwrites *d_amax_out. [UE5M3 approach: per-operand amax sampled every D steps]
 */
fp4_status fp4_tensor_amax(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                           int32_t hadamard_n, float* d_amax_out, void* stream);

/*
 * amax_cache_update - sample-and-hold [UE5M3 approach]: if the cache is empty or
 * step % D == 0, A <- *d_amax_obs and the cache becomes valid; otherwise A is held.
 * The decision is taken on the device (the host need not know the valid flag).
 */
fp4_status amax_cache_update(const fp4_amax_cache* cache, int64_t step, const float* d_amax_obs, void* stream);

/* amax_cache_reset - mark the cache empty (a resumed run samples on first use). */
fp4_status amax_cache_reset(const fp4_amax_cache* cache, void* stream);

/*
 * The three GEMMs [UE5M3 approach, GEMM model; MXFP4 method]. Each computes
 * C[M x N] = A[M x K] . B[N x K]^T into row-major float32 c (ldc = N) from two operands
 * with the same fmt and block, K % 64 == 0:
 *   for every 64-product group: block partials T_b = S_a S_b sum(q_a q_b) are exact; the
 *   group's partials are added in K order in float32 with round-to-nearest-even; groups
 *   are accumulated in K order with float32 round-toward-zero; optionally the result is
 *   canonicalised to round_half_even(1024 c)/1024 (canon != 0); finally
 *   c = acc * float32(g_a * g_b) [* 1/hadamard_n for wgrad], rounded to nearest-even; with
 *   tile-local operands g_a = a->g[m / a->g_stripe], g_b = b->g[n / b->g_stripe].
 * Exact results require every block partial and group sum to stay inside the float32
 * normal range (always true for UE5M3/E4M3; for E8M0, combined block exponents Ea + Eb in
 * [-124, 116], which fp4_scale_range + fp4_gemm_check_range verify). K = 0 writes +0 to every
 * output (an empty sum).
 *
 * fp4_gemm_fprop: Y = X . W^T. x: ROW-view activation (1D scales); w: weight forward view
 *                 (TILE2D q with FP4_SCALES_2D, or a ROW-view weight with 1D scales).
 * fp4_gemm_dgrad: dX = dY . W. dy: ROW-view upstream gradient; wt: the weight's transposed
 *                 payload q_t with FP4_SCALES_2D_T (or any 1D-scaled [N x K] operand).
 * fp4_gemm_wgrad: dW = dY^T . X. dyt, xt: COL-view operands (1D scales along tokens);
 *                 hadamard_n (0/16/32) must match the rotation used to quantize both.
 */
fp4_status fp4_gemm_fprop(const fp4_operand* x, const fp4_operand* w, float* y, int32_t canon, void* stream);
fp4_status fp4_gemm_dgrad(const fp4_operand* dy, const fp4_operand* wt, float* dx, int32_t canon, void* stream);
fp4_status fp4_gemm_wgrad(const fp4_operand* dyt, const fp4_operand* xt, float* dw, int32_t hadamard_n,
                          int32_t canon, void* stream);

/*
 * fp4_gemm_fprop_q / fp4_gemm_dgrad_q - fprop / dgrad whose epilogue also writes C as the next
 * GEMM's quantized ROW-view operand [FUSION abstract: the producer emits the FP4 payload,
 * scales and layout its consumer reads, instead of a float32 round trip through HBM; HOPPER
 * methodology: FP4 copies kept in the consumer's format]. Y = X . W^T feeds the next layer's
 * fprop; dX = dY . W feeds the previous layer's dgrad (stochastic rounding, as for dY).
 *   x, w / dy, wt, canon  as in fp4_gemm_fprop / fp4_gemm_dgrad
 *   y / dx    float32 [M x N] output as before, or NULL to write only the quantized operand
 *             (0.5 + 1/B bytes per output element instead of 4)
 *   out_cfg   recipe of the output operand: view FP4_VIEW_ROW, hadamard_n 0, any fmt / block /
 *             T / stochastic / seed / offset of fp4_quantize
 *   d_amax_out  device float: the output operand's cached amax (delayed scaling: known before
 *             the GEMM runs); may be NULL for E8M0
 *   q, s      device [M x N/2] payload and [M x N/B] scale codes, as fp4_quantize ROW writes
 *   d_g, d_amax_obs, d_stats  optional, as in fp4_quantize: g, the observed max|C| (for the
 *             cache's next sample) and the health counts of the output operand
 * q, s and g are byte-identical to fp4_quantize(ROW) applied to the float32 C that y holds
 * (the SR counter is the element's index in C [M x N]). Requires N % B == 0 and K > 0.
 */
fp4_status fp4_gemm_fprop_q(const fp4_operand* x, const fp4_operand* w, float* y, int32_t canon,
                            const fp4_quant_cfg* out_cfg, const float* d_amax_out, uint8_t* q, uint8_t* s, float* d_g,
                            float* d_amax_obs, uint32_t* d_stats, void* stream);
fp4_status fp4_gemm_dgrad_q(const fp4_operand* dy, const fp4_operand* wt, float* dx, int32_t canon,
                            const fp4_quant_cfg* out_cfg, const float* d_amax_out, uint8_t* q, uint8_t* s, float* d_g,
                            float* d_amax_obs, uint32_t* d_stats, void* stream);

/*
 * fp4_decode_f16 - the operand a (UE5M3 or E4M3, any scale layout) decoded to fp16 [rows x K],
 * K-contiguous: out[r][k] = E2M1(q[r][k]) * S(r, k) * 2^-3, exactly (S is the block scale
 * value, without the tensor factor g; every such value has at most 6 significant bits and lies
 * in [2^-21, 46080], so fp16, subnormals included, holds it exactly) [UE5M3 approach: the
 * software GEMM model; UE5M3 limits: no native UE5M3 hardware, hence an exact software route].
 *   out  device, 16-byte aligned, 2 * rows * K bytes, caller-owned.
 * Returns FP4_EUNSUPPORTED for E8M0 operands (the MXFP4 GEMM reads FP4 natively).
 *
 * fp4_gemm_f16 - C = A . B^T for UE5M3/E4M3 operands a [M x K] and b [N x K] whose fp16
 * decodes (fp4_decode_f16) are a16 and b16: the same group model, rounding and epilogue as
 * fp4_gemm_fprop / _dgrad / _wgrad on the same operands (hadamard_n as in fp4_gemm_wgrad, 0
 * otherwise), bit for bit, from a kernel that reads the decoded values instead of decoding
 * each operand tile in every workgroup that uses it. a and b supply format, block, sizes and g
 * (their q and s are not read). c as in the other GEMMs.
 */
fp4_status fp4_decode_f16(const fp4_operand* a, void* out, void* stream);
fp4_status fp4_gemm_f16(const fp4_operand* a, const void* a16, const fp4_operand* b, const void* b16, float* c,
                        int32_t hadamard_n, int32_t canon, void* stream);

/*
 * fp4_scale_range - d_range[0] = smallest and d_range[1] = largest scale code of operand a
 * (device int32[2], overwritten; 255 and 0 for an empty operand). Reads the scale codes only
 * (1/64 of the payload bytes for MXFP4). Together with fp4_gemm_check_range it is the checked
 * mode of the MXFP4 GEMMs.
 *
 * fp4_gemm_check_range - host-only check that a GEMM between operands of format fmt whose
 * scale codes lie in range_a / range_b (host int32[2], e.g. copied from fp4_scale_range) stays
 * exact under the GEMM model [UE5M3 approach, GEMM model; MXFP4 method]. MXFP4 block partials
 * 2^(Ea+Eb) * sum(q_a q_b) have nonzero magnitudes in [0.25, 1152] * 2^(Ea+Eb) and group sums
 * below 2304 * 2^(Ea+Eb); every one stays a normal float32 (the kernels' exactness condition)
 * iff -124 <= Ea + Eb <= 116 for every block pair, i.e. min_a + min_b >= 130 and
 * max_a + max_b <= 370 in codes. Returns FP4_OK inside, FP4_ERANGE outside (with the range
 * in fp4_last_error). UE5M3 / E4M3 partials are always inside: FP4_OK. Launches nothing.
 */
fp4_status fp4_scale_range(const fp4_operand* a, int32_t* d_range, void* stream);
fp4_status fp4_gemm_check_range(int32_t fmt, const int32_t* range_a, const int32_t* range_b);

/*
 * fp4_debug_encode - runs the device encoders on n float32 inputs, for parity tests only.
 *   which 0: E2M1 nearest-even payload code of x (one byte per input, sign in bit 3)
 *   which 1: UE5M3 scale code of x (x >= 0), nearest-even, saturating (no zero rule)
 *   which 2: E4M3 scale code of x (x >= 0), nearest-even, saturating (no zero rule)
 *   which 3: E8M0 block exponent code of x (x >= 0) as used for a block maximum
 *   which 4: stochastic E2M1 code of x with 16-bit draw u16[i] (u16 required)
 */
fp4_status fp4_debug_encode(const float* x, const uint16_t* u16, int64_t n, int32_t which, uint8_t* out,
                            void* stream);

/* Thread-local description of the last error on this thread ("" if none). */
const char* fp4_last_error(void);

/* FP4BS_ABI_VERSION of the loaded library. */
int32_t fp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4BS_H */
