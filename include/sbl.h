/*
 * sbl.h — C ABI of the Sparse-BitLinear forward path for AMD Instinct MI355X
 * (gfx950).  libsbl.so implements every function declared here with
 * hand-written HIP kernels.
 *
 * The operator (Sparse-BitLinear, W1.58A8 with N:M structured sparsity):
 *   mask   keep the n largest |w| of every m contiguous input-dim weights
 *          ("Sparse-BitNet" README, "How It Works" / "N:M Structured
 *          Sparsity"; "Sparse-BitNet Guide", "Mathematical Formulation of
 *          Sparse-BitLinear", step 1);
 *   gamma  per-row mean |w| ("halo-sparse-bitnet-3:4-500m" model card,
 *          "Recipe"; guide step 2), clamped below at 1e-5 (guide,
 *          "End-to-End Implementation");
 *   codes  Clip(Round(w / gamma), -1, 1) (.) mask (guide step 3; README
 *          "BitLinear (1.58-bit Quantization)"), packed 2 bits per weight
 *          (model card, "Packed vs raw");
 *   x~     per-token absmax int8, x~ = Clip(Round(x * 127/beta), -128, 127)
 *          (guide step 4);
 *   y      (x~ . codes^T) * beta * gamma / 127 with an int32 accumulator
 *          (guide step 4, "linear output").
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer owned by the caller (for example the
 *     data_ptr() of a PyTorch tensor) unless its comment says "host".
 *     The library allocates nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous; outputs are valid once the stream reaches the call.
 *     Calls enqueued on one stream run in order; calls that overlap on
 *     different streams and share an output race.
 *   - Arguments are validated before anything is enqueued: a call that
 *     returns an error has written nothing.  Nothing is printed and nothing
 *     aborts.
 *   - Matrices are dense row-major with no padding between rows.  A weight
 *     matrix is [rows = out_features, cols = in_features] (the Linear
 *     convention of the guide, "Mathematical Formulation"); activations are
 *     [tokens, in_features].
 *   - cols (= K, in_features) must be a positive multiple of 64; row and
 *     token counts may be any value >= 0 (0 is a no-op).  Base pointers must
 *     be 16-byte aligned.
 *   - Inputs are finite by precondition; NaN and infinities give
 *     deterministic but unspecified results.
 *
 * Layouts
 *   mask bits : uint8 [rows*cols/8]; weight (r, j) is bit (j % 8) of byte
 *               (r*cols + j) / 8.
 *   packed    : uint8 [rows, cols/4]; weight (r, j) is the 2-bit field at
 *               bits [2*(j%4), 2*(j%4)+1] of byte (r, j/4); 00 = 0,
 *               01 = +1, 10 = -1.  11 is never written and reads as 0.
 *   row scale : float [rows], and optionally its bfloat16 copy (round to
 *               nearest even) as uint16 bits [rows] — the model card's
 *               NAME.row_scale.
 *   x         : bfloat16 bits, uint16 [tokens, cols].
 *   x~, beta  : int8 [tokens, cols] and float [tokens].
 *   y, acc    : float / int32 [tokens, rows].
 */
#ifndef SBL_H_
#define SBL_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define SBL_OK 0
#define SBL_ERR_ARG (-1)         /* null pointer where one is required, negative size */
#define SBL_ERR_SHAPE (-2)       /* cols not a positive multiple of 64, or too large   */
#define SBL_ERR_ALIGN (-3)       /* a base pointer is not 16-byte aligned              */
#define SBL_ERR_UNSUPPORTED (-4) /* (n, m) or option outside what is implemented       */
#define SBL_ERR_HIP (-5)         /* the HIP runtime reported an error at launch        */
#define SBL_ERR_TOO_LARGE (-6)   /* needs more than the library's fixed scratch holds  */

/* Largest cols (K) accepted: keeps |acc| <= 127*K well inside int32 and the
 * per-row work of the weight kernels bounded. */
#define SBL_MAX_COLS 65536

/* Flags of ternary_quant_pack / nm_mask_quant_pack. */
#define SBL_SCALE_FROM_MASKED 1u /* gamma = sum(|w| * mask) / cols instead of sum(|w|) / cols */
#define SBL_SCALE_PER_TENSOR 2u  /* one gamma for the whole matrix (guide "Mathematical
                                    Formulation", step 2, and its module): mean |w| over
                                    rows*cols, written into every row_scale entry; W is read
                                    twice and `packed` holds per-row partial sums in between.
                                    Not accepted by nm_mask_quant_pack_grouped. */

/* Row-scale dtype selector of the products. */
#define SBL_SCALE_F32 0
#define SBL_SCALE_BF16 1

/* Text for a status code (static storage, never NULL). */
const char* sbl_status_str(int status);

/* ------------------------------------------------------------------------
 * N:M magnitude mask.
 * README "N:M Structured Sparsity"; guide "Mathematical Formulation", step 1;
 * model card "Recipe" (every group keeps exactly n).
 * In every group of m consecutive weights of a row, set the bits of the n
 * weights of largest |w|; among equal magnitudes the lower index wins.
 *   W         float [rows, cols]
 *   n, m      m in {4, 8}, 0 <= n <= m
 *   mask_bits uint8 [rows*cols/8] (written completely)
 * ------------------------------------------------------------------------ */
int nm_mask_create(const float* W, int64_t rows, int64_t cols, int n, int m,
                   uint8_t* mask_bits, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-row absmean ternary quantisation and 2-bit packing.
 * Model card "Recipe" (per-row absmean) and "Packed vs raw" (layout);
 * guide "Mathematical Formulation", steps 2-3; README "Sparse-BitNet".
 *   gamma_r  = max(mean_j |W_rj|, 1e-5), the mean rounded once to float
 *              (sum of |w| * mask_rj with SBL_SCALE_FROM_MASKED; the mean over
 *              the whole matrix, the same in every row, with
 *              SBL_SCALE_PER_TENSOR);
 *   code_rj  = Clip(Round(W_rj / gamma_r), -1, 1), 0 where the mask bit is
 *              0 (Round = half to even).
 *   mask_bits   uint8 [rows*cols/8] or NULL (dense BitNet: every weight
 *               kept; SBL_SCALE_FROM_MASKED then needs a mask)
 *   packed      uint8 [rows, cols/4]
 *   row_scale   float [rows]
 *   row_scale_bf16  uint16 [rows] or NULL
 * ------------------------------------------------------------------------ */
int ternary_quant_pack(const float* W, const uint8_t* mask_bits, int64_t rows,
                       int64_t cols, unsigned flags, uint8_t* packed,
                       float* row_scale, uint16_t* row_scale_bf16,
                       hipStream_t stream);

/* Mask creation and quantisation in one pass over W (the mask never
 * round-trips through memory).  Same results as nm_mask_create followed by
 * ternary_quant_pack.  mask_bits may be NULL when the caller does not need
 * the mask. */
int nm_mask_quant_pack(const float* W, int64_t rows, int64_t cols, int n, int m,
                       unsigned flags, uint8_t* mask_bits, uint8_t* packed,
                       float* row_scale, uint16_t* row_scale_bf16,
                       hipStream_t stream);

/* One launch of nm_mask_quant_pack over several weight matrices (for
 * example every linear of a model).  `descs_host` and `descs_dev` hold the
 * same `count` descriptors, in host and in device memory; the host copy is
 * validated and sized, the device copy is read by the kernel and must stay
 * valid until the stream reaches the call. */
typedef struct sbl_refresh_desc {
  const float* W;            /* float [rows, cols]                 */
  uint8_t* mask_bits;        /* uint8 [rows*cols/8] or NULL        */
  uint8_t* packed;           /* uint8 [rows, cols/4]               */
  float* row_scale;          /* float [rows]                       */
  uint16_t* row_scale_bf16;  /* uint16 [rows] or NULL              */
  int64_t rows;
  int64_t cols;
} sbl_refresh_desc;

int nm_mask_quant_pack_grouped(const sbl_refresh_desc* descs_host,
                               const sbl_refresh_desc* descs_dev, int count,
                               int n, int m, unsigned flags, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token absmax int8 activation quantisation (W1.58A8).
 * Guide "Mathematical Formulation", step 4, and its module in
 * "End-to-End Implementation"; "BitNet TinyDialogues 1.58b", "O que é".
 *   beta_t = max(max_j |x_tj|, 1e-5);  s_t = 127 / beta_t (one correctly
 *   rounded float division);  x~_tj = Clip(Round(x_tj * s_t), -128, 127)
 *   (float multiply, half-to-even).  |x~| <= 127 always holds.
 *   x_bf16 uint16 [tokens, cols];  xq int8 [tokens, cols];  beta float [tokens]
 * ------------------------------------------------------------------------ */
int act_quant_i8(const uint16_t* x_bf16, int64_t tokens, int64_t cols,
                 int8_t* xq, float* beta, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RMSNorm, then per-token absmax int8 quantisation, in one pass over x.
 * Guide "Mathematical Formulation", step 4 (activations are normalised with
 * RMSNorm before the absmax quantisation) and its module in "End-to-End
 * Implementation" (nn.RMSNorm with a per-channel weight in front of the
 * absmax step); the model card's model uses norm_eps 1e-6.
 *   r_t    = float(1 / sqrt(sum_j x_tj^2 / cols + eps))   (exact squares,
 *            every step in double, one rounding to float; 0 when the
 *            root's argument is 0)
 *   n_tj   = (x_tj * r_t) * norm_weight_j    (two float multiplies)
 *   then beta_t, x~_tj from n as in act_quant_i8.
 *   x_bf16 uint16 [tokens, cols];  norm_weight float [cols];  eps >= 0
 *   xq int8 [tokens, cols];  beta float [tokens]
 * Errors: SBL_ERR_ARG also for a negative or non-finite eps.
 * ------------------------------------------------------------------------ */
int rmsnorm_act_quant_i8(const uint16_t* x_bf16, const float* norm_weight, float eps,
                         int64_t tokens, int64_t cols, int8_t* xq, float* beta,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Mask monitoring: change count between two masks and a verify count.
 * README "Key Training Options" (the mask change rate is monitored every
 * few steps); model card "Recipe" (mask-verify; every group keeps exactly
 * n).
 *   stats[0] = number of weights whose bit differs between old_bits and
 *              new_bits (0 when old_bits is NULL); the change rate is
 *              stats[0] / (rows*cols)
 *   stats[1] = number of m-groups of new_bits that do not hold exactly n
 *              set bits
 *   old_bits, new_bits  uint8 [rows*cols/8] (layout of nm_mask_create);
 *                       old_bits may be NULL (and new_bits too when rows
 *                       is 0: the counts are then zeroed)
 *   stats               int64 [2], device memory; overwritten (zeroed by the
 *                       call itself before counting)
 * ------------------------------------------------------------------------ */
int nm_mask_stats(const uint8_t* old_bits, const uint8_t* new_bits, int64_t rows,
                  int64_t cols, int n, int m, int64_t* stats, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Packed-code validator.
 * Model card "Packed vs raw": a weight is stored as one of the 2-bit codes
 * 00 (0), 01 (+1), 10 (-1), so the field 11 never occurs in a valid matrix;
 * model card "Recipe" and README "N:M Structured Sparsity": under an n:m
 * mask every group of m consecutive weights of a row holds at most n
 * nonzeros (codes may add zeros inside the kept positions).
 *   stats[0] = number of 2-bit fields equal to 11 (the products read them
 *              as 0)
 *   stats[1] = number of m-groups of a row with more than n codes 01 or 10
 *   packed  uint8 [rows, cols/4] (layout of ternary_quant_pack); may be
 *           NULL when rows is 0 (the counts are then zeroed)
 *   n, m    m in {4, 8}, 0 <= n <= m
 *   stats   int64 [2], device memory, 8-byte aligned; overwritten (zeroed by
 *           the call itself before counting)
 * ------------------------------------------------------------------------ */
int packed_codes_check(const uint8_t* packed, int64_t rows, int64_t cols, int n, int m,
                       int64_t* stats, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Packed-ternary x int8 product, prefill (dense int8 matrix cores).
 * Guide "Mathematical Formulation", step 4 (integer product, rescale).
 *   acc[t, o] = sum_k xq[t, k] * code[o, k]   (int32, exact)
 *   y[t, o]   = acc[t, o] * beta[t] * gamma[o] / 127   (float; within
 *               1e-6 relative of the exactly rounded value)
 *   xq     int8 [T, K];  beta float [T]
 *   packed uint8 [N, K/4];  row_scale float [N] (SBL_SCALE_F32) or bf16
 *          bits uint16 [N] (SBL_SCALE_BF16)
 *   y      float [T, N]
 *   acc    int32 [T, N] or NULL (exact integer accumulators, for checking)
 * ------------------------------------------------------------------------ */
int sparse_bitlinear_gemm(const int8_t* xq, const float* beta,
                          const uint8_t* packed, const void* row_scale,
                          int scale_dtype, int64_t T, int64_t K, int64_t N,
                          float* y, int32_t* acc, hipStream_t stream);

/* ------------------------------------------------------------------------
 * 2:4 variant on gfx950 sparse int8 matrix cores (smfmac).
 * Guide "The Hardware Mechanics of 2:4 Sparsity": a 2:4 weight is carried
 * as its kept values plus 2-bit in-group indices.  Here the weights are
 * first compressed from the packed codes into a private operand image of
 * sparse24_bytes(N, K) bytes; the product then gives the same acc and y as
 * sparse_bitlinear_gemm on the packed codes.
 * sparse24_compress: every group of 4 codes must hold at most 2 nonzeros
 * (true for a 2:4 mask); each group that holds more is counted into
 * *bad_groups (int32 device counter, may be NULL; the caller zeroes it) and
 * compressed with its first two nonzeros only.
 * ------------------------------------------------------------------------ */
size_t sparse24_bytes(int64_t N, int64_t K);
int sparse24_compress(const uint8_t* packed, int64_t N, int64_t K, void* sparse24,
                      int32_t* bad_groups, hipStream_t stream);
int sparse_bitlinear_gemm_sparse24(const int8_t* xq, const float* beta,
                                   const void* sparse24, const void* row_scale,
                                   int scale_dtype, int64_t T, int64_t K,
                                   int64_t N, float* y, int32_t* acc,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode product (GEMV), 1 <= T <= 16 tokens; same contract as
 * sparse_bitlinear_gemm, including the optional int32 accumulators.
 * Model card "What does NOT ship" (the serve path needs a kernel that reads
 * the packed layout directly).  One token with K <= 8192 streams on the
 * vector ALU (int8 dot products); other cases run on the int8 matrix cores;
 * both give the same exact acc and y.
 * Errors: SBL_ERR_UNSUPPORTED for T outside [1, 16]; SBL_ERR_SHAPE for
 * N > SBL_GEMV_MAX_ROWS.
 * ------------------------------------------------------------------------ */
#define SBL_GEMV_MAX_TOKENS 16
#define SBL_GEMV_MAX_ROWS (1 << 28)
int sparse_bitlinear_gemv(const int8_t* xq, const float* beta,
                          const uint8_t* packed, const void* row_scale,
                          int scale_dtype, int64_t T, int64_t K, int64_t N,
                          float* y, int32_t* acc, hipStream_t stream);

/* Many decode products in one launch (for example every linear of every
 * layer).  Host and device copies of the same descriptors, as for
 * nm_mask_quant_pack_grouped.  All share the token count T. */
typedef struct sbl_gemv_desc {
  const int8_t* xq;       /* int8 [T, K]                          */
  const float* beta;      /* float [T]                            */
  const uint8_t* packed;  /* uint8 [N, K/4]                       */
  const void* row_scale;  /* float or bf16 [N], per scale_dtype   */
  float* y;               /* float [T, N]                         */
  int32_t* acc;           /* int32 [T, N] or NULL                 */
  int64_t K;
  int64_t N;
  int32_t scale_dtype;    /* SBL_SCALE_F32 or SBL_SCALE_BF16      */
  int32_t reserved;       /* must be 0                            */
} sbl_gemv_desc;

int sparse_bitlinear_gemv_grouped(const sbl_gemv_desc* descs_host,
                                  const sbl_gemv_desc* descs_dev, int count,
                                  int64_t T, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward pass with the straight-through estimator (training).
 * Guide "Training Stability & The Straight-Through Estimator" (the gradient
 * passes through the mask and the ternary rounding to the latent weights)
 * and its module's backward; README "BitLinear" (gradients flow through by
 * STE).  With dy = dL/dy [T, N] of y = acc * beta * gamma / 127:
 *   dw[o,k] = gamma_o * sum_t (dy[t,o] * (beta_t/127)) * x~[t,k]
 *             (dL/dW~, passed straight to the latent weight W)
 *   dx[t,k] = sum_o (dy[t,o] * gamma_o) * code[o,k]
 *             (the activation quantiser passed straight through:
 *             x~ * beta/127 stands for x)
 * dy*gamma, beta/127 and dy*(beta/127) are float operations; the sums are
 * accumulated in float on bf16 matrix cores from an exact three-piece bf16
 * split of the float factor (every product exact).  A matrix-core step adds
 * 16 exact products of one piece to the accumulator, three steps per 16
 * terms; dw adds at most 32 partial sums in a fixed order and then rounds
 * the product with gamma.  With one rounding per step, each entry is within
 * (3R/16 + 36) * 2^-24 * sum|terms| of the exact sum (R the reduction
 * length: N for dx, T for dw).
 *   dy       float [T, N]
 *   xq, beta int8 [T, K], float [T]            (needed for dw)
 *   packed   uint8 [N, K/4]                    (needed for dx)
 *   row_scale float [N]
 *   dx       float [T, K] or NULL;  dw  float [N, K] or NULL
 *   workspace  16-byte aligned device memory of at least
 *              sparse_bitlinear_ste_workspace_bytes(T, K, N) bytes when dw is
 *              requested (it holds beta/127 per token and, when the token
 *              reduction of dw is split across the GPU, the partial sums,
 *              added afterwards in a fixed order); NULL when that size is 0
 *              or dw is NULL.  Its contents on entry do not matter.
 * An empty reduction (N = 0 for dx, T = 0 for dw) writes zeros; the
 * operands it would read may then be NULL.
 * Errors: SBL_ERR_ARG also for a workspace smaller than required;
 * SBL_ERR_SHAPE for N > 2^22 or K outside the column limits.
 * ------------------------------------------------------------------------ */
size_t sparse_bitlinear_ste_workspace_bytes(int64_t T, int64_t K, int64_t N);
int sparse_bitlinear_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                                  const uint8_t* packed, const float* row_scale, int64_t T,
                                  int64_t K, int64_t N, float* dx, float* dw, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or training loops, harnesses
 * that forbid hipMalloc).  Same contract and the same results, bit for bit,
 * as sparse_bitlinear_ste_backward, without a workspace argument: the
 * workspace is a device array owned by the library, SBL_STE_SCRATCH_BYTES
 * per GPU, which comes with the library's code object and is held until the
 * process ends.  The call itself allocates nothing.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (different streams) race.  The array keeps the last call's contents; a
 * call writes every byte of it that it reads.
 * Errors: as sparse_bitlinear_ste_backward; SBL_ERR_TOO_LARGE when dw is
 * requested and sparse_bitlinear_ste_workspace_bytes(T, K, N) exceeds
 * SBL_STE_SCRATCH_BYTES (the 0.5B skeleton's linears at 32768 tokens need
 * at most 53 MB); SBL_ERR_HIP when the array's device address cannot be
 * obtained.
 * ------------------------------------------------------------------------ */
#define SBL_STE_SCRATCH_BYTES ((size_t)64 << 20)
int sparse_bitlinear_ste_backward_noalloc(const float* dy, const int8_t* xq, const float* beta,
                                          const uint8_t* packed, const float* row_scale,
                                          int64_t T, int64_t K, int64_t N, float* dx, float* dw,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement probe (not part of the operator): the int8 matrix-core rate
 * the device sustains, for the benchmark's roofline beside the datasheet
 * peak.  `blocks` blocks of 4 waves; every wave runs 4 independent chains
 * of `iters` v_mfma_i32_32x32x32_i8 with no memory traffic, i.e.
 * blocks * 4 * 4 * iters * 65536 int8 operations.  The caller times the
 * launch on `stream`.
 *   sink  int32 [blocks * 4] device memory (overwritten)
 * Errors: SBL_ERR_ARG for iters < 1, blocks < 1 or a NULL sink.
 * ------------------------------------------------------------------------ */
int sbl_probe_mfma_i8(int64_t iters, int blocks, int32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SBL_H_ */
