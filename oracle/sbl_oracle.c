/*
 * Plain CPU oracle for the Sparse-BitLinear forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library: everything here is written out from the method's definition
 * as the source pages state it.
 *
 * Sources (the pages are cited by title and section):
 *   [halo]  "halo-sparse-bitnet-3:4-500m — research preview" model card:
 *           "Recipe" (3:4 N:M, per-row absmean) and "Packed vs raw"
 *           (2-bit codes 00=0, 01=+1, 10=-1, four per byte; bf16 row scale).
 *   [repo]  "Sparse-BitNet" README, "How It Works": "BitLinear (1.58-bit
 *           Quantization)", "N:M Structured Sparsity", "Sparse-BitNet".
 *   [guide] "Sparse-BitNet Guide: 1.58-Bit LLMs Meet 2:4 Sparsity",
 *           "Mathematical Formulation of Sparse-BitLinear" (items 1-4: mask,
 *           absmean scale, joint sparse-ternary weight, int8 activation and
 *           the rescaled integer product) and "End-to-End Implementation"
 *           (the PyTorch module: clamp(min=1e-5) on both scales, half-to-even
 *           rounding, x * (127/beta)).
 *
 * Precision: every step is the plain definition.  Sums and the output
 * rescale are evaluated in double and rounded once to float; the two
 * decisions that turn reals into integers (the ternary code and the int8
 * activation) are taken in float, the precision the guide's module computes
 * in, one correctly rounded operation at a time.  Build with
 * -ffp-contract=off and without fast-math.
 *
 * Parity pins (which test fixes each function against something other than
 * itself) are listed in the docstring of oracle/__init__.py; no function
 * here is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_SCALE_EPS 1e-5f

/* |w| as a float.  Comparisons below use ordinary float ordering, so +0 and
 * -0 tie; inputs are finite by precondition. */
static float absf(float w) { return w < 0.0f ? -w : w; }

/* ------------------------------------------------------------------------ *
 * N:M magnitude mask.
 * [repo] "N:M Structured Sparsity": within every M consecutive elements keep
 * the N of largest magnitude.  [guide] item 1: groups are contiguous along
 * the input dimension of a row.  [halo] "Recipe": every group keeps exactly
 * N.  Equal magnitudes: the lower index wins (the pages leave ties open).
 *
 * Element j of group g is kept iff fewer than n other elements of the group
 * beat it, where k beats j when |w_k| > |w_j|, or |w_k| == |w_j| and k < j.
 * Output: bit (j % 8) of byte (row*cols + j) / 8, one bit per weight.
 * ------------------------------------------------------------------------ */
void oracle_nm_mask(const float* W, int64_t rows, int64_t cols, int n, int m,
                    uint8_t* mask_bits) {
  memset(mask_bits, 0, (size_t)((rows * cols + 7) / 8));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < cols / m; ++g) {
      const float* grp = W + r * cols + g * m;
      for (int j = 0; j < m; ++j) {
        int beaten_by = 0;
        for (int k = 0; k < m; ++k) {
          if (k == j) continue;
          float ak = absf(grp[k]), aj = absf(grp[j]);
          if (ak > aj || (ak == aj && k < j)) beaten_by++;
        }
        if (beaten_by < n) {
          int64_t bit = r * cols + g * m + j;
          /* Rows are disjoint in whole bytes only when cols % 8 == 0; the
           * atomic keeps the general case race-free. */
#pragma omp atomic
          mask_bits[bit >> 3] |= (uint8_t)(1u << (bit & 7));
        }
      }
    }
  }
}

static int mask_bit(const uint8_t* mask_bits, int64_t idx) {
  return (mask_bits[idx >> 3] >> (idx & 7)) & 1;
}

/* ------------------------------------------------------------------------ *
 * bf16 rounding of a float, round-to-nearest-even on the upper 16 bits.
 * [halo] "Packed vs raw": the stored row scale is bfloat16.
 * ------------------------------------------------------------------------ */
uint16_t oracle_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) {          /* inf / nan: truncate */
    uint16_t h = (uint16_t)(u >> 16);
    if (u & 0x007fffffu) h |= 0x0040u;              /* keep nan a nan */
    return h;
  }
  uint32_t lower = u & 0xffffu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
  return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ *
 * Per-row absmean scale.
 * [halo] "Recipe": the absmean scale is taken per row.  [guide] item 2
 * writes gamma as the mean of |W_ij| (over the whole tensor there; the model
 * card's per-row reading is the one followed).  [guide] module: the mean is
 * clamped below at 1e-5.
 *
 * gamma_i = max( float( sum_j |W_ij| / cols ), 1e-5f ), sum and division in
 * double, one rounding to float.  With from_masked != 0 the sum runs over
 * |W_ij| * mask_ij instead ([repo] "Sparse-BitNet": mask first, then
 * quantise) and is still divided by cols.
 * ------------------------------------------------------------------------ */
void oracle_row_scale(const float* W, const uint8_t* mask_bits, int from_masked,
                      int64_t rows, int64_t cols, float* gamma,
                      uint16_t* gamma_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      if (from_masked && !mask_bit(mask_bits, r * cols + j)) continue;
      s += (double)absf(W[r * cols + j]);
    }
    float g = (float)(s / (double)cols);
    if (!(g >= ORACLE_SCALE_EPS)) g = ORACLE_SCALE_EPS;
    gamma[r] = g;
    if (gamma_bf16) gamma_bf16[r] = oracle_bf16_rne(g);
  }
}

/* ------------------------------------------------------------------------ *
 * Ternary codes.
 * [guide] item 3: W~ = M (.) Clip(Round(W / gamma), -1, 1); [repo]
 * "BitLinear": round then clamp to [-1, 1].  Round is half-to-even (the
 * guide's module uses torch.round).  The division is one correctly rounded
 * float division, as in the module.  mask_bits may be NULL (dense BitNet).
 * ------------------------------------------------------------------------ */
void oracle_ternary_codes(const float* W, const uint8_t* mask_bits,
                          const float* gamma, int64_t rows, int64_t cols,
                          int8_t* codes) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < cols; ++j) {
      float q = W[r * cols + j] / gamma[r];
      float t = rintf(q);
      if (t > 1.0f) t = 1.0f;
      if (t < -1.0f) t = -1.0f;
      int8_t c = (int8_t)t;
      if (mask_bits && !mask_bit(mask_bits, r * cols + j)) c = 0;
      codes[r * cols + j] = c;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * 2-bit packing.  [halo] "Packed vs raw": four codes per byte, 00 = 0,
 * 01 = +1, 10 = -1.  Order inside the byte is not stated; the reading taken:
 * column 4b + r of a row sits in bits [2r, 2r+1] of byte b of that row.
 * ------------------------------------------------------------------------ */
void oracle_pack_codes(const int8_t* codes, int64_t rows, int64_t cols,
                       uint8_t* packed) {
  int64_t bpr = cols / 4;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < bpr; ++b) {
      unsigned byte = 0;
      for (int i = 0; i < 4; ++i) {
        int8_t c = codes[r * cols + 4 * b + i];
        unsigned f = c == 1 ? 1u : (c == -1 ? 2u : 0u);
        byte |= f << (2 * i);
      }
      packed[r * bpr + b] = (uint8_t)byte;
    }
  }
}

/* Inverse of oracle_pack_codes; the unused field 11 reads as 0. */
void oracle_unpack_codes(const uint8_t* packed, int64_t rows, int64_t cols,
                         int8_t* codes) {
  int64_t bpr = cols / 4;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < cols; ++j) {
      unsigned f = (packed[r * bpr + j / 4] >> (2 * (j % 4))) & 3u;
      codes[r * cols + j] = f == 1u ? 1 : (f == 2u ? -1 : 0);
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Packed-code validator.  [halo] "Packed vs raw": the 2-bit fields 00, 01
 * and 10 are the codes 0, +1 and -1, so 11 is no code at all; [halo]
 * "Recipe" and [repo] "N:M Structured Sparsity": under an n:m mask at most
 * n of every m consecutive weights of a row are nonzero.
 * stats[0] = number of fields equal to 11; stats[1] = number of m-groups of
 * a row holding more than n fields equal to 01 or 10.
 * ------------------------------------------------------------------------ */
void oracle_packed_check(const uint8_t* packed, int64_t rows, int64_t cols,
                         int n, int m, int64_t* stats) {
  int64_t bpr = cols / 4, not_code = 0, over_n = 0;
#pragma omp parallel for schedule(static) reduction(+ : not_code, over_n)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < cols / m; ++g) {
      int nonzero = 0;
      for (int i = 0; i < m; ++i) {
        int64_t j = g * m + i;
        unsigned f = (packed[r * bpr + j / 4] >> (2 * (j % 4))) & 3u;
        if (f == 3u) not_code++;
        else if (f != 0u) nonzero++;
      }
      if (nonzero > n) over_n++;
    }
  }
  stats[0] = not_code;
  stats[1] = over_n;
}

/* ------------------------------------------------------------------------ *
 * Per-token absmax int8 activation quantisation.
 * [guide] item 4: beta = max_j |x_j|, x~ = Clip(Round(x * 127/beta), -128, 127);
 * the module clamps beta below at 1e-5 and scales by (127/beta) computed
 * first.  Input is bfloat16 (raw bits); widening to float is exact.
 * ------------------------------------------------------------------------ */
static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void oracle_act_quant(const uint16_t* x_bf16, int64_t tokens, int64_t cols,
                      int8_t* xq, float* beta) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t) {
    float b = 0.0f;
    for (int64_t j = 0; j < cols; ++j) {
      float a = absf(bf16_to_float(x_bf16[t * cols + j]));
      if (a > b) b = a;
    }
    if (!(b >= ORACLE_SCALE_EPS)) b = ORACLE_SCALE_EPS;
    beta[t] = b;
    float s = 127.0f / b;
    for (int64_t j = 0; j < cols; ++j) {
      float v = rintf(bf16_to_float(x_bf16[t * cols + j]) * s);
      if (v > 127.0f) v = 127.0f;
      if (v < -128.0f) v = -128.0f;
      xq[t * cols + j] = (int8_t)v;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Integer product.  [guide] item 4: the output is x~ W~^T evaluated with
 * integer additions.  acc[t, o] = sum_k x~[t, k] * code[o, k], exact in
 * int32 for cols <= 2^24 / 127.
 * ------------------------------------------------------------------------ */
void oracle_gemm_acc(const int8_t* xq, const int8_t* codes, int64_t tokens,
                     int64_t cols, int64_t out_features, int32_t* acc) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t o = 0; o < out_features; ++o) {
      int32_t s = 0;
      for (int64_t k = 0; k < cols; ++k)
        s += (int32_t)xq[t * cols + k] * (int32_t)codes[o * cols + k];
      acc[t * out_features + o] = s;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Rescale.  [guide] item 4: y = (x~ W~^T) * beta * gamma / 127, here with
 * the per-token beta and per-row gamma.  Evaluated in double, rounded once
 * to float.  gamma is the value the product was given (float, or the bf16
 * row scale widened to float).
 * ------------------------------------------------------------------------ */
void oracle_dequant(const int32_t* acc, const float* beta, const float* gamma,
                    int64_t tokens, int64_t out_features, float* y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t)
    for (int64_t o = 0; o < out_features; ++o)
      y[t * out_features + o] =
          (float)((double)acc[t * out_features + o] * (double)beta[t] *
                  (double)gamma[o] / 127.0);
}

/* ------------------------------------------------------------------------ *
 * RMSNorm, then per-token absmax int8 quantisation of the normalised row.
 * [guide] item 4: the activations are normalised with RMSNorm before the
 * absmax quantisation; its module applies nn.RMSNorm(in_features) (a learned
 * per-channel weight) to x first.  The model card's model uses norm_eps
 * 1e-6 ([halo], "How to load"); eps is an argument here.
 *
 * Reading (the pages give no precision or order): with x_j the bf16 inputs
 * widened to float (exact),
 *   r   = float( 1 / sqrt(sum_j x_j^2 / cols + eps) )   every step in double
 *         (squares exact), one rounding to float at the end; r = 0 when
 *         sum/cols + eps is 0 (an all-zero row at eps = 0 then normalises to
 *         0 instead of 0 * inf).  Double keeps the mean of squares of any
 *         bf16 row in range;
 *   n_j = (x_j * r) * w_j                 two float multiplies;
 * then beta = max(max_j |n_j|, 1e-5), s = 127/beta and
 * x~_j = Clip(Round(n_j * s), -128, 127) exactly as oracle_act_quant does on
 * its input.  `normed` (nullable) receives n.
 * ------------------------------------------------------------------------ */
void oracle_rmsnorm_act_quant(const uint16_t* x_bf16, const float* weight, float eps,
                              int64_t tokens, int64_t cols, int8_t* xq, float* beta,
                              float* normed) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t) {
    const uint16_t* xr = x_bf16 + t * cols;
    double ss = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      double v = (double)bf16_to_float(xr[j]);
      ss += v * v;
    }
    double d = ss / (double)cols + (double)eps;
    float r = d > 0.0 ? (float)(1.0 / sqrt(d)) : 0.0f;
    float b = 0.0f;
    for (int64_t j = 0; j < cols; ++j) {
      float n = (bf16_to_float(xr[j]) * r) * weight[j];
      if (normed) normed[t * cols + j] = n;
      float a = absf(n);
      if (a > b) b = a;
    }
    if (!(b >= ORACLE_SCALE_EPS)) b = ORACLE_SCALE_EPS;
    beta[t] = b;
    float s = 127.0f / b;
    for (int64_t j = 0; j < cols; ++j) {
      float n = (bf16_to_float(xr[j]) * r) * weight[j];
      float v = rintf(n * s);
      if (v > 127.0f) v = 127.0f;
      if (v < -128.0f) v = -128.0f;
      xq[t * cols + j] = (int8_t)v;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Mask monitoring.  [repo] "Key Training Options": the mask change rate is
 * monitored every few steps (--sparse_mask_monitor_interval); [halo]
 * "Recipe": a mask-verify runs every 500 steps.  Reading: the change count
 * is the number of weights whose kept/dropped state differs between two
 * masks of the same matrix (the rate is that over rows*cols), and the verify
 * count is the number of M-groups of the new mask that do not keep exactly
 * N weights (the model card's "keep exactly N").  old_bits may be NULL
 * (verify only; the change count is then 0).
 * stats[0] = changed weights, stats[1] = groups not keeping exactly n.
 * ------------------------------------------------------------------------ */
void oracle_mask_stats(const uint8_t* old_bits, const uint8_t* new_bits, int64_t rows,
                       int64_t cols, int n, int m, int64_t* stats) {
  int64_t changed = 0, bad = 0;
  const int64_t total = rows * cols;
  for (int64_t i = 0; i < total; ++i)
    if (old_bits && mask_bit(old_bits, i) != mask_bit(new_bits, i)) changed++;
  for (int64_t g = 0; g < total / m; ++g) {
    int kept = 0;
    for (int j = 0; j < m; ++j) kept += mask_bit(new_bits, g * m + j);
    if (kept != n) bad++;
  }
  stats[0] = changed;
  stats[1] = bad;
}

/* ------------------------------------------------------------------------ *
 * Per-tensor absmean scale.  [guide] item 2 and its module: gamma is the
 * mean of |W| over all d_out * d_in weights, clamped below at 1e-5 (the
 * model card's per-row scale is the default elsewhere).  Sum and division
 * in double, one rounding to float; from_masked sums |W| * mask and still
 * divides by rows * cols.
 * ------------------------------------------------------------------------ */
float oracle_tensor_scale(const float* W, const uint8_t* mask_bits, int from_masked,
                          int64_t rows, int64_t cols) {
  double s = 0.0;
  for (int64_t i = 0; i < rows * cols; ++i) {
    if (from_masked && !mask_bit(mask_bits, i)) continue;
    s += (double)absf(W[i]);
  }
  float g = (float)(s / ((double)rows * (double)cols));
  if (!(g >= ORACLE_SCALE_EPS)) g = ORACLE_SCALE_EPS;
  return g;
}

/* ------------------------------------------------------------------------ *
 * Backward pass with the straight-through estimator.
 * [guide] "Training Stability & The Straight-Through Estimator": gradients
 * pass through the 2:4 mask and the ternary rounding unchanged to the
 * latent weights (dL/dW = dL/dW~); the module's backward returns the
 * gradient of the sparse ternary weight as the weight gradient.  [repo]
 * "BitLinear": gradients flow through by STE.
 *
 * With y[t,o] = acc[t,o] * beta_t * gamma_o / 127 and acc = x~ . W~^T, and
 * dy the gradient of the loss with respect to y:
 *   dw[o,k] = gamma_o * sum_t (dy[t,o] * (beta_t/127)) * x~[t,k]
 *             (the exact gradient with respect to W~, passed straight to W)
 *   dx[t,k] = sum_o (dy[t,o] * gamma_o) * code[o,k]
 *             (reading: the activation quantiser is passed straight
 *             through as well, x~ * beta / 127 standing in for x; the guide's
 *             module rounds without an estimator, which would give 0)
 * Reading of the precision: the scaled factors dy*gamma, beta/127 and
 * dy*(beta/127) are float products / quotients (one rounding each), the
 * sums are exact real sums (here double, one rounding to float), and dw's
 * final product with gamma is one float multiply.  dx or dw may be NULL.
 * ------------------------------------------------------------------------ */
void oracle_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                         const int8_t* codes, const float* gamma, int64_t T, int64_t K,
                         int64_t N, float* dx, float* dw) {
  if (dx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t k = 0; k < K; ++k) {
        double s = 0.0;
        for (int64_t o = 0; o < N; ++o) {
          int8_t c = codes[o * K + k];
          if (c == 0) continue;
          float a = dy[t * N + o] * gamma[o];
          s += c > 0 ? (double)a : -(double)a;
        }
        dx[t * K + k] = (float)s;
      }
    }
  }
  if (dw) {
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < N; ++o) {
      for (int64_t k = 0; k < K; ++k) {
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) {
          float b = dy[t * N + o] * (beta[t] / 127.0f);
          s += (double)b * (double)xq[t * K + k];
        }
        dw[o * K + k] = (float)s * gamma[o];
      }
    }
  }
}

/* Number of OpenMP threads the oracle runs with (1 when built without it). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
