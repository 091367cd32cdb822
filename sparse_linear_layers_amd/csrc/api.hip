// extern "C" entry points of libsbl (declared in include/sbl.h): argument
// validation, then one launch on the caller's stream.  Validation finishes
// before anything is enqueued, so a call that fails writes nothing.
#include <stdint.h>

#include "sbl.h"
#include "sbl_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned16_or_null(const void* p) { return p == nullptr || aligned16(p); }

// cols: positive multiple of 64, at most SBL_MAX_COLS.
int check_cols(int64_t cols) {
  if (cols <= 0 || cols % 64 != 0 || cols > SBL_MAX_COLS) return SBL_ERR_SHAPE;
  return SBL_OK;
}

int check_nm(int n, int m) {
  if (m != 4 && m != 8) return SBL_ERR_UNSUPPORTED;
  if (n < 0 || n > m) return SBL_ERR_UNSUPPORTED;
  return SBL_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SBL_OK : SBL_ERR_HIP; }

// Row counts: any value >= 0 whose grid fits the launch limits.
constexpr int64_t kMaxRows = int64_t(1) << 30;

}  // namespace

extern "C" {

const char* sbl_status_str(int status) {
  switch (status) {
    case SBL_OK: return "ok";
    case SBL_ERR_ARG: return "invalid argument (null pointer or negative size)";
    case SBL_ERR_SHAPE: return "unsupported shape (cols must be a positive multiple of 64, at most 65536)";
    case SBL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SBL_ERR_UNSUPPORTED: return "unsupported option (n, m, flags, scale dtype or token count)";
    case SBL_ERR_HIP: return "HIP runtime error at launch";
    case SBL_ERR_TOO_LARGE: return "problem needs more than the library's fixed scratch (SBL_STE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int nm_mask_create(const float* W, int64_t rows, int64_t cols, int n, int m, uint8_t* mask_bits,
                   hipStream_t stream) {
  if (rows < 0 || rows > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (int s = check_nm(n, m)) return s;
  if (rows == 0) return SBL_OK;
  if (!W || !mask_bits) return SBL_ERR_ARG;
  if (!aligned16(W) || !aligned16(mask_bits)) return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_nm_mask(W, rows, cols, n, m, mask_bits, stream));
}

int ternary_quant_pack(const float* W, const uint8_t* mask_bits, int64_t rows, int64_t cols,
                       unsigned flags, uint8_t* packed, float* row_scale, uint16_t* row_scale_bf16,
                       hipStream_t stream) {
  if (rows < 0 || rows > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (flags & ~(SBL_SCALE_FROM_MASKED | SBL_SCALE_PER_TENSOR)) return SBL_ERR_UNSUPPORTED;
  if (rows == 0) return SBL_OK;
  if (!W || !packed || !row_scale) return SBL_ERR_ARG;
  if ((flags & SBL_SCALE_FROM_MASKED) && !mask_bits) return SBL_ERR_ARG;
  if (!aligned16(W) || !aligned16_or_null(mask_bits) || !aligned16(packed) ||
      !aligned16(row_scale) || !aligned16_or_null(row_scale_bf16))
    return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_quant_pack(W, mask_bits, rows, cols, 0, 4, 0, flags, nullptr,
                                           packed, row_scale, row_scale_bf16, stream));
}

int nm_mask_quant_pack(const float* W, int64_t rows, int64_t cols, int n, int m, unsigned flags,
                       uint8_t* mask_bits, uint8_t* packed, float* row_scale,
                       uint16_t* row_scale_bf16, hipStream_t stream) {
  if (rows < 0 || rows > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (int s = check_nm(n, m)) return s;
  if (flags & ~(SBL_SCALE_FROM_MASKED | SBL_SCALE_PER_TENSOR)) return SBL_ERR_UNSUPPORTED;
  if (rows == 0) return SBL_OK;
  if (!W || !packed || !row_scale) return SBL_ERR_ARG;
  if (!aligned16(W) || !aligned16_or_null(mask_bits) || !aligned16(packed) ||
      !aligned16(row_scale) || !aligned16_or_null(row_scale_bf16))
    return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_quant_pack(W, nullptr, rows, cols, n, m, 1, flags, mask_bits,
                                           packed, row_scale, row_scale_bf16, stream));
}

int nm_mask_quant_pack_grouped(const sbl_refresh_desc* descs_host,
                               const sbl_refresh_desc* descs_dev, int count, int n, int m,
                               unsigned flags, hipStream_t stream) {
  if (count < 0) return SBL_ERR_ARG;
  if (count == 0) return SBL_OK;
  if (!descs_host || !descs_dev) return SBL_ERR_ARG;
  if (int s = check_nm(n, m)) return s;
  if (flags & ~SBL_SCALE_FROM_MASKED) return SBL_ERR_UNSUPPORTED;
  int64_t total_blocks = 0;
  for (int i = 0; i < count; ++i) {
    const sbl_refresh_desc& d = descs_host[i];
    if (d.rows < 0 || d.rows > kMaxRows) return SBL_ERR_ARG;
    if (int s = check_cols(d.cols)) return s;
    if (d.rows == 0) continue;
    if (!d.W || !d.packed || !d.row_scale) return SBL_ERR_ARG;
    if (!aligned16(d.W) || !aligned16_or_null(d.mask_bits) || !aligned16(d.packed) ||
        !aligned16(d.row_scale) || !aligned16_or_null(d.row_scale_bf16))
      return SBL_ERR_ALIGN;
    // rows of 2049..32768 columns take a block each, shorter ones a wave
    const int64_t need = (d.cols / 4 + 63) / 64;
    total_blocks += need > 8 && need <= 128 ? d.rows : (d.rows + 3) / 4;
  }
  if (total_blocks > INT32_MAX / 2) return SBL_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(sbl::launch_quant_pack_grouped(descs_host, descs_dev, count, n, m, flags, stream));
}

int rmsnorm_act_quant_i8(const uint16_t* x_bf16, const float* norm_weight, float eps,
                         int64_t tokens, int64_t cols, int8_t* xq, float* beta,
                         hipStream_t stream) {
  if (tokens < 0 || tokens > kMaxRows) return SBL_ERR_ARG;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return SBL_ERR_ARG;  // rejects NaN and inf
  if (int s = check_cols(cols)) return s;
  if (tokens == 0) return SBL_OK;
  if (!x_bf16 || !norm_weight || !xq || !beta) return SBL_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(norm_weight) || !aligned16(xq) || !aligned16(beta))
    return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_rmsnorm_act_quant(x_bf16, norm_weight, eps, tokens, cols, xq, beta,
                                                  stream));
}

int nm_mask_stats(const uint8_t* old_bits, const uint8_t* new_bits, int64_t rows, int64_t cols,
                  int n, int m, int64_t* stats, hipStream_t stream) {
  if (rows < 0 || rows > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (int s = check_nm(n, m)) return s;
  if (!stats || (rows > 0 && !new_bits)) return SBL_ERR_ARG;
  if (!aligned16_or_null(old_bits) || !aligned16(new_bits) || (reinterpret_cast<uintptr_t>(stats) & 7u))
    return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_mask_stats(old_bits, new_bits, rows, cols, n, m, stats, stream));
}

int packed_codes_check(const uint8_t* packed, int64_t rows, int64_t cols, int n, int m,
                       int64_t* stats, hipStream_t stream) {
  if (rows < 0 || rows > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (int s = check_nm(n, m)) return s;
  if (!stats || (rows > 0 && !packed)) return SBL_ERR_ARG;
  if (!aligned16_or_null(packed) || (reinterpret_cast<uintptr_t>(stats) & 7u)) return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_packed_check(packed, rows, cols, n, m, stats, stream));
}

int act_quant_i8(const uint16_t* x_bf16, int64_t tokens, int64_t cols, int8_t* xq, float* beta,
                 hipStream_t stream) {
  if (tokens < 0 || tokens > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(cols)) return s;
  if (tokens == 0) return SBL_OK;
  if (!x_bf16 || !xq || !beta) return SBL_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(xq) || !aligned16(beta)) return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_act_quant(x_bf16, tokens, cols, xq, beta, stream));
}

static int check_product(const int8_t* xq, const float* beta, const void* w, const void* scale,
                         int scale_dtype, int64_t T, int64_t K, int64_t N, const float* y,
                         const int32_t* acc) {
  if (T < 0 || N < 0 || T > kMaxRows || N > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(K)) return s;
  if (scale_dtype != SBL_SCALE_F32 && scale_dtype != SBL_SCALE_BF16) return SBL_ERR_UNSUPPORTED;
  if (T == 0 || N == 0) return SBL_OK;  // empty: no pointer is dereferenced
  if (!xq || !beta || !w || !scale || !y) return SBL_ERR_ARG;
  if (!aligned16(xq) || !aligned16(beta) || !aligned16(w) || !aligned16(scale) || !aligned16(y) ||
      !aligned16_or_null(acc))
    return SBL_ERR_ALIGN;
  return SBL_OK;
}

int sparse_bitlinear_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                          const void* row_scale, int scale_dtype, int64_t T, int64_t K, int64_t N,
                          float* y, int32_t* acc, hipStream_t stream) {
  if (int s = check_product(xq, beta, packed, row_scale, scale_dtype, T, K, N, y, acc)) return s;
  if (T == 0 || N == 0) return SBL_OK;
  (void)hipGetLastError();
  return hip_status(sbl::launch_gemm(xq, beta, packed, row_scale, scale_dtype == SBL_SCALE_BF16, T,
                                     K, N, y, acc, stream));
}

size_t sparse24_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return (size_t)N * (size_t)K / 4;
}

int sparse24_compress(const uint8_t* packed, int64_t N, int64_t K, void* sparse24,
                      int32_t* bad_groups, hipStream_t stream) {
  if (N < 0 || N > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(K)) return s;
  if (N == 0) return SBL_OK;
  if (!packed || !sparse24) return SBL_ERR_ARG;
  if (!aligned16(packed) || !aligned16(sparse24) ||
      (bad_groups && (reinterpret_cast<uintptr_t>(bad_groups) & 3u)))
    return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_sparse24_compress(packed, N, K, sparse24, bad_groups, stream));
}

int sparse_bitlinear_gemm_sparse24(const int8_t* xq, const float* beta, const void* sparse24,
                                   const void* row_scale, int scale_dtype, int64_t T, int64_t K,
                                   int64_t N, float* y, int32_t* acc, hipStream_t stream) {
  if (int s = check_product(xq, beta, sparse24, row_scale, scale_dtype, T, K, N, y, acc)) return s;
  if (T == 0 || N == 0) return SBL_OK;
  (void)hipGetLastError();
  return hip_status(sbl::launch_gemm_sparse24(xq, beta, sparse24, row_scale,
                                              scale_dtype == SBL_SCALE_BF16, T, K, N, y, acc,
                                              stream));
}

int sparse_bitlinear_gemv(const int8_t* xq, const float* beta, const uint8_t* packed,
                          const void* row_scale, int scale_dtype, int64_t T, int64_t K, int64_t N,
                          float* y, int32_t* acc, hipStream_t stream) {
  if (T < 1 || T > SBL_GEMV_MAX_TOKENS) return SBL_ERR_UNSUPPORTED;
  if (int s = check_product(xq, beta, packed, row_scale, scale_dtype, T, K, N, y, acc)) return s;
  if (N > SBL_GEMV_MAX_ROWS) return SBL_ERR_SHAPE;
  if (N == 0) return SBL_OK;
  sbl_gemv_desc d{xq, beta, packed, row_scale, y, acc, K, N, scale_dtype, 0};
  (void)hipGetLastError();
  return hip_status(sbl::launch_gemv(&d, nullptr, 1, T, stream));
}

int sparse_bitlinear_gemv_grouped(const sbl_gemv_desc* descs_host, const sbl_gemv_desc* descs_dev,
                                  int count, int64_t T, hipStream_t stream) {
  if (count < 0) return SBL_ERR_ARG;
  if (count == 0) return SBL_OK;
  if (!descs_host || !descs_dev) return SBL_ERR_ARG;
  if (T < 1 || T > SBL_GEMV_MAX_TOKENS) return SBL_ERR_UNSUPPORTED;
  int64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    const sbl_gemv_desc& d = descs_host[i];
    if (int s = check_product(d.xq, d.beta, d.packed, d.row_scale, d.scale_dtype, T, d.K, d.N, d.y,
                              d.acc))
      return s;
    if (d.N > SBL_GEMV_MAX_ROWS) return SBL_ERR_SHAPE;
    if (d.reserved != 0) return SBL_ERR_ARG;
    blocks += sbl::gemv_blocks(d.N, T);
  }
  if (blocks > INT32_MAX / 2) return SBL_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(sbl::launch_gemv(descs_host, descs_dev, count, T, stream));
}

size_t sparse_bitlinear_ste_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  if (T <= 0 || N <= 0 || check_cols(K) != SBL_OK) return 0;
  return sbl::ste_workspace_bytes(T, K, N);
}

// Checks of the backward's arguments other than its workspace; on success
// *dx_out / *dw_out are the outputs to compute (NULL when empty) and *need
// the workspace bytes.
static int check_ste(const float* dy, const int8_t* xq, const float* beta, const uint8_t* packed,
                     const float* row_scale, int64_t T, int64_t K, int64_t N, float** dx_out,
                     float** dw_out, size_t* need) {
  if (T < 0 || N < 0 || T > kMaxRows || N > kMaxRows) return SBL_ERR_ARG;
  if (int s = check_cols(K)) return s;
  if (N > (int64_t(1) << 22)) return SBL_ERR_SHAPE;  // 32-bit per-lane offsets into dy tiles
  float* dx = T == 0 ? nullptr : *dx_out;            // empty outputs
  float* dw = N == 0 ? nullptr : *dw_out;
  *dx_out = dx;
  *dw_out = dw;
  *need = 0;
  if (!dx && !dw) return SBL_OK;
  const bool reads = T > 0 && N > 0;  // otherwise the reduction is empty: zeros
  if (reads && !dy) return SBL_ERR_ARG;
  if (N > 0 && !row_scale) return SBL_ERR_ARG;
  if (dx && reads && !packed) return SBL_ERR_ARG;
  if (dw && reads && (!xq || !beta)) return SBL_ERR_ARG;
  if (!aligned16_or_null(dy) || !aligned16_or_null(row_scale) || !aligned16_or_null(xq) ||
      !aligned16_or_null(beta) || !aligned16_or_null(packed) || !aligned16_or_null(dx) ||
      !aligned16_or_null(dw))
    return SBL_ERR_ALIGN;
  *need = dw ? sbl::ste_workspace_bytes(T, K, N) : 0;
  return SBL_OK;
}

int sparse_bitlinear_ste_backward_noalloc(const float* dy, const int8_t* xq, const float* beta,
                                          const uint8_t* packed, const float* row_scale,
                                          int64_t T, int64_t K, int64_t N, float* dx, float* dw,
                                          hipStream_t stream) {
  size_t need = 0;
  if (int s = check_ste(dy, xq, beta, packed, row_scale, T, K, N, &dx, &dw, &need)) return s;
  if (!dx && !dw) return SBL_OK;
  if (need > SBL_STE_SCRATCH_BYTES) return SBL_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0 && sbl::ste_scratch(sbl::stream_device(stream), &ws) != hipSuccess) {
    (void)hipGetLastError();
    return SBL_ERR_HIP;
  }
  (void)hipGetLastError();
  return hip_status(sbl::launch_ste_backward(dy, xq, beta, packed, row_scale, T, K, N, dx, dw, ws,
                                             stream));
}

int sparse_bitlinear_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                                  const uint8_t* packed, const float* row_scale, int64_t T,
                                  int64_t K, int64_t N, float* dx, float* dw, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  if (int s = check_ste(dy, xq, beta, packed, row_scale, T, K, N, &dx, &dw, &need)) return s;
  if (!dx && !dw) return SBL_OK;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SBL_ERR_ARG;
  if (need > 0 && !aligned16(workspace)) return SBL_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(sbl::launch_ste_backward(dy, xq, beta, packed, row_scale, T, K, N, dx, dw,
                                             need > 0 ? workspace : nullptr, stream));
}

int sbl_probe_mfma_i8(int64_t iters, int blocks, int32_t* sink, hipStream_t stream) {
  if (iters < 1 || blocks < 1 || !sink) return SBL_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(sbl::launch_probe_mfma_i8(iters, blocks, sink, stream));
}

}  // extern "C"
