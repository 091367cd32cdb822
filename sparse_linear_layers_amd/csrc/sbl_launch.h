// Host-side launchers of the gfx950 kernels (internal to libsbl).  Each
// returns the hipError_t of its launch(es); argument validation happens in
// api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "sbl.h"

namespace sbl {

// Per-device cache of a positive host query (CU count, occupancy): slot
// `dev` holds the answer once asked; devices past the table are asked every
// time.  Lock-free: concurrent first calls may both query and store the
// same value.
constexpr int kMaxDevices = 64;
template <typename F>
inline int per_device_cached(std::atomic<int> (&cache)[kMaxDevices], int dev, F&& query) {
  if (dev < 0 || dev >= kMaxDevices) return query();
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    v = query();
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// The queries below fall back to a default when they fail and then clear the
// error they left, so that the launcher's hipGetLastError() after its launch
// reports only the launch.

// Device a launch on `stream` runs on (the current device for the null
// stream).
inline int stream_device(hipStream_t stream) {
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) == hipSuccess) return (int)d;
    (void)hipGetLastError();
  }
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) return dev;
  (void)hipGetLastError();
  return 0;
}

// Compute units of device `dev` (256, the MI355X count, if the query fails).
inline int device_cus(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  return per_device_cached(cache, dev, [dev] {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      return c;
    (void)hipGetLastError();
    return 256;
  });
}

// Resident blocks per CU of `kernel` at `threads` threads and no dynamic
// LDS, on the current device (`fallback` if the query fails).
inline int kernel_occupancy(const void* kernel, int threads, int fallback) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) == hipSuccess && occ > 0)
    return occ;
  (void)hipGetLastError();
  return fallback;
}

// Descriptors per grouped launch (their block offsets travel in the kernel
// argument block); longer lists are split into several launches.
constexpr int kMaxGroupedRefresh = 256;
constexpr int kMaxGroupedGemv = 256;

hipError_t launch_nm_mask(const float* W, int64_t rows, int64_t cols, int n, int m,
                          uint8_t* mask_bits, hipStream_t stream);
hipError_t launch_quant_pack(const float* W, const uint8_t* mask_in, int64_t rows, int64_t cols,
                             int n, int m, int fuse_mask, unsigned flags, uint8_t* mask_out,
                             uint8_t* packed, float* scale, uint16_t* scale_bf16,
                             hipStream_t stream);
hipError_t launch_quant_pack_grouped(const sbl_refresh_desc* host, const sbl_refresh_desc* dev,
                                     int count, int n, int m, unsigned flags, hipStream_t stream);
hipError_t launch_mask_stats(const uint8_t* old_bits, const uint8_t* new_bits, int64_t rows,
                             int64_t cols, int n, int m, int64_t* stats, hipStream_t stream);
hipError_t launch_packed_check(const uint8_t* packed, int64_t rows, int64_t cols, int n, int m,
                               int64_t* stats, hipStream_t stream);
hipError_t launch_rmsnorm_act_quant(const uint16_t* x, const float* w, float eps, int64_t tokens,
                                    int64_t cols, int8_t* xq, float* beta, hipStream_t stream);
hipError_t launch_act_quant(const uint16_t* x, int64_t tokens, int64_t cols, int8_t* xq,
                            float* beta, hipStream_t stream);
hipError_t launch_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                       const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N, float* y,
                       int32_t* acc, hipStream_t stream);
hipError_t launch_sparse24_compress(const uint8_t* packed, int64_t N, int64_t K, void* out,
                                    int32_t* bad_groups, hipStream_t stream);
hipError_t launch_gemm_sparse24(const int8_t* xq, const float* beta, const void* sp,
                                const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N,
                                float* y, int32_t* acc, hipStream_t stream);
size_t ste_workspace_bytes(int64_t T, int64_t K, int64_t N);
// Device address of the library's SBL_STE_SCRATCH_BYTES workspace on device
// `dev` (set up on the first call for that device).
hipError_t ste_scratch(int dev, void** out);
hipError_t launch_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                               const uint8_t* packed, const float* gamma, int64_t T, int64_t K,
                               int64_t N, float* dx, float* dw, void* workspace,
                               hipStream_t stream);
int64_t gemv_blocks(int64_t N, int64_t T);  // work units of the decode product over N rows
hipError_t launch_gemv(const sbl_gemv_desc* host, const sbl_gemv_desc* dev_or_null, int count,
                       int64_t T, hipStream_t stream);
hipError_t launch_probe_mfma_i8(int64_t iters, int blocks, int32_t* sink, hipStream_t stream);

}  // namespace sbl
