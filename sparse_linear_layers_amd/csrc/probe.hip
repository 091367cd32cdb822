// Measurement probe: the int8 matrix-core rate this device sustains, next to
// its datasheet peak.  Not part of the operator; the benchmark reports it
// beside the product kernels' rates.
//
// Every wave keeps four independent accumulator chains of
// v_mfma_i32_32x32x32_i8 (no memory traffic in the loop), so the matrix
// cores are never waiting on a dependency; one lane of each wave stores a
// sum of its accumulators so the work cannot be dropped.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int64_t iters, int32_t* sink) {
  const int lane = threadIdx.x & 63;
  v4i a = {lane, lane + 1, lane + 2, lane + 3};
  v4i b = {3 * lane, 5, 7, lane ^ 9};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  if (lane == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

hipError_t launch_probe_mfma_i8(int64_t iters, int blocks, int32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace sbl
