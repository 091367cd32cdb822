// Wave-level helpers on DPP lane exchanges for the activation quantisers and
// the weight refresh (internal header).
#pragma once

#include "sbl_device.h"

namespace sbl {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Wave reductions through DPP lane exchanges (no LDS round trips): within
// each 16-lane row, exchanges with lane i^1, i^2 (quad permutations), 7-i
// and 15-i (half-row and row mirrors) leave every lane of the row with the
// row's total; the four row totals are then read from lanes 0, 16, 32, 48
// and combined as (r0 + r1) + (r2 + r3).  Each exchange pairs lanes whose
// operands are the same two values, so all lanes end with bit-identical
// results, also for floating-point sums.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// The exchanges above stay within 16-lane rows and every lane is enabled,
// so no lane keeps its old value: the 64-bit form leaves the old operand
// undefined, which spares the zeroing moves of the destination halves.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32_nold(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32_nold<CTRL>((uint32_t)b), hi = dpp_u32_nold<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

}  // namespace sbl
