// Device helpers shared by the gfx950 kernels of libsbl (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbl {

constexpr int kWave = 64;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// v_perm_b32: result byte i = byte sel_i of the 8-byte value {hi:lo}, where
// selectors 0-3 address `lo` and 4-7 address `hi`; selector 8 replicates bit
// 15 of `lo`, 12 gives 0x00 (and 13 and up 0xFF).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Byte table of the 2-bit weight code (model card "Packed vs raw"):
// 00 -> 0, 01 -> +1, 10 -> -1 (0xFF), 11 (never written) -> 0.
constexpr uint32_t kCodeLut = 0x00FF0100u;
constexpr uint32_t kLow2 = 0x03030303u;
// The same table for a code held in bits [3:2] of a selector byte, whose
// values 0, 4, 8, 12 pick: byte 0 of lo (0x00), byte 0 of hi (0x01), bit 15
// of lo replicated (0xFF), the constant 0x00.
constexpr uint32_t kCodeLutB2Hi = 0x00000001u;
constexpr uint32_t kCodeLutB2Lo = 0x00008000u;

// 16 packed codes -> 16 int8 in "strided" order: dword m, byte j holds the
// code of column 4*j + m.  Nine ALU ops: codes 1 and 3 of each byte select
// through the second table without being shifted down.
__device__ __forceinline__ void expand16_strided(uint32_t w, uint32_t out[4]) {
  const uint32_t w4 = w >> 4;
  out[0] = perm(kCodeLut, kCodeLut, w & kLow2);
  out[1] = perm(kCodeLutB2Hi, kCodeLutB2Lo, w & (kLow2 << 2));
  out[2] = perm(kCodeLut, kCodeLut, w4 & kLow2);
  out[3] = perm(kCodeLutB2Hi, kCodeLutB2Lo, w4 & (kLow2 << 2));
}

// Transpose the 4x4 byte matrix held in four dwords: out[j].byte[m] =
// in[m].byte[j].  Eight v_perm.
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  uint32_t p01l = perm(in[1], in[0], 0x05010400u);
  uint32_t p01h = perm(in[1], in[0], 0x07030602u);
  uint32_t p23l = perm(in[3], in[2], 0x05010400u);
  uint32_t p23h = perm(in[3], in[2], 0x07030602u);
  out[0] = perm(p23l, p01l, 0x05040100u);
  out[1] = perm(p23l, p01l, 0x07060302u);
  out[2] = perm(p23h, p01h, 0x05040100u);
  out[3] = perm(p23h, p01h, 0x07060302u);
}

// 16 packed codes -> 16 int8 in column order (dword j holds columns
// 4j..4j+3).
__device__ __forceinline__ void expand16_natural(uint32_t w, uint32_t out[4]) {
  uint32_t t[4];
  expand16_strided(w, t);
  transpose4x4(t, out);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += shfl_xor(v, s);
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = max(v, (uint32_t)shfl_xor((int)v, s));
  return v;
}

// float -> bfloat16 bits, round to nearest even (finite inputs; NaN kept NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Row scale read for the products: float or bf16 bits.
__device__ __forceinline__ float load_scale(const void* s, int bf16, int64_t i) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(s)[i])
              : reinterpret_cast<const float*>(s)[i];
}

// Rank-based N-of-M keep mask over magnitude keys (|w| bits, an unsigned
// order equal to the float order of |w| for finite w): element j is kept
// iff fewer than n elements beat it, where i beats j when key_i > key_j, or
// key_i == key_j and i < j.
template <int M>
__device__ __forceinline__ uint32_t keep_mask(const uint32_t (&key)[M], int n) {
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    int beaten = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (i < j) beaten += key[i] >= key[j];
      else if (i > j) beaten += key[i] > key[j];
    }
    bits |= (uint32_t)(beaten < n) << j;
  }
  return bits;
}

__device__ __forceinline__ uint32_t abs_key(float w) { return __float_as_uint(w) & 0x7fffffffu; }

}  // namespace sbl
