// Weight-side kernels: N:M magnitude mask, per-row absmean ternary
// quantisation with 2-bit packing, and both fused in one pass.
//
// N:M mask: "Sparse-BitNet" README, "N:M Structured Sparsity"; "Sparse-BitNet
// Guide", "Mathematical Formulation of Sparse-BitLinear", step 1.
// Absmean ternary codes: model card "halo-sparse-bitnet-3:4-500m", "Recipe"
// (per row) and "Packed vs raw" (2-bit layout); guide steps 2-3.
//
// All three are HBM-bound streams over fp32 W (4 B/weight in; 1/8 B mask,
// 1/4 B codes out).  The row kernels keep a whole row in registers (one
// wave per row, 128-bit loads, lane l owning 4-column chunks l, l+64, ...),
// so W is read exactly once even though the scale must be known before any
// code is decided.
#include "sbl_device.h"
#include "sbl_wave.h"
#include "sbl_launch.h"

namespace sbl {

// ---------------------------------------------------------------------------
// Mask only: a flat stream over groups of M (M = 4: one float4 per lane;
// M = 8: two).  Bits of 32/M adjacent lanes are OR-ed into one dword store.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(256) void nm_mask_kernel(const float* __restrict__ W,
                                                      int64_t groups, int n,
                                                      uint32_t* __restrict__ out) {
  constexpr int kLanesPerWord = 32 / M;
  const int lane = lane_id();
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t base = wave * kWave; base < groups; base += nwaves * kWave) {
    const int64_t g = base + lane;
    uint32_t bits = 0;
    if (g < groups) {
      const float4* p = reinterpret_cast<const float4*>(W) + g * (M / 4);
      uint32_t key[M];
#pragma unroll
      for (int q = 0; q < M / 4; ++q) {
        float4 v = p[q];
        key[4 * q + 0] = abs_key(v.x);
        key[4 * q + 1] = abs_key(v.y);
        key[4 * q + 2] = abs_key(v.z);
        key[4 * q + 3] = abs_key(v.w);
      }
      bits = keep_mask<M>(key, n);
    }
    uint32_t word = bits << (M * (lane % kLanesPerWord));
#pragma unroll
    for (int s = 1; s < kLanesPerWord; s <<= 1) word |= (uint32_t)shfl_xor((int)word, s);
    if ((lane % kLanesPerWord) == 0 && g < groups) out[g / kLanesPerWord] = word;
  }
}

// ---------------------------------------------------------------------------
// Row kernel: scale, codes, packing, and optionally the mask.
//   MODE 0: mask read from mask_in (or none when mask_in is null)
//   MODE 1: mask computed here, m = 4 (one chunk = one group)
//   MODE 2: mask computed here, m = 8 (a group spans lanes 2i and 2i+1)
//   MODE 3, 4: as MODE 1 for n = 3 and n = 2 (the common ratios), with the
//           keep decisions as lane masks (quant_pack_row_m4); each has its
//           own kernels, so the registers of one do not burden the others.
// kMaskMode maps MODE 3 and 4 back to 1 where only the mask rule matters.
template <int MODE> constexpr int kMaskMode = MODE >= 3 ? 1 : MODE;
// CPL = 4-column chunks per lane held in registers; cols <= 256 * CPL.
// ---------------------------------------------------------------------------
struct RowJob {
  const float* W;
  const uint8_t* mask_in;
  uint8_t* mask_out;
  uint8_t* packed;
  float* scale;
  uint16_t* scale_bf16;
  int64_t rows;
  int64_t cols;
  const float* scale_in;  // non-null: the row's scale is given (per-tensor gamma)
};

// 16 bytes of latent weights read with the non-temporal policy: a refresh
// reads W once, and streaming it measured faster than cached loads (also
// for a layer's matrices that fit in the Infinity Cache).
__device__ __forceinline__ float4 load_w4_stream(const float4* p, int64_t idx) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p) + idx);
  return make_float4(t.x, t.y, t.z, t.w);
}

// Buffer resource over a row's bytes: loads past the end read zeros and
// stores past it are dropped (rows here are at most 256 KB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wrow_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kWLoadNonTemporal = 2;  // the cache-policy bit load_w4_stream sets

typedef unsigned long long lanemask;  // one bit per lane of the wave
__device__ __forceinline__ lanemask lanes(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ bool mine(lanemask m) { return __builtin_amdgcn_inverse_ballot_w64(m); }

// Dropped elements of each lane's group of four (m = 4), as lane masks, by
// the rank rule of keep_mask<4>: for i < j, i beats j iff key_i >= key_j,
// and otherwise j beats i, so six compares decide all twelve pairs.  An
// element is dropped iff at least NK of the other three beat it (NK = 2 or
// 3); the count is boolean logic on the compare masks, which live in scalar
// registers and keep that work off the vector ALU.
template <int NK>
__device__ __forceinline__ void drop4(const float4& v, lanemask (&d)[4]) {
  static_assert(NK == 2 || NK == 3, "the n = 2 and n = 3 rules");
  const uint32_t k0 = abs_key(v.x), k1 = abs_key(v.y), k2 = abs_key(v.z), k3 = abs_key(v.w);
  const lanemask c01 = lanes(k0 >= k1), c02 = lanes(k0 >= k2), c03 = lanes(k0 >= k3);
  const lanemask c12 = lanes(k1 >= k2), c13 = lanes(k1 >= k3), c23 = lanes(k2 >= k3);
  // the three "beaten by" masks of each element
  const lanemask a[4] = {~c01, c01, c02, c03}, b[4] = {~c02, ~c12, c12, c13};
  const lanemask c[4] = {~c03, ~c13, ~c23, c23};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (NK == 3)
      d[j] = a[j] & b[j] & c[j];  // beaten by all three
    else
      d[j] = (a[j] & b[j]) | (c[j] & (a[j] | b[j]));  // by at least two
  }
}

// The row kernel for an n:4 mask computed in the same pass, laid out like
// quant_pack_row below but with every lane running the same straight-line
// code: chunks past the row's end read zeros through the buffer resource
// (they add nothing to the sum) and their stores fall outside it.  Keep
// decisions are lane masks, recomputed from the loaded values in each loop
// that needs them rather than held across the row.
template <int CPL, bool BLOCK, int NK>
__device__ __forceinline__ void quant_pack_row_m4(const RowJob& job, int64_t row_in,
                                                 bool from_masked) {
  // the row is the same for the whole wave: scalar registers (the buffer
  // resources below must be)
  const int64_t row = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(row_in >> 32)) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((int)row_in));
  constexpr int NTH = BLOCK ? 256 : kWave;
  const int lane = lane_id();
  const int tid = BLOCK ? (int)threadIdx.x : lane;
  const int64_t cols = job.cols;
  const __amdgpu_buffer_rsrc_t rw = wrow_rsrc(job.W + row * cols, 4 * cols);
  float4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v t = __builtin_bit_cast(
        f4v, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(16u * (uint32_t)(tid + NTH * c)), 0,
                                                   kWLoadNonTemporal));
    v[c] = make_float4(t.x, t.y, t.z, t.w);
  }
  // Each loop takes its own copy of a chunk through an empty asm statement,
  // so the compiler neither merges the two loops' mask computations nor
  // hoists them: their lane masks would overflow the scalar registers.
  auto chunk = [&](int c) {
    float4 x = v[c];
    __asm__ volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
    return x;
  };
  // ---- scale: sum of |w| in double, lane partials then DPP exchanges ----
  // (a dropped element adds +0.0, which leaves the sum as skipping it would)
  float g;
  if (job.scale_in) {
    g = job.scale_in[row];
  } else {
    double s = 0.0;
    if (from_masked) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float4 x = chunk(c);
        lanemask d[4];
        drop4<NK>(x, d);
        const float a[4] = {fabsf(x.x), fabsf(x.y), fabsf(x.z), fabsf(x.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) s += (double)(mine(d[e]) ? 0.f : a[e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float a[4] = {fabsf(v[c].x), fabsf(v[c].y), fabsf(v[c].z), fabsf(v[c].w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) s += (double)a[e];
      }
    }
    s = wave_sum_dpp(s);
    if constexpr (BLOCK) {
      __shared__ double red[4];
      if (lane == 0) red[threadIdx.x >> 6] = s;
      __syncthreads();
      s = (red[0] + red[1]) + (red[2] + red[3]);
    }
    g = fmaxf((float)(s / (double)cols), 1e-5f);
  }
  // Clip(Round(w/g), -1, 1) is +-1 exactly when |w| > g/2 (g/2 is exact for
  // g >= 1e-5, and w/g rounded to float exceeds 1/2 iff |w| > g/2): code 01
  // for +1 and 10 for -1.
  const float thr = g * 0.5f;
  // ---- codes, packed 4 per byte; 4 lanes' bytes form one dword store ----
  const __amdgpu_buffer_rsrc_t rp = wrow_rsrc(job.packed + row * (cols >> 2), cols >> 2);
  const __amdgpu_buffer_rsrc_t rm = wrow_rsrc(job.mask_out + ((row * cols) >> 3), cols >> 3);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint32_t idx = (uint32_t)(tid + NTH * c);
    const float4 x = chunk(c);
    const float w[4] = {x.x, x.y, x.z, x.w};
    lanemask d[4];
    drop4<NK>(x, d);
    uint32_t byte = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const lanemask nz = lanes(fabsf(w[e]) > thr) & ~d[e];
      const lanemask neg = lanes((int)__float_as_uint(w[e]) < 0);
      byte |= mine(nz & ~neg) ? (1u << (2 * e)) : 0u;
      byte |= mine(nz & neg) ? (2u << (2 * e)) : 0u;
    }
    uint32_t word = byte << (8 * (lane & 3));
    word |= dpp_u32<kDppXor1>(word);
    word |= dpp_u32<kDppXor2>(word);
    if ((lane & 3) == 0) __builtin_amdgcn_raw_buffer_store_b32(word, rp, (int)idx, 0, 0);
    if (job.mask_out) {
      uint32_t k4 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) k4 |= mine(d[e]) ? 0u : (1u << e);
      uint32_t mw = k4 << (4 * (lane & 7));
      mw |= dpp_u32<kDppXor1>(mw);
      mw |= dpp_u32<kDppXor2>(mw);
      mw |= dpp_u32<kDppHalfMirror>(mw);  // the other quad of the 8 lanes
      if ((lane & 7) == 0) __builtin_amdgcn_raw_buffer_store_b32(mw, rm, (int)(idx >> 1), 0, 0);
    }
    // one chunk's lane masks at a time (scalar registers run short otherwise)
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tid == 0) {
    job.scale[row] = g;
    if (job.scale_bf16) job.scale_bf16[row] = f32_to_bf16_rne(g);
  }
}

// One row per wave (BLOCK = false), or per block of 256 threads for long rows
// (BLOCK = true: the four waves' double sums meet in LDS in a fixed order).
// Chunk idx = thread + threads * c, so the chunks of a wave are consecutive
// and the lane exchanges below (n:8 groups, code and mask packing) stay
// inside a wave.
template <int CPL, int MODE, bool BLOCK>
__device__ __forceinline__ void quant_pack_row_bits(const RowJob& job, int64_t row, int n,
                                                    bool from_masked) {
  constexpr int NTH = BLOCK ? 256 : kWave;
  const int lane = lane_id();
  const int tid = BLOCK ? (int)threadIdx.x : lane;
  const int64_t cols = job.cols;
  const int64_t nchunks = cols >> 2;
  const float4* src = reinterpret_cast<const float4*>(job.W + row * cols);
  float4 v[CPL];
  uint32_t keep[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t idx = tid + (int64_t)NTH * c;
    v[c] = idx < nchunks ? load_w4_stream(src, idx) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // ---- mask ----
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t idx = tid + (int64_t)NTH * c;
    if constexpr (MODE == 0) {
      if (job.mask_in && idx < nchunks) {
        const int64_t bit = row * cols + 4 * idx;
        keep[c] = (job.mask_in[bit >> 3] >> (bit & 7)) & 0xFu;
      } else {
        keep[c] = 0xFu;
      }
    } else if constexpr (MODE == 1) {
      uint32_t key[4] = {abs_key(v[c].x), abs_key(v[c].y), abs_key(v[c].z), abs_key(v[c].w)};
      keep[c] = keep_mask<4>(key, n);
    } else {
      uint32_t mine[4] = {abs_key(v[c].x), abs_key(v[c].y), abs_key(v[c].z), abs_key(v[c].w)};
      uint32_t other[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) other[e] = dpp_u32<kDppXor1>(mine[e]);
      const bool low_half = (lane & 1) == 0;
      uint32_t key[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = low_half ? mine[e] : other[e];
        key[4 + e] = low_half ? other[e] : mine[e];
      }
      const uint32_t k8 = keep_mask<8>(key, n);
      keep[c] = low_half ? (k8 & 0xFu) : (k8 >> 4);
    }
  }
  // ---- scale: sum of |w| in double, lane partials then DPP exchanges ----
  float g;
  if (job.scale_in) {
    g = job.scale_in[row];
  } else {
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float a[4] = {fabsf(v[c].x), fabsf(v[c].y), fabsf(v[c].z), fabsf(v[c].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!from_masked || ((keep[c] >> e) & 1u)) s += (double)a[e];
    }
    s = wave_sum_dpp(s);
    if constexpr (BLOCK) {
      __shared__ double red[4];
      if (lane == 0) red[threadIdx.x >> 6] = s;
      __syncthreads();
      s = (red[0] + red[1]) + (red[2] + red[3]);
    }
    g = fmaxf((float)(s / (double)cols), 1e-5f);
  }
  // Clip(Round(w/g), -1, 1) is +-1 exactly when |w| > g/2 (g/2 is exact for
  // g >= 1e-5, and w/g rounded to float exceeds 1/2 iff |w| > g/2).
  const float thr = g * 0.5f;
  // ---- codes, packed 4 per byte; 4 lanes' bytes form one dword store ----
  uint32_t* dst = reinterpret_cast<uint32_t*>(job.packed + row * (cols >> 2));
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int64_t idx = tid + (int64_t)NTH * c;
    const float w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    uint32_t byte = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t f = fabsf(w[e]) > thr ? (w[e] < 0.f ? 2u : 1u) : 0u;
      f = ((keep[c] >> e) & 1u) ? f : 0u;
      byte |= f << (2 * e);
    }
    uint32_t word = byte << (8 * (lane & 3));
    word |= dpp_u32<kDppXor1>(word);
    word |= dpp_u32<kDppXor2>(word);
    if ((lane & 3) == 0 && idx < nchunks) dst[idx >> 2] = word;
    if constexpr (MODE != 0) {
      if (job.mask_out) {
        uint32_t mw = keep[c] << (4 * (lane & 7));
        mw |= dpp_u32<kDppXor1>(mw);
        mw |= dpp_u32<kDppXor2>(mw);
        mw |= dpp_u32<kDppHalfMirror>(mw);  // the other quad of the 8 lanes
        if ((lane & 7) == 0 && idx < nchunks)
          reinterpret_cast<uint32_t*>(job.mask_out)[(row * cols + 4 * idx) >> 5] = mw;
      }
    }
  }
  if (tid == 0) {
    job.scale[row] = g;
    if (job.scale_bf16) job.scale_bf16[row] = f32_to_bf16_rne(g);
  }
}

template <int CPL, int MODE, bool BLOCK>
__device__ __forceinline__ void quant_pack_row(const RowJob& job, int64_t row, int n,
                                               bool from_masked) {
  if constexpr (MODE == 3)
    quant_pack_row_m4<CPL, BLOCK, 3>(job, row, from_masked);
  else if constexpr (MODE == 4)
    quant_pack_row_m4<CPL, BLOCK, 2>(job, row, from_masked);
  else
    quant_pack_row_bits<CPL, MODE, BLOCK>(job, row, n, from_masked);
}

// Rows longer than 256*32 columns: two passes over the row (the second
// read is expected to hit L2), same arithmetic.
template <int MODE>
__device__ void quant_pack_row_long(const RowJob& job, int64_t row, int n, bool from_masked) {
  const int lane = lane_id();
  const int64_t cols = job.cols;
  const int64_t nchunks = cols >> 2;
  const float4* src = reinterpret_cast<const float4*>(job.W + row * cols);
  auto mask_of = [&](int64_t idx, const float4& x) -> uint32_t {
    if constexpr (MODE == 0) {
      if (!job.mask_in) return 0xFu;
      const int64_t bit = row * cols + 4 * idx;
      return (job.mask_in[bit >> 3] >> (bit & 7)) & 0xFu;
    } else if constexpr (MODE == 1) {
      uint32_t key[4] = {abs_key(x.x), abs_key(x.y), abs_key(x.z), abs_key(x.w)};
      return keep_mask<4>(key, n);
    } else {
      uint32_t mine[4] = {abs_key(x.x), abs_key(x.y), abs_key(x.z), abs_key(x.w)};
      uint32_t other[4];
      for (int e = 0; e < 4; ++e) other[e] = dpp_u32<kDppXor1>(mine[e]);
      const bool low_half = (lane & 1) == 0;
      uint32_t key[8];
      for (int e = 0; e < 4; ++e) {
        key[e] = low_half ? mine[e] : other[e];
        key[4 + e] = low_half ? other[e] : mine[e];
      }
      const uint32_t k8 = keep_mask<8>(key, n);
      return low_half ? (k8 & 0xFu) : (k8 >> 4);
    }
  };
  float g;
  if (job.scale_in) {
    g = job.scale_in[row];
  } else {
    double s = 0.0;
    for (int64_t base = 0; base < nchunks; base += kWave) {  // nchunks % 16 == 0
      const int64_t idx = base + lane;
      float4 x = idx < nchunks ? src[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
      uint32_t k = mask_of(idx, x);
      const float a[4] = {fabsf(x.x), fabsf(x.y), fabsf(x.z), fabsf(x.w)};
      for (int e = 0; e < 4; ++e)
        if (!from_masked || ((k >> e) & 1u)) s += (double)a[e];
    }
    s = wave_sum_dpp(s);
    g = fmaxf((float)(s / (double)cols), 1e-5f);
  }
  const float thr = g * 0.5f;
  uint32_t* dst = reinterpret_cast<uint32_t*>(job.packed + row * (cols >> 2));
  for (int64_t base = 0; base < nchunks; base += kWave) {
    const int64_t idx = base + lane;
    float4 x = idx < nchunks ? load_w4_stream(src, idx) : make_float4(0.f, 0.f, 0.f, 0.f);  // last read
    uint32_t k = mask_of(idx, x);
    const float w[4] = {x.x, x.y, x.z, x.w};
    uint32_t byte = 0;
    for (int e = 0; e < 4; ++e) {
      uint32_t f = fabsf(w[e]) > thr ? (w[e] < 0.f ? 2u : 1u) : 0u;
      f = ((k >> e) & 1u) ? f : 0u;
      byte |= f << (2 * e);
    }
    uint32_t word = byte << (8 * (lane & 3));
    word |= dpp_u32<kDppXor1>(word);
    word |= dpp_u32<kDppXor2>(word);
    if ((lane & 3) == 0 && idx < nchunks) dst[idx >> 2] = word;
    if constexpr (MODE != 0) {
      if (job.mask_out) {
        uint32_t mw = k << (4 * (lane & 7));
        mw |= dpp_u32<kDppXor1>(mw);
        mw |= dpp_u32<kDppXor2>(mw);
        mw |= dpp_u32<kDppHalfMirror>(mw);  // the other quad of the 8 lanes
        if ((lane & 7) == 0 && idx < nchunks)
          reinterpret_cast<uint32_t*>(job.mask_out)[(row * cols + 4 * idx) >> 5] = mw;
      }
    }
  }
  if (lane == 0) {
    job.scale[row] = g;
    if (job.scale_bf16) job.scale_bf16[row] = f32_to_bf16_rne(g);
  }
}

template <int CPL, int MODE>
__device__ __forceinline__ void quant_pack_dispatch(const RowJob& job, int64_t row, int n,
                                                    bool from_masked) {
  if constexpr (CPL == 0)
    quant_pack_row_long<kMaskMode<MODE>>(job, row, n, from_masked);
  else
    quant_pack_row<CPL, MODE, false>(job, row, n, from_masked);
}

constexpr int kRowsPerBlock = 4;  // one wave per row

template <int CPL, int MODE>
__global__ __launch_bounds__(256) void quant_pack_kernel(RowJob job, int n, int from_masked) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= job.rows) return;  // whole wave leaves; no block barrier below
  quant_pack_dispatch<CPL, MODE>(job, row, n, from_masked != 0);
}

// Grouped: the blocks of all matrices laid end to end; block_start[d] is the
// first block of entry d (kept in the kernel argument).  An entry's rows
// take one wave each (four per block), or, for rows longer than 8 chunks
// per lane (whole_block), one block each.
struct GroupedRefreshArgs {
  const sbl_refresh_desc* descs;
  int count;
  int block_start[kMaxGroupedRefresh + 1];
  int descs_idx[kMaxGroupedRefresh];            // index into descs of each entry
  unsigned char whole_block[kMaxGroupedRefresh];  // one row per block
};

template <int CPL, int MODE>
__global__ __launch_bounds__(256) void quant_pack_grouped_kernel(GroupedRefreshArgs args, int n,
                                                                 int from_masked) {
  const int b = blockIdx.x;
  int lo = 0, hi = args.count - 1;  // last d with block_start[d] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.block_start[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const sbl_refresh_desc d = args.descs[args.descs_idx[lo]];
  RowJob job{d.W, nullptr, d.mask_bits, d.packed, d.row_scale, d.row_scale_bf16, d.rows, d.cols};
  if constexpr (CPL > 0) {
    if (args.whole_block[lo]) {  // block-uniform: every wave reaches the barrier inside
      quant_pack_row<CPL, MODE, true>(job, b - args.block_start[lo], n, from_masked != 0);
      return;
    }
  }
  const int64_t row = (int64_t)(b - args.block_start[lo]) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= d.rows) return;
  quant_pack_dispatch<CPL, MODE>(job, row, n, from_masked != 0);
}

// ---------------------------------------------------------------------------
// Per-tensor absmean ("Sparse-BitNet Guide", "Mathematical Formulation",
// step 2, and its module: one gamma = mean |W| over the whole matrix).
// Three launches, because no code can be decided before the whole tensor
// is summed: (1) one wave per row sums |w| (or |w| * mask) in double and
// parks the sum in the first 8 bytes of the row's packed output, which the
// codes overwrite later; (2) one block adds the row sums in a fixed order
// and writes gamma into every row scale; (3) the row kernel quantises with
// the given scale.  W is read twice (8.25 B per weight instead of 4.25).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void row_abs_sum_kernel(RowJob job, int n, int from_masked) {
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= job.rows) return;
  const int64_t cols = job.cols;
  const int64_t nchunks = cols >> 2;
  const float4* src = reinterpret_cast<const float4*>(job.W + row * cols);
  double s = 0.0;
  for (int64_t base = 0; base < nchunks; base += kWave) {  // nchunks % 16 == 0
    const int64_t idx = base + lane;
    const float4 x = idx < nchunks ? src[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t k = 0xFu;
    if (from_masked) {
      if constexpr (MODE == 0) {
        const int64_t bit = row * cols + 4 * idx;
        k = idx < nchunks ? (job.mask_in[bit >> 3] >> (bit & 7)) & 0xFu : 0u;
      } else if constexpr (MODE == 1) {
        uint32_t key[4] = {abs_key(x.x), abs_key(x.y), abs_key(x.z), abs_key(x.w)};
        k = keep_mask<4>(key, n);
      } else {
        uint32_t mine[4] = {abs_key(x.x), abs_key(x.y), abs_key(x.z), abs_key(x.w)};
        uint32_t other[4];
        for (int e = 0; e < 4; ++e) other[e] = dpp_u32<kDppXor1>(mine[e]);
        const bool low_half = (lane & 1) == 0;
        uint32_t key[8];
        for (int e = 0; e < 4; ++e) {
          key[e] = low_half ? mine[e] : other[e];
          key[4 + e] = low_half ? other[e] : mine[e];
        }
        const uint32_t k8 = keep_mask<8>(key, n);
        k = low_half ? (k8 & 0xFu) : (k8 >> 4);
      }
    }
    const float a[4] = {fabsf(x.x), fabsf(x.y), fabsf(x.z), fabsf(x.w)};
    for (int e = 0; e < 4; ++e)
      if ((k >> e) & 1u) s += (double)a[e];
  }
  s = wave_sum(s);
  if (lane == 0) *reinterpret_cast<double*>(job.packed + row * (cols >> 2)) = s;
}

__global__ __launch_bounds__(256) void tensor_scale_kernel(RowJob job) {
  __shared__ double part[256];
  const int t = threadIdx.x;
  const int64_t stride = job.cols >> 2;
  double s = 0.0;
  for (int64_t r = t; r < job.rows; r += 256)
    s += *reinterpret_cast<const double*>(job.packed + r * stride);
  part[t] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {  // fixed pairing order: deterministic
    if (t < h) part[t] += part[t + h];
    __syncthreads();
  }
  const float g = fmaxf((float)(part[0] / ((double)job.rows * (double)job.cols)), 1e-5f);
  for (int64_t r = t; r < job.rows; r += 256) {
    job.scale[r] = g;
    if (job.scale_bf16) job.scale_bf16[r] = f32_to_bf16_rne(g);
  }
}

// ---------------------------------------------------------------------------
// Mask monitoring (README "Key Training Options": the mask change rate is
// monitored every few steps; model card "Recipe": a mask-verify every 500
// steps).  stats[0] += weights whose mask bit differs between two masks,
// stats[1] += M-groups of the new mask that do not keep exactly n.  The
// masks are flat bit streams (groups never straddle rows, cols % 64 == 0),
// read 16 bytes per lane; group counts come from in-register popcounts.
// ---------------------------------------------------------------------------
__global__ void zero_stats_kernel(unsigned long long* stats) {
  if (threadIdx.x < 2) stats[threadIdx.x] = 0ull;
}

template <int M>
__device__ __forceinline__ uint32_t groups_not_n(uint32_t w, uint32_t n) {
  uint32_t v = w - ((w >> 1) & 0x55555555u);           // 2-bit counts
  v = (v & 0x33333333u) + ((v >> 2) & 0x33333333u);    // 4-bit counts (groups of 4)
  uint32_t x;
  if constexpr (M == 4) {
    x = v ^ (n * 0x11111111u);
    x = (x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x11111111u;
  } else {
    v = (v + (v >> 4)) & 0x0F0F0F0Fu;                   // 8-bit counts (groups of 8)
    x = v ^ (n * 0x01010101u);
    x = (x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x01010101u;
  }
  return (uint32_t)__popc(x);
}

// Mask words are read once: non-temporal loads.
__device__ __forceinline__ uint4 load_u4_stream(const uint4* p, int64_t idx) {
  const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p) + idx);
  return make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
}

// Per-word counters of the two stream kernels below.  `a` is a word of
// the stream that is checked, `b` the matching word of the second stream
// (the old mask; equal to `a` when there is none).
template <int M>
struct MaskStatsOp {
  __device__ __forceinline__ static void word(uint32_t a, uint32_t b, uint32_t n, uint32_t& c0, uint32_t& c1) {
    c0 += (uint32_t)__popc(a ^ b);
    c1 += groups_not_n<M>(a, n);
  }
};

// Packed-code validator (model card "Packed vs raw": the field 11 is not a
// code; "Recipe": at most n nonzero codes per group of m).  A 32-bit word
// holds 16 fields; with lo/hi the low and high bit of every field, 11 is
// lo & hi and a nonzero code (01 or 10) is lo ^ hi.  Groups of 4 fields are
// the bytes of the word, groups of 8 its 16-bit halves, so no group
// straddles two words (a row is a whole number of 16-byte chunks).
template <int M>
struct PackedCheckOp {
  __device__ __forceinline__ static void word(uint32_t a, uint32_t, uint32_t n, uint32_t& c0, uint32_t& c1) {
    const uint32_t lo = a & 0x55555555u, hi = (a >> 1) & 0x55555555u;
    c0 += (uint32_t)__popc(lo & hi);
    const uint32_t nz = lo ^ hi;
    uint32_t v = (nz & 0x33333333u) + ((nz >> 2) & 0x33333333u);  // per 4 bits: 0..2
    v = (v + (v >> 4)) & 0x0F0F0F0Fu;                              // per byte: 0..4
    if constexpr (M == 4) {
      // byte + (127 - n) reaches bit 7 iff the byte's count exceeds n
      c1 += (uint32_t)__popc((v + (0x7Fu - n) * 0x01010101u) & 0x80808080u);
    } else {
      v = (v + (v >> 8)) & 0x001F001Fu;                            // per 16 bits: 0..8
      c1 += (uint32_t)__popc((v + (0x7FFFu - n) * 0x00010001u) & 0x80008000u);
    }
  }
};

// One block of 1024 threads per CU at most: few blocks keep the two 64-bit
// atomics per block cheap (they serialise on one address), and four 16-byte
// loads per operand and lane keep enough bytes in flight.
constexpr int kStatsThreads = 1024;

template <typename Op>
__global__ __launch_bounds__(kStatsThreads) void word_stats_kernel(const uint32_t* __restrict__ old_w,
                                                                   const uint32_t* __restrict__ new_w,
                                                                   int64_t words, int n,
                                                                   unsigned long long* stats) {
  __shared__ unsigned long long part[2][kStatsThreads / kWave];
  uint32_t c0 = 0, c1 = 0;
  const int64_t nvec = words >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * blockDim.x;
  auto word = [&](uint32_t a, uint32_t b) { Op::word(a, b, (uint32_t)n, c0, c1); };
  const uint4* nv = reinterpret_cast<const uint4*>(new_w);
  const uint4* ov = reinterpret_cast<const uint4*>(old_w);
  int64_t i = gid;
  // four 16-byte loads per operand in flight per lane
  for (; i + 3 * gsz < nvec; i += 4 * gsz) {
    uint4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = load_u4_stream(nv, i + u * gsz);
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = old_w ? load_u4_stream(ov, i + u * gsz) : a[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      word(a[u].x, b[u].x);
      word(a[u].y, b[u].y);
      word(a[u].z, b[u].z);
      word(a[u].w, b[u].w);
    }
  }
  for (; i < nvec; i += gsz) {
    const uint4 a = nv[i];
    const uint4 b = old_w ? ov[i] : a;
    word(a.x, b.x);
    word(a.y, b.y);
    word(a.z, b.z);
    word(a.w, b.w);
  }
  for (int64_t i = 4 * nvec + gid; i < words; i += gsz) word(new_w[i], old_w ? old_w[i] : new_w[i]);
  // A lane's counts stay below 2^32 (at most 2^46 bits over 2^18 lanes);
  // wave and block sums are 64-bit, then one atomic per counter.
  unsigned long long c64 = c0, g64 = c1;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    c64 += (unsigned long long)__shfl_xor((long long)c64, d, kWave);
    g64 += (unsigned long long)__shfl_xor((long long)g64, d, kWave);
  }
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) {
    part[0][wave] = c64;
    part[1][wave] = g64;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long c = 0, g = 0;
#pragma unroll
    for (int w = 0; w < kStatsThreads / kWave; ++w) {
      c += part[0][w];
      g += part[1][w];
    }
    if (c) atomicAdd(&stats[0], c);
    if (g) atomicAdd(&stats[1], g);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
// Register footprint class of a row: 4-column chunks each lane holds.
static int chunks_per_lane(int64_t cols) {
  const int64_t need = (cols / 4 + kWave - 1) / kWave;
  constexpr int kClasses[] = {1, 2, 4, 8, 12, 16, 20, 24, 28, 32};
  for (int c : kClasses)
    if (need <= c) return c;
  return 0;  // long-row path
}

hipError_t launch_nm_mask(const float* W, int64_t rows, int64_t cols, int n, int m,
                          uint8_t* mask_bits, hipStream_t stream) {
  const int64_t groups = rows * cols / m;
  const int64_t blocks = std::min<int64_t>((groups + 255) / 256, 256 * 32);
  if (m == 4)
    hipLaunchKernelGGL(nm_mask_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, W,
                       groups, n, reinterpret_cast<uint32_t*>(mask_bits));
  else
    hipLaunchKernelGGL(nm_mask_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, W,
                       groups, n, reinterpret_cast<uint32_t*>(mask_bits));
  return hipGetLastError();
}

template <int MODE>
static void launch_row(int cpl, dim3 grid, hipStream_t stream, const RowJob& job, int n,
                       int from_masked) {
  switch (cpl) {
#define SBL_CASE(C)                                                                        \
  case C:                                                                                  \
    hipLaunchKernelGGL((quant_pack_kernel<C, MODE>), grid, dim3(256), 0, stream, job, n, \
                       from_masked);                                                       \
    break;
    SBL_CASE(1) SBL_CASE(2) SBL_CASE(4) SBL_CASE(8) SBL_CASE(12) SBL_CASE(16) SBL_CASE(20)
    SBL_CASE(24) SBL_CASE(28) SBL_CASE(32)
#undef SBL_CASE
    case 0:  // the two-pass long-row path has no lane-mask variant
      hipLaunchKernelGGL((quant_pack_kernel<0, kMaskMode<MODE>>), grid, dim3(256), 0, stream, job, n,
                         from_masked);
      break;
  }
}

// Mode of a row kernel with the mask computed in it (fuse_mask).
static int fused_mode(int n, int m) { return m == 8 ? 2 : n == 3 ? 3 : n == 2 ? 4 : 1; }

hipError_t launch_quant_pack(const float* W, const uint8_t* mask_in, int64_t rows, int64_t cols,
                             int n, int m, int fuse_mask, unsigned flags, uint8_t* mask_out,
                             uint8_t* packed, float* scale, uint16_t* scale_bf16,
                             hipStream_t stream) {
  RowJob job{W, mask_in, mask_out, packed, scale, scale_bf16, rows, cols, nullptr};
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const int cpl = chunks_per_lane(cols);
  const int fm = (flags & SBL_SCALE_FROM_MASKED) ? 1 : 0;
  if (flags & SBL_SCALE_PER_TENSOR) {
    if (!fuse_mask)
      hipLaunchKernelGGL(row_abs_sum_kernel<0>, grid, dim3(256), 0, stream, job, n, fm);
    else if (m == 4)
      hipLaunchKernelGGL(row_abs_sum_kernel<1>, grid, dim3(256), 0, stream, job, n, fm);
    else
      hipLaunchKernelGGL(row_abs_sum_kernel<2>, grid, dim3(256), 0, stream, job, n, fm);
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, stream, job);
    job.scale_in = scale;
  }
  switch (fuse_mask ? fused_mode(n, m) : 0) {
    case 0: launch_row<0>(cpl, grid, stream, job, n, fm); break;
    case 1: launch_row<1>(cpl, grid, stream, job, n, fm); break;
    case 2: launch_row<2>(cpl, grid, stream, job, n, fm); break;
    case 3: launch_row<3>(cpl, grid, stream, job, n, fm); break;
    default: launch_row<4>(cpl, grid, stream, job, n, fm); break;
  }
  return hipGetLastError();
}

template <int MODE>
static void launch_grouped(int cpl, dim3 grid, hipStream_t stream, const GroupedRefreshArgs& a,
                           int n, int fm) {
  switch (cpl) {
#define SBL_CASE(C)                                                                              \
  case C:                                                                                        \
    hipLaunchKernelGGL((quant_pack_grouped_kernel<C, MODE>), grid, dim3(256), 0, stream, a, n, \
                       fm);                                                                      \
    break;
    SBL_CASE(1) SBL_CASE(2) SBL_CASE(4) SBL_CASE(8) SBL_CASE(12) SBL_CASE(16) SBL_CASE(20)
    SBL_CASE(24) SBL_CASE(28) SBL_CASE(32)
#undef SBL_CASE
    case 0:
      hipLaunchKernelGGL((quant_pack_grouped_kernel<0, kMaskMode<MODE>>), grid, dim3(256), 0, stream,
                         a, n, fm);
      break;
  }
}

// Zero the two counters, then one pass of word_stats_kernel<Op> over
// `words` 32-bit words.
template <template <int> class Op>
static hipError_t launch_word_stats(const uint32_t* ow, const uint32_t* nw, int64_t words, int n, int m,
                                    int64_t* stats, hipStream_t stream) {
  unsigned long long* st = reinterpret_cast<unsigned long long*>(stats);
  hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, stream, st);
  if (words > 0) {
    const int64_t blocks =
        std::max<int64_t>(1, std::min<int64_t>((words / 16 + kStatsThreads - 1) / kStatsThreads, 256));
    if (m == 4)
      hipLaunchKernelGGL(word_stats_kernel<Op<4>>, dim3((unsigned)blocks), dim3(kStatsThreads), 0, stream, ow, nw, words, n, st);
    else
      hipLaunchKernelGGL(word_stats_kernel<Op<8>>, dim3((unsigned)blocks), dim3(kStatsThreads), 0, stream, ow, nw, words, n, st);
  }
  return hipGetLastError();
}

hipError_t launch_mask_stats(const uint8_t* old_bits, const uint8_t* new_bits, int64_t rows,
                             int64_t cols, int n, int m, int64_t* stats, hipStream_t stream) {
  return launch_word_stats<MaskStatsOp>(reinterpret_cast<const uint32_t*>(old_bits),
                                        reinterpret_cast<const uint32_t*>(new_bits), rows * cols / 32, n, m,
                                        stats, stream);
}

hipError_t launch_packed_check(const uint8_t* packed, int64_t rows, int64_t cols, int n, int m,
                               int64_t* stats, hipStream_t stream) {
  return launch_word_stats<PackedCheckOp>(nullptr, reinterpret_cast<const uint32_t*>(packed),
                                          rows * cols / 16, n, m, stats, stream);
}

hipError_t launch_quant_pack_grouped(const sbl_refresh_desc* host, const sbl_refresh_desc* dev,
                                     int count, int n, int m, unsigned flags,
                                     hipStream_t stream) {
  // Each matrix gets a register class (16-byte chunks per thread): rows of
  // up to 8 chunks per lane take one wave per row; longer rows (up to 32
  // chunks per thread) take a whole block per row; longer still, the
  // two-pass long-row path.  When no class exceeds 8 chunks (the layers of
  // both benchmark stacks) every matrix goes into one launch of the largest
  // class, long-row blocks first; otherwise there is one launch per class,
  // so a narrow row never carries the registers of the widest.  The block
  // offsets of a launch travel in its argument block (at most
  // kMaxGroupedRefresh entries per launch).
  const int fm = (flags & SBL_SCALE_FROM_MASKED) ? 1 : 0;
  constexpr int kClasses[] = {1, 2, 4, 8, 12, 16, 20, 24, 28, 32, 0};
  auto class_of = [&](int64_t need) {
    for (int c : kClasses)
      if (c > 0 && need <= c) return c;
    return 0;
  };
  auto plan = [&](const sbl_refresh_desc& h, bool& whole) {
    const int64_t need = (h.cols / 4 + kWave - 1) / kWave;
    whole = need > 8 && need <= 4 * 32;
    return class_of(whole ? (need + 3) / 4 : need);
  };
  int max_cls = 0;
  bool merge = true;
  for (int d = 0; d < count; ++d) {
    if (host[d].rows == 0) continue;
    bool whole;
    const int c = plan(host[d], whole);
    if (c == 0 || c > 8) merge = false;
    max_cls = std::max(max_cls, c);
  }
  for (int cls : kClasses) {
    if (merge && cls != max_cls) continue;
    GroupedRefreshArgs a;
    a.descs = dev;
    int cnt = 0;
    int64_t blocks = 0;
    auto flush = [&]() -> hipError_t {
      if (cnt == 0) return hipSuccess;
      a.count = cnt;
      a.block_start[cnt] = (int)blocks;
      if (blocks > 0) {
        const dim3 grid((unsigned)blocks);
        switch (fused_mode(n, m)) {
          case 1: launch_grouped<1>(cls, grid, stream, a, n, fm); break;
          case 2: launch_grouped<2>(cls, grid, stream, a, n, fm); break;
          case 3: launch_grouped<3>(cls, grid, stream, a, n, fm); break;
          default: launch_grouped<4>(cls, grid, stream, a, n, fm); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      cnt = 0;
      blocks = 0;
      return hipSuccess;
    };
    for (int pass = 0; pass < 2; ++pass) {  // whole-block rows first
      for (int d = 0; d < count; ++d) {
        if (host[d].rows == 0) continue;
        bool whole;
        const int c = plan(host[d], whole);
        if ((!merge && c != cls) || whole != (pass == 0)) continue;
        if (cnt == kMaxGroupedRefresh) {
          hipError_t e = flush();
          if (e != hipSuccess) return e;
        }
        a.descs_idx[cnt] = d;
        a.whole_block[cnt] = whole ? 1 : 0;
        a.block_start[cnt] = (int)blocks;
        blocks += whole ? host[d].rows : (host[d].rows + kRowsPerBlock - 1) / kRowsPerBlock;
        ++cnt;
      }
    }
    hipError_t e = flush();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbl
