// Per-token absmax int8 activation quantisation (W1.58A8).
// "Sparse-BitNet Guide", "Mathematical Formulation of Sparse-BitLinear",
// step 4, and its module in "End-to-End Implementation": beta = max|x|
// clamped below at 1e-5, x~ = Clip(Round(x * (127/beta)), -128, 127).
//
// One wave per token; the token row (bf16) stays in registers between the
// absmax reduction and the quantisation, so x is read once (2 B/element in,
// 1 B/element out).  The absmax is an integer max over the magnitude bits,
// exact and order-free.
#include "sbl_device.h"
#include "sbl_wave.h"
#include "sbl_launch.h"

namespace sbl {

// 16 bytes of x on their last read, with the non-temporal policy: x is read
// once and would only evict the weights and x~ that the products read next
// (a layer step with streaming activation loads ran ~5% faster, although a
// lone quantisation of an x that is still cached is a little slower).
__device__ __forceinline__ uint4 load_x16(const uint4* p, int64_t idx) {
  const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p) + idx);
  return make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
}

// The short-row kernels address a token's row through buffer resources
// (base, byte count): loads past the end read zeros and stores past it are
// dropped, so the lanes whose chunk lies past the row's end run the same
// straight-line code as the others and need no branch or zeroing.
constexpr int kLoadNonTemporal = 2;  // the cache-policy bit load_x16 sets
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int POLICY>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
  return make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
}
__device__ __forceinline__ float4 bload16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const uint4 u = bload16<0>(r, off);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
__device__ __forceinline__ void bstore8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)v.x, (int)v.y}, r, (int)off, 0, 0);
}

// x~ codes of 8 values: Clip(Round(v * s), -128, 127) as bytes.  The product
// is rounded to float, then 1.5 * 2^23 is added: the sum's unit in the last
// place is 1, so the addition rounds v * s to the nearest integer, ties to
// even, as rintf does, and the low byte of the sum's bits is that integer in
// two's complement.  With s = 127 / beta and beta >= max |v|, |v * s| stays
// below 127.5, so the clip never acts and the byte is the code.
__device__ __forceinline__ uint2 quant8_codes(const float (&v)[8], float s) {
  constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = v[e] * s;  // rounded to float first (no contraction)
    q[e] = __float_as_uint(p + kRound);
  }
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = perm(q[4 * h + 1], q[4 * h], 0x0C0C0400u);      // bytes q0, q1
    const uint32_t hi = perm(q[4 * h + 3], q[4 * h + 2], 0x0C0C0400u);  // bytes q2, q3
    out[h] = perm(hi, lo, 0x05040100u);
  }
  return make_uint2(out[0], out[1]);
}

template <int CPL>  // 8-element (16-byte) chunks per lane; 0 = long-row loop
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t tokens, int64_t cols,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ beta) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (t >= tokens) return;
  const int64_t nchunks = cols >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * cols);
  uint2* dst = reinterpret_cast<uint2*>(xq + t * cols);
  // max of the magnitude bits of both bf16 halves of each dword, kept per
  // half in packed 16-bit lanes (folded to one value after the loop)
  auto chunk_max = [](const uint4& d, us2 m) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7fff7fffu));
    return m;
  };
  auto fold = [](us2 m) { return (uint32_t)max(m.x, m.y); };
  auto quant8 = [](const uint4& d, float s) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return quant8_codes(f, s);
  };
  us2 mh = {0, 0};
  uint32_t m;
  if constexpr (CPL > 0) {
    // chunks past the row's end read as zeros (no effect on the max) and
    // their codes are dropped by the store's range check
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + t * cols, 2 * cols);
    const __amdgpu_buffer_rsrc_t rq = row_rsrc(xq + t * cols, cols);
    uint4 v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      v[c] = bload16<kLoadNonTemporal>(rx, 16u * (uint32_t)(lane + kWave * c));
      mh = chunk_max(v[c], mh);
    }
    m = wave_max_dpp(fold(mh));
    const float b = fmaxf(__uint_as_float(m << 16), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
#pragma unroll
    for (int c = 0; c < CPL; ++c) bstore8(quant8(v[c], s), rq, 8u * (uint32_t)(lane + kWave * c));
    if (lane == 0) beta[t] = b;
  } else {
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) mh = chunk_max(src[idx], mh);
    }
    m = wave_max_dpp(fold(mh));
    const float b = fmaxf(__uint_as_float(m << 16), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) dst[idx] = quant8(load_x16(src, idx), s);  // second, last read
    }
    if (lane == 0) beta[t] = b;
  }
}

// ---------------------------------------------------------------------------
// RMSNorm (per-channel weight w, epsilon) fused in front of the absmax
// quantisation: the guide's module normalises x with nn.RMSNorm before the
// absmax step ("Mathematical Formulation", step 4; "End-to-End
// Implementation").  One pass over x: the row stays in registers while
//   r  = float(1 / sqrt(sum x^2 / cols + eps))   (exact squares, double lane
//        partials (two chains each) summed across the wave by DPP exchanges,
//        the rest in double, one rounding to float; 0 when the root's
//        argument is 0),
//   n  = (x * r) * w             (two float multiplies),
// then beta, s and x~ exactly as act_quant_kernel does on n.  The weight
// (4 B per channel) is shared by every token and stays in L2; a lane
// requests its weights together with its x chunks.
// ---------------------------------------------------------------------------
template <int CPL>  // 8-element chunks per lane; 0 = long rows (three passes)
__global__ __launch_bounds__(256) void rmsnorm_act_quant_kernel(const uint16_t* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                float eps, int64_t tokens,
                                                                int64_t cols,
                                                                int8_t* __restrict__ xq,
                                                                float* __restrict__ beta) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (t >= tokens) return;
  const int64_t nchunks = cols >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * cols);
  const float4* wsrc = reinterpret_cast<const float4*>(w);
  uint2* dst = reinterpret_cast<uint2*>(xq + t * cols);
  auto widen = [](const uint4& d, float (&f)[8]) {
    const uint32_t q[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(q[i] << 16);
      f[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  };
  // exact squares in double (a float square can overflow or lose bits),
  // even and odd elements summed in two chains; a bf16 square has at most
  // 16 significant bits and stays in double's normal range, so the fused
  // multiply-add rounds exactly as the separate add of the exact product
  auto chunk_ss = [&](const uint4& d, double (&s)[2]) {
    float f[8];
    widen(d, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e & 1] = __builtin_fma((double)f[e], (double)f[e], s[e & 1]);
  };
  auto normalise = [&](const uint4& d, int64_t idx, float r, float (&n)[8]) {
    float f[8];
    widen(d, f);
    const float4 w0 = wsrc[2 * idx], w1 = wsrc[2 * idx + 1];
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = (f[e] * r) * wv[e];
  };
  auto normalise_w = [&](const uint4& d, const float4 (&wq)[2], float r, float (&n)[8]) {
    float f[8];
    widen(d, f);
    const float wv[8] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w, wq[1].x, wq[1].y, wq[1].z, wq[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = (f[e] * r) * wv[e];
  };
  // max |n| as a float (finite, non-negative: ordered like its bits)
  auto nmax = [](const float (&n)[8], float m) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(n[e]));
    return m;
  };
  auto quant8 = [](const float (&n)[8], float s) { return quant8_codes(n, s); };
  // r = float(1 / sqrt(sum/cols + eps)) in double (correctly rounded divide
  // and root), one rounding to float; 0 for an all-zero row at eps = 0
  auto inv_rms = [&](double ss) {
    const double d = ss / (double)cols + (double)eps;
    return d > 0.0 ? (float)(1.0 / sqrt(d)) : 0.0f;
  };
  if constexpr (CPL > 0) {
    // With at most two chunks per lane, the lane's weights are requested
    // together with its x chunks (a longer row would hold too many
    // registers: 183 instead of 122 VGPRs at ten chunks).  Chunks past the
    // row's end read x = 0 and w = 0: their squares add nothing, their n is
    // 0 or NaN (0 * r with r = inf), neither of which moves the float max
    // of magnitudes, and their codes are dropped by the store's range check.
    constexpr bool kEarlyW = CPL <= 2;
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + t * cols, 2 * cols);
    const __amdgpu_buffer_rsrc_t rw = row_rsrc(w, 4 * cols);
    const __amdgpu_buffer_rsrc_t rq = row_rsrc(xq + t * cols, cols);
    uint4 v[CPL];
    float4 wl[kEarlyW ? CPL : 1][2];
    double ss[2] = {0.0, 0.0};
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint32_t idx = (uint32_t)(lane + kWave * c);
      v[c] = bload16<kLoadNonTemporal>(rx, 16u * idx);
      if constexpr (kEarlyW) {
        wl[c][0] = bload16f(rw, 32u * idx);
        wl[c][1] = bload16f(rw, 32u * idx + 16u);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) chunk_ss(v[c], ss);
    const float r = inv_rms(wave_sum_dpp(ss[0] + ss[1]));
    // Longer rows request their weights only now, in two halves: hoisted
    // above the reduction, or all at once, they would hold their registers
    // alongside x (at ten chunks 133 VGPRs, three waves per SIMD, instead
    // of 128 and four).
    if constexpr (!kEarlyW) __builtin_amdgcn_sched_barrier(0);
    float n[CPL][8];
    float mf = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint32_t idx = (uint32_t)(lane + kWave * c);
      if constexpr (kEarlyW) {
        normalise_w(v[c], wl[c], r, n[c]);
      } else {
        if (c == CPL / 2) __builtin_amdgcn_sched_barrier(0);
        const float4 wq[2] = {bload16f(rw, 32u * idx), bload16f(rw, 32u * idx + 16u)};
        normalise_w(v[c], wq, r, n[c]);
      }
      mf = nmax(n[c], mf);
    }
    const uint32_t m = wave_max_dpp(__float_as_uint(mf));
    const float b = fmaxf(__uint_as_float(m), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
#pragma unroll
    for (int c = 0; c < CPL; ++c) bstore8(quant8(n[c], s), rq, 8u * (uint32_t)(lane + kWave * c));
    if (lane == 0) beta[t] = b;
  } else {
    double ss[2] = {0.0, 0.0};
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) chunk_ss(src[idx], ss);
    }
    const float r = inv_rms(wave_sum_dpp(ss[0] + ss[1]));
    float mf = 0.f;
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) {
        float n[8];
        normalise(src[idx], idx, r, n);
        mf = nmax(n, mf);
      }
    }
    const uint32_t m = wave_max_dpp(__float_as_uint(mf));
    const float b = fmaxf(__uint_as_float(m), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) {
        float n[8];
        normalise(load_x16(src, idx), idx, r, n);  // third, last read
        dst[idx] = quant8(n, s);
      }
    }
    if (lane == 0) beta[t] = b;
  }
}

hipError_t launch_rmsnorm_act_quant(const uint16_t* x, const float* w, float eps, int64_t tokens,
                                    int64_t cols, int8_t* xq, float* beta, hipStream_t stream) {
  const int64_t need = (cols / 8 + kWave - 1) / kWave;
  const dim3 grid((unsigned)((tokens + 3) / 4)), block(256);
#define SBL_RQ(C) \
  hipLaunchKernelGGL(rmsnorm_act_quant_kernel<C>, grid, block, 0, stream, x, w, eps, tokens, cols, xq, beta)
  if (need <= 1) SBL_RQ(1);
  else if (need <= 2) SBL_RQ(2);
  else if (need <= 4) SBL_RQ(4);
  else if (need <= 6) SBL_RQ(6);
  else if (need <= 8) SBL_RQ(8);
  else if (need <= 10) SBL_RQ(10);
  else if (need <= 12) SBL_RQ(12);
  else SBL_RQ(0);
#undef SBL_RQ
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* x, int64_t tokens, int64_t cols, int8_t* xq,
                            float* beta, hipStream_t stream) {
  const int64_t need = (cols / 8 + kWave - 1) / kWave;
  const dim3 grid((unsigned)((tokens + 3) / 4)), block(256);
#define SBL_AQ(C) hipLaunchKernelGGL(act_quant_kernel<C>, grid, block, 0, stream, x, tokens, cols, xq, beta)
  if (need <= 1) SBL_AQ(1);
  else if (need <= 2) SBL_AQ(2);
  else if (need <= 4) SBL_AQ(4);
  else if (need <= 6) SBL_AQ(6);
  else if (need <= 8) SBL_AQ(8);
  else if (need <= 10) SBL_AQ(10);
  else if (need <= 12) SBL_AQ(12);
  else if (need <= 16) SBL_AQ(16);
  else SBL_AQ(0);
#undef SBL_AQ
  return hipGetLastError();
}

}  // namespace sbl
