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

template <int CPL>  // 8-element (16-byte) chunks per lane; 0 = long-row loop
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                        int64_t tokens, int64_t cols,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ beta) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const int64_t nchunks = cols >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * cols);
  uint2* dst = reinterpret_cast<uint2*>(xq + t * cols);
  auto chunk_max = [](const uint4& d, uint32_t m) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
    return m;
  };
  auto quant8 = [](const uint4& d, float s) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float f = __uint_as_float(h ? (w[i] & 0xffff0000u) : (w[i] << 16));
        float q = rintf(f * s);
        q = fminf(fmaxf(q, -128.f), 127.f);
        const uint32_t b = (uint32_t)(int32_t)q & 0xffu;
        out[i >> 1] |= b << (8 * (2 * (i & 1) + h));
      }
    }
    return make_uint2(out[0], out[1]);
  };
  uint32_t m = 0;
  if constexpr (CPL > 0) {
    uint4 v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t idx = lane + (int64_t)kWave * c;
      v[c] = idx < nchunks ? load_x16(src, idx) : make_uint4(0u, 0u, 0u, 0u);
      m = chunk_max(v[c], m);
    }
    m = wave_max(m);
    const float b = fmaxf(__uint_as_float(m << 16), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t idx = lane + (int64_t)kWave * c;
      if (idx < nchunks) dst[idx] = quant8(v[c], s);
    }
    if (lane == 0) beta[t] = b;
  } else {
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) m = chunk_max(src[idx], m);
    }
    m = wave_max(m);
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
//        partials + butterfly, the rest in double, one rounding to float;
//        0 when the root's argument is 0),
//   n  = (x * r) * w             (two float multiplies),
// then beta, s and x~ exactly as act_quant_kernel does on n.  The weight
// (4 B per channel) is shared by every token and stays in L2.
// ---------------------------------------------------------------------------
template <int CPL>  // 8-element chunks per lane; 0 = long rows (three passes)
__global__ __launch_bounds__(256) void rmsnorm_act_quant_kernel(const uint16_t* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                float eps, int64_t tokens,
                                                                int64_t cols,
                                                                int8_t* __restrict__ xq,
                                                                float* __restrict__ beta) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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
  auto chunk_ss = [&](const uint4& d, double s) {
    float f[8];
    widen(d, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (double)f[e] * (double)f[e];
    return s;
  };
  auto normalise = [&](const uint4& d, int64_t idx, float r, float (&n)[8]) {
    float f[8];
    widen(d, f);
    const float4 w0 = wsrc[2 * idx], w1 = wsrc[2 * idx + 1];
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = (f[e] * r) * wv[e];
  };
  auto nmax = [](const float (&n)[8], uint32_t m) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(n[e]) & 0x7fffffffu);
    return m;
  };
  auto quant8 = [](const float (&n)[8], float s) {
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = rintf(n[e] * s);
      q = fminf(fmaxf(q, -128.f), 127.f);
      out[e >> 2] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (e & 3));
    }
    return make_uint2(out[0], out[1]);
  };
  // r = float(1 / sqrt(sum/cols + eps)) in double (correctly rounded divide
  // and root), one rounding to float; 0 for an all-zero row at eps = 0
  auto inv_rms = [&](double ss) {
    const double d = ss / (double)cols + (double)eps;
    return d > 0.0 ? (float)(1.0 / sqrt(d)) : 0.0f;
  };
  if constexpr (CPL > 0) {
    uint4 v[CPL];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t idx = lane + (int64_t)kWave * c;
      v[c] = idx < nchunks ? load_x16(src, idx) : make_uint4(0u, 0u, 0u, 0u);
      ss = chunk_ss(v[c], ss);
    }
    const float r = inv_rms(wave_sum(ss));
    float n[CPL][8];
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t idx = lane + (int64_t)kWave * c;
      if (idx < nchunks) {
        normalise(v[c], idx, r, n[c]);
        m = nmax(n[c], m);
      }
    }
    m = wave_max(m);
    const float b = fmaxf(__uint_as_float(m), 1e-5f);
    const float s = __fdiv_rn(127.0f, b);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t idx = lane + (int64_t)kWave * c;
      if (idx < nchunks) dst[idx] = quant8(n[c], s);
    }
    if (lane == 0) beta[t] = b;
  } else {
    double ss = 0.0;
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) ss = chunk_ss(src[idx], ss);
    }
    const float r = inv_rms(wave_sum(ss));
    uint32_t m = 0;
    for (int64_t base = 0; base < nchunks; base += kWave) {
      const int64_t idx = base + lane;
      if (idx < nchunks) {
        float n[8];
        normalise(src[idx], idx, r, n);
        m = nmax(n, m);
      }
    }
    m = wave_max(m);
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
