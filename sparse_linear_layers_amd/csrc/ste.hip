// Backward pass of the layer with the straight-through estimator ("Sparse-
// BitNet Guide", "Training Stability & The Straight-Through Estimator": the
// gradient passes through the mask and the ternary rounding to the latent
// weights; README "BitLinear": gradients flow through by STE):
//   dw[o,k] = gamma_o * sum_t (dy[t,o] * (beta_t/127)) * x~[t,k]
//   dx[t,k] = sum_o (dy[t,o] * gamma_o) * code[o,k]
//
// Both are products of a float operand with an operand that bf16 holds
// exactly (ternary codes, int8 x~).  They run on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16): each float is split into three bf16 pieces
// (hi = top 8 significant bits, mid, lo), which represent it exactly, so
// every product is exact and only the fp32 accumulation rounds.
//
// One kernel computes C[m, n] = sum_r A(r, m) * B(r, n) over 128 x 128
// output tiles and 32-wide reduction steps staged through LDS, 4 waves of
// 64 x 64:
//   dx: m = token, n = k, r = o;  A = dy * gamma (rows of dy), B = codes
//       (packed rows, expanded and transposed while staged);
//   dw: m = o, n = k, r = token;  A = dy * beta/127 (transposed while
//       staged), B = x~ (transposed while staged).  The token reduction is
//       split over S chunks whose partial tiles go to a caller workspace; a
//       second kernel adds them in chunk order and multiplies by gamma, so
//       the result does not depend on scheduling.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

namespace ste {
constexpr int BM = 128, BN = 128, BR = 32, NT = 256;
constexpr int LS = BR + 8;  // bf16 per staged row (80 B): 16-lane fragment reads hit every bank once
}  // namespace ste

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct SteArgs {
  const float* dy;
  const int8_t* xq;
  const float* beta;
  const uint8_t* packed;
  const float* gamma;
  float* out;        // dx [T, K], or the workspace [S, N, K] of dw partials
  int64_t T, K, N;
  int64_t r_chunk;   // reduction length of one split (dw)
  int tiles_n;
};

// exact three-piece bf16 split of a float
__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t b = __float_as_uint(v);
  const float h = __uint_as_float(b & 0xffff0000u);
  const float r1 = v - h;  // exact: at most 16 significant bits remain
  const float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
  const float r2 = r1 - m;  // exact: at most 8 significant bits
  hi = (uint16_t)(b >> 16);
  mid = (uint16_t)(__float_as_uint(m) >> 16);
  lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

__device__ __forceinline__ uint16_t code_bf16(uint32_t c) {  // 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0
  return c == 1u ? (uint16_t)0x3F80u : c == 2u ? (uint16_t)0xBF80u : (uint16_t)0u;
}

template <int DW>
__global__ __launch_bounds__(ste::NT, 2) void ste_kernel(SteArgs a) {
  using namespace ste;
  __shared__ __attribute__((aligned(16))) uint16_t sA[3][BM * LS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int64_t M = DW ? N : T;     // output rows
  const int64_t R = DW ? T : N;     // reduction length
  const int tile = blockIdx.x;
  const int64_t m0 = (int64_t)(tile / a.tiles_n) * BM;
  const int64_t n0 = (int64_t)(tile % a.tiles_n) * BN;
  const int64_t r_begin = DW ? (int64_t)blockIdx.y * a.r_chunk : 0;
  const int64_t r_end = DW ? min(R, r_begin + a.r_chunk) : R;
  const int64_t kbytes = K >> 2;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int64_t r0 = r_begin; r0 < r_end; r0 += BR) {
    // ---- stage A (three bf16 pieces) and B, [row][r] with r contiguous ----
    if constexpr (!DW) {
      // A[m = t][r = o] = dy[t][o] * gamma[o]: thread: row t = tid/2, o 16*(tid&1)..+16
      const int row = tid >> 1, part = (tid & 1) * 16;
      const int64_t t = min(m0 + row, T - 1);
      uint16_t h[16], md[16], l[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t o = r0 + part + 4 * q + e;
          const float v = o < r_end ? a.dy[t * N + o] * a.gamma[o] : 0.0f;
          split3(v, h[4 * q + e], md[4 * q + e], l[4 * q + e]);
        }
      }
      uint16_t* d0 = &sA[0][row * LS + part];
      uint16_t* d1 = &sA[1][row * LS + part];
      uint16_t* d2 = &sA[2][row * LS + part];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        d0[e] = h[e];
        d1[e] = md[e];
        d2[e] = l[e];
      }
      // B[n = k][r = o] = code[o][k]: thread: row o = tid/8, 16 codes at k = 16*(tid&7)
      const int orow = tid >> 3, kc = (tid & 7) * 16;
      const int64_t o = r0 + orow;
      const bool kin = n0 + kc < K;  // (K % 128 == 64: half of the last k tile is past the row)
      uint32_t w = 0;
      if (o < r_end && kin) w = *reinterpret_cast<const uint32_t*>(a.packed + o * kbytes + (n0 + kc) / 4);
#pragma unroll
      for (int e = 0; e < 16; ++e) sB[(kc + e) * LS + orow] = kin ? code_bf16((w >> (2 * e)) & 3u) : 0;
    } else {
      // A[m = o][r = t] = dy[t][o] * (beta_t/127): thread: row t = tid/8, o 16*(tid&7)..+16
      const int trow = tid >> 3, oc = (tid & 7) * 16;
      const int64_t t = r0 + trow;
      const bool tin = t < r_end;
      const float s = tin ? a.beta[t] / 127.0f : 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t o = m0 + oc + e;
        const float v = (tin && o < N) ? a.dy[t * N + o] * s : 0.0f;
        uint16_t h, md, l;
        split3(v, h, md, l);
        sA[0][(oc + e) * LS + trow] = h;
        sA[1][(oc + e) * LS + trow] = md;
        sA[2][(oc + e) * LS + trow] = l;
      }
      // B[n = k][r = t] = x~[t][k]: 16 bytes at k = 16*(tid&7)... of row t
      uint4 xv = make_uint4(0u, 0u, 0u, 0u);
      if (tin && n0 + oc < K) xv = *reinterpret_cast<const uint4*>(a.xq + t * K + n0 + oc);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int8_t q = (int8_t)((xw[e >> 2] >> (8 * (e & 3))) & 0xffu);
        sB[(oc + e) * LS + trow] = (uint16_t)(__float_as_uint((float)q) >> 16);  // exact
      }
    }
    __syncthreads();
    // ---- products: 2 x 16 of r, three pieces, 2 x 2 tiles of 32 x 32 ----
#pragma unroll
    for (int kk = 0; kk < BR / 16; ++kk) {
      const int koff = kk * 16 + 8 * (lane >> 5);
      bf16x8 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[(wn * 64 + 32 * j + (lane & 31)) * LS + koff]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sA[p][(wm * 64 + 32 * i + (lane & 31)) * LS + koff]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- store: lane holds C[m = 8*(r/4) + 4*(lane/32) + r%4][n = lane%32] ----
  float* out = a.out + (DW ? (int64_t)blockIdx.y * N * K : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < K) out[m * K + n] = acc[i][j][r];
      }
    }
}

// dw[o, k] = (sum over the S partials, in chunk order) * gamma_o
__global__ __launch_bounds__(256) void ste_dw_reduce_kernel(const float* __restrict__ ws,
                                                            const float* __restrict__ gamma,
                                                            int64_t N, int64_t K, int S,
                                                            float* __restrict__ dw) {
  const int64_t total = N * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = ws[i];
    for (int c = 1; c < S; ++c) s += ws[(int64_t)c * total + i];
    dw[i] = s * gamma[i / K];
  }
}

// Split of the token reduction of dw: enough blocks to cover the CUs twice,
// chunks of at least 512 tokens (a multiple of the 32-token step).
static int ste_splits(int64_t T, int64_t K, int64_t N, int64_t* chunk) {
  if (T <= 0) {  // empty reduction: one pass that writes zeros
    *chunk = ste::BR;
    return 1;
  }
  const int64_t tiles = ((N + ste::BM - 1) / ste::BM) * ((K + ste::BN - 1) / ste::BN);
  int64_t S = std::max<int64_t>(1, std::min<int64_t>((512 + tiles - 1) / tiles, 32));
  S = std::max<int64_t>(1, std::min<int64_t>(S, (T + 511) / 512));
  int64_t c = (T + S - 1) / S;
  c = (c + ste::BR - 1) / ste::BR * ste::BR;
  S = std::max<int64_t>(1, (T + c - 1) / c);
  *chunk = c;
  return (int)S;
}

size_t ste_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  int64_t chunk = 0;
  const int S = ste_splits(T, K, N, &chunk);
  return S > 1 ? (size_t)S * (size_t)N * (size_t)K * sizeof(float) : 0;
}

hipError_t launch_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                               const uint8_t* packed, const float* gamma, int64_t T, int64_t K,
                               int64_t N, float* dx, float* dw, void* workspace,
                               hipStream_t stream) {
  const int tiles_k = (int)((K + ste::BN - 1) / ste::BN);
  if (dx && T > 0) {
    SteArgs a{dy, xq, beta, packed, gamma, dx, T, K, N, 0, tiles_k};
    const int64_t tiles = ((T + ste::BM - 1) / ste::BM) * tiles_k;
    hipLaunchKernelGGL(ste_kernel<0>, dim3((unsigned)tiles), dim3(ste::NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dw && N > 0) {
    int64_t chunk = 0;
    const int S = ste_splits(T, K, N, &chunk);
    float* part = S > 1 ? reinterpret_cast<float*>(workspace) : dw;
    SteArgs a{dy, xq, beta, packed, gamma, part, T, K, N, chunk, tiles_k};
    const int64_t tiles = ((N + ste::BM - 1) / ste::BM) * tiles_k;
    hipLaunchKernelGGL(ste_kernel<1>, dim3((unsigned)tiles, (unsigned)S), dim3(ste::NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = std::min<int64_t>((N * K + 255) / 256, 4096);
    hipLaunchKernelGGL(ste_dw_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       part, gamma, N, K, S, dw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbl
