// Prefill product: packed ternary weights x int8 activations on the dense
// int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8).
// "Sparse-BitNet Guide", "Mathematical Formulation of Sparse-BitLinear",
// step 4: y = (x~ W~^T) * beta * gamma / 127 with an integer accumulator.
//
// Design
//  * Weights are the MFMA A operand (rows = output features o), tokens the B
//    operand, so a lane's accumulators hold four consecutive o of one token:
//    the epilogue writes y[t][o..o+3] as one 16-byte store.
//  * Per 64-wide k step a block loads BM rows x 16 B of packed codes (one
//    128-bit load per row) and BN rows x 64 B of x~, expands the codes to
//    int8 with a v_perm table (00->0, 01->+1, 10->-1) and stages both tiles
//    in LDS; global loads of step k+1 are in flight while step k computes.
//  * LDS rows are padded to 80 B so the 16-byte fragment reads of 16
//    consecutive lanes cover all 64 banks once.
//  * Blocks are renumbered so that the tiles sharing one token tile run on
//    the same XCD (each XCD has its own L2).
//  * Epilogue: y = ((float)acc * (beta_t / 127)) * gamma_o in float; acc is
//    exact (|acc| <= 127*K < 2^24) so y is within 3 float roundings of the
//    exact product.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

constexpr int kBK = 64;           // k per LDS stage
constexpr int kLdsStride = 80;    // bytes per staged row (64 + 16 pad)

struct GemmArgs {
  const int8_t* xq;
  const float* beta;
  const uint8_t* packed;
  const void* scale;
  float* y;
  int32_t* acc;
  int64_t T, K, N;
  int scale_bf16;
  int vec_store;   // N % 4 == 0: 16-byte stores
  int tiles_o;     // number of o tiles
  int nblocks;
};

// Map the hardware block id to a logical tile so that consecutive logical
// tiles (same token tile, neighbouring o tiles) land on one XCD: hardware
// dispatches block b to XCD b % 8.
__device__ __forceinline__ int xcd_swizzle(int b, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;
  if (b >= per * kXcd) return b;  // ragged tail keeps its id
  return (b % kXcd) * per + b / kXcd;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_i8_kernel(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int A_PER = (BM + NT - 1) / NT;    // packed rows per thread
  constexpr int B_PER = BN * 4 / NT;           // 16-byte x~ chunks per thread
  static_assert(BN * 4 % NT == 0, "B tile split");
  static_assert(BM % NT == 0 || NT % BM == 0, "A tile split");

  __shared__ __attribute__((aligned(16))) int8_t sA[BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int tile = xcd_swizzle(blockIdx.x, a.nblocks);
  const int64_t o0 = (int64_t)(tile % a.tiles_o) * BM;
  const int64_t t0 = (int64_t)(tile / a.tiles_o) * BN;
  const int64_t K = a.K;
  const int64_t kbytes = K >> 2;  // packed bytes per weight row

  // global source rows (clamped: rows past the edge compute garbage that is
  // never stored)
  const uint8_t* a_src[A_PER];
  int a_row[A_PER];
  bool a_on[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int r = tid + i * NT;
    a_on[i] = r < BM;
    a_row[i] = r;
    const int64_t o = min(o0 + r, a.N - 1);
    a_src[i] = a.packed + o * kbytes;
  }
  const int8_t* b_src[B_PER];
  int b_dst[B_PER];
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int ci = tid + i * NT;
    const int r = ci >> 2, part = ci & 3;
    const int64_t t = min(t0 + r, a.T - 1);
    b_src[i] = a.xq + t * K + part * 16;
    b_dst[i] = r * kLdsStride + part * 16;
  }

  uint4 a_reg[A_PER];
  uint4 b_reg[B_PER];
  auto load_tile = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      if (a_on[i]) a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + kt * 16);
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      b_reg[i] = *reinterpret_cast<const uint4*>(b_src[i] + kt * kBK);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      if (!a_on[i]) continue;
      const uint32_t w[4] = {a_reg[i].x, a_reg[i].y, a_reg[i].z, a_reg[i].w};
      int8_t* dst = sA + a_row[i] * kLdsStride;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t e[4];
        expand16_natural(w[q], e);
        *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(e[0], e[1], e[2], e[3]);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) *reinterpret_cast<uint4*>(sB + b_dst[i]) = b_reg[i];
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  const int64_t KT = K / kBK;
  load_tile(0);
  for (int64_t kt = 0; kt < KT; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i af[TM], bf[TN];
      const int koff = kk * 32 + (lane >> 5) * 16;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(sA + (wm * WTM + i * 32 + (lane & 31)) * kLdsStride + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(sB + (wn * WTN + j * 32 + (lane & 31)) * kLdsStride + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds C[o = 8*(r/4) + 4*(lane/32) + r%4][t = lane%32]
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t t = t0 + wn * WTN + j * 32 + (lane & 31);
    if (t >= a.T) continue;
    const float bt = __fdiv_rn(a.beta[t], 127.0f);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t o = o0 + wm * WTM + i * 32 + 8 * r4 + 4 * (lane >> 5);
        if (o >= a.N) continue;
        int32_t c[4];
        float yv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = acc[i][j][4 * r4 + e];
          const int64_t oe = min(o + e, a.N - 1);
          yv[e] = ((float)c[e] * bt) * load_scale(a.scale, a.scale_bf16, oe);
        }
        float* yp = a.y + t * a.N + o;
        int32_t* ap = a.acc ? a.acc + t * a.N + o : nullptr;
        if (a.vec_store) {
          *reinterpret_cast<float4*>(yp) = make_float4(yv[0], yv[1], yv[2], yv[3]);
          if (ap) *reinterpret_cast<int4*>(ap) = make_int4(c[0], c[1], c[2], c[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (o + e < a.N) {
              yp[e] = yv[e];
              if (ap) ap[e] = c[e];
            }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  a.tiles_o = (int)((a.N + BM - 1) / BM);
  const int64_t tiles_t = (a.T + BN - 1) / BN;
  const int64_t nb = (int64_t)a.tiles_o * tiles_t;
  a.nblocks = (int)nb;
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN>), dim3((unsigned)nb), dim3(WM * WN * 64), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                       const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N, float* y,
                       int32_t* acc, hipStream_t stream) {
  GemmArgs a{xq, beta, packed, scale, y, acc, T, K, N, scale_bf16, (N % 4) == 0, 0, 0};
  if (N >= 1024 && (N % 256 == 0 || N > 2048)) return launch_cfg<256, 128, 2, 2>(a, stream);
  return launch_cfg<128, 128, 2, 2>(a, stream);
}

}  // namespace sbl
