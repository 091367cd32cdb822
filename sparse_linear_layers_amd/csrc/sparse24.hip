// 2:4 prefill product on the gfx950 sparse int8 matrix cores
// (v_smfmac_i32_32x32x64_i8).
// "Sparse-BitNet Guide", "The Hardware Mechanics of 2:4 Sparsity": a 2:4
// weight is carried as its kept values plus 2-bit in-group indices, and the
// matrix unit skips the zero half.  The page's layout is NVIDIA's; this one
// is the gfx950 operand image, built here from the packed codes.
//
// Compressed operand ("sparse24", sparse24_bytes(N, K) = N*K/4 bytes, the
// same size as the packed codes): for weight row o, 64-wide k block kb and
// lane half G in {0, 1}, eight bytes
//     word 0: 16 kept values as 2-bit codes (00/01/10), value of slot s at
//             bits [2p, 2p+1] with p = 4*(s%4) + s/4, so that the 3-op
//             strided expansion yields the int8 values in slot order;
//     word 1: the smfmac index word: bits [4*gq + 2*h] = in-group index of
//             slot 2*gq + h (h = 0, 1, ascending within the group).
// Slot group gq = 4*hh + q (hh, q in 0..3 / 0..1) holds the dense columns
//     kb*64 + 32*hh + 16*G + 4*q + {0..3}.
// With that image, the A operand of lane (row o%32, half G) pairs slot
// group gq with B lane group gq/4 bytes 16*G + 4*(gq%4) + index, and B lane
// group h is given x~ columns 32*h .. 32*h + 31 of the block: every kept
// weight meets its own activation.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

__global__ __launch_bounds__(256) void sparse24_compress_kernel(const uint8_t* __restrict__ packed,
                                                                int64_t N, int64_t K,
                                                                uint2* __restrict__ out,
                                                                int32_t* bad_groups) {
  const int64_t kblocks = K >> 6;
  const int64_t total = N * kblocks * 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int G = (int)(i & 1);
  const int64_t kb = (i >> 1) % kblocks;
  const int64_t o = (i >> 1) / kblocks;
  const uint8_t* row = packed + o * (K >> 2);
  uint32_t vals = 0, idxw = 0;
  int bad = 0;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    // 16 codes = 4 bytes: dense columns kb*64 + 32*hh + 16*G + 0..15
    const uint32_t w = *reinterpret_cast<const uint32_t*>(row + kb * 16 + 8 * hh + 4 * G);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t grp = (w >> (8 * q)) & 0xffu;  // 4 codes of one group
      int sel[2];
      int nsel = 0, nnz = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t c = (grp >> (2 * e)) & 3u;
        const bool nz = (c == 1u || c == 2u);
        nnz += nz;
        if (nz && nsel < 2) sel[nsel++] = e;
      }
      bad += nnz > 2;
      // pad with the lowest unused indices, then keep ascending order
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nsel < 2 && !(nsel == 1 && sel[0] == e)) sel[nsel++] = e;
      if (sel[0] > sel[1]) { const int t = sel[0]; sel[0] = sel[1]; sel[1] = t; }
      const int gq = 4 * hh + q;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int s = 2 * gq + h;
        uint32_t c = (grp >> (2 * sel[h])) & 3u;
        if (c == 3u) c = 0u;
        const int p = 4 * (s & 3) + (s >> 2);
        vals |= c << (2 * p);
        idxw |= (uint32_t)sel[h] << (4 * gq + 2 * h);
      }
    }
  }
  out[(o * kblocks + kb) * 2 + G] = make_uint2(vals, idxw);
  if (bad && bad_groups) atomicAdd(bad_groups, bad);
}

hipError_t launch_sparse24_compress(const uint8_t* packed, int64_t N, int64_t K, void* out,
                                    int32_t* bad_groups, hipStream_t stream) {
  const int64_t total = N * (K >> 6) * 2;
  hipLaunchKernelGGL(sparse24_compress_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, packed, N, K, reinterpret_cast<uint2*>(out), bad_groups);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// smfmac GEMM: same block structure as the dense kernel, one 64-wide k step
// per stage and one smfmac per 32x32 tile pair per stage.
// ---------------------------------------------------------------------------
constexpr int kSpBK = 64;
constexpr int kSpAStride = 48;  // bytes per staged weight row: 2 x 16 values + pad
constexpr int kSpBStride = 80;  // bytes per staged token row: 64 + pad

struct Sp24Args {
  const int8_t* xq;
  const float* beta;
  const uint2* sp;
  const void* scale;
  float* y;
  int32_t* acc;
  int64_t T, K, N;
  int scale_bf16;
  int vec_store;
  int tiles_o;
  int nblocks;
};

__device__ __forceinline__ int xcd_swizzle24(int b, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;
  if (b >= per * kXcd) return b;
  return (b % kXcd) * per + b / kXcd;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_sp24_kernel(Sp24Args a) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_PER = (BM + NT - 1) / NT;  // weight rows per thread (16 B each)
  constexpr int B_PER = BN * 4 / NT;
  static_assert(BN * 4 % NT == 0, "B tile split");

  __shared__ __attribute__((aligned(16))) int8_t sAv[BM * kSpAStride];
  __shared__ uint32_t sAi[BM * 2];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * kSpBStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int tile = xcd_swizzle24(blockIdx.x, a.nblocks);
  const int64_t o0 = (int64_t)(tile % a.tiles_o) * BM;
  const int64_t t0 = (int64_t)(tile / a.tiles_o) * BN;
  const int64_t K = a.K;
  const int64_t kblocks = K >> 6;

  const uint4* a_src[A_PER];
  int a_row[A_PER];
  bool a_on[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int r = tid + i * NT;
    a_on[i] = r < BM;
    a_row[i] = r;
    const int64_t o = min(o0 + r, a.N - 1);
    a_src[i] = reinterpret_cast<const uint4*>(a.sp + o * kblocks * 2);
  }
  const int8_t* b_src[B_PER];
  int b_dst[B_PER];
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int ci = tid + i * NT;
    const int r = ci >> 2, part = ci & 3;
    const int64_t t = min(t0 + r, a.T - 1);
    b_src[i] = a.xq + t * K + part * 16;
    b_dst[i] = r * kSpBStride + part * 16;
  }
  uint4 a_reg[A_PER];
  uint4 b_reg[B_PER];
  auto load_tile = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      if (a_on[i]) a_reg[i] = a_src[i][kt];
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      b_reg[i] = *reinterpret_cast<const uint4*>(b_src[i] + kt * kSpBK);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      if (!a_on[i]) continue;
      const uint32_t vw[2] = {a_reg[i].x, a_reg[i].z};
      const uint32_t iw[2] = {a_reg[i].y, a_reg[i].w};
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        uint32_t e[4];
        expand16_strided(vw[G], e);
        *reinterpret_cast<uint4*>(sAv + a_row[i] * kSpAStride + 16 * G) = make_uint4(e[0], e[1], e[2], e[3]);
        sAi[a_row[i] * 2 + G] = iw[G];
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

  load_tile(0);
  for (int64_t kt = 0; kt < kblocks; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < kblocks) load_tile(kt + 1);
    const int G = lane >> 5;
    v4i af[TM];
    int ai[TM];
    v8i bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      af[i] = *reinterpret_cast<const v4i*>(sAv + r * kSpAStride + 16 * G);
      ai[i] = (int)sAi[r * 2 + G];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int8_t* p = sB + (wn * WTN + j * 32 + (lane & 31)) * kSpBStride + 32 * G;
      const v4i lo = *reinterpret_cast<const v4i*>(p);
      const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(af[i], bf[j], acc[i][j], ai[i], 0, 0);
  }

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
static hipError_t launch_sp_cfg(Sp24Args a, hipStream_t stream) {
  a.tiles_o = (int)((a.N + BM - 1) / BM);
  const int64_t nb = (int64_t)a.tiles_o * ((a.T + BN - 1) / BN);
  a.nblocks = (int)nb;
  hipLaunchKernelGGL((gemm_sp24_kernel<BM, BN, WM, WN>), dim3((unsigned)nb), dim3(WM * WN * 64),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_sparse24(const int8_t* xq, const float* beta, const void* sp,
                                const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N,
                                float* y, int32_t* acc, hipStream_t stream) {
  Sp24Args a{xq, beta, reinterpret_cast<const uint2*>(sp), scale, y, acc, T, K, N, scale_bf16,
             (N % 4) == 0, 0, 0};
  if (N >= 1024 && (N % 256 == 0 || N > 2048)) return launch_sp_cfg<256, 128, 2, 2>(a, stream);
  return launch_sp_cfg<128, 128, 2, 2>(a, stream);
}

}  // namespace sbl
