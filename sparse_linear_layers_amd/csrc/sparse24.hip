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
// smfmac GEMM: the structure of the dense product kernel (persistent blocks
// over XCD-contiguous tile ranges, flattened (tile, k-step) loop, two
// register stages, double-buffered LDS), one 64-wide k step per stage and
// one smfmac per 32x32 tile pair per step.
// ---------------------------------------------------------------------------
struct Sp24Args {
  const int8_t* xq;
  const float* beta;
  const uint8_t* sp;
  const void* scale;
  float* y;
  int32_t* acc;
  int64_t T, K, N;
  int scale_bf16;
  int vec_store;
  int tiles_o;
  int ntiles;
};

struct SpTileRange {
  int first, step, end;
};
__device__ __forceinline__ SpTileRange sp_tile_range(int b, int G, int ntiles) {
  constexpr int kXcd = 8;
  const int X = G < kXcd ? G : kXcd;
  const int x = b % X;
  SpTileRange r;
  r.step = (G - x + X - 1) / X;
  r.first = (int)((int64_t)ntiles * x / X) + b / X;
  r.end = (int)((int64_t)ntiles * (x + 1) / X);
  return r;
}

template <int BM, int BN>
__global__ __launch_bounds__(256, 2) void gemm_sp24_kernel(Sp24Args a) {
  constexpr int AST = 48;                      // bytes per staged weight row: 2 x 16 values + pad
  constexpr int BST = 80;                      // bytes per staged token row: 64 + pad
  constexpr int NT = 256;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int B_PER = BN * 4 / NT;
  static_assert(BM <= NT && B_PER == 2, "tile split");

  __shared__ __attribute__((aligned(16))) int8_t sAv[2][BM * AST];
  __shared__ uint32_t sAi[2][BM * 2];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * BST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t K = a.K;
  const int64_t rowbytes = K >> 2;  // image bytes per weight row (16 per 64-wide k block)
  const int KT = (int)(K >> 6);

  const SpTileRange tr = sp_tile_range(blockIdx.x, gridDim.x, a.ntiles);
  if (tr.first >= tr.end) return;
  const int total = ((tr.end - tr.first + tr.step - 1) / tr.step) * KT;
  int ld_tile = tr.first, ld_kt = 0;
  int64_t ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BM, ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BN;
  int cp_tile = tr.first, cp_kt = 0;

  const bool a_on = tid < BM;
  const int a_row = tid;
  const int b_row0 = tid >> 2, b_part = (tid & 3) * 16;

  uint4 ra_0, rb0_0, rb1_0;
  uint4 ra_1, rb0_1, rb1_1;

#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    if (a_on) {                                                                         \
      const int r_ = (int)min((int64_t)a_row, a.N - 1 - ld_o0);                         \
      ra_##S = *reinterpret_cast<const uint4*>(a.sp + (ld_o0 + r_) * rowbytes + ld_kt * 16); \
    }                                                                                   \
    const int8_t* xb_ = a.xq + ld_t0 * K + ld_kt * 64 + b_part;                         \
    const int last_ = (int)min((int64_t)(BN - 1), a.T - 1 - ld_t0);                     \
    rb0_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0, last_) * (int)K);       \
    rb1_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0 + 64, last_) * (int)K);  \
    if (++ld_kt == KT) {                                                                \
      ld_kt = 0;                                                                        \
      ld_tile += tr.step;                                                               \
      ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BM;                                      \
      ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BN;                                      \
    }                                                                                   \
  }

#define SBL_STORE(S, buf)                                                               \
  {                                                                                     \
    if (a_on) {                                                                         \
      uint32_t e_[4];                                                                   \
      expand16_strided(ra_##S.x, e_);                                                   \
      *reinterpret_cast<uint4*>(sAv[buf] + a_row * AST) = make_uint4(e_[0], e_[1], e_[2], e_[3]); \
      expand16_strided(ra_##S.z, e_);                                                   \
      *reinterpret_cast<uint4*>(sAv[buf] + a_row * AST + 16) = make_uint4(e_[0], e_[1], e_[2], e_[3]); \
      *reinterpret_cast<uint2*>(&sAi[buf][a_row * 2]) = make_uint2(ra_##S.y, ra_##S.w);  \
    }                                                                                   \
    int8_t* s_ = sB[buf] + b_row0 * BST + b_part;                                       \
    *reinterpret_cast<uint4*>(s_) = rb0_##S;                                            \
    *reinterpret_cast<uint4*>(s_ + 64 * BST) = rb1_##S;                                 \
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  auto compute = [&](int buf) {
    const int G = lane >> 5;
    v4i af[TM];
    int ai[TM];
    v8i bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      af[i] = *reinterpret_cast<const v4i*>(sAv[buf] + r * AST + 16 * G);
      ai[i] = (int)sAi[buf][r * 2 + G];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int8_t* p = sB[buf] + (wn * WTN + j * 32 + (lane & 31)) * BST + 32 * G;
      const v4i lo = *reinterpret_cast<const v4i*>(p);
      const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(af[i], bf[j], acc[i][j], ai[i], 0, 0);
  };

  auto epilogue = [&]() {
    const int64_t o0 = (int64_t)(cp_tile % a.tiles_o) * BM;
    const int64_t t0 = (int64_t)(cp_tile / a.tiles_o) * BN;
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) {
      const int64_t t = t0 + wn * WTN + jn * 32 + (lane & 31);
      const bool t_ok = t < a.T;
      const float bt = __fdiv_rn(a.beta[t_ok ? t : 0], 127.0f);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int64_t o = o0 + wm * WTM + i * 32 + 8 * r4 + 4 * (lane >> 5);
          if (!t_ok || o >= a.N) continue;
          int32_t c[4];
          float yv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            c[e] = acc[i][jn][4 * r4 + e];
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
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) acc[i][jn] = v16i{};
  };

#define SBL_ITER(S)                                                                     \
  {                                                                                     \
    compute(it & 1);                                                                    \
    if (it + 1 < total) SBL_STORE(S, (it + 1) & 1);                                     \
    if (it + 3 < total) SBL_LOAD(S);                                                    \
    if (++cp_kt == KT) {                                                                \
      cp_kt = 0;                                                                        \
      epilogue();                                                                       \
      cp_tile += tr.step;                                                               \
    }                                                                                   \
    __syncthreads();                                                                    \
    ++it;                                                                               \
  }

  SBL_LOAD(0);
  SBL_STORE(0, 0);
  if (total > 1) SBL_LOAD(1);
  if (total > 2) SBL_LOAD(0);
  __syncthreads();
  int it = 0;
  while (it < total) {
    SBL_ITER(1);
    if (it >= total) break;
    SBL_ITER(0);
  }
#undef SBL_ITER
#undef SBL_LOAD
#undef SBL_STORE
}

static int sp_num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

hipError_t launch_gemm_sparse24(const int8_t* xq, const float* beta, const void* sp,
                                const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N,
                                float* y, int32_t* acc, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  Sp24Args a{xq, beta, reinterpret_cast<const uint8_t*>(sp), scale, y, acc, T, K, N, scale_bf16,
             (N % 4) == 0, 0, 0};
  a.tiles_o = (int)((N + BM - 1) / BM);
  a.ntiles = (int)((int64_t)a.tiles_o * ((T + BN - 1) / BN));
  int occ = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_sp24_kernel<BM, BN>, 256, 0) !=
          hipSuccess || occ < 1)
    occ = 1;
  const int grid = (int)std::min<int64_t>(a.ntiles, (int64_t)occ * sp_num_cus());
  hipLaunchKernelGGL((gemm_sp24_kernel<BM, BN>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sbl
