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
#include <type_traits>

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
// smfmac GEMM for problems with fewer 256 x 256 tiles than CUs (or N % 4 !=
// 0): the structure of the dense small-tile kernel (persistent blocks over
// XCD-contiguous tile ranges, flattened (tile, k-step) loop, two register
// stages, double-buffered LDS), one 64-wide k step per stage and one smfmac
// per 32x32 tile pair per step.
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

// ---------------------------------------------------------------------------
// Warp-specialised smfmac kernel for problems with at least one 256 x 256
// tile per CU: the structure of the dense warp-specialised product (one
// persistent 768-thread block per CU, 8 math and 4 loader waves, 128-wide
// k steps two ahead in registers, double-buffered LDS, XCD-contiguous tile
// ranges), with the weights as the sparse A operand.
//  * Math wave w holds 128 (o) x 64 (t) int32 accumulators (waves 2 (o) x
//    4 (t) over the tile) and runs two smfmac blocks of 64 k per step.
//  * Per step and weight row a loader thread reads the 32 image bytes of
//    the two blocks and stores the four packed 16-value halves and the four
//    index words as they are, each as [block][row][half] dwords, so one
//    32-bit read per lane covers 64 banks; the math waves expand a half's
//    values to int8 right before its smfmac (a quarter of the LDS bytes of
//    staging int8 values: down 896 x 4864 ran 10% faster).  Every fragment
//    address is one per-lane base plus a constant.
//  * Epilogue: the A-operand layout gives lane l token l%32 and four
//    consecutive features per register group, so each 32 x 32 block passes
//    through a per-wave LDS patch (row = token) and returns as 16-byte
//    pieces, eight lanes per 128-byte row of y: every store writes whole
//    lines.
namespace spws {
constexpr int BO = 256, BT = 256, BK = 128, NT = 768;
constexpr int MATH = 8;
constexpr int XS = BK + 16;  // bytes per staged x~ row
constexpr int WO = 128, WT = 64;
constexpr int TO = WO / 32, TT = WT / 32;
constexpr int XQ = BT / 32;
constexpr int ES = 144;  // bytes per row of the epilogue patch (padded: 16 rows x 16 B hit all banks)
}  // namespace spws

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sp_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)min(bytes, (int64_t)INT32_MAX), 0x00020000);
}

__device__ __forceinline__ uint4 sp_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// y is written once and never read back: its stores carry the non-temporal
// policy (bit 1 of the policy operand).
constexpr int kSpStoreNonTemporal = 2;

template <bool SCALE_BF16>
__global__ __launch_bounds__(spws::NT, 1) void gemm_sp24_ws_kernel(Sp24Args a) {
  using namespace spws;
  __shared__ __attribute__((aligned(16))) int8_t sX[2][BT * XS];       // x~ rows (tokens)
  __shared__ __attribute__((aligned(16))) uint32_t sV[2][2][BO * 2];   // packed kept values, [row][half]
  __shared__ __attribute__((aligned(16))) uint32_t sI[2][2][BO * 2];   // index words
  __shared__ __attribute__((aligned(16))) float sG[2][BO];             // row scales, by tile parity
  __shared__ __attribute__((aligned(16))) float sBt[2][BT];            // beta/127, by tile parity
  __shared__ __attribute__((aligned(16))) int8_t sE[MATH][32 * ES];          // epilogue patches

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = a.K, N = a.N, T = a.T;
  const int rowbytes = (int)(K >> 2);
  const int KB = (int)(K >> 6);  // 64-wide smfmac blocks
  const int KT = (KB + 1) >> 1;  // 128-wide steps

  const SpTileRange tr = sp_tile_range(blockIdx.x, gridDim.x, a.ntiles);
  if (tr.first >= tr.end) return;
  const int total = ((tr.end - tr.first + tr.step - 1) / tr.step) * KT;
  const int total2 = (total + 1) & ~1;  // both roles pass the same (even) number of barriers

  if (wave < MATH) {
    // ------------------------------ math waves ------------------------------
    const int wo = wave & 1, wt = wave >> 1;
    const int G = lane >> 5, l32 = lane & 31;
    v16i acc[TO][TT];
#pragma unroll
    for (int i = 0; i < TO; ++i)
#pragma unroll
      for (int j = 0; j < TT; ++j) acc[i][j] = v16i{};

    auto epilogue = [&](int tile, int par) {
      const int64_t o0 = (int64_t)(tile % a.tiles_o) * BO;
      const int64_t t0 = (int64_t)(tile / a.tiles_o) * BT;
      const int64_t rows_t = min((int64_t)BT, T - t0);
      const int N4 = (int)N * 4;
      const __amdgpu_buffer_rsrc_t ry = sp_rsrc(a.y + t0 * N, rows_t * N * 4);
      const __amdgpu_buffer_rsrc_t ra =
          sp_rsrc(a.acc ? static_cast<const void*>(a.acc + t0 * N) : a.y, a.acc ? rows_t * N * 4 : 0);
      int8_t* const e = sE[wave];
      // the patch addresses are recomputed here from an opaque copy of the
      // lane (kept live through the products they would spill)
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
      const int G = ln >> 5, l32 = ln & 31;
      const int rr = ln >> 3, cc = ln & 7;  // read-back: rows rr + 8v, 16-byte unit cc
#pragma unroll
      for (int i = 0; i < TO; ++i) {
        const int ol = wo * WO + i * 32 + 4 * cc;
        const float4 g = *reinterpret_cast<const float4*>(&sG[par][ol]);
        const uint32_t vo = o0 + ol < N ? (uint32_t)((o0 + ol) * 4) : 0x80000000u;  // past N: dropped
#pragma unroll
        for (int j = 0; j < TT; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<v4i*>(e + l32 * ES + 16 * (2 * q + G)) =
                v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = 8 * v + rr;
            const v4i c = *reinterpret_cast<const v4i*>(e + r * ES + 16 * cc);
            const int tl = wt * WT + j * 32 + r;
            const float bt = sBt[par][tl];
            const uint32_t off = vo + (uint32_t)(tl * N4);
            const v4i yv = v4i{(int)__float_as_uint(((float)c.x * bt) * g.x),
                               (int)__float_as_uint(((float)c.y * bt) * g.y),
                               (int)__float_as_uint(((float)c.z * bt) * g.z),
                               (int)__float_as_uint(((float)c.w * bt) * g.w)};
            __builtin_amdgcn_raw_buffer_store_b128(yv, ry, (int)off, 0, kSpStoreNonTemporal);
            if (a.acc) __builtin_amdgcn_raw_buffer_store_b128(c, ra, (int)off, 0, 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < TO; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j) acc[i][j] = v16i{};
    };

    // per-lane fragment bases: weight row wo*WO + l32 (+32 i), half G
    // (swapped on rows with bit 3 set); token row wt*WT + l32 (+32 j)
    const int i_off = 2 * (wo * WO + l32) + G;
    const int x_off = (wt * WT + l32) * XS + 32 * G;
    auto mma = [&](auto bufc) {
      constexpr int buf = decltype(bufc)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // the token fragments stay in registers, the weight fragments
        // stream through one 32-row block at a time
        v8i bf[TT];
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          const int8_t* p = sX[buf] + x_off + j * 32 * XS + 64 * kb;
          const v4i lo = *reinterpret_cast<const v4i*>(p);
          const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
          bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < TO; ++i) {
          // the row half's 16 kept values, expanded here (a quarter of the
          // LDS bytes of staging them as int8)
          uint32_t e[4];
          expand16_strided(sV[buf][kb][i_off + 64 * i], e);
          const v4i af = v4i{(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
          const int ix = (int)sI[buf][kb][i_off + 64 * i];
#pragma unroll
          for (int j = 0; j < TT; ++j)
            acc[i][j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(af, bf[j], acc[i][j], ix, 0, 0);
        }
      }
    };

    int tile = tr.first, kt = 0, par = 0;
    auto advance = [&]() {
      if (++kt == KT) {
        epilogue(tile, par);
        kt = 0;
        tile += tr.step;
        par ^= 1;
      }
    };
    __syncthreads();  // step 0 staged
    for (int s = 0; s < total2; s += 2) {
      if (s < total) {
        mma(std::integral_constant<int, 0>{});
        advance();
      }
      __syncthreads();
      if (s + 1 < total) {
        mma(std::integral_constant<int, 1>{});
        advance();
      }
      __syncthreads();
    }
  } else {
    // ----------------------------- loader waves -----------------------------
    // Thread lt stages image row lt (32 bytes per step) and x~ rows
    // x_row + 32 q (q < 8), bytes x_part..+16 of the step's 128.  The values
    // of a block past K (K % 128 == 64) are zeroed when staged, which makes
    // whatever x~ and index bits sit there irrelevant.
    const int lt = tid - MATH * 64;
    const int x_row = lt >> 3, x_part = (lt & 7) * 16;
    const int c_vbase = lt * rowbytes;
    const int x_vbase = x_row * (int)K + x_part;
    const int x_q = 32 * (int)K;
    int8_t* const xdst = &sX[0][x_row * XS + x_part];

    int ld_tile = tr.first, ld_kt = 0, ld_par = 0;
    int64_t ld_o0 = 0, ld_t0 = 0;
    __amdgpu_buffer_rsrc_t rc, rx;
    auto rebase = [&]() {
      ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BO;
      ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BT;
      rc = sp_rsrc(a.sp + ld_o0 * rowbytes, min((int64_t)BO, N - ld_o0) * rowbytes);
      rx = sp_rsrc(a.xq + ld_t0 * K, min((int64_t)BT, T - ld_t0) * K);
    };
    rebase();

    uint4 c0, c1, d0, d1, x0[XQ], x1[XQ];
    uint32_t g0, g1, b0, b1;
    int kt0, kt1, par0, par1;
#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    kt##S = ld_kt;                                                                      \
    par##S = ld_par;                                                                    \
    c##S = sp_load16(rc, c_vbase + 32 * ld_kt);                                         \
    d##S = sp_load16(rc, c_vbase + 32 * ld_kt + 16);                                    \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q) x##S[q] = sp_load16(rx, x_vbase + q * x_q + BK * ld_kt); \
    const int64_t so_ = min(ld_o0 + lt, N - 1);                                         \
    g##S = SCALE_BF16 ? (uint32_t)reinterpret_cast<const uint16_t*>(a.scale)[so_] << 16 \
                      : reinterpret_cast<const uint32_t*>(a.scale)[so_];                \
    b##S = reinterpret_cast<const uint32_t*>(a.beta)[min(ld_t0 + lt, T - 1)];           \
    if (++ld_kt == KT) {                                                                \
      if (ld_tile + tr.step < tr.end) {                                                 \
        ld_kt = 0;                                                                      \
        ld_tile += tr.step;                                                             \
        ld_par ^= 1;                                                                    \
        rebase();                                                                       \
      } else {                                                                          \
        ld_kt = KT - 1;                                                                 \
      }                                                                                 \
    }                                                                                   \
  }
#define SBL_WRITE(S, buf)                                                               \
  {                                                                                     \
    const bool ka_ = 2 * kt##S < KB, kb_ = 2 * kt##S + 1 < KB;                          \
    *reinterpret_cast<uint2*>(&sV[buf][0][2 * lt]) = ka_ ? make_uint2(c##S.x, c##S.z) : make_uint2(0u, 0u); \
    *reinterpret_cast<uint2*>(&sV[buf][1][2 * lt]) = kb_ ? make_uint2(d##S.x, d##S.z) : make_uint2(0u, 0u); \
    *reinterpret_cast<uint2*>(&sI[buf][0][2 * lt]) = make_uint2(c##S.y, c##S.w);       \
    *reinterpret_cast<uint2*>(&sI[buf][1][2 * lt]) = make_uint2(d##S.y, d##S.w);       \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q)                                      \
      *reinterpret_cast<uint4*>(xdst + (buf) * (BT * XS) + q * 32 * XS) = x##S[q];      \
    if (kt##S == 0) {                                                                   \
      sBt[par##S][lt] = __fdiv_rn(__uint_as_float(b##S), 127.0f);                       \
      sG[par##S][lt] = __uint_as_float(g##S);                                           \
    }                                                                                   \
  }

    SBL_LOAD(0);
    SBL_WRITE(0, 0);
    SBL_LOAD(1);
    SBL_LOAD(0);
    __syncthreads();
    for (int s = 0; s < total2; s += 2) {
      if (s + 1 < total) SBL_WRITE(1, 1);  // step s+1
      SBL_LOAD(1);                         // step s+3
      __asm__ volatile("" ::: "memory");
      __syncthreads();
      if (s + 2 < total) SBL_WRITE(0, 0);  // step s+2
      SBL_LOAD(0);                         // step s+4
      __asm__ volatile("" ::: "memory");
      __syncthreads();
    }
#undef SBL_LOAD
#undef SBL_WRITE
  }
}

hipError_t launch_gemm_sparse24(const int8_t* xq, const float* beta, const void* sp,
                                const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N,
                                float* y, int32_t* acc, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  Sp24Args a{xq, beta, reinterpret_cast<const uint8_t*>(sp), scale, y, acc, T, K, N, scale_bf16,
             (N % 4) == 0, 0, 0};
  const int64_t ws_o = (N + spws::BO - 1) / spws::BO, ws_t = (T + spws::BT - 1) / spws::BT;
  if (ws_o * ws_t > INT32_MAX) return hipErrorInvalidValue;
  // the warp-specialised kernel stores whole 16-byte pieces (N % 4 == 0) and
  // keeps 32-bit buffer offsets within a tile's rows of y
  const int dev = stream_device(stream);
  const int cus = device_cus(dev);
  if (N % 4 == 0 && ws_o * ws_t >= cus && (int64_t)spws::BT * N * 4 < INT32_MAX / 2) {
    a.tiles_o = (int)ws_o;
    a.ntiles = (int)(ws_o * ws_t);
    const int grid = (int)std::min<int64_t>(a.ntiles, cus);
    if (scale_bf16)
      hipLaunchKernelGGL(gemm_sp24_ws_kernel<true>, dim3((unsigned)grid), dim3(spws::NT), 0, stream, a);
    else
      hipLaunchKernelGGL(gemm_sp24_ws_kernel<false>, dim3((unsigned)grid), dim3(spws::NT), 0, stream, a);
    return hipGetLastError();
  }
  a.tiles_o = (int)((N + BM - 1) / BM);
  a.ntiles = (int)((int64_t)a.tiles_o * ((T + BN - 1) / BN));
  static std::atomic<int> occ_cache[kMaxDevices];
  const int occ = per_device_cached(occ_cache, dev, [] {
    return kernel_occupancy(reinterpret_cast<const void*>(gemm_sp24_kernel<BM, BN>), 256, 1);
  });
  const int grid = (int)std::min<int64_t>(a.ntiles, (int64_t)occ * cus);
  hipLaunchKernelGGL((gemm_sp24_kernel<BM, BN>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sbl
