// Prefill product: packed ternary weights x int8 activations on the dense
// int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8).
// "Sparse-BitNet Guide", "Mathematical Formulation of Sparse-BitLinear",
// step 4: y = (x~ W~^T) * beta * gamma / 127 with an integer accumulator.
//
// Design
//  * Weights are the MFMA A operand (rows = output features o), tokens the B
//    operand, so a lane's accumulators hold four consecutive o of one token:
//    the epilogue writes y[t][o..o+3] as one 16-byte store.
//  * 128 x 128 output tiles, 4 waves of 64 x 64.  Blocks are persistent
//    (as many per CU as fit: 126 VGPRs and 40 KB of LDS allow 4) and walk a
//    list of tiles; the (tile, k-step) loop is flattened so the global loads
//    run three 64-wide k steps ahead, across tile boundaries, in two register
//    stages, and the fp32 stores of a finished tile drain while the next
//    tile computes.
//  * Per k step a block loads 128 rows x 16 B of packed codes (one 128-bit
//    load per row) and 128 rows x 64 B of x~, expands the codes to int8 with
//    a v_perm table (00 -> 0, 01 -> +1, 10 -> -1) while writing them to LDS
//    (double-buffered, one barrier per k step).
//  * LDS rows are padded to 80 B so the 16-byte fragment reads of 16
//    consecutive lanes cover all 64 banks once.
//  * Tiles are cut into one contiguous range per XCD (hardware block b runs
//    on XCD b % 8), so the blocks sharing an XCD's L2 work on neighbouring
//    tiles of the same token rows.
//  * Epilogue: y = ((float)acc * (beta_t / 127)) * gamma_o in float; acc is
//    exact (|acc| <= 127*K < 2^24) so y is within 3 float roundings of the
//    exact product.
#include "sbl_device.h"
#include "sbl_launch.h"


namespace sbl {

constexpr int kXcd = 8;

struct GemmArgs {
  const int8_t* xq;
  const float* beta;
  const uint8_t* packed;
  const void* scale;
  float* y;
  int32_t* acc;
  int64_t T, K, N;
  int scale_bf16;
  int vec_store;  // N % 4 == 0: 16-byte stores
  int tiles_o;
  int ntiles;
};

// Tiles of hardware block b in a grid of G blocks: the tiles are cut into
// X = min(8, G) contiguous ranges, one per XCD (block b runs on XCD b % 8);
// the blocks of a range interleave over it, so block b takes tiles
// first, first + step, ... below end.
struct TileRange {
  int first, step, end;
};
__device__ __forceinline__ TileRange tile_range(int b, int G, int ntiles) {
  const int X = G < kXcd ? G : kXcd;
  const int x = b % X;
  TileRange r;
  r.step = (G - x + X - 1) / X;  // blocks in range x
  r.first = (int)((int64_t)ntiles * x / X) + b / X;
  r.end = (int)((int64_t)ntiles * (x + 1) / X);
  return r;
}

template <int BM, int BN, int NSET>
__global__ __launch_bounds__(256, (BM * BN <= 128 * 128) ? 2 : 1) void gemm_i8_kernel(GemmArgs a) {
  constexpr int BK = 64;                       // k per LDS stage
  constexpr int STRIDE = 80;                   // bytes per staged row (64 + 16 pad)
  constexpr int NT = 256;                      // 4 waves, 2 x 2
  constexpr int WTM = BM / 2, WTN = BN / 2;    // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int B_PER = BN * 4 / NT;           // 16-byte x~ chunks per thread
  static_assert(BM <= NT && (B_PER == 2 || B_PER == 4) && (NSET == 1 || NSET == 2), "tile split");

  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * STRIDE];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t K = a.K;
  const int64_t kbytes = K >> 2;  // packed bytes per weight row
  const int KT = (int)(K / BK);

  const TileRange tr = tile_range(blockIdx.x, gridDim.x, a.ntiles);
  if (tr.first >= tr.end) return;
  const int total = ((tr.end - tr.first + tr.step - 1) / tr.step) * KT;
  // load cursor (runs NSET + 1 k steps ahead of the compute cursor)
  int ld_tile = tr.first, ld_kt = 0;
  int64_t ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BM, ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BN;
  // compute cursor
  int cp_tile = tr.first, cp_kt = 0;

  // fixed per-thread parts of the addresses: thread t stages packed row t
  // (t < BM) and x~ chunks (row t/4 + 64 i, 16-byte part t%4)
  const bool a_on = tid < BM;
  const int a_row = tid;
  const int b_row0 = tid >> 2, b_part = (tid & 3) * 16;

  // register stages: set S holds the global data of the k steps it with
  // it % NSET == S until they are written to LDS
  uint4 ra_0, rb0_0, rb1_0, rb2_0, rb3_0;
  uint4 ra_1, rb0_1, rb1_1, rb2_1, rb3_1;

#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    if (a_on) {                                                                         \
      const int r_ = (int)min((int64_t)a_row, a.N - 1 - ld_o0);                         \
      ra_##S = *reinterpret_cast<const uint4*>(a.packed + (ld_o0 + r_) * kbytes + ld_kt * 16); \
    }                                                                                   \
    const int8_t* xb_ = a.xq + ld_t0 * K + ld_kt * BK + b_part;                         \
    const int last_ = (int)min((int64_t)(BN - 1), a.T - 1 - ld_t0);                     \
    rb0_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0, last_) * (int)K);       \
    rb1_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0 + 64, last_) * (int)K);  \
    if constexpr (B_PER == 4) {                                                         \
      rb2_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0 + 128, last_) * (int)K); \
      rb3_##S = *reinterpret_cast<const uint4*>(xb_ + min(b_row0 + 192, last_) * (int)K); \
    }                                                                                   \
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
      int8_t* d_ = sA[buf] + a_row * STRIDE;                                            \
      uint32_t e_[4];                                                                   \
      expand16_natural(ra_##S.x, e_);                                                   \
      *reinterpret_cast<uint4*>(d_) = make_uint4(e_[0], e_[1], e_[2], e_[3]);           \
      expand16_natural(ra_##S.y, e_);                                                   \
      *reinterpret_cast<uint4*>(d_ + 16) = make_uint4(e_[0], e_[1], e_[2], e_[3]);      \
      expand16_natural(ra_##S.z, e_);                                                   \
      *reinterpret_cast<uint4*>(d_ + 32) = make_uint4(e_[0], e_[1], e_[2], e_[3]);      \
      expand16_natural(ra_##S.w, e_);                                                   \
      *reinterpret_cast<uint4*>(d_ + 48) = make_uint4(e_[0], e_[1], e_[2], e_[3]);      \
    }                                                                                   \
    int8_t* s_ = sB[buf] + b_row0 * STRIDE + b_part;                                    \
    *reinterpret_cast<uint4*>(s_) = rb0_##S;                                            \
    *reinterpret_cast<uint4*>(s_ + 64 * STRIDE) = rb1_##S;                              \
    if constexpr (B_PER == 4) {                                                         \
      *reinterpret_cast<uint4*>(s_ + 128 * STRIDE) = rb2_##S;                           \
      *reinterpret_cast<uint4*>(s_ + 192 * STRIDE) = rb3_##S;                           \
    }                                                                                   \
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i af[TM], bf[TN];
      const int koff = kk * 32 + (lane >> 5) * 16;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(sA[buf] + (wm * WTM + i * 32 + (lane & 31)) * STRIDE + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(sB[buf] + (wn * WTN + j * 32 + (lane & 31)) * STRIDE + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  auto epilogue = [&]() {
    const int64_t o0 = (int64_t)(cp_tile % a.tiles_o) * BM;
    const int64_t t0 = (int64_t)(cp_tile / a.tiles_o) * BN;
    // lane holds C[o = 8*(r/4) + 4*(lane/32) + r%4][t = lane%32] of each tile
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

  // one k step: compute from LDS, stage the next step from register set S
  // into the other LDS buffer, refill set S, finish the tile if done
#define SBL_ITER(S)                                                                     \
  {                                                                                     \
    compute(it & 1);                                                                    \
    if (it + 1 < total) SBL_STORE(S, (it + 1) & 1);                                     \
    if (it + 1 + NSET < total) SBL_LOAD(S);                                             \
    if (++cp_kt == KT) {                                                                \
      cp_kt = 0;                                                                        \
      epilogue();                                                                       \
      cp_tile += tr.step;                                                               \
    }                                                                                   \
    __syncthreads();                                                                    \
    ++it;                                                                               \
  }

  // prologue: step 0 staged, steps 1..NSET in registers
  SBL_LOAD(0);
  SBL_STORE(0, 0);
  if constexpr (NSET == 1) {
    if (total > 1) SBL_LOAD(0);
  } else {
    if (total > 1) SBL_LOAD(1);
    if (total > 2) SBL_LOAD(0);
  }
  __syncthreads();

  int it = 0;
  if constexpr (NSET == 1) {
    while (it < total) SBL_ITER(0);
  } else {
    while (it < total) {
      SBL_ITER(1);  // it even: data of step it+1 sits in set 1
      if (it >= total) break;
      SBL_ITER(0);
    }
  }
#undef SBL_ITER
#undef SBL_LOAD
#undef SBL_STORE
}

static int g_num_cus = 0;

static int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <int BM, int BN, int NSET>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  a.tiles_o = (int)((a.N + BM - 1) / BM);
  const int64_t tiles_t = (a.T + BN - 1) / BN;
  a.ntiles = (int)((int64_t)a.tiles_o * tiles_t);
  int occ = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_i8_kernel<BM, BN, NSET>, 256, 0) !=
          hipSuccess || occ < 1)
    occ = 1;
  const int grid = (int)std::min<int64_t>(a.ntiles, (int64_t)occ * num_cus());
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, NSET>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                       const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N, float* y,
                       int32_t* acc, hipStream_t stream) {
  GemmArgs a{xq, beta, packed, scale, y, acc, T, K, N, scale_bf16, (N % 4) == 0, 0, 0};
  return launch_cfg<128, 128, 2>(a, stream);
}

}  // namespace sbl
