// Prefill product: packed ternary weights x int8 activations on the dense
// int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8).
// "Sparse-BitNet Guide", "Mathematical Formulation of Sparse-BitLinear",
// step 4: y = (x~ W~^T) * beta * gamma / 127 with an integer accumulator.
//
// Two kernels share the contract:
//  * gemm_i8_ws_kernel (below) for problems with at least one 256 x 256 tile
//    per CU: warp-specialised math and loader waves, one block per CU.
//  * gemm_i8_kernel for smaller problems: 128 x 128 tiles, several blocks per
//    CU.  Design of the small kernel:
//  * Weights are the MFMA A operand (rows = output features o), tokens the B
//    operand, so a lane's accumulators hold four consecutive o of one token:
//    the epilogue writes y[t][o..o+3] as one 16-byte store.
//  * 4 waves of 64 x 64.  Blocks are persistent (as many per CU as fit:
//    126 VGPRs and 40 KB of LDS allow 4) and walk a list of tiles; the
//    (tile, k-step) loop is flattened so the global loads run three 64-wide
//    k steps ahead, across tile boundaries, in two register stages, and the
//    fp32 stores of a finished tile drain while the next tile computes.
//  * Per k step a block loads 128 rows x 16 B of packed codes (8 bytes per
//    thread) and 128 rows x 64 B of x~, expands the codes to int8 with
//    a v_perm table (00 -> 0, 01 -> +1, 10 -> -1) while writing them to LDS
//    (double-buffered, one barrier per k step).
//  * LDS rows are padded to 80 B so the 16-byte fragment reads of 16
//    consecutive lanes cover all 64 banks once.
//  * Tiles are cut into one contiguous range per XCD (hardware block b runs
//    on XCD b % 8), so the blocks sharing an XCD's L2 work on neighbouring
//    tiles of the same token rows (both kernels).
//  * Epilogue: y = ((float)acc * (beta_t / 127)) * gamma_o in float; acc is
//    exact (|acc| <= 127*K < 2^24) so y is within 3 float roundings of the
//    exact product (both kernels).
#include <type_traits>

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
  int ntiles;  // whole tiles
  int nhalf;   // warp-specialised kernel: half tiles (along t) after the whole ones
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

// Four consecutive row scales as floats.
__device__ __forceinline__ float4 load_scale4(const void* s, int bf16, int64_t i) {
  if (bf16) {
    const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(s) + i);
    return make_float4(__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                       __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s) + i);
}

template <int BM, int BN, int NSET>
__global__ __launch_bounds__(256, (BM * BN <= 128 * 128) ? 2 : 1) void gemm_i8_kernel(GemmArgs a) {
  constexpr int BK = 64;                       // k per LDS stage
  constexpr int STRIDE = 80;                   // bytes per staged row (64 + 16 pad)
  constexpr int NT = 256;                      // 4 waves, 2 x 2
  constexpr int WTM = BM / 2, WTN = BN / 2;    // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int B_PER = BN * 4 / NT;           // 16-byte x~ chunks per thread
  static_assert(BM * 2 == NT && (B_PER == 2 || B_PER == 4) && (NSET == 1 || NSET == 2), "tile split");

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

  // fixed per-thread parts of the addresses: thread t stages 8 bytes (32
  // codes) of packed row t/2 and x~ chunks (row t/4 + 64 i, 16-byte part t%4)
  const int a_row = tid >> 1, a_part = (tid & 1) * 8;
  const int b_row0 = tid >> 2, b_part = (tid & 3) * 16;

  // register stages: set S holds the global data of the k steps it with
  // it % NSET == S until they are written to LDS
  uint2 ra_0, ra_1;
  uint4 rb0_0, rb1_0, rb2_0, rb3_0;
  uint4 rb0_1, rb1_1, rb2_1, rb3_1;

  // Every load is unconditional and in bounds, so the compiler can wait for
  // exactly the older register set: rows past N or T repeat the last row
  // (their outputs are never stored) and past the block's last step the
  // cursor stays on that step.
#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    const int64_t r_ = min((int64_t)a_row, a.N - 1 - ld_o0);                            \
    ra_##S = *reinterpret_cast<const uint2*>(a.packed + (ld_o0 + r_) * kbytes + ld_kt * 16 + a_part); \
    const int8_t* xb_ = a.xq + ld_t0 * K + ld_kt * BK + b_part;                         \
    const int64_t last_ = min((int64_t)(BN - 1), a.T - 1 - ld_t0);                      \
    rb0_##S = *reinterpret_cast<const uint4*>(xb_ + min((int64_t)b_row0, last_) * K);   \
    rb1_##S = *reinterpret_cast<const uint4*>(xb_ + min((int64_t)b_row0 + 64, last_) * K); \
    if constexpr (B_PER == 4) {                                                         \
      rb2_##S = *reinterpret_cast<const uint4*>(xb_ + min((int64_t)b_row0 + 128, last_) * K); \
      rb3_##S = *reinterpret_cast<const uint4*>(xb_ + min((int64_t)b_row0 + 192, last_) * K); \
    }                                                                                   \
    if (++ld_kt == KT) {                                                                \
      if (ld_tile + tr.step < tr.end) {                                                 \
        ld_kt = 0;                                                                      \
        ld_tile += tr.step;                                                             \
        ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BM;                                    \
        ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BN;                                    \
      } else {                                                                          \
        ld_kt = KT - 1;                                                                 \
      }                                                                                 \
    }                                                                                   \
  }

#define SBL_STORE(S, buf)                                                               \
  {                                                                                     \
    int8_t* d_ = sA[buf] + a_row * STRIDE + 4 * a_part;                                 \
    uint32_t e_[4];                                                                     \
    expand16_natural(ra_##S.x, e_);                                                     \
    *reinterpret_cast<uint4*>(d_) = make_uint4(e_[0], e_[1], e_[2], e_[3]);             \
    expand16_natural(ra_##S.y, e_);                                                     \
    *reinterpret_cast<uint4*>(d_ + 16) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
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

  // lane holds C[o = 8*(r/4) + 4*(lane/32) + r%4][t = lane%32] of each
  // 32 x 32 tile: y[t][o..o+3] is one 16-byte store
  auto epilogue = [&]() {
    const int64_t o0 = (int64_t)(cp_tile % a.tiles_o) * BM;
    const int64_t t0 = (int64_t)(cp_tile / a.tiles_o) * BN;
    const int64_t ob = o0 + wm * WTM + 4 * (lane >> 5);
    int64_t tj[TN];
    float bt[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      tj[j] = t0 + wn * WTN + j * 32 + (lane & 31);
      bt[j] = __fdiv_rn(a.beta[min(tj[j], a.T - 1)], 127.0f);
    }
    if (a.vec_store && o0 + BM <= a.N && t0 + BN <= a.T) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t o = ob + i * 32 + 8 * q;
          const float4 g = load_scale4(a.scale, a.scale_bf16, o);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const v16i& c = acc[i][j];
            const float4 yv = make_float4(((float)c[4 * q] * bt[j]) * g.x, ((float)c[4 * q + 1] * bt[j]) * g.y,
                                          ((float)c[4 * q + 2] * bt[j]) * g.z, ((float)c[4 * q + 3] * bt[j]) * g.w);
            *reinterpret_cast<float4*>(a.y + tj[j] * a.N + o) = yv;
            if (a.acc)
              *reinterpret_cast<int4*>(a.acc + tj[j] * a.N + o) =
                  make_int4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t o = ob + i * 32 + 8 * q + e;
              if (o < a.N && tj[j] < a.T) {
                const int32_t c = acc[i][j][4 * q + e];
                a.y[tj[j] * a.N + o] = ((float)c * bt[j]) * load_scale(a.scale, a.scale_bf16, o);
                if (a.acc) a.acc[tj[j] * a.N + o] = c;
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
    SBL_LOAD(S);                                                                        \
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
    SBL_LOAD(0);
  } else {
    SBL_LOAD(1);
    SBL_LOAD(0);
  }
  __syncthreads();

  int it = 0;
  if constexpr (NSET == 1) {
    while (it < total) SBL_ITER(0);
  } else {
    // steps in pairs with no exit between the halves (an exit there would
    // make the compiler assume only one register set can be in flight and
    // wait for both), then the odd last step
    while (it + 1 < total) {
      SBL_ITER(1);  // it even: data of step it+1 sits in set 1
      SBL_ITER(0);
    }
    if (it < total) SBL_ITER(1);
  }
#undef SBL_ITER
#undef SBL_LOAD
#undef SBL_STORE
}

// ---------------------------------------------------------------------------
// Warp-specialised kernel for problems with at least one tile per block slot:
// BO (o) x BT (t) output tiles, 128-code k steps, persistent blocks of MATH
// math waves and LOADERS loader waves (layout in WsCfg).
//
//  * Math waves each hold a 64 (o) x 128 (t) block of int32 accumulators,
//    read their MFMA fragments from LDS and write their finished outputs
//    themselves.  They issue no global loads, so a math wave never waits on
//    the memory counter for a load queued behind its own fp32 stores (loads
//    and stores share one in-order counter on this architecture).
//  * Loader waves stream x~ and the packed codes of the k steps two ahead
//    into registers (two register sets) and write them to LDS (double
//    buffered, one barrier per k step), with each tile's row scales and
//    beta/127 for the math waves' epilogue.
//  * The packed codes are staged as they are (a quarter of the bytes of
//    int8 codes) and expanded by the math waves right before their
//    products, in the order the three-op expansion produces; the loaders
//    stage x~ with each 16-byte group transposed 4 x 4 to match.  (Staging
//    int8 codes expanded by the loaders moved 40% more LDS bytes per step
//    and measured 4-7% slower.)
//  * Tokens are the MFMA A operand and weights the B operand, so register r
//    of a lane holds output (token 8*(r/4) + 4*(lane/32) + r%4, feature
//    lane%32) of a 32 x 32 block: one dword store per register writes two
//    whole 128-byte row segments of y, with no transposition.  (Weights as
//    A with one 16-byte store per four features measured 17% slower on the
//    layer's gate/up projection with the default cache policy, and 3x
//    slower with the streaming policy: its 32-byte row pieces reach memory
//    as partial lines.)
//  * Loads and stores go through buffer resources rebased per tile; rows
//    past N or T read as zero and their stores are dropped by the hardware
//    range check.
template <int BO_, int BT_, int MATH_, int LOADERS_, int BLOCKS_PER_CU_, int WO_ = 64, int WT_ = 128>
struct WsCfg {
  static constexpr int BO = BO_, BT = BT_, BK = 128;
  static constexpr int MATH = MATH_, LOADERS = LOADERS_;
  static constexpr int NT = 64 * (MATH + LOADERS);
  static constexpr int LT = 64 * LOADERS;  // loader threads
  static constexpr int BLOCKS_PER_CU = BLOCKS_PER_CU_;
  // waves each SIMD must hold for BLOCKS_PER_CU blocks per CU (the second
  // launch bound is a minimum of waves per SIMD, which caps the registers)
  static constexpr int WAVES_PER_SIMD = (NT / 64 * BLOCKS_PER_CU + 3) / 4;
  static constexpr int STRIDE = BK + 16;       // bytes per staged x~ row: 16-lane fragment reads hit all 64 banks once
  static constexpr int WSTRIDE = BK / 4 + 16;  // bytes per staged row of packed codes (same property)
  static constexpr int WO = WO_, WT = WT_;     // math wave tile
  static constexpr int WAVES_O = BO / WO;      // math waves along o
  static constexpr int TI = WT / 32, TJ = WO / 32;
  static constexpr int CW = BK / 64;         // 16-byte code chunks per weight row and k step
  static constexpr int CR = BO / LT;         // weight rows per loader thread
  static constexpr int XP = BK / 16;         // 16-byte x~ parts per token row and k step
  static constexpr int XQ = BT * XP / LT;    // x~ chunks per loader thread and k step
  static constexpr int NB = (BT + LT - 1) / LT;  // beta entries per loader thread
  static_assert(CR * LT == BO, "weight rows split evenly over the loader threads");
  static_assert(WAVES_O * (BT / WT) == MATH, "math waves cover the tile");
  static_assert(XQ * LT == BT * XP, "x~ chunks split evenly");
};
// The layout the large products run on: 256 x 256 tiles, 8 math and 4
// loader waves, one block per CU (three waves per SIMD: 168 VGPRs each).
// LDS: x~ 2 x 256 x 144 B, codes 2 x 256 x 48 B, scales 4 KB: 100 KB.
// (Two blocks per CU on 256 x 128 tiles, 4 math + 2 loader waves each, so
// that one block's stores overlap the other's products, measured 16%
// slower on the gate/up projection; so did starting half of the blocks
// half a tile late.)
using WsMain = WsCfg<256, 256, 8, 4, 1>;
// Problems whose 256 x 256 tiles leave a partial last round can take
// 256 x 128 tiles instead (8 math waves of 32 x 128: the same code-expansion
// work per MFMA, twice the x~ fragment reads), in rounds of half the cost.
using WsHalf = WsCfg<256, 128, 8, 4, 1, 32, 128>;

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// stores past it are dropped.  Callers keep every offset in the per-lane
// operand (scalar offset 0), which the range check covers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)min(bytes, (int64_t)INT32_MAX), 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// Output stores carry the streaming (non-temporal) policy: y is written once
// and not read back by the kernel, and each store instruction writes whole
// 128-byte row segments.
constexpr int kStoreNonTemporal = 2;
__device__ __forceinline__ void buffer_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, (int)soff, kStoreNonTemporal);
}

template <class C, bool SCALE_BF16>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_SIMD) void gemm_i8_ws_kernel(GemmArgs a) {
  constexpr int BO = C::BO, BT = C::BT, BK = C::BK, MATH = C::MATH, LT = C::LT;
  constexpr int STRIDE = C::STRIDE, WSTRIDE = C::WSTRIDE;
  constexpr int WO = C::WO, WT = C::WT, TI = C::TI, TJ = C::TJ, CW = C::CW, CR = C::CR;
  constexpr int XP = C::XP, XQ = C::XQ, NB = C::NB;
  __shared__ __attribute__((aligned(16))) int8_t sX[2][BT * STRIDE];    // x~ rows (tokens)
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][BO * WSTRIDE];  // packed codes (features)
  __shared__ __attribute__((aligned(16))) float sG[2][BO];              // row scales, by tile parity
  __shared__ __attribute__((aligned(16))) float sBt[2][BT];             // beta/127, by tile parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = a.K, N = a.N, T = a.T;
  const int kbytes = (int)(K >> 2);
  const int KT = (int)((K + BK - 1) / BK);

  // This block's work items: its whole tiles, then its half tile, if any
  // (the last tiles of the problem cut in two along t, so that the grid's
  // last round costs half a tile: at most one per block).
  const TileRange tr = tile_range(blockIdx.x, gridDim.x, a.ntiles);
  const TileRange th = tile_range(blockIdx.x, gridDim.x, a.nhalf);
  const int nfull = tr.first < tr.end ? (tr.end - tr.first + tr.step - 1) / tr.step : 0;
  const int items = nfull + (th.first < th.end ? (th.end - th.first + th.step - 1) / th.step : 0);
  if (items == 0) return;
  const int total = items * KT;
  // item -> first feature, first token and token rows (0 for the empty
  // second half of a ragged last tile row)
  auto geom = [&](int item, int64_t& o0, int64_t& t0, int64_t& rows) {
    int tile, half = -1;
    if (item < nfull) {
      tile = tr.first + item * tr.step;
    } else {
      const int h = th.first + (item - nfull) * th.step;
      tile = a.ntiles + (h >> 1);
      half = h & 1;
    }
    o0 = (int64_t)(tile % a.tiles_o) * BO;
    t0 = (int64_t)(tile / a.tiles_o) * BT + (half > 0 ? BT / 2 : 0);
    rows = max((int64_t)0, min((int64_t)(half < 0 ? BT : BT / 2), T - t0));
  };
  const int total2 = (total + 1) & ~1;  // both roles pass the same (even) number of barriers

  if (wave < MATH) {
    // ------------------------------ math waves ------------------------------
    const int wo = wave % C::WAVES_O, wt = wave / C::WAVES_O;
    v16i acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

    // y = ((float)acc * beta/127) * gamma, one dword per register: lanes
    // 0-31 and 32-63 each write 128 contiguous bytes of one token row
    auto epilogue = [&](int item, int par) {
      int64_t o0, t0, rows_t;
      geom(item, o0, t0, rows_t);
      const int N4 = (int)N * 4;
      const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(a.y + t0 * N, rows_t * N * 4);
      const int ol = wo * WO + (lane & 31);
      const int tl = wt * WT + 4 * (lane >> 5);
      uint32_t vo[TJ];
      float g[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int64_t o = o0 + ol + 32 * j;
        g[j] = sG[par][ol + 32 * j];
        vo[j] = o < N ? (uint32_t)(tl * N4 + (int)o * 4) : 0x80000000u;  // past N: dropped
      }
      // A tile that lies wholly inside T passes the row offset as the
      // scalar operand (no per-store address arithmetic); the last, partial
      // tile adds it to the per-lane offset so that the range check drops
      // the rows past T.
      auto store_all = [&](auto full) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 b = *reinterpret_cast<const float4*>(&sBt[par][tl + 32 * i + 8 * q]);
            const float bq[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t roff = (uint32_t)((32 * i + 8 * q + e) * N4);
#pragma unroll
              for (int j = 0; j < TJ; ++j) {
                const uint32_t v = __float_as_uint(((float)acc[i][j][4 * q + e] * bq[e]) * g[j]);
                if constexpr (decltype(full)::value) buffer_store4(v, ry, vo[j], roff);
                else buffer_store4(v, ry, vo[j] + roff, 0);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      };
      if (rows_t == BT) store_all(std::true_type{});
      else store_all(std::false_type{});
      if (a.acc) {  // int32 accumulator hook (a test aid)
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.acc + t0 * N, rows_t * N * 4);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              buffer_store4((uint32_t)acc[i][j][r], ra, vo[j] + (uint32_t)((32 * i + 8 * (r >> 2) + (r & 3)) * N4), 0);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};
    };
    int item = 0, kt = 0, par = 0;
    // on a half tile the waves of the second 128 tokens have nothing to do
    bool idle = nfull == 0 && wt * WT >= BT / 2;
    __syncthreads();  // step 0 staged
    for (int s = 0; s < total2; ++s) {
      if (s < total && !idle) {
        const int buf = s & 1;
        // k order inside a step: lane half h takes k in [64h, 64h + 64), and
        // for product kk its 16 values [64h + 16kk, +16), in the byte order
        // the code expansion produces (byte j of register m is k = 4j + m of
        // the 16); x~ is staged in that order, so both operands of every
        // product see the same k at the same place.  A lane's packed codes
        // of the whole step are one 16-byte read (dword kk).
        const int8_t* px = sX[buf] + (wt * WT + (lane & 31)) * STRIDE + (lane >> 5) * 64;
        const uint8_t* pw = sW[buf] + (wo * WO + (lane & 31)) * WSTRIDE + (lane >> 5) * 16;
        constexpr int KK = BK / 32;
        uint4 wc[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) wc[j] = *reinterpret_cast<const uint4*>(pw + j * 32 * WSTRIDE);
        v4i xf[2];
        xf[0] = *reinterpret_cast<const v4i*>(px);
        // The x~ fragment of the next product pair is requested before the
        // current pair is issued, so every LDS read has two MFMAs (and the
        // other math waves of the SIMD) to hide behind.
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          v4i wf[TJ];
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const uint32_t w = kk == 0 ? wc[j].x : kk == 1 ? wc[j].y : kk == 2 ? wc[j].z : wc[j].w;
            uint32_t e[4];
            expand16_strided(w, e);
            wf[j] = v4i{(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
          }
#pragma unroll
          for (int i = 0; i < TI; ++i) {
            const int c = (kk * TI + i) & 1;
            if (i + 1 < TI)
              xf[c ^ 1] = *reinterpret_cast<const v4i*>(px + (i + 1) * 32 * STRIDE + kk * 16);
            else if (kk + 1 < KK)
              xf[c ^ 1] = *reinterpret_cast<const v4i*>(px + (kk + 1) * 16);
            // keep the read above in front of these products (the scheduler
            // would otherwise sink it to save registers)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[c], wf[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if (s < total && ++kt == KT) {
        // (an idle wave's stores lie past the half tile's rows: dropped)
        epilogue(item, par);
        kt = 0;
        ++item;
        par ^= 1;
        idle = item >= nfull && wt * WT >= BT / 2;
      }
      __syncthreads();
    }
  } else {
    // ----------------------------- loader waves -----------------------------
    // Thread lt stages the BK/4 bytes (BK codes) at byte (BK/4)*kt of packed
    // rows lt + LT r (r < CR), and x~ rows x_row + (LT/XP) q (q < XQ), bytes
    // x_part..+16 of the step's BK, each 16-byte group transposed 4 x 4.
    // Codes of a k tail (K % BK == 64) are zeroed when staged, which makes
    // whatever x~ sits there irrelevant.
    const int lt = tid - MATH * 64;
    const int x_row = lt / XP, x_part = (lt % XP) * 16;
    const int c_vbase = lt * kbytes;
    const int c_r = LT * kbytes;
    const int x_vbase = x_row * (int)K + x_part;
    const int x_q = (LT / XP) * (int)K;
    uint8_t* const wdst = &sW[0][lt * WSTRIDE];
    int8_t* const xdst = &sX[0][x_row * STRIDE + x_part];

    int ld_item = 0, ld_kt = 0, ld_par = 0;
    int64_t ld_o0 = 0, ld_t0 = 0;
    __amdgpu_buffer_rsrc_t rc, rx, rg, rb;
    constexpr int GB = SCALE_BF16 ? 2 : 4;  // bytes per row scale
    auto rebase = [&]() {
      int64_t rows_t;
      geom(ld_item, ld_o0, ld_t0, rows_t);
      rc = buffer_rsrc(a.packed + ld_o0 * kbytes, min((int64_t)BO, N - ld_o0) * kbytes);
      rx = buffer_rsrc(a.xq + ld_t0 * K, rows_t * K);
      // the tile's row scales and beta: entries past N or T read as zero
      rg = buffer_rsrc(static_cast<const char*>(a.scale) + ld_o0 * GB, min((int64_t)BO, N - ld_o0) * GB);
      rb = buffer_rsrc(a.beta + ld_t0, rows_t * 4);
    };
    rebase();

    // Two register sets; every load is unconditional (past the block's last
    // step the cursor stays on that step), so the compiler can wait for
    // exactly the older set.
    uint4 c0[CR][CW], c1[CR][CW], x0[XQ], x1[XQ];
    uint32_t g0[CR], g1[CR], b0[NB], b1[NB];
    int kt0, kt1, par0, par1;
#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    kt##S = ld_kt;                                                                      \
    par##S = ld_par;                                                                    \
    _Pragma("unroll") for (int r = 0; r < CR; ++r)                                      \
      _Pragma("unroll") for (int ci = 0; ci < CW; ++ci)                                 \
        c##S[r][ci] = buffer_load16(rc, c_vbase + r * c_r + (BK / 4) * ld_kt + 16 * ci); \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q) x##S[q] = buffer_load16(rx, x_vbase + q * x_q + BK * ld_kt); \
    _Pragma("unroll") for (int r = 0; r < CR; ++r)                                      \
      g##S[r] = SCALE_BF16                                                              \
          ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rg, (lt + r * LT) * GB, 0, 0) << 16 \
          : __builtin_amdgcn_raw_buffer_load_b32(rg, (lt + r * LT) * GB, 0, 0);         \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                   \
      b##S[nb] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lt + nb * LT) * 4, 0, 0);    \
    if (++ld_kt == KT) {                                                                \
      if (ld_item + 1 < items) {                                                        \
        ld_kt = 0;                                                                      \
        ++ld_item;                                                                      \
        ld_par ^= 1;                                                                    \
        rebase();                                                                       \
      } else {                                                                          \
        ld_kt = KT - 1;                                                                 \
      }                                                                                 \
    }                                                                                   \
  }
#define SBL_WRITE(S, buf)                                                               \
  {                                                                                     \
    uint8_t* d_ = wdst + (buf) * (BO * WSTRIDE);                                        \
    _Pragma("unroll") for (int r = 0; r < CR; ++r)                                      \
      _Pragma("unroll") for (int ci = 0; ci < CW; ++ci) {                               \
        /* a chunk past K (K % BK == 64) is overwritten with zeros (uniform) */         \
        *reinterpret_cast<uint4*>(d_ + r * LT * WSTRIDE + 16 * ci) = c##S[r][ci];       \
        if ((BK / 4) * kt##S + 16 * ci >= kbytes)                                       \
          *reinterpret_cast<uint4*>(d_ + r * LT * WSTRIDE + 16 * ci) = make_uint4(0u, 0u, 0u, 0u); \
      }                                                                                 \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q) {                                    \
      const uint32_t in_[4] = {x##S[q].x, x##S[q].y, x##S[q].z, x##S[q].w};             \
      uint32_t t_[4];                                                                   \
      transpose4x4(in_, t_);                                                            \
      *reinterpret_cast<uint4*>(xdst + (buf) * (BT * STRIDE) + q * (LT / XP) * STRIDE) = \
          make_uint4(t_[0], t_[1], t_[2], t_[3]);                                       \
    }                                                                                   \
    if (kt##S == 0) {                                                                   \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                 \
        if (lt + nb * LT < BT) sBt[par##S][lt + nb * LT] = __fdiv_rn(__uint_as_float(b##S[nb]), 127.0f); \
      _Pragma("unroll") for (int r = 0; r < CR; ++r) sG[par##S][lt + r * LT] = __uint_as_float(g##S[r]); \
    }                                                                                   \
  }

    // prologue: step 0 staged, steps 1 and 2 in register sets 1 and 0
    SBL_LOAD(0);
    SBL_WRITE(0, 0);
    SBL_LOAD(1);
    SBL_LOAD(0);
    __syncthreads();
    // The empty asm statements keep the compiler from sinking a step's loads
    // past the barrier and the next write (which would shorten the prefetch
    // distance to one step).
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

template <int BM, int BN, int NSET>
static hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  a.tiles_o = (int)((a.N + BM - 1) / BM);
  const int64_t tiles_t = (a.T + BN - 1) / BN;
  a.ntiles = (int)((int64_t)a.tiles_o * tiles_t);
  static std::atomic<int> occ_cache[kMaxDevices];
  const int dev = stream_device(stream);
  const int occ = per_device_cached(occ_cache, dev, [] {
    return kernel_occupancy(reinterpret_cast<const void*>(gemm_i8_kernel<BM, BN, NSET>), 256, 1);
  });
  const int grid = (int)std::min<int64_t>(a.ntiles, (int64_t)occ * device_cus(dev));
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, NSET>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// The warp-specialised kernel on configuration C: tiles dealt to one block
// per CU, the last half-full round as half tiles where that pays (below).
template <class C>
static hipError_t launch_ws(GemmArgs a, int64_t tiles_o, int64_t tiles_t, int64_t slots, bool halves,
                            hipStream_t stream) {
  a.tiles_o = (int)tiles_o;
  const int64_t tiles = tiles_o * tiles_t;
  const int64_t rem = tiles % slots;
  a.nhalf = (halves && rem > 0 && 2 * rem <= slots) ? (int)(2 * rem) : 0;
  a.ntiles = (int)(tiles - a.nhalf / 2);
  const int grid = (int)std::min<int64_t>(tiles, slots);
  if (a.scale_bf16)
    hipLaunchKernelGGL((gemm_i8_ws_kernel<C, true>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_i8_ws_kernel<C, false>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                       const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N, float* y,
                       int32_t* acc, hipStream_t stream) {
  GemmArgs a{xq, beta, packed, scale, y, acc, T, K, N, scale_bf16, (N % 4) == 0, 0, 0};
  const int64_t ws_o = (N + WsMain::BO - 1) / WsMain::BO, ws_t = (T + WsMain::BT - 1) / WsMain::BT;
  const int64_t wh_t = (T + WsHalf::BT - 1) / WsHalf::BT;
  const int64_t slots = device_cus(stream_device(stream));  // one block per CU in both layouts
  if (ws_o * wh_t > INT32_MAX || ((N + 127) / 128) * ((T + 127) / 128) > INT32_MAX)
    return hipErrorInvalidValue;
  // the warp-specialised kernel keeps 32-bit buffer offsets within a tile's
  // rows of y and x~
  const bool offsets_ok = (int64_t)WsMain::BT * N * 4 < INT32_MAX / 2;
  if (offsets_ok && ws_o * ws_t >= slots) {
    // When the last round of tiles fills at most half the grid, an
    // HBM-bound product runs it as twice as many half tiles, one per block,
    // instead of whole tiles on half the blocks: a half tile stores half the
    // bytes (measured 7% faster on a 1152 x 896 product at 32768 tokens).
    // A product bound by the matrix cores keeps whole tiles: its tile time is
    // set per wave, and a half tile leaves each SIMD one math wave, which
    // takes about as long as two.  The bound is the product's intensity
    // against the ridge of 5 int8 POP/s over 8 TB/s (625 ops per byte).
    const double ops = 2.0 * (double)T * (double)N * (double)K;
    const double bytes = (double)T * K + (double)N * K / 4 + 4.0 * N + 4.0 * T + 4.0 * T * N;
    const bool hbm_bound = ops < 625.0 * bytes;
    // Rounds of whole tiles (a half-full last round at half cost where it
    // runs as half tiles), against rounds of 256 x 128 tiles at 0.575 of a
    // whole round each: at equal work the narrower tiles measured 5-12%
    // slower (2048 x 2048 and 2048 x 7168 at 8192 tokens, one wide tile per
    // CU), and 5-9% faster where they save a partial round (12288 tokens;
    // a ragged last token row).
    const int64_t full = ws_o * ws_t / slots, rem = ws_o * ws_t % slots;
    const double main_rounds = (double)full + (rem == 0 ? 0.0 : (hbm_bound && 2 * rem <= slots) ? 0.5 : 1.0);
    const double half_rounds = 0.575 * (double)((ws_o * wh_t + slots - 1) / slots);
    if (half_rounds < main_rounds) return launch_ws<WsHalf>(a, ws_o, wh_t, slots, false, stream);
    return launch_ws<WsMain>(a, ws_o, ws_t, slots, hbm_bound, stream);
  }
  if (offsets_ok && ws_o * wh_t >= slots) return launch_ws<WsHalf>(a, ws_o, wh_t, slots, false, stream);
  return launch_cfg<128, 128, 2>(a, stream);
}

}  // namespace sbl
