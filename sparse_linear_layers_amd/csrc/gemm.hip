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
//  * Per k step a block loads 128 rows x 16 B of packed codes (8 bytes per
//    thread) and 128 rows x 64 B of x~, expands the codes to int8 with
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
// Large-tile variant for problems with at least one tile per CU:
// 256 (o) x 256 (t) output tiles, 8 waves of 128 x 64, 128-code k steps, one
// persistent 512-thread block per CU (2 x 72 KB of LDS stages).
//
// Per k step a block moves 8 KB of packed codes and 32 KB of x~ from L2.
// Against the 128 x 128 x 64 step above this quadruples the work done per
// L2 request (each x~ request is now a whole 128-byte row segment, and each
// code request feeds 256 tokens instead of 128), which is what bounds the
// small-tile kernel: its L1 runs out of outstanding misses long before the
// matrix cores or HBM are busy.
namespace big {
constexpr int BM = 256, BN = 256, BK = 128, NT = 512;
constexpr int STRIDE = BK + 16;           // bytes per staged row: 16-lane reads hit all 64 banks once
constexpr int WTM = 128, WTN = 64;        // wave tile: waves are 2 (o) x 4 (t)
constexpr int TM = WTM / 32, TN = WTN / 32;
constexpr int NSET = 1;                   // register stages of global data
}  // namespace big

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)min(bytes, (int64_t)INT32_MAX), 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

template <bool SCALE_BF16, int NSET>
__global__ __launch_bounds__(big::NT, 1) void gemm_i8_big_kernel(GemmArgs a) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * STRIDE];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t K = a.K, N = a.N, T = a.T;
  const int64_t kbytes = K >> 2;  // packed bytes per weight row
  const int KT = (int)((K + BK - 1) / BK);

  const TileRange tr = tile_range(blockIdx.x, gridDim.x, a.ntiles);
  if (tr.first >= tr.end) return;
  const int total = ((tr.end - tr.first + tr.step - 1) / tr.step) * KT;
  int cp_tile = tr.first, cp_kt = 0;

  // Staging roles: 16 bytes (64 codes) of packed row a_row at byte
  // 32*kt + 16*a_half; x~ rows b_row0 + 64 q (q < 4), bytes b_part..+16 of
  // the step's 128.  Loads go through buffer resources rebased at each tile
  // (offsets stay 32-bit and the k step is a scalar offset), so a step's
  // loads cost no vector ALU.  Rows past N or T repeat the last row (their
  // outputs are never stored); the codes of a k tail (K % 128 == 64) are
  // zeroed when staged, which makes whatever x~ sits there irrelevant.
  const int a_row = tid >> 1, a_half = tid & 1;
  const int b_row0 = tid >> 3, b_part = (tid & 7) * 16;
  int ld_tile = tr.first, ld_kt = 0;
  __amdgpu_buffer_rsrc_t rs_a, rs_b;
  int a_off, b_off0, b_off1, b_off2, b_off3;
  auto ld_rebase = [&]() {
    const int64_t o0 = (int64_t)(ld_tile % a.tiles_o) * BM;
    const int64_t t0 = (int64_t)(ld_tile / a.tiles_o) * BN;
    const int rows_o = (int)min((int64_t)BM, N - o0), rows_t = (int)min((int64_t)BN, T - t0);
    rs_a = buffer_rsrc(a.packed + o0 * kbytes, (int64_t)rows_o * kbytes);
    rs_b = buffer_rsrc(a.xq + t0 * K, (int64_t)rows_t * K);
    a_off = min(a_row, rows_o - 1) * (int)kbytes + 16 * a_half;
    b_off0 = min(b_row0, rows_t - 1) * (int)K + b_part;
    b_off1 = min(b_row0 + 64, rows_t - 1) * (int)K + b_part;
    b_off2 = min(b_row0 + 128, rows_t - 1) * (int)K + b_part;
    b_off3 = min(b_row0 + 192, rows_t - 1) * (int)K + b_part;
  };
  ld_rebase();

  uint4 ra_0, rb0_0, rb1_0, rb2_0, rb3_0;
  uint4 ra_1, rb0_1, rb1_1, rb2_1, rb3_1;
  bool ka_0 = true, ka_1 = true;  // the set's codes lie inside K

  // Past the block's last step the cursor stays on that step: the extra
  // loads are in bounds and their data is never computed with.
#define SBL_BLOAD(S)                                                                    \
  {                                                                                     \
    ka_##S = ld_kt * (BK / 4) + 16 * a_half < kbytes;                                   \
    ra_##S = buffer_load16(rs_a, a_off, ld_kt * (BK / 4));                              \
    rb0_##S = buffer_load16(rs_b, b_off0, ld_kt * BK);                                  \
    rb1_##S = buffer_load16(rs_b, b_off1, ld_kt * BK);                                  \
    rb2_##S = buffer_load16(rs_b, b_off2, ld_kt * BK);                                  \
    rb3_##S = buffer_load16(rs_b, b_off3, ld_kt * BK);                                  \
    if (++ld_kt == KT) {                                                                \
      if (ld_tile + tr.step < tr.end) {                                                 \
        ld_kt = 0;                                                                      \
        ld_tile += tr.step;                                                             \
        ld_rebase();                                                                    \
      } else {                                                                          \
        ld_kt = KT - 1;                                                                 \
      }                                                                                 \
    }                                                                                   \
  }

  // staging piece d (0..3) of set S into LDS buffer buf: codes of dword d
  // of the packed chunk (16 codes) and x~ chunk d
#define SBL_BPIECE(S, buf, d, comp, rbd)                                                \
  {                                                                                     \
    uint32_t e_[4];                                                                     \
    expand16_natural(ka_##S ? ra_##S.comp : 0u, e_);                                    \
    *reinterpret_cast<uint4*>(sA[buf] + a_row * STRIDE + 64 * a_half + 16 * (d)) =      \
        make_uint4(e_[0], e_[1], e_[2], e_[3]);                                         \
    *reinterpret_cast<uint4*>(sB[buf] + (b_row0 + 64 * (d)) * STRIDE + b_part) = rbd##_##S; \
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  // 32 k of the product from LDS buffer buf
#define SBL_BKK(buf, kk)                                                                \
  {                                                                                     \
    const int8_t* pa_ = sA[buf] + (wm * WTM + (lane & 31)) * STRIDE + (lane >> 5) * 16 + (kk) * 32; \
    const int8_t* pb_ = sB[buf] + (wn * WTN + (lane & 31)) * STRIDE + (lane >> 5) * 16 + (kk) * 32; \
    v4i af_[TM], bf_[TN];                                                               \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) af_[i] = *reinterpret_cast<const v4i*>(pa_ + i * 32 * STRIDE); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) bf_[j] = *reinterpret_cast<const v4i*>(pb_ + j * 32 * STRIDE); \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                      \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                    \
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af_[i], bf_[j], acc[i][j], 0, 0, 0); \
  }

  // lane holds C[o = 8*(r/4) + 4*(lane/32) + r%4][t = lane%32] of each
  // 32 x 32 tile: y[t][o..o+3] is one 16-byte store
  // Epilogue of a finished tile, through the LDS buffer the tile's last step
  // was computed from (free once every wave is past it): per 32-row slab i
  // of its 128 x 64 wave tile, each wave writes y = (acc * beta/127) * gamma
  // as [64 tokens][32 rows] floats into its own 9 KB, reads it back by token
  // row and stores whole 128-byte row segments (8 per instruction).  The
  // MFMA layout (lane holds rows 8*(r/4) + 4*(lane/32) + r%4 of token
  // lane%32) would otherwise give 32-byte pieces of 32 different lines per
  // store.  N % 4 != 0 takes a per-element path; the int32 accumulator
  // hook, a test aid, is written directly.
  auto epilogue = [&](int buf) {
    const int64_t o0 = (int64_t)(cp_tile % a.tiles_o) * BM;
    const int64_t t0 = (int64_t)(cp_tile / a.tiles_o) * BN;
    const int64_t ob = o0 + wm * WTM + 4 * (lane >> 5);
    const int64_t tw = t0 + wn * WTN;  // first token of the wave tile
    float bt[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bt[j] = __fdiv_rn(a.beta[min(tw + j * 32 + (lane & 31), T - 1)], 127.0f);
    if (a.vec_store) {
      constexpr int ES = 36;  // floats per staged token row (32 + 4 pad)
      float* st = reinterpret_cast<float*>((wave < 4 ? sA[buf] : sB[buf]) + (wave & 3) * (WTN * ES * 4));
      const int rr = lane >> 3, cc = (lane & 7) * 4;  // read-back: token row rr + 8 s, floats cc..cc+3
      float* yrow = a.y + (tw + rr) * N + (o0 + wm * WTM + cc);
      const int64_t oc0 = o0 + wm * WTM + cc;
      const int rows_ok = (int)min((int64_t)WTN, T - tw);  // token rows of the wave tile inside T
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        __builtin_amdgcn_sched_barrier(0);  // one slab's scales live at a time
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t o = min(ob + i * 32 + 8 * q, N - 4);
          float4 g;
          if constexpr (SCALE_BF16) {
            const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.scale) + o);
            g = make_float4(__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                            __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u));
          } else {
            g = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.scale) + o);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const v16i& c = acc[i][j];
            *reinterpret_cast<float4*>(st + (j * 32 + (lane & 31)) * ES + 8 * q + 4 * (lane >> 5)) =
                make_float4(((float)c[4 * q] * bt[j]) * g.x, ((float)c[4 * q + 1] * bt[j]) * g.y,
                            ((float)c[4 * q + 2] * bt[j]) * g.z, ((float)c[4 * q + 3] * bt[j]) * g.w);
          }
        }
        const bool o_ok = oc0 + i * 32 < N;
#pragma unroll
        for (int r8 = 0; r8 < WTN / 8; ++r8) {
          const float4 v = *reinterpret_cast<const float4*>(st + (rr + 8 * r8) * ES + cc);
          if (o_ok && rr + 8 * r8 < rows_ok)
            *reinterpret_cast<float4*>(yrow + (int64_t)(8 * r8) * N + i * 32) = v;
        }
      }
      if (a.acc) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int64_t o = ob + i * 32 + 8 * q, t = tw + j * 32 + (lane & 31);
              const v16i& c = acc[i][j];
              if (t < T && o < N)
                *reinterpret_cast<int4*>(a.acc + t * N + o) = make_int4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
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
              const int64_t o = ob + i * 32 + 8 * q + e, t = tw + j * 32 + (lane & 31);
              if (o < N && t < T) {
                const int32_t c = acc[i][j][4 * q + e];
                a.y[t * N + o] = ((float)c * bt[j]) * load_scale(a.scale, SCALE_BF16, o);
                if (a.acc) a.acc[t * N + o] = c;
              }
            }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};
  };

  // One k step: the product of LDS buffer it&1, with the staging of set S
  // into the other buffer woven between its four 32-k pieces (one straight
  // block, so the compiler can overlap the expansion ALU with the matrix
  // core), then the refill of set S, the epilogue when a tile is done, and
  // one barrier.  Staging on the last step writes data nobody reads.
#define SBL_BITER(S)                                                                    \
  {                                                                                     \
    const int cur_ = it & 1, nxt_ = cur_ ^ 1;                                           \
    SBL_BKK(cur_, 0);                                                                   \
    SBL_BPIECE(S, nxt_, 0, x, rb0);                                                     \
    SBL_BKK(cur_, 1);                                                                   \
    SBL_BPIECE(S, nxt_, 1, y, rb1);                                                     \
    SBL_BKK(cur_, 2);                                                                   \
    SBL_BPIECE(S, nxt_, 2, z, rb2);                                                     \
    SBL_BKK(cur_, 3);                                                                   \
    SBL_BPIECE(S, nxt_, 3, w, rb3);                                                     \
    SBL_BLOAD(S);                                                                       \
    if (++cp_kt == KT) {                                                                \
      cp_kt = 0;                                                                        \
      __syncthreads();                                                                  \
      epilogue(cur_);                                                                   \
      cp_tile += tr.step;                                                               \
    }                                                                                   \
    __syncthreads();                                                                    \
    ++it;                                                                               \
  }

  int it = 0;
  if constexpr (NSET == 2) {
    // prologue: step 0 staged, steps 1 and 2 in register sets 1 and 0
    SBL_BLOAD(0);
    SBL_BPIECE(0, 0, 0, x, rb0);
    SBL_BPIECE(0, 0, 1, y, rb1);
    SBL_BPIECE(0, 0, 2, z, rb2);
    SBL_BPIECE(0, 0, 3, w, rb3);
    SBL_BLOAD(1);
    SBL_BLOAD(0);
    __syncthreads();
    // steps in pairs with no exit between the halves (an exit there would
    // make the compiler assume only one register set can be in flight and
    // wait for both), then the odd last step
    while (it + 1 < total) {
      SBL_BITER(1);  // it even: data of step it+1 sits in set 1
      SBL_BITER(0);
    }
    if (it < total) SBL_BITER(1);
  } else {
    // one register set: step it+1 is loaded while step it computes
    SBL_BLOAD(0);
    SBL_BPIECE(0, 0, 0, x, rb0);
    SBL_BPIECE(0, 0, 1, y, rb1);
    SBL_BPIECE(0, 0, 2, z, rb2);
    SBL_BPIECE(0, 0, 3, w, rb3);
    SBL_BLOAD(0);
    __syncthreads();
    while (it < total) SBL_BITER(0);
  }
#undef SBL_BITER
#undef SBL_BKK
#undef SBL_BPIECE
#undef SBL_BLOAD
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
  const int64_t big_o = (N + big::BM - 1) / big::BM, big_t = (T + big::BN - 1) / big::BN;
  const int cus = num_cus();
  if (big_o * big_t > INT32_MAX || ((N + 127) / 128) * ((T + 127) / 128) > INT32_MAX)
    return hipErrorInvalidValue;
  if (big_o * big_t >= cus) {
    a.tiles_o = (int)big_o;
    a.ntiles = (int)(big_o * big_t);
    const int grid = (int)std::min<int64_t>(a.ntiles, cus);
    if (scale_bf16)
      hipLaunchKernelGGL((gemm_i8_big_kernel<true, big::NSET>), dim3((unsigned)grid), dim3(big::NT), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_i8_big_kernel<false, big::NSET>), dim3((unsigned)grid), dim3(big::NT), 0, stream, a);
    return hipGetLastError();
  }
  return launch_cfg<128, 128, 2>(a, stream);
}

}  // namespace sbl
