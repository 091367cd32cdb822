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
// Warp-specialised kernel for problems with at least one tile per CU:
// 256 (o) x 256 (t) output tiles, 128-code k steps, one persistent 768-thread
// block per CU.
//
//  * Waves 0-7 are math waves (two per SIMD): each holds a 64 (o) x 128 (t)
//    block of int32 accumulators, reads its MFMA fragments from LDS and
//    writes its finished outputs itself.  They issue no global loads, so a
//    math wave never waits on the memory counter for a load queued behind
//    its own fp32 stores (loads and stores share one in-order counter on
//    this architecture): the stores of a finished tile drain while the next
//    tile computes.
//  * Waves 8-11 are loader waves: they stream x~ and the packed codes of the
//    k steps two ahead into registers (two register sets), expand the codes
//    to int8 with the v_perm table while writing them to LDS (double
//    buffered, one barrier per k step), and stage each tile's row scales and
//    beta/127 for the math waves' epilogue.
//  * Tokens are the MFMA A operand and weights the B operand, so register r
//    of a lane holds output (token 8*(r/4) + 4*(lane/32) + r%4, feature
//    lane%32) of a 32 x 32 block: one dword store per register writes two
//    whole 128-byte row segments of y, with no transposition.
//  * Loads and stores go through buffer resources rebased per tile; rows
//    past N or T read as zero and their stores are dropped by the hardware
//    range check.
//  * LDS: x~ and expanded codes, 2 stages x 256 rows x 144 B each (147 KB),
//    plus 4 KB of scales: 151.5 KB of the 160 KB.  Three waves per SIMD leave
//    168 VGPRs per wave: 128 accumulators and one set of fragments.
namespace ws {
constexpr int BO = 256, BT = 256, BK = 128, NT = 768;
constexpr int MATH = 8;  // math waves (2 per SIMD); the 4 waves after them load
constexpr int STRIDE = BK + 16;  // bytes per staged row: 16-lane fragment reads hit all 64 banks once
constexpr int WO = 64, WT = 128;  // math wave tile; the 8 math waves are 4 (o) x 2 (t)
constexpr int TI = WT / 32, TJ = WO / 32;
constexpr int XQ = BT / 32;  // 16-byte x~ chunks per loader thread and k step (8)
}  // namespace ws

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

// Output stores carry the non-temporal cache policy (bit 1 of the policy
// operand): y is written once and not read back by the kernel, and streaming
// it past the caches shortened the fp32-output-bound products by ~10%.
constexpr int kStoreNonTemporal = 2;
__device__ __forceinline__ void buffer_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, (int)soff, kStoreNonTemporal);
}

template <bool SCALE_BF16>
__global__ __launch_bounds__(ws::NT, 1) void gemm_i8_ws_kernel(GemmArgs a) {
  using namespace ws;
  __shared__ __attribute__((aligned(16))) int8_t sX[2][BT * STRIDE];  // x~ rows (tokens)
  __shared__ __attribute__((aligned(16))) int8_t sW[2][BO * STRIDE];  // expanded codes (features)
  __shared__ __attribute__((aligned(16))) float sG[2][BO];            // row scales, by tile parity
  __shared__ __attribute__((aligned(16))) float sBt[2][BT];           // beta/127, by tile parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = a.K, N = a.N, T = a.T;
  const int kbytes = (int)(K >> 2);
  const int KT = (int)((K + BK - 1) / BK);

  const TileRange tr = tile_range(blockIdx.x, gridDim.x, a.ntiles);
  if (tr.first >= tr.end) return;
  const int total = ((tr.end - tr.first + tr.step - 1) / tr.step) * KT;
  const int total2 = (total + 1) & ~1;  // both roles pass the same (even) number of barriers

  if (wave < MATH) {
    // ------------------------------ math waves ------------------------------
    const int wo = wave & 3, wt = wave >> 2;
    v16i acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

    // y = ((float)acc * beta/127) * gamma, one dword per register: lanes
    // 0-31 and 32-63 each write 128 contiguous bytes of one token row
    auto epilogue = [&](int tile, int par) {
      const int64_t o0 = (int64_t)(tile % a.tiles_o) * BO;
      const int64_t t0 = (int64_t)(tile / a.tiles_o) * BT;
      const int64_t rows_t = min((int64_t)BT, T - t0);
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

    int tile = tr.first, kt = 0, par = 0;
    __syncthreads();  // step 0 staged
    for (int s = 0; s < total2; ++s) {
      if (s < total) {
        const int buf = s & 1;
        const int8_t* px = sX[buf] + (wt * WT + (lane & 31)) * STRIDE + (lane >> 5) * 16;
        const int8_t* pw = sW[buf] + (wo * WO + (lane & 31)) * STRIDE + (lane >> 5) * 16;
        v4i xf[1][TI], wf[1][TJ];
#define SBL_FRAG(S, kk)                                                                 \
  {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < TI; ++i) xf[S][i] = *reinterpret_cast<const v4i*>(px + i * 32 * STRIDE + (kk) * 32); \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j) wf[S][j] = *reinterpret_cast<const v4i*>(pw + j * 32 * STRIDE + (kk) * 32); \
  }
#define SBL_MMA(S)                                                                      \
  {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < TI; ++i)                                      \
      _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                    \
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[S][i], wf[S][j], acc[i][j], 0, 0, 0); \
  }
        SBL_FRAG(0, 0);
        SBL_MMA(0);
        SBL_FRAG(0, 1);
        SBL_MMA(0);
        SBL_FRAG(0, 2);
        SBL_MMA(0);
        SBL_FRAG(0, 3);
        SBL_MMA(0);
#undef SBL_FRAG
#undef SBL_MMA
        if (++kt == KT) {
          epilogue(tile, par);
          kt = 0;
          tile += tr.step;
          par ^= 1;
        }
      }
      __syncthreads();
    }
  } else {
    // ----------------------------- loader waves -----------------------------
    // Thread lt stages the 32 bytes (128 codes) of packed row lt at byte
    // 32*kt, and x~ rows x_row + 32 q (q < 8), bytes x_part..+16 of the
    // step's 128.  Codes of a k tail (K % 128 == 64) are zeroed when staged,
    // which makes whatever x~ sits there irrelevant.
    const int lt = tid - MATH * 64;
    const int c_row = lt;
    const int x_row = lt >> 3, x_part = (lt & 7) * 16;
    const int c_vbase = c_row * kbytes;
    const int x_vbase = x_row * (int)K + x_part;
    const int x_q = 32 * (int)K;
    int8_t* const wdst = &sW[0][c_row * STRIDE];
    int8_t* const xdst = &sX[0][x_row * STRIDE + x_part];
    const int sl = lt;  // scale slot of this thread

    int ld_tile = tr.first, ld_kt = 0, ld_par = 0;
    int64_t ld_o0 = 0, ld_t0 = 0;
    __amdgpu_buffer_rsrc_t rc, rx;
    auto rebase = [&]() {
      ld_o0 = (int64_t)(ld_tile % a.tiles_o) * BO;
      ld_t0 = (int64_t)(ld_tile / a.tiles_o) * BT;
      rc = buffer_rsrc(a.packed + ld_o0 * kbytes, min((int64_t)BO, N - ld_o0) * kbytes);
      rx = buffer_rsrc(a.xq + ld_t0 * K, min((int64_t)BT, T - ld_t0) * K);
    };
    rebase();

    // Two register sets; every load is unconditional (past the block's last
    // step the cursor stays on that step), so the compiler can wait for
    // exactly the older set.
    uint4 c0, c1, d0, d1, x0[XQ], x1[XQ];
    uint32_t g0, g1, b0, b1;
    int kt0, kt1, par0, par1;
#define SBL_LOAD(S)                                                                     \
  {                                                                                     \
    kt##S = ld_kt;                                                                      \
    par##S = ld_par;                                                                    \
    c##S = buffer_load16(rc, c_vbase + 32 * ld_kt);                                     \
    d##S = buffer_load16(rc, c_vbase + 32 * ld_kt + 16);                                \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q) x##S[q] = buffer_load16(rx, x_vbase + q * x_q + BK * ld_kt); \
    const int64_t so_ = min(ld_o0 + sl, N - 1);                                         \
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
    int8_t* d_ = wdst + (buf) * (BO * STRIDE);                                          \
    const bool ka_ = 32 * kt##S < kbytes, kb_ = 32 * kt##S + 16 < kbytes;               \
    uint32_t e_[4];                                                                     \
    expand16_natural(ka_ ? c##S.x : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_) = make_uint4(e_[0], e_[1], e_[2], e_[3]);             \
    expand16_natural(ka_ ? c##S.y : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 16) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(ka_ ? c##S.z : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 32) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(ka_ ? c##S.w : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 48) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(kb_ ? d##S.x : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 64) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(kb_ ? d##S.y : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 80) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(kb_ ? d##S.z : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 96) = make_uint4(e_[0], e_[1], e_[2], e_[3]);        \
    expand16_natural(kb_ ? d##S.w : 0u, e_);                                            \
    *reinterpret_cast<uint4*>(d_ + 112) = make_uint4(e_[0], e_[1], e_[2], e_[3]);       \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q)                                      \
      *reinterpret_cast<uint4*>(xdst + (buf) * (BT * STRIDE) + q * 32 * STRIDE) = x##S[q]; \
    if (kt##S == 0) {                                                                   \
      sBt[par##S][lt] = __fdiv_rn(__uint_as_float(b##S), 127.0f);                       \
      sG[par##S][lt] = __uint_as_float(g##S);                                           \
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

hipError_t launch_gemm(const int8_t* xq, const float* beta, const uint8_t* packed,
                       const void* scale, int scale_bf16, int64_t T, int64_t K, int64_t N, float* y,
                       int32_t* acc, hipStream_t stream) {
  GemmArgs a{xq, beta, packed, scale, y, acc, T, K, N, scale_bf16, (N % 4) == 0, 0, 0};
  const int64_t ws_o = (N + ws::BO - 1) / ws::BO, ws_t = (T + ws::BT - 1) / ws::BT;
  const int cus = device_cus(stream_device(stream));
  if (ws_o * ws_t > INT32_MAX || ((N + 127) / 128) * ((T + 127) / 128) > INT32_MAX)
    return hipErrorInvalidValue;
  // the warp-specialised kernel keeps 32-bit buffer offsets within a tile's
  // rows of y and x~
  if (ws_o * ws_t >= cus && (int64_t)ws::BT * N * 4 < INT32_MAX / 2) {
    a.tiles_o = (int)ws_o;
    a.ntiles = (int)(ws_o * ws_t);
    const int grid = (int)std::min<int64_t>(a.ntiles, cus);
    if (scale_bf16)
      hipLaunchKernelGGL(gemm_i8_ws_kernel<true>, dim3((unsigned)grid), dim3(ws::NT), 0, stream, a);
    else
      hipLaunchKernelGGL(gemm_i8_ws_kernel<false>, dim3((unsigned)grid), dim3(ws::NT), 0, stream, a);
    return hipGetLastError();
  }
  return launch_cfg<128, 128, 2>(a, stream);
}

}  // namespace sbl
