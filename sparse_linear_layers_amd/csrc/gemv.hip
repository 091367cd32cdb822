// Decode product (1 <= T <= 16 tokens) over packed ternary weights, single
// or grouped over many matrices in one launch.  Same contract as the
// prefill product ("Sparse-BitNet Guide", "Mathematical Formulation of
// Sparse-BitLinear", step 4); the model card "halo-sparse-bitnet-3:4-500m"
// ("What does NOT ship") notes that serving needs a kernel that reads the
// packed 2-bit layout directly, which this is.
//
// The stream of packed codes (1/4 B per weight) is the whole cost.  Two
// kernels share the contract:
//  * gemv_valu_kernel<B> (T <= 4): no matrix cores.  Codes are expanded to
//    int8 with the v_perm table and multiplied with v_dot4 on the vector
//    ALU; every wave streams its own rows with two k steps of loads in
//    flight, with no LDS and no barrier (design below).
//  * gemv_kernel<G> (T > 4): int8 matrix cores (v_mfma_i32_16x16x64_i8)
//    with the token count in the MFMA's N dimension.
//
// Design of the matrix-core kernel:
//  * A unit is 16*G consecutive weight rows of one matrix (G = 4 row groups
//    of 16).
//    Persistent blocks (4 waves, as many per CU as fit) walk the units; the
//    waves split K into four contiguous ranges of 256-code steps, and each
//    wave walks all G row groups over its range.
//  * Within a step, lane l holds 16 bytes (64 codes) of row l%16 of a row
//    group at k offset 64*(l/16); dword i of them is the A operand of one
//    v_mfma_i32_16x16x64_i8, whose lane group l/16 then covers
//    k = 256*s + 64*(l/16) + 16*i .. +16 on both operands.  The token count
//    (1..16) rides in the MFMA's N dimension for free.
//  * Codes are expanded in "strided" byte order (3 ALU ops per 4 weights
//    instead of 5).  The matching x~ bytes (token l%16, same k) are loaded by
//    each wave straight into registers and byte-transposed once per step;
//    the same fragments then serve all G row groups, so no LDS staging or
//    barrier sits in front of the products.
//  * A wave loads up to two steps at a time (most waves have one step:
//    K <= 1024), which keeps enough blocks resident per CU to hide memory
//    latency; the row scales and beta are loaded before the first step, the
//    descriptor of a block's next unit is read while the current one
//    computes, and the unit-to-matrix table is read once per block.
//  * The four partial int32 accumulators of a row group meet in LDS after
//    the last step (one barrier); integer sums are exact in any order.
//  * Grouped launches run the blocks of the longest-K matrices first, so
//    the slowest blocks do not form the tail.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

constexpr int kGemvWaves = 4;

struct GemvArgs {
  const sbl_gemv_desc* descs;  // device descriptors, or null: use `single`
  sbl_gemv_desc single;
  int count;
  int T;
  int block_start[kMaxGroupedGemv + 1];  // first unit of each launch position
  int16_t order[kMaxGroupedGemv];        // launch position -> descriptor index
};

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// Descriptor fields a unit needs (scalar registers).
struct GemvUnit {
  const int8_t* xq;
  const float* beta;
  const uint8_t* packed;
  const void* row_scale;
  float* y;
  int32_t* acc;
  int K, N, bf16;
  int64_t row0;
};

typedef const __attribute__((address_space(4))) sbl_gemv_desc* const_desc_ptr;  // scalar loads

// Unit u (ROWS consecutive rows of one matrix) -> its descriptor fields.
// The launch position of a unit is the last j with block_start[j] <= u:
// every lane keeps four entries of the table (read once per wave), so a
// unit's position is four ballots away.
template <int ROWS>
struct UnitTable {
  int bs[4];   // block_start[q * 64 + lane]
  int ord[4];  // order[q * 64 + lane]
  __device__ __forceinline__ void init(const GemvArgs& a, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = q * kWave + lane;
      const bool in = a.descs && idx < a.count;
      bs[q] = in ? a.block_start[idx] : INT32_MAX;
      ord[q] = in ? a.order[idx] : 0;
    }
  }
  // entry j (uniform) of a table held four entries per lane
  __device__ __forceinline__ static int entry(const int (&t)[4], int j) {
    const int q = j >> 6, l = j & 63;
    const int v = q == 0 ? t[0] : q == 1 ? t[1] : q == 2 ? t[2] : t[3];
    return __builtin_amdgcn_readlane(v, l);
  }
  __device__ __forceinline__ GemvUnit fetch(const GemvArgs& a, int u) const {
    GemvUnit f;
    if (a.descs) {
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) cnt += __popcll(__ballot(bs[q] <= u));
      const int j = cnt - 1;
      const const_desc_ptr dp = (const_desc_ptr)(uintptr_t)a.descs + entry(ord, j);
      f.xq = dp->xq;
      f.beta = dp->beta;
      f.packed = dp->packed;
      f.row_scale = dp->row_scale;
      f.y = dp->y;
      f.acc = dp->acc;
      f.K = (int)dp->K;
      f.N = (int)dp->N;
      f.bf16 = dp->scale_dtype == SBL_SCALE_BF16;
      f.row0 = (int64_t)(u - entry(bs, j)) * ROWS;
    } else {
      f.xq = a.single.xq;
      f.beta = a.single.beta;
      f.packed = a.single.packed;
      f.row_scale = a.single.row_scale;
      f.y = a.single.y;
      f.acc = a.single.acc;
      f.K = (int)a.single.K;
      f.N = (int)a.single.N;
      f.bf16 = a.single.scale_dtype == SBL_SCALE_BF16;
      f.row0 = (int64_t)u * ROWS;
    }
    return f;
  }
};
static_assert(kMaxGroupedGemv <= 4 * kWave, "four table entries per lane");

constexpr uint32_t kOut = 0x80000000u;  // a buffer offset past every range: reads 0

// ---------------------------------------------------------------------------
// Vector-ALU kernel, T <= B tokens (B = 1, 2 or 4).
//  * A unit is 32 consecutive rows of one matrix and belongs to one wave.
//    Lanes form 8 groups of 8: group r owns rows r, r+8, r+16, r+24 of the
//    unit, and lane j of a group reads the 16-byte code chunks j, j+8, ...
//    of its rows (a k step is one such chunk of every row: 128 contiguous
//    bytes of 8 rows per load instruction, so every load moves whole cache
//    lines).  One step of x~ (64 bytes per token) serves the four rows.
//  * Codes are expanded to int8 in "strided" byte order (11 ALU ops per 16
//    codes) and x~ is byte-transposed to the same order (8 ops per 16 bytes
//    per token, shared by the four rows); v_dot4 then adds 4 products per op.
//  * Waves run independently (no LDS, no barrier) over a flattened sequence
//    of (unit, k step) with two steps of loads in flight, across unit
//    boundaries; a wave's units come in snake order over the launch
//    (longest K first), which evens out the bytes per wave.
//  * The 8 partial int32 sums of a row (one per lane of its group) are
//    added with lane exchanges; integer sums are exact in any order.
// ---------------------------------------------------------------------------
namespace gv {
constexpr int ROWS = 32;      // rows per unit
constexpr int LANES_ROW = 8;  // lanes per row group
constexpr int RPL = 4;        // rows per lane
}  // namespace gv

template <int B>
__global__ __launch_bounds__(256) void gemv_valu_kernel(GemvArgs a, int units) {
  using namespace gv;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 3;  // row group
  const int j = lane & 7;     // chunk lane
  const int W = (int)gridDim.x * kGemvWaves;
  const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kGemvWaves + (int)(threadIdx.x >> 6));
  const int T = a.T;

  // k-th unit of this wave: round k covers units [kW, kW + W), walked
  // forwards in even rounds and backwards in odd ones
  auto unit_at = [&](int k) { return k * W + ((k & 1) ? W - 1 - gw : gw); };
  if (unit_at(0) >= units) return;

  UnitTable<ROWS> tab;
  tab.init(a, lane);

  // One k step's operands.  The row scale of the row the lane stores and
  // beta ride along with every step (cache hits after the first), so the
  // epilogue after a unit's last step needs nothing that step did not load
  // and never waits on the loads in flight behind it.
  struct Set {
    uint4 c[RPL];     // code chunk of each of the lane's rows
    uint4 x[B][4];    // x~ of the chunk: 64 bytes per token
    uint32_t sh, sf;  // raw row scale: bf16 bits, float bits (the other reads 0)
    uint32_t bt[B];   // raw beta of each token
  };
  // rows past N and chunks past K read as zeros: their offsets are moved
  // past the end of the resource (an OR of the top bit, no branch)
  auto load = [&](const GemvUnit& d, int s, Set& S) {
    const int kbytes = d.K >> 2;
    const int rows_left = (int)min((int64_t)ROWS, (int64_t)d.N - d.row0);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(d.packed + d.row0 * kbytes), (short)0, rows_left * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(d.xq), (short)0, T * d.K, 0x00020000);
    const int es = d.bf16 ? 1 : 2;  // log2 of the scale's bytes
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(d.row_scale)) + (d.row0 << es), (short)0,
        rows_left << es, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(d.beta), (short)0, 4 * T, 0x00020000);
    // Scale and beta first: the memory counter completes in issue order,
    // so the wait for a step's codes covers them too.  Both scale loads
    // are issued, the unused one past the end (a load behind a branch would
    // be waited for inside it).
    const uint32_t srow = (uint32_t)(grp + 8 * (j >> 1));
    S.sh = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(d.bf16 ? srow << 1 : kOut), 0, 0);
    S.sf = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(d.bf16 ? kOut : srow << 2), 0, 0);
#pragma unroll
    for (int b = 0; b < B; ++b) S.bt[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * b, 0, 0);
    const int chunk = j + LANES_ROW * s;
    const uint32_t k_out = chunk < (d.K >> 6) ? 0u : kOut;
#pragma unroll
    for (int q = 0; q < RPL; ++q)
      S.c[q] = bload16(rw, (uint32_t)((grp + 8 * q) * kbytes + 16 * chunk) | k_out);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        S.x[b][p] = bload16(rx, (uint32_t)(b * d.K + 64 * chunk + 16 * p) | k_out);
  };

  int acc[RPL][B];
#pragma unroll
  for (int q = 0; q < RPL; ++q)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[q][b] = 0;

  auto compute = [&](const Set& S) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t xt[B][4];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint32_t xin[4] = {S.x[b][p].x, S.x[b][p].y, S.x[b][p].z, S.x[b][p].w};
        transpose4x4(xin, xt[b]);
      }
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        const uint32_t wd = p == 0 ? S.c[q].x : p == 1 ? S.c[q].y : p == 2 ? S.c[q].z : S.c[q].w;
        uint32_t e[4];
        expand16_strided(wd, e);
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[q][b] = __builtin_amdgcn_sdot4((int)e[m], (int)xt[b][m], acc[q][b], false);
      }
    }
  };

  // y (and acc) of the unit.  The 8 lanes of a group hold partial sums of
  // its 4 rows; three exchange rounds (lane bits 2, 1, 0) halve the rows a
  // lane keeps and add the partner's share of them, so that lane j ends
  // with the whole sum of row q = j/2 (both lanes of a pair hold it) and
  // every lane does the same work.  Lanes with even j store row
  // grp + 8*(j/2) for every token.
  auto epilogue = [&](const GemvUnit& d, const Set& S) {
    const bool hi2 = (j & 4) != 0, hi1 = (j & 2) != 0;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      // round 1: keep rows {2,3} (bit 2 set) or {0,1}; send the other two
      const int k0 = hi2 ? acc[2][b] : acc[0][b], k1 = hi2 ? acc[3][b] : acc[1][b];
      const int s0 = hi2 ? acc[0][b] : acc[2][b], s1 = hi2 ? acc[1][b] : acc[3][b];
      const int m0 = k0 + __shfl_xor(s0, 4, kWave), m1 = k1 + __shfl_xor(s1, 4, kWave);
      // round 2: keep one of the two
      int v = (hi1 ? m1 : m0) + __shfl_xor(hi1 ? m0 : m1, 2, kWave);
      // round 3: the pair's two halves
      v += __shfl_xor(v, 1, kWave);
      acc[0][b] = v;
    }
    // Stores go through buffer resources over the unit's rows of each
    // token row (global-memory stores only, so the counters of the loads in
    // flight stay exact); rows past N and odd lanes fall outside them.
    const int rows_left = (int)min((int64_t)ROWS, (int64_t)d.N - d.row0);
    const uint32_t soff = (j & 1) ? kOut : (uint32_t)(4 * (grp + 8 * (j >> 1)));
    const float g = __uint_as_float(d.bf16 ? (uint32_t)S.sh << 16 : S.sf);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (b < T) {
        const int c = acc[0][b];
        const float bt = __fdiv_rn(__uint_as_float(S.bt[b]), 127.0f);
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            d.y + (int64_t)b * d.N + d.row0, (short)0, 4 * rows_left, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(((float)c * bt) * g), ry, (int)soff, 0, 0);
        if (d.acc) {
          const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
              d.acc + (int64_t)b * d.N + d.row0, (short)0, 4 * rows_left, 0x00020000);
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)c, ra, (int)soff, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < RPL; ++q)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[q][b] = 0;
  };

  auto nsteps = [](const GemvUnit& d) { return (d.K + 64 * LANES_ROW - 1) / (64 * LANES_ROW); };

  // load cursor: unit index lk of this wave, step ls of it; it stays on the
  // last step once the wave's units run out (those loads are never used)
  int lk = 0, ls = 0;
  GemvUnit ld = tab.fetch(a, unit_at(0));
  int lsteps = nsteps(ld);
  auto advance_load = [&]() {
    if (++ls == lsteps) {
      const int u = unit_at(lk + 1);
      if (u < units) {
        ++lk;
        ls = 0;
        ld = tab.fetch(a, u);
        lsteps = nsteps(ld);
      } else {
        ls = lsteps - 1;
      }
    }
  };
  // compute cursor
  int ck = 0, cs = 0;
  GemvUnit cd = ld;
  int csteps = lsteps;

  // steps of all this wave's units: the loop below runs them in pairs with
  // no exit between the halves (an exit there would make the compiler
  // assume that either register set may have been loaded last, and wait
  // for both)
  int total = 0;
  for (int k = 0;; ++k) {
    const int u = unit_at(k);
    if (u >= units) break;
    total += nsteps(k == 0 ? ld : tab.fetch(a, u));
  }

  Set s0, s1;
  load(ld, ls, s0);
  advance_load();
  load(ld, ls, s1);
  advance_load();
  auto step = [&](Set& S) {
    compute(S);
    if (++cs == csteps) {
      epilogue(cd, S);
      const int u = unit_at(ck + 1);
      if (u < units) {
        ++ck;
        cs = 0;
        cd = tab.fetch(a, u);
        csteps = nsteps(cd);
      }
    }
    load(ld, ls, S);
    advance_load();
  };
  int it = 0;
  for (; it + 1 < total; it += 2) {
    step(s0);
    step(s1);
  }
  if (it < total) step(s0);
}

// ---------------------------------------------------------------------------
// Matrix-core kernel (T > 4), units of 16*G rows per block.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256, G <= 4 ? 4 : 2) void gemv_kernel(GemvArgs a, int units) {
  __shared__ __attribute__((aligned(16))) v4i sacc[kGemvWaves][G][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int tok = lane & 15;
  const int T = a.T;
  const bool tok_ok = tok < T;
  constexpr int E = G / kGemvWaves;  // row groups this wave finishes

  // Units (16*G rows of one matrix) u = blockIdx.x + k * gridDim.x.
  UnitTable<16 * G> tab;
  tab.init(a, lane);
  auto fetch = [&](int u) { return tab.fetch(a, u); };
  // this wave's 256-code steps of a unit
  auto step_range = [&](const GemvUnit& d, int& lo, int& hi) {
    const int nsteps = (d.K + 255) >> 8;
    lo = nsteps * wave / kGemvWaves;
    hi = nsteps * (wave + 1) / kGemvWaves;
  };
  // One step's operands: codes of every row group (rows past N repeat row
  // N-1; their outputs are never stored), x~ of the lane's token.  Every
  // load goes through a buffer resource (scalar base and size): a lane that
  // must read zeros (k past K in a partial last step, a token slot >= T)
  // gets an offset past the end, which the hardware range check turns into
  // zeros without a branch.
  auto load_step = [&](const GemvUnit& d, int s, uint4 (&w)[G], uint4 (&x)[4]) {
    const int kbytes = d.K >> 2;
    const int rows_left = (int)min((int64_t)(16 * G), (int64_t)d.N - d.row0);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(d.packed + d.row0 * kbytes), (short)0, rows_left * kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(d.xq), (short)0, T * d.K, 0x00020000);
    const bool k_ok = 256 * s + 64 * g < d.K;
#pragma unroll
    for (int rg = 0; rg < G; ++rg)
      w[rg] = bload16(rw, k_ok ? (uint32_t)(min(16 * rg + tok, rows_left - 1) * kbytes + 16 * g + 64 * s) : kOut);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = bload16(rx, (k_ok && tok_ok) ? (uint32_t)(tok * d.K + 64 * g + 256 * s + 16 * i) : kOut);
  };

  int u = blockIdx.x;
  if (u >= units) return;
  GemvUnit dc = fetch(u);
  int un = u + (int)gridDim.x;
  GemvUnit dn = un < units ? fetch(un) : dc;  // read while this unit computes
  for (;;) {
    const int N = dc.N;
    const int64_t row0 = dc.row0;

    // Row scales of this lane's four rows per finished row group (rows past
    // N clamped) and beta, loaded now and converted only at the epilogue, so
    // that their memory round trip overlaps the code loads.  Both scale
    // types are requested, the unused one at an offset past the buffer;
    // every offset and the resource are uniform in structure, so no load
    // sits behind a branch that would force an early wait.
    // The resource covers this unit's rows only, so its offsets stay small
    // whatever N is.
    const int bf16 = __builtin_amdgcn_readfirstlane(dc.bf16);
    const int unit_rows = (int)min((int64_t)(16 * G), (int64_t)N - row0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(dc.row_scale)) + (row0 << (bf16 ? 1 : 2)), (short)0,
        __builtin_amdgcn_readfirstlane(unit_rows << (bf16 ? 1 : 2)), 0x00020000);
    uint32_t sh[E][4], sf[E][4];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int oc = min(16 * (wave * E + e) + 4 * g + r, unit_rows - 1);
        sh[e][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(bf16 ? 2u * oc : kOut), 0, 0);
        sf[e][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(bf16 ? kOut : 4u * oc), 0, 0);
      }
    const float beta_raw = dc.beta[min(tok, T - 1)];

    int s_lo, s_hi;
    step_range(dc, s_lo, s_hi);
    v4i acc[G];
#pragma unroll
    for (int rg = 0; rg < G; ++rg) acc[rg] = v4i{0, 0, 0, 0};
    auto compute = [&](const uint4 (&w)[G], const uint4 (&x)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t xin[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
        uint32_t xt[4];
        transpose4x4(xin, xt);
        const v4i bv = {(int)xt[0], (int)xt[1], (int)xt[2], (int)xt[3]};
#pragma unroll
        for (int rg = 0; rg < G; ++rg) {
          const uint32_t wd = i == 0 ? w[rg].x : i == 1 ? w[rg].y : i == 2 ? w[rg].z : w[rg].w;
          uint32_t e4[4];
          expand16_strided(wd, e4);
          const v4i av = {(int)e4[0], (int)e4[1], (int)e4[2], (int)e4[3]};
          acc[rg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[rg], 0, 0, 0);
        }
      }
    };
    // steps in pairs: both pairs' loads in flight together (long-K units
    // wait for half as many memory round trips); a lone last step reads
    // only its own operands
    for (int s = s_lo; s < s_hi; s += 2) {
      uint4 w0[G], x0[4], w1[G], x1[4];
      load_step(dc, s, w0, x0);
      const bool two = s + 1 < s_hi;
      if (two) load_step(dc, s + 1, w1, x1);
      compute(w0, x0);
      if (two) compute(w1, x1);
    }

    const float bt = __fdiv_rn(beta_raw, 127.0f);
    // partial sums of the four K ranges
#pragma unroll
    for (int rg = 0; rg < G; ++rg) sacc[wave][rg][lane] = acc[rg];
    __syncthreads();
    // lane holds C[row = 4*(lane/16) + r][token = lane%16] of its row group
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int rg = wave * E + e;
      const v4i c = sacc[0][rg][lane] + sacc[1][rg][lane] + sacc[2][rg][lane] + sacc[3][rg][lane];
      const int64_t o = row0 + 16 * rg + 4 * g;
      if (tok_ok && o < N) {
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = bf16 ? __uint_as_float(sh[e][r] << 16) : __uint_as_float(sf[e][r]);
        float* yp = dc.y + (int64_t)tok * N + o;
        const float v0 = ((float)c[0] * bt) * sc[0], v1 = ((float)c[1] * bt) * sc[1];
        const float v2 = ((float)c[2] * bt) * sc[2], v3 = ((float)c[3] * bt) * sc[3];
        int32_t* ap = dc.acc ? dc.acc + (int64_t)tok * N + o : nullptr;
        if ((N & 3) == 0) {  // o + 3 < N and 16-byte aligned
          *reinterpret_cast<float4*>(yp) = make_float4(v0, v1, v2, v3);
          if (ap) *reinterpret_cast<int4*>(ap) = make_int4(c[0], c[1], c[2], c[3]);
        } else {
          yp[0] = v0;
          if (o + 1 < N) yp[1] = v1;
          if (o + 2 < N) yp[2] = v2;
          if (o + 3 < N) yp[3] = v3;
          if (ap) {
            ap[0] = c[0];
            if (o + 1 < N) ap[1] = c[1];
            if (o + 2 < N) ap[2] = c[2];
            if (o + 3 < N) ap[3] = c[3];
          }
        }
      }
    }
    if (un >= units) break;
    __syncthreads();  // sacc is rewritten by the next unit
    u = un;
    dc = dn;
    un += (int)gridDim.x;
    if (un < units) dn = fetch(un);
  }
}

// Resident blocks of a decode kernel on the device of `stream`: as many
// per CU as the register file holds.
template <typename K>
static int resident_slots(K kernel, std::atomic<int> (&cache)[kMaxDevices], hipStream_t stream) {
  const int dev = stream_device(stream);
  const int occ = per_device_cached(cache, dev, [kernel] {
    return kernel_occupancy(reinterpret_cast<const void*>(kernel), 256, 2);
  });
  return occ * device_cus(dev);
}

// Tokens up to which the vector-ALU kernel runs; above, the matrix cores.
constexpr int64_t kGemvValuMaxTokens = 4;

// Rows per unit of the kernel that serves T tokens.
static int64_t gemv_unit_rows(int64_t T) { return T <= kGemvValuMaxTokens ? gv::ROWS : 64; }

int64_t gemv_blocks(int64_t N, int64_t T) {
  const int64_t rows = gemv_unit_rows(T);
  return (N + rows - 1) / rows;
}

template <int B>
static hipError_t launch_valu(const GemvArgs& a, int64_t units, hipStream_t stream) {
  static std::atomic<int> cache[kMaxDevices];
  const int64_t waves = std::min<int64_t>(units, (int64_t)resident_slots(gemv_valu_kernel<B>, cache, stream) * kGemvWaves);
  const int grid = (int)((waves + kGemvWaves - 1) / kGemvWaves);
  hipLaunchKernelGGL(gemv_valu_kernel<B>, dim3((unsigned)grid), dim3(256), 0, stream, a, (int)units);
  return hipGetLastError();
}

hipError_t launch_gemv(const sbl_gemv_desc* host, const sbl_gemv_desc* dev, int count, int64_t T,
                       hipStream_t stream) {
  for (int first = 0; first < count;) {
    const int last = std::min(count, first + kMaxGroupedGemv);
    const int n = last - first;
    GemvArgs a{};
    a.descs = dev ? dev + first : nullptr;
    if (!dev) a.single = host[first];
    a.count = n;
    a.T = (int)T;
    // launch order: longest K first (stable), so the longest units start
    // first and shorter ones fill in behind them
    int16_t ord[kMaxGroupedGemv];
    for (int i = 0; i < n; ++i) ord[i] = (int16_t)i;
    std::stable_sort(ord, ord + n, [&](int16_t x, int16_t y) { return host[first + x].K > host[first + y].K; });
    int64_t units = 0;
    for (int i = 0; i < n; ++i) {
      a.order[i] = ord[i];
      a.block_start[i] = (int)units;
      units += gemv_blocks(host[first + ord[i]].N, T);
    }
    a.block_start[n] = (int)units;
    if (units > 0) {
      hipError_t e;
      if (T <= kGemvValuMaxTokens) {
        e = T == 1 ? launch_valu<1>(a, units, stream)
                   : T == 2 ? launch_valu<2>(a, units, stream) : launch_valu<4>(a, units, stream);
      } else {
        static std::atomic<int> cache[kMaxDevices];
        const int grid = (int)std::min<int64_t>(units, (int64_t)resident_slots(gemv_kernel<4>, cache, stream));
        hipLaunchKernelGGL(gemv_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, a, (int)units);
        e = hipGetLastError();
      }
      if (e != hipSuccess) return e;
    }
    first = last;
  }
  return hipSuccess;
}

}  // namespace sbl
