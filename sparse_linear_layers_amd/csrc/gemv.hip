// Decode product (1 <= T <= 16 tokens) over packed ternary weights, single
// or grouped over many matrices in one launch.  Same contract as the
// prefill product ("Sparse-BitNet Guide", "Mathematical Formulation of
// Sparse-BitLinear", step 4); the model card "halo-sparse-bitnet-3:4-500m"
// ("What does NOT ship") notes that serving needs a kernel that reads the
// packed 2-bit layout directly, which this is.
//
// The stream of packed codes (1/4 B per weight) is the whole cost.  Two
// kernels share the contract:
//  * gemv_stream_kernel (T == 1, K <= 8192): no matrix cores.  Fully
//    coalesced code loads over whole consecutive rows, v_perm expansion and
//    v_dot4 products on the vector ALU, row sums through LDS atomics
//    (design below).
//  * gemv_kernel<G> (every other case): int8 matrix cores
//    (v_mfma_i32_16x16x64_i8) with the token count in the MFMA's N
//    dimension.
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
//  * Codes are expanded in "strided" byte order (9 ALU ops per 16 weights
//    instead of 19).  The matching x~ bytes (token l%16, same k) are loaded by
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
  int16_t kblocks[kMaxGroupedGemv];      // launch position -> K / 64
  int16_t urows[kMaxGroupedGemv];        // launch position -> rows per unit (streaming kernel)
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
  int rows;  // rows per unit
  int64_t row0;
};

typedef const __attribute__((address_space(4))) sbl_gemv_desc* const_desc_ptr;  // scalar loads

// Unit u (ROWS consecutive rows of one matrix; ROWS = 0: the launch
// position's own row count) -> its descriptor fields.  The launch position
// of a unit is the last j with block_start[j] <= u: every lane keeps four
// entries of each table (read once per wave), so a unit's position is four
// ballots away.
template <int ROWS>
struct UnitTable {
  int bs[4];   // block_start[q * 64 + lane]
  int ord[4];  // order[q * 64 + lane]
  int kb[4];   // kblocks[q * 64 + lane]
  int ur[4];   // urows[q * 64 + lane]
  __device__ __forceinline__ void init(const GemvArgs& a, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = q * kWave + lane;
      const bool in = a.descs && idx < a.count;
      bs[q] = in ? a.block_start[idx] : INT32_MAX;
      ord[q] = in ? a.order[idx] : 0;
      kb[q] = in ? a.kblocks[idx] : 0;
      ur[q] = in ? a.urows[idx] : 0;
    }
  }
  // launch position of unit u (grouped launches)
  __device__ __forceinline__ int position(int u) const {
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt += __popcll(__ballot(bs[q] <= u));
    return cnt - 1;
  }
  // K / 64 of unit u's matrix, from the tables alone (no memory access)
  __device__ __forceinline__ int kblocks_of(const GemvArgs& a, int u) const {
    return a.descs ? entry(kb, position(u)) : (int)(a.single.K >> 6);
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
      const int j = position(u);
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
      f.rows = ROWS > 0 ? ROWS : entry(ur, j);
      f.row0 = (int64_t)(u - entry(bs, j)) * f.rows;
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
      f.rows = ROWS > 0 ? ROWS : a.urows[0];
      f.row0 = (int64_t)u * f.rows;
    }
    return f;
  }
};
static_assert(kMaxGroupedGemv <= 4 * kWave, "four table entries per lane");

constexpr uint32_t kOut = 0x80000000u;  // a buffer offset past every range: reads 0

// ---------------------------------------------------------------------------
// Streaming kernel, one token (T == 1, K <= 8192).
//  * A unit is `rows` consecutive rows of one matrix (chosen per matrix on
//    the host so that units carry about equal bytes, about one unit per
//    resident wave) and belongs to one wave.  Rows are contiguous in
//    memory, so one load instruction covers whole consecutive rows: with
//    c = K/64 16-byte chunks per row and c <= 64, lane l reads chunk l % c
//    of row l / c of a group of 64 / c rows, i.e. bytes 16*l.. of the
//    group (one contiguous run of whole cache lines); with 64 < c <= 128 a
//    row takes two instructions (chunks l and 64 + l).  Every lane so keeps
//    the same one or two chunks of x~ for the whole unit, loaded once and
//    held in registers in the expanded byte order.
//  * Two code loads (2 KB, non-temporal) form a step; two steps are in
//    flight (with four loads per step the kernel needed 114 VGPRs and ran
//    5% slower at four waves per SIMD than this at five).  Codes are
//    expanded with the v_perm tables (9 ops per 16 codes) and multiplied
//    with v_dot4 (4 products per op).
//  * A lane's sum for one instruction belongs to one row: the lanes of a
//    row add theirs into the wave's row accumulators in LDS (integer
//    atomics: exact in any order; a row of two instructions is summed over
//    the wave with lane exchanges instead); lane l then finishes rows l and
//    64 + l.
// ---------------------------------------------------------------------------
namespace gs {
// Codes are read once: the non-temporal policy (bit 1 of the cache-policy
// operand) streamed the one-token sweep 11% faster.
constexpr int kLoadNonTemporal = 2;
constexpr int MAX_ROWS = 128;    // rows per unit
constexpr int MAX_CHUNKS = 128;  // K / 64, i.e. K <= 8192
constexpr int STEP = 2;          // code loads per step
}  // namespace gs

template <bool TWO>  // TWO: a row takes two load instructions (64 < K/64 <= 128)
__device__ __forceinline__ void stream_unit(const GemvUnit& d, int lane, int* racc) {
  using namespace gs;
  const int kbytes = d.K >> 2, cpr = d.K >> 6;
  const int rpi = TWO ? 1 : 64 / cpr;  // rows per load group
  const int rows = (int)min((int64_t)d.rows, (int64_t)d.N - d.row0);
  const int n_instr = ((rows + rpi - 1) / rpi) * (TWO ? 2 : 1);
  const int nsteps = (n_instr + STEP - 1) / STEP;
  const int slot = TWO ? 0 : lane / cpr;  // row of the lane within a load group
  const int kc = TWO ? lane : lane % cpr;
  const bool act0 = TWO || lane < rpi * cpr;
  const bool act1 = TWO && 64 + lane < cpr;

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(d.packed + d.row0 * kbytes), (short)0, rows * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(d.xq), (short)0, d.K, 0x00020000);
  const int es = d.bf16 ? 1 : 2;  // log2 of the scale's bytes
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(d.row_scale)) + (d.row0 << es), (short)0,
      rows << es, 0x00020000);

  // x~ chunk(s) of the lane and the scales of the two rows it finishes go
  // first (the memory counter completes in issue order); both scale types
  // are requested, the unused one past the end
  uint4 x0[4], x1[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) x0[p] = bload16(rx, act0 ? (uint32_t)(64 * kc + 16 * p) : kOut);
  if constexpr (TWO) {
#pragma unroll
    for (int p = 0; p < 4; ++p) x1[p] = bload16(rx, act1 ? (uint32_t)(64 * (64 + kc) + 16 * p) : kOut);
  }
  uint32_t sh[2], sf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t r = (uint32_t)(lane + 64 * h);
    sh[h] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(d.bf16 ? r << 1 : kOut), 0, 0);
    sf[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(d.bf16 ? kOut : r << 2), 0, 0);
  }
  const float beta = d.beta[0];

  // code loads of instruction i (rows past the unit's end read zeros)
  auto load = [&](int s, uint4 (&c)[STEP]) {
#pragma unroll
    for (int q = 0; q < STEP; ++q) {
      const int i = STEP * s + q;
      const bool seg1 = TWO && (q & 1);  // STEP is even: the segment is q's parity
      const int grp = TWO ? (i >> 1) : i;
      const bool on = i < n_instr && (seg1 ? act1 : act0);
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
          rw, (int)((uint32_t)(grp * rpi * kbytes + (seg1 ? 1024 : 0) + 16 * lane) | (on ? 0u : kOut)), 0,
          kLoadNonTemporal);
      c[q] = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
    }
  };

  // accumulators of the unit's rows (and a slot for inactive lanes)
  racc[lane] = 0;
  racc[64 + lane] = 0;
  if (lane == 0) racc[MAX_ROWS] = 0;

  uint4 c0[STEP], c1[STEP];
  load(0, c0);
  load(1, c1);

  // x~ in the expanded byte order: transposed 4x4 byte blocks
  uint32_t xt0[4][4], xt1[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t in0[4] = {x0[p].x, x0[p].y, x0[p].z, x0[p].w};
    transpose4x4(in0, xt0[p]);
    if constexpr (TWO) {
      const uint32_t in1[4] = {x1[p].x, x1[p].y, x1[p].z, x1[p].w};
      transpose4x4(in1, xt1[p]);
    }
  }

  int prev = 0;  // first half of a row's sum (TWO)
  auto compute = [&](int s, const uint4 (&c)[STEP]) {
#pragma unroll
    for (int q = 0; q < STEP; ++q) {
      const int i = STEP * s + q;
      const bool seg1 = TWO && (q & 1);
      const int grp = TWO ? (i >> 1) : i;
      int part = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t wd = p == 0 ? c[q].x : p == 1 ? c[q].y : p == 2 ? c[q].z : c[q].w;
        uint32_t e[4];
        expand16_strided(wd, e);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          part = __builtin_amdgcn_sdot4((int)e[m], (int)(seg1 ? xt1[p][m] : xt0[p][m]), part, false);
      }
      if constexpr (TWO) {
        // one row per instruction pair, all lanes: a wave sum after the
        // pair's second half (lane exchanges; exact integer adds)
        if (seg1) {
          part += prev;
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) part += __shfl_xor(part, d, kWave);
          if (lane == 0 && i < n_instr) racc[grp] = part;
        } else {
          prev = part;
        }
      } else {
        // the lanes of a row add their sums into its accumulator
        const bool on = i < n_instr && act0;
        atomicAdd(&racc[on ? grp * rpi + slot : MAX_ROWS], part);
      }
    }
  };
  // Steps in pairs with no exit between the halves (an exit there would
  // make the compiler assume either register set may have been loaded
  // last).  The scheduling barriers keep each refill ahead of the next
  // step's products: the scheduler would otherwise start consuming the
  // other set first, and wait for every load in flight.
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    compute(s, c0);
    load(s + 2, c0);
    __builtin_amdgcn_sched_barrier(0);
    compute(s + 1, c1);
    load(s + 3, c1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s < nsteps) compute(s, c0);

  // epilogue: rows lane and 64 + lane; stores through resources over the
  // unit's rows (rows past its end fall outside them)
  const float bt = __fdiv_rn(beta, 127.0f);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(d.y + d.row0, (short)0, 4 * rows, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(d.acc + d.row0, (short)0, 4 * rows, 0x00020000);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = lane + 64 * h;
    const int c = racc[r];
    const float g = __uint_as_float(d.bf16 ? sh[h] << 16 : sf[h]);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(((float)c * bt) * g), ry, 4 * r, 0, 0);
    if (d.acc) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)c, ra, 4 * r, 0, 0);
  }
}

__global__ __launch_bounds__(256) void gemv_stream_kernel(GemvArgs a, int units) {
  __shared__ int sacc[kGemvWaves][gs::MAX_ROWS + 1];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int W = (int)gridDim.x * kGemvWaves;
  UnitTable<0> tab;
  tab.init(a, lane);
  for (int u = (int)blockIdx.x * kGemvWaves + wv; u < units; u += W) {
    const GemvUnit d = tab.fetch(a, u);
    if (d.K > 64 * 64)
      stream_unit<true>(d, lane, sacc[wv]);
    else
      stream_unit<false>(d, lane, sacc[wv]);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel (every case the streaming kernel does not take), units
// of 16*G rows per block.
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

// The streaming kernel serves one token and K <= 8192; everything else
// runs on the matrix cores (units of 64 rows).
static bool gemv_streams(int64_t T, int64_t maxK) { return T == 1 && maxK <= 64 * gs::MAX_CHUNKS; }

// Rows per unit of the streaming kernel for a matrix of K columns: about
// `target` bytes, a whole number of load groups, at most MAX_ROWS.
static int stream_unit_rows(int64_t K, int64_t target) {
  const int64_t kbytes = K / 4, cpr = K / 64;
  const int64_t rpi = cpr > 64 ? 1 : 64 / cpr;
  const int64_t cap = gs::MAX_ROWS / rpi * rpi;
  int64_t rows = (target / kbytes + rpi / 2) / rpi * rpi;
  return (int)std::min(cap, std::max(rpi, rows));
}

int64_t gemv_blocks(int64_t N, int64_t T) {
  (void)T;
  return N;  // at least one row per unit: an upper bound on the units of either kernel
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
    int64_t maxK = 0, bytes = 0;
    for (int i = 0; i < n; ++i) {
      maxK = std::max<int64_t>(maxK, host[first + i].K);
      bytes += host[first + i].N * (host[first + i].K / 4);
    }
    const bool streams = gemv_streams(T, maxK);
    static std::atomic<int> cache_s[kMaxDevices], cache_m[kMaxDevices];
    const int64_t slots = streams ? resident_slots(gemv_stream_kernel, cache_s, stream)
                                  : resident_slots(gemv_kernel<4>, cache_m, stream);
    const int64_t target = std::max<int64_t>(4096, bytes / std::max<int64_t>(1, slots * kGemvWaves));
    int64_t units = 0;
    for (int i = 0; i < n; ++i) {
      const sbl_gemv_desc& d = host[first + ord[i]];
      const int rows = streams ? stream_unit_rows(d.K, target) : 64;
      a.order[i] = ord[i];
      a.kblocks[i] = (int16_t)(d.K >> 6);
      a.urows[i] = (int16_t)rows;
      a.block_start[i] = (int)units;
      units += (d.N + rows - 1) / rows;
    }
    a.block_start[n] = (int)units;
    if (units > INT32_MAX / 2) return hipErrorInvalidValue;
    if (units > 0) {
      if (streams) {
        const int64_t waves = std::min<int64_t>(units, slots * kGemvWaves);
        hipLaunchKernelGGL(gemv_stream_kernel, dim3((unsigned)((waves + kGemvWaves - 1) / kGemvWaves)),
                           dim3(256), 0, stream, a, (int)units);
      } else {
        hipLaunchKernelGGL(gemv_kernel<4>, dim3((unsigned)std::min<int64_t>(units, slots)), dim3(256), 0,
                           stream, a, (int)units);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    first = last;
  }
  return hipSuccess;
}

}  // namespace sbl
