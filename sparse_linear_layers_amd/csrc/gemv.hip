// Decode product (1 <= T <= 16 tokens) over packed ternary weights, single
// or grouped over many matrices in one launch.  Same contract as the
// prefill product ("Sparse-BitNet Guide", "Mathematical Formulation of
// Sparse-BitLinear", step 4); the model card "halo-sparse-bitnet-3:4-500m"
// ("What does NOT ship") notes that serving needs a kernel that reads the
// packed 2-bit layout directly, which this is.
//
// The stream of packed codes (1/4 B per weight) is the whole cost, so the
// kernel is built to keep many code loads in flight per CU with few
// dependent memory round trips and little ALU per byte:
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
  int block_start[kMaxGroupedGemv + 1];  // by launch position
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
  int K, N, bf16;
  int64_t row0;
};

template <int G>
__global__ __launch_bounds__(256, G <= 4 ? 4 : 2) void gemv_kernel(GemvArgs a, int units) {
  __shared__ __attribute__((aligned(16))) v4i sacc[kGemvWaves][G][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int tok = lane & 15;
  const int T = a.T;
  const bool tok_ok = tok < T;
  constexpr uint32_t kOut = 0x80000000u;
  constexpr int E = G / kGemvWaves;  // row groups this wave finishes

  // Units (16*G rows of one matrix) u = blockIdx.x + k * gridDim.x.  The
  // launch position of a unit is the last j with block_start[j] <= u: every
  // lane keeps four entries of the table (one round of loads for all of the
  // block's units) and a unit's position is four ballots away.
  int bs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = q * kWave + lane;
    bs[q] = (a.descs && idx < a.count) ? a.block_start[idx] : INT32_MAX;
  }
  static_assert(kMaxGroupedGemv <= 4 * kWave, "four table entries per lane");
  typedef const __attribute__((address_space(4))) sbl_gemv_desc* const_desc_ptr;  // scalar loads
  auto fetch = [&](int u) {
    GemvUnit f;
    if (a.descs) {
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) cnt += __popcll(__ballot(bs[q] <= u));
      const int j = cnt - 1;
      const const_desc_ptr dp = (const_desc_ptr)(uintptr_t)a.descs + a.order[j];
      f.xq = dp->xq;
      f.beta = dp->beta;
      f.packed = dp->packed;
      f.row_scale = dp->row_scale;
      f.y = dp->y;
      f.K = (int)dp->K;
      f.N = (int)dp->N;
      f.bf16 = dp->scale_dtype == SBL_SCALE_BF16;
      f.row0 = (int64_t)(u - a.block_start[j]) * (16 * G);
    } else {
      f.xq = a.single.xq;
      f.beta = a.single.beta;
      f.packed = a.single.packed;
      f.row_scale = a.single.row_scale;
      f.y = a.single.y;
      f.K = (int)a.single.K;
      f.N = (int)a.single.N;
      f.bf16 = a.single.scale_dtype == SBL_SCALE_BF16;
      f.row0 = (int64_t)u * (16 * G);
    }
    return f;
  };

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
    const int bf16 = __builtin_amdgcn_readfirstlane(dc.bf16);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(dc.row_scale), (short)0, __builtin_amdgcn_readfirstlane(N << (bf16 ? 1 : 2)),
        0x00020000);
    uint32_t sh[E][4], sf[E][4];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int oc = (int)min(row0 + 16 * (wave * E + e) + 4 * g + r, (int64_t)N - 1);
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
        if ((N & 3) == 0) {  // o + 3 < N and 16-byte aligned
          *reinterpret_cast<float4*>(yp) = make_float4(v0, v1, v2, v3);
        } else {
          yp[0] = v0;
          if (o + 1 < N) yp[1] = v1;
          if (o + 2 < N) yp[2] = v2;
          if (o + 3 < N) yp[3] = v3;
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

// Persistent blocks of the decode kernel on the device of `stream`: as
// many per CU as the register file holds.
static int gemv_resident_slots(hipStream_t stream) {
  static std::atomic<int> occ_cache[kMaxDevices];
  const int dev = stream_device(stream);
  const int occ = per_device_cached(occ_cache, dev, [] {
    return kernel_occupancy(reinterpret_cast<const void*>(gemv_kernel<4>), 256, 2);
  });
  return occ * device_cus(dev);
}

// Row groups per block for a token count.
static int gemv_groups(int64_t T) {
  (void)T;  // 8 row groups per unit (less x~ traffic at T = 16) measured no faster
  return 4;
}

int64_t gemv_blocks(int64_t N, int64_t T) {
  const int64_t rows = 16 * gemv_groups(T);
  return (N + rows - 1) / rows;
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
    // launch order: longest K first (stable), so the longest blocks start
    // first and shorter ones fill in behind them
    int16_t ord[kMaxGroupedGemv];
    for (int i = 0; i < n; ++i) ord[i] = (int16_t)i;
    std::stable_sort(ord, ord + n, [&](int16_t x, int16_t y) { return host[first + x].K > host[first + y].K; });
    int64_t blocks = 0;
    for (int i = 0; i < n; ++i) {
      a.order[i] = ord[i];
      a.block_start[i] = (int)blocks;
      blocks += gemv_blocks(host[first + ord[i]].N, T);
    }
    a.block_start[n] = (int)blocks;
    if (blocks > 0) {
      const int grid = (int)std::min<int64_t>(blocks, (int64_t)gemv_resident_slots(stream));
      hipLaunchKernelGGL(gemv_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, a, (int)blocks);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    first = last;
  }
  return hipSuccess;
}

}  // namespace sbl
