// Backward pass of the layer with the straight-through estimator ("Sparse-
// BitNet Guide", "Training Stability & The Straight-Through Estimator": the
// gradient passes through the mask and the ternary rounding to the latent
// weights; README "BitLinear": gradients flow through by STE):
//   dw[o,k] = gamma_o * sum_t (dy[t,o] * (beta_t/127)) * x~[t,k]
//   dx[t,k] = sum_o (dy[t,o] * gamma_o) * code[o,k]
//
// Both are products of a float operand with an operand that bf16 holds
// exactly (ternary codes, int8 x~).  They run on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16): each float is split into three bf16 pieces
// (hi = top 8 significant bits, mid, lo), which represent it exactly, so
// every product is exact and only the fp32 accumulation rounds.
//
// One kernel computes C[m, n] = sum_r A(r, m) * B(r, n) over 128 x 256
// output tiles and 32-wide reduction steps staged through LDS, 4 waves of
// 64 x 128 (the three A pieces share each B fragment):
//   dx: m = token, n = k, r = o;  A = dy * gamma (rows of dy), B = codes
//       (packed rows, expanded and transposed while staged);
//   dw: m = o, n = k, r = token;  A = dy * beta/127 (transposed while
//       staged), B = x~ (transposed while staged).  The token reduction is
//       split over S chunks whose partial tiles go to a caller workspace; a
//       second kernel adds them in chunk order and multiplies by gamma, so
//       the result does not depend on scheduling.
// Each thread stages a 4 x 4 (A) and 4 x 8 (B) block per step: the
// transposes happen in registers, every LDS write is 8 bytes, and the
// global loads of the next step are in flight during the products.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

namespace ste {
constexpr int BM = 128, BN = 256, BR = 32, NT = 256;
constexpr int LS = BR + 8;  // bf16 per staged row (80 B): 16-lane fragment reads hit every bank once
}  // namespace ste

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct SteArgs {
  const float* dy;
  const int8_t* xq;
  const float* beta;
  const uint8_t* packed;
  const float* gamma;
  const float* tscale;  // dw: beta_t / 127 per token
  float* out;        // dx [T, K], or the workspace [S, N, K] of dw partials
  int64_t T, K, N;
  int64_t r_chunk;   // reduction length of one split (dw)
  int tiles_n;       // column tiles
  int tiles_mn;      // output tiles (per split)
};

// Block b of a G-block grid runs on XCD b % 8.  Each XCD gets a contiguous
// range of work units (unit order: split, row tile, column tile), so the
// blocks that share an operand tile also share an L2.
__device__ __forceinline__ int xcd_unit(int b, int G) {
  constexpr int X = 8;
  const int base = G / X, rem = G % X;
  const int x = b % X;
  return x * base + min(x, rem) + b / X;
}

// Exact three-piece bf16 split of two floats: hi = the top 16 bits, mid =
// the top 16 bits of the remainder, lo = what is left (at most 8
// significant bits).  Returns each piece of the pair packed in a dword.
__device__ __forceinline__ void split3x2(float x0, float x1, uint32_t& hi, uint32_t& mid,
                                         uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
  const float r0 = x0 - __uint_as_float(b0 & 0xffff0000u);  // exact
  const float r1 = x1 - __uint_as_float(b1 & 0xffff0000u);
  const uint32_t c0 = __float_as_uint(r0), c1 = __float_as_uint(r1);
  const float q0 = r0 - __uint_as_float(c0 & 0xffff0000u);  // exact
  const float q1 = r1 - __uint_as_float(c1 & 0xffff0000u);
  hi = perm(b1, b0, 0x07060302u);
  mid = perm(c1, c0, 0x07060302u);
  lo = perm(__float_as_uint(q1), __float_as_uint(q0), 0x07060302u);
}

// Byte tables of the 2-bit code's bf16 (00 -> 0, 01 -> +1.0 = 0x3F80,
// 10 -> -1.0 = 0xBF80, 11 -> 0): high bytes and low bytes.
constexpr uint32_t kCodeBf16Hi = 0x00BF3F00u;
constexpr uint32_t kCodeBf16Lo = 0x00808000u;

// One thread's share of a reduction step, held in registers between the
// global loads and the LDS writes.
struct SteStage {
  float a[16];     // dy values, [i][j]
  float s[4];      // dx: gamma of 4 reduction rows o; dw: beta/127 of 4 tokens
  uint32_t b[8];   // dx: b[i] = 2 packed bytes (8 codes) of row o_i;
                   // dw: b[2i], b[2i+1] = 8 bytes of x~ of token t_i
};

// Raw buffer resource over [base, base + bytes): loads past the end return
// 0.  Offsets are per lane (scalar offset 0); kOut lies past every buffer.
constexpr uint32_t kOut = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ste_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)max((int64_t)0, min(bytes, (int64_t)INT32_MAX)),
                                           0x00020000);
}
__device__ __forceinline__ void bload_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, float* d) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  d[0] = __int_as_float(v.x); d[1] = __int_as_float(v.y);
  d[2] = __int_as_float(v.z); d[3] = __int_as_float(v.w);
}
__device__ __forceinline__ float bload_f1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// Thread roles within a step (tid = 0..255, f = tid & 7, g = tid >> 3):
//   dx  A: tokens m0 + g + 32 i, reduction rows o = r0 + 4 f + j
//       B: reduction rows o = r0 + 4 f + i, columns k = n0 + 8 g + j
//   dw  A: tokens t = r0 + 4 f + i, output rows o = m0 + 4 g + j
//       B: tokens t = r0 + 4 f + i, columns k = n0 + 8 g + j
// Eight consecutive lanes read 128 contiguous bytes of one dy row (dx) or
// one 16-byte piece of 8 rows (dw); 16 consecutive lanes write 128
// distinct LDS bytes.  Each step's buffers start at its first row, so the
// per-lane offsets stay small and constant; a buffer ends at the last row
// the step may read (T, N or the split's last token), and columns past the
// matrix take kOut.
template <int DW>
__device__ __forceinline__ void ste_load(const SteArgs& a, SteStage& st, int64_t r0, int64_t r_end,
                                         int64_t m0, int64_t n0, int f, int g, bool vec) {
  const int64_t T = a.T, K = a.K, N = a.N;
  const uint32_t rowA = (uint32_t)N * 4u;  // bytes per dy row
  if constexpr (!DW) {
    const auto rA = ste_rsrc(a.dy + m0 * N + r0, ((T - m0) * N - r0) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(g + 32 * i) * rowA + 16u * f;
      if (vec) {
        bload_f4(rA, r0 + 4 * f < N ? off : kOut, &st.a[4 * i]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) st.a[4 * i + j] = bload_f1(rA, r0 + 4 * f + j < N ? off + 4u * j : kOut);
      }
    }
    const auto rG = ste_rsrc(a.gamma + r0, (N - r0) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) st.s[j] = bload_f1(rG, 16u * f + 4u * j);
    const uint32_t kb = (uint32_t)(K >> 2);  // bytes per packed row
    const auto rB = ste_rsrc(a.packed + r0 * kb + (n0 >> 2), (N - r0) * (int64_t)kb - (n0 >> 2));
    const bool kin = n0 + 8 * g < K;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b16(rB, (int)(kin ? (4u * f + i) * kb + 2u * g : kOut), 0, 0);
  } else {
    const auto rA = ste_rsrc(a.dy + r0 * N + m0, ((r_end - r0) * N - m0) * 4);
    const bool oin = m0 + 4 * g < N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (uint32_t)(4 * f + i) * rowA + 16u * g;
      if (vec) {
        bload_f4(rA, oin ? off : kOut, &st.a[4 * i]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) st.a[4 * i + j] = bload_f1(rA, m0 + 4 * g + j < N ? off + 4u * j : kOut);
      }
    }
    const auto rS = ste_rsrc(a.tscale + r0, (r_end - r0) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.s[i] = bload_f1(rS, 16u * f + 4u * i);
    const uint32_t kr = (uint32_t)K;  // bytes per x~ row
    const auto rB = ste_rsrc(a.xq + r0 * K + n0, (r_end - r0) * K - n0);
    const bool kin = n0 + 8 * g < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2i x = __builtin_amdgcn_raw_buffer_load_b64(rB, (int)(kin ? (4u * f + i) * kr + 8u * g : kOut), 0, 0);
      st.b[2 * i] = (uint32_t)x.x;
      st.b[2 * i + 1] = (uint32_t)x.y;
    }
  }
}

template <int DW>
__device__ __forceinline__ void ste_store_lds(const SteStage& st, uint16_t (*sA)[ste::BM * ste::LS],
                                              uint16_t* sB, int f, int g) {
  using namespace ste;
  if constexpr (!DW) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h0, m0, l0, h1, m1, l1;
      split3x2(st.a[4 * i + 0] * st.s[0], st.a[4 * i + 1] * st.s[1], h0, m0, l0);
      split3x2(st.a[4 * i + 2] * st.s[2], st.a[4 * i + 3] * st.s[3], h1, m1, l1);
      const int off = (g + 32 * i) * LS + 4 * f;
      *reinterpret_cast<uint2*>(&sA[0][off]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(&sA[1][off]) = make_uint2(m0, m1);
      *reinterpret_cast<uint2*>(&sA[2][off]) = make_uint2(l0, l1);
    }
    // gather byte q of the four rows into G[q]: G[q].byte[i] = b[i].byte[q]
    const uint32_t p01 = perm(st.b[1], st.b[0], 0x05010400u);
    const uint32_t p23 = perm(st.b[3], st.b[2], 0x05010400u);
    const uint32_t G[2] = {perm(p23, p01, 0x05040100u), perm(p23, p01, 0x07060302u)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = (G[j >> 2] >> (2 * (j & 3))) & kLow2;  // code of column j, rows 0..3
      const uint32_t hb = perm(0u, kCodeBf16Hi, c);
      const uint32_t lb = perm(0u, kCodeBf16Lo, c);
      *reinterpret_cast<uint2*>(&sB[(8 * g + j) * LS + 4 * f]) =
          make_uint2(perm(hb, lb, 0x05010400u), perm(hb, lb, 0x07030602u));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t h0, m0, l0, h1, m1, l1;
      split3x2(st.a[j] * st.s[0], st.a[4 + j] * st.s[1], h0, m0, l0);
      split3x2(st.a[8 + j] * st.s[2], st.a[12 + j] * st.s[3], h1, m1, l1);
      const int off = (4 * g + j) * LS + 4 * f;
      *reinterpret_cast<uint2*>(&sA[0][off]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(&sA[1][off]) = make_uint2(m0, m1);
      *reinterpret_cast<uint2*>(&sA[2][off]) = make_uint2(l0, l1);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = (int)(st.b[2 * i + (j >> 2)] << (24 - 8 * (j & 3))) >> 24;  // x~, sign-extended
        v[i] = __float_as_uint((float)q);                                            // exact
      }
      *reinterpret_cast<uint2*>(&sB[(8 * g + j) * LS + 4 * f]) =
          make_uint2(perm(v[1], v[0], 0x07060302u), perm(v[3], v[2], 0x07060302u));
    }
  }
}

template <int DW>
__global__ __launch_bounds__(ste::NT, 2) void ste_kernel(SteArgs a) {
  using namespace ste;
  __shared__ __attribute__((aligned(16))) uint16_t sA[3][BM * LS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int f = tid & 7, g = tid >> 3;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int64_t M = DW ? N : T;     // output rows
  const int64_t R = DW ? T : N;     // reduction length
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int split = unit / a.tiles_mn;
  const int tile = unit - split * a.tiles_mn;
  const int64_t m0 = (int64_t)(tile / a.tiles_n) * BM;
  const int64_t n0 = (int64_t)(tile % a.tiles_n) * BN;
  const int64_t r_begin = DW ? (int64_t)split * a.r_chunk : 0;
  const int64_t r_end = DW ? min(R, r_begin + a.r_chunk) : R;
  const bool vec = (N & 3) == 0;   // dy rows start 16-byte aligned: 4-float loads
  // a wave whose 128 columns all lie past K only helps to stage
  const bool active = n0 + wn * 128 < K;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  SteStage st;
  if (r_begin < r_end) ste_load<DW>(a, st, r_begin, r_end, m0, n0, f, g, vec);
  for (int64_t r0 = r_begin; r0 < r_end; r0 += BR) {
    ste_store_lds<DW>(st, sA, sB, f, g);
    __syncthreads();
    if (r0 + BR < r_end) ste_load<DW>(a, st, r0 + BR, r_end, m0, n0, f, g, vec);  // in flight during the products
    if (active) {
      // ---- products: 2 x 16 of r, three pieces, 2 x 4 tiles of 32 x 32 ----
#pragma unroll
      for (int kk = 0; kk < BR / 16; ++kk) {
        const int koff = kk * 16 + 8 * (lane >> 5);
        bf16x8 bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[(wn * 128 + 32 * j + (lane & 31)) * LS + koff]);
#pragma unroll
        for (int p = 0; p < 3; ++p) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sA[p][(wm * 64 + 32 * i + (lane & 31)) * LS + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;

  // ---- store: lane holds C[m = 8*(r/4) + 4*(lane/32) + r%4][n = lane%32] ----
  float* out = a.out + (DW ? (int64_t)split * N * K : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < K) {
          // dx is final and written once: stream it past the caches; dw
          // partials are read back by the reduction right after
          if constexpr (DW) out[m * K + n] = acc[i][j][r];
          else __builtin_nontemporal_store(acc[i][j][r], &out[m * K + n]);
        }
      }
    }
}

// dw[o, k] = (sum over the S partials, in chunk order) * gamma_o
__global__ __launch_bounds__(256) void ste_dw_reduce_kernel(const float* __restrict__ ws,
                                                            const float* __restrict__ gamma,
                                                            int64_t N, int64_t K, int S,
                                                            float* __restrict__ dw) {
  const int64_t total = N * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = ws[i];
    for (int c = 1; c < S; ++c) s += ws[(int64_t)c * total + i];
    dw[i] = s * gamma[i / K];
  }
}

// Blocks of the dw kernel resident at once on the current device (the
// workspace-size query has no stream, so both it and the launch use the
// current device).
static int64_t ste_slots() {
  static std::atomic<int> occ_cache[kMaxDevices];
  const int dev = stream_device(nullptr);
  const int occ = per_device_cached(occ_cache, dev, [] {
    return kernel_occupancy(reinterpret_cast<const void*>(ste_kernel<1>), ste::NT, 2);
  });
  return (int64_t)device_cus(dev) * occ;
}

// Split of the token reduction of dw: as many splits as fit the output
// tiles into one round of resident blocks (a second, partial round would
// leave most CUs idle for a whole block), at most 32, with chunks of at
// least 512 tokens (a multiple of the 32-token step).
static int ste_splits(int64_t T, int64_t K, int64_t N, int64_t* chunk) {
  if (T <= 0) {  // empty reduction: one pass that writes zeros
    *chunk = ste::BR;
    return 1;
  }
  const int64_t tiles = ((N + ste::BM - 1) / ste::BM) * ((K + ste::BN - 1) / ste::BN);
  const int64_t slots = ste_slots();
  int64_t S = tiles >= slots ? 1 : std::min<int64_t>(slots / tiles, 32);
  S = std::max<int64_t>(1, std::min<int64_t>(S, (T + 511) / 512));
  int64_t c = (T + S - 1) / S;
  c = (c + ste::BR - 1) / ste::BR * ste::BR;
  S = std::max<int64_t>(1, (T + c - 1) / c);
  *chunk = c;
  return (int)S;
}

// Workspace of dw: the S partial sums [S, N, K] (when S > 1), then, from a
// 256-byte boundary, beta_t / 127 for every token.
static size_t ste_partials_bytes(int64_t T, int64_t K, int64_t N) {
  int64_t chunk = 0;
  const int S = ste_splits(T, K, N, &chunk);
  const size_t b = S > 1 ? (size_t)S * (size_t)N * (size_t)K * sizeof(float) : 0;
  return (b + 255) / 256 * 256;
}

size_t ste_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  if (T <= 0) return 0;
  return ste_partials_bytes(T, K, N) + (size_t)T * sizeof(float);
}

// beta_t / 127 (one IEEE division per token, as the definition states)
__global__ __launch_bounds__(256) void ste_token_scale_kernel(const float* __restrict__ beta,
                                                              int64_t T, float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) out[t] = beta[t] / 127.0f;
}

// ---------------------------------------------------------------------------
// Workspace of the allocation-free entry point: a device array that comes
// with the code object (each GPU the library runs on holds its own copy
// until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress reports for the device the work runs on, queried once
// per device with that device current.
static __device__ __align__(256) uint8_t scratch[SBL_STE_SCRATCH_BYTES];

static std::atomic<uintptr_t> scratch_addr[kMaxDevices];

hipError_t ste_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uintptr_t v = scratch_addr[dev].load(std::memory_order_acquire);
  if (v == 0) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    v = reinterpret_cast<uintptr_t>(p);
    scratch_addr[dev].store(v, std::memory_order_release);  // concurrent first calls store the same value
  }
  *out = reinterpret_cast<void*>(v);
  return hipSuccess;
}

hipError_t launch_ste_backward(const float* dy, const int8_t* xq, const float* beta,
                               const uint8_t* packed, const float* gamma, int64_t T, int64_t K,
                               int64_t N, float* dx, float* dw, void* workspace,
                               hipStream_t stream) {
  const int tiles_k = (int)((K + ste::BN - 1) / ste::BN);
  if (dx && T > 0) {
    const int64_t tiles = ((T + ste::BM - 1) / ste::BM) * tiles_k;
    if (tiles > INT32_MAX) return hipErrorInvalidConfiguration;
    SteArgs a{dy, xq, beta, packed, gamma, nullptr, dx, T, K, N, 0, tiles_k, (int)tiles};
    hipLaunchKernelGGL(ste_kernel<0>, dim3((unsigned)tiles), dim3(ste::NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dw && N > 0) {
    int64_t chunk = 0;
    const int S = ste_splits(T, K, N, &chunk);
    float* part = S > 1 ? reinterpret_cast<float*>(workspace) : dw;
    float* tscale = nullptr;
    if (T > 0) {
      tscale = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ste_partials_bytes(T, K, N));
      hipLaunchKernelGGL(ste_token_scale_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0,
                         stream, beta, T, tscale);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t tiles = ((N + ste::BM - 1) / ste::BM) * tiles_k;
    if (tiles * S > INT32_MAX) return hipErrorInvalidConfiguration;
    SteArgs a{dy, xq, beta, packed, gamma, tscale, part, T, K, N, chunk, tiles_k, (int)tiles};
    hipLaunchKernelGGL(ste_kernel<1>, dim3((unsigned)(tiles * S)), dim3(ste::NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = std::min<int64_t>((N * K + 255) / 256, 4096);
    hipLaunchKernelGGL(ste_dw_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       part, gamma, N, K, S, dw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbl
