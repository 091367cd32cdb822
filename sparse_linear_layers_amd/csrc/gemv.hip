// Decode product (1 <= T <= 16 tokens) over packed ternary weights, single
// or grouped over many matrices in one launch.  Same contract as the
// prefill product ("Sparse-BitNet Guide", "Mathematical Formulation of
// Sparse-BitLinear", step 4); the model card "halo-sparse-bitnet-3:4-500m"
// ("What does NOT ship") notes that serving needs a kernel that reads the
// packed 2-bit layout directly, which this is.
//
// The stream of packed codes (1/4 B per weight) is the whole cost, so the
// kernel is built around reading it once at full HBM rate with as little
// ALU per byte as possible:
//  * A wave owns 16 weight rows; lane l reads 16 bytes (64 codes) of row
//    l%16 at k offset 64*(l/16) of each 256-code step.  The v_mfma
//    i32_16x16x64_i8 then does the whole k reduction in the matrix core:
//    no cross-lane reduction, and the token count (1..16) rides in the
//    MFMA's N dimension for free.
//  * Codes are expanded in "strided" byte order (3 ALU ops per 4 weights
//    instead of 5); the matching x~ slab is staged in LDS once per block in
//    the same order, so the pairing of weights and activations is exact.
#include "sbl_device.h"
#include "sbl_launch.h"

namespace sbl {

constexpr int kGemvRowsPerWave = 16;
constexpr int kGemvWaves = 4;
constexpr int kGemvRowsPerBlock = kGemvRowsPerWave * kGemvWaves;
constexpr int kGemvSlab = 1024;                  // codes per staged x~ slab
constexpr int kGemvLdsStride = kGemvSlab + 16;   // bytes per staged token

struct GemvArgs {
  const sbl_gemv_desc* descs;  // device descriptors, or null: use `single`
  sbl_gemv_desc single;
  int count;
  int T;
  int block_start[kMaxGroupedGemv + 1];
};

__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t xs[SBL_GEMV_MAX_TOKENS * kGemvLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  // descriptor of this block: the last d with block_start[d] <= b, found
  // with one round of parallel reads and a ballot count (one memory latency
  // instead of a dependent binary search)
  int d = 0;
  if (a.descs) {
    int cnt = 0;
    for (int j = 0; j < a.count; j += kWave) {
      const int idx = j + lane;
      const bool le = idx < a.count && a.block_start[idx] <= b;
      cnt += __popcll(__ballot(le));
    }
    d = cnt - 1;
  }
  const sbl_gemv_desc desc = a.descs ? a.descs[d] : a.single;
  const int64_t K = desc.K, N = desc.N;
  const int T = a.T;
  const int64_t row0 = (int64_t)(b - a.block_start[d]) * kGemvRowsPerBlock + wave * kGemvRowsPerWave;
  const int g = lane >> 4;  // k group within a step
  const int tok = lane & 15;
  const uint8_t* wrow = desc.packed + min(row0 + (lane & 15), N - 1) * (K >> 2);
  const int xrow = min(tok, T - 1) * kGemvLdsStride;  // LDS row this lane's B operand reads

  // Weight codes of one slab: super-step s (0..3) is 16 bytes = 64 codes of
  // row lane%16 at k offset s*256 + 64*g of the slab (4 lanes cover 64
  // contiguous bytes of a row).  Its dword i feeds MFMA i, whose lane group g
  // then covers k = s*256 + 64*g + 16*i .. +16 on both operands.  The loads
  // of slab n+1 are issued before slab n is computed.
  constexpr int kSteps = kGemvSlab / 256;
  uint4 w0, w1, w2, w3;
#define SBL_WLD(s, ks_)                                                                 \
  w##s = ((ks_) + (s) * 256 + 64 * g < K)                                               \
             ? *reinterpret_cast<const uint4*>(wrow + (((ks_) + (s) * 256 + 64 * g) >> 2)) \
             : make_uint4(0u, 0u, 0u, 0u);
#define SBL_WLOAD(ks_)                                                                  \
  { SBL_WLD(0, ks_) SBL_WLD(1, ks_) SBL_WLD(2, ks_) SBL_WLD(3, ks_) }
  static_assert(kSteps == 4, "four super-steps per slab");

  v4i acc = {0, 0, 0, 0};
  SBL_WLOAD((int64_t)0);
  for (int64_t ks = 0; ks < K; ks += kGemvSlab) {
    const int width = (int)min<int64_t>(kGemvSlab, K - ks);  // multiple of 64
    __syncthreads();
    // stage x~[0:T, ks:ks+width] with each 16-byte chunk byte-transposed
    const int cpt = width >> 4;
    for (int t = 0; t < T; ++t)
      for (int q = tid; q < cpt; q += 256) {
        const uint4 v = *reinterpret_cast<const uint4*>(desc.xq + (int64_t)t * K + ks + 16 * q);
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
        transpose4x4(in, o);
        *reinterpret_cast<uint4*>(xs + t * kGemvLdsStride + 16 * q) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    __syncthreads();
    const uint4 wv[kSteps] = {w0, w1, w2, w3};
    if (ks + kGemvSlab < K) SBL_WLOAD(ks + kGemvSlab);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s * 256 >= width) break;  // uniform: whole super-steps past the slab end
      const int kin = s * 256 + 64 * g;  // k offset of this lane group inside the slab
      const uint32_t wd[4] = {wv[s].x, wv[s].y, wv[s].z, wv[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t e[4];
        expand16_strided(wd[i], e);
        const v4i av = {(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
        // lanes of token slots >= T read a real row (their output columns
        // are never stored); past the k tail the codes are zero
        const v4i bv = *reinterpret_cast<const v4i*>(xs + xrow + kin + 16 * i);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
      }
    }
  }
#undef SBL_WLD
#undef SBL_WLOAD
  // lane holds C[row = 4*(lane/16) + r][token = lane%16]
  if (tok < T) {
    const float bt = __fdiv_rn(desc.beta[tok], 127.0f);
    const int64_t o = row0 + 4 * g;
    float* yp = desc.y + (int64_t)tok * N;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (o + r < N) yp[o + r] = ((float)acc[r] * bt) * load_scale(desc.row_scale, desc.scale_dtype, o + r);
  }
}

hipError_t launch_gemv(const sbl_gemv_desc* host, const sbl_gemv_desc* dev, int count, int64_t T,
                       hipStream_t stream) {
  for (int first = 0; first < count;) {
    const int last = std::min(count, first + kMaxGroupedGemv);
    GemvArgs a{};
    a.descs = dev ? dev + first : nullptr;
    if (!dev) a.single = host[first];
    a.count = last - first;
    a.T = (int)T;
    int64_t blocks = 0;
    for (int d = first; d < last; ++d) {
      a.block_start[d - first] = (int)blocks;
      blocks += (host[d].N + kGemvRowsPerBlock - 1) / kGemvRowsPerBlock;
    }
    a.block_start[last - first] = (int)blocks;
    if (blocks > 0) {
      hipLaunchKernelGGL(gemv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    first = last;
  }
  return hipSuccess;
}

}  // namespace sbl
