// Projection GEMM: y[b, m, n] = sum_k x[b, m, k] w[n, k] + bias[n].
//
// The to_q / to_k / to_v / to_out projections of the wrapped attention
// module (DistriSelfAttentionPP, DistriFusion architecture article, attention
// section).  Row and batch strides are free, so the K/V projection of the
// fresh patch can write straight into its rows of the private full-image K/V
// buffer (the splice, fused into the projection epilogue).
//
// bf16 path: MFMA v_mfma_f32_16x16x32_bf16 with A = weight rows (output
// channels, K-contiguous) and B = token rows (K-contiguous).  A workgroup owns
// 128 channels x 128 tokens; eight waves, each 32 channels x 64 tokens (2 x 4
// accumulator tiles).  K is walked in 64-wide slices staged in LDS (XOR-
// swizzled rows, double-buffered), the next slice fetched into registers
// during the current one's MFMAs; one barrier per slice.  Each lane's
// accumulator holds four consecutive channels of one token: one 8-byte store.
//
// f32 path: one thread per output, direct loop (small shapes).
#include "dpp_common.h"

namespace dpp {

__global__ __launch_bounds__(256) void linear_f32_kernel(float* __restrict__ y, const float* __restrict__ x,
                                                         const float* __restrict__ w, const float* __restrict__ bias,
                                                         int64_t M, int64_t K, int64_t N, int64_t ld_x, int64_t bs_x,
                                                         int64_t ld_y, int64_t bs_y) {
  const int64_t b = blockIdx.y;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < M * N;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = idx / N, n = idx % N;
    const float* xr = x + b * bs_x + m * ld_x;
    const float* wr = w + n * K;
    float acc = bias ? bias[n] : 0.f;
    for (int64_t k = 0; k < K; ++k) acc = fmaf(xr[k], wr[k], acc);
    y[b * bs_y + m * ld_y + n] = acc;
  }
}

constexpr int kLinBN = 128;   // output channels per workgroup
constexpr int kLinBM = 128;   // tokens per workgroup
constexpr int kLinKC = 64;    // K slice (8 x 16-byte vectors per row)
constexpr int kLinThreads = 512;
constexpr int kLinCG = 2;     // 16-channel MFMA groups per wave
constexpr int kLinTG = 4;     // 16-token MFMA groups per wave
constexpr int kLinIters = kLinBN * 8 / kLinThreads;  // staged vectors per thread per operand

struct LinArgs {
  const uint16_t* x;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  int64_t M, K, N, ld_x, bs_x, ld_y, bs_y;
};

// LDS row of 8 x 16-byte slots, slot XOR-swizzled by the row index.
__device__ __forceinline__ int lin_swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

__global__ __launch_bounds__(kLinThreads) void linear_bf16_mfma_kernel(LinArgs a) {
  __shared__ uint4 As[2][kLinBN * 8];
  __shared__ uint4 Bs[2][kLinBM * 8];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wn = wave % 4, wm = wave / 4;
  const int64_t b = blockIdx.z;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kLinBN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kLinBM;
  const uint16_t* xb = a.x + b * a.bs_x;

  // staging map: vector id -> (row, 16-byte slot) of a 128 x 64 slice
  const uint16_t* a_src[kLinIters];
  const uint16_t* b_src[kLinIters];
#pragma unroll
  for (int u = 0; u < kLinIters; ++u) {
    const int id = tid + u * kLinThreads;
    const int row = id >> 3, slot = id & 7;
    a_src[u] = (n0 + row < a.N) ? a.w + (n0 + row) * a.K + slot * 8 : nullptr;
    b_src[u] = (m0 + row < a.M) ? xb + (m0 + row) * a.ld_x + slot * 8 : nullptr;
  }
  uint4 a_reg[kLinIters], b_reg[kLinIters];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < kLinIters; ++u) {
      const int slot = (tid + u * kLinThreads) & 7;
      const bool in_k = k0 + slot * 8 < a.K;  // K % 8 == 0: a vector is wholly in or out
      a_reg[u] = (a_src[u] != nullptr && in_k) ? *reinterpret_cast<const uint4*>(a_src[u] + k0) : make_uint4(0, 0, 0, 0);
      b_reg[u] = (b_src[u] != nullptr && in_k) ? *reinterpret_cast<const uint4*>(b_src[u] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kLinIters; ++u) {
      const int id = tid + u * kLinThreads;
      As[buf][lin_swz(id >> 3, id & 7)] = a_reg[u];
      Bs[buf][lin_swz(id >> 3, id & 7)] = b_reg[u];
    }
  };

  f32x4 acc[kLinCG][kLinTG];
#pragma unroll
  for (int i = 0; i < kLinCG; ++i)
#pragma unroll
    for (int j = 0; j < kLinTG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kg = lane >> 4, pl = lane & 15;
  // fragment rows r = base + 16 i + pl share (r & 7) = (pl & 7)
  const int a_row0 = wn * 32 + pl, b_row0 = wm * 64 + pl;
  const int nslices = static_cast<int>((a.K + kLinKC - 1) / kLinKC);
  load(0);
  store(0);
  if (nslices > 1) load(kLinKC);
  __syncthreads();
  for (int s = 0; s < nslices; ++s) {
    const int buf = s & 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int slot = (ks * 4 + kg) ^ (pl & 7);
      bf16x8 af[kLinCG], bfr[kLinTG];
#pragma unroll
      for (int i = 0; i < kLinCG; ++i) af[i] = __builtin_bit_cast(bf16x8, As[buf][(a_row0 + 16 * i) * 8 + slot]);
#pragma unroll
      for (int j = 0; j < kLinTG; ++j) bfr[j] = __builtin_bit_cast(bf16x8, Bs[buf][(b_row0 + 16 * j) * 8 + slot]);
#pragma unroll
      for (int i = 0; i < kLinCG; ++i)
#pragma unroll
        for (int j = 0; j < kLinTG; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // stage slice s+1 (in registers) into the other buffer, last read before
    // the previous barrier; then fetch slice s+2
    if (s + 1 < nslices) store(buf ^ 1);
    __syncthreads();
    if (s + 2 < nslices) load(static_cast<int64_t>(s + 2) * kLinKC);
  }

  // epilogue: lane holds channels n0 + wn*32 + 16 i + 4 kg + 0..3 of token m0 + wm*64 + 16 j + pl
#pragma unroll
  for (int j = 0; j < kLinTG; ++j) {
    const int64_t m = m0 + wm * 64 + 16 * j + pl;
    if (m >= a.M) continue;
    uint16_t* yp = a.y + b * a.bs_y + m * a.ld_y;
#pragma unroll
    for (int i = 0; i < kLinCG; ++i) {
      const int64_t n = n0 + wn * 32 + 16 * i + 4 * kg;
      if (n >= a.N) continue;
      float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
      if (a.bias) { v0 += a.bias[n]; v1 += a.bias[n + 1]; v2 += a.bias[n + 2]; v3 += a.bias[n + 3]; }
      uint2 out;
      out.x = pack_bf16x2(v0, v1);
      out.y = pack_bf16x2(v2, v3);
      *reinterpret_cast<uint2*>(yp + n) = out;
    }
  }
}

hipError_t launch_linear(void* y, const void* x, const void* w, const float* bias, int64_t B, int64_t M, int64_t K,
                         int64_t N, int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, bool bf16, hipStream_t s) {
  if (!bf16) {
    int64_t blocks = ceil_div(M * N, 256);
    if (blocks > 65535) blocks = 65535;
    hipLaunchKernelGGL(linear_f32_kernel, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(B)), dim3(256), 0,
                       s, static_cast<float*>(y), static_cast<const float*>(x), static_cast<const float*>(w), bias, M,
                       K, N, ld_x, bs_x, ld_y, bs_y);
    return hipGetLastError();
  }
  LinArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.bias = bias;
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.K = K;
  a.N = N;
  a.ld_x = ld_x;
  a.bs_x = bs_x;
  a.ld_y = ld_y;
  a.bs_y = bs_y;
  dim3 grid(static_cast<unsigned>(ceil_div(M, kLinBM)), static_cast<unsigned>(ceil_div(N, kLinBN)),
            static_cast<unsigned>(B));
  hipLaunchKernelGGL(linear_bf16_mfma_kernel, grid, dim3(kLinThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dpp
