// a5 -- classifier-free guidance combine and denoising discrepancy.
//
// eps = eps_u + w (eps_c - eps_u) elementwise, and rel-MAE = sum|eps_c -
// eps_u| / sum|eps_u| (Hybridiff technical summary, sections 2A and 2B).
// HBM-bound: one streaming read of each branch, one streaming write.  The reduction is
// deterministic: a grid whose size depends only on n writes one float64 pair
// per workgroup, and a single workgroup sums those pairs in a fixed order.
#include "dpp_common.h"

namespace dpp {

constexpr int kCfgThreads = 256;
constexpr int kCfgMaxBlocks = 1024;
constexpr int kCfgVecPerThread = 1;  // target vectors per thread per pass

static int cfg_blocks(int64_t n) {
  // 8 elements per 16-byte bf16 vector; the same grid serves fp32.
  const int64_t nvec = ceil_div(n, 8);
  const int64_t want = ceil_div(nvec, static_cast<int64_t>(kCfgThreads) * kCfgVecPerThread);
  return static_cast<int>(want < 1 ? 1 : (want > kCfgMaxBlocks ? kCfgMaxBlocks : want));
}

size_t cfg_workspace_bytes(int64_t n) { return static_cast<size_t>(cfg_blocks(n)) * 2 * sizeof(double); }

__device__ __forceinline__ void block_pair_to_partial(float sd, float su, double* partial) {
  __shared__ double red[kCfgThreads / kWave][2];
  double d = wave_sum_d(static_cast<double>(sd));
  double u = wave_sum_d(static_cast<double>(su));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) { red[w][0] = d; red[w][1] = u; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, c = 0.0;
    for (int i = 0; i < kCfgThreads / kWave; ++i) { a += red[i][0]; c += red[i][1]; }
    partial[2 * blockIdx.x] = a;
    partial[2 * blockIdx.x + 1] = c;
  }
}

template <typename T, bool kVecPath>
__global__ __launch_bounds__(kCfgThreads) void cfg_kernel(T* eps, const T* eps_c, const T* eps_u, int64_t n,
                                                          float w, double* partial) {
  float sd = 0.f, su = 0.f;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCfgThreads;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kCfgThreads + threadIdx.x;
  int64_t tail0 = 0;
  if constexpr (kVecPath) {
    constexpr int V = Elem<T>::kVec;
    const int64_t nvec = n / V;
    tail0 = nvec * V;
    const uint4* c4 = reinterpret_cast<const uint4*>(eps_c);
    const uint4* u4 = reinterpret_cast<const uint4*>(eps_u);
    uint4* e4 = reinterpret_cast<uint4*>(eps);
    for (int64_t i = tid; i < nvec; i += stride) {
      float c[V], u[V], e[V];
      Elem<T>::unpack(ld_stream(c4 + i), c);
      Elem<T>::unpack(ld_stream(u4 + i), u);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float d = c[j] - u[j];
        e[j] = fmaf(w, d, u[j]);
        sd += fabsf(d);
        su += fabsf(u[j]);
      }
      st_stream(e4 + i, Elem<T>::pack(e));
    }
    // elements past the last whole vector: first threads of block 0
    if (blockIdx.x == 0 && tail0 + threadIdx.x < n) {
      const int64_t i = tail0 + threadIdx.x;
      const float c = Elem<T>::load(eps_c, i), u = Elem<T>::load(eps_u, i);
      const float d = c - u;
      Elem<T>::store(eps, i, fmaf(w, d, u));
      sd += fabsf(d);
      su += fabsf(u);
    }
  } else {
    for (int64_t i = tid; i < n; i += stride) {
      const float c = Elem<T>::load(eps_c, i), u = Elem<T>::load(eps_u, i);
      const float d = c - u;
      Elem<T>::store(eps, i, fmaf(w, d, u));
      sd += fabsf(d);
      su += fabsf(u);
    }
  }
  if (partial != nullptr) block_pair_to_partial(sd, su, partial);
}

__global__ __launch_bounds__(kCfgThreads) void cfg_final_kernel(const double* partial, int nblk, float* relmae) {
  __shared__ double red[kCfgThreads / kWave][2];
  double d = 0.0, u = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kCfgThreads) {
    d += partial[2 * i];
    u += partial[2 * i + 1];
  }
  d = wave_sum_d(d);
  u = wave_sum_d(u);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) { red[w][0] = d; red[w][1] = u; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, c = 0.0;
    for (int i = 0; i < kCfgThreads / kWave; ++i) { a += red[i][0]; c += red[i][1]; }
    *relmae = static_cast<float>(a / c);  // IEEE: 0/0 -> NaN, x/0 -> inf
  }
}

hipError_t launch_cfg(void* eps, float* relmae, const void* eps_c, const void* eps_u, int64_t n,
                      float guidance, void* ws, bool bf16, hipStream_t s) {
  const int nblk = cfg_blocks(n);
  double* partial = relmae ? static_cast<double*>(ws) : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(eps) % 16 == 0) && (reinterpret_cast<uintptr_t>(eps_c) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(eps_u) % 16 == 0);
  if (bf16) {
    auto* e = static_cast<uint16_t*>(eps);
    auto* c = static_cast<const uint16_t*>(eps_c);
    auto* u = static_cast<const uint16_t*>(eps_u);
    if (vec)
      hipLaunchKernelGGL((cfg_kernel<uint16_t, true>), dim3(nblk), dim3(kCfgThreads), 0, s, e, c, u, n, guidance, partial);
    else
      hipLaunchKernelGGL((cfg_kernel<uint16_t, false>), dim3(nblk), dim3(kCfgThreads), 0, s, e, c, u, n, guidance, partial);
  } else {
    auto* e = static_cast<float*>(eps);
    auto* c = static_cast<const float*>(eps_c);
    auto* u = static_cast<const float*>(eps_u);
    if (vec)
      hipLaunchKernelGGL((cfg_kernel<float, true>), dim3(nblk), dim3(kCfgThreads), 0, s, e, c, u, n, guidance, partial);
    else
      hipLaunchKernelGGL((cfg_kernel<float, false>), dim3(nblk), dim3(kCfgThreads), 0, s, e, c, u, n, guidance, partial);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || relmae == nullptr) return err;
  hipLaunchKernelGGL(cfg_final_kernel, dim3(1), dim3(kCfgThreads), 0, s, static_cast<const double*>(ws), nblk, relmae);
  return hipGetLastError();
}

}  // namespace dpp
