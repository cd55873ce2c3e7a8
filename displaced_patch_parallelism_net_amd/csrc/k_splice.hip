// a1 -- splice the fresh patch into the full-image buffer.
//
// The one-device stand-in for gathering each device's patch output and
// concatenating along the height axis into the reused full-image buffer
// (DistriFusion architecture article, communication section).  In NHWC the
// row band of one batch entry is a single contiguous slab, so the splice is B
// slab copies: HBM-bound, 16-byte streaming (non-temporal) loads/stores,
// four vectors in flight per thread.
#include "dpp_common.h"

namespace dpp {

constexpr int kSpliceThreads = 256;
constexpr int kSpliceUnroll = 4;

__global__ __launch_bounds__(kSpliceThreads) void splice_vec_kernel(
    uint4* __restrict__ full, const uint4* __restrict__ patch, int64_t slab, int64_t full_bstride,
    int64_t off) {
  const int64_t b = blockIdx.y;
  uint4* dst = full + b * full_bstride + off;
  const uint4* src = patch + b * slab;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSpliceThreads * kSpliceUnroll + threadIdx.x;
  uint4 r[kSpliceUnroll];
#pragma unroll
  for (int u = 0; u < kSpliceUnroll; ++u) {
    const int64_t i = base + u * kSpliceThreads;
    if (i < slab) r[u] = ld_stream(src + i);
  }
#pragma unroll
  for (int u = 0; u < kSpliceUnroll; ++u) {
    const int64_t i = base + u * kSpliceThreads;
    if (i < slab) st_stream(dst + i, r[u]);
  }
}

// Fallback for slabs that are not 16-byte aligned: one element per thread.
template <typename T>
__global__ __launch_bounds__(kSpliceThreads) void splice_elem_kernel(
    T* __restrict__ full, const T* __restrict__ patch, int64_t slab, int64_t full_bstride, int64_t off) {
  const int64_t b = blockIdx.y;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kSpliceThreads + threadIdx.x; i < slab;
       i += static_cast<int64_t>(gridDim.x) * kSpliceThreads)
    full[b * full_bstride + off + i] = patch[b * slab + i];
}

hipError_t launch_splice(void* full, const void* patch, int64_t B, int64_t H, int64_t W, int64_t C,
                         int64_t row0, int64_t rows, int esize, hipStream_t s) {
  const int64_t slab_bytes = rows * W * C * esize;
  const int64_t bstride_bytes = H * W * C * esize;
  const int64_t off_bytes = row0 * W * C * esize;
  const bool vec = (reinterpret_cast<uintptr_t>(full) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(patch) % 16 == 0) && slab_bytes % 16 == 0 &&
                   bstride_bytes % 16 == 0 && off_bytes % 16 == 0;
  if (vec) {
    const int64_t slab = slab_bytes / 16;
    dim3 grid(static_cast<unsigned>(ceil_div(slab, kSpliceThreads * kSpliceUnroll)), static_cast<unsigned>(B));
    hipLaunchKernelGGL(splice_vec_kernel, grid, dim3(kSpliceThreads), 0, s, static_cast<uint4*>(full),
                       static_cast<const uint4*>(patch), slab, bstride_bytes / 16, off_bytes / 16);
  } else {
    const int64_t slab = slab_bytes / esize;
    const int64_t blocks = ceil_div(slab, kSpliceThreads);
    dim3 grid(static_cast<unsigned>(blocks < 4096 ? blocks : 4096), static_cast<unsigned>(B));
    if (esize == 2)
      hipLaunchKernelGGL(splice_elem_kernel<uint16_t>, grid, dim3(kSpliceThreads), 0, s,
                         static_cast<uint16_t*>(full), static_cast<const uint16_t*>(patch), slab,
                         bstride_bytes / 2, off_bytes / 2);
    else
      hipLaunchKernelGGL(splice_elem_kernel<uint32_t>, grid, dim3(kSpliceThreads), 0, s,
                         static_cast<uint32_t*>(full), static_cast<const uint32_t*>(patch), slab,
                         bstride_bytes / 4, off_bytes / 4);
  }
  return hipGetLastError();
}

}  // namespace dpp
