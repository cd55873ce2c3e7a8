// a3 -- 3x3 convolution of the patch rows with halo rows from the stale image.
//
// DistriConv2dPP (DistriFusion architecture article, conv section): each
// device convolves only its own rows (DistriFusion reading notes,
// Introduction, fourth paragraph); the rows just above and below its band
// belong to neighbouring patches and come from the previous step's
// activations.
//
// bf16 path: implicit GEMM on MFMA.  M = output channels (A = weights,
// [Cout][tap][Cin] rows are K-contiguous), N = output pixels (B = input
// pixels, channel-contiguous in NHWC), K = 9 taps x Cin.  A workgroup owns a
// 128-channel x 128-pixel tile, the pixels being TR rows x TC columns of the
// patch.  For each 64-channel slice of Cin the (TR+2) x (TC+2) input band,
// halos included, is staged once in LDS and reused by all nine taps; the
// weights of one tap are staged per step.  Four waves each compute 64 x 64
// with v_mfma_f32_16x16x32_bf16; the accumulator's lane layout gives each lane
// four consecutive output channels of one pixel, stored as one 8-byte write.
// Loads for the next step are issued before the current step's MFMAs.
//
// f32 path: one thread per output element, direct loops (small shapes).
#include "dpp_common.h"

namespace dpp {

// ------------------------------------------------------------------ fp32 direct
__global__ __launch_bounds__(256) void conv3x3_f32_kernel(float* __restrict__ y, const float* __restrict__ x,
                                                          const float* __restrict__ stale,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ bias, int64_t B, int64_t H,
                                                          int64_t W, int64_t Cin, int64_t Cout, int64_t row0,
                                                          int64_t rows) {
  const int64_t total = B * rows * W * Cout;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t o = idx % Cout;
    const int64_t pix = idx / Cout;
    const int64_t col = pix % W;
    const int64_t i = (pix / W) % rows;
    const int64_t b = pix / (W * rows);
    float acc = bias ? bias[o] : 0.f;
    for (int dy = 0; dy < 3; ++dy) {
      const int64_t r = i + dy - 1;      // patch-relative row
      const int64_t ir = row0 + r;       // image row
      if (ir < 0 || ir >= H) continue;   // zero padding
      const float* src = (r >= 0 && r < rows) ? x + (b * rows + r) * W * Cin : stale + (b * H + ir) * W * Cin;
      for (int dx = 0; dx < 3; ++dx) {
        const int64_t c = col + dx - 1;
        if (c < 0 || c >= W) continue;
        const float* px = src + c * Cin;
        const float* wr = w + ((o * 3 + dy) * 3 + dx) * Cin;
        for (int64_t ci = 0; ci < Cin; ++ci) acc = fmaf(wr[ci], px[ci], acc);
      }
    }
    y[idx] = acc;
  }
}

// ------------------------------------------------------------------ bf16 MFMA implicit GEMM
constexpr int kConvThreads = 256;
constexpr int kConvBM = 128;  // output channels per workgroup
constexpr int kConvBN = 128;  // output pixels per workgroup
constexpr int kConvKC = 64;   // input channels per slice (8 x 16-byte vectors)

struct ConvArgs {
  const uint16_t* x;
  const uint16_t* stale;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  int H, W, Cin, Cout, row0, rows;
  int tiles_c;  // column tiles per patch row band
};

// LDS row of 8 x 16-byte slots, slot index XOR-swizzled by the row index so
// that 16 lanes reading the same logical slot of consecutive rows spread over
// the banks.
__device__ __forceinline__ int swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

template <int TC>
__global__ __launch_bounds__(kConvThreads) void conv3x3_bf16_mfma_kernel(ConvArgs a) {
  constexpr int TR = kConvBN / TC;
  constexpr int BW = TC + 2;           // band columns
  constexpr int BPIX = (TR + 2) * BW;  // band pixels
  constexpr int BAND_VEC = BPIX * 8;   // 16-byte vectors per band
  constexpr int BAND_ITERS = (BAND_VEC + kConvThreads - 1) / kConvThreads;
  constexpr int W_VEC = kConvBM * 8;
  constexpr int W_ITERS = W_VEC / kConvThreads;  // 4

  __shared__ uint4 band[BPIX * 8];
  __shared__ uint4 wts[kConvBM * 8];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.z;
  const int m0 = blockIdx.y * kConvBM;
  const int tile_r = blockIdx.x / a.tiles_c, tile_c = blockIdx.x % a.tiles_c;
  const int pr0 = tile_r * TR, pc0 = tile_c * TC;  // patch-relative origin of the pixel tile
  const int H = a.H, W = a.W, Cin = a.Cin;
  const int64_t ktot = 9LL * Cin;

  // -------- global -> register staging
  uint4 band_reg[BAND_ITERS];
  uint4 w_reg[W_ITERS];

  auto load_band = [&](int c0) {
#pragma unroll
    for (int u = 0; u < BAND_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (id < BAND_VEC) {
        const int pix = id >> 3, slot = id & 7;
        const int br = pix / BW, bc = pix % BW;
        const int r = pr0 - 1 + br;  // patch-relative
        const int ir = a.row0 + r;   // image row
        const int col = pc0 - 1 + bc;
        if (ir >= 0 && ir < H && col >= 0 && col < W) {
          const uint16_t* src = (r >= 0 && r < a.rows)
                                    ? a.x + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * Cin
                                    : a.stale + ((static_cast<int64_t>(b) * H + ir) * W + col) * Cin;
          v = *reinterpret_cast<const uint4*>(src + c0 + slot * 8);
        }
      }
      band_reg[u] = v;
    }
  };
  auto load_w = [&](int tap, int c0) {
#pragma unroll
    for (int u = 0; u < W_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      const int m = id >> 3, slot = id & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + m < a.Cout) v = *reinterpret_cast<const uint4*>(a.w + (m0 + m) * ktot + tap * Cin + c0 + slot * 8);
      w_reg[u] = v;
    }
  };
  auto store_band = [&]() {
#pragma unroll
    for (int u = 0; u < BAND_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      if (id < BAND_VEC) band[swz(id >> 3, id & 7)] = band_reg[u];
    }
  };
  auto store_w = [&]() {
#pragma unroll
    for (int u = 0; u < W_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      wts[swz(id >> 3, id & 7)] = w_reg[u];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane pixel coordinates of the four 16-pixel groups of this wave.
  int pix_tr[4], pix_tc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pt = wn * 64 + j * 16 + (lane & 15);
    pix_tr[j] = pt / TC;
    pix_tc[j] = pt % TC;
  }
  const int kg = lane >> 4;  // 0..3: which 8-element k group of the 32-wide MFMA step

  const int nslices = Cin / kConvKC;
  const int nsteps = nslices * 9;
  load_band(0);
  load_w(0, 0);
  for (int step = 0; step < nsteps; ++step) {
    const int slice = step / 9, tap = step % 9;
    __syncthreads();  // previous step's LDS reads are done
    if (tap == 0) store_band();
    store_w();
    __syncthreads();
    if (step + 1 < nsteps) {
      const int ns = step + 1, nslice = ns / 9, ntap = ns % 9;
      if (ntap == 0) load_band(nslice * kConvKC);
      load_w(ntap, nslice * kConvKC);
    }
    (void)slice;
    const int dy = tap / 3, dx = tap % 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + i * 16 + (lane & 15);
        af[i] = __builtin_bit_cast(bf16x8, wts[swz(m, ks * 4 + kg)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bp = (pix_tr[j] + dy) * BW + pix_tc[j] + dx;
        bfr[j] = __builtin_bit_cast(bf16x8, band[swz(bp, ks * 4 + kg)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // -------- epilogue: lane holds channels m0 + wm*64 + i*16 + 4*(lane/16) + 0..3 of one pixel
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = pr0 + pix_tr[j], col = pc0 + pix_tc[j];
    if (r >= a.rows || col >= W) continue;
    uint16_t* yp = a.y + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * a.Cout;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + i * 16 + 4 * kg;
      if (m >= a.Cout) continue;
      float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
      if (a.bias) { v0 += a.bias[m]; v1 += a.bias[m + 1]; v2 += a.bias[m + 2]; v3 += a.bias[m + 3]; }
      uint2 out;
      out.x = pack_bf16x2(v0, v1);
      out.y = pack_bf16x2(v2, v3);
      *reinterpret_cast<uint2*>(yp + m) = out;
    }
  }
}

hipError_t launch_conv3x3(void* y, const void* x, const void* stale_full, const void* weight, const float* bias,
                          int64_t B, int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows,
                          bool bf16, hipStream_t s) {
  if (!bf16) {
    const int64_t total = B * rows * W * Cout;
    int64_t blocks = ceil_div(total, 256);
    if (blocks > 65535) blocks = 65535;
    hipLaunchKernelGGL(conv3x3_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<float*>(y), static_cast<const float*>(x), static_cast<const float*>(stale_full),
                       static_cast<const float*>(weight), bias, B, H, W, Cin, Cout, row0, rows);
    return hipGetLastError();
  }
  ConvArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.stale = static_cast<const uint16_t*>(stale_full);
  a.w = static_cast<const uint16_t*>(weight);
  a.bias = bias;
  a.y = static_cast<uint16_t*>(y);
  a.H = static_cast<int>(H);
  a.W = static_cast<int>(W);
  a.Cin = static_cast<int>(Cin);
  a.Cout = static_cast<int>(Cout);
  a.row0 = static_cast<int>(row0);
  a.rows = static_cast<int>(rows);
  const int TC = W > 32 ? 64 : (W > 16 ? 32 : 16);
  const int TR = kConvBN / TC;
  a.tiles_c = static_cast<int>(ceil_div(W, TC));
  const int64_t tiles = ceil_div(rows, TR) * a.tiles_c;
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(ceil_div(Cout, kConvBM)), static_cast<unsigned>(B));
  if (TC == 64)
    hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<64>, grid, dim3(kConvThreads), 0, s, a);
  else if (TC == 32)
    hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<32>, grid, dim3(kConvThreads), 0, s, a);
  else
    hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<16>, grid, dim3(kConvThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dpp
