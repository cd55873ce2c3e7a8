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
// pixels, channel-contiguous in NHWC), K = 9 taps x Cin.  A workgroup owns 2
// patch rows x 16*TG columns x 128 output channels (TG chosen per width so
// the tiles cover the rows exactly where possible: 240 columns -> 3 tiles of
// 80, one workgroup per CU).  For each 64-channel slice of Cin the halo band
// (4 rows x 16*TG+2 columns, halo rows from the stale image) is staged once in
// LDS and reused by all nine taps; the weights of one tap are staged per
// step; both double-buffered in LDS, weights fetched two steps ahead into
// registers.  Eight waves (two per SIMD) each compute 32 channels x 16*TG
// pixels of one tile row with v_mfma_f32_16x16x32_bf16; the accumulator's
// lane layout gives each lane four consecutive output channels of one pixel,
// stored as one 8-byte write.
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
// Workgroup tile: 2 patch rows x 16*TG columns of output pixels x 128 output
// channels; 2 x kConvWN waves, wave (wr, wn) owns tile row wr and channels
// [CW wn, CW wn + CW): TG x CW/16 accumulator tiles of 16 x 16.  The host picks TG
// (1..5) so that the tiles cover the row width with the least waste and the
// workgroup count fills the 256 CUs in whole rounds (e.g. 240 columns ->
// TG 5: three tiles per row pair).
// K loop: step = (64-channel slice, tap).  The (2+2) x (16 TG + 2) halo band
// of a slice is staged once and reused by its nine taps; the weights of one
// tap (128 x 64) per step.  Both are double-buffered in LDS; weights are
// fetched into registers two steps ahead, right after a step's single
// barrier.
constexpr int kConvWN = 4;                      // waves across the 128 output channels
constexpr int kConvCW = 128 / kConvWN;          // output channels per wave
constexpr int kConvCG = kConvCW / 16;           // 16-channel MFMA groups per wave
constexpr int kConvThreads = 2 * kConvWN * 64;  // 2 tile rows x kConvWN
constexpr int kConvBM = 128;  // output channels per workgroup
constexpr int kConvKC = 64;   // input channels per slice (8 x 16-byte vectors)
constexpr int kConvTR = 2;    // patch rows per workgroup
constexpr int kConvTPS = 2;   // taps per barrier step

struct ConvArgs {
  const uint16_t* x;
  const uint16_t* stale;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  int H, W, Cin, Cout, row0, rows;
  int tiles_c;  // column tiles per row pair
};

// LDS row of 8 x 16-byte slots, slot index XOR-swizzled by the row index so
// that 16 lanes reading the same logical slot of consecutive rows spread over
// the banks.
__device__ __forceinline__ int swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

template <int TG>
__global__ __launch_bounds__(kConvThreads, 1) void conv3x3_bf16_mfma_kernel(ConvArgs a) {
  constexpr int TC = 16 * TG;           // output columns per tile
  constexpr int BW = TC + 2;            // band columns
  constexpr int BPIX = (kConvTR + 2) * BW;
  constexpr int BAND_VEC = BPIX * 8;    // 16-byte vectors per band
  constexpr int BAND_ITERS = (BAND_VEC + kConvThreads - 1) / kConvThreads;
  constexpr int W_ITERS = kConvBM * 8 / kConvThreads;

  __shared__ uint4 band[2][BPIX * 8];
  __shared__ uint4 wts[2][kConvTPS][kConvBM * 8];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wr = wave / kConvWN, wn = wave % kConvWN;
  const int b = blockIdx.z;
  const int m0 = blockIdx.y * kConvBM;
  const int tile_r = blockIdx.x / a.tiles_c, tile_c = blockIdx.x % a.tiles_c;
  const int pr0 = tile_r * kConvTR, pc0 = tile_c * TC;  // patch-relative origin of the pixel tile
  const int H = a.H, W = a.W, Cin = a.Cin;
  const int64_t ktot = 9LL * Cin;

  uint4 band_reg[BAND_ITERS];
  uint4 w_regA[kConvTPS][W_ITERS], w_regB[kConvTPS][W_ITERS];  // weights of the next two steps

  // Per-thread source pointers, computed once: band vector u of the first
  // slice (x for patch rows, the stale image for halo rows; nullptr = zero
  // padding) and the four weight rows.  Each step only adds a uniform offset.
  const uint16_t* band_src[BAND_ITERS];
#pragma unroll
  for (int u = 0; u < BAND_ITERS; ++u) {
    const int id = tid + u * kConvThreads;
    band_src[u] = nullptr;
    if (id < BAND_VEC) {
      const int pix = id >> 3, slot = id & 7;
      const int br = pix / BW, bc = pix % BW;
      const int r = pr0 - 1 + br;  // patch-relative
      const int ir = a.row0 + r;   // image row
      const int col = pc0 - 1 + bc;
      if (ir >= 0 && ir < H && col >= 0 && col < W)
        band_src[u] = ((r >= 0 && r < a.rows) ? a.x + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * Cin
                                              : a.stale + ((static_cast<int64_t>(b) * H + ir) * W + col) * Cin) +
                      slot * 8;
    }
  }
  const uint16_t* w_src[W_ITERS];
#pragma unroll
  for (int u = 0; u < W_ITERS; ++u) {
    const int id = tid + u * kConvThreads;
    const int m = id >> 3, slot = id & 7;
    w_src[u] = (m0 + m < a.Cout) ? a.w + (m0 + m) * ktot + slot * 8 : nullptr;
  }

  auto load_band = [&](int c0) {
#pragma unroll
    for (int u = 0; u < BAND_ITERS; ++u) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (band_src[u] != nullptr) v = *reinterpret_cast<const uint4*>(band_src[u] + c0);
      band_reg[u] = v;
    }
  };
  const int nslices = Cin / kConvKC;
  const int nflat = nslices * 9;  // (slice, tap) pairs
  const int nsteps = (nflat + kConvTPS - 1) / kConvTPS;
  auto load_w = [&](uint4 (&w_reg)[kConvTPS][W_ITERS], int step) {
#pragma unroll
    for (int i = 0; i < kConvTPS; ++i) {
      const int f = step * kConvTPS + i;
      const int sl = f / 9;
      const int off = (f - sl * 9) * Cin + sl * kConvKC;
#pragma unroll
      for (int u = 0; u < W_ITERS; ++u) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (w_src[u] != nullptr && f < nflat) v = *reinterpret_cast<const uint4*>(w_src[u] + off);
        w_reg[i][u] = v;
      }
    }
  };
  auto store_band = [&](int buf) {
#pragma unroll
    for (int u = 0; u < BAND_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      if (id < BAND_VEC) band[buf][swz(id >> 3, id & 7)] = band_reg[u];
    }
  };
  auto store_w = [&](const uint4 (&w_reg)[kConvTPS][W_ITERS], int buf) {
#pragma unroll
    for (int i = 0; i < kConvTPS; ++i)
#pragma unroll
      for (int u = 0; u < W_ITERS; ++u) {
        const int id = tid + u * kConvThreads;
        wts[buf][i][swz(id >> 3, id & 7)] = w_reg[i][u];
      }
  };

  f32x4 acc[kConvCG][TG];
#pragma unroll
  for (int i = 0; i < kConvCG; ++i)
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kg = lane >> 4;     // 0..3: which 8-element k group of the 32-wide MFMA step
  const int pl = lane & 15;     // pixel (B) / channel (A) row within a 16-group
  // A fragment rows m = wn*CW + 16 i + pl share (m & 7) = (pl & 7): one swizzled
  // slot per k step, fragment i at a fixed +16 rows.
  const int a_row0 = wn * kConvCW + pl;
  const int a_slot[2] = {(0 + kg) ^ (pl & 7), (4 + kg) ^ (pl & 7)};
  // One step = kConvTPS consecutive (slice, tap) pairs f: MFMAs on the
  // staged weights of the step and the band of each f's slice; then stage
  // the weights of step+1 (held in wnext) and, once per slice (at its tap
  // 6, at least a step before the slice's end), the next slice's band into
  // the other band buffer, which the previous slice last used before an
  // earlier barrier; barrier; then fetch the weights of step+3 into wnext
  // (two steps of latency cover).
  auto do_step = [&](int step, uint4 (&wnext)[kConvTPS][W_ITERS]) {
    const int wb = step & 1;
    int next_band = -1;  // slice whose band is stored at this step's end
#pragma unroll
    for (int sub = 0; sub < kConvTPS; ++sub) {
      const int f = step * kConvTPS + sub;
      if (f < nflat) {
        const int slice = f / 9, tap = f - slice * 9;
        const int bb = slice & 1;
        if (tap == 0 && slice + 1 < nslices) load_band((slice + 1) * kConvKC);
        if (tap == 6 && slice + 1 < nslices) next_band = slice + 1;
        const int dy = tap / 3, dx = tap - dy * 3;
        // B fragment rows bp = (wr + dy) * BW + dx + 16 j + pl: all fragments
        // of a tap share (bp & 7), so one swizzled slot per k step serves all j
        const int bp0 = (wr + dy) * BW + dx + pl;
        const int b_x = bp0 & 7;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 af[kConvCG], bfr[TG];
          const int bslot = (ks * 4 + kg) ^ b_x;
#pragma unroll
          for (int i = 0; i < kConvCG; ++i)
            af[i] = __builtin_bit_cast(bf16x8, wts[wb][sub][(a_row0 + 16 * i) * 8 + a_slot[ks]]);
#pragma unroll
          for (int j = 0; j < TG; ++j) bfr[j] = __builtin_bit_cast(bf16x8, band[bb][(bp0 + 16 * j) * 8 + bslot]);
#pragma unroll
          for (int i = 0; i < kConvCG; ++i)
#pragma unroll
            for (int j = 0; j < TG; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (step + 1 < nsteps) store_w(wnext, wb ^ 1);
    if (next_band >= 0) store_band(next_band & 1);
    __syncthreads();
    if (step + 3 < nsteps) load_w(wnext, step + 3);
  };

  // prologue: step 0 staged; steps 1 and 2 in registers
  load_band(0);
  load_w(w_regB, 0);
  store_band(0);
  store_w(w_regB, 0);
  if (nsteps > 1) load_w(w_regA, 1);
  if (nsteps > 2) load_w(w_regB, 2);
  __syncthreads();
  for (int step = 0; step < nsteps; step += 2) {
    do_step(step, w_regA);
    if (step + 1 < nsteps) do_step(step + 1, w_regB);
  }

  // -------- epilogue: lane holds channels m0 + wn*CW + i*16 + 4*(lane/16) + 0..3 of one pixel
  const int r = pr0 + wr;
  if (r >= a.rows) return;
#pragma unroll
  for (int j = 0; j < TG; ++j) {
    const int col = pc0 + j * 16 + pl;
    if (col >= W) continue;
    uint16_t* yp = a.y + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * a.Cout;
#pragma unroll
    for (int i = 0; i < kConvCG; ++i) {
      const int m = m0 + wn * kConvCW + i * 16 + 4 * kg;
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

// Column-tile choice: the TG (1..5 groups of 16 columns) whose tiles waste the
// fewest columns; ties go to the larger tile.
static int conv_pick_tg(int64_t W) {
  int best = 1;
  int64_t best_waste = -1;
  for (int tg = 1; tg <= 5; ++tg) {
    const int64_t tc = 16 * tg;
    const int64_t waste = ceil_div(W, tc) * tc - W;
    if (best_waste < 0 || waste < best_waste || (waste == best_waste && tg > best)) {
      best = tg;
      best_waste = waste;
    }
  }
  return best;
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
  const int tg = conv_pick_tg(W);
  a.tiles_c = static_cast<int>(ceil_div(W, 16 * tg));
  const int64_t tiles = ceil_div(rows, kConvTR) * a.tiles_c;
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(ceil_div(Cout, kConvBM)), static_cast<unsigned>(B));
  switch (tg) {
    case 1: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<1>, grid, dim3(kConvThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<2>, grid, dim3(kConvThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<3>, grid, dim3(kConvThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<4>, grid, dim3(kConvThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<5>, grid, dim3(kConvThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace dpp
