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
// LDS and reused by all nine taps; one barrier step covers the three taps of
// one kernel row, whose weights are double-buffered in LDS and fetched two
// steps ahead into registers.  Eight waves (two per SIMD) each compute 32 channels x 16*TG
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
//
// K loop: step = (64-channel slice, kernel row dy), three taps (dx = 0..2)
// each, one barrier per step.  The weights of a step (3 x 128 x 64) are
// double-buffered in LDS and fetched into registers two steps ahead.  The
// (2+2) x (16 TG + 2) halo band of a slice has one LDS buffer: step dy reads
// band rows dy and dy+1 only, so rows 0-1 of the next slice's band are
// written during its dy = 2 step (they were last read at dy = 1) and rows 2-3
// during the next slice's dy = 0 step; each half is fetched into registers
// two steps before it is written.  Every global load is unconditional (weight
// rows past Cout read zero through the buffer resource's range check; band
// vectors in the zero padding load a valid address and are zeroed when
// staged), and a pair of slices is one straight-line loop body, so each wait
// before a staging store covers only the loads it needs.
constexpr int kConvWN = 4;                      // waves across the 128 output channels
constexpr int kConvCW = 128 / kConvWN;          // output channels per wave
constexpr int kConvCG = kConvCW / 16;           // 16-channel MFMA groups per wave
constexpr int kConvThreads = 2 * kConvWN * 64;  // 2 tile rows x kConvWN
constexpr int kConvBM = 128;  // output channels per workgroup
constexpr int kConvKC = 64;   // input channels per slice (8 x 16-byte vectors)
constexpr int kConvTR = 2;    // patch rows per workgroup
constexpr int kConvBufWord3 = 0x00020000;  // raw 32-bit buffer access, no swizzle

struct ConvArgs {
  const uint16_t* x;
  const uint16_t* stale;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  float* part;  // split-K: float32 partial outputs [nsplit][B][rows][W][Cout], else NULL
  int H, W, Cin, Cout, row0, rows;
  int tiles_c;  // column tiles per row pair
  int nsplit;   // input-channel splits (blockIdx.z = b * nsplit + split)
  int spl;      // 64-channel slices per split
};

// LDS row of 8 x 16-byte slots, slot index XOR-swizzled by the row index so
// that 16 lanes reading the same logical slot of consecutive rows spread over
// the banks.
__device__ __forceinline__ int swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

template <int TG>
__global__ __launch_bounds__(kConvThreads, 1) void conv3x3_bf16_mfma_kernel(ConvArgs a) {
  constexpr int TC = 16 * TG;              // output columns per tile
  constexpr int BW = TC + 2;               // band columns
  constexpr int HALF_VEC = 2 * BW * 8;     // 16-byte vectors in two band rows
  constexpr int HB_ITERS = (HALF_VEC + kConvThreads - 1) / kConvThreads;
  constexpr int W_ITERS = kConvBM * 8 / kConvThreads;

  // band: 4 rows x BW pixels x 8 slots, plus one dummy slot that absorbs the
  // stores of the threads past the last vector of a half
  __shared__ uint4 band[2 * HALF_VEC + 1];
  __shared__ uint4 wts[2][3][kConvBM * 8];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wr = wave / kConvWN, wn = wave % kConvWN;
  const int b = blockIdx.z / a.nsplit, split = blockIdx.z % a.nsplit;
  const int m0 = blockIdx.y * kConvBM;
  const int tile_r = blockIdx.x / a.tiles_c, tile_c = blockIdx.x % a.tiles_c;
  const int pr0 = tile_r * kConvTR, pc0 = tile_c * TC;  // patch-relative origin of the pixel tile
  const int H = a.H, W = a.W, Cin = a.Cin;
  // this workgroup's input-channel slices: [s0, s0 + nslices)
  const int s0 = split * a.spl;
  const int nslices = min(a.spl, Cin / kConvKC - s0);
  const int nsteps = nslices * 3;

  // Band staging map, fixed for the kernel: vector u of half hf (rows 2hf,
  // 2hf+1) -> source address of the first slice (x for patch rows, the stale
  // image for halo rows; zero padding loads x and is masked) and LDS slot.
  const uint16_t* band_src[2][HB_ITERS];
  int band_dst[2][HB_ITERS];
  uint32_t band_ok = 0;  // bit hf*HB_ITERS+u: the vector is inside the image
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int u = 0; u < HB_ITERS; ++u) {
      const int id = tid + u * kConvThreads;
      const int pix = hf * 2 * BW + (id >> 3), slot = id & 7;
      const int br = pix / BW, bc = pix % BW;
      const int r = pr0 - 1 + br;  // patch-relative
      const int ir = a.row0 + r;   // image row
      const int col = pc0 - 1 + bc;
      band_src[hf][u] = a.x + slot * 8;
      band_dst[hf][u] = 2 * HALF_VEC;
      if (id < HALF_VEC) {
        band_dst[hf][u] = swz(pix, slot);
        if (ir >= 0 && ir < H && col >= 0 && col < W) {
          band_src[hf][u] = ((r >= 0 && r < a.rows) ? a.x + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * Cin
                                                    : a.stale + ((static_cast<int64_t>(b) * H + ir) * W + col) * Cin) +
                            slot * 8;
          band_ok |= 1u << (hf * HB_ITERS + u);
        }
      }
    }
  // Weight staging map: vector u -> byte offset of row m0 + m, slot, at tap 0
  // of slice 0; rows past Cout lie beyond the resource and read zero.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w), 0, a.Cout * 9 * Cin * 2, kConvBufWord3);
  int w_off[W_ITERS];
#pragma unroll
  for (int u = 0; u < W_ITERS; ++u) {
    const int id = tid + u * kConvThreads;
    w_off[u] = ((m0 + (id >> 3)) * 9 * Cin + (id & 7) * 8) * 2;
  }

  uint4 band_lo[HB_ITERS], band_hi[HB_ITERS];
  uint4 w_regA[3][W_ITERS], w_regB[3][W_ITERS];  // weights of the next two steps
  // Loads never touch their results until the staging store.
  auto load_half = [&](uint4 (&reg)[HB_ITERS], int hf, int slice) {
    const int c0 = (s0 + min(slice, nslices - 1)) * kConvKC;
#pragma unroll
    for (int u = 0; u < HB_ITERS; ++u) reg[u] = *reinterpret_cast<const uint4*>(band_src[hf][u] + c0);
  };
  auto store_half = [&](uint4 (&reg)[HB_ITERS], int hf) {
#pragma unroll
    for (int u = 0; u < HB_ITERS; ++u) {
      const uint32_t keep = 0u - ((band_ok >> (hf * HB_ITERS + u)) & 1u);
      // pins the mask here: hoisted next to the load, it would make the
      // wave wait for the load there
      asm volatile("" : "+v"(reg[u].x), "+v"(reg[u].y), "+v"(reg[u].z), "+v"(reg[u].w));
      band[band_dst[hf][u]] = make_uint4(reg[u].x & keep, reg[u].y & keep, reg[u].z & keep, reg[u].w & keep);
    }
  };
  auto load_w = [&](uint4 (&reg)[3][W_ITERS], int step) {
    const int st = min(step, nsteps - 1);
    const int sl = st / 3, dy = st - sl * 3;  // local slice, kernel row
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
      const int soff = ((dy * 3 + dx) * Cin + (s0 + sl) * kConvKC) * 2;
#pragma unroll
      for (int u = 0; u < W_ITERS; ++u)
        reg[dx][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[u] + soff, 0, 0));
    }
  };
  auto store_w = [&](const uint4 (&reg)[3][W_ITERS], int buf) {
#pragma unroll
    for (int dx = 0; dx < 3; ++dx)
#pragma unroll
      for (int u = 0; u < W_ITERS; ++u) {
        const int id = tid + u * kConvThreads;
        wts[buf][dx][swz(id >> 3, id & 7)] = reg[dx][u];
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

  // The three taps of kernel row dy on the staged weights of buffer wb.
  auto compute = [&](int dy, int wb) {
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
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
          af[i] = __builtin_bit_cast(bf16x8, wts[wb][dx][(a_row0 + 16 * i) * 8 + a_slot[ks]]);
#pragma unroll
        for (int j = 0; j < TG; ++j) bfr[j] = __builtin_bit_cast(bf16x8, band[(bp0 + 16 * j) * 8 + bslot]);
#pragma unroll
        for (int i = 0; i < kConvCG; ++i)
#pragma unroll
          for (int j = 0; j < TG; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  // Step st = 3 slice + dy (st & 1 == P): compute on weight buffer P, stage
  // the weights of st+1 (held in wnext) into the other buffer, barrier, fetch
  // the weights of st+3 into wnext.  Around it, the band halves of the next
  // slice: loads at dy = 0 (rows 0-1) and dy = 1 (rows 2-3); rows 0-1 are
  // staged at dy = 2, rows 2-3 at the next slice's dy = 0.
  auto slice_steps = [&](int slice, uint4 (&w0)[3][W_ITERS], uint4 (&w1)[3][W_ITERS], int p) {
    const int st = slice * 3;
    // dy = 0
    store_half(band_hi, 1);
    load_half(band_lo, 0, slice + 1);
    compute(0, p);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 3);
    // dy = 1
    load_half(band_hi, 1, slice + 1);
    compute(1, p ^ 1);
    store_w(w1, p);
    __syncthreads();
    load_w(w1, st + 4);
    // dy = 2
    compute(2, p);
    store_half(band_lo, 0);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 5);
  };

  // prologue: band rows 0-1 and the weights of step 0 staged; rows 2-3 in
  // registers (staged at the first step); steps 1 and 2 in registers
  load_half(band_lo, 0, 0);
  load_half(band_hi, 1, 0);
  load_w(w_regB, 0);
  store_half(band_lo, 0);
  store_w(w_regB, 0);
  load_w(w_regA, 1);
  load_w(w_regB, 2);
  __syncthreads();
  // slice pairs: the first slice of a pair starts at an even step (weights
  // of its steps st+1, st+3 in A; st+2 in B), the second at an odd one
  int slice = 0;
  for (; slice + 1 < nslices; slice += 2) {
    slice_steps(slice, w_regA, w_regB, 0);
    slice_steps(slice + 1, w_regB, w_regA, 1);
  }
  if (slice < nslices) slice_steps(slice, w_regA, w_regB, 0);

  // -------- epilogue: lane holds channels m0 + wn*CW + i*16 + 4*(lane/16) + 0..3 of one pixel
  const int r = pr0 + wr;
  if (a.part != nullptr) {  // split-K: float32 partials, bias added by the reduction
    if (r < a.rows) {
      const int64_t nb = gridDim.z / a.nsplit;
#pragma unroll
      for (int j = 0; j < TG; ++j) {
        const int col = pc0 + j * 16 + pl;
        if (col >= W) continue;
        float* pp = a.part + (((static_cast<int64_t>(split) * nb + b) * a.rows + r) * W + col) * a.Cout;
#pragma unroll
        for (int i = 0; i < kConvCG; ++i) {
          const int m = m0 + wn * kConvCW + i * 16 + 4 * kg;
          if (m < a.Cout) *reinterpret_cast<f32x4*>(pp + m) = acc[i][j];
        }
      }
    }
    return;  // uniform over the workgroup: no barrier follows
  }
  // bf16 output: bias added and rounded in registers, the tile (2 rows x TC
  // pixels x 128 channels) staged in LDS ([pixel][channel]; pixels padded by
  // 16 bytes, a stride of 4 banks mod 64, so the 16 pixels of a tile write
  // fall on distinct banks), then stored so that each wave store
  // writes the 256 contiguous bytes of two whole pixels instead of 32-byte
  // pieces of 16 pixels.  The slice loop ended with a barrier, so the weight
  // buffers are free.
  constexpr int kPixU2 = kConvBM / 4 + 2;  // uint2 per padded LDS pixel
  uint2* const tile = reinterpret_cast<uint2*>(&wts[0][0][0]);
#pragma unroll
  for (int i = 0; i < kConvCG; ++i) {
    const int c = wn * kConvCW + i * 16 + 4 * kg;
    const int m = m0 + c;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.bias && m < a.Cout) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = a.bias[m + e];
    }
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      uint2 out;
      out.x = pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
      out.y = pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
      tile[(wr * TC + j * 16 + pl) * kPixU2 + c / 4] = out;
    }
  }
  __syncthreads();
  constexpr int kChunks = kConvTR * TC * (kConvBM / 4);  // 8-byte chunks of the tile
  static_assert(kChunks % kConvThreads == 0, "whole chunks per thread");
#pragma unroll
  for (int u = 0; u < kChunks / kConvThreads; ++u) {
    const int id = tid + u * kConvThreads;
    const int pix = id / (kConvBM / 4), q = id % (kConvBM / 4);
    const int row = pr0 + pix / TC, col = pc0 + pix % TC, m = m0 + 4 * q;
    if (row < a.rows && col < W && m < a.Cout)
      *reinterpret_cast<uint2*>(a.y + ((static_cast<int64_t>(b) * a.rows + row) * W + col) * a.Cout + m) =
          tile[pix * kPixU2 + q];
  }
}

// Split-K reduction: y = bf16(bias + sum over splits of the float32 partials),
// the splits added in order; thread per 4 output channels of one pixel.
__global__ __launch_bounds__(256) void conv_splitk_reduce_kernel(const float* __restrict__ part,
                                                                 uint16_t* __restrict__ y,
                                                                 const float* __restrict__ bias, int nsplit,
                                                                 int64_t npix, int Cout) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int cq = Cout / 4;
  if (idx >= npix * cq) return;
  const int64_t pix = idx / cq;
  const int m = static_cast<int>(idx % cq) * 4;
  f32x4 acc = bias ? f32x4{bias[m], bias[m + 1], bias[m + 2], bias[m + 3]} : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nsplit; ++sp) acc += *reinterpret_cast<const f32x4*>(part + (sp * npix + pix) * Cout + m);
  uint2 out;
  out.x = pack_bf16x2(acc[0], acc[1]);
  out.y = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(y + pix * Cout + m) = out;
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

struct ConvSplit {
  int nsplit, spl;
};

// Input-channel split for grids that would leave CUs idle.  Cost of a launch
// in slice-rounds: ceil(workgroups x splits / 256) rounds of spl 64-channel
// slices each, a slice-round being about 3.2 us on MI355X.  A split adds its
// float32 partials, written and read back by the reduction (counted at
// 5 TB/s, 16 MB per slice-round), and one slice-round for the reduction's
// launch.  Gains under 10% go to fewer splits.  The model picks the measured
// fastest split count at every shape of a forced-split sweep (B = 1-2,
// 8-240 rows, 64-240 px wide, 320 and 640 channels): 3840 px 8-patch band,
// 225 workgroups -> no split; 16-patch band, 120 -> 2 (60 -> 47 us); 1024 px
// 8-patch band, 20 -> 10 (54 -> 29 us); full images never split.
static ConvSplit conv_split(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout) {
  constexpr double kSliceRoundBytes = 16e6;
  const int tg = conv_pick_tg(W);
  const int64_t wgs = ceil_div(rows, kConvTR) * ceil_div(W, 16 * tg) * ceil_div(Cout, kConvBM) * B;
  const int64_t nsl = Cin / kConvKC;
  const double out_bytes = static_cast<double>(B) * rows * W * Cout * sizeof(float);
  ConvSplit best{1, static_cast<int>(nsl)};
  double best_cost = static_cast<double>(ceil_div(wgs, 256) * nsl);
  const double bar = 0.9 * best_cost;
  for (int64_t ns = 2; ns <= nsl; ++ns) {
    const int64_t spl = ceil_div(nsl, ns), nse = ceil_div(nsl, spl);
    if (B * nse > 65535) break;
    const double cost = static_cast<double>(ceil_div(wgs * nse, 256) * spl) + 1.0 +
                        2.0 * nse * out_bytes / kSliceRoundBytes;
    if (cost < bar && cost < best_cost) {
      best_cost = cost;
      best = ConvSplit{static_cast<int>(nse), static_cast<int>(spl)};
    }
  }
  return best;
}

size_t conv_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout) {
  const ConvSplit sp = conv_split(B, rows, W, Cin, Cout);
  if (sp.nsplit <= 1) return 0;
  return static_cast<size_t>(sp.nsplit) * B * rows * W * Cout * sizeof(float);
}

hipError_t launch_conv3x3(void* y, const void* x, const void* stale_full, const void* weight, const float* bias,
                          int64_t B, int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows,
                          void* ws, size_t ws_bytes, bool bf16, hipStream_t s) {
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
  ConvSplit sp = conv_split(B, rows, W, Cin, Cout);
  if (sp.nsplit > 1 && (ws == nullptr || ws_bytes < conv_workspace_bytes(B, rows, W, Cin, Cout)))
    sp = ConvSplit{1, static_cast<int>(Cin / kConvKC)};
  a.nsplit = sp.nsplit;
  a.spl = sp.spl;
  a.part = sp.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(ceil_div(Cout, kConvBM)),
            static_cast<unsigned>(B * sp.nsplit));
  switch (tg) {
    case 1: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<1>, grid, dim3(kConvThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<2>, grid, dim3(kConvThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<3>, grid, dim3(kConvThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<4>, grid, dim3(kConvThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(conv3x3_bf16_mfma_kernel<5>, grid, dim3(kConvThreads), 0, s, a); break;
  }
  if (sp.nsplit > 1) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t npix = B * rows * W;
    hipLaunchKernelGGL(conv_splitk_reduce_kernel, dim3(static_cast<unsigned>(ceil_div(npix * (Cout / 4), 256))),
                       dim3(256), 0, s, static_cast<const float*>(ws), static_cast<uint16_t*>(y), bias, sp.nsplit,
                       npix, static_cast<int>(Cout));
  }
  return hipGetLastError();
}

}  // namespace dpp
