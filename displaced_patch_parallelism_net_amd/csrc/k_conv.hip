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
// pixels, channel-contiguous in NHWC), K = 9 taps x Cin.  Two tile kernels
// share the K loop's structure and the epilogue.  The four-row kernel's
// workgroup owns 4 patch rows x 16*TG columns x 64 output channels (TG
// chosen per width so the tiles cover the rows exactly where possible: 240
// columns -> 3 tiles of 80), eight waves (two per SIMD) each computing 32
// channels x 16*TG pixels of one tile row.  The six-row kernel's workgroup
// owns 6 rows x 48 columns x 64 channels with twelve waves (three per SIMD);
// it covers the 30-row band of a 240 x 240 image in 8 patches exactly (250
// workgroups, one per CU).  For each 64-channel slice of Cin the halo band
// (halo rows from the stale image) is staged once in LDS and reused by all
// nine taps; one barrier step covers the three taps of one kernel row,
// whose weights are double-buffered in LDS and fetched two steps ahead into
// registers.  MFMA v_mfma_f32_16x16x32_bf16; the accumulator's lane layout
// gives each lane four consecutive output channels of one pixel.
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
// Workgroup tile: 4 patch rows x 16*TG columns of output pixels x 64 output
// channels; eight waves, wave (wr, wn) owns tile row wr and channels
// [32 wn, 32 wn + 32): TG x 2 accumulator tiles of 16 x 16.  The host picks
// TG (1..5) so that the tiles cover the row width with the least waste (e.g.
// 240 columns -> TG 5: three tiles per row).
//
// K loop: step = (64-channel slice, kernel row dy), three taps (dx = 0..2)
// each, one barrier per step.  The weights of a step (3 x 64 x 64) are
// double-buffered in LDS and fetched into registers two steps ahead.  The
// 6 x (16 TG + 2) halo band of a slice is staged once and read by all nine
// taps, from a ring of eight LDS rows: slice s's band row i sits in ring row
// (6s + i) mod 8, and step dy reads band rows dy .. dy+3.  The band goes in
// two-row pieces A, B, C (rows 0-1, 2-3, 4-5), each fetched into registers
// two steps before it is written: C(s) during slice s's dy = 0 step (into the
// ring rows of slice s-1's rows 2-3), A(s+1) during dy = 1 (ring rows slice s
// does not use), B(s+1) during dy = 2 (slice s's rows 0-1, last read at
// dy = 1).
//
// Staging loads carry no predicates: a weight row past Cout and a band
// vector outside the image lie beyond the range of their buffer resource,
// which returns zeros.  Each band row has one source (x for patch rows, the
// stale image for halo rows, nothing above or below the image), so the four
// waves that load a row use one resource based at that row's first pixel
// at the slice's channels; a lane's offsets are fixed for the kernel, and
// its LDS slot is the ring row's base plus a fixed column part.  A pair of
// slices is one straight-line loop body, so each wait before a staging store
// covers only the loads it needs.
constexpr int kConvTR = 4;                  // patch rows per workgroup
constexpr int kConvBM = 64;                 // output channels per workgroup
constexpr int kConvCW = 32;                 // output channels per wave
constexpr int kConvCG = kConvCW / 16;       // 16-channel MFMA groups per wave
constexpr int kConvWN = kConvBM / kConvCW;  // waves across the channels
constexpr int kConvThreads = 512;           // 8 waves: 4 rows x 2 channel halves
constexpr int kConvKC = 64;                 // input channels per slice (8 x 16-byte vectors)
constexpr int kConvRing = 8;                // band rows held in LDS
constexpr int kConvBufWord3 = 0x00020000;   // raw 32-bit buffer access, no swizzle

struct ConvArgs {
  const uint16_t* x;
  const uint16_t* stale;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  float* part;  // split-K: float32 partial outputs [nsplit][B][rows][W][Cout], else NULL
  int H, W, Cin, Cout, row0, rows;
  int tiles_c;  // column tiles per row band
  int nsplit;   // input-channel splits (blockIdx.z = b * nsplit + split)
  int spl;      // 64-channel slices per split
  float* gn_part;  // GroupNorm partial sums of y [B][conv_gn_chunks][G][2], or NULL (unsplit only)
  int G;
};

// LDS row of 8 x 16-byte slots, slot index XOR-swizzled by the row index so
// that 16 lanes reading the same logical slot of consecutive rows spread over
// the banks (weights: a row is an output channel; band: a row is a pixel,
// keyed by its column, which within one ring row is the same spread).
__device__ __forceinline__ int swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

// Epilogue of the bf16 conv kernels.  Lane (kg = lane / 16, pl = lane % 16)
// of the wave owning tile row `row` and channels [m0 + cw0, m0 + cw0 + 32)
// holds, in acc[i][j], channels m0 + cw0 + 16 i + 4 kg + 0..3 of pixel column
// pc0 + 16 j + pl.  Split-K: the float32 partials go straight to a.part (the
// bias is added by the reduction).  Otherwise the bias is added and the
// result rounded in registers, the TR x 16 TG pixel x 64 channel tile is
// staged in LDS at `tile` ([pixel][channel]; pixels padded by 16 bytes, so
// that the 16 pixels of a tile write fall on distinct banks), then stored so
// that each wave store writes whole 128-byte pixels instead of 32-byte pieces
// of 16 pixels; with a.gn_part the tile's GroupNorm partial sums follow as
// chunk `chunk` of `nchunk` per batch entry, the LDS past the staged tile
// being their scratch.
constexpr int kConvPixU2 = kConvBM / 4 + 2;  // uint2 per padded LDS pixel

template <int TR, int TG, int NT>
constexpr size_t conv_epilogue_bytes() {
  return static_cast<size_t>(TR * 16 * TG * kConvPixU2) * 8 + 4 * tile_group_sums_scratch_floats<NT, kConvBM>();
}

template <int TR, int TG, int NT>
__device__ __forceinline__ void conv_epilogue(const ConvArgs& a, const f32x4 (&acc)[kConvCG][TG], uint2* tile, int b,
                                              int split, int m0, int row, int pc0, int cw0, int pr0, int64_t chunk,
                                              int64_t nchunk) {
  constexpr int TC = 16 * TG;
  constexpr int kTileU2 = TR * TC * kConvPixU2;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int kg = lane >> 4, pl = lane & 15;
  const int W = a.W;
  if (a.part != nullptr) {  // split-K: float32 partials, bias added by the reduction
    if (row < a.rows) {
      const int64_t nb = gridDim.z / a.nsplit;
#pragma unroll
      for (int j = 0; j < TG; ++j) {
        const int col = pc0 + j * 16 + pl;
        if (col >= W) continue;
        float* pp = a.part + (((static_cast<int64_t>(split) * nb + b) * a.rows + row) * W + col) * a.Cout;
#pragma unroll
        for (int i = 0; i < kConvCG; ++i) {
          const int m = m0 + cw0 + i * 16 + 4 * kg;
          if (m < a.Cout) *reinterpret_cast<f32x4*>(pp + m) = acc[i][j];
        }
      }
    }
    return;  // uniform over the workgroup: no barrier follows
  }
  const int trow = row - pr0;  // tile row
#pragma unroll
  for (int i = 0; i < kConvCG; ++i) {
    const int c = cw0 + i * 16 + 4 * kg;
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
      tile[(trow * TC + j * 16 + pl) * kConvPixU2 + c / 4] = out;
    }
  }
  __syncthreads();
  constexpr int kChunks = TR * TC * (kConvBM / 4);  // 8-byte chunks of the tile
  static_assert(kChunks % NT == 0, "whole chunks per thread");
#pragma unroll
  for (int u = 0; u < kChunks / NT; ++u) {
    const int id = tid + u * NT;
    const int pix = id / (kConvBM / 4), q = id % (kConvBM / 4);
    const int r = pr0 + pix / TC, col = pc0 + pix % TC, m = m0 + 4 * q;
    if (r < a.rows && col < W && m < a.Cout)
      *reinterpret_cast<uint2*>(a.y + ((static_cast<int64_t>(b) * a.rows + r) * W + col) * a.Cout + m) =
          tile[pix * kConvPixU2 + q];
  }
  if (a.gn_part != nullptr) {
    // GroupNorm partial sums of this tile's stored values, one chunk per
    // tile (chunk = channel tile * pixel tiles + pixel tile)
    float* out = a.gn_part + (static_cast<int64_t>(b) * nchunk + chunk) * a.G * 2;
    tile_group_sums<NT, TR * TC, kConvBM>(
        reinterpret_cast<const uint16_t*>(tile), 4 * kConvPixU2,
        [&](int p) { return pr0 + p / TC < a.rows && pc0 + p % TC < W; }, m0, a.Cout, a.Cout / a.G, a.G,
        reinterpret_cast<float*>(tile + kTileU2), out);
  }
}

template <int TG>
__global__ __launch_bounds__(kConvThreads, 1) void conv3x3_bf16_mfma_kernel(ConvArgs a) {
  constexpr int TC = 16 * TG;                   // output columns per tile
  constexpr int BW = TC + 2;                    // band columns
  constexpr int ROW_VEC = BW * 8;               // 16-byte vectors in one band row
  constexpr int RB_ITERS = (ROW_VEC + 255) / 256;  // per lane, four waves per row
  constexpr int W_ITERS = kConvBM * 8 / kConvThreads;
  constexpr int BAND_VEC = kConvRing * ROW_VEC;

  __shared__ uint4 band[BAND_VEC];
  __shared__ uint4 wts[2][3][kConvBM * 8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
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

  // Band staging map.  Waves 0-3 load the first row of a piece, waves 4-7
  // the second; lane vector u -> band column bc, slot: byte offset from the
  // row's first pixel (beyond the resource for columns outside the image and
  // for lanes past the row) and the column part of its LDS slot.
  const int prow = wave >> 2;  // row within a piece
  int b_off[RB_ITERS], b_col[RB_ITERS];
#pragma unroll
  for (int u = 0; u < RB_ITERS; ++u) {
    const int id = (wave & 3) * kWave + lane + u * 256;
    const int bc = id >> 3, slot = id & 7;
    const int col = pc0 - 1 + bc;
    b_off[u] = (id < ROW_VEC && col >= 0 && col < W) ? (col * Cin + slot * 8) * 2 : 0x7ffffff0;
    b_col[u] = id < ROW_VEC ? bc * 8 + (slot ^ (bc & 7)) : -1;
  }
  // source row of this wave's row of piece pc (band row 2 pc + prow), or NULL
  // above and below the image
  auto band_row_src = [&](int pc) -> const uint16_t* {
    const int r = pr0 - 1 + 2 * pc + prow;  // patch-relative
    const int ir = a.row0 + r;              // image row
    if (ir < 0 || ir >= H) return nullptr;
    return (r >= 0 && r < a.rows) ? a.x + (static_cast<int64_t>(b) * a.rows + r) * W * Cin
                                  : a.stale + (static_cast<int64_t>(b) * H + ir) * W * Cin;
  };
  const uint16_t* const row_src[3] = {band_row_src(0), band_row_src(1), band_row_src(2)};
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

  uint4 band_ra[RB_ITERS], band_rb[RB_ITERS];  // two band pieces in flight
  uint4 w_regA[3][W_ITERS], w_regB[3][W_ITERS];  // weights of the next two steps
  // Loads never touch their results until the staging store.
  auto load_piece = [&](uint4 (&reg)[RB_ITERS], int pc, int slice) {
    const int c0 = (s0 + min(slice, nslices - 1)) * kConvKC;
    const uint16_t* src = row_src[pc];
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src ? src + c0 : a.x), 0, src ? (W * Cin - c0) * 2 : 0, kConvBufWord3);
#pragma unroll
    for (int u = 0; u < RB_ITERS; ++u)
      reg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[u], 0, 0));
  };
  // piece pc into ring rows (base + 2 pc + prow) mod 8
  auto store_piece = [&](const uint4 (&reg)[RB_ITERS], int pc, int base) {
    const int row_base = ((base + 2 * pc + prow) & (kConvRing - 1)) * ROW_VEC;
#pragma unroll
    for (int u = 0; u < RB_ITERS; ++u)
      if (u + 1 < RB_ITERS || b_col[u] >= 0) band[row_base + b_col[u]] = reg[u];
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

  // The three taps of kernel row dy on the staged weights of buffer wb: six
  // batches n = (dx, 32-wide k step ks), each two A and TG B fragments and
  // 2 TG MFMAs.  The fragments of batch n+1 are read from LDS before the
  // MFMAs of batch n issue; the scheduling groups keep the compiler from
  // sinking those reads next to their use.
  auto frag_load = [&](int dy, int wb, int base, int n, bf16x8 (&af)[kConvCG], bf16x8 (&bfr)[TG]) {
    const int dx = n >> 1, ks = n & 1;
    // B fragment j: band column dx + 16 j + pl of ring row (base + wr + dy)
    // mod 8; the columns of a tap share (column & 7), so one swizzled slot per
    // k step serves all j
    const int brow = (base + wr + dy) & (kConvRing - 1);
    const int col0 = dx + pl;
    const int bslot = (ks * 4 + kg) ^ (col0 & 7);
#pragma unroll
    for (int i = 0; i < kConvCG; ++i)
      af[i] = __builtin_bit_cast(bf16x8, wts[wb][dx][(a_row0 + 16 * i) * 8 + a_slot[ks]]);
#pragma unroll
    for (int j = 0; j < TG; ++j)
      bfr[j] = __builtin_bit_cast(bf16x8, band[brow * ROW_VEC + (col0 + 16 * j) * 8 + bslot]);
  };
  auto mfma_batch = [&](const bf16x8 (&af)[kConvCG], const bf16x8 (&bfr)[TG]) {
#pragma unroll
    for (int i = 0; i < kConvCG; ++i)
#pragma unroll
      for (int j = 0; j < TG; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  constexpr int kSgDsRead = 0x100, kSgMfma = 0x008;  // sched_group_barrier masks
  auto compute = [&](int dy, int wb, int base) {
    bf16x8 a0[kConvCG], b0[TG], a1[kConvCG], b1[TG];
    frag_load(dy, wb, base, 0, a0, b0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
#pragma unroll
    for (int n = 0; n < 6; n += 2) {
      frag_load(dy, wb, base, n + 1, a1, b1);
      mfma_batch(a0, b0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, kConvCG * TG, 0);
      if (n + 2 < 6) frag_load(dy, wb, base, n + 2, a0, b0);
      mfma_batch(a1, b1);
      if (n + 2 < 6) __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, kConvCG * TG, 0);
    }
  };
  // Step st = 3 slice + dy (st & 1 == p): compute on weight buffer p, stage
  // the weights of st+1 (held in wnext) into the other buffer, barrier, fetch
  // the weights of st+3 into wnext.  Before it, the band pieces (e and o hold
  // the pieces fetched at even and odd steps): dy = 0 stages C(s) and
  // fetches B(s+1), dy = 1 stages A(s+1) and fetches C(s+1), dy = 2 stages
  // B(s+1) and fetches A(s+2).
  auto slice_steps = [&](int slice, uint4 (&w0)[3][W_ITERS], uint4 (&w1)[3][W_ITERS], int p,
                         uint4 (&e)[RB_ITERS], uint4 (&o)[RB_ITERS]) {
    const int st = slice * 3;
    const int base = (6 * slice) & (kConvRing - 1), nbase = (base + 6) & (kConvRing - 1);
    // dy = 0
    store_piece(e, 2, base);
    load_piece(e, 1, slice + 1);
    compute(0, p, base);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 3);
    // dy = 1
    store_piece(o, 0, nbase);
    load_piece(o, 2, slice + 1);
    compute(1, p ^ 1, base);
    store_w(w1, p);
    __syncthreads();
    load_w(w1, st + 4);
    // dy = 2
    store_piece(e, 1, nbase);
    load_piece(e, 0, slice + 2);
    compute(2, p, base);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 5);
  };

  // prologue: band rows 0-3 of slice 0 and the weights of step 0 staged;
  // C(0), A(1) and the weights of steps 1 and 2 in registers
  load_piece(band_ra, 0, 0);
  load_piece(band_rb, 1, 0);
  load_w(w_regB, 0);
  store_piece(band_ra, 0, 0);
  store_piece(band_rb, 1, 0);
  store_w(w_regB, 0);
  load_piece(band_ra, 2, 0);  // C(0), staged at step 0
  load_piece(band_rb, 0, 1);  // A(1), staged at step 1
  load_w(w_regA, 1);
  load_w(w_regB, 2);
  __syncthreads();
  // slice pairs: the first slice of a pair starts at an even step (weights
  // of its steps st+1, st+3 in A; st+2 in B), the second at an odd one
  int slice = 0;
  for (; slice + 1 < nslices; slice += 2) {
    slice_steps(slice, w_regA, w_regB, 0, band_ra, band_rb);
    slice_steps(slice + 1, w_regB, w_regA, 1, band_rb, band_ra);
  }
  if (slice < nslices) slice_steps(slice, w_regA, w_regB, 0, band_ra, band_rb);

  // -------- epilogue (the slice loop ended with a barrier: the band and
  // weight buffers are free; the staged tile and the statistics scratch go
  // into the larger of the two)
  constexpr bool kTileInBand = sizeof(band) >= sizeof(wts);
  static_assert(conv_epilogue_bytes<kConvTR, TG, kConvThreads>() <= (kTileInBand ? sizeof(band) : sizeof(wts)),
                "staged tile and statistics scratch fit");
  uint2* const tile = kTileInBand ? reinterpret_cast<uint2*>(&band[0]) : reinterpret_cast<uint2*>(&wts[0][0][0]);
  conv_epilogue<kConvTR, TG, kConvThreads>(a, acc, tile, b, split, m0, pr0 + wr, pc0, wn * kConvCW, pr0,
                                           static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x,
                                           static_cast<int64_t>(gridDim.x) * gridDim.y);
}

// Six-row tile: 6 patch rows x 16*TG columns x 64 output channels, twelve
// waves (three per SIMD), wave (wr, wn) owning tile row wr and channels
// [32 wn, 32 wn + 32): TG x 2 accumulator tiles.  Chosen where it covers the
// band exactly (rows a multiple of 6, width a multiple of 48, TG = 3): the
// 30-row x 240-column band is 5 x 5 x 10 = 250 workgroups of 288 pixels
// instead of 240 of 320 (the last four-row tile half empty), and three waves
// per SIMD hide more of the LDS and barrier latency than two.
//
// Same K loop as the four-row kernel (one barrier step per 64-channel slice
// and kernel row; weights double-buffered in LDS, fetched two steps ahead),
// but the slice's halo band is 8 rows: the band is double-buffered (two
// halves of 8 LDS rows, slice s in half s & 1), and slice s+1's band is
// staged during slice s in three pieces -- rows 0-2, 3-5 and 6-7, one per
// step dy -- each fetched into registers two steps before it is stored.
// Waves 4k .. 4k+3 load and store row k of a piece; the last piece has two
// rows, so waves 8-11 skip it.
constexpr int kConv6TR = 6;
constexpr int kConv6Threads = 768;  // 12 waves: 6 rows x 2 channel halves
constexpr int kConv6Half = 8;       // band rows per slice

template <int TG>
__global__ __launch_bounds__(kConv6Threads, 1) void conv3x3_bf16_mfma6_kernel(ConvArgs a) {
  constexpr int TC = 16 * TG;                      // output columns per tile
  constexpr int BW = TC + 2;                       // band columns
  constexpr int ROW_VEC = BW * 8;                  // 16-byte vectors in one band row
  constexpr int RB_ITERS = (ROW_VEC + 255) / 256;  // per lane, four waves per row
  constexpr int W_VEC = 3 * kConvBM * 8;           // weight vectors of one step (3 taps)
  constexpr int W_ITERS = W_VEC / kConv6Threads;
  static_assert(W_VEC % kConv6Threads == 0, "whole weight vectors per thread");

  __shared__ uint4 band[2 * kConv6Half * ROW_VEC];
  __shared__ uint4 wts[2][3][kConvBM * 8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int wr = wave / kConvWN, wn = wave % kConvWN;
  // 1-D grid over (b, pixel tile, channel tile).  Workgroup ids are dealt
  // round-robin to the 8 XCDs; each XCD takes a contiguous range of tiles,
  // channel tile fastest, so the channel tiles of a pixel tile (which read
  // the same band rows) share an L2.
  const int nct = (a.Cout + kConvBM - 1) / kConvBM;
  const int npt = a.tiles_c * (a.rows / kConv6TR);
  const int ntot = gridDim.x, xcd = blockIdx.x % 8, per = ntot / 8, rem = ntot % 8;
  const int logical = xcd * per + min(xcd, rem) + static_cast<int>(blockIdx.x) / 8;
  const int b = logical / (npt * nct), split = 0;
  const int ptile = logical % (npt * nct) / nct, ctile = logical % nct;
  const int m0 = ctile * kConvBM;
  const int tile_r = ptile / a.tiles_c, tile_c = ptile % a.tiles_c;
  const int pr0 = tile_r * kConv6TR, pc0 = tile_c * TC;
  const int H = a.H, W = a.W, Cin = a.Cin;
  const int s0 = 0;
  const int nslices = min(a.spl, Cin / kConvKC - s0);
  const int nsteps = nslices * 3;

  // Band staging map (as in the four-row kernel): lane vector u -> byte
  // offset from its row's first pixel (beyond the resource outside the image
  // and past the row) and the column part of its LDS slot.
  const int prow = wave >> 2;  // row within a piece: 0..2
  int b_off[RB_ITERS], b_col[RB_ITERS];
#pragma unroll
  for (int u = 0; u < RB_ITERS; ++u) {
    const int id = (wave & 3) * kWave + lane + u * 256;
    const int bc = id >> 3, slot = id & 7;
    const int col = pc0 - 1 + bc;
    b_off[u] = (id < ROW_VEC && col >= 0 && col < W) ? (col * Cin + slot * 8) * 2 : 0x7ffffff0;
    b_col[u] = id < ROW_VEC ? bc * 8 + (slot ^ (bc & 7)) : -1;
  }
  // source of this wave's row of piece pc (band row 3 pc + prow), or NULL
  // above and below the image and for the missing third row of piece 2
  auto band_row_src = [&](int pc) -> const uint16_t* {
    const int br = 3 * pc + prow;
    if (br >= kConv6Half) return nullptr;
    const int r = pr0 - 1 + br;  // patch-relative
    const int ir = a.row0 + r;   // image row
    if (ir < 0 || ir >= H) return nullptr;
    return (r >= 0 && r < a.rows) ? a.x + (static_cast<int64_t>(b) * a.rows + r) * W * Cin
                                  : a.stale + (static_cast<int64_t>(b) * H + ir) * W * Cin;
  };
  const uint16_t* const row_src[3] = {band_row_src(0), band_row_src(1), band_row_src(2)};
  // Weight staging map: vector u -> tap dx, output-channel row m and slot of
  // the step's 3 x 64 x 64 block; rows past Cout read zero.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w), 0, a.Cout * 9 * Cin * 2, kConvBufWord3);
  int w_off[W_ITERS], w_dst[W_ITERS];
#pragma unroll
  for (int u = 0; u < W_ITERS; ++u) {
    const int id = tid + u * kConv6Threads;
    const int dx = id / (kConvBM * 8), r = id % (kConvBM * 8);
    w_off[u] = ((m0 + (r >> 3)) * 9 * Cin + dx * Cin + (r & 7) * 8) * 2;
    w_dst[u] = dx * (kConvBM * 8) + swz(r >> 3, r & 7);
  }

  uint4 band_ra[RB_ITERS], band_rb[RB_ITERS];
  uint4 w_regA[W_ITERS], w_regB[W_ITERS];
  auto load_piece = [&](uint4 (&reg)[RB_ITERS], int pc, int slice) {
    const int c0 = (s0 + min(slice, nslices - 1)) * kConvKC;
    const uint16_t* src = row_src[pc];
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src ? src + c0 : a.x), 0, src ? (W * Cin - c0) * 2 : 0, kConvBufWord3);
#pragma unroll
    for (int u = 0; u < RB_ITERS; ++u)
      reg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[u], 0, 0));
  };
  // piece pc of a slice into band half `half` (wave-uniform skip for the
  // missing row of piece 2)
  auto store_piece = [&](const uint4 (&reg)[RB_ITERS], int pc, int half) {
    if (3 * pc + prow >= kConv6Half) return;
    const int row_base = (half * kConv6Half + 3 * pc + prow) * ROW_VEC;
#pragma unroll
    for (int u = 0; u < RB_ITERS; ++u)
      if (u + 1 < RB_ITERS || b_col[u] >= 0) band[row_base + b_col[u]] = reg[u];
  };
  auto load_w = [&](uint4 (&reg)[W_ITERS], int step) {
    const int st = min(step, nsteps - 1);
    const int sl = st / 3, dy = st - sl * 3;
    const int soff = (dy * 3 * Cin + (s0 + sl) * kConvKC) * 2;
#pragma unroll
    for (int u = 0; u < W_ITERS; ++u)
      reg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[u] + soff, 0, 0));
  };
  auto store_w = [&](const uint4 (&reg)[W_ITERS], int buf) {
#pragma unroll
    for (int u = 0; u < W_ITERS; ++u) (&wts[buf][0][0])[w_dst[u]] = reg[u];
  };

  f32x4 acc[kConvCG][TG];
#pragma unroll
  for (int i = 0; i < kConvCG; ++i)
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kg = lane >> 4, pl = lane & 15;
  const int a_row0 = wn * kConvCW + pl;
  const int a_slot[2] = {(0 + kg) ^ (pl & 7), (4 + kg) ^ (pl & 7)};
  auto frag_load = [&](int dy, int wb, int half, int n, bf16x8 (&af)[kConvCG], bf16x8 (&bfr)[TG]) {
    const int dx = n >> 1, ks = n & 1;
    const int brow = half * kConv6Half + wr + dy;
    const int col0 = dx + pl;
    const int bslot = (ks * 4 + kg) ^ (col0 & 7);
#pragma unroll
    for (int i = 0; i < kConvCG; ++i)
      af[i] = __builtin_bit_cast(bf16x8, wts[wb][dx][(a_row0 + 16 * i) * 8 + a_slot[ks]]);
#pragma unroll
    for (int j = 0; j < TG; ++j)
      bfr[j] = __builtin_bit_cast(bf16x8, band[brow * ROW_VEC + (col0 + 16 * j) * 8 + bslot]);
  };
  auto mfma_batch = [&](const bf16x8 (&af)[kConvCG], const bf16x8 (&bfr)[TG]) {
#pragma unroll
    for (int i = 0; i < kConvCG; ++i)
#pragma unroll
      for (int j = 0; j < TG; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  constexpr int kSgDsRead = 0x100, kSgMfma = 0x008;  // sched_group_barrier masks
  auto compute = [&](int dy, int wb, int half) {
    bf16x8 a0[kConvCG], b0[TG], a1[kConvCG], b1[TG];
    frag_load(dy, wb, half, 0, a0, b0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
#pragma unroll
    for (int n = 0; n < 6; n += 2) {
      frag_load(dy, wb, half, n + 1, a1, b1);
      mfma_batch(a0, b0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, kConvCG * TG, 0);
      if (n + 2 < 6) frag_load(dy, wb, half, n + 2, a0, b0);
      mfma_batch(a1, b1);
      if (n + 2 < 6) __builtin_amdgcn_sched_group_barrier(kSgDsRead, kConvCG + TG, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, kConvCG * TG, 0);
    }
  };
  // Step st = 3 slice + dy: store piece dy of slice+1 (fetched two steps
  // earlier) into the other band half and fetch the piece stored two steps
  // later into the same registers (e at the slice's dy = 0 and 2, o at
  // dy = 1; the caller swaps e and o for odd slices), compute on weight
  // buffer st & 1 and band half slice & 1, stage the weights of st+1 into
  // the other weight buffer, barrier, fetch the weights of st+3.
  auto slice_steps = [&](int slice, uint4 (&w0)[W_ITERS], uint4 (&w1)[W_ITERS], int p, uint4 (&e)[RB_ITERS],
                         uint4 (&o)[RB_ITERS]) {
    const int st = slice * 3;
    const int half = slice & 1, nhalf = half ^ 1;
    // dy = 0: store piece 0 of slice+1, fetch piece 2 of slice+1
    store_piece(e, 0, nhalf);
    load_piece(e, 2, slice + 1);
    compute(0, p, half);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 3);
    // dy = 1: store piece 1 of slice+1, fetch piece 0 of slice+2
    store_piece(o, 1, nhalf);
    load_piece(o, 0, slice + 2);
    compute(1, p ^ 1, half);
    store_w(w1, p);
    __syncthreads();
    load_w(w1, st + 4);
    // dy = 2: store piece 2 of slice+1, fetch piece 1 of slice+2
    store_piece(e, 2, nhalf);
    load_piece(e, 1, slice + 2);
    compute(2, p, half);
    store_w(w0, p ^ 1);
    __syncthreads();
    load_w(w0, st + 5);
  };

  // prologue: slice 0's band in half 0 and the weights of step 0 staged;
  // pieces 0 and 1 of slice 1 and the weights of steps 1 and 2 in registers
  load_piece(band_ra, 0, 0);
  load_piece(band_rb, 1, 0);
  load_w(w_regB, 0);
  store_piece(band_ra, 0, 0);
  store_piece(band_rb, 1, 0);
  store_w(w_regB, 0);
  load_piece(band_ra, 2, 0);
  store_piece(band_ra, 2, 0);
  load_piece(band_ra, 0, 1);  // stored at step 0
  load_piece(band_rb, 1, 1);  // stored at step 1
  load_w(w_regA, 1);
  load_w(w_regB, 2);
  __syncthreads();
  int slice = 0;
  for (; slice + 1 < nslices; slice += 2) {
    slice_steps(slice, w_regA, w_regB, 0, band_ra, band_rb);
    slice_steps(slice + 1, w_regB, w_regA, 1, band_rb, band_ra);
  }
  if (slice < nslices) slice_steps(slice, w_regA, w_regB, 0, band_ra, band_rb);

  // -------- epilogue (the slice loop ended with a barrier)
  static_assert(conv_epilogue_bytes<kConv6TR, TG, kConv6Threads>() <= sizeof(band),
                "staged tile and statistics scratch fit in the band");
  conv_epilogue<kConv6TR, TG, kConv6Threads>(a, acc, reinterpret_cast<uint2*>(&band[0]), b, split, m0, pr0 + wr, pc0,
                                             wn * kConvCW, pr0, static_cast<int64_t>(ctile) * npt + ptile,
                                             static_cast<int64_t>(npt) * nct);
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

static int64_t conv_tiles(int64_t rows, int64_t W, int64_t Cout) {
  return ceil_div(rows, kConvTR) * ceil_div(W, 16 * conv_pick_tg(W)) * ceil_div(Cout, kConvBM);
}

struct ConvSplit {
  int nsplit, spl;
};

// Input-channel split for grids that would leave CUs idle.  Cost of a launch
// in slice-rounds: ceil(workgroups x splits / 256) rounds of spl 64-channel
// slices each, a slice-round being about 3.2 us on MI355X.  A split adds its
// float32 partials, written and read back by the reduction (counted at
// 5 TB/s, 16 MB per slice-round), and one slice-round for the reduction's
// launch.  Gains under 10% go to fewer splits.  In a forced-split sweep on
// MI355X (seven bands of 8-240 rows, 64-240 px wide, 320 and 640 channels)
// the model picks the measured fastest count at six shapes and one within 4 %:
// 240 x 240 image, 30-row band, 240 four-row workgroups -> no split; 15-row band, 120
// -> 2 (42 -> 35 us); 64 x 64 image, 8-row band, 20 -> 10 (36 -> 19 us;
// 5 splits: 18 us); full images never split.
static ConvSplit conv_split(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout) {
  constexpr double kSliceRoundBytes = 16e6;
  const int64_t wgs = conv_tiles(rows, W, Cout) * B;
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

// Six-row tiles (48 columns) where they cover the band exactly and take fewer
// pixel-rounds than the four-row tiles: ceil(workgroups / 256) rounds of the
// tile's pixels, the six-row tile's pixels counted at 0.9 for its third wave
// per SIMD (an LDS-fed MFMA probe with the conv's fragment ratios: 74 % of the
// matrix pipe busy against 67 %).  Depends on the shape of one batch entry
// only, so that the GroupNorm chunk count does too.  (The 30 x 240 band:
// 250 six-row tiles against 240 four-row ones, the last row of those half
// empty.)
static int64_t conv_tiles6(int64_t rows, int64_t W, int64_t Cout) {
  return rows / kConv6TR * (W / 48) * ceil_div(Cout, kConvBM);
}

static bool conv_six_rows(int64_t rows, int64_t W, int64_t Cout) {
  if (rows % kConv6TR != 0 || W % 48 != 0) return false;
  const double cost4 = static_cast<double>(ceil_div(conv_tiles(rows, W, Cout), 256) * kConvTR * 16 * conv_pick_tg(W));
  const double cost6 = 0.9 * static_cast<double>(ceil_div(conv_tiles6(rows, W, Cout), 256) * kConv6TR * 48);
  return cost6 < cost4;
}

int64_t conv_gn_chunks(int64_t rows, int64_t W, int64_t Cout) {
  return conv_six_rows(rows, W, Cout) ? conv_tiles6(rows, W, Cout) : conv_tiles(rows, W, Cout);
}

size_t conv_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout) {
  const ConvSplit sp = conv_split(B, rows, W, Cin, Cout);
  if (sp.nsplit <= 1) return 0;
  return static_cast<size_t>(sp.nsplit) * B * rows * W * Cout * sizeof(float);
}

hipError_t launch_conv3x3(void* y, const void* x, const void* stale_full, const void* weight, const float* bias,
                          int64_t B, int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows,
                          void* ws, size_t ws_bytes, bool bf16, hipStream_t s, float* gn_part, int G) {
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
  if (sp.nsplit > 1 && (gn_part != nullptr || ws == nullptr || ws_bytes < conv_workspace_bytes(B, rows, W, Cin, Cout)))
    sp = ConvSplit{1, static_cast<int>(Cin / kConvKC)};
  a.gn_part = gn_part;
  a.G = G;
  a.nsplit = sp.nsplit;
  a.spl = sp.spl;
  a.part = sp.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  if (sp.nsplit == 1 && conv_six_rows(rows, W, Cout)) {
    a.tiles_c = static_cast<int>(W / 48);
    hipLaunchKernelGGL(conv3x3_bf16_mfma6_kernel<3>, dim3(static_cast<unsigned>(B * conv_tiles6(rows, W, Cout))),
                       dim3(kConv6Threads), 0, s, a);
    return hipGetLastError();
  }
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
