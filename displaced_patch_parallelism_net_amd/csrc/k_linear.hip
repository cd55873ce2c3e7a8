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
// 64*CG channels x 160 tokens, eight waves of 16*CG channels x 80 tokens (CG x
// 5 accumulator tiles); with few token tiles, 80 tokens and four waves.  CG = 2 (128 channels) for 7200 tokens x 640 channels:
// 225 workgroups, one round on 256 CUs; CG = 4 (256 channels) for the fused
// K/V projection (1280 channels): again 225 workgroups instead of two rounds
// of 225, and each token row is loaded once.  K is walked in 64-wide slices staged in LDS (XOR-
// swizzled rows, double-buffered); for K = 320, 640, 1280 the slice loop is
// unrolled and the global loads run four slices ahead (their latency is long
// against one slice's MFMAs at these sizes); one barrier per slice.  Each lane's
// accumulator holds four consecutive channels of one token: one 8-byte store.
// Workgroups map to tiles in an XCD-aware order: each XCD takes a contiguous
// range of tiles, channel tile fastest, so the channel tiles of one token
// tile share an L2 (7200 x 640 x 640: 14.8 -> 12.4 us).
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

constexpr int kLinBM = 160;   // tokens per workgroup (kLinBMSmall for few token tiles)
constexpr int kLinBMSmall = 80;
constexpr int kLinKC = 64;    // K slice (8 x 16-byte vectors per row)
constexpr int kLinThreads = 512;  // 8 waves: 2 token halves x 4 channel groups (4 waves at kLinBMSmall)
constexpr int kLinTG = 5;     // 16-token MFMA groups per wave

struct LinArgs {
  const uint16_t* x;
  const uint16_t* w;
  const float* bias;
  uint16_t* y;
  int64_t M, K, N, ld_x, bs_x, ld_y, bs_y;
  float* gn_part;  // GroupNorm partial sums of y [B][gridDim.x * gridDim.y][G][2], or NULL
  int G;
};

// LDS row of 8 x 16-byte slots, slot XOR-swizzled by the row index.
__device__ __forceinline__ int lin_swz(int row, int slot) { return row * 8 + (slot ^ (row & 7)); }

constexpr int kLinBufWord3 = 0x00020000;  // raw 32-bit buffer access, no swizzle
constexpr int kLinAhead = 4;              // K slices in flight (fully unrolled instantiations, CG = 2)

// NSL > 0: the K loop has exactly NSL slices and is fully unrolled, with the
// global loads kLinAhead slices ahead in a ring of registers (every count is
// a constant, so each wait covers exactly the slice it needs).  NSL == 0:
// any K, loads one slice ahead.  Loads are raw buffer loads against
// resources that end at the last element of w and of x's batch entry: rows
// past N or M read as zero, so no load is predicated; the K tail (k >= K in
// the last slice) is zeroed by a select.
template <int NSL, int CG, int BM>
__global__ __launch_bounds__(BM / 80 * 256) void linear_bf16_mfma_kernel(LinArgs a) {
  constexpr int kLinBM = BM;                             // tokens per workgroup
  constexpr int kLinThreads = BM / 80 * 256;             // waves: BM / 80 token groups x 4 channel groups
  constexpr int kLinItersB = (kLinBM * 8 + kLinThreads - 1) / kLinThreads;  // token vectors per thread
  constexpr int kLinBN = 64 * CG;                        // output channels per workgroup
  constexpr int kLinCG = CG;                             // 16-channel MFMA groups per wave
  constexpr int kLinItersA = kLinBN * 8 / kLinThreads;   // weight vectors per thread
  // the wider tile holds twice the weight vectors per slice: one slice less in flight
  constexpr int kAhead = CG == 2 ? kLinAhead : kLinAhead - 1;
  constexpr int AHEAD = NSL > 0 ? (NSL < kAhead ? NSL : kAhead) : 1;
  // LDS: the two weight and two token slice buffers; after the K loop the
  // same memory holds the output tile for the coalesced store
  __shared__ uint4 smem[2 * kLinBN * 8 + 2 * kLinBM * 8];
  uint4* const As = smem;                     // [2][kLinBN * 8]
  uint4* const Bs = smem + 2 * kLinBN * 8;    // [2][kLinBM * 8]
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wn = wave % 4, wm = wave / 4;
  const int64_t b = blockIdx.z;
  // XCD-aware tile order: the hardware deals workgroup ids round-robin to the
  // 8 XCDs; give each XCD a contiguous range of logical tiles, channel tile
  // fastest, so the channel tiles of one token tile share an L2 and read
  // their token rows from beyond it once.
  const int total = gridDim.x * gridDim.y, lid = blockIdx.y * gridDim.x + blockIdx.x;
  const int per = total / 8, rem = total % 8, xcd = lid % 8;
  const int logical = xcd * per + min(xcd, rem) + lid / 8;
  const int mt = logical / gridDim.y, nt = logical % gridDim.y;
  const int64_t n0 = static_cast<int64_t>(nt) * kLinBN;
  const int64_t m0 = static_cast<int64_t>(mt) * kLinBM;
  const int nslices = NSL > 0 ? NSL : static_cast<int>((a.K + kLinKC - 1) / kLinKC);

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w), 0, static_cast<int>(a.N * a.K * 2), kLinBufWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x + b * a.bs_x), 0, static_cast<int>(((a.M - 1) * a.ld_x + a.K) * 2), kLinBufWord3);
  // staging map: vector id -> (row, 16-byte slot) of a slice (rows x 64);
  // byte offsets of the slice at k = 0
  const int slot8 = tid & 7;  // the same for every staged vector of a thread
  int a_off[kLinItersA], b_off[kLinItersB];
#pragma unroll
  for (int u = 0; u < kLinItersA; ++u) {
    const int row = (tid + u * kLinThreads) >> 3;
    a_off[u] = static_cast<int>(((n0 + row) * a.K + slot8 * 8) * 2);
  }
#pragma unroll
  for (int u = 0; u < kLinItersB; ++u) {
    const int row = (tid + u * kLinThreads) >> 3;
    b_off[u] = row < kLinBM ? static_cast<int>(((m0 + row) * a.ld_x + slot8 * 8) * 2) : 0x7ffffff0;
  }
  // Loaded values are not touched until they are staged (a select right
  // after a load would make the wave wait for it there).
  uint4 a_reg[AHEAD][kLinItersA], b_reg[AHEAD][kLinItersB];
  auto load = [&](int r, int s) {
    const int kb = s * kLinKC * 2;
#pragma unroll
    for (int u = 0; u < kLinItersA; ++u)
      a_reg[r][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, a_off[u] + kb, 0, 0));
#pragma unroll
    for (int u = 0; u < kLinItersB; ++u)
      b_reg[r][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, b_off[u] + kb, 0, 0));
  };
  // stage slice s from ring slot r; vectors past K (last slice only) are
  // masked to zero (a bit mask, not a branch, keeps the ring in registers)
  auto masked = [](const uint4& v, unsigned m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); };
  auto store = [&](int r, int s, int buf) {
    const unsigned m = (s * kLinKC + slot8 * 8 < a.K) ? 0xffffffffu : 0u;  // K % 8 == 0: whole vectors
#pragma unroll
    for (int u = 0; u < kLinItersA; ++u) {
      const int id = tid + u * kLinThreads;
      As[buf * kLinBN * 8 + lin_swz(id >> 3, id & 7)] = masked(a_reg[r][u], m);
    }
#pragma unroll
    for (int u = 0; u < kLinItersB; ++u) {
      const int id = tid + u * kLinThreads;
      if (id < kLinBM * 8) Bs[buf * kLinBM * 8 + lin_swz(id >> 3, id & 7)] = masked(b_reg[r][u], m);
    }
  };

  f32x4 acc[kLinCG][kLinTG];
#pragma unroll
  for (int i = 0; i < kLinCG; ++i)
#pragma unroll
    for (int j = 0; j < kLinTG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kg = lane >> 4, pl = lane & 15;
  // fragment rows r = base + 16 i + pl share (r & 7) = (pl & 7)
  const int a_row0 = wn * 16 * kLinCG + pl, b_row0 = wm * (16 * kLinTG) + pl;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int slot = (ks * 4 + kg) ^ (pl & 7);
      bf16x8 af[kLinCG], bfr[kLinTG];
#pragma unroll
      for (int i = 0; i < kLinCG; ++i) af[i] = __builtin_bit_cast(bf16x8, As[buf * kLinBN * 8 + (a_row0 + 16 * i) * 8 + slot]);
#pragma unroll
      for (int j = 0; j < kLinTG; ++j) bfr[j] = __builtin_bit_cast(bf16x8, Bs[buf * kLinBM * 8 + (b_row0 + 16 * j) * 8 + slot]);
#pragma unroll
      for (int i = 0; i < kLinCG; ++i)
#pragma unroll
        for (int j = 0; j < kLinTG; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  if constexpr (NSL > 0) {
    // prologue: slices 0 .. AHEAD-1 requested, slice 0 staged, slice AHEAD
    // requested into the freed ring slot
#pragma unroll
    for (int r = 0; r < AHEAD; ++r) load(r, r);
    store(0, 0, 0);
    if (AHEAD < NSL) load(0, AHEAD);
    __syncthreads();
    // slice s: MFMAs from buffer s & 1; slice s+1 (ring slot (s+1) % AHEAD)
    // into the other buffer, last read before the previous barrier; slice
    // s+1+AHEAD requested into the freed slot
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
      compute(s & 1);
      if (s + 1 < NSL) {
        store((s + 1) % AHEAD, s + 1, (s + 1) & 1);
        if (s + 1 + AHEAD < NSL) load((s + 1) % AHEAD, s + 1 + AHEAD);
      }
      __syncthreads();
    }
  } else {
    load(0, 0);
    store(0, 0, 0);
    if (nslices > 1) load(0, 1);
    __syncthreads();
    for (int s = 0; s < nslices; ++s) {
      compute(s & 1);
      if (s + 1 < nslices) store(0, s + 1, (s + 1) & 1);
      __syncthreads();
      if (s + 2 < nslices) load(0, s + 2);
    }
  }

  // epilogue: lane holds channels wn*16*CG + 16 i + 4 kg + 0..3 (of the tile)
  // of token wm*80 + 16 j + pl.  Bias added and rounded here, then the tile
  // goes through LDS ([token][channel]; rows padded by 16 bytes, a stride of
  // 4 banks mod 64, so the 16 tokens of a tile write fall on distinct banks)
  // so that every wave store writes whole rows: 64 lanes x 8 bytes
  // = 2 (CG = 2) or 1 (CG = 4) full tile rows, instead of 32-byte pieces of
  // 16 rows.  The K loop ended with a barrier: the slice buffers are free.
  constexpr int kRowU2 = kLinBN / 4 + 2;  // uint2 per padded LDS row
  uint2* const tile = reinterpret_cast<uint2*>(smem);
#pragma unroll
  for (int i = 0; i < kLinCG; ++i) {
    const int c = wn * 16 * kLinCG + 16 * i + 4 * kg;
    const int64_t n = n0 + c;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.bias && n < a.N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = a.bias[n + e];
    }
#pragma unroll
    for (int j = 0; j < kLinTG; ++j) {
      const int r = wm * (16 * kLinTG) + 16 * j + pl;
      uint2 out;
      out.x = pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
      out.y = pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
      tile[r * kRowU2 + c / 4] = out;
    }
  }
  __syncthreads();
  constexpr int kChunks = kLinBM * (kLinBN / 4);  // 8-byte chunks of the tile
  static_assert(kChunks % kLinThreads == 0, "whole chunks per thread");
#pragma unroll
  for (int u = 0; u < kChunks / kLinThreads; ++u) {
    const int id = tid + u * kLinThreads;
    const int r = id / (kLinBN / 4), q = id % (kLinBN / 4);
    const int64_t m = m0 + r, n = n0 + 4 * q;
    if (m < a.M && n < a.N)
      *reinterpret_cast<uint2*>(a.y + b * a.bs_y + m * a.ld_y + n) = tile[r * kRowU2 + q];
  }
  if (a.gn_part != nullptr) {
    // GroupNorm partial sums of this tile's stored values (tokens = pixels),
    // one chunk per workgroup; the LDS past the output tile is the scratch
    const int64_t nchunk = static_cast<int64_t>(gridDim.x) * gridDim.y;
    const int64_t chunk = static_cast<int64_t>(nt) * gridDim.x + mt;
    static_assert((kLinBM * kRowU2 * 8 + 4 * tile_group_sums_scratch_floats<kLinThreads, kLinBN>()) <= sizeof(smem),
                  "statistics scratch fits after the staged tile");
    tile_group_sums<kLinThreads, kLinBM, kLinBN>(
        reinterpret_cast<const uint16_t*>(tile), 4 * kRowU2, [&](int r) { return m0 + r < a.M; },
        static_cast<int>(n0), static_cast<int>(a.N), static_cast<int>(a.N / a.G), a.G,
        reinterpret_cast<float*>(tile + kLinBM * kRowU2), a.gn_part + (b * nchunk + chunk) * a.G * 2);
  }
}

// Token tile: 160 tokens (8 waves), or 80 tokens (4 waves) when the
// 160-token grid would fill at most half of the 256 CUs.  Each workgroup
// runs the whole K chain serially, so at few tiles more, smaller
// workgroups finish sooner (1024 and 2048 tokens x 640 x 640: 10.2-10.5 ->
// 8.4-8.7 us); with a full grid the larger tile is faster.
static int linear_bm(int64_t B, int64_t M, int64_t N) {
  return ceil_div(M, kLinBM) * B * ceil_div(N, 128) <= 128 ? kLinBMSmall : kLinBM;
}

// Channel tile of the bf16 kernel: the one with the fewer rounds of
// workgroups times tile width (one workgroup per CU); ties go to the wider
// tile (fewer loads of the token rows, one prologue instead of several).
static bool linear_wide(int64_t B, int64_t M, int64_t N) {
  const int64_t tm = ceil_div(M, linear_bm(B, M, N)) * B;
  const int64_t cost2 = ceil_div(tm * ceil_div(N, 128), 256) * 128;
  const int64_t cost4 = ceil_div(tm * ceil_div(N, 256), 256) * 256;
  return cost4 <= cost2;
}

int64_t linear_gn_chunks(int64_t B, int64_t M, int64_t N) {
  return ceil_div(M, linear_bm(B, M, N)) * ceil_div(N, linear_wide(B, M, N) ? 256 : 128);
}

template <int BM>
static void launch_linear_bf16(const LinArgs& a, int64_t K, bool wide, dim3 grid, hipStream_t s) {
  const dim3 blk(BM / 80 * 256);
  switch (ceil_div(K, kLinKC) * 2 + (wide ? 1 : 0)) {
    case 10: hipLaunchKernelGGL((linear_bf16_mfma_kernel<5, 2, BM>), grid, blk, 0, s, a); break;
    case 11: hipLaunchKernelGGL((linear_bf16_mfma_kernel<5, 4, BM>), grid, blk, 0, s, a); break;
    case 20: hipLaunchKernelGGL((linear_bf16_mfma_kernel<10, 2, BM>), grid, blk, 0, s, a); break;
    case 21: hipLaunchKernelGGL((linear_bf16_mfma_kernel<10, 4, BM>), grid, blk, 0, s, a); break;
    case 40: hipLaunchKernelGGL((linear_bf16_mfma_kernel<20, 2, BM>), grid, blk, 0, s, a); break;
    case 41: hipLaunchKernelGGL((linear_bf16_mfma_kernel<20, 4, BM>), grid, blk, 0, s, a); break;
    default:
      if (wide) hipLaunchKernelGGL((linear_bf16_mfma_kernel<0, 4, BM>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((linear_bf16_mfma_kernel<0, 2, BM>), grid, blk, 0, s, a);
      break;
  }
}

hipError_t launch_linear(void* y, const void* x, const void* w, const float* bias, int64_t B, int64_t M, int64_t K,
                         int64_t N, int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, bool bf16, hipStream_t s,
                         float* gn_part, int G) {
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
  a.gn_part = gn_part;
  a.G = G;
  const bool wide = linear_wide(B, M, N);
  const int bm = linear_bm(B, M, N);
  dim3 grid(static_cast<unsigned>(ceil_div(M, bm)), static_cast<unsigned>(ceil_div(N, wide ? 256 : 128)),
            static_cast<unsigned>(B));
  if (bm == kLinBM)
    launch_linear_bf16<kLinBM>(a, K, wide, grid, s);
  else
    launch_linear_bf16<kLinBMSmall>(a, K, wide, grid, s);
  return hipGetLastError();
}

}  // namespace dpp
