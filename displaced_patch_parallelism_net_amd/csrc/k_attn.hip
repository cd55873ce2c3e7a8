// a4 -- displaced self-attention: the patch's queries against all tokens of
// the spliced full-image K/V buffer.
//
// DistriSelfAttentionPP (DistriFusion architecture article, attention
// section); the K/V rows of other patches are the previous step's
// (DistriFusion reading notes, Introduction, fourth paragraph).  Per batch b,
// head h and query i: o = softmax(scale q k^T) v over every key.
//
// bf16 path (head_dim 64): one pass over the keys with an online softmax
// (running max m, running sum l, rescaled output), all on MFMA
// v_mfma_f32_32x32x16_bf16:
//  * a workgroup owns 256 queries of one (b, h) and a range of keys; each of
//    its four waves owns 64 queries (two 32-query blocks) whose Q fragments
//    stay in registers for the whole pass;
//  * K and V tiles of 64 keys are double-buffered in LDS; the next tile's
//    global loads are issued before the current tile's math;
//  * scores are computed transposed, S^T = K Q^T, so each lane holds the
//    scores of one query: the row max needs one cross-lane exchange, the row
//    sum stays lane-local until the end, and the rescale of O^T is per lane;
//  * the accumulator layout of S^T is reused as the B operand of
//    O^T = V^T P^T after conversion to bf16: within every 16 keys the MFMA's
//    k index runs over the keys in the order 0-3, 8-11, 4-7, 12-15, so V is
//    written to LDS transposed ([d][key]) in that order;
//  * scores are scaled by scale*log2(e) and exponentiated with exp2.
// When the workspace allows, the key range is split over several workgroups
// (fills the GPU when there are few query tiles); a second kernel merges the
// partial (m, l, O) triples.
//
// f32 path: one thread per query, scalar online softmax (small shapes).
#include "dpp_common.h"

namespace dpp {

// ------------------------------------------------------------------ fp32 reference-style kernel
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, float* __restrict__ o, int n_q,
                                                      int n_kv, int heads, int64_t ld_q, int64_t ld_kv, int64_t ld_o,
                                                      float scale) {
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh % heads;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n_q) return;
  const float* qp = q + (static_cast<int64_t>(b) * n_q + i) * ld_q + h * D;
  const float* kb = k + static_cast<int64_t>(b) * n_kv * ld_kv + h * D;
  const float* vb = v + static_cast<int64_t>(b) * n_kv * ld_kv + h * D;
  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qr[d] = qp[d] * scale; acc[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < n_kv; ++j) {
    const float* kr = kb + static_cast<int64_t>(j) * ld_kv;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qr[d], kr[d], s);
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);
    const float p = expf(s - mn);
    l = l * alpha + p;
    const float* vr = vb + static_cast<int64_t>(j) * ld_kv;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], alpha, p * vr[d]);
    m = mn;
  }
  float* op = o + (static_cast<int64_t>(b) * n_q + i) * ld_o + h * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

// ------------------------------------------------------------------ bf16 MFMA flash kernel
constexpr int kAttD = 64;
constexpr int kAttKT = 64;                      // keys per tile
constexpr int kAttWaves = 4;
constexpr int kAttQW = 64;                      // queries per wave
constexpr int kAttQT = kAttQW * kAttWaves;      // queries per workgroup
constexpr int kAttThreads = kAttWaves * kWave;
constexpr int kAttRow = 72;                     // padded LDS row (bf16): 144 bytes
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* o_part;   // [nsplit][B*heads][n_q][64] unnormalised, split mode only
  float* ml_part;  // [nsplit][B*heads][n_q][2] (m, l), split mode only
  int n_q, n_kv, heads;
  int64_t ld_q, ld_kv, ld_o;
  float c;          // scale * log2(e)
  int keys_per_split;
  int n_qt, n_bh;   // query tiles, batch*heads
};

// Position of key (0..15) inside its 16-key group in the MFMA k order.
__device__ __forceinline__ int kperm16(int key) {
  const int g = (key >> 3) & 1, a = (key >> 2) & 1;
  return (key & ~15) | (a << 3) | (g << 2) | (key & 3);
}

// Lazy rescaling.  The running reference m of a query only moves when a
// tile's max exceeds it by more than kTau (log2 units); softmax does not
// depend on the reference point, so this is exact as long as P = 2^(s - m)
// stays finite and representable.  The fast path therefore skips the tile
// max entirely: it exponentiates with the current m and checks the lane's
// partial row sum -- if that sum is <= kSumCap every P in it is too.  A lane
// above the cap (or inf/NaN: the first tile, m = -inf) sends the whole wave
// through the exact path for that tile: true tile max, rescale, recompute.
constexpr float kTau = 8.0f;
constexpr float kSumCap = 4096.0f;

// gfx9 buffer resource word 3 (32-bit raw access, no swizzle).
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Software pipeline over "units" u = (tile t, key half kb): 32 keys x 64
// queries per wave.  Within unit u the wave exponentiates S_u on the VALU
// while the MFMA pipe computes S_{u+1} = K_{u+1} Q^T and O += V_{u-1} P_{u-1}:
// the two instruction streams are interleaved in four chunks of four MFMAs
// and one eighth of the exponentials each, so one wave keeps both pipes busy.
// A tile is read from LDS during three consecutive iterations (K of the next
// unit, V of the previous one), so four LDS buffers rotate and one barrier
// per tile suffices: tile t+2 is written at the start of iteration t into the
// buffer tile t-2 used, which every wave left before the previous barrier.
constexpr int kAttBufs = 4;

__global__ __launch_bounds__(kAttThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  __shared__ __align__(16) uint16_t Ks[kAttBufs][kAttKT * kAttRow];
  __shared__ __align__(16) uint16_t Vt[kAttBufs][kAttD * kAttRow];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int g = lane >> 5, l32 = lane & 31;
  // XCD-aware order: the hardware deals workgroup ids round-robin to the 8
  // XCDs; give each XCD a contiguous range of logical ids, query tile
  // fastest, so workgroups sharing a (head, key range) share one L2.
  const int total = gridDim.x, lid = blockIdx.x;
  const int per = total / 8, rem = total % 8, xcd = lid % 8;
  const int logical = xcd * per + min(xcd, rem) + lid / 8;
  const int qtile = logical % a.n_qt;
  const int bh = (logical / a.n_qt) % a.n_bh;
  const int split = logical / (a.n_qt * a.n_bh);
  const int b = bh / a.heads, h = bh % a.heads;
  const int k_begin = split * a.keys_per_split;
  const int k_end = min(a.n_kv, k_begin + a.keys_per_split);
  const int q0 = qtile * kAttQT + wave * kAttQW;
  const bool active = q0 < a.n_q;  // waves wholly past the queries only stage tiles

  const uint16_t* qb = a.q + static_cast<int64_t>(b) * a.n_q * a.ld_q + h * kAttD;
  const uint16_t* kb = a.k + static_cast<int64_t>(b) * a.n_kv * a.ld_kv + h * kAttD;
  const uint16_t* vb = a.v + static_cast<int64_t>(b) * a.n_kv * a.ld_kv + h * kAttD;
  const int row_bytes = static_cast<int>(a.ld_kv) * 2;

  // Q^T fragments (B operand of S^T = K Q^T): lane -> query l32, d = 16 ks + 8 g + 0..7
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    const int qi = q0 + qb2 * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(qb + static_cast<int64_t>(min(qi, a.n_q - 1)) * a.ld_q + ks * 16 + g * 8);
      if (qi >= a.n_q) u = make_uint4(0, 0, 0, 0);
      qf[qb2][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // Tile loader: buffer loads against a per-tile resource ending at the last
  // valid key; rows past it read as zero.  K: thread -> keys kk and kk+32,
  // 16-byte column dv (8 lanes per 128-byte row; the two rows of a 16-lane
  // group land 32 words apart in LDS).  V: thread -> key pair (2kp, 2kp+1),
  // column dvv; a wave's lanes walk all 32 key pairs of two columns, so its
  // transposed 32-bit LDS writes cover 64 distinct banks.
  const int kk = tid >> 3, dv = tid & 7;
  const int kp = tid & 31, dvv = tid >> 5;
  const int koff0 = kk * row_bytes + dv * 16, koff1 = koff0 + 32 * row_bytes;
  const int voff0 = (2 * kp) * row_bytes + dvv * 16, voff1 = voff0 + row_bytes;
  uint4 kr0, kr1, vr0, vr1;
  auto load_tile = [&](int t0) {
    const int valid = min(k_end - t0, kAttKT);
    const int nrec = (valid - 1) * row_bytes + kAttD * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kb + static_cast<int64_t>(t0) * a.ld_kv), 0, nrec, kBufWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vb + static_cast<int64_t>(t0) * a.ld_kv), 0, nrec, kBufWord3);
    kr0 = buffer_load16(rk, koff0);
    kr1 = buffer_load16(rk, koff1);
    vr0 = buffer_load16(rv, voff0);
    vr1 = buffer_load16(rv, voff1);
  };
  const int vpos = kperm16(2 * kp);
  auto store_tile = [&](int buf) {
    *reinterpret_cast<uint4*>(&Ks[buf][kk * kAttRow + dv * 8]) = kr0;
    *reinterpret_cast<uint4*>(&Ks[buf][(kk + 32) * kAttRow + dv * 8]) = kr1;
    const uint32_t a0[4] = {vr0.x, vr0.y, vr0.z, vr0.w};
    const uint32_t a1[4] = {vr1.x, vr1.y, vr1.z, vr1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
      *reinterpret_cast<uint32_t*>(&Vt[buf][(dvv * 8 + 2 * e) * kAttRow + vpos]) = lo;
      *reinterpret_cast<uint32_t*>(&Vt[buf][(dvv * 8 + 2 * e + 1) * kAttRow + vpos]) = hi;
    }
  };
  auto k_frag = [&](int buf, int kh, int ks) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Ks[buf][(kh * 32 + l32) * kAttRow + ks * 16 + g * 8]));
  };
  auto v_frag = [&](int buf, int db, int kh, int t16) {
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(&Vt[buf][(db * 32 + l32) * kAttRow + kh * 32 + t16 * 16 + g * 8]));
  };

  f32x16 O[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[i][j][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  // One eighth of a unit's exponentials: query block qb2, keys 16*t16 .. +15
  // of the half.  The row sum adds the float32 weights (before their bf16
  // rounding) in a short tree: on gfx950 plain adds issue beside a running
  // MFMA far better than the packed bf16 dot product, and the normaliser
  // then differs from the sum of the rounded weights only by their
  // independent rounding errors.
  // The first chunk of a query block (t16 == 0) starts its partial sum
  // instead of adding to a zero: 0 + x is not x for x = -0, so an add of
  // zero would stay in the code.
  auto exp_chunk = [&](const f32x16 (&S)[2], int qb2, int t16, const float (&m)[2], bf16x8 (&P)[2][2], float (&ls)[2]) {
    uint32_t w[4];
    float s2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(S[qb2][t16 * 8 + 2 * e], a.c, -m[qb2]));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(S[qb2][t16 * 8 + 2 * e + 1], a.c, -m[qb2]));
      w[e] = pack_bf16x2(p0, p1);
      s2[e] = p0 + p1;
    }
    const float sum = (s2[0] + s2[1]) + (s2[2] + s2[3]);
    ls[qb2] = t16 == 0 ? sum : ls[qb2] + sum;
    P[qb2][t16] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  };
  // scores of a unit in the ragged last tile: keys past the range -> -inf
  auto mask_unit = [&](f32x16 (&S)[2], int t0, int kh) {
    if (t0 + kAttKT > k_end) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + kh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= k_end) { S[0][r] = -INFINITY; S[1][r] = -INFINITY; }
      }
    }
  };
  // One unit: exponentiate Scur (reference m_run) into Pcur while issuing
  // Snext = K(buf_k, kh_next) Q^T and O += V(buf_v, kh_prev) Pprev.  Then the
  // overflow guard / exact path for Pcur.  Returns nothing; updates l_run.
  auto unit = [&](const f32x16 (&Scur)[2], bf16x8 (&Pcur)[2][2], f32x16 (&Snext)[2], int buf_k, int kh_next,
                  const bf16x8 (&Pprev)[2][2], int buf_v, int kh_prev) {
    const bf16x8 kf0 = k_frag(buf_k, kh_next, 0), kf1 = k_frag(buf_k, kh_next, 1);
    const bf16x8 kf2 = k_frag(buf_k, kh_next, 2), kf3 = k_frag(buf_k, kh_next, 3);
    const bf16x8 vf00 = v_frag(buf_v, 0, kh_prev, 0), vf01 = v_frag(buf_v, 0, kh_prev, 1);
    const bf16x8 vf10 = v_frag(buf_v, 1, kh_prev, 0), vf11 = v_frag(buf_v, 1, kh_prev, 1);
    float ls[2];
    const float m[2] = {m_run[0], m_run[1]};
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    // chunk 0
    Snext[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0][0], z, 0, 0, 0);
    Snext[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[1][0], z, 0, 0, 0);
    Snext[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[0][1], Snext[0], 0, 0, 0);
    Snext[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[1][1], Snext[1], 0, 0, 0);
    exp_chunk(Scur, 0, 0, m, Pcur, ls);
    // chunk 1
    Snext[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf2, qf[0][2], Snext[0], 0, 0, 0);
    Snext[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf2, qf[1][2], Snext[1], 0, 0, 0);
    Snext[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf3, qf[0][3], Snext[0], 0, 0, 0);
    Snext[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf3, qf[1][3], Snext[1], 0, 0, 0);
    exp_chunk(Scur, 0, 1, m, Pcur, ls);
    // chunk 2
    O[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf00, Pprev[0][0], O[0][0], 0, 0, 0);
    O[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf00, Pprev[1][0], O[1][0], 0, 0, 0);
    O[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf01, Pprev[0][1], O[0][0], 0, 0, 0);
    O[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf01, Pprev[1][1], O[1][0], 0, 0, 0);
    exp_chunk(Scur, 1, 0, m, Pcur, ls);
    // chunk 3
    O[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf10, Pprev[0][0], O[0][1], 0, 0, 0);
    O[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf10, Pprev[1][0], O[1][1], 0, 0, 0);
    O[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf11, Pprev[0][1], O[0][1], 0, 0, 0);
    O[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf11, Pprev[1][1], O[1][1], 0, 0, 0);
    exp_chunk(Scur, 1, 1, m, Pcur, ls);
    // Materialise the packed weights before the guard branch: the exact path
    // overwrites them, so the compiler would otherwise sink their conversion
    // past the branch, where no MFMA is left to overlap it.
    asm volatile("" ::"v"(Pcur[0][0]), "v"(Pcur[0][1]), "v"(Pcur[1][0]), "v"(Pcur[1][1]));
    // overflow guard; the exact path runs after this unit's MFMAs were issued,
    // so the O rescale applies to everything accumulated so far
    if (__builtin_amdgcn_ballot_w64(!(ls[0] <= kSumCap) || !(ls[1] <= kSumCap)) != 0) {
      float mn[2];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        float mx = Scur[qb2][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, Scur[qb2][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * a.c;
        mn[qb2] = (mx > m_run[qb2] + kTau) ? mx : m_run[qb2];
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb2] - mn[qb2]);
        m_run[qb2] = mn[qb2];
        l_run[qb2] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[qb2][db][r] *= alpha;
      }
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16) exp_chunk(Scur, qb2, t16, mn, Pcur, ls);
    }
    l_run[0] += ls[0];
    l_run[1] += ls[1];
  };

  const int ntiles = (k_end - k_begin + kAttKT - 1) / kAttKT;
  // prologue: tiles 0 and 1 into buffers 0 and 1, tile 2 into registers; the
  // V^T buffer of "tile -1" (buffer 3) holds zeros for the first unit's
  // (empty) O update
  load_tile(k_begin);
  store_tile(0);
  if (ntiles > 1) {
    load_tile(k_begin + kAttKT);
    store_tile(1);
  }
  for (int i = tid; i < kAttD * kAttRow / 2; i += kAttThreads) reinterpret_cast<uint32_t*>(Vt[3])[i] = 0u;
  if (ntiles > 2) load_tile(k_begin + 2 * kAttKT);
  __syncthreads();

  f32x16 S0[2], S1[2];   // scores of the current tile's first / second key half
  bf16x8 P0[2][2], P1[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P0[i][j] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      P1[i][j] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    S0[0] = z;
    S0[1] = z;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kf = k_frag(0, 0, ks);
      S0[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][ks], S0[0], 0, 0, 0);
      S0[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[1][ks], S0[1], 0, 0, 0);
    }
  }

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = k_begin + t * kAttKT;
    if (t + 2 < ntiles) {
      store_tile((t + 2) & 3);
      if (t + 3 < ntiles) load_tile(t0 + 3 * kAttKT);
    }
    const int bt = t & 3, bprev = (t + 3) & 3, bnext = (t + 1) & 3;
    // unit (t, 0): softmax S0 -> P0; S1 = K(t, half 1) Q^T; O += V(t-1, half 1) P1
    if (active) {
      mask_unit(S0, t0, 0);
      unit(S0, P0, S1, bt, 1, P1, bprev, 1);
      // unit (t, 1): softmax S1 -> P1; S0 = K(t+1, half 0) Q^T (unused after
      // the last tile); O += V(t, half 0) P0
      mask_unit(S1, t0, 1);
      unit(S1, P1, S0, bnext, 0, P0, bt, 0);
    }
    __syncthreads();
  }
  // drain: O += V(last, half 1) P1
  {
    const int bl = (ntiles - 1) & 3;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int t16 = 0; t16 < 2; ++t16) {
        const bf16x8 vf = v_frag(bl, db, 1, t16);
        O[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P1[0][t16], O[0][db], 0, 0, 0);
        O[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P1[1][t16], O[1][db], 0, 0, 0);
      }
  }

  // ---- epilogue: lane holds query l32, d = db*32 + 8*(r/4) + 4*g + r%4
  if (a.o_part == nullptr) {
#pragma unroll
    for (int qb2 = 0; qb2 < 2; ++qb2) {
      const int qi = q0 + qb2 * 32 + l32;
      const float l_tot = l_run[qb2] + __shfl_xor(l_run[qb2], 32, kWave);
      if (qi >= a.n_q) continue;
      const float inv = 1.f / l_tot;
      uint16_t* op = a.o + (static_cast<int64_t>(b) * a.n_q + qi) * a.ld_o + h * kAttD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + 8 * r4 + 4 * g;
          uint2 u;
          u.x = pack_bf16x2(O[qb2][db][r4 * 4 + 0] * inv, O[qb2][db][r4 * 4 + 1] * inv);
          u.y = pack_bf16x2(O[qb2][db][r4 * 4 + 2] * inv, O[qb2][db][r4 * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + d) = u;
        }
    }
    return;
  }
  // Split partials: each wave's 64 x 64 float32 block goes through LDS (the
  // tile buffers, free once every wave has finished the drain; rows padded
  // to 68 floats, a stride of 4 banks mod 64) so that each store writes four
  // whole 256-byte rows, which are consecutive in o_part, instead of 16-byte
  // pieces of 32 rows.
  constexpr int kStageRow = kAttD + 4;
  __syncthreads();
  float* const stage = reinterpret_cast<float*>(wave < 2 ? &Ks[0][0] : &Vt[0][0]) + (wave & 1) * kAttQW * kStageRow;
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    const int qi = q0 + qb2 * 32 + l32;
    const float l_tot = l_run[qb2] + __shfl_xor(l_run[qb2], 32, kWave);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(stage + (qb2 * 32 + l32) * kStageRow + db * 32 + 8 * r4 + 4 * g) =
            make_float4(O[qb2][db][r4 * 4 + 0], O[qb2][db][r4 * 4 + 1], O[qb2][db][r4 * 4 + 2], O[qb2][db][r4 * 4 + 3]);
    if (g == 0 && qi < a.n_q) {
      const int64_t row = (static_cast<int64_t>(split) * a.n_bh + bh) * a.n_q + qi;
      a.ml_part[row * 2] = m_run[qb2];
      a.ml_part[row * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  const int64_t row0 = (static_cast<int64_t>(split) * a.n_bh + bh) * a.n_q + q0;
#pragma unroll
  for (int it = 0; it < kAttQW / 4; ++it) {
    const int r = it * 4 + (lane >> 4), c = lane & 15;
    if (q0 + r < a.n_q)
      *reinterpret_cast<float4*>(a.o_part + (row0 + r) * kAttD + 4 * c) =
          *reinterpret_cast<const float4*>(stage + r * kStageRow + 4 * c);
  }
}

// Merge of key-range splits: thread per (b*heads, query, 4 channels).  All
// of a thread's partial loads are issued before any is used (the split count
// is at most MAXS), so a thread waits for one memory round trip, not nsplit.
template <int MAXS>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ ml_part, uint16_t* __restrict__ o,
                                                         int nsplit, int n_q, int heads, int64_t ld_o, int64_t rows) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * 16) return;
  const int64_t row = idx / 16;  // bh * n_q + qi
  const int dq = static_cast<int>(idx % 16);
  float2 ml[MAXS];
  f32x4 ov[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < nsplit) {
      const int64_t r = s * rows + row;
      ml[s] = *reinterpret_cast<const float2*>(ml_part + r * 2);
      ov[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_part + r * kAttD + dq * 4));
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < nsplit) M = fmaxf(M, ml[s].x);
  float L = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < nsplit) {
      const float w = __builtin_amdgcn_exp2f(ml[s].x - M);
      L = fmaf(w, ml[s].y, L);
      acc[0] = fmaf(w, ov[s].x, acc[0]);
      acc[1] = fmaf(w, ov[s].y, acc[1]);
      acc[2] = fmaf(w, ov[s].z, acc[2]);
      acc[3] = fmaf(w, ov[s].w, acc[3]);
    }
  }
  const float inv = 1.f / L;
  const int64_t bh = row / n_q, qi = row % n_q;
  const int64_t b = bh / heads, h = bh % heads;
  uint16_t* op = o + (b * n_q + qi) * ld_o + h * kAttD + dq * 4;
  uint2 u;
  u.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  u.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(op) = u;
}

// Key-range split policy: depends on the shape only (so the workspace query
// needs no device).  An MI355X holds 256 CUs x 2 resident workgroups of this
// kernel; pick the smallest split count whose workgroup count fills the
// resident slots in whole rounds to >= 97 % (else the best one), keeping
// >= 8 key tiles per split.  (At 7200 queries x 57600 keys x 10 heads: 7
// splits, 2030 workgroups, 99 % of four rounds.)
constexpr int64_t kAttSlots = 256 * 2;
struct AttnSplit {
  int nsplit;
  int keys_per_split;
};
static AttnSplit attn_split(int64_t B, int64_t n_q, int64_t n_kv, int64_t heads) {
  const int64_t qtiles = ceil_div(n_q, kAttQT) * B * heads;
  const int64_t ktiles = ceil_div(n_kv, kAttKT);
  const int64_t max_ns = ktiles / 8 > 1 ? (ktiles / 8 < 16 ? ktiles / 8 : 16) : 1;
  int64_t best = 1;
  double best_eff = 0.0;
  for (int64_t ns = 1; ns <= max_ns; ++ns) {
    const int64_t kps_t = ceil_div(ktiles, ns);
    const int64_t ns_eff = ceil_div(ktiles, kps_t);
    const int64_t total = qtiles * ns_eff;
    const double eff = static_cast<double>(total) / static_cast<double>(ceil_div(total, kAttSlots) * kAttSlots);
    if (eff > best_eff + 1e-9) { best_eff = eff; best = ns; }
    if (eff >= 0.97) break;
  }
  const int64_t kps = ceil_div(ktiles, best) * kAttKT;
  const int64_t ns = ceil_div(n_kv, kps);
  return AttnSplit{static_cast<int>(ns), static_cast<int>(kps)};
}

size_t attn_workspace_bytes(int64_t B, int64_t n_q, int64_t n_kv, int64_t heads, int64_t D, bool bf16) {
  if (!bf16 || D != kAttD) return 0;
  const AttnSplit sp = attn_split(B, n_q, n_kv, heads);
  if (sp.nsplit <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(sp.nsplit) * B * heads * n_q;
  return static_cast<size_t>(rows * (kAttD + 2)) * sizeof(float);
}

hipError_t launch_attention(void* o, const void* q, const void* k, const void* v, int64_t B, int64_t n_q, int64_t n_kv,
                            int64_t heads, int64_t D, int64_t ld_q, int64_t ld_kv, int64_t ld_o, float scale, void* ws,
                            size_t ws_bytes, bool bf16, hipStream_t s) {
  if (!bf16) {
    dim3 grid(static_cast<unsigned>(ceil_div(n_q, 64)), static_cast<unsigned>(B * heads));
    auto* qq = static_cast<const float*>(q);
    auto* kk = static_cast<const float*>(k);
    auto* vv = static_cast<const float*>(v);
    auto* oo = static_cast<float*>(o);
    const int nq = static_cast<int>(n_q), nkv = static_cast<int>(n_kv), hh = static_cast<int>(heads);
    switch (D) {
      case 16: hipLaunchKernelGGL(attn_f32_kernel<16>, grid, dim3(64), 0, s, qq, kk, vv, oo, nq, nkv, hh, ld_q, ld_kv, ld_o, scale); break;
      case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, s, qq, kk, vv, oo, nq, nkv, hh, ld_q, ld_kv, ld_o, scale); break;
      case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, qq, kk, vv, oo, nq, nkv, hh, ld_q, ld_kv, ld_o, scale); break;
      default: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, qq, kk, vv, oo, nq, nkv, hh, ld_q, ld_kv, ld_o, scale); break;
    }
    return hipGetLastError();
  }
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.n_q = static_cast<int>(n_q);
  a.n_kv = static_cast<int>(n_kv);
  a.heads = static_cast<int>(heads);
  a.ld_q = ld_q;
  a.ld_kv = ld_kv;
  a.ld_o = ld_o;
  a.c = scale * kLog2e;
  AttnSplit sp = attn_split(B, n_q, n_kv, heads);
  const size_t need = attn_workspace_bytes(B, n_q, n_kv, heads, D, true);
  if (sp.nsplit > 1 && (ws == nullptr || ws_bytes < need)) {
    sp.nsplit = 1;
    sp.keys_per_split = static_cast<int>(ceil_div(n_kv, kAttKT) * kAttKT);
  }
  a.keys_per_split = sp.keys_per_split;
  const int64_t rows = B * heads * n_q;
  if (sp.nsplit > 1) {
    a.o_part = static_cast<float*>(ws);
    a.ml_part = a.o_part + static_cast<int64_t>(sp.nsplit) * rows * kAttD;
  } else {
    a.o_part = nullptr;
    a.ml_part = nullptr;
  }
  a.n_qt = static_cast<int>(ceil_div(n_q, kAttQT));
  a.n_bh = static_cast<int>(B * heads);
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.n_qt) * a.n_bh * sp.nsplit));
  hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(kAttThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || sp.nsplit <= 1) return err;
  const dim3 mgrid(static_cast<unsigned>(ceil_div(rows * 16, 256)));
  if (sp.nsplit <= 8)
    hipLaunchKernelGGL(attn_merge_kernel<8>, mgrid, dim3(256), 0, s, a.o_part, a.ml_part, a.o, sp.nsplit, a.n_q,
                       a.heads, ld_o, rows);
  else
    hipLaunchKernelGGL(attn_merge_kernel<16>, mgrid, dim3(256), 0, s, a.o_part, a.ml_part, a.o, sp.nsplit, a.n_q,
                       a.heads, ld_o, rows);
  return hipGetLastError();
}

}  // namespace dpp
