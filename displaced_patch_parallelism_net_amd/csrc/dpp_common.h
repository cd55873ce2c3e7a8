// Internal helpers shared by the libdpp kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// 8 bf16 in a uint4 -> 8 floats.
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16);
  f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16);
  f[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static float load(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  __device__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
  __device__ static void unpack(const uint4& u, float* f) { unpack8(u, f); }
  __device__ static uint4 pack(const float* f) { return pack8(f); }
};

// Streaming (non-temporal) 16-byte access for data touched once: it does not
// displace reusable lines from the caches, and measured faster for large
// cold copies on gfx950.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint4* p, const uint4& u) {
  const u32x4 v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// GroupNorm partial sums of a bf16 output tile staged in LDS, taken from the
// stored (rounded) values because those are what a following GroupNorm
// reads.  For every group g of G (output channels [g*cg, (g+1)*cg)):
//   out[2g] = sum of y, out[2g+1] = sum of y^2
// over the tile's valid pixels and its valid channels of group g; zero for a
// group the tile does not touch.  Tile element (pixel p, channel c) is
// tile[p * stride + c] (bf16 bits; stride a multiple of 4) for p < NPIX,
// c < NCH; pixel p counts when pix_ok(p); channel c is output channel m0 + c
// and counts when m0 + c < n_valid.  Fixed summation order, no atomics:
//   1. thread (quad q, lane k) adds channels 4q..4q+3 over pixels k, k + KP, ...
//   2. thread c adds the KP lane sums of channel c in lane order;
//   3. eight lanes per group add its channels j, j + 8, ... and an xor
//      butterfly joins the eight.
// red is LDS scratch of 2 * (NTHREADS * 4 + NCH) floats that nothing else
// uses during the call; all threads of the workgroup must call (barriers
// inside).
template <int NTHREADS, int NCH>
constexpr int tile_group_sums_scratch_floats() { return 2 * ((NTHREADS / (NCH / 4)) * NCH + NCH); }

template <int NTHREADS, int NPIX, int NCH, typename PixOk>
__device__ __forceinline__ void tile_group_sums(const uint16_t* tile, int stride, PixOk pix_ok, int m0, int n_valid,
                                                int cg, int G, float* red, float* out) {
  constexpr int NQ = NCH / 4;
  static_assert(NCH % 4 == 0 && NTHREADS % NQ == 0, "whole channel quads and pixel lanes");
  constexpr int KP = NTHREADS / NQ;
  const int t = threadIdx.x;
  const int q = t % NQ, k = t / NQ;
  float s1[4] = {0.f, 0.f, 0.f, 0.f}, s2[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p = k; p < NPIX; p += KP) {
    if (pix_ok(p)) {
      const uint2 u = *reinterpret_cast<const uint2*>(tile + p * stride + 4 * q);
      const float v[4] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                          __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s1[e] += v[e];
        s2[e] = fmaf(v[e], v[e], s2[e]);
      }
    }
  }
  float* lane_sums = red;                       // [KP][NCH][2]
  float* chan_sums = red + 2 * KP * NCH;        // [NCH][2]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = m0 + 4 * q + e < n_valid;
    lane_sums[2 * (k * NCH + 4 * q + e)] = ok ? s1[e] : 0.f;
    lane_sums[2 * (k * NCH + 4 * q + e) + 1] = ok ? s2[e] : 0.f;
  }
  __syncthreads();
  for (int c = t; c < NCH; c += NTHREADS) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) {
      a += lane_sums[2 * (kk * NCH + c)];
      b += lane_sums[2 * (kk * NCH + c) + 1];
    }
    chan_sums[2 * c] = a;
    chan_sums[2 * c + 1] = b;
  }
  __syncthreads();
  const int cend = min(NCH, n_valid - m0);
  const int j = t % 8;
  for (int g = t / 8; g < G; g += NTHREADS / 8) {  // uniform within each set of eight lanes
    float a = 0.f, b = 0.f;
    const int c0 = max(g * cg - m0, 0), c1 = min((g + 1) * cg - m0, cend);
    for (int c = c0 + j; c < c1; c += 8) {
      a += chan_sums[2 * c];
      b += chan_sums[2 * c + 1];
    }
#pragma unroll
    for (int off = 4; off > 0; off >>= 1) {
      a += __shfl_xor(a, off, 8);
      b += __shfl_xor(b, off, 8);
    }
    if (j == 0) {
      out[2 * g] = a;
      out[2 * g + 1] = b;
    }
  }
}

}  // namespace dpp

// Launchers (host side, one per kernel family).  They assume validated
// arguments and return the hipError_t of the launch.
namespace dpp {
hipError_t launch_splice(void* full, const void* patch, int64_t B, int64_t H, int64_t W, int64_t C,
                         int64_t row0, int64_t rows, int esize, hipStream_t s);

size_t gn_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t C, int64_t G);
size_t gn_scratch_bytes();
hipError_t gn_scratch_ptr(void** out);
hipError_t launch_groupnorm(void* y, float* stats_out, const void* x, const float* stale_stats,
                            const float* gamma, const float* beta, int64_t B, int64_t H, int64_t W,
                            int64_t C, int64_t G, int64_t P, int64_t p, int64_t rows, float eps,
                            void* ws, bool bf16, bool silu, hipStream_t s);
// GroupNorm whose fresh sums come from a producer's partials [B][nchunk][G][2]:
// one fused finalize + apply launch, no workspace
hipError_t launch_groupnorm_presummed(void* y, float* stats_out, const void* x, const float* partials,
                                      int64_t nchunk, const float* stale_stats, const float* gamma,
                                      const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G,
                                      int64_t P, int64_t p, int64_t rows, float eps, bool bf16, bool silu,
                                      hipStream_t s);

size_t conv_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout);
// gn_part != NULL: GroupNorm partial sums of y, [B][conv_gn_chunks][G][2]
// (bf16 only, always unsplit)
int64_t conv_gn_chunks(int64_t rows, int64_t W, int64_t Cout);
hipError_t launch_conv3x3(void* y, const void* x, const void* stale_full, const void* weight,
                          const float* bias, int64_t B, int64_t H, int64_t W, int64_t Cin,
                          int64_t Cout, int64_t row0, int64_t rows, void* ws, size_t ws_bytes, bool bf16,
                          hipStream_t s, float* gn_part = nullptr, int G = 0);

size_t attn_workspace_bytes(int64_t B, int64_t n_q, int64_t n_kv, int64_t heads, int64_t D, bool bf16);
hipError_t launch_attention(void* o, const void* q, const void* k, const void* v, int64_t B,
                            int64_t n_q, int64_t n_kv, int64_t heads, int64_t D, int64_t ld_q,
                            int64_t ld_kv, int64_t ld_o, float scale, void* ws, size_t ws_bytes,
                            bool bf16, hipStream_t s);

// gn_part != NULL: GroupNorm partial sums of y, [B][linear_gn_chunks][G][2] (bf16 only)
int64_t linear_gn_chunks(int64_t B, int64_t M, int64_t N);
hipError_t launch_linear(void* y, const void* x, const void* w, const float* bias, int64_t B, int64_t M,
                         int64_t K, int64_t N, int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, bool bf16,
                         hipStream_t s, float* gn_part = nullptr, int G = 0);

size_t cfg_workspace_bytes(int64_t n);
hipError_t launch_cfg(void* eps, float* relmae, const void* eps_c, const void* eps_u, int64_t n,
                      float guidance, void* ws, bool bf16, hipStream_t s);
}  // namespace dpp
