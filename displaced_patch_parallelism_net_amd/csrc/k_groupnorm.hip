// a2 -- GroupNorm of one patch with statistics corrected by stale sums.
//
// DistriGroupNorm (DistriFusion architecture article, normalisation section):
// the group statistics are those of the spliced image -- the other patches'
// raw sums (sum x, sum x^2) from the previous step plus the own patch's fresh
// sums (DistriFusion reading notes, Introduction, fourth paragraph).
//
// Two launches, deterministic (no atomics):
//   1. partial: workgroup (chunk, b) sums its pixels per channel in float32
//      registers (each thread owns one 16-byte channel vector and walks
//      pixels, eight loads in flight), folds channels into groups through
//      LDS in a fixed order and writes one (s1, s2) per group to the
//      workspace;
//   2. apply: a workgroup owns 64 channels of batch entry b; it adds the
//      chunk partials of the few groups those channels touch in float64 in
//      a fixed order (the fresh sums, stored to stats_out[b, p]), forms
//      mean/rstd from them and the other patches' stale sums, and streams
//      y = x * a_c + b_c (then SiLU when asked).
// The second read of x (step 2) normally hits the 256 MB last-level cache.
// When the kernel that wrote x also wrote its group partial sums (the conv
// and projection epilogues), step 1 is skipped and x is read once, in one
// launch.  The statistics-only call (no y) runs the float64 sums as a
// kernel of its own (gn_stats_kernel): the same order, the same bits.
#include <mutex>

#include "dpp_common.h"

// Scratch of the allocation-free GroupNorm entry point (the chunk partial
// sums, exactly the workspace the other entry points take from the caller).  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kGnScratchBytes = size_t(1) << 20;   // DPP_GN_NOALLOC_MAX_BYTES
static __device__ __align__(256) unsigned char scratch[kGnScratchBytes];

namespace dpp {

size_t gn_scratch_bytes() { return kGnScratchBytes; }

// Device address of this device's scratch array, looked up on the first call
// made with that device current and kept for later calls.
hipError_t gn_scratch_ptr(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

constexpr int kGnMaxThreads = 256;
constexpr int kGnStatChunks = 256;    // total partial workgroups (over B)
constexpr int kGnInFlight = 8;        // 16-byte loads in flight per thread

struct GnGeom {
  int vec;      // elements per 16-byte vector
  int V;        // vectors per pixel = C / vec
  int KP;       // pixels walked in parallel per workgroup
  int threads;  // KP * V
  int64_t npix;
  int64_t nstat, stat_ppc;    // partial chunks per b, pixels per chunk
};

static GnGeom gn_geom(int64_t B, int64_t rows, int64_t W, int64_t C, bool bf16) {
  GnGeom g;
  g.vec = bf16 ? 8 : 4;
  g.V = static_cast<int>(C / g.vec);
  g.KP = kGnMaxThreads / g.V;
  if (g.KP < 1) g.KP = 1;
  g.threads = g.KP * g.V;
  g.npix = rows * W;
  const int64_t maxc = ceil_div(g.npix, g.KP);
  const int64_t want = ceil_div(kGnStatChunks, B);
  g.nstat = want < maxc ? want : maxc;
  if (g.nstat < 1) g.nstat = 1;
  g.stat_ppc = ceil_div(g.npix, g.nstat);
  g.nstat = ceil_div(g.npix, g.stat_ppc);
  return g;
}

size_t gn_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t C, int64_t G) {
  // bf16 and f32 differ in chunking; size for the larger of the two that
  // the channel count admits.
  int64_t nstat = gn_geom(B, rows, W, C, false).nstat;
  if (C % 8 == 0) {
    const int64_t nb = gn_geom(B, rows, W, C, true).nstat;
    if (nb > nstat) nstat = nb;
  }
  return static_cast<size_t>(B * nstat * G * 2) * sizeof(float);
}

template <typename T>
__global__ __launch_bounds__(kGnMaxThreads) void gn_partial_kernel(const T* __restrict__ x, float* __restrict__ partial,
                                                                   int64_t npix, int C, int G, int V, int KP,
                                                                   int64_t ppc, int64_t nchunk) {
  constexpr int VEC = Elem<T>::kVec;
  __shared__ float red1[kGnMaxThreads * 8];
  __shared__ float red2[kGnMaxThreads * 8];
  const int b = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int t = threadIdx.x;
  const int v = t % V, k = t / V;
  const int64_t p0 = chunk * ppc;
  const int64_t p1 = (p0 + ppc < npix) ? p0 + ppc : npix;
  const uint4* xv = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(b) * npix * C);
  float s1[VEC], s2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) { s1[j] = 0.f; s2[j] = 0.f; }
  if (k < KP) {
    int64_t pix = p0 + k;
    // kGnInFlight vectors in flight per iteration
    for (; pix + (kGnInFlight - 1) * KP < p1; pix += kGnInFlight * KP) {
      uint4 u[kGnInFlight];
#pragma unroll
      for (int q = 0; q < kGnInFlight; ++q) u[q] = xv[(pix + q * KP) * V + v];
#pragma unroll
      for (int q = 0; q < kGnInFlight; ++q) {
        float f[VEC];
        Elem<T>::unpack(u[q], f);
#pragma unroll
        for (int j = 0; j < VEC; ++j) { s1[j] += f[j]; s2[j] = fmaf(f[j], f[j], s2[j]); }
      }
    }
    for (; pix < p1; pix += KP) {
      float fa[VEC];
      Elem<T>::unpack(xv[pix * V + v], fa);
#pragma unroll
      for (int j = 0; j < VEC; ++j) { s1[j] += fa[j]; s2[j] = fmaf(fa[j], fa[j], s2[j]); }
    }
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      red1[k * C + v * VEC + j] = s1[j];
      red2[k * C + v * VEC + j] = s2[j];
    }
  }
  __syncthreads();
  // Fold channels into groups: eight consecutive lanes per group, lane j
  // summing the group's (pixel column, channel) values j, j + 8, ..., then a
  // fixed xor butterfly over the eight lanes.  Only whole eight-lane sets
  // take part (blockDim need not be a multiple of 8).
  constexpr int kFold = 8;
  const int cg = C / G, nv = KP * cg;
  const int sets = static_cast<int>(blockDim.x) / kFold;
  const int j = t % kFold;
  if (t < sets * kFold) {
    for (int g = t / kFold; g < G; g += sets) {
      float a = 0.f, c = 0.f;
      for (int i = j; i < nv; i += kFold) {
        const int kk = i / cg, ch = g * cg + i % cg;
        a += red1[kk * C + ch];
        c += red2[kk * C + ch];
      }
#pragma unroll
      for (int off = kFold / 2; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, kFold);
        c += __shfl_xor(c, off, kFold);
      }
      if (j == 0) {
        float* out = partial + ((static_cast<int64_t>(b) * nchunk + chunk) * G + g) * 2;
        out[0] = a;
        out[1] = c;
      }
    }
  }
}

// Fresh group sums of a patch from its chunk partials, in one fixed order: a
// wave handles one (b, g); lane j adds the chunk partials j, j + 64,
// j + 128, ... in float64 in increasing order (batches of kGnFinLoads loads
// issued before any is used; chunks past the end read as zero, which leaves
// the sums unchanged), and a 64-lane xor butterfly (offsets 32, 16, ..., 1)
// joins the lanes, every lane ending with the same sums.  The apply kernel
// forms the same sums in the same order.
constexpr int kGnFinLoads = 4;
constexpr int kGnSet = 64;

__device__ __forceinline__ double2 gn_fresh_sums(const float* __restrict__ partial, int64_t nchunk, int G, int b,
                                                 int g, int j) {
  double a = 0.0, c = 0.0;
  const float* base = partial + (static_cast<int64_t>(b) * nchunk * G + g) * 2;
  for (int64_t ch = j; ch < nchunk; ch += kGnFinLoads * kGnSet) {
    float2 v[kGnFinLoads];
#pragma unroll
    for (int i = 0; i < kGnFinLoads; ++i) {
      const int64_t ci = ch + i * kGnSet;
      v[i] = ci < nchunk ? *reinterpret_cast<const float2*>(base + ci * G * 2) : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kGnFinLoads; ++i) { a += v[i].x; c += v[i].y; }
  }
#pragma unroll
  for (int off = kGnSet / 2; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, kGnSet);
    c += __shfl_xor(c, off, kGnSet);
  }
  return make_double2(a, c);
}

// The fresh sums of every group to stats_out[b, p] (the next step's stale
// sums; alone, the first half of the synchronous step): one group per
// 64-lane workgroup.  Only the statistics-only call runs it.
__global__ __launch_bounds__(kWave) void gn_stats_kernel(const float* __restrict__ partial, int64_t nchunk,
                                                         float* __restrict__ stats_out, int G, int P, int p) {
  const int b = blockIdx.y;
  const int g = blockIdx.x * (kWave / kGnSet) + threadIdx.x / kGnSet, j = threadIdx.x % kGnSet;
  if (g >= G) return;  // uniform within each lane set
  const double2 r = gn_fresh_sums(partial, nchunk, G, b, g, j);
  if (j == 0) {
    float* so = stats_out + ((static_cast<int64_t>(b) * P + p) * G + g) * 2;
    so[0] = static_cast<float>(r.x);
    so[1] = static_cast<float>(r.y);
  }
}

// SiLU z sigmoid(z) = z / (1 + 2^(-z log2 e)): large negative z gives
// z * (1/inf) = -0, large positive z gives z.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// Apply, with the fresh sums formed in the same launch.  A workgroup owns a
// tile of 64 channels (blockIdx.y) of batch entry b (blockIdx.z) and walks
// pixels; it needs the statistics of only the few groups its channels
// touch.  It first issues its first batch of x loads, then
//  1. adds the chunk partials of those groups into their fresh sums, bit for
//     bit as gn_stats_kernel does (task (j, g) adds chunks j, j+64, ... in
//     float64 in increasing order, as gn_fresh_sums' lane j; the 64 lane sums
//     are then added in the order of its xor butterfly, one LDS stage per
//     offset 32, 16, ..., 1), rounded to float32 as stored; the workgroups of
//     pixel block 0 store them to stats_out[b, p] (each group by the tile
//     holding its first channel);
//  2. forms each group's total over patches q in increasing order, in
//     float64, from those fresh sums for q == p and the stale sums for
//     q != p, and the mean/rstd from it -- the same values in every
//     workgroup;
//  3. streams y = x * a_c + b_c (a_c = rstd_g gamma_c, b_c = beta_c - mean_g
//     a_c; then SiLU when asked: the GroupNorm + SiLU pair opening an SDXL
//     residual block) with streaming 16-byte loads and stores.  Each wave
//     access covers whole 128-byte runs of eight pixels.  Pixels go in
//     grid-stride order: workgroup w takes pixels w*KP .. w*KP+KP-1 of every
//     run of gridDim.x*KP consecutive pixels, so the workgroups in flight
//     stream one window of x and y.
constexpr int kGnApplyThreads = 256;
constexpr int kGnApplyWgs = 2560;     // total apply workgroups over B and the channel tiles
constexpr int kGnApplyInFlight = 8;   // 16-byte loads in flight per thread
constexpr int kGnCt = 64;             // channels per workgroup tile
constexpr int kGnCtMaxGroups = kGnCt + 1;  // groups a 64-channel tile can touch
constexpr int kGnFreshBlock = 4;      // groups per fresh-sum block (LDS scratch 64 x 4 double2)
constexpr int kGnQb = 16;             // patches staged per pass

template <typename T, bool SILU>
__global__ __launch_bounds__(kGnApplyThreads) void gn_apply_kernel(
    const T* __restrict__ x, T* __restrict__ y, const float* __restrict__ partial, int64_t nchunk,
    float* __restrict__ stats_out, const float* __restrict__ stale, const float* __restrict__ gamma,
    const float* __restrict__ beta, int64_t npix, int C, int G, int P, int p, double n, float eps) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int VT = kGnCt / VEC;           // vectors per pixel of the tile
  constexpr int KP = kGnApplyThreads / VT;  // pixels per pass
  __shared__ double2 red[kGnSet * kGnFreshBlock];
  __shared__ float2 fresh[kGnCtMaxGroups];
  __shared__ float2 gstat[kGnCtMaxGroups];  // (mean, rstd) per group of the tile
  __shared__ double2 tot[kGnCtMaxGroups];
  __shared__ float2 stage[kGnQb * kGnCtMaxGroups];
  const int b = blockIdx.z;
  const int t = threadIdx.x, nt = blockDim.x;
  const int v = t % VT, k = t / VT;
  const int c0 = blockIdx.y * kGnCt;
  const int cg = C / G;
  const int g_lo = c0 / cg, g_hi = (min(c0 + kGnCt, C) - 1) / cg, ng = g_hi - g_lo + 1;
  const int V = C / VEC;                    // vectors per pixel
  const int vi = c0 / VEC + v;              // this thread's vector within a pixel
  const bool active = k < KP && vi < V;
  const int64_t off = static_cast<int64_t>(b) * npix * V;
  const uint4* xv = reinterpret_cast<const uint4*>(x) + off;
  uint4* yv = reinterpret_cast<uint4*>(y) + off;
  const int64_t step = static_cast<int64_t>(gridDim.x) * KP;
  int64_t pix = static_cast<int64_t>(blockIdx.x) * KP + k;
  uint4 u[kGnApplyInFlight];
  float gm[VEC], bt[VEC];
  // the first batch and the affine parameters do not depend on the
  // statistics: in flight while they form
  if (active) {
#pragma unroll
    for (int q = 0; q < kGnApplyInFlight; ++q)
      if (pix + q * step < npix) u[q] = ld_stream(xv + (pix + q * step) * V + vi);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      gm[e] = gamma[vi * VEC + e];
      bt[e] = beta[vi * VEC + e];
    }
  }
  // 1. fresh sums of groups g_lo .. g_hi
  const float* pbase = partial + static_cast<int64_t>(b) * nchunk * G * 2;
  for (int h0 = 0; h0 < ng; h0 += kGnFreshBlock) {
    const int gb = ng - h0 < kGnFreshBlock ? ng - h0 : kGnFreshBlock;
    for (int q = t; q < kGnSet * gb; q += nt) {
      const int j = q / gb, h = q % gb, g = g_lo + h0 + h;
      double a = 0.0, c = 0.0;
      for (int64_t ch = j; ch < nchunk; ch += kGnFinLoads * kGnSet) {
        float2 pv[kGnFinLoads];
#pragma unroll
        for (int i = 0; i < kGnFinLoads; ++i) {
          const int64_t ci = ch + i * kGnSet;
          pv[i] = ci < nchunk ? *reinterpret_cast<const float2*>(pbase + (ci * G + g) * 2) : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < kGnFinLoads; ++i) { a += pv[i].x; c += pv[i].y; }
      }
      red[j * kGnFreshBlock + h] = make_double2(a, c);
    }
    for (int o = kGnSet / 2; o > 0; o >>= 1) {
      __syncthreads();
      for (int q = t; q < o * gb; q += nt) {
        const int j = q / gb, h = q % gb;
        const double2 r0 = red[j * kGnFreshBlock + h], r1 = red[(j + o) * kGnFreshBlock + h];
        red[j * kGnFreshBlock + h] = make_double2(r0.x + r1.x, r0.y + r1.y);
      }
    }
    __syncthreads();
    for (int h = t; h < gb; h += nt)
      fresh[h0 + h] = make_float2(static_cast<float>(red[h].x), static_cast<float>(red[h].y));
    __syncthreads();
  }
  // 2. totals over the patches, mean and rstd; pixel block 0 stores the fresh
  // sums.  The stale sums are staged in LDS by all threads, kGnQb patches
  // per pass, then added per group in patch order.
  for (int h = t; h < ng; h += nt) {
    const int g = g_lo + h;
    if (blockIdx.x == 0 && g * cg >= c0)
      *reinterpret_cast<float2*>(stats_out + ((static_cast<int64_t>(b) * P + p) * G + g) * 2) = fresh[h];
    tot[h] = make_double2(0.0, 0.0);
  }
  for (int q0 = 0; q0 < P; q0 += kGnQb) {
    const int nq = P - q0 < kGnQb ? P - q0 : kGnQb;
    for (int i = t; i < nq * ng; i += nt) {
      const int q = q0 + i / ng, h = i % ng;
      stage[i] = q == p ? fresh[h]
                        : *reinterpret_cast<const float2*>(stale + ((static_cast<int64_t>(b) * P + q) * G + g_lo + h) * 2);
    }
    __syncthreads();
    for (int h = t; h < ng; h += nt) {
      double2 a = tot[h];
      for (int i = 0; i < nq; ++i) {
        a.x += stage[i * ng + h].x;
        a.y += stage[i * ng + h].y;
      }
      tot[h] = a;
    }
    __syncthreads();
  }
  for (int h = t; h < ng; h += nt) {
    const double mean = tot[h].x / n;
    double var = tot[h].y / n - mean * mean;
    if (var < 0.0) var = 0.0;
    gstat[h] = make_float2(static_cast<float>(mean), static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps))));
  }
  __syncthreads();
  if (!active) return;
  float ac[VEC], sh[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float2 mr = gstat[(vi * VEC + e) / cg - g_lo];
    ac[e] = mr.y * gm[e];
    sh[e] = fmaf(-mr.x, ac[e], bt[e]);
  }
  // 3. stream
  for (;;) {
#pragma unroll
    for (int q = 0; q < kGnApplyInFlight; ++q) {
      const int64_t pq = pix + q * step;
      if (pq < npix) {
        float f[VEC];
        Elem<T>::unpack(u[q], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          f[e] = fmaf(f[e], ac[e], sh[e]);
          if (SILU) f[e] = silu_f(f[e]);
        }
        st_stream(yv + pq * V + vi, Elem<T>::pack(f));
      }
    }
    pix += kGnApplyInFlight * step;
    if (pix >= npix) break;
#pragma unroll
    for (int q = 0; q < kGnApplyInFlight; ++q)
      if (pix + q * step < npix) u[q] = ld_stream(xv + (pix + q * step) * V + vi);
  }
}

// y == NULL: the fresh sums to stats_out[b, p] (gn_stats_kernel).  Else the
// apply, which forms the same sums itself and stores them.
template <typename T>
static hipError_t gn_finish(T* y, float* stats_out, const T* x, const float* partial, int64_t nchunk,
                            const float* stale, const float* gamma, const float* beta, int64_t B, int64_t H, int64_t W,
                            int64_t C, int64_t G, int64_t P, int64_t p, int64_t rows, float eps, bool silu,
                            hipStream_t s) {
  if (y == nullptr) {
    hipLaunchKernelGGL(gn_stats_kernel, dim3(static_cast<unsigned>(ceil_div(G, kWave / kGnSet)),
                                             static_cast<unsigned>(B)),
                       dim3(kWave), 0, s, partial, nchunk, stats_out, static_cast<int>(G), static_cast<int>(P),
                       static_cast<int>(p));
    return hipGetLastError();
  }
  constexpr int KP = kGnApplyThreads / (kGnCt / Elem<T>::kVec);
  const int64_t npix = rows * W;
  const int64_t nct = ceil_div(C, kGnCt);
  int64_t npb = ceil_div(kGnApplyWgs, B * nct);
  const int64_t full = ceil_div(npix, static_cast<int64_t>(KP) * kGnApplyInFlight);  // one full batch per thread
  if (npb > full) npb = full;
  const double n = static_cast<double>(H) * static_cast<double>(W) * static_cast<double>(C / G);
  const dim3 grid(static_cast<unsigned>(npb), static_cast<unsigned>(nct), static_cast<unsigned>(B));
  if (silu)
    hipLaunchKernelGGL((gn_apply_kernel<T, true>), grid, dim3(kGnApplyThreads), 0, s, x, y, partial, nchunk,
                       stats_out, stale, gamma, beta, npix, static_cast<int>(C), static_cast<int>(G),
                       static_cast<int>(P), static_cast<int>(p), n, eps);
  else
    hipLaunchKernelGGL((gn_apply_kernel<T, false>), grid, dim3(kGnApplyThreads), 0, s, x, y, partial, nchunk,
                       stats_out, stale, gamma, beta, npix, static_cast<int>(C), static_cast<int>(G),
                       static_cast<int>(P), static_cast<int>(p), n, eps);
  return hipGetLastError();
}

template <typename T>
static hipError_t gn_run(T* y, float* stats_out, const T* x, const float* stale, const float* gamma,
                         const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P,
                         int64_t p, int64_t rows, float eps, void* ws, bool silu, hipStream_t s) {
  const GnGeom g = gn_geom(B, rows, W, C, sizeof(T) == 2);
  float* partial = static_cast<float*>(ws);
  hipLaunchKernelGGL(gn_partial_kernel<T>, dim3(static_cast<unsigned>(g.nstat), static_cast<unsigned>(B)),
                     dim3(g.threads), 0, s, x, partial, g.npix, static_cast<int>(C), static_cast<int>(G), g.V, g.KP,
                     g.stat_ppc, g.nstat);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return gn_finish(y, stats_out, x, partial, g.nstat, stale, gamma, beta, B, H, W, C, G, P, p, rows, eps, silu, s);
}

// Fresh sums from a producer's partials: one kernel (or the statistics-only
// one), x read once.
hipError_t launch_groupnorm_presummed(void* y, float* stats_out, const void* x, const float* partials, int64_t nchunk,
                                      const float* stale_stats, const float* gamma, const float* beta, int64_t B,
                                      int64_t H, int64_t W, int64_t C, int64_t G, int64_t P, int64_t p, int64_t rows,
                                      float eps, bool bf16, bool silu, hipStream_t s) {
  if (bf16)
    return gn_finish(static_cast<uint16_t*>(y), stats_out, static_cast<const uint16_t*>(x), partials, nchunk,
                     stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, silu, s);
  return gn_finish(static_cast<float*>(y), stats_out, static_cast<const float*>(x), partials, nchunk, stale_stats,
                   gamma, beta, B, H, W, C, G, P, p, rows, eps, silu, s);
}

hipError_t launch_groupnorm(void* y, float* stats_out, const void* x, const float* stale_stats, const float* gamma,
                            const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P,
                            int64_t p, int64_t rows, float eps, void* ws, bool bf16, bool silu, hipStream_t s) {
  if (bf16)
    return gn_run(static_cast<uint16_t*>(y), stats_out, static_cast<const uint16_t*>(x), stale_stats, gamma, beta, B,
                  H, W, C, G, P, p, rows, eps, ws, silu, s);
  return gn_run(static_cast<float*>(y), stats_out, static_cast<const float*>(x), stale_stats, gamma, beta, B, H, W, C,
                G, P, p, rows, eps, ws, silu, s);
}

}  // namespace dpp
