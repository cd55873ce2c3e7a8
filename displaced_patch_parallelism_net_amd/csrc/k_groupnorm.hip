// a2 -- GroupNorm of one patch with statistics corrected by stale sums.
//
// DistriGroupNorm (DistriFusion architecture article, normalisation section):
// the group statistics are those of the spliced image -- the other patches'
// raw sums (sum x, sum x^2) from the previous step plus the own patch's fresh
// sums (DistriFusion reading notes, Introduction, fourth paragraph).
//
// Three launches, all deterministic (no atomics):
//   1. partial: workgroup (chunk, b) sums its pixels per channel in float32
//      registers (each thread owns one 16-byte channel vector and walks
//      pixels, eight loads in flight), folds channels into groups through LDS in a fixed order and
//      writes one (s1, s2) per group to the workspace;
//   2. finalize: one wave per (group, b) adds the chunk partials in float64
//      (fixed order), adds the other patches' stale sums, writes the fresh
//      sums to stats_out[b,p] and mean/rstd to the workspace;
//   3. apply: y = x * a_c + b_c with a_c = rstd_g gamma_c, b_c = beta_c -
//      mean_g a_c (then SiLU when asked: the GroupNorm + SiLU pair opening
//      an SDXL residual block); one 16-byte load and one streaming store per
//      vector.
// The second read of x (step 3) normally hits the 256 MB last-level cache.
#include <mutex>

#include "dpp_common.h"

// Scratch of the allocation-free GroupNorm entry point (chunk partial sums
// and per-group mean/rstd, exactly the workspace the other entry points take
// from the caller).  Each GPU the library runs on holds its own copy until
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
constexpr int kGnApplyChunks = 1024;  // total apply workgroups (over B)
constexpr int kGnInFlight = 8;        // 16-byte loads in flight per thread

struct GnGeom {
  int vec;      // elements per 16-byte vector
  int V;        // vectors per pixel = C / vec
  int KP;       // pixels walked in parallel per workgroup
  int threads;  // KP * V
  int64_t npix;
  int64_t nstat, stat_ppc;    // partial chunks per b, pixels per chunk
  int64_t napply, apply_ppc;  // apply chunks per b, pixels per chunk
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
  int64_t want = ceil_div(kGnStatChunks, B);
  g.nstat = want < maxc ? want : maxc;
  if (g.nstat < 1) g.nstat = 1;
  g.stat_ppc = ceil_div(g.npix, g.nstat);
  g.nstat = ceil_div(g.npix, g.stat_ppc);
  want = ceil_div(kGnApplyChunks, B);
  g.napply = want < maxc ? want : maxc;
  if (g.napply < 1) g.napply = 1;
  g.apply_ppc = ceil_div(g.npix, g.napply);
  g.napply = ceil_div(g.npix, g.apply_ppc);
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
  return static_cast<size_t>(B * nstat * G * 2 + B * G * 2) * sizeof(float);
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

// Finalize: one wave per (group g, batch entry b).  Lane l sums chunks l,
// l + 64, ... of the group's partials in float64 (kGnFinLoads loads issued
// before they are summed, then a remainder loop) and, issued with the first
// of them, the stale sums of patches l, l + 64, ... other than p; two fixed
// xor butterflies add the lanes (every lane ends with the same totals); lane
// 0 writes the fresh sums and (mean, rstd).  Deterministic, no atomics.
constexpr int kGnFinLoads = 8;

__global__ __launch_bounds__(kWave) void gn_finalize_kernel(
    const float* __restrict__ partial, int64_t nchunk, const float* __restrict__ stale, float* __restrict__ stats_out,
    float* __restrict__ coef, int G, int P, int p, double n, float eps) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int l = threadIdx.x;
  const float* base = partial + (static_cast<int64_t>(b) * nchunk * G + g) * 2;
  double sa = 0.0, sc = 0.0;  // stale sums of the other patches
  if (stale != nullptr && coef != nullptr)
    for (int q = l; q < P; q += kWave)
      if (q != p) {
        const float2 st = *reinterpret_cast<const float2*>(stale + ((static_cast<int64_t>(b) * P + q) * G + g) * 2);
        sa += st.x;
        sc += st.y;
      }
  double a = 0.0, c = 0.0;
  int64_t ch = l;
  for (; ch + (kGnFinLoads - 1) * kWave < nchunk; ch += kGnFinLoads * kWave) {
    float2 v[kGnFinLoads];
#pragma unroll
    for (int j = 0; j < kGnFinLoads; ++j) v[j] = *reinterpret_cast<const float2*>(base + (ch + j * kWave) * G * 2);
#pragma unroll
    for (int j = 0; j < kGnFinLoads; ++j) { a += v[j].x; c += v[j].y; }
  }
  for (; ch < nchunk; ch += kWave) {
    const float2 v = *reinterpret_cast<const float2*>(base + ch * G * 2);
    a += v.x;
    c += v.y;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, kWave);
    c += __shfl_xor(c, off, kWave);
    sa += __shfl_xor(sa, off, kWave);
    sc += __shfl_xor(sc, off, kWave);
  }
  if (l != 0) return;
  float* so = stats_out + ((static_cast<int64_t>(b) * P + p) * G + g) * 2;
  so[0] = static_cast<float>(a);
  so[1] = static_cast<float>(c);
  if (coef == nullptr) return;
  const double T1 = a + sa, T2 = c + sc;
  const double mean = T1 / n;
  double var = T2 / n - mean * mean;
  if (var < 0.0) var = 0.0;
  const double rstd = 1.0 / sqrt(var + static_cast<double>(eps));
  coef[(static_cast<int64_t>(b) * G + g) * 2] = static_cast<float>(mean);
  coef[(static_cast<int64_t>(b) * G + g) * 2 + 1] = static_cast<float>(rstd);
}

// SiLU z sigmoid(z) = z / (1 + 2^(-z log2 e)): large negative z gives
// z * (1/inf) = -0, large positive z gives z.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

template <typename T, bool SILU>
__global__ __launch_bounds__(kGnMaxThreads) void gn_apply_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                                 const float* __restrict__ coef,
                                                                 const float* __restrict__ gamma,
                                                                 const float* __restrict__ beta, int64_t npix, int C,
                                                                 int G, int V, int KP, int64_t ppc) {
  constexpr int VEC = Elem<T>::kVec;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int v = t % V, k = t / V;
  if (k >= KP) return;
  const int cg = C / G;
  float a[VEC], sh[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int c = v * VEC + j;
    const int g = c / cg;
    const float mean = coef[(b * G + g) * 2], rstd = coef[(b * G + g) * 2 + 1];
    a[j] = rstd * gamma[c];
    sh[j] = fmaf(-mean, a[j], beta[c]);
  }
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * ppc;
  const int64_t p1 = (p0 + ppc < npix) ? p0 + ppc : npix;
  const int64_t off = static_cast<int64_t>(b) * npix * V;
  const uint4* xv = reinterpret_cast<const uint4*>(x) + off;
  uint4* yv = reinterpret_cast<uint4*>(y) + off;
  int64_t pix = p0 + k;
  for (; pix + (kGnInFlight - 1) * KP < p1; pix += kGnInFlight * KP) {
    uint4 u[kGnInFlight];
#pragma unroll
    for (int q = 0; q < kGnInFlight; ++q) u[q] = xv[(pix + q * KP) * V + v];
#pragma unroll
    for (int q = 0; q < kGnInFlight; ++q) {
      float f[VEC];
      Elem<T>::unpack(u[q], f);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        f[j] = fmaf(f[j], a[j], sh[j]);
        if (SILU) f[j] = silu_f(f[j]);
      }
      st_stream(yv + (pix + q * KP) * V + v, Elem<T>::pack(f));
    }
  }
  for (; pix < p1; pix += KP) {
    float f0[VEC];
    Elem<T>::unpack(xv[pix * V + v], f0);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      f0[j] = fmaf(f0[j], a[j], sh[j]);
      if (SILU) f0[j] = silu_f(f0[j]);
    }
    st_stream(yv + pix * V + v, Elem<T>::pack(f0));
  }
}

template <typename T>
static hipError_t gn_run(T* y, float* stats_out, const T* x, const float* stale, const float* gamma,
                         const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P,
                         int64_t p, int64_t rows, float eps, void* ws, bool silu, hipStream_t s) {
  const GnGeom g = gn_geom(B, rows, W, C, sizeof(T) == 2);
  float* partial = static_cast<float*>(ws);
  float* coef = partial + B * g.nstat * G * 2;
  hipLaunchKernelGGL(gn_partial_kernel<T>, dim3(static_cast<unsigned>(g.nstat), static_cast<unsigned>(B)),
                     dim3(g.threads), 0, s, x, partial, g.npix, static_cast<int>(C), static_cast<int>(G), g.V, g.KP,
                     g.stat_ppc, g.nstat);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const double n = static_cast<double>(H) * static_cast<double>(W) * static_cast<double>(C / G);
  hipLaunchKernelGGL(gn_finalize_kernel, dim3(static_cast<unsigned>(G), static_cast<unsigned>(B)), dim3(kWave), 0, s,
                     partial, g.nstat,
                     stale, stats_out, y ? coef : nullptr, static_cast<int>(G), static_cast<int>(P),
                     static_cast<int>(p), n, eps);
  err = hipGetLastError();
  if (err != hipSuccess || y == nullptr) return err;
  const dim3 agrid(static_cast<unsigned>(g.napply), static_cast<unsigned>(B));
  if (silu)
    hipLaunchKernelGGL((gn_apply_kernel<T, true>), agrid, dim3(g.threads), 0, s, x, y, coef, gamma, beta, g.npix,
                       static_cast<int>(C), static_cast<int>(G), g.V, g.KP, g.apply_ppc);
  else
    hipLaunchKernelGGL((gn_apply_kernel<T, false>), agrid, dim3(g.threads), 0, s, x, y, coef, gamma, beta, g.npix,
                       static_cast<int>(C), static_cast<int>(G), g.V, g.KP, g.apply_ppc);
  return hipGetLastError();
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
