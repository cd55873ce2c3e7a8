// C ABI of libdpp: argument validation on the host, then the launch
// sequence of each call on the caller's stream.  No call allocates, frees,
// synchronises or keeps state.  Validation runs before any HIP call, so an
// invalid call returns its error code without touching the device.
#include "../../include/dpp.h"
#include "dpp_common.h"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int esize_of(int dtype) { return dtype == DPP_BF16 ? 2 : 4; }

// Byte ranges [lo, hi) overlap?
inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? DPP_OK : DPP_ERR_LAUNCH; }

inline bool bad_dtype(int dtype) { return dtype != DPP_BF16 && dtype != DPP_F32; }

}  // namespace

extern "C" {

const char* dpp_strerror(int status) {
  switch (status) {
    case DPP_OK: return "DPP_OK";
    case DPP_ERR_NULL: return "DPP_ERR_NULL: required pointer is NULL";
    case DPP_ERR_SHAPE: return "DPP_ERR_SHAPE: invalid sizes";
    case DPP_ERR_DTYPE: return "DPP_ERR_DTYPE: unknown dtype";
    case DPP_ERR_ALIGN: return "DPP_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case DPP_ERR_ALIAS: return "DPP_ERR_ALIAS: output overlaps an input";
    case DPP_ERR_WORKSPACE: return "DPP_ERR_WORKSPACE: workspace missing or too small";
    case DPP_ERR_UNSUPPORTED: return "DPP_ERR_UNSUPPORTED: no kernel for this shape/dtype";
    case DPP_ERR_LAUNCH: return "DPP_ERR_LAUNCH: kernel launch failed";
    default: return "DPP: unknown status";
  }
}

int dpp_version(void) { return DPP_VERSION; }

// ------------------------------------------------------------------ a1
int dpp_splice_patch(void* full, const void* patch, int64_t B, int64_t H, int64_t W, int64_t C, int64_t row0,
                     int64_t rows, int dtype, void* stream) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!full || !patch) return DPP_ERR_NULL;
  if (B <= 0 || H <= 0 || W <= 0 || C <= 0 || rows <= 0 || row0 < 0 || row0 + rows > H) return DPP_ERR_SHAPE;
  if (B > 65535) return DPP_ERR_UNSUPPORTED;
  const int es = esize_of(dtype);
  if (overlap(full, B * H * W * C * es, patch, B * rows * W * C * es)) return DPP_ERR_ALIAS;
  return launch_status(dpp::launch_splice(full, patch, B, H, W, C, row0, rows, es, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ a2
size_t dpp_groupnorm_stale_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t C, int64_t G) {
  if (B <= 0 || rows <= 0 || W <= 0 || C <= 0 || G <= 0 || C % G != 0 || C % 4 != 0) return 0;
  return dpp::gn_workspace_bytes(B, rows, W, C, G);
}

}  // extern "C"

namespace {
// Every check of a GroupNorm call except those of its workspace.
int groupnorm_validate(void* y, float* stats_out, const void* x, const float* stale_stats, const float* gamma,
                       const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P, int64_t p,
                       int64_t rows, float eps, int dtype) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!x || !stats_out) return DPP_ERR_NULL;
  if (y && (!gamma || !beta)) return DPP_ERR_NULL;
  if (y && P > 1 && !stale_stats) return DPP_ERR_NULL;
  if (B <= 0 || H <= 0 || W <= 0 || C <= 0 || G <= 0 || P <= 0 || rows <= 0 || rows > H || p < 0 || p >= P ||
      C % G != 0 || !(eps >= 0.f))
    return DPP_ERR_SHAPE;
  const int vec = dtype == DPP_BF16 ? 8 : 4;
  if (C % vec != 0 || C / vec > 256 || G > 256 || B > 65535) return DPP_ERR_UNSUPPORTED;
  if (!aligned16(x) || (y && !aligned16(y))) return DPP_ERR_ALIGN;
  const int es = esize_of(dtype);
  const int64_t act = B * rows * W * C * es;
  const int64_t st = B * P * G * 2 * 4;
  if (overlap(stats_out, st, x, act)) return DPP_ERR_ALIAS;
  if (stale_stats && overlap(stats_out, st, stale_stats, st)) return DPP_ERR_ALIAS;
  if (y && (overlap(y, act, x, act) || overlap(y, act, stats_out, st))) return DPP_ERR_ALIAS;
  if (y && stale_stats && overlap(y, act, stale_stats, st)) return DPP_ERR_ALIAS;
  return DPP_OK;
}

int groupnorm_call(void* y, float* stats_out, const void* x, const float* stale_stats, const float* gamma,
                   const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P, int64_t p,
                   int64_t rows, float eps, void* workspace, size_t workspace_bytes, int dtype, bool silu,
                   void* stream) {
  const int rc = groupnorm_validate(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, dtype);
  if (rc != DPP_OK) return rc;
  const int es = esize_of(dtype);
  const int64_t act = B * rows * W * C * es;
  const int64_t st = B * P * G * 2 * 4;
  const size_t need = dpp::gn_workspace_bytes(B, rows, W, C, G);
  if (!workspace || workspace_bytes < need) return DPP_ERR_WORKSPACE;
  if (overlap(workspace, static_cast<int64_t>(need), x, act) || overlap(workspace, static_cast<int64_t>(need), stats_out, st) ||
      (y && overlap(workspace, static_cast<int64_t>(need), y, act)))
    return DPP_ERR_ALIAS;
  return launch_status(dpp::launch_groupnorm(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps,
                                             workspace, dtype == DPP_BF16, silu, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

int dpp_groupnorm_stale(void* y, float* stats_out, const void* x, const float* stale_stats, const float* gamma,
                        const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P, int64_t p,
                        int64_t rows, float eps, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  return groupnorm_call(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, workspace,
                        workspace_bytes, dtype, false, stream);
}

int dpp_groupnorm_silu_stale(void* y, float* stats_out, const void* x, const float* stale_stats, const float* gamma,
                             const float* beta, int64_t B, int64_t H, int64_t W, int64_t C, int64_t G, int64_t P,
                             int64_t p, int64_t rows, float eps, void* workspace, size_t workspace_bytes, int dtype,
                             void* stream) {
  return groupnorm_call(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, workspace,
                        workspace_bytes, dtype, true, stream);
}

int dpp_groupnorm_stale_presummed(void* y, float* stats_out, const void* x, const float* partials, int64_t nchunk,
                                  const float* stale_stats, const float* gamma, const float* beta, int64_t B,
                                  int64_t H, int64_t W, int64_t C, int64_t G, int64_t P, int64_t p, int64_t rows,
                                  float eps, int silu, int dtype, void* stream) {
  const int rc = groupnorm_validate(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, dtype);
  if (rc != DPP_OK) return rc;
  if (!partials) return DPP_ERR_NULL;
  if (nchunk <= 0 || nchunk > (1LL << 30)) return DPP_ERR_SHAPE;
  const int es = esize_of(dtype);
  const int64_t act = B * rows * W * C * es;
  const int64_t st = B * P * G * 2 * 4;
  const int64_t pb = B * nchunk * G * 2 * 4;
  if (overlap(stats_out, st, partials, pb) || (y && overlap(y, act, partials, pb))) return DPP_ERR_ALIAS;
  return launch_status(dpp::launch_groupnorm_presummed(y, stats_out, x, partials, nchunk, stale_stats, gamma, beta, B,
                                                       H, W, C, G, P, p, rows, eps, dtype == DPP_BF16, silu != 0,
                                                       static_cast<hipStream_t>(stream)));
}

int dpp_groupnorm_stale_noalloc(void* y, float* stats_out, const void* x, const float* stale_stats,
                                const float* gamma, const float* beta, int64_t B, int64_t H, int64_t W, int64_t C,
                                int64_t G, int64_t P, int64_t p, int64_t rows, float eps, int dtype, void* stream) {
  const int rc = groupnorm_validate(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps, dtype);
  if (rc != DPP_OK) return rc;
  // the shape's scratch must fit the library's static array
  static_assert(DPP_GN_NOALLOC_MAX_BYTES == (1u << 20), "header limit and scratch size agree");
  if (dpp::gn_workspace_bytes(B, rows, W, C, G) > dpp::gn_scratch_bytes()) return DPP_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (dpp::gn_scratch_ptr(&scratch) != hipSuccess) return DPP_ERR_LAUNCH;
  return launch_status(dpp::launch_groupnorm(y, stats_out, x, stale_stats, gamma, beta, B, H, W, C, G, P, p, rows, eps,
                                             scratch, dtype == DPP_BF16, false, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ a3
size_t dpp_conv3x3_halo_workspace_bytes(int64_t B, int64_t rows, int64_t W, int64_t Cin, int64_t Cout) {
  if (B <= 0 || rows <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || Cin % 64 != 0 || Cout % 16 != 0) return 0;
  return dpp::conv_workspace_bytes(B, rows, W, Cin, Cout);
}

int dpp_conv3x3_halo(void* y, const void* x, const void* stale_full, const void* weight, const float* bias, int64_t B,
                     int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows, int dtype,
                     void* stream) {
  return dpp_conv3x3_halo_ws(y, x, stale_full, weight, bias, B, H, W, Cin, Cout, row0, rows, nullptr, 0, dtype,
                             stream);
}

}  // extern "C"

namespace {
// Every check of a conv call except those of its workspace.
int conv_validate(void* y, const void* x, const void* stale_full, const void* weight, const float* bias, int64_t B,
                  int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows, int dtype) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!y || !x || !weight) return DPP_ERR_NULL;
  if (B <= 0 || H <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || rows <= 0 || row0 < 0 || row0 + rows > H)
    return DPP_ERR_SHAPE;
  const bool needs_stale = row0 > 0 || row0 + rows < H;
  if (needs_stale && !stale_full) return DPP_ERR_NULL;
  if (B > 65535 || W > (1 << 24) || H > (1 << 24) || Cin > (1 << 20) || Cout > (1 << 20)) return DPP_ERR_UNSUPPORTED;
  if (dtype == DPP_BF16) {
    if (Cin % 64 != 0 || Cout % 16 != 0) return DPP_ERR_UNSUPPORTED;
    // weight byte offsets (rows padded to a multiple of 128) and byte offsets
    // within one band row (W + 2 pixels) are 32-bit
    if ((Cout + 128) * 9 * Cin * 2 > 0x7fffffffLL) return DPP_ERR_UNSUPPORTED;
    if ((W + 2) * Cin * 2 > 0x7fffffffLL) return DPP_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(y) || !aligned16(weight) || (stale_full && !aligned16(stale_full)))
      return DPP_ERR_ALIGN;
  }
  const int es = esize_of(dtype);
  const int64_t ybytes = B * rows * W * Cout * es;
  if (overlap(y, ybytes, x, B * rows * W * Cin * es) || overlap(y, ybytes, weight, Cout * 9 * Cin * es) ||
      (stale_full && overlap(y, ybytes, stale_full, B * H * W * Cin * es)) || (bias && overlap(y, ybytes, bias, Cout * 4)))
    return DPP_ERR_ALIAS;
  return DPP_OK;
}
}  // namespace

extern "C" {

int dpp_conv3x3_halo_ws(void* y, const void* x, const void* stale_full, const void* weight, const float* bias,
                        int64_t B, int64_t H, int64_t W, int64_t Cin, int64_t Cout, int64_t row0, int64_t rows,
                        void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  const int rc = conv_validate(y, x, stale_full, weight, bias, B, H, W, Cin, Cout, row0, rows, dtype);
  if (rc != DPP_OK) return rc;
  const int es = esize_of(dtype);
  const int64_t ybytes = B * rows * W * Cout * es;
  if (workspace && workspace_bytes > 0) {
    const int64_t wb = static_cast<int64_t>(workspace_bytes);
    if (!aligned16(workspace)) return DPP_ERR_ALIGN;
    if (overlap(workspace, wb, y, ybytes) || overlap(workspace, wb, x, B * rows * W * Cin * es) ||
        overlap(workspace, wb, weight, Cout * 9 * Cin * es) ||
        (stale_full && overlap(workspace, wb, stale_full, B * H * W * Cin * es)) ||
        (bias && overlap(workspace, wb, bias, Cout * 4)))
      return DPP_ERR_ALIAS;
  }
  return launch_status(dpp::launch_conv3x3(y, x, stale_full, weight, bias, B, H, W, Cin, Cout, row0, rows, workspace,
                                           workspace_bytes, dtype == DPP_BF16, static_cast<hipStream_t>(stream)));
}

int64_t dpp_conv3x3_halo_gn_chunks(int64_t rows, int64_t W, int64_t Cout) {
  if (rows <= 0 || W <= 0 || Cout <= 0) return 0;
  return dpp::conv_gn_chunks(rows, W, Cout);
}

int dpp_conv3x3_halo_gn(void* y, float* gn_partials, int64_t G, const void* x, const void* stale_full,
                        const void* weight, const float* bias, int64_t B, int64_t H, int64_t W, int64_t Cin,
                        int64_t Cout, int64_t row0, int64_t rows, int dtype, void* stream) {
  const int rc = conv_validate(y, x, stale_full, weight, bias, B, H, W, Cin, Cout, row0, rows, dtype);
  if (rc != DPP_OK) return rc;
  if (!gn_partials) return DPP_ERR_NULL;
  if (G <= 0 || Cout % G != 0) return DPP_ERR_SHAPE;
  if (dtype != DPP_BF16) return DPP_ERR_UNSUPPORTED;
  const int64_t pbytes = B * dpp::conv_gn_chunks(rows, W, Cout) * G * 2 * 4;
  const int64_t ybytes = B * rows * W * Cout * 2;
  if (overlap(gn_partials, pbytes, y, ybytes) || overlap(gn_partials, pbytes, x, B * rows * W * Cin * 2) ||
      overlap(gn_partials, pbytes, weight, Cout * 9 * Cin * 2) ||
      (stale_full && overlap(gn_partials, pbytes, stale_full, B * H * W * Cin * 2)) ||
      (bias && overlap(gn_partials, pbytes, bias, Cout * 4)))
    return DPP_ERR_ALIAS;
  return launch_status(dpp::launch_conv3x3(y, x, stale_full, weight, bias, B, H, W, Cin, Cout, row0, rows, nullptr, 0,
                                           true, static_cast<hipStream_t>(stream), gn_partials, static_cast<int>(G)));
}

// ------------------------------------------------------------------ a4
size_t dpp_self_attn_workspace_bytes(int64_t B, int64_t n_q, int64_t n_kv, int64_t heads, int64_t head_dim, int dtype) {
  if (B <= 0 || n_q <= 0 || n_kv <= 0 || heads <= 0 || head_dim <= 0 || bad_dtype(dtype)) return 0;
  return dpp::attn_workspace_bytes(B, n_q, n_kv, heads, head_dim, dtype == DPP_BF16);
}

int dpp_self_attn_displaced(void* o, const void* q, const void* k, const void* v, int64_t B, int64_t n_q, int64_t n_kv,
                            int64_t heads, int64_t head_dim, int64_t ld_q, int64_t ld_kv, int64_t ld_o, float scale,
                            void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!o || !q || !k || !v) return DPP_ERR_NULL;
  if (B <= 0 || n_q <= 0 || n_kv <= 0 || heads <= 0 || head_dim <= 0) return DPP_ERR_SHAPE;
  const int64_t hd = heads * head_dim;
  if (ld_q < hd || ld_kv < hd || ld_o < hd) return DPP_ERR_SHAPE;
  if (B * heads > 65535 || n_q > (1LL << 30) || n_kv > (1LL << 30)) return DPP_ERR_UNSUPPORTED;
  // bf16 grid: 256-query tiles x B*heads x up to 16 key splits, one int32 id each
  if (((n_q + 255) / 256) * B * heads * 16 > 0x7fffffffLL) return DPP_ERR_UNSUPPORTED;
  if (dtype == DPP_BF16) {
    if (head_dim != 64) return DPP_ERR_UNSUPPORTED;
    if (ld_q > (1LL << 24) || ld_kv > (1LL << 24) || ld_o > (1LL << 24)) return DPP_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ld_q % 8 || ld_kv % 8 || ld_o % 8)
      return DPP_ERR_ALIGN;
  } else if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128) {
    return DPP_ERR_UNSUPPORTED;
  }
  const int es = esize_of(dtype);
  const int64_t obytes = B * n_q * ld_o * es;
  const int64_t kvbytes = B * n_kv * ld_kv * es;
  if (overlap(o, obytes, q, B * n_q * ld_q * es) || overlap(o, obytes, k, kvbytes) || overlap(o, obytes, v, kvbytes))
    return DPP_ERR_ALIAS;
  if (workspace && workspace_bytes > 0) {
    const int64_t wb = static_cast<int64_t>(workspace_bytes);
    if (overlap(workspace, wb, o, obytes) || overlap(workspace, wb, q, B * n_q * ld_q * es) ||
        overlap(workspace, wb, k, kvbytes) || overlap(workspace, wb, v, kvbytes))
      return DPP_ERR_ALIAS;
  }
  if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(head_dim));
  return launch_status(dpp::launch_attention(o, q, k, v, B, n_q, n_kv, heads, head_dim, ld_q, ld_kv, ld_o, scale,
                                             workspace, workspace ? workspace_bytes : 0, dtype == DPP_BF16,
                                             static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ projections
}  // extern "C"

namespace {
int linear_validate(void* y, const void* x, const void* w, const float* bias, int64_t B, int64_t M, int64_t K,
                    int64_t N, int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, int dtype) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!y || !x || !w) return DPP_ERR_NULL;
  if (B <= 0 || M <= 0 || K <= 0 || N <= 0 || ld_x < K || ld_y < N || bs_x < 0 || bs_y < 0) return DPP_ERR_SHAPE;
  // batches of the output must not overlap one another
  if (B > 1 && bs_y < (M - 1) * ld_y + N) return DPP_ERR_SHAPE;
  if (B > 65535 || M > (1LL << 30) || N > (1LL << 30) || K > (1LL << 30)) return DPP_ERR_UNSUPPORTED;
  if (dtype == DPP_BF16) {
    if (K % 8 != 0 || N % 4 != 0) return DPP_ERR_UNSUPPORTED;
    // the kernel addresses w and one batch entry of x with 32-bit byte offsets
    // (rows padded to its tile of up to 256 channels x 160 tokens, plus the
    // last K slice; 0x7ffffff0 marks rows past M)
    if ((N + 256) * K * 2 + 128 > 0x7fffffffLL || ((M + 160) * ld_x + K) * 2 > 0x7fffffefLL)
      return DPP_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || (reinterpret_cast<uintptr_t>(y) & 7u) || ld_x % 8 || bs_x % 8 ||
        ld_y % 4 || bs_y % 4)
      return DPP_ERR_ALIGN;
  }
  const int es = esize_of(dtype);
  const int64_t xbytes = ((B - 1) * bs_x + (M - 1) * ld_x + K) * es;
  const int64_t ybytes = ((B - 1) * bs_y + (M - 1) * ld_y + N) * es;
  const int64_t wbytes = N * K * es;
  if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, w, wbytes) || (bias && overlap(y, ybytes, bias, N * 4)))
    return DPP_ERR_ALIAS;
  return DPP_OK;
}
}  // namespace

extern "C" {

int dpp_linear(void* y, const void* x, const void* w, const float* bias, int64_t B, int64_t M, int64_t K, int64_t N,
               int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, int dtype, void* stream) {
  const int rc = linear_validate(y, x, w, bias, B, M, K, N, ld_x, bs_x, ld_y, bs_y, dtype);
  if (rc != DPP_OK) return rc;
  return launch_status(dpp::launch_linear(y, x, w, bias, B, M, K, N, ld_x, bs_x, ld_y, bs_y, dtype == DPP_BF16,
                                          static_cast<hipStream_t>(stream)));
}

int64_t dpp_linear_gn_chunks(int64_t B, int64_t M, int64_t N) {
  if (B <= 0 || M <= 0 || N <= 0) return 0;
  return dpp::linear_gn_chunks(B, M, N);
}

int dpp_linear_gn(void* y, float* gn_partials, int64_t G, const void* x, const void* w, const float* bias, int64_t B,
                  int64_t M, int64_t K, int64_t N, int64_t ld_x, int64_t bs_x, int64_t ld_y, int64_t bs_y, int dtype,
                  void* stream) {
  const int rc = linear_validate(y, x, w, bias, B, M, K, N, ld_x, bs_x, ld_y, bs_y, dtype);
  if (rc != DPP_OK) return rc;
  if (!gn_partials) return DPP_ERR_NULL;
  if (G <= 0 || N % G != 0) return DPP_ERR_SHAPE;
  if (dtype != DPP_BF16) return DPP_ERR_UNSUPPORTED;
  const int64_t pbytes = B * dpp::linear_gn_chunks(B, M, N) * G * 2 * 4;
  if (overlap(gn_partials, pbytes, y, ((B - 1) * bs_y + (M - 1) * ld_y + N) * 2) ||
      overlap(gn_partials, pbytes, x, ((B - 1) * bs_x + (M - 1) * ld_x + K) * 2) ||
      overlap(gn_partials, pbytes, w, N * K * 2) || (bias && overlap(gn_partials, pbytes, bias, N * 4)))
    return DPP_ERR_ALIAS;
  return launch_status(dpp::launch_linear(y, x, w, bias, B, M, K, N, ld_x, bs_x, ld_y, bs_y, true,
                                          static_cast<hipStream_t>(stream), gn_partials, static_cast<int>(G)));
}

// ------------------------------------------------------------------ a5
size_t dpp_cfg_combine_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return dpp::cfg_workspace_bytes(n);
}

int dpp_cfg_combine_relmae(void* eps, float* relmae, const void* eps_c, const void* eps_u, int64_t n, float guidance,
                           void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (bad_dtype(dtype)) return DPP_ERR_DTYPE;
  if (!eps || !eps_c || !eps_u) return DPP_ERR_NULL;
  if (n <= 0) return DPP_ERR_SHAPE;
  const int es = esize_of(dtype);
  const int64_t nb = n * es;
  if ((eps != eps_c && overlap(eps, nb, eps_c, nb)) || (eps != eps_u && overlap(eps, nb, eps_u, nb)))
    return DPP_ERR_ALIAS;
  if (relmae) {
    const size_t need = dpp::cfg_workspace_bytes(n);
    if (!workspace || workspace_bytes < need) return DPP_ERR_WORKSPACE;
    const int64_t wb = static_cast<int64_t>(need);
    if (overlap(workspace, wb, eps, nb) || overlap(workspace, wb, eps_c, nb) || overlap(workspace, wb, eps_u, nb) ||
        overlap(relmae, 4, eps, nb) || overlap(relmae, 4, workspace, wb))
      return DPP_ERR_ALIAS;
  }
  return launch_status(dpp::launch_cfg(eps, relmae, eps_c, eps_u, n, guidance, workspace, dtype == DPP_BF16,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
