/*
 * Plain-C use of the library's C ABI, with no Python and no PyTorch: device
 * buffers from the HIP runtime API, calls through include/dpp.h, results
 * checked on the host.  Built by displaced_patch_parallelism_net_amd/build.py
 * (gcc, C11) and run by tests/test_gpu_capi.py; prints "capi ok" on success.
 *
 * Checks:
 *  - dpp_version / dpp_strerror;
 *  - an invalid call returns its error code and launches nothing;
 *  - dpp_splice_patch on bf16 bits: the patch rows replaced, every other
 *    element unchanged (bit-exact);
 *  - dpp_cfg_combine_relmae on float32: eps = u + w (c - u) elementwise and
 *    rel-MAE = sum|c - u| / sum|u|, against a double-precision host loop;
 *  - dpp_conv3x3_halo_ws on bf16 with the workspace its query asks for (a
 *    shape whose input channels are split): the halo rows from the stale
 *    image, against a double-precision host loop over the same bf16 values;
 *  - the calls run on a caller-created stream passed as void*.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dpp.h"

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
      return 1;                                                           \
    }                                                                     \
  } while (0)

#define CHECK(cond, ...)              \
  do {                                \
    if (!(cond)) {                    \
      fprintf(stderr, __VA_ARGS__);   \
      fprintf(stderr, "\n");          \
      return 1;                       \
    }                                 \
  } while (0)

/* xorshift32: a small deterministic host generator */
static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}
static float next_f(void) { return (float)(next_u32() & 0xffffff) / 16777216.0f * 2.0f - 1.0f; }

/* bf16 <-> float: round to nearest even (finite values only) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int main(void) {
  printf("dpp_version %d\n", dpp_version());
  CHECK(dpp_strerror(DPP_ERR_SHAPE) != NULL, "dpp_strerror returned NULL");

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  /* ---- error path: NULL operand, nothing launched ---- */
  CHECK(dpp_splice_patch(NULL, NULL, 1, 4, 4, 8, 0, 2, DPP_BF16, stream) == DPP_ERR_NULL,
        "NULL splice did not return DPP_ERR_NULL");

  /* ---- splice: B=2, H=12, W=10, C=64, rows [4, 8) ---- */
  const int64_t B = 2, H = 12, W = 10, C = 64, row0 = 4, rows = 4;
  const size_t nfull = (size_t)(B * H * W * C), npatch = (size_t)(B * rows * W * C);
  uint16_t* hfull = (uint16_t*)malloc(nfull * 2);
  uint16_t* hpatch = (uint16_t*)malloc(npatch * 2);
  uint16_t* hout = (uint16_t*)malloc(nfull * 2);
  for (size_t i = 0; i < nfull; ++i) hfull[i] = (uint16_t)next_u32();
  for (size_t i = 0; i < npatch; ++i) hpatch[i] = (uint16_t)next_u32();
  void *dfull, *dpatch;
  HIP_OK(hipMalloc(&dfull, nfull * 2));
  HIP_OK(hipMalloc(&dpatch, npatch * 2));
  HIP_OK(hipMemcpy(dfull, hfull, nfull * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dpatch, hpatch, npatch * 2, hipMemcpyHostToDevice));
  int st = dpp_splice_patch(dfull, dpatch, B, H, W, C, row0, rows, DPP_BF16, stream);
  CHECK(st == DPP_OK, "dpp_splice_patch -> %d (%s)", st, dpp_strerror(st));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hout, dfull, nfull * 2, hipMemcpyDeviceToHost));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t i = 0; i < W * C; ++i) {
        const size_t f = (size_t)((b * H + h) * W * C + i);
        uint16_t want = hfull[f];
        if (h >= row0 && h < row0 + rows) want = hpatch[(size_t)((b * rows + (h - row0)) * W * C + i)];
        CHECK(hout[f] == want, "splice mismatch at b=%lld h=%lld i=%lld", (long long)b, (long long)h,
              (long long)i);
      }

  /* ---- CFG combine + rel-MAE, float32, n = 100003 ---- */
  const int64_t n = 100003;
  const float w = 7.5f;
  float* hc = (float*)malloc((size_t)n * 4);
  float* hu = (float*)malloc((size_t)n * 4);
  float* he = (float*)malloc((size_t)n * 4);
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    hu[i] = next_f();
    hc[i] = hu[i] + 0.05f * next_f();
    num += fabs((double)hc[i] - (double)hu[i]);
    den += fabs((double)hu[i]);
  }
  void *dc, *du, *de, *dws;
  float* drel;
  const size_t wsb = dpp_cfg_combine_workspace_bytes(n);
  HIP_OK(hipMalloc(&dc, (size_t)n * 4));
  HIP_OK(hipMalloc(&du, (size_t)n * 4));
  HIP_OK(hipMalloc(&de, (size_t)n * 4));
  HIP_OK(hipMalloc(&dws, wsb));
  HIP_OK(hipMalloc((void**)&drel, 4));
  HIP_OK(hipMemcpy(dc, hc, (size_t)n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(du, hu, (size_t)n * 4, hipMemcpyHostToDevice));
  st = dpp_cfg_combine_relmae(de, drel, dc, du, n, w, dws, wsb, DPP_F32, stream);
  CHECK(st == DPP_OK, "dpp_cfg_combine_relmae -> %d (%s)", st, dpp_strerror(st));
  HIP_OK(hipStreamSynchronize(stream));
  float rel;
  HIP_OK(hipMemcpy(he, de, (size_t)n * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&rel, drel, 4, hipMemcpyDeviceToHost));
  double max_err = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double want = (double)hu[i] + (double)w * ((double)hc[i] - (double)hu[i]);
    const double err = fabs((double)he[i] - want);
    if (err > max_err) max_err = err;
  }
  CHECK(max_err <= 1e-4, "cfg combine max-abs-err %.3e > 1e-4", max_err);
  const double rel_want = num / den;
  CHECK(fabs((double)rel - rel_want) <= 1e-3 * rel_want, "rel-MAE %.7g vs %.7g", (double)rel, rel_want);

  /* ---- conv 3x3 with halo rows, bf16, split input channels ---- */
  {
    const int64_t cB = 2, cH = 9, cW = 5, Ci = 192, Co = 80, r0 = 3, R = 3;
    const size_t nx = (size_t)(cB * R * cW * Ci), ns = (size_t)(cB * cH * cW * Ci), nw = (size_t)(Co * 9 * Ci);
    const size_t ny = (size_t)(cB * R * cW * Co);
    uint16_t* hx = (uint16_t*)malloc(nx * 2);
    uint16_t* hs = (uint16_t*)malloc(ns * 2);
    uint16_t* hw = (uint16_t*)malloc(nw * 2);
    uint16_t* hy = (uint16_t*)malloc(ny * 2);
    float* hb = (float*)malloc((size_t)Co * 4);
    for (size_t i = 0; i < nx; ++i) hx[i] = to_bf16(next_f());
    for (size_t i = 0; i < ns; ++i) hs[i] = to_bf16(next_f());
    for (size_t i = 0; i < nw; ++i) hw[i] = to_bf16(0.05f * next_f());
    for (int64_t i = 0; i < Co; ++i) hb[i] = 0.1f * next_f();
    const size_t cwsb = dpp_conv3x3_halo_workspace_bytes(cB, R, cW, Ci, Co);
    CHECK(cwsb > 0, "this conv shape is expected to split its input channels");
    void *dx, *ds, *dw, *dy, *dws2;
    float* db;
    HIP_OK(hipMalloc(&dx, nx * 2));
    HIP_OK(hipMalloc(&ds, ns * 2));
    HIP_OK(hipMalloc(&dw, nw * 2));
    HIP_OK(hipMalloc(&dy, ny * 2));
    HIP_OK(hipMalloc((void**)&db, (size_t)Co * 4));
    HIP_OK(hipMalloc(&dws2, cwsb));
    HIP_OK(hipMemcpy(dx, hx, nx * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(ds, hs, ns * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, hw, nw * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, hb, (size_t)Co * 4, hipMemcpyHostToDevice));
    st = dpp_conv3x3_halo_ws(dy, dx, ds, dw, db, cB, cH, cW, Ci, Co, r0, R, dws2, cwsb, DPP_BF16, stream);
    CHECK(st == DPP_OK, "dpp_conv3x3_halo_ws -> %d (%s)", st, dpp_strerror(st));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(hy, dy, ny * 2, hipMemcpyDeviceToHost));
    double cmax = 0.0, cref_max = 0.0;
    for (int64_t b = 0; b < cB; ++b)
      for (int64_t i = 0; i < R; ++i)
        for (int64_t w = 0; w < cW; ++w)
          for (int64_t o = 0; o < Co; ++o) {
            double acc = hb[o];
            for (int64_t dy_ = -1; dy_ <= 1; ++dy_)
              for (int64_t dx_ = -1; dx_ <= 1; ++dx_) {
                const int64_t ir = r0 + i + dy_, ic = w + dx_;
                if (ir < 0 || ir >= cH || ic < 0 || ic >= cW) continue;
                const int fresh = ir >= r0 && ir < r0 + R;
                for (int64_t c = 0; c < Ci; ++c) {
                  const uint16_t xv = fresh ? hx[(size_t)(((b * R + (ir - r0)) * cW + ic) * Ci + c)]
                                            : hs[(size_t)(((b * cH + ir) * cW + ic) * Ci + c)];
                  acc += from_bf16(hw[(size_t)((o * 9 + (dy_ + 1) * 3 + (dx_ + 1)) * Ci + c)]) * from_bf16(xv);
                }
              }
            const double got = from_bf16(hy[(size_t)(((b * R + i) * cW + w) * Co + o)]);
            if (fabs(got - acc) > cmax) cmax = fabs(got - acc);
            if (fabs(acc) > cref_max) cref_max = fabs(acc);
          }
    /* one bf16 rounding of the output: |err| <= 2^-8 |ref| plus float32 summation error */
    CHECK(cmax <= 5e-3 * cref_max + 1e-4, "conv max-abs-err %.3e (max |ref| %.3e)", cmax, cref_max);
    printf("conv split-K (workspace %zu B) max-abs-err %.3e of max |ref| %.3e\n", cwsb, cmax, cref_max);
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(ds));
    HIP_OK(hipFree(dw));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(db));
    HIP_OK(hipFree(dws2));
    free(hx);
    free(hs);
    free(hw);
    free(hy);
    free(hb);
  }

  HIP_OK(hipFree(dfull));
  HIP_OK(hipFree(dpatch));
  HIP_OK(hipFree(dc));
  HIP_OK(hipFree(du));
  HIP_OK(hipFree(de));
  HIP_OK(hipFree(dws));
  HIP_OK(hipFree(drel));
  HIP_OK(hipStreamDestroy(stream));
  free(hfull);
  free(hpatch);
  free(hout);
  free(hc);
  free(hu);
  free(he);
  printf("splice bit-exact; cfg max-abs-err %.3e; rel-MAE %.7g (host %.7g)\n", max_err, (double)rel, rel_want);
  printf("capi ok\n");
  return 0;
}
