/*
 * dpp.h -- C ABI of libdpp: one device's share of a displaced-patch-parallel
 * diffusion denoising step, as gfx950 (MI355X) HIP kernels.
 *
 * The method (DistriFusion reading notes, Introduction, fourth paragraph):
 * the image is split into patches, one per device; after a synchronous first
 * step, each device computes only its own patch from fresh activations and
 * takes the rest of the image (global context, patch interaction) from the
 * activations of the previous denoising step.  The layers that need the rest
 * of the image are GroupNorm, 3x3 convolution and self-attention
 * (DistriFusion architecture article: DistriGroupNorm, DistriConv2dPP,
 * DistriSelfAttentionPP); after each layer the patch outputs are gathered and
 * concatenated along the height axis into a reused full-image buffer
 * (same article, communication section).  On one device that gather becomes
 * dpp_splice_patch.  Classifier-free guidance combines a conditional and an
 * unconditional branch, and the relative error between their noise
 * predictions (rel-MAE) is the denoising discrepancy that drives
 * condition-split scheduling (Hybridiff technical summary, sections 2A, 2B).
 *
 * Conventions for every call:
 *  - Layout is token-major (NHWC): an activation is [B,H,W,C], row-major,
 *    contiguous; a patch is the row band [row0, row0+rows) of it, stored
 *    contiguously as [B,rows,W,C]; token t = row*W + col.
 *  - Every pointer is a device pointer owned by the caller.  The library
 *    allocates, frees and synchronises nothing, keeps no state between calls,
 *    and may be called from several host threads.
 *  - dtype selects the storage type of activations and conv weights:
 *    DPP_BF16 (bf16 bit patterns) or DPP_F32.  GroupNorm gamma/beta, conv
 *    bias, group statistics and the rel-MAE scalar are always float32.
 *    Arithmetic is float32 (group statistics finalised in float64); every
 *    bf16 output is stored with one round-to-nearest-even conversion of its
 *    float32 result.  The one rounding inside a call is the attention's: its
 *    softmax weights enter the bf16 weight x value product as bf16, while
 *    the normaliser sums the same weights in float32 before that rounding.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it and the call returns at once; faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - Return value: DPP_OK, or a negative DPP_ERR_* code.  Arguments are
 *    validated on the host before anything is enqueued: on an error nothing
 *    is launched and nothing is written.
 *  - Workspaces are caller-owned device scratch, at least the size the
 *    matching *_workspace_bytes() returns, 256-byte aligned.  They need no
 *    initialisation and hold nothing useful after the call.  Calls that
 *    share a workspace must be ordered (same stream).
 */
#ifndef DPP_H_
#define DPP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DPP_VERSION 1

enum dpp_dtype { DPP_BF16 = 0, DPP_F32 = 1 };

enum dpp_status {
  DPP_OK = 0,
  DPP_ERR_NULL = -1,        /* a required pointer is NULL                    */
  DPP_ERR_SHAPE = -2,       /* non-positive size, band outside the image,
                               C % G != 0, heads*head_dim > ld, ...          */
  DPP_ERR_DTYPE = -3,       /* dtype is neither DPP_BF16 nor DPP_F32         */
  DPP_ERR_ALIGN = -4,       /* a pointer or row stride is not 16-byte aligned
                               where the kernel reads 16-byte vectors        */
  DPP_ERR_ALIAS = -5,       /* an output overlaps an input it may not alias  */
  DPP_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required       */
  DPP_ERR_UNSUPPORTED = -7, /* valid shape the library has no kernel for    */
  DPP_ERR_LAUNCH = -8       /* the HIP runtime rejected a launch             */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* dpp_strerror(int status);

/* DPP_VERSION of the built library. */
int dpp_version(void);

/*
 * a1 -- splice.  Writes the fresh patch into rows [row0, row0+rows) of the
 * full-image buffer: full[b, row0+i, w, c] = patch[b, i, w, c].  Other rows
 * are left untouched.  This is the local stand-in for gathering every
 * device's patch output and concatenating along the height axis into the
 * reused full-image buffer (DistriFusion architecture article, communication
 * section); on one device, only the own patch is fresh, so the buffer holds
 * fresh own rows and the previous step's rows elsewhere (DistriFusion reading
 * notes, Introduction, fourth paragraph).
 *   full  [B,H,W,C] in/out.   patch [B,rows,W,C] in; must not overlap full.
 *   Requires 0 <= row0, rows >= 1, row0 + rows <= H.  Bit-exact copy.
 */
int dpp_splice_patch(void* full, const void* patch,
                     int64_t B, int64_t H, int64_t W, int64_t C,
                     int64_t row0, int64_t rows, int dtype, void* stream);

/*
 * a2 -- GroupNorm with stale statistics (DistriGroupNorm; DistriFusion
 * architecture article, normalisation section).  Normalises patch p with the
 * group statistics of the spliced image: the other patches' contribution is
 * their raw sums from the previous step, the own patch's is recomputed from
 * the fresh x.  Per batch b and group g (C/G channels each):
 *   s1, s2   = sum of x, x^2 over the patch (rows x W x C/G values)
 *   T_k      = s_k + sum_{q != p} stale_stats[b,q,g,k]
 *   mean     = T_1/n,  var = max(T_2/n - mean^2, 0),  n = H*W*C/G
 *   y        = (x - mean)/sqrt(var + eps) * gamma[c] + beta[c]
 *   stats_out[b,p,g,:] = (s1, s2)   (the next step's stale_stats slot p;
 *                                    other slots are not written)
 *   x, y        [B,rows,W,C]   (y may equal NULL: only stats_out is produced,
 *                               the first half of the synchronous step; then
 *                               gamma, beta and stale_stats may be NULL)
 *   stale_stats [B,P,G,2] float32, slot p ignored; NULL allowed when P == 1
 *   stats_out   [B,P,G,2] float32; must not overlap stale_stats or y
 *   gamma, beta [C] float32
 *   Requires C % G == 0, 0 <= p < P, 1 <= rows <= H, C <= 8*256 (bf16) or
 *   4*256 (f32), C % 8 == 0 (bf16) or C % 4 == 0 (f32), x and y 16-byte
 *   aligned.  Workspace: dpp_groupnorm_stale_workspace_bytes().
 */
size_t dpp_groupnorm_stale_workspace_bytes(int64_t B, int64_t rows, int64_t W,
                                           int64_t C, int64_t G);
int dpp_groupnorm_stale(void* y, float* stats_out, const void* x,
                        const float* stale_stats, const float* gamma,
                        const float* beta, int64_t B, int64_t H, int64_t W,
                        int64_t C, int64_t G, int64_t P, int64_t p,
                        int64_t rows, float eps, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream);

/*
 * GroupNorm with stale statistics followed by SiLU, y = z * sigmoid(z) of
 * the dpp_groupnorm_stale output z: the GroupNorm + SiLU pair that opens an
 * SDXL residual block (the normalisation layer wrapped by DistriGroupNorm,
 * DistriFusion architecture article, normalisation section).  Arguments,
 * statistics, requirements and workspace exactly as dpp_groupnorm_stale;
 * stats_out holds the sums of x (before normalisation).
 */
int dpp_groupnorm_silu_stale(void* y, float* stats_out, const void* x,
                             const float* stale_stats, const float* gamma,
                             const float* beta, int64_t B, int64_t H,
                             int64_t W, int64_t C, int64_t G, int64_t P,
                             int64_t p, int64_t rows, float eps,
                             void* workspace, size_t workspace_bytes,
                             int dtype, void* stream);

/*
 * GroupNorm with stale statistics whose fresh sums come from the kernel that
 * produced x, so x is read once (DistriGroupNorm; DistriFusion architecture
 * article, normalisation section).  The producers dpp_conv3x3_halo_gn and
 * dpp_linear_gn write, besides their output, its GroupNorm partial sums:
 *   partials [B,nchunk,G,2] float32: per chunk and group (sum y, sum y^2) of
 *            the stored output values over the chunk's pixels and the
 *            group's channels (zero where the chunk does not touch it).
 * This call adds the chunks in float64 in one fixed order (64 lanes, lane j
 * adding chunks j, j+64, j+128, ... in increasing order, then the 64 lane
 * sums pairwise at offsets 32, 16, ..., 1) as the fresh sums s1, s2 of
 * dpp_groupnorm_stale, and continues exactly as that call (stale
 * correction, mean/var, normalisation, stats_out[b,p] = the fresh sums);
 * silu != 0 applies SiLU to the result as dpp_groupnorm_silu_stale does.
 *   x, y [B,rows,W,C] as dpp_groupnorm_stale (y == NULL: stats_out only);
 *   partials as written by the producer of x for the same
 *   B, G and shape; nchunk >= 1 its chunk count (the producer's *_gn_chunks).
 *   The result depends on partials only through their per-group sums: with
 *   partials of values other than x's, it normalises x with those sums.
 *   No workspace: one launch (the group totals are formed on chip by every
 *   workgroup, in one fixed order).  Requirements and errors otherwise as
 *   dpp_groupnorm_stale; partials must not overlap y or stats_out.
 */
int dpp_groupnorm_stale_presummed(void* y, float* stats_out, const void* x,
                                  const float* partials, int64_t nchunk,
                                  const float* stale_stats, const float* gamma,
                                  const float* beta, int64_t B, int64_t H,
                                  int64_t W, int64_t C, int64_t G, int64_t P,
                                  int64_t p, int64_t rows, float eps,
                                  int silu, int dtype, void* stream);

/*
 * dpp_groupnorm_stale without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The scratch it needs (the chunk partial
 * sums that dpp_groupnorm_stale keeps in its workspace) lives in a static
 * device array of DPP_GN_NOALLOC_MAX_BYTES inside the
 * library; each GPU holds its own copy from the first call made with that
 * device current until the process ends.  The call allocates and frees
 * nothing.  Shapes whose scratch
 * (dpp_groupnorm_stale_workspace_bytes) exceeds DPP_GN_NOALLOC_MAX_BYTES
 * return DPP_ERR_WORKSPACE -- e.g. G = 32 fits every B <= 4096.  All calls on
 * one GPU share that GPU's array: calls that may overlap on one GPU (several
 * streams, several host threads without ordering) race and must be ordered
 * by the caller.  Nothing in the array needs clearing: every element a call
 * reads was written earlier in the same call.  DPP_ERR_LAUNCH also reports a
 * failed lookup of the array's device address.  Arguments, statistics,
 * requirements and results otherwise exactly as dpp_groupnorm_stale.
 */
#define DPP_GN_NOALLOC_MAX_BYTES (1u << 20)
int dpp_groupnorm_stale_noalloc(void* y, float* stats_out, const void* x,
                                const float* stale_stats, const float* gamma,
                                const float* beta, int64_t B, int64_t H,
                                int64_t W, int64_t C, int64_t G, int64_t P,
                                int64_t p, int64_t rows, float eps, int dtype,
                                void* stream);

/*
 * a3 -- 3x3 convolution of the patch rows with halo rows from the stale image
 * (DistriConv2dPP; DistriFusion architecture article, conv section; only the
 * own region is computed: DistriFusion reading notes, Introduction, fourth
 * paragraph).  Stride 1, zero padding 1 at the image border, cross-
 * correlation:
 *   y[b,i,w,o] = bias[o] + sum_{dy,dx in 0..2} sum_c
 *                weight[o,dy,dx,c] * S[b, row0+i+dy-1, w+dx-1, c]
 * where S is the spliced image: rows [row0, row0+rows) from x, rows row0-1
 * and row0+rows (the halos) from stale_full, zero outside the image.  No
 * other row of stale_full is read.
 *   x          [B,rows,W,Cin]
 *   stale_full [B,H,W,Cin]; may be NULL when both halo rows are outside the
 *              image (row0 == 0 and rows == H)
 *   weight     [Cout,3,3,Cin] (dtype)   bias [Cout] float32 or NULL
 *   y          [B,rows,W,Cout]; must not overlap any input
 *   bf16 requires Cin % 64 == 0, Cout % 16 == 0 and 16-byte aligned x,
 *   stale_full, weight, y (else DPP_ERR_UNSUPPORTED / DPP_ERR_ALIGN), and
 *   (Cout + 128) * 9 * Cin * 2 < 2^31 and (W + 2) * Cin * 2 < 2^31 (32-bit
 *   weight and image-row offsets; else DPP_ERR_UNSUPPORTED).  f32 has no
 *   divisibility requirement.
 */
int dpp_conv3x3_halo(void* y, const void* x, const void* stale_full,
                     const void* weight, const float* bias, int64_t B,
                     int64_t H, int64_t W, int64_t Cin, int64_t Cout,
                     int64_t row0, int64_t rows, int dtype, void* stream);

/*
 * dpp_conv3x3_halo with an optional float32 workspace.  When the bf16 patch
 * is too small to fill the GPU with output tiles (e.g. the 1024 px level: 40
 * tiles), the input channels are split across workgroups that write float32
 * partial outputs to the workspace, and a second kernel adds them (in a
 * fixed order) with the bias; results match the oracle to the same bar, not
 * bit for bit the unsplit call.  workspace_bytes >=
 * dpp_conv3x3_halo_workspace_bytes(B, rows, W, Cin, Cout) enables the split
 * (0 = the shape needs none); NULL / smaller runs unsplit.  The workspace
 * must be 16-byte aligned (else DPP_ERR_ALIGN) and must not overlap any
 * operand (else DPP_ERR_ALIAS); calls sharing one must be ordered.
 * Everything else exactly as dpp_conv3x3_halo.
 */
size_t dpp_conv3x3_halo_workspace_bytes(int64_t B, int64_t rows, int64_t W,
                                        int64_t Cin, int64_t Cout);
int dpp_conv3x3_halo_ws(void* y, const void* x, const void* stale_full,
                        const void* weight, const float* bias, int64_t B,
                        int64_t H, int64_t W, int64_t Cin, int64_t Cout,
                        int64_t row0, int64_t rows, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream);

/*
 * dpp_conv3x3_halo that also writes the GroupNorm partial sums of its output
 * for a GroupNorm that follows (dpp_groupnorm_stale_presummed), from the
 * stored bf16 values, one chunk per output tile:
 *   gn_partials [B, dpp_conv3x3_halo_gn_chunks(rows, W, Cout), G, 2] float32
 * G groups of Cout/G channels (Cout % G == 0, else DPP_ERR_SHAPE).  y is
 * bit-identical to dpp_conv3x3_halo's; always unsplit (no workspace).  bf16
 * only (DPP_F32: DPP_ERR_UNSUPPORTED).  gn_partials must not overlap an
 * operand.  Everything else exactly as dpp_conv3x3_halo.
 */
int64_t dpp_conv3x3_halo_gn_chunks(int64_t rows, int64_t W, int64_t Cout);
int dpp_conv3x3_halo_gn(void* y, float* gn_partials, int64_t G, const void* x,
                        const void* stale_full, const void* weight,
                        const float* bias, int64_t B, int64_t H, int64_t W,
                        int64_t Cin, int64_t Cout, int64_t row0, int64_t rows,
                        int dtype, void* stream);

/*
 * a4 -- displaced self-attention (DistriSelfAttentionPP; DistriFusion
 * architecture article, attention section).  The patch's queries attend over
 * all tokens of the spliced full-image K/V buffer (fresh own rows, previous
 * step's rows elsewhere: DistriFusion reading notes, Introduction, fourth
 * paragraph).  Per batch b, head h (channels [h*D, (h+1)*D)) and query i:
 *   o[b,i,h] = sum_j softmax_j(scale * <q[b,i,h], k[b,j,h]>) v[b,j,h]
 *   q [B,n_q,ld_q], k and v [B,n_kv,ld_kv], o [B,n_q,ld_o]: row strides in
 *   elements, ld >= heads*head_dim; k and v may be the same pointer.
 *   scale <= 0 selects 1/sqrt(head_dim).  o must not overlap q, k or v.
 *   bf16 requires head_dim == 64, 16-byte aligned pointers and ld % 8 == 0.
 *   f32 requires head_dim in {16, 32, 64, 128}.
 *   Limits (else DPP_ERR_UNSUPPORTED): B*heads <= 65535, n_q and n_kv <=
 *   2^30, ceil(n_q/256)*B*heads*16 < 2^31; bf16 row strides ld_q, ld_kv,
 *   ld_o <= 2^24 elements (64 key rows of K/V are addressed with 32-bit byte
 *   offsets).
 *   workspace: optional.  With workspace_bytes >=
 *   dpp_self_attn_workspace_bytes(...) the key range may be split across
 *   workgroups and merged in a second pass (more parallelism for short query
 *   ranges); with NULL / 0 the call runs unsplit.
 */
size_t dpp_self_attn_workspace_bytes(int64_t B, int64_t n_q, int64_t n_kv,
                                     int64_t heads, int64_t head_dim,
                                     int dtype);
int dpp_self_attn_displaced(void* o, const void* q, const void* k,
                            const void* v, int64_t B, int64_t n_q,
                            int64_t n_kv, int64_t heads, int64_t head_dim,
                            int64_t ld_q, int64_t ld_kv, int64_t ld_o,
                            float scale, void* workspace,
                            size_t workspace_bytes, int dtype, void* stream);

/*
 * Projection: y[b,m,n] = sum_k x[b,m,k] * w[n,k] + bias[n].  The to_q, to_k,
 * to_v and to_out projections of the self-attention module that
 * DistriSelfAttentionPP wraps (DistriFusion architecture article, attention
 * section).  Element (b,m,k) of x is x[b*bs_x + m*ld_x + k]; element (b,m,n)
 * of y is y[b*bs_y + m*ld_y + n] (strides in elements).  Free strides let the
 * K/V projection of the fresh patch write straight into its rows of the
 * private full-image K/V buffer: y = buffer + row0*W*ld_y with bs_y the
 * buffer's batch stride -- the splice fused into the projection.
 *   x [B,M,K] (dtype), w [N,K] (dtype, output-major), bias [N] float32 or
 *   NULL, y [B,M,N] (dtype); y must not overlap x, w or bias, and output
 *   batches must not overlap (bs_y >= (M-1)*ld_y + N when B > 1).
 *   Requires ld_x >= K, ld_y >= N.  bf16 requires K % 8 == 0, N % 4 == 0,
 *   x and w 16-byte aligned, ld_x and bs_x multiples of 8, y 8-byte aligned,
 *   ld_y and bs_y multiples of 4, and 32-bit byte offsets within w and within
 *   one batch entry of x: (N + 256) * K * 2 + 128 < 2^31 and ((M + 160) * ld_x +
 *   K) * 2 < 2^31 - 16 (else DPP_ERR_UNSUPPORTED).  Limits for both dtypes:
 *   B <= 65535, M, K, N <= 2^30.  Float32 accumulation, one rounding.
 */
int dpp_linear(void* y, const void* x, const void* w, const float* bias,
               int64_t B, int64_t M, int64_t K, int64_t N, int64_t ld_x,
               int64_t bs_x, int64_t ld_y, int64_t bs_y, int dtype,
               void* stream);

/*
 * dpp_linear that also writes the GroupNorm partial sums of its output (the
 * M rows of a batch entry are the pixels, the N columns the channels) for a
 * GroupNorm that follows, e.g. the out projection feeding the next block's
 * GroupNorm (dpp_groupnorm_stale_presummed), from the stored bf16 values:
 *   gn_partials [B, dpp_linear_gn_chunks(B, M, N), G, 2] float32
 * G groups of N/G channels (N % G == 0, else DPP_ERR_SHAPE).  y is
 * bit-identical to dpp_linear's.  bf16 only (DPP_F32:
 * DPP_ERR_UNSUPPORTED).  gn_partials must not overlap an operand.
 * Everything else exactly as dpp_linear.
 */
int64_t dpp_linear_gn_chunks(int64_t B, int64_t M, int64_t N);
int dpp_linear_gn(void* y, float* gn_partials, int64_t G, const void* x,
                  const void* w, const float* bias, int64_t B, int64_t M,
                  int64_t K, int64_t N, int64_t ld_x, int64_t bs_x,
                  int64_t ld_y, int64_t bs_y, int dtype, void* stream);

/*
 * a5 -- classifier-free guidance combine and denoising discrepancy
 * (Hybridiff technical summary, section 2A: conditional and unconditional
 * branches; section 2B: rel-MAE between their noise predictions).
 *   eps[i]  = eps_u[i] + guidance * (eps_c[i] - eps_u[i])
 *   *relmae = sum_i |eps_c[i] - eps_u[i]| / sum_i |eps_u[i]|
 *             (deterministic order: each thread first adds its own
 *              elements in float32 -- about 8 * ceil(n / 2^21) of them, 8
 *              at n = 65536 -- then the workgroup and grid sums are
 *              float64; 0/0 -> NaN, x/0 -> +inf)
 *   eps, eps_c, eps_u: n elements; eps may be exactly eps_c or eps_u, and
 *   must not partly overlap them.  relmae: one device float32, or NULL to
 *   skip the reduction.  Workspace: dpp_cfg_combine_workspace_bytes(n)
 *   (may be NULL when relmae is NULL).
 */
size_t dpp_cfg_combine_workspace_bytes(int64_t n);
int dpp_cfg_combine_relmae(void* eps, float* relmae, const void* eps_c,
                           const void* eps_u, int64_t n, float guidance,
                           void* workspace, size_t workspace_bytes, int dtype,
                           void* stream);

/*
 * Adaptive parallelism switching (Hybridiff technical summary, section 2B):
 * the per-step denoising discrepancy (the rel-MAE of
 * dpp_cfg_combine_relmae) selects, for each denoising step, the warm-up
 * stage (0: branches run serially), the parallel stage (1: conditional and
 * unconditional branches on two devices) or the fully-connecting stage (2).
 * The stage boundaries are where the discrepancy's decline slows (tau1) and
 * where it starts to rise again (tau2); the pages give no thresholds, so the
 * rule is:
 *   drop[i]  = relmae[i-1] - relmae[i],  maxdrop[i] = max(drop[1..i], 0)
 *   tau1     = first i >= min_warmup with maxdrop[i] > 0 and
 *              drop[i] <= rho * maxdrop[i]
 *   tau2     = first i > tau1 with relmae[i] > (1 + eps) *
 *              min(relmae[tau1..i-1])
 *   stage[i] = 0 for i < tau1, 1 for tau1 <= i < tau2, 2 for i >= tau2
 * (T when a boundary never comes).  float32 arithmetic; NaN entries (0/0
 * discrepancy) never trigger a boundary.  Causal: stage[i] depends on
 * relmae[0..i] only, so the call can be repeated on the growing trace.
 *   relmae [T] host float32, in denoising order (index 0 = the first step);
 *   stage  [T] host int32 out; tau1, tau2 host int64 out.
 *   Requires T >= 1, min_warmup >= 1, 0 <= rho <= 1, eps >= 0.  Host code:
 *   no device work, no stream.  Typical rho = 0.25, eps = 0.02.
 */
int dpp_hybrid_schedule(const float* relmae, int64_t T, float rho, float eps,
                        int64_t min_warmup, int32_t* stage, int64_t* tau1,
                        int64_t* tau2);

#ifdef __cplusplus
}
#endif

#endif /* DPP_H_ */
