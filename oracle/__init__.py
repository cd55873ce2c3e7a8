"""CPU oracle for one device's share of a displaced-patch-parallel denoising step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it.

Everything is plain float64 numpy; each function is the definition of its step
written out, with a library matmul/exp as the only primitives.  Sources (the
page titles are those of the reference pages):

* "DistriFusion reading notes" -- CSDN blog notes on "DistriFusion: Distributed
  Parallel Inference for High-Resolution Diffusion Models", Introduction fourth
  paragraph: the image is split into patches, one per device; after a
  synchronous first step, each device reuses the previous step's activations
  for global context and patch interaction, and runs conv and attention only
  on its own region.
* "DistriFusion architecture article" -- mqxn.cn article on DistriFusion's
  distributed UNet design: module wrappers DistriConv2dPP, DistriSelfAttentionPP
  and DistriGroupNorm (sections on conv, attention and normalisation layer
  splitting), and the gather of patch outputs concatenated along the height
  axis into a reused full-image buffer (section on communication).
* "AsyncDiff abstract" -- arxivdaily.com summary and abstract of arXiv 2406.06911:
  the noise-prediction model split into components on separate devices, each
  fed the previous step's hidden state of the component before it.
* "Hybridiff technical summary" -- gist.science summary of arXiv 2602.21760,
  section 2A (conditional and unconditional CFG branches as parallel units) and
  2B (denoising discrepancy: relative error rel-MAE between the conditional and
  unconditional noise predictions).

Readings where the pages are silent (each also listed in the design notes):
  R1  a displaced layer is the ordinary full-image layer applied to the spliced
      image S_p (stale image with patch p's rows replaced by the fresh patch),
      restricted to patch p's rows;
  R2  GroupNorm statistics: per-patch raw sums (sum x, sum x^2) per group; the
      other patches' sums come from the previous step, the own patch's are
      fresh; biased variance, clamped at 0; eps = 1e-5;
  R3  conv: 3x3, stride 1, zero padding 1 at the image border, bias;
      cross-correlation; halo rows from the stale image;
  R4  attention: softmax(scale Q K^T) V per head, scale = 1/sqrt(D), no mask;
      Q from the patch, K/V over all tokens of the spliced buffer;
  R5  CFG: eps = eps_u + w (eps_c - eps_u); rel-MAE = sum|eps_c - eps_u| /
      sum|eps_u|;
  R6  chained block GN -> conv -> splice -> attention with identity Q/K/V
      projections; bf16 configurations round each stored layer output to bf16;
      the previous step is the synchronous full-image run of the same block on
      the stale input.
  R11 projected attention: q/k/v/out are linear maps x W^T + b of the wrapped
      attention module; the patch's fresh k and v replace its tokens in the
      previous step's projected K and V (splicing rows commutes with a
      row-wise linear map, so this equals projecting the spliced input);
  R12 GroupNorm + SiLU: z * sigmoid(z) applied to the GroupNorm output.
  R13 stage switching: the warm-up ends at the first step (at or after a
      minimum warm-up) whose decline d[i-1] - d[i] is at most rho times the
      fastest decline so far; the parallel stage ends at the first later step
      whose discrepancy exceeds (1 + eps) times that stage's running minimum
      (rho = 0.25, eps = 0.02 by default).
  R14 component step: a component is the full-image block (P = 1) GN -> conv
      -> attention with identity projections; its input after the warm-up is
      the previous step's stored output of the component before it.
  R15 attention block: GroupNorm + SiLU -> conv -> q projection, fresh k, v
      projections spliced into the previous step's projected K, V -> attention
      -> out projection; the previous step is the synchronous full-image run
      of the same block on the stale input, whose projected K, V every patch
      starts from.
"""
from .dpp_oracle import (  # noqa: F401
    bf16_round,
    splice,
    patch_sums,
    groupnorm_stale,
    conv3x3_halo,
    conv3x3_halo_sampled,
    self_attn_displaced,
    cfg_combine_relmae,
    hybrid_schedule,
    silu,
    groupnorm_silu_stale,
    linear,
    projected_attention,
    previous_step_state,
    displaced_block,
    component_block,
    async_component_chain,
    previous_block_state,
    displaced_attention_block,
)
