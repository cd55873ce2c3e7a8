"""Call sequences of one device's share of a displaced-patch-parallel step.

One emulated device (patch p of P row bands) runs GroupNorm -> 3x3 conv ->
splice -> self-attention with identity Q/K/V projections: the conv output of
its rows is the query set, and K = V = its private full-image buffer, i.e. the
previous step's conv output with its own rows replaced by the fresh ones.  The
previous step is the synchronous first step (DistriFusion reading notes,
Introduction, fourth paragraph): per-patch raw GroupNorm sums of the stale
input, GroupNorm and conv of the whole stale image.

DisplacedBlock is the same share of the attention block with its
projections: GroupNorm + SiLU -> conv -> q and fused K/V projections into the
private K/V buffer -> attention -> out projection.  ComponentChain sequences
the full-image components of an asynchronous component chain.

Every arithmetic step runs in libdpp's kernels; this module only allocates
device buffers (torch) and issues the calls on the current stream.  Each
emulated patch owns a private K/V buffer so that one patch's fresh rows never
reach another patch within the same step (on real devices they arrive with the
next step's exchange).
"""
from __future__ import annotations

import torch

from . import _lib as L


def capture_graph(fn, warmup: int = 1):
    """Record the kernel launches of `fn` -- a sequence of libdpp calls, which
    launch on the current stream and allocate, copy and synchronise nothing --
    into a HIP graph (torch.cuda.CUDAGraph) and return it; `graph.replay()`
    then issues the whole sequence with one launch from the host.  `fn` runs
    `warmup` times eagerly on a side stream first.  The graph keeps the
    device pointers it was captured with: replays read and write the same
    buffers, so the caller refills the input buffers in place between
    replays.  Every libdpp kernel writes its outputs in full (no memset
    nodes), so each replay recomputes them from the inputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


class DisplacedLayer:
    def __init__(self, B, H, W, C, P, G, heads, dtype, device="cuda", eps=1e-5, head_dim=64):
        if H % P:
            raise ValueError("H must divide into P equal row bands")
        self.B, self.H, self.W, self.C, self.P, self.G = B, H, W, C, P, G
        self.heads, self.D, self.eps = heads, head_dim, eps
        self.R = H // P
        self.dtype = dtype
        self.device = device
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dtype, device=device)
        self.stats_prev = torch.zeros(B, P, G, 2, **f32)   # stale sums (previous step)
        self.stats_next = torch.zeros(B, P, G, 2, **f32)   # fresh sums (this step)
        self.a1 = torch.empty(B, H, W, C, **act)           # previous GN output (conv halo source)
        self.a2 = torch.empty(B, H, W, C, **act)           # previous conv output (stale K/V)
        self.kv = [None] * P                               # private spliced K/V buffers
        self.y1 = torch.empty(B, self.R, W, C, **act)
        self.y2 = torch.empty(B, self.R, W, C, **act)
        self.o = torch.empty(B, self.R * W, C, **act)
        gw = max(L.dpp_groupnorm_stale_workspace_bytes(B, H, W, C, G),
                 L.dpp_groupnorm_stale_workspace_bytes(B, self.R, W, C, G))
        self.gn_ws = torch.empty(max(gw, 256), dtype=torch.uint8, device=device)
        aw = L.dpp_self_attn_workspace_bytes(B, self.R * W, H * W, heads, head_dim,
                                             L.DPP_BF16 if dtype == torch.bfloat16 else L.DPP_F32)
        self.attn_ws = torch.empty(aw, dtype=torch.uint8, device=device) if aw else None
        cw = max(L.dpp_conv3x3_halo_workspace_bytes(B, self.R, W, C, C),
                 L.dpp_conv3x3_halo_workspace_bytes(B, H, W, C, C)) if dtype == torch.bfloat16 else 0
        self.conv_ws = torch.empty(cw, dtype=torch.uint8, device=device) if cw else None   # split-K partials
        self._stats_full = torch.zeros(B, 1, G, 2, **f32)

    def band(self, x, p):
        """Rows of patch p of a [B,H,W,C] tensor, contiguous."""
        return x[:, p * self.R:(p + 1) * self.R].contiguous()

    def synchronous_step(self, x_stale, gamma, beta, weight, bias):
        """Previous-step state from the stale input (every patch fresh)."""
        for q in range(self.P):
            L.dpp_groupnorm_stale(None, self.stats_prev, self.band(x_stale, q), None, None, None,
                                  self.H, self.G, self.P, q, self.eps, self.gn_ws)
        L.dpp_groupnorm_stale(self.a1, self._stats_full, x_stale, None, gamma, beta,
                              self.H, self.G, 1, 0, self.eps, self.gn_ws)
        L.dpp_conv3x3_halo(self.a2, self.a1, None, weight, bias, self.H, 0, workspace=self.conv_ws)
        for p in range(self.P):
            if self.kv[p] is None:
                self.kv[p] = torch.empty_like(self.a2)
            self.kv[p].copy_(self.a2)

    def patch_step(self, p, x_patch, gamma, beta, weight, bias):
        """Patch p's share of the current step; returns the attention output
        [B, R*W, C] (a buffer reused by the next call)."""
        r0 = p * self.R
        L.dpp_groupnorm_stale(self.y1, self.stats_next, x_patch, self.stats_prev, gamma, beta,
                              self.H, self.G, self.P, p, self.eps, self.gn_ws)
        L.dpp_conv3x3_halo(self.y2, self.y1, self.a1, weight, bias, self.H, r0, workspace=self.conv_ws)
        L.dpp_splice_patch(self.kv[p], self.y2, r0)
        kv = self.kv[p].view(self.B, self.H * self.W, self.C)
        L.dpp_self_attn_displaced(self.o, self.y2.view(self.B, self.R * self.W, self.C), kv, kv,
                                  self.heads, self.D, 0.0, self.attn_ws)
        return self.o


class DisplacedBlock:
    """One device's share of the attention block with its projections: GroupNorm
    + SiLU with stale statistics -> 3x3 conv with stale halos -> q projection
    and the fused K/V projection written straight into the patch's rows of its
    private K/V buffer (the splice fused into the projection) -> attention over
    the whole buffer -> out projection.  DistriGroupNorm, DistriConv2dPP and
    DistriSelfAttentionPP wrapping the whole attention module (DistriFusion
    architecture article); the rest of each private buffer is the previous
    step's projected K/V (DistriFusion reading notes, Introduction, fourth
    paragraph).  The K/V buffer is [B, N, 2C]: K in channels [0, C), V in
    [C, 2C), so one GEMM writes both.

    Buffer plumbing and call order only; every step runs in libdpp's kernels.
    """

    def __init__(self, B, H, W, C, P, G, heads, dtype=None, device="cuda", eps=1e-5, head_dim=64):
        if H % P:
            raise ValueError("H must divide into P equal row bands")
        dtype = dtype or torch.bfloat16
        self.B, self.H, self.W, self.C, self.P, self.G = B, H, W, C, P, G
        self.heads, self.D, self.eps = heads, head_dim, eps
        self.R = H // P
        self.N, self.Nq = H * W, self.R * W
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dtype, device=device)
        self.stats_prev = torch.zeros(B, P, G, 2, **f32)
        self.stats_next = torch.zeros(B, P, G, 2, **f32)
        self.a1 = torch.empty(B, H, W, C, **act)           # previous GroupNorm + SiLU output (conv halo source)
        self.kv = [None] * P                               # private [B, N, 2C] K/V buffers
        self.y1 = torch.empty(B, self.R, W, C, **act)
        self.y2 = torch.empty(B, self.R, W, C, **act)
        self.q = torch.empty(B, self.Nq, C, **act)
        self.o = torch.empty(B, self.Nq, C, **act)
        self.out = torch.empty(B, self.Nq, C, **act)
        gw = max(L.dpp_groupnorm_stale_workspace_bytes(B, H, W, C, G),
                 L.dpp_groupnorm_stale_workspace_bytes(B, self.R, W, C, G))
        self.gn_ws = torch.empty(max(gw, 256), dtype=torch.uint8, device=device)
        dt = L.DPP_BF16 if dtype == torch.bfloat16 else L.DPP_F32
        aw = L.dpp_self_attn_workspace_bytes(B, self.Nq, self.N, heads, head_dim, dt)
        self.attn_ws = torch.empty(aw, dtype=torch.uint8, device=device) if aw else None
        cw = max(L.dpp_conv3x3_halo_workspace_bytes(B, self.R, W, C, C),
                 L.dpp_conv3x3_halo_workspace_bytes(B, H, W, C, C)) if dtype == torch.bfloat16 else 0
        self.conv_ws = torch.empty(cw, dtype=torch.uint8, device=device) if cw else None
        self._stats_full = torch.zeros(B, 1, G, 2, **f32)

    def band(self, x, p):
        """Rows of patch p of a [B,H,W,C] tensor, contiguous."""
        return x[:, p * self.R:(p + 1) * self.R].contiguous()

    def synchronous_step(self, x_stale, gamma, beta, conv_w, conv_b, w_kv, b_kv):
        """Previous-step state from the stale input (every patch fresh): the
        per-patch sums, GroupNorm + SiLU of the whole image, its conv, and
        the projected K/V every private buffer starts from."""
        B, H, W, C = self.B, self.H, self.W, self.C
        for q in range(self.P):
            L.dpp_groupnorm_stale(None, self.stats_prev, self.band(x_stale, q), None, None, None,
                                  H, self.G, self.P, q, self.eps, self.gn_ws)
        L.dpp_groupnorm_silu_stale(self.a1, self._stats_full, x_stale, None, gamma, beta, H, self.G, 1, 0, self.eps,
                                   self.gn_ws)
        a2 = torch.empty_like(self.a1)
        L.dpp_conv3x3_halo(a2, self.a1, None, conv_w, conv_b, H, 0, workspace=self.conv_ws)
        kv0 = torch.empty(B, self.N, 2 * C, dtype=self.a1.dtype, device=self.a1.device)
        L.dpp_linear(kv0, a2.view(B, self.N, C), w_kv, b_kv)
        for p in range(self.P):
            if self.kv[p] is None:
                self.kv[p] = torch.empty_like(kv0)
            self.kv[p].copy_(kv0)

    def patch_step(self, p, x_patch, gamma, beta, conv_w, conv_b, w_q, b_q, w_kv, b_kv, w_o, b_o,
                   next_gn_partials=None):
        """Patch p's share of the current step; returns the out projection
        [B, R*W, C] (a buffer reused by the next call).  With
        next_gn_partials ([B, dpp_linear_gn_chunks(B, R*W, C), G', 2]) the out
        projection also writes the GroupNorm partial sums of its output for
        the next block's GroupNorm (dpp_groupnorm_stale_presummed)."""
        B, C, Nq = self.B, self.C, self.Nq
        r0 = p * self.R
        L.dpp_groupnorm_silu_stale(self.y1, self.stats_next, x_patch, self.stats_prev, gamma, beta, self.H, self.G,
                                   self.P, p, self.eps, self.gn_ws)
        L.dpp_conv3x3_halo(self.y2, self.y1, self.a1, conv_w, conv_b, self.H, r0, workspace=self.conv_ws)
        tok = self.y2.view(B, Nq, C)
        L.dpp_linear(self.q, tok, w_q, b_q)
        kv = self.kv[p]
        L.dpp_linear(kv[:, r0 * self.W:r0 * self.W + Nq, :], tok, w_kv, b_kv)
        L.dpp_self_attn_displaced(self.o, self.q, kv[:, :, :C], kv[:, :, C:], self.heads, self.D, 0.0, self.attn_ws)
        if next_gn_partials is None:
            L.dpp_linear(self.out, self.o, w_o, b_o)
        else:
            L.dpp_linear_gn(self.out, next_gn_partials, self.o, w_o, b_o)
        return self.out


class ComponentChain:
    """Asynchronous denoising over K full-image components (AsyncDiff
    abstract): the noise-prediction model is cut into components, one per
    device; after the warm-up, component k at step t consumes the output that
    component k-1 produced at step t-1, so on K devices all components run at
    once.  One device's work per step is one component: GroupNorm -> 3x3 conv
    -> self-attention over the whole image (one patch, identity projections,
    Q = K = V = the conv output), through the same kernels as the displaced
    layer.  This class runs the K components of a step one after the other on
    the current stream; outputs are kept per component for the next step.
    """

    def __init__(self, K, B, H, W, C, G, heads, dtype, device="cuda", eps=1e-5, head_dim=64):
        self.K, self.B, self.H, self.W, self.C, self.G = K, B, H, W, C, G
        self.heads, self.D, self.eps = heads, head_dim, eps
        act = dict(dtype=dtype, device=device)
        self.y1 = [torch.empty(B, H, W, C, **act) for _ in range(K)]
        self.y2 = [torch.empty(B, H, W, C, **act) for _ in range(K)]
        self.out = [torch.empty(B, H, W, C, **act) for _ in range(K)]     # this step
        self.prev = [torch.empty(B, H, W, C, **act) for _ in range(K)]    # previous step
        self._stats = torch.empty(B, 1, G, 2, dtype=torch.float32, device=device)
        gw = L.dpp_groupnorm_stale_workspace_bytes(B, H, W, C, G)
        self.gn_ws = torch.empty(max(gw, 256), dtype=torch.uint8, device=device)
        aw = L.dpp_self_attn_workspace_bytes(B, H * W, H * W, heads, head_dim,
                                             L.DPP_BF16 if dtype == torch.bfloat16 else L.DPP_F32)
        self.attn_ws = torch.empty(aw, dtype=torch.uint8, device=device) if aw else None
        cw = L.dpp_conv3x3_halo_workspace_bytes(B, H, W, C, C) if dtype == torch.bfloat16 else 0
        self.conv_ws = torch.empty(cw, dtype=torch.uint8, device=device) if cw else None
        self._steps = 0

    def component(self, k, x, gamma, beta, weight, bias):
        """Component k on input x [B,H,W,C]; output in self.out[k]."""
        L.dpp_groupnorm_stale(self.y1[k], self._stats, x, None, gamma, beta, self.H, self.G, 1, 0, self.eps,
                              self.gn_ws)
        L.dpp_conv3x3_halo(self.y2[k], self.y1[k], None, weight, bias, self.H, 0, workspace=self.conv_ws)
        t = self.y2[k].view(self.B, self.H * self.W, self.C)
        L.dpp_self_attn_displaced(self.out[k].view(self.B, self.H * self.W, self.C), t, t, t, self.heads, self.D,
                                  0.0, self.attn_ws)
        return self.out[k]

    def step(self, x, params, synchronous=False):
        """One denoising step.  params: K tuples (gamma, beta, weight, bias).
        synchronous (the warm-up): component k takes component k-1's output
        of this step; otherwise the one of the previous step.  Returns the
        last component's output (valid until the next step).  The first
        step must be synchronous: there is no previous output yet."""
        if self._steps == 0 and not synchronous and self.K > 1:
            raise ValueError("the first step of a component chain must be synchronous")
        self._steps += 1
        for k in range(self.K):
            src = x if k == 0 else (self.out[k - 1] if synchronous else self.prev[k - 1])
            self.component(k, src, *params[k])
        self.out, self.prev = self.prev, self.out
        return self.prev[self.K - 1]
