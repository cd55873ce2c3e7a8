"""ctypes binding of libdpp (include/dpp.h).

Argument marshalling only: each Python function has the name of the C entry
point, takes device tensors instead of pointers, reads sizes from their shapes,
passes the current HIP stream, and raises DppError on a non-zero status.  All
computation happens in the library's HIP kernels.  Importing this module
fails loudly when libdpp.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpp.so")

DPP_BF16 = 0
DPP_F32 = 1

STATUS = {
    0: "DPP_OK", -1: "DPP_ERR_NULL", -2: "DPP_ERR_SHAPE", -3: "DPP_ERR_DTYPE", -4: "DPP_ERR_ALIGN",
    -5: "DPP_ERR_ALIAS", -6: "DPP_ERR_WORKSPACE", -7: "DPP_ERR_UNSUPPORTED", -8: "DPP_ERR_LAUNCH",
}

# Every symbol include/dpp.h declares: name -> (restype, argtypes)
_vp, _i64, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "dpp_strerror": (ctypes.c_char_p, [_i]),
    "dpp_version": (_i, []),
    "dpp_splice_patch": (_i, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp]),
    "dpp_groupnorm_stale_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "dpp_groupnorm_stale": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _f,
                                 _vp, _sz, _i, _vp]),
    "dpp_groupnorm_silu_stale": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _f, _vp, _sz, _i, _vp]),
    "dpp_groupnorm_stale_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                         _i64, _f, _i, _vp]),
    "dpp_conv3x3_halo": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp]),
    "dpp_conv3x3_halo_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "dpp_conv3x3_halo_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _sz, _i,
                                 _vp]),
    "dpp_self_attn_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i]),
    "dpp_self_attn_displaced": (_i, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _f, _vp, _sz,
                                     _i, _vp]),
    "dpp_linear": (_i, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp]),
    "dpp_cfg_combine_workspace_bytes": (_sz, [_i64]),
    "dpp_cfg_combine_relmae": (_i, [_vp, _vp, _vp, _vp, _i64, _f, _vp, _sz, _i, _vp]),
    "dpp_hybrid_schedule": (_i, [_vp, _i64, _f, _f, _i64, _vp, _vp, _vp]),
    "dpp_groupnorm_stale_presummed": (_i, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                           _i64, _i64, _i64, _f, _i, _i, _vp]),
    "dpp_conv3x3_halo_gn_chunks": (_i64, [_i64, _i64, _i64]),
    "dpp_conv3x3_halo_gn": (_i, [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i,
                                 _vp]),
    "dpp_linear_gn_chunks": (_i64, [_i64, _i64, _i64]),
    "dpp_linear_gn": (_i, [_vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp]),
}


class DppError(RuntimeError):
    def __init__(self, name: str, status: int):
        self.status = status
        super().__init__(f"{name} -> {status} ({STATUS.get(status, '?')})")


def _load():
    # PyTorch brings its own HIP runtime (libamdhip64.so.7 under torch/lib).
    # Loading it first makes libdpp's libamdhip64.so.7 dependency resolve to
    # that same runtime; otherwise the process would hold two HIP runtimes and
    # torch's streams and allocations would be foreign to libdpp's launches.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdpp.so not built at {LIB_PATH}: run `python displaced_patch_parallelism_net_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _check(name, status):
    if status != 0:
        raise DppError(name, status)


def _dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DPP_BF16
    if t.dtype == torch.float32:
        return DPP_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    """Device pointer of a GPU tensor (None -> NULL).  A host tensor is
    refused here: the kernels would dereference its address on the GPU."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _same_dtype(*ts):
    ts = [t for t in ts if t is not None]
    if any(t.dtype != ts[0].dtype for t in ts):
        raise TypeError("activation and weight tensors must share one dtype: " + ", ".join(str(t.dtype) for t in ts))


def _f32(*ts):
    import torch
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"statistics, affine parameters and biases are float32, got {t.dtype}")


def _shape(t, want, what):
    if t is not None and tuple(t.shape) != tuple(want):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(want)}")


def _numel(t, n, what):
    if t is not None and t.numel() != n:
        raise ValueError(f"{what}: {t.numel()} elements, expected {n}")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


# ------------------------------------------------------------------ calls
def dpp_splice_patch(full, patch, row0: int, stream=None):
    _contig(full, patch)
    _same_dtype(full, patch)
    B, H, W, C = full.shape
    rows = patch.shape[1]
    _shape(patch, (B, rows, W, C), "patch")
    _check("dpp_splice_patch", LIB.dpp_splice_patch(_ptr(full), _ptr(patch), B, H, W, C, row0, rows, _dtype(full),
                                                    _stream(stream)))


def dpp_groupnorm_stale_workspace_bytes(B, rows, W, C, G) -> int:
    return int(LIB.dpp_groupnorm_stale_workspace_bytes(B, rows, W, C, G))


def _gn_args(y, stats_out, x, stale_stats, gamma, beta, G, P):
    """The library indexes both statistics arrays as [B,P,G,2] with the P and
    G it is passed, so anything but exactly that shape is refused here."""
    _contig(y, stats_out, x, stale_stats, gamma, beta)
    _same_dtype(y, x)
    _f32(stats_out, stale_stats, gamma, beta)
    B, rows, W, C = x.shape
    _shape(y, x.shape, "y")
    _numel(gamma, C, "gamma")
    _numel(beta, C, "beta")
    for t, what in ((stats_out, "stats_out"), (stale_stats, "stale_stats")):
        _shape(t, (B, P, G, 2), what)


def dpp_groupnorm_stale(y, stats_out, x, stale_stats, gamma, beta, H: int, G: int, P: int, p: int, eps: float,
                        workspace, stream=None):
    _gn_args(y, stats_out, x, stale_stats, gamma, beta, G, P)
    B, rows, W, C = x.shape
    _check("dpp_groupnorm_stale",
           LIB.dpp_groupnorm_stale(_ptr(y), _ptr(stats_out), _ptr(x), _ptr(stale_stats), _ptr(gamma), _ptr(beta), B, H,
                                   W, C, G, P, p, rows, eps, _ptr(workspace),
                                   0 if workspace is None else workspace.numel() * workspace.element_size(),
                                   _dtype(x), _stream(stream)))


def dpp_groupnorm_silu_stale(y, stats_out, x, stale_stats, gamma, beta, H: int, G: int, P: int, p: int, eps: float,
                             workspace, stream=None):
    _gn_args(y, stats_out, x, stale_stats, gamma, beta, G, P)
    B, rows, W, C = x.shape
    _check("dpp_groupnorm_silu_stale",
           LIB.dpp_groupnorm_silu_stale(_ptr(y), _ptr(stats_out), _ptr(x), _ptr(stale_stats), _ptr(gamma), _ptr(beta),
                                        B, H, W, C, G, P, p, rows, eps, _ptr(workspace),
                                        0 if workspace is None else workspace.numel() * workspace.element_size(),
                                        _dtype(x), _stream(stream)))


GN_NOALLOC_MAX_BYTES = 1 << 20   # DPP_GN_NOALLOC_MAX_BYTES


def dpp_groupnorm_stale_noalloc(y, stats_out, x, stale_stats, gamma, beta, H: int, G: int, P: int, p: int,
                                eps: float, stream=None):
    """dpp_groupnorm_stale with the library's static per-device scratch
    instead of a caller workspace (no device allocation in the call)."""
    _gn_args(y, stats_out, x, stale_stats, gamma, beta, G, P)
    B, rows, W, C = x.shape
    _check("dpp_groupnorm_stale_noalloc",
           LIB.dpp_groupnorm_stale_noalloc(_ptr(y), _ptr(stats_out), _ptr(x), _ptr(stale_stats), _ptr(gamma),
                                           _ptr(beta), B, H, W, C, G, P, p, rows, eps, _dtype(x), _stream(stream)))


def dpp_groupnorm_stale_presummed(y, stats_out, x, partials, stale_stats, gamma, beta, H: int, G: int, P: int, p: int,
                                  eps: float, silu: bool = False, stream=None):
    """GroupNorm of x with the fresh sums taken from partials [B,nchunk,G,2]
    written by the producer of x (dpp_conv3x3_halo_gn, dpp_linear_gn)."""
    _gn_args(y, stats_out, x, stale_stats, gamma, beta, G, P)
    _contig(partials)
    _f32(partials)
    B, rows, W, C = x.shape
    if partials.dim() != 4 or tuple(partials.shape[::2]) != (B, G) or partials.shape[3] != 2:
        raise ValueError(f"partials: shape {tuple(partials.shape)}, expected [B, nchunk, G, 2] with B = {B}, G = {G}")
    _check("dpp_groupnorm_stale_presummed",
           LIB.dpp_groupnorm_stale_presummed(_ptr(y), _ptr(stats_out), _ptr(x), _ptr(partials), partials.shape[1],
                                             _ptr(stale_stats), _ptr(gamma), _ptr(beta), B, H, W, C, G, P, p, rows,
                                             eps, 1 if silu else 0, _dtype(x), _stream(stream)))


def dpp_conv3x3_halo_gn_chunks(rows, W, Cout) -> int:
    return int(LIB.dpp_conv3x3_halo_gn_chunks(rows, W, Cout))


def dpp_conv3x3_halo_gn(y, gn_partials, x, stale_full, weight, bias, H: int, row0: int, stream=None):
    """dpp_conv3x3_halo plus the GroupNorm partial sums of y,
    gn_partials [B, dpp_conv3x3_halo_gn_chunks(rows, W, Cout), G, 2]."""
    _contig(y, x, stale_full, weight, bias, gn_partials)
    _same_dtype(y, x, stale_full, weight)
    _f32(bias, gn_partials)
    B, rows, W, Cin = x.shape
    Cout = weight.shape[0]
    _shape(weight, (Cout, 3, 3, Cin), "weight")
    _shape(y, (B, rows, W, Cout), "y")
    _shape(stale_full, (B, H, W, Cin), "stale_full")
    _numel(bias, Cout, "bias")
    if gn_partials.dim() != 4:
        raise ValueError("gn_partials must be [B, nchunk, G, 2]")
    G = gn_partials.shape[2]
    _shape(gn_partials, (B, dpp_conv3x3_halo_gn_chunks(rows, W, Cout), G, 2), "gn_partials")
    _check("dpp_conv3x3_halo_gn",
           LIB.dpp_conv3x3_halo_gn(_ptr(y), _ptr(gn_partials), G, _ptr(x), _ptr(stale_full), _ptr(weight), _ptr(bias),
                                   B, H, W, Cin, Cout, row0, rows, _dtype(x), _stream(stream)))


def dpp_linear_gn_chunks(B, M, N) -> int:
    return int(LIB.dpp_linear_gn_chunks(B, M, N))


def _lin3(y, x, w, bias):
    _contig(w, bias)
    _same_dtype(y, x, w)
    _f32(bias)
    x3 = x if x.dim() == 3 else x.unsqueeze(0)
    y3 = y if y.dim() == 3 else y.unsqueeze(0)
    B, M, K = x3.shape
    N = w.shape[0]
    if tuple(y3.shape) != (B, M, N) or tuple(w.shape) != (N, K):
        raise ValueError(f"shape mismatch: x {tuple(x3.shape)}, w {tuple(w.shape)}, y {tuple(y3.shape)}")
    if x3.stride(2) != 1 or y3.stride(2) != 1:
        raise ValueError("last dimension of x and y must be contiguous")
    _numel(bias, N, "bias")
    return x3, y3, B, M, K, N


def dpp_linear_gn(y, gn_partials, x, w, bias=None, stream=None):
    """dpp_linear plus the GroupNorm partial sums of y,
    gn_partials [B, dpp_linear_gn_chunks(B, M, N), G, 2]."""
    x3, y3, B, M, K, N = _lin3(y, x, w, bias)
    _contig(gn_partials)
    _f32(gn_partials)
    if gn_partials.dim() != 4:
        raise ValueError("gn_partials must be [B, nchunk, G, 2]")
    G = gn_partials.shape[2]
    _shape(gn_partials, (B, dpp_linear_gn_chunks(B, M, N), G, 2), "gn_partials")
    _check("dpp_linear_gn", LIB.dpp_linear_gn(_ptr(y3), _ptr(gn_partials), G, _ptr(x3), _ptr(w), _ptr(bias), B, M, K,
                                              N, x3.stride(1), x3.stride(0), y3.stride(1), y3.stride(0), _dtype(x),
                                              _stream(stream)))


def dpp_linear(y, x, w, bias=None, stream=None):
    """y = x w^T + bias over the last dimension.  x [M,K] or [B,M,K] and y
    [M,N] or [B,M,N] may be strided views (last dimension contiguous), e.g. y
    a row band of a larger K/V buffer; w [N,K] contiguous; bias [N] float32."""
    x3, y3, B, M, K, N = _lin3(y, x, w, bias)
    _check("dpp_linear", LIB.dpp_linear(_ptr(y3), _ptr(x3), _ptr(w), _ptr(bias), B, M, K, N, x3.stride(1),
                                        x3.stride(0), y3.stride(1), y3.stride(0), _dtype(x), _stream(stream)))


def dpp_conv3x3_halo_workspace_bytes(B, rows, W, Cin, Cout) -> int:
    return int(LIB.dpp_conv3x3_halo_workspace_bytes(B, rows, W, Cin, Cout))


def dpp_conv3x3_halo(y, x, stale_full, weight, bias, H: int, row0: int, workspace=None, stream=None):
    """With a workspace (dpp_conv3x3_halo_workspace_bytes) small patches may
    split the input channels across workgroups (dpp_conv3x3_halo_ws)."""
    _contig(y, x, stale_full, weight, bias)
    _same_dtype(y, x, stale_full, weight)
    _f32(bias)
    B, rows, W, Cin = x.shape
    Cout = weight.shape[0]
    _shape(weight, (Cout, 3, 3, Cin), "weight")
    _shape(y, (B, rows, W, Cout), "y")
    _shape(stale_full, (B, H, W, Cin), "stale_full")
    _numel(bias, Cout, "bias")
    if workspace is None:
        _check("dpp_conv3x3_halo",
               LIB.dpp_conv3x3_halo(_ptr(y), _ptr(x), _ptr(stale_full), _ptr(weight), _ptr(bias), B, H, W, Cin, Cout,
                                    row0, rows, _dtype(x), _stream(stream)))
    else:
        _check("dpp_conv3x3_halo_ws",
               LIB.dpp_conv3x3_halo_ws(_ptr(y), _ptr(x), _ptr(stale_full), _ptr(weight), _ptr(bias), B, H, W, Cin,
                                       Cout, row0, rows, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _dtype(x), _stream(stream)))


def dpp_self_attn_workspace_bytes(B, n_q, n_kv, heads, head_dim, dtype) -> int:
    return int(LIB.dpp_self_attn_workspace_bytes(B, n_q, n_kv, heads, head_dim, dtype))


def dpp_self_attn_displaced(o, q, k, v, heads: int, head_dim: int = 64, scale: float = 0.0, workspace=None,
                            stream=None):
    """q [B,n_q,*], k/v [B,n_kv,*], o [B,n_q,*]; row strides from the tensors
    (last dimension contiguous, batch stride = rows * row stride)."""
    for t in (o, q, k, v):
        if t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError("attention tensors must be [B,N,ld] row-major with unit channel stride")
    _same_dtype(o, q, k, v)
    B, n_q = q.shape[0], q.shape[1]
    n_kv = k.shape[1]
    hd = heads * head_dim
    if tuple(o.shape[:2]) != (B, n_q) or tuple(k.shape[:2]) != (B, n_kv) or tuple(v.shape[:2]) != (B, n_kv):
        raise ValueError(f"shape mismatch: o {tuple(o.shape)}, q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    if min(o.shape[2], q.shape[2], k.shape[2], v.shape[2]) < hd or k.stride(1) != v.stride(1):
        raise ValueError(f"rows must hold heads * head_dim = {hd} channels, k and v one row stride")
    _check("dpp_self_attn_displaced",
           LIB.dpp_self_attn_displaced(_ptr(o), _ptr(q), _ptr(k), _ptr(v), B, n_q, n_kv, heads, head_dim, q.stride(1),
                                       k.stride(1), o.stride(1), scale, _ptr(workspace),
                                       0 if workspace is None else workspace.numel() * workspace.element_size(),
                                       _dtype(q), _stream(stream)))


def dpp_cfg_combine_workspace_bytes(n) -> int:
    return int(LIB.dpp_cfg_combine_workspace_bytes(n))


def dpp_cfg_combine_relmae(eps, relmae, eps_c, eps_u, guidance: float, workspace=None, stream=None):
    _contig(eps, eps_c, eps_u)
    _same_dtype(eps, eps_c, eps_u)
    _f32(relmae)
    n = eps_c.numel()
    _numel(eps, n, "eps")
    _numel(eps_u, n, "eps_u")
    _check("dpp_cfg_combine_relmae",
           LIB.dpp_cfg_combine_relmae(_ptr(eps), _ptr(relmae), _ptr(eps_c), _ptr(eps_u), n, guidance, _ptr(workspace),
                                      0 if workspace is None else workspace.numel() * workspace.element_size(),
                                      _dtype(eps_c), _stream(stream)))


def dpp_hybrid_schedule(relmae, rho: float = 0.25, eps: float = 0.02, min_warmup: int = 1):
    """Stages (0 warm-up, 1 parallel, 2 fully-connecting) for a host
    sequence of per-step rel-MAE values; returns (stage int32 array, tau1,
    tau2).  Host-only call."""
    import numpy as np
    d = np.ascontiguousarray(relmae, dtype=np.float32)
    T = d.shape[0]
    stage = np.empty(T, dtype=np.int32)
    t1, t2 = ctypes.c_int64(), ctypes.c_int64()
    _check("dpp_hybrid_schedule", LIB.dpp_hybrid_schedule(d.ctypes.data_as(ctypes.c_void_p), T, rho, eps, min_warmup,
                                                          stage.ctypes.data_as(ctypes.c_void_p), ctypes.byref(t1),
                                                          ctypes.byref(t2)))
    return stage, t1.value, t2.value


def dpp_strerror(status: int) -> str:
    return LIB.dpp_strerror(status).decode()


def dpp_version() -> int:
    return int(LIB.dpp_version())
