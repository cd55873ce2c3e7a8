"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments with the documented status
before touching the device (these calls never launch anything, so they run
without a GPU).  Pointers here are fake aligned addresses: validation reads no
memory."""
import ctypes
import os
import re

import pytest

import displaced_patch_parallelism_net_amd as dpp
from displaced_patch_parallelism_net_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.LIB
OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WS, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7
BF16, F32 = 0, 1
A = 0x10000000        # fake 16-byte aligned device addresses, far apart
Bp = 0x20000000
Cp = 0x30000000
Dp = 0x40000000
Ep = 0x50000000
WSP = 0x60000000


def _no_launch(rc):
    # the helpers pass fake device addresses: every call must stop at a
    # validation check, never at (or past) a kernel launch
    assert rc not in (OK, -8), f"validation let a call with fake pointers through (status {rc})"
    return rc


def header_symbols():
    text = open(os.path.join(ROOT, "include", "dpp.h")).read()
    return sorted(set(re.findall(r"\b(dpp_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    syms = header_symbols()
    assert len(syms) == 21, syms
    for s in syms:
        assert hasattr(L, s), s
        assert s in _lib.SIGNATURES, s
    assert set(_lib.SIGNATURES) == set(syms)


def test_exported_symbols_via_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dpp_[a-z0-9_]+)", out))
    assert set(header_symbols()) <= exported


def test_version_and_strerror():
    assert dpp.dpp_version() == 1
    for code in range(0, -9, -1):
        assert dpp.dpp_strerror(code).startswith("DPP")
    assert "unknown" in dpp.dpp_strerror(17)


# ----------------------------------------------------------------- splice
def splice(full=A, patch=Bp, B=1, H=8, W=4, C=16, row0=0, rows=2, dtype=BF16):
    return _no_launch(L.dpp_splice_patch(full, patch, B, H, W, C, row0, rows, dtype, None))


def test_splice_validation():
    assert splice(dtype=7) == DTYPE
    assert splice(full=None) == NULL
    assert splice(patch=None) == NULL
    assert splice(rows=0) == SHAPE
    assert splice(row0=-1) == SHAPE
    assert splice(row0=7, rows=2) == SHAPE
    assert splice(W=0) == SHAPE
    assert splice(patch=A + 64) == ALIAS          # patch inside the full buffer
    assert splice(B=70000) == UNSUP


# ----------------------------------------------------------------- GroupNorm
def gn(y=A, so=Bp, x=Cp, st=Dp, gamma=Ep, beta=Ep + 4096, B=1, H=8, W=4, C=64, G=8, P=2, p=0, rows=4, eps=1e-5,
       ws=WSP, wsb=1 << 20, dtype=BF16):
    return _no_launch(L.dpp_groupnorm_stale(y, so, x, st, gamma, beta, B, H, W, C, G, P, p, rows, eps, ws, wsb, dtype, None))


def test_groupnorm_validation():
    assert gn(dtype=2) == DTYPE
    assert gn(x=None) == NULL
    assert gn(so=None) == NULL
    assert gn(gamma=None) == NULL
    assert gn(st=None) == NULL                     # P > 1 needs stale sums
    assert gn(C=60, G=8) == SHAPE                  # C % G
    assert gn(p=2) == SHAPE
    assert gn(rows=9) == SHAPE
    assert gn(eps=-1.0) == SHAPE
    assert gn(C=20, G=4) == UNSUP                  # bf16 needs C % 8
    assert gn(C=4096, G=32) == UNSUP               # more than 256 vectors per pixel
    assert gn(x=Cp + 2) == ALIGN
    assert gn(y=A + 8) == ALIGN
    assert gn(so=Dp) == ALIAS                      # stats_out == stale_stats
    assert gn(y=Cp) == ALIAS                       # in place is not allowed
    assert gn(ws=None) == WS
    assert gn(wsb=16) == WS
    assert gn(ws=Cp) == ALIAS


def test_groupnorm_stats_only_mode_needs_no_affine():
    # y == NULL: gamma/beta/stale may be NULL; validation passes all the way
    # to the workspace check
    assert gn(y=None, gamma=None, beta=None, st=None, ws=None) == WS
    assert gn(y=None, st=None, P=1, wsb=8) == WS   # gets past every pointer check; never reaches a launch


def test_groupnorm_workspace_query():
    assert dpp.dpp_groupnorm_stale_workspace_bytes(1, 30, 240, 640, 32) > 0
    assert dpp.dpp_groupnorm_stale_workspace_bytes(1, 30, 240, 630, 32) == 0
    assert dpp.dpp_groupnorm_stale_workspace_bytes(0, 30, 240, 640, 32) == 0


# ----------------------------------------------------------------- conv
def conv(y=A, x=Bp, st=Cp, w=Dp, bias=Ep, B=1, H=8, W=16, Cin=64, Cout=64, row0=2, rows=2, dtype=BF16):
    return _no_launch(L.dpp_conv3x3_halo(y, x, st, w, bias, B, H, W, Cin, Cout, row0, rows, dtype, None))


def test_conv_validation():
    assert conv(dtype=-1) == DTYPE
    assert conv(y=None) == NULL
    assert conv(w=None) == NULL
    assert conv(st=None) == NULL                   # halos inside the image need the stale image
    assert conv(row0=6, rows=3) == SHAPE
    assert conv(Cout=0) == SHAPE
    assert conv(Cin=32) == UNSUP                   # bf16 needs Cin % 64
    assert conv(Cout=24) == UNSUP                  # bf16 needs Cout % 16
    assert conv(W=1 << 21, Cin=640) == UNSUP       # bf16 image-row byte offsets are 32-bit
    assert conv(Cin=1 << 18, Cout=512) == UNSUP    # and so are weight byte offsets
    assert conv(x=Bp + 4) == ALIGN
    assert conv(y=Bp) == ALIAS
    assert conv(y=Cp + 256) == ALIAS               # inside the stale image
    assert conv(y=Dp) == ALIAS
    # f32 has no divisibility or alignment requirement
    assert conv(Cin=3, Cout=5, dtype=F32, x=None) == NULL


def test_conv_workspace_query_and_alias():
    # the 3840 px 8-patch band fills the GPU unsplit; the 16-patch band
    # splits in two, the 1024 px band in five; full images never split (the
    # float32 partials would cost more than the idle CUs)
    assert dpp.dpp_conv3x3_halo_workspace_bytes(1, 30, 240, 640, 640) == 0
    assert dpp.dpp_conv3x3_halo_workspace_bytes(1, 15, 240, 640, 640) == 2 * 15 * 240 * 640 * 4
    assert dpp.dpp_conv3x3_halo_workspace_bytes(1, 16, 64, 640, 640) == 5 * 16 * 64 * 640 * 4
    for hw in (64, 128, 240):
        assert dpp.dpp_conv3x3_halo_workspace_bytes(1, hw, hw, 640, 640) == 0
    assert dpp.dpp_conv3x3_halo_workspace_bytes(1, 128, 128, 320, 320) == 0
    assert dpp.dpp_conv3x3_halo_workspace_bytes(1, 16, 64, 630, 640) == 0   # Cin % 64 != 0
    ws_rc = _no_launch(L.dpp_conv3x3_halo_ws(A, Bp, Cp, Dp, Ep, 1, 8, 16, 64, 64, 2, 2, A + 64, 1 << 20, BF16, None))
    assert ws_rc == ALIAS                                                    # workspace over y
    assert _no_launch(L.dpp_conv3x3_halo_ws(A, Bp, Cp, Dp, Ep, 1, 8, 16, 64, 64, 2, 2, WSP + 4, 1 << 20, BF16,
                                            None)) == ALIGN
    assert _no_launch(L.dpp_conv3x3_halo_ws(A, Bp, Cp, Dp, Ep, 1, 8, 16, 64, 64, 2, 2, None, 0, 7, None)) == DTYPE


def test_conv_whole_image_needs_no_stale():
    assert conv(st=None, row0=0, rows=8, y=None) == NULL   # reaches the pointer checks only
    assert conv(st=None, row0=0, rows=7) == NULL


# ----------------------------------------------------------------- attention
def attn(o=A, q=Bp, k=Cp, v=Dp, B=1, nq=100, nkv=300, heads=2, D=64, ldq=128, ldkv=128, ldo=128, scale=0.0, ws=None,
         wsb=0, dtype=BF16):
    return _no_launch(L.dpp_self_attn_displaced(o, q, k, v, B, nq, nkv, heads, D, ldq, ldkv, ldo, scale, ws, wsb, dtype, None))


def test_attention_validation():
    assert attn(dtype=3) == DTYPE
    assert attn(q=None) == NULL
    assert attn(v=None) == NULL
    assert attn(nq=0) == SHAPE
    assert attn(ldq=64) == SHAPE
    assert attn(D=32) == UNSUP                     # bf16 kernels are head_dim 64
    assert attn(D=48, dtype=F32, ldq=96, ldkv=96, ldo=96) == UNSUP
    assert attn(q=Bp + 2) == ALIGN
    assert attn(ldkv=132) == ALIGN
    assert attn(o=Cp) == ALIAS
    assert attn(o=Bp + 128) == ALIAS
    assert attn(ws=A, wsb=1024) == ALIAS


def test_attention_huge_row_stride_unsupported():
    big = (1 << 24) + 8
    assert attn(ldkv=big) == UNSUP
    assert attn(ldq=big) == UNSUP
    assert attn(ldo=big) == UNSUP


def test_attention_workspace_query():
    # short query ranges are split over the keys; the split needs workspace
    assert dpp.dpp_self_attn_workspace_bytes(1, 1024, 4096, 10, 64, BF16) > 0
    assert dpp.dpp_self_attn_workspace_bytes(1, 1024, 4096, 10, 64, F32) == 0
    assert dpp.dpp_self_attn_workspace_bytes(1, 1024, 4096, 10, 32, BF16) == 0
    assert dpp.dpp_self_attn_workspace_bytes(1, 0, 4096, 10, 64, BF16) == 0


# ----------------------------------------------------------------- CFG
def cfg(eps=A, rel=Bp, c=Cp, u=Dp, n=1000, w=7.5, ws=WSP, wsb=1 << 16, dtype=BF16):
    return _no_launch(L.dpp_cfg_combine_relmae(eps, rel, c, u, n, w, ws, wsb, dtype, None))


def test_cfg_validation():
    assert cfg(dtype=5) == DTYPE
    assert cfg(c=None) == NULL
    assert cfg(n=0) == SHAPE
    assert cfg(eps=Cp + 2) == ALIAS                # partial overlap with eps_c
    assert cfg(ws=None) == WS
    assert cfg(wsb=8) == WS
    assert cfg(ws=A) == ALIAS
    assert cfg(rel=A + 16) == ALIAS
    # relmae == NULL skips the reduction: no workspace needed (reaches launch)
    assert dpp.dpp_cfg_combine_workspace_bytes(1 << 16) >= 16
    assert dpp.dpp_cfg_combine_workspace_bytes(0) == 0


def test_binding_raises_on_error_status():
    with pytest.raises(dpp.DppError) as ei:
        _lib._check("dpp_splice_patch", -2)
    assert ei.value.status == -2


# ----------------------------------------------------------------- GroupNorm + SiLU
def test_groupnorm_silu_validation_matches_groupnorm():
    def gs(**kw):
        args = dict(y=A, so=Bp, x=Cp, st=Dp, gamma=Ep, beta=Ep + 4096, B=1, H=8, W=4, C=64, G=8, P=2, p=0, rows=4,
                    eps=1e-5, ws=WSP, wsb=1 << 20, dtype=BF16)
        args.update(kw)
        a = args
        return L.dpp_groupnorm_silu_stale(a["y"], a["so"], a["x"], a["st"], a["gamma"], a["beta"], a["B"], a["H"],
                                          a["W"], a["C"], a["G"], a["P"], a["p"], a["rows"], a["eps"], a["ws"],
                                          a["wsb"], a["dtype"], None)
    for kw, code in [(dict(dtype=2), DTYPE), (dict(x=None), NULL), (dict(gamma=None), NULL), (dict(C=60), SHAPE),
                     (dict(C=20, G=4), UNSUP), (dict(x=Cp + 2), ALIGN), (dict(y=Cp), ALIAS), (dict(ws=None), WS)]:
        assert gs(**kw) == code, kw
        assert gn(**kw) == code, kw


# ----------------------------------------------------------------- projections
def lin(y=A, x=Bp, w=Cp, bias=Dp, B=1, M=100, K=64, N=64, ldx=64, bsx=6400, ldy=64, bsy=6400, dtype=BF16):
    return _no_launch(L.dpp_linear(y, x, w, bias, B, M, K, N, ldx, bsx, ldy, bsy, dtype, None))


def test_linear_32bit_offset_limits():
    # w of 2^31 bytes and an x batch entry of 2^31 bytes need 64-bit offsets
    assert lin(N=32768, K=32768, ldx=32768, M=10, bsx=327680, ldy=32768, bsy=327680) == UNSUP
    assert lin(M=1 << 20, K=1024, ldx=1024, bsx=1 << 30, ldy=64, bsy=64 << 20) == UNSUP
    # a w just inside the limit passes the size checks: with y placed inside w
    # the aliasing check, which comes after them, is the one that answers (no
    # host test may reach a launch: these pointers are not device memory)
    assert lin(N=7932, K=1 << 17, ldx=1 << 17, M=4, bsx=1 << 19, ldy=8064, bsy=1 << 15, y=Cp + 64) == ALIAS
    assert lin(N=7936, K=1 << 17, ldx=1 << 17, M=4, bsx=1 << 19, ldy=8064, bsy=1 << 15, y=Cp + 64) == UNSUP


def test_linear_validation():
    assert lin(dtype=3) == DTYPE
    assert lin(y=None) == NULL
    assert lin(x=None) == NULL
    assert lin(w=None) == NULL
    assert lin(bias=None, x=None) == NULL          # bias is optional; x is not
    assert lin(M=0) == SHAPE
    assert lin(ldx=32) == SHAPE                    # ld_x < K
    assert lin(ldy=32) == SHAPE                    # ld_y < N
    assert lin(B=2, bsy=64) == SHAPE               # output batches overlap
    assert lin(B=70000, bsy=1 << 20) == UNSUP
    assert lin(K=60, ldx=64) == UNSUP              # bf16 needs K % 8
    assert lin(N=62, ldy=64) == UNSUP              # bf16 needs N % 4
    assert lin(x=Bp + 8) == ALIGN
    assert lin(ldx=68) == ALIGN                    # row stride not a multiple of 8 elements
    assert lin(y=A + 2) == ALIGN
    assert lin(y=Bp) == ALIAS                      # in place
    assert lin(y=Cp + 64) == ALIAS                 # inside the weights
    # f32: no divisibility or alignment requirement beyond the shapes
    assert lin(K=60, ldx=60, N=62, ldy=62, bsx=6000, bsy=6200, dtype=F32, w=None) == NULL


# ----------------------------------------------------------------- binding checks (no GPU needed)
def test_binding_refuses_host_tensors_and_mismatches():
    import torch
    bf = torch.bfloat16
    full, patch = torch.zeros(1, 8, 4, 16, dtype=bf), torch.zeros(1, 2, 4, 16, dtype=bf)
    with pytest.raises(ValueError, match="GPU"):
        dpp.dpp_splice_patch(full, patch, 0)
    with pytest.raises(ValueError, match="patch"):
        dpp.dpp_splice_patch(full, torch.zeros(1, 2, 4, 8, dtype=bf), 0)
    with pytest.raises(TypeError):
        dpp.dpp_splice_patch(full, patch.float(), 0)
    x, w = torch.zeros(1, 2, 4, 64, dtype=bf), torch.zeros(64, 3, 3, 64, dtype=bf)
    with pytest.raises(ValueError, match="weight"):
        dpp.dpp_conv3x3_halo(torch.zeros(1, 2, 4, 64, dtype=bf), x, None, torch.zeros(64, 2, 3, 64, dtype=bf), None, 2, 0)
    with pytest.raises(ValueError, match="y"):
        dpp.dpp_conv3x3_halo(torch.zeros(1, 2, 4, 32, dtype=bf), x, None, w, None, 2, 0)
    with pytest.raises(TypeError):
        dpp.dpp_conv3x3_halo(torch.zeros(1, 2, 4, 64, dtype=bf), x, None, w, torch.zeros(64, dtype=bf), 2, 0)
    g = torch.ones(64)
    with pytest.raises(TypeError):
        dpp.dpp_groupnorm_stale(x.clone(), None, x, None, g.to(bf), g, 2, 8, 1, 0, 1e-5, None)
    with pytest.raises(ValueError, match="stats_out"):
        dpp.dpp_groupnorm_stale(x.clone(), torch.zeros(1, 1, 8, 3), x, None, g, g, 2, 8, 1, 0, 1e-5, None)
    q, kv = torch.zeros(1, 8, 64, dtype=bf), torch.zeros(1, 16, 128, dtype=bf)
    with pytest.raises(ValueError, match="row stride"):
        dpp.dpp_self_attn_displaced(q.clone(), q, kv[:, :, :64], torch.zeros(1, 16, 64, dtype=bf), 1)
    with pytest.raises(ValueError, match="shape"):
        dpp.dpp_self_attn_displaced(torch.zeros(1, 4, 64, dtype=bf), q, kv, kv, 1)
    with pytest.raises(ValueError, match="eps"):
        dpp.dpp_cfg_combine_relmae(torch.zeros(10, dtype=bf), None, torch.zeros(12, dtype=bf),
                                   torch.zeros(12, dtype=bf), 7.5)
    with pytest.raises(ValueError, match="bias"):
        dpp.dpp_linear(torch.zeros(4, 8, dtype=bf), torch.zeros(4, 16, dtype=bf), torch.zeros(8, 16, dtype=bf),
                       torch.zeros(4))


def test_binding_requires_exact_statistics_shape():
    # The library indexes stats_out and stale_stats as [B,P,G,2] with the P
    # and G it is passed: fewer groups would be written past their end, more
    # patch slots (B > 1) in the wrong layout.  The binding refuses both.
    import torch
    bf = torch.bfloat16
    x = torch.zeros(2, 2, 4, 64, dtype=bf)
    g = torch.ones(64)
    good = torch.zeros(2, 3, 8, 2)
    for bad, what in ((torch.zeros(2, 3, 4, 2), "stats_out"),      # fewer groups than G
                      (torch.zeros(2, 4, 8, 2), "stats_out"),      # more patch slots than P
                      (torch.zeros(1, 3, 8, 2), "stats_out"),      # batch mismatch
                      (torch.zeros(2, 3, 8, 3), "stats_out")):     # not (sum, sum of squares)
        with pytest.raises(ValueError, match=what):
            dpp.dpp_groupnorm_stale(x.clone(), bad, x, good, g, g, 6, 8, 3, 1, 1e-5, None)
        with pytest.raises(ValueError, match=what):
            dpp.dpp_groupnorm_silu_stale(x.clone(), bad, x, good, g, g, 6, 8, 3, 1, 1e-5, None)
    for bad in (torch.zeros(2, 3, 16, 2), torch.zeros(2, 2, 8, 2)):
        with pytest.raises(ValueError, match="stale_stats"):
            dpp.dpp_groupnorm_stale(x.clone(), good, x, bad, g, g, 6, 8, 3, 1, 1e-5, None)
    # the exact shape passes every binding check and stops at the host-tensor check
    with pytest.raises(ValueError, match="GPU"):
        dpp.dpp_groupnorm_stale(x.clone(), good, x, torch.zeros(2, 3, 8, 2), g, g, 6, 8, 3, 1, 1e-5, None)


def gn_noalloc(y=A, so=Bp, x=Cp, st=Dp, gamma=Ep, beta=Ep + 4096, B=1, H=8, W=4, C=64, G=8, P=2, p=0, rows=4,
               eps=1e-5, dtype=BF16):
    return _no_launch(L.dpp_groupnorm_stale_noalloc(y, so, x, st, gamma, beta, B, H, W, C, G, P, p, rows, eps, dtype,
                                                    None))


def test_groupnorm_noalloc_validation():
    # the same argument checks as dpp_groupnorm_stale, before any HIP call
    assert gn_noalloc(dtype=2) == DTYPE
    assert gn_noalloc(x=None) == NULL
    assert gn_noalloc(st=None) == NULL
    assert gn_noalloc(C=60, G=8) == SHAPE
    assert gn_noalloc(p=2) == SHAPE
    assert gn_noalloc(C=20, G=4) == UNSUP
    assert gn_noalloc(x=Cp + 2) == ALIGN
    assert gn_noalloc(so=Dp) == ALIAS
    assert gn_noalloc(y=Cp) == ALIAS
    # shapes whose scratch exceeds the static array: refused, nothing launched
    need = dpp.dpp_groupnorm_stale_workspace_bytes(4097, 4, 4, 64, 32)
    assert need > _lib.GN_NOALLOC_MAX_BYTES
    assert gn_noalloc(B=4097, H=8, W=4, C=64, G=32, P=2, rows=4) == WS
    assert dpp.dpp_groupnorm_stale_workspace_bytes(4096, 4, 4, 64, 32) <= _lib.GN_NOALLOC_MAX_BYTES


def test_producer_statistics_and_presummed_validation():
    # conv with GroupNorm partials: the conv's own checks, then its own
    assert L.dpp_conv3x3_halo_gn_chunks(30, 240, 640) == 250          # 5 six-row tiles x 5 48-column tiles x 10 channel tiles
    assert L.dpp_conv3x3_halo_gn_chunks(240, 240, 640) == 2000        # six-row tiles: 40 x 5 x 10 (8 rounds of 288 px)
    assert L.dpp_conv3x3_halo_gn_chunks(6, 48, 64) == 2               # six rows fit, but two four-row tiles finish first
    assert L.dpp_conv3x3_halo_gn_chunks(28, 240, 640) == 210          # 7 four-row tiles x 3 x 10
    assert L.dpp_conv3x3_halo_gn_chunks(16, 64, 320) == 20            # 4 x 1 x 5
    assert L.dpp_linear_gn_chunks(1, 7200, 640) == 225                 # 45 token tiles x 5 channel tiles
    assert L.dpp_linear_gn_chunks(1, 7200, 1280) == 225                # 256-channel tiles: 45 x 5
    assert L.dpp_linear_gn_chunks(1, 1024, 640) == 65                  # few tiles: 80-token tiles, 13 x 5
    assert L.dpp_conv3x3_halo_gn_chunks(0, 240, 640) == 0

    def cgn(y=A, part=WSP, G=32, x=Bp, st=Cp, w=Dp, bias=Ep, B=1, H=8, W=16, Cin=64, Cout=64, row0=2, rows=2,
            dtype=BF16):
        return _no_launch(L.dpp_conv3x3_halo_gn(y, part, G, x, st, w, bias, B, H, W, Cin, Cout, row0, rows, dtype,
                                                None))
    assert cgn(part=None) == NULL
    assert cgn(G=0) == SHAPE
    assert cgn(G=24) == SHAPE                      # Cout % G
    assert cgn(dtype=F32, Cin=12, Cout=12, G=4) == UNSUP
    assert cgn(part=A + 64) == ALIAS               # inside y
    assert cgn(rows=0) == SHAPE                    # the conv's own checks first
    assert cgn(y=None) == NULL

    def lgn(y=A, part=WSP, G=32, x=Bp, w=Cp, bias=Dp, B=1, M=64, K=64, N=64, ldx=64, bsx=4096, ldy=64, bsy=4096,
            dtype=BF16):
        return _no_launch(L.dpp_linear_gn(y, part, G, x, w, bias, B, M, K, N, ldx, bsx, ldy, bsy, dtype, None))
    assert lgn(part=None) == NULL
    assert lgn(G=48) == SHAPE                      # N % G
    assert lgn(dtype=F32) == UNSUP
    assert lgn(part=Cp + 16) == ALIAS              # inside the weights
    assert lgn(ldx=60) == SHAPE                    # the GEMM's own checks first

    def pgn(y=A, so=Bp, x=Cp, part=WSP + (1 << 20), nchunk=5, st=Dp, gamma=Ep, beta=Ep + 4096, B=1, H=8, W=4, C=64,
            G=8, P=2, p=0, rows=4, eps=1e-5, silu=0, dtype=BF16):
        return _no_launch(L.dpp_groupnorm_stale_presummed(y, so, x, part, nchunk, st, gamma, beta, B, H, W, C, G, P, p,
                                                          rows, eps, silu, dtype, None))
    assert pgn(part=None) == NULL
    assert pgn(nchunk=0) == SHAPE
    assert pgn(part=Bp) == ALIAS                   # partials == stats_out
    assert pgn(part=A + 64) == ALIAS               # partials inside y
    assert pgn(C=60) == SHAPE                      # GroupNorm's own checks first
    assert pgn(st=None) == NULL
