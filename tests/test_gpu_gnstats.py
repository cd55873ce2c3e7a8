"""GPU parity of the producer-side GroupNorm statistics (DistriGroupNorm,
DistriFusion architecture article, normalisation section): the conv and the
projection GEMM write the per-group partial sums of their stored output, and
dpp_groupnorm_stale_presummed normalises with them, reading its input once.

* the producers' outputs are bit-identical to the plain calls;
* the chunk partials add up to the oracle's raw group sums of the stored
  output (oracle.patch_sums), and every (chunk, group) a chunk's channels do
  not touch is exactly zero;
* the presummed GroupNorm (with and without SiLU) meets the bar against the
  oracle's GroupNorm with stale statistics of the stored producer output, and
  writes the fresh sums to its stats slot;
* guard bands around every output stay intact.
Each test prints the case it runs before touching the GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import Config, f32_to_bf16_bits, layer_inputs, rows_of, values
from tests._helpers import bits, check_guards, guarded_empty, parity, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import displaced_patch_parallelism_net_amd as dpp  # fails loudly without libdpp.so
    return dpp


def say(*a):
    print("[case]", *a, flush=True)


def _check_partials(part, y_vals, G, chunk_groups, what):
    """part [B,nchunk,G,2] against the raw group sums of y_vals [B,rows,W,C];
    chunk_groups[c] = the set of groups chunk c may touch (others must be 0)."""
    got = part.astype(np.float64).sum(axis=1)
    want = oracle.patch_sums(y_vals, G)
    n = y_vals.shape[1] * y_vals.shape[2] * y_vals.shape[3] // G
    e1 = np.abs(got[..., 0] - want[..., 0]).max()
    e2 = (np.abs(got[..., 1] - want[..., 1]) / np.maximum(np.abs(want[..., 1]), 1e-30)).max()
    print(f"{what}: sum err {e1:.3e} (n {n}), sumsq rel err {e2:.3e}", flush=True)
    assert e1 <= 1e-5 * n and e2 <= 1e-5
    for c, groups in enumerate(chunk_groups):
        others = np.setdiff1d(np.arange(G), np.asarray(sorted(groups), dtype=np.int64))
        assert np.all(part[:, c, others] == 0.0), f"{what}: chunk {c} wrote groups it does not touch"


def _conv_pixel_tiles(rows, W):
    """Pixel tiles of the conv: four patch rows x 16 tg columns, tg (1..5) the
    width that wastes the fewest columns, ties to the wider tile; or six rows
    x 48 columns where those cover the band exactly."""
    tg = min(range(1, 6), key=lambda t: (-(-W // (16 * t)) * 16 * t - W, -t))
    four = -(-rows // 4) * -(-W // (16 * tg))
    six = rows // 6 * (W // 48) if rows % 6 == 0 and W % 48 == 0 else None
    return four, six


def _conv_chunk_groups(nchunk, rows, W, Cout, G):
    """Conv chunks are (channel tile) * pixel tiles + pixel tile, with
    64-channel tiles and one of the two pixel tilings: the one whose chunk
    count the call reports."""
    ctiles = -(-Cout // 64)
    assert nchunk in [ctiles * t for t in _conv_pixel_tiles(rows, W) if t], f"no tiling gives {nchunk} chunks"
    ptiles = nchunk // ctiles
    cg = Cout // G
    out = []
    for c in range(nchunk):
        ct = c // ptiles
        lo, hi = ct * 64, min(Cout, ct * 64 + 64)
        out.append(set(range(lo // cg, (hi - 1) // cg + 1)))
    return out


CONV_CASES = [
    # (config, patch, G) -- G sets the channels per group: 20, 10, 6 (groups straddle
    # 4-channel quads and 64-channel tiles), 1 (one group), C (one channel each)
    (Config("gs_1024", B=1, H=64, W=64, C=640, P=4), 1, 32),
    (Config("gs_c320", B=1, H=16, W=48, C=320, P=2, G=32, heads=5, D=64), 1, 32),
    (Config("gs_w37", B=2, H=12, W=37, C=192, P=4, G=8, heads=3, D=64), 2, 32),
    (Config("gs_g1", B=1, H=9, W=20, C=128, P=3, G=1, heads=2, D=64), 0, 1),
    (Config("gs_gc", B=1, H=6, W=19, C=64, P=2, G=64, heads=1, D=64), 1, 64),
    (Config("gs_r6", B=1, H=24, W=240, C=128, P=2, G=16, heads=2, D=64), 1, 16),   # six-row tiles
]


@pytest.mark.parametrize("cfg,p,G", CONV_CASES, ids=[c[0].name for c in CONV_CASES])
def test_conv_gn_partials(cfg, p, G):
    import displaced_patch_parallelism_net_amd as dpp
    say("conv gn partials", cfg.name, "patch", p, "G", G)
    inp = layer_inputs(cfg)
    r0 = cfg.row0(p)
    x_np = rows_of(inp["x_fresh"], r0, cfg.rows)
    x, st, w = to_dev(x_np, "bf16"), to_dev(inp["x_stale"], "bf16"), to_dev(inp["conv_w"], "bf16")
    b = torch.from_numpy(inp["conv_b"]).cuda()
    nchunk = dpp.dpp_conv3x3_halo_gn_chunks(cfg.rows, cfg.W, cfg.C)
    ybase, y = guarded_empty((cfg.B, cfg.rows, cfg.W, cfg.C), torch.bfloat16)
    pbase, part = guarded_empty((cfg.B, nchunk, G, 2), torch.float32)
    part.fill_(-3.0)
    y_ref = torch.empty(cfg.B, cfg.rows, cfg.W, cfg.C, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_conv3x3_halo_gn(y, part, x, st, w, b, cfg.H, r0)
    dpp.dpp_conv3x3_halo(y_ref, x, st, w, b, cfg.H, r0)
    torch.cuda.synchronize()
    check_guards(ybase, f"conv gn {cfg.name} y")
    check_guards(pbase, f"conv gn {cfg.name} partials")
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    _check_partials(part.cpu().numpy(), to_host(y), G, _conv_chunk_groups(nchunk, cfg.rows, cfg.W, cfg.C, G),
                    f"conv gn {cfg.name}")


LIN_CASES = [(2, 300, 640, 640, 32), (1, 7200, 640, 640, 32), (1, 1024, 320, 320, 32), (1, 333, 128, 1280, 32),
             (1, 50, 64, 96, 12)]


@pytest.mark.parametrize("B,M,K,N,G", LIN_CASES)
def test_linear_gn_partials(B, M, K, N, G):
    import displaced_patch_parallelism_net_amd as dpp
    say("linear gn partials", B, M, K, N, G)
    rng = np.random.default_rng(41)
    x = f32_to_bf16_bits(rng.standard_normal((B, M, K)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    bias = (0.02 * rng.standard_normal(N)).astype(np.float32)
    xd, wd, bd = to_dev(x, "bf16"), to_dev(w, "bf16"), torch.from_numpy(bias).cuda()
    nchunk = dpp.dpp_linear_gn_chunks(B, M, N)
    ybase, y = guarded_empty((B, M, N), torch.bfloat16)
    pbase, part = guarded_empty((B, nchunk, G, 2), torch.float32)
    part.fill_(-3.0)
    y_ref = torch.empty(B, M, N, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_linear_gn(y, part, xd, wd, bd)
    dpp.dpp_linear(y_ref, xd, wd, bd)
    torch.cuda.synchronize()
    check_guards(ybase, "linear gn y")
    check_guards(pbase, "linear gn partials")
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    # chunks are (channel tile) * token tiles + token tile; the token tile is
    # 160 tokens, or 80 when the 160-token grid has at most 128 tiles, and
    # the channel tile 128 or 256 wide (the call's choice): check the sums,
    # and that no chunk writes a group outside either width's reach
    bm = 80 if -(-M // 160) * B * -(-N // 128) <= 128 else 160
    ptiles = -(-M // bm)
    ctiles = nchunk // ptiles
    assert ctiles * ptiles == nchunk
    bn = 128 if -(-N // 128) == ctiles else 256
    cg = N // G
    groups = []
    for c in range(nchunk):
        ct = c // ptiles
        lo, hi = ct * bn, min(N, ct * bn + bn)
        groups.append(set(range(lo // cg, (hi - 1) // cg + 1)))
    _check_partials(part.cpu().numpy(), to_host(y).reshape(B, M, 1, N), G, groups, f"linear gn {B}x{M}x{K}x{N}")


PRESUMMED = [
    (Config("ps_1024", B=1, H=64, W=64, C=640, P=4), 2, False),
    (Config("ps_1024_silu", B=1, H=64, W=64, C=640, P=4), 3, True),
    (Config("ps_pair", B=2, H=32, W=40, C=320, P=4, G=32, heads=5, D=64), 0, False),
    (Config("ps_rag", B=2, H=9, W=37, C=192, P=3, G=12, heads=3, D=64), 1, True),
]


@pytest.mark.parametrize("cfg,p,silu", PRESUMMED, ids=[c[0].name for c in PRESUMMED])
def test_groupnorm_presummed_after_conv(cfg, p, silu):
    """conv (with partials) -> presummed GroupNorm of the conv output, against
    the oracle's GroupNorm of the stored conv output with the stale sums of
    the stale image; stats_out slot p holds the conv output's fresh sums."""
    import displaced_patch_parallelism_net_amd as dpp
    say("presummed gn after conv", cfg.name, "patch", p, "silu" if silu else "")
    inp = layer_inputs(cfg)
    r0 = cfg.row0(p)
    x_np = rows_of(inp["x_fresh"], r0, cfg.rows)
    x, st, w = to_dev(x_np, "bf16"), to_dev(inp["x_stale"], "bf16"), to_dev(inp["conv_w"], "bf16")
    b = torch.from_numpy(inp["conv_b"]).cuda()
    nchunk = dpp.dpp_conv3x3_halo_gn_chunks(cfg.rows, cfg.W, cfg.C)
    part = torch.empty(cfg.B, nchunk, cfg.G, 2, device="cuda")
    h = torch.empty(cfg.B, cfg.rows, cfg.W, cfg.C, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_conv3x3_halo_gn(h, part, x, st, w, b, cfg.H, r0)
    # stale sums: raw sums of the other patches of the stale image (seeded)
    xs = values(cfg, inp["x_stale"]).astype(np.float64)
    stale = np.stack([oracle.patch_sums(xs[:, cfg.row0(q):cfg.row0(q) + cfg.rows], cfg.G) for q in range(cfg.P)],
                     axis=1).astype(np.float32)
    gamma, beta = torch.from_numpy(inp["gamma"]).cuda(), torch.from_numpy(inp["beta"]).cuda()
    ybase, y = guarded_empty((cfg.B, cfg.rows, cfg.W, cfg.C), torch.bfloat16)
    sbase, so = guarded_empty((cfg.B, cfg.P, cfg.G, 2), torch.float32)
    so.fill_(7.0)
    dpp.dpp_groupnorm_stale_presummed(y, so, h, part, torch.from_numpy(stale).cuda(), gamma, beta, cfg.H, cfg.G,
                                      cfg.P, p, cfg.gn_eps, silu=silu)
    torch.cuda.synchronize()
    check_guards(ybase, f"presummed gn {cfg.name} y")
    check_guards(sbase, f"presummed gn {cfg.name} stats_out")
    hv = to_host(h)
    fn = oracle.groupnorm_silu_stale if silu else oracle.groupnorm_stale
    want_y, want_s = fn(hv, stale, inp["gamma"], inp["beta"], cfg.H, cfg.G, p, cfg.gn_eps)
    parity(to_host(y), want_y, "bf16", f"presummed gn {cfg.name} p{p}")
    so_h = so.cpu().numpy()
    n = cfg.rows * cfg.W * cfg.C // cfg.G
    e1 = np.abs(so_h[:, p, :, 0] - want_s[..., 0]).max()
    e2 = (np.abs(so_h[:, p, :, 1] - want_s[..., 1]) / np.abs(want_s[..., 1])).max()
    print(f"presummed gn {cfg.name} stats: sum err {e1:.3e} (n {n}), sumsq rel err {e2:.3e}", flush=True)
    assert e1 <= 1e-5 * n and e2 <= 1e-5
    assert np.all(np.delete(so_h, p, axis=1) == 7.0), "stats_out slots of other patches were written"
    # the stats-only form writes the same sums
    so2 = torch.full((cfg.B, cfg.P, cfg.G, 2), 7.0, device="cuda")
    dpp.dpp_groupnorm_stale_presummed(None, so2, h, part, None, None, None, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(so2.cpu().numpy(), so_h)


def test_groupnorm_presummed_after_out_projection():
    """out projection (with partials) -> the next block's presummed GroupNorm +
    SiLU over the projected tokens viewed as the patch [B,rows,W,C]."""
    import displaced_patch_parallelism_net_amd as dpp
    B, H, W, C, G, P, p = 1, 60, 48, 640, 32, 4, 1
    R = H // P
    say("presummed gn after out projection", B, R * W, C)
    rng = np.random.default_rng(43)
    o = f32_to_bf16_bits(rng.standard_normal((B, R * W, C)).astype(np.float32))
    wo = f32_to_bf16_bits((rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32))
    bo = (0.02 * rng.standard_normal(C)).astype(np.float32)
    nchunk = dpp.dpp_linear_gn_chunks(B, R * W, C)
    part = torch.empty(B, nchunk, G, 2, device="cuda")
    out = torch.empty(B, R * W, C, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_linear_gn(out, part, to_dev(o, "bf16"), to_dev(wo, "bf16"), torch.from_numpy(bo).cuda())
    stale = np.zeros((B, P, G, 2), dtype=np.float32)
    stale[..., 1] = R * W * C // G            # other patches: unit variance around zero
    gamma = (1.0 + 0.02 * rng.standard_normal(C)).astype(np.float32)
    beta = (0.02 * rng.standard_normal(C)).astype(np.float32)
    y = torch.empty(B, R, W, C, dtype=torch.bfloat16, device="cuda")
    so = torch.zeros(B, P, G, 2, device="cuda")
    dpp.dpp_groupnorm_stale_presummed(y, so, out.view(B, R, W, C), part, torch.from_numpy(stale).cuda(),
                                      torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda(), H, G, P, p, 1e-5,
                                      silu=True)
    torch.cuda.synchronize()
    want_y, _ = oracle.groupnorm_silu_stale(to_host(out).reshape(B, R, W, C), stale, gamma, beta, H, G, p, 1e-5)
    parity(to_host(y), want_y, "bf16", "presummed gn+silu after out projection")


def test_groupnorm_presummed_matches_plain_groupnorm():
    """On the same x, the presummed call (partials from the conv that wrote
    x) and dpp_groupnorm_stale (its own partial pass) agree to the bar: only
    the chunking of the float32 partial sums differs."""
    import displaced_patch_parallelism_net_amd as dpp
    cfg = Config("ps_eq", B=1, H=240, W=240, C=640, P=8)
    p = 3
    say("presummed vs plain gn", cfg.name, "patch", p)
    inp = layer_inputs(cfg)
    r0 = cfg.row0(p)
    x, st, w = (to_dev(rows_of(inp["x_fresh"], r0, cfg.rows), "bf16"), to_dev(inp["x_stale"], "bf16"),
                to_dev(inp["conv_w"], "bf16"))
    b = torch.from_numpy(inp["conv_b"]).cuda()
    nchunk = dpp.dpp_conv3x3_halo_gn_chunks(cfg.rows, cfg.W, cfg.C)
    assert nchunk == 250  # 5 six-row tiles x 5 48-column tiles x 10 channel tiles
    part = torch.empty(cfg.B, nchunk, cfg.G, 2, device="cuda")
    h = torch.empty(cfg.B, cfg.rows, cfg.W, cfg.C, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_conv3x3_halo_gn(h, part, x, st, w, b, cfg.H, r0)
    stale = torch.zeros(cfg.B, cfg.P, cfg.G, 2, device="cuda")
    stale[..., 1] = float(cfg.rows * cfg.W * cfg.C // cfg.G) * 2.0
    gamma, beta = torch.from_numpy(inp["gamma"]).cuda(), torch.from_numpy(inp["beta"]).cuda()
    y1, y2 = torch.empty_like(h), torch.empty_like(h)
    s1, s2 = torch.zeros_like(stale), torch.zeros_like(stale)
    ws = torch.empty(dpp.dpp_groupnorm_stale_workspace_bytes(cfg.B, cfg.rows, cfg.W, cfg.C, cfg.G), dtype=torch.uint8,
                     device="cuda")
    dpp.dpp_groupnorm_stale_presummed(y1, s1, h, part, stale, gamma, beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps)
    dpp.dpp_groupnorm_stale(y2, s2, h, stale, gamma, beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps, ws)
    torch.cuda.synchronize()
    want, _ = oracle.groupnorm_stale(to_host(h), stale.cpu().numpy(), inp["gamma"], inp["beta"], cfg.H, cfg.G, p,
                                     cfg.gn_eps)
    parity(to_host(y1), want, "bf16", "presummed gn 3840 px")
    parity(to_host(y2), want, "bf16", "plain gn 3840 px")
    np.testing.assert_allclose(s1.cpu().numpy()[:, p], s2.cpu().numpy()[:, p], rtol=2e-5, atol=1e-2)
