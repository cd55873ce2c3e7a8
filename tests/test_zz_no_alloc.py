"""GPU test of the allocation-free GroupNorm entry point
(dpp_groupnorm_stale_noalloc): its output and fresh sums equal those of
dpp_groupnorm_stale with a caller workspace, bit for bit, and meet the oracle
bar, on calls in a row whose second input is smaller than the first (the
static scratch keeps the previous call's contents), in bf16 and fp32, and in
the stats-only mode of the synchronous step.  Each case prints what it runs
before touching the GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import Config, layer_inputs, rows_of, values
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


def _stale(cfg, xs):
    return np.stack([oracle.patch_sums(xs[:, cfg.row0(q):cfg.row0(q) + cfg.rows], cfg.G) for q in range(cfg.P)],
                    axis=1).astype(np.float32)


def _one(cfg, p, stats_only=False):
    import displaced_patch_parallelism_net_amd as dpp
    say("groupnorm noalloc", cfg.name, "patch", p, "stats only" if stats_only else "")
    inp = layer_inputs(cfg)
    stale = torch.from_numpy(_stale(cfg, values(cfg, inp["x_stale"]).astype(np.float64))).cuda()
    gamma, beta = torch.from_numpy(inp["gamma"]).cuda(), torch.from_numpy(inp["beta"]).cuda()
    x_np = rows_of(inp["x_fresh"], cfg.row0(p), cfg.rows)
    x = to_dev(x_np, cfg.dtype)
    dt = x.dtype
    ws = torch.empty(dpp.dpp_groupnorm_stale_workspace_bytes(cfg.B, cfg.rows, cfg.W, cfg.C, cfg.G), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() <= dpp._lib.GN_NOALLOC_MAX_BYTES
    y_ref = None if stats_only else torch.empty_like(x)
    s_ref = torch.full((cfg.B, cfg.P, cfg.G, 2), 7.0, device="cuda")
    dpp.dpp_groupnorm_stale(y_ref, s_ref, x, None if stats_only else stale, None if stats_only else gamma,
                            None if stats_only else beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps, ws)
    ybase, y = (None, None) if stats_only else guarded_empty(tuple(x.shape), dt)
    sbase, s = guarded_empty((cfg.B, cfg.P, cfg.G, 2), torch.float32)
    s.fill_(7.0)
    dpp.dpp_groupnorm_stale_noalloc(y, s, x, None if stats_only else stale, None if stats_only else gamma,
                                    None if stats_only else beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps)
    torch.cuda.synchronize()
    check_guards(sbase, f"noalloc {cfg.name} stats_out")
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref.cpu().numpy())
    if stats_only:
        return
    check_guards(ybase, f"noalloc {cfg.name} y")
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    want, _ = oracle.groupnorm_stale(values(cfg, x_np), _stale(cfg, values(cfg, inp["x_stale"]).astype(np.float64)),
                                     inp["gamma"], inp["beta"], cfg.H, cfg.G, p, cfg.gn_eps)
    parity(to_host(y), want, cfg.dtype, f"noalloc gn {cfg.name} p{p}")


def test_groupnorm_noalloc_matches_workspace_entry_on_consecutive_calls():
    big = Config("noalloc_1024", B=2, H=64, W=64, C=640, P=4)        # 256 partial chunks over the batch
    small = Config("noalloc_small", B=1, H=9, W=7, C=96, P=3, G=12, heads=1, D=96)
    tiny_f32 = Config("noalloc_f32", B=2, H=10, W=3, C=12, P=5, G=3, heads=1, D=12, dtype="f32")
    _one(big, 1)
    _one(small, 2)          # smaller input: the scratch still holds the first call's sums
    _one(tiny_f32, 4)
    _one(big, 3, stats_only=True)
    _one(small, 0)
