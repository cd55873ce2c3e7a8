"""A displaced layer step captured into a HIP graph (step.capture_graph) and
replayed must write exactly what the eager calls write: the same kernels on
the same inputs, bit for bit.  The step is every patch's GroupNorm -> conv ->
splice -> attention of the 1024 px and 3840 px workloads plus the CFG
combine, as the benchmark runs it.  Between replays the test overwrites
every output buffer from the host side (eager fills, synchronised), so a
replay that skipped a kernel or left a node stale would show up; three
replays are checked."""
import numpy as np
import pytest

from dpp_synth import CONFIGS, cfg_inputs, layer_inputs
from tests._helpers import bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import displaced_patch_parallelism_net_amd as dpp  # fails loudly without libdpp.so
    return dpp


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("name", ["sdxl_1024", "sdxl_3840"])
def test_graph_replay_matches_eager_step(gpu, name):
    dpp = gpu
    from displaced_patch_parallelism_net_amd.step import DisplacedLayer, capture_graph
    cfg = CONFIGS[name]
    say("graph replay of the", cfg.name, "step: eager reference")
    li = layer_inputs(cfg)
    n_lat = 2 * cfg.H * 2 * cfg.W * 4
    ci = cfg_inputs(cfg, n=n_lat)
    layer = DisplacedLayer(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, cfg.G, cfg.heads, torch.bfloat16, eps=cfg.gn_eps,
                           head_dim=cfg.D)
    gamma, beta = torch.from_numpy(li["gamma"]).cuda(), torch.from_numpy(li["beta"]).cuda()
    w, b = to_dev(li["conv_w"], "bf16"), torch.from_numpy(li["conv_b"]).cuda()
    layer.synchronous_step(to_dev(li["x_stale"], "bf16"), gamma, beta, w, b)
    xf = to_dev(li["x_fresh"], "bf16")
    xp = [layer.band(xf, p) for p in range(cfg.P)]
    eps_c, eps_u = to_dev(ci["eps_c"], "bf16"), to_dev(ci["eps_u"], "bf16")
    eps = torch.empty_like(eps_c)
    rel = torch.zeros(1, dtype=torch.float32, device="cuda")
    cfg_ws = torch.empty(dpp.dpp_cfg_combine_workspace_bytes(n_lat), dtype=torch.uint8, device="cuda")

    def step():
        for p in range(cfg.P):
            layer.patch_step(p, xp[p], gamma, beta, w, b)
        dpp.dpp_cfg_combine_relmae(eps, rel, eps_c, eps_u, cfg.guidance, cfg_ws)

    step()
    torch.cuda.synchronize()
    # outputs of the step: every patch's spliced rows of its K/V buffer (GN,
    # conv, splice), the fresh statistics, the last patch's attention output
    # and the CFG results
    rows = [(p * layer.R, (p + 1) * layer.R) for p in range(cfg.P)]
    ref = {"kv": [bits(layer.kv[p][:, r0:r1]) for p, (r0, r1) in enumerate(rows)],
           "stats": layer.stats_next.cpu().numpy().copy(), "o": bits(layer.o), "eps": bits(eps),
           "rel": rel.cpu().numpy().copy()}

    say("graph replay of the", cfg.name, "step: capture")
    g = capture_graph(step)
    torch.cuda.synchronize()
    for rep in range(3):
        for p, (r0, r1) in enumerate(rows):
            layer.kv[p][:, r0:r1].fill_(float(rep + 3))
        layer.stats_next.fill_(-1.0)
        layer.o.fill_(float(rep + 5))
        layer.y1.fill_(0.5)
        layer.y2.fill_(0.25)
        eps.fill_(9.0)
        rel.fill_(-2.0)
        torch.cuda.synchronize()
        say("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for p, (r0, r1) in enumerate(rows):
            assert np.array_equal(bits(layer.kv[p][:, r0:r1]), ref["kv"][p]), f"replay {rep}: patch {p} rows"
        assert np.array_equal(layer.stats_next.cpu().numpy(), ref["stats"]), f"replay {rep}: statistics"
        assert np.array_equal(bits(layer.o), ref["o"]), f"replay {rep}: attention output"
        assert np.array_equal(bits(eps), ref["eps"]), f"replay {rep}: CFG output"
        assert np.array_equal(rel.cpu().numpy(), ref["rel"]), f"replay {rep}: rel-MAE"
        print(f"graph replay {rep}: bit-identical to the eager step", flush=True)
    del g
