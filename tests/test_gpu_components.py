"""GPU parity of the asynchronous component chain (AsyncDiff abstract): K
full-image components (GroupNorm -> conv -> self-attention, one patch), run
through the library's kernels in the order ComponentChain issues them.

Checks per step and component:
* data flow, bit-exact: every component's output equals a separate call of
  the same component on the buffer it should have read (this step's output
  of the component before it during the warm-up, the previous step's after);
* every stage against the single-operation oracle fed the device's own
  stored input of that stage (the component's source tensor, the stored
  GroupNorm output, the stored conv output), at the single-operation bar, in
  bf16 and fp32 alike: GroupNorm, conv and self-attention of all K
  components at every step;
* fp32 only: every stage against the oracle's own chain as well (the two
  sides store nothing rounded, so the chains agree to the fp32 bar; in bf16
  they round stored tensors independently and a one-ulp flip of an input
  element moves the attention with Q = K = V by up to 12% of its output RMS,
  so the chain-against-chain comparison is not a bf16 bar).
Each test prints the case it runs before touching the GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import Config, component_chain_inputs, values
from tests._helpers import parity, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import displaced_patch_parallelism_net_amd as dpp  # fails loudly without libdpp.so
    return dpp


def say(*a):
    print("[case]", *a, flush=True)


CHAINS = [
    # (config, components, steps, warm-up steps)
    (Config("chain_tiny_f32", B=1, H=12, W=10, C=64, P=1, G=32, heads=1, D=64, dtype="f32"), 3, 4, 1),
    (Config("chain_32px", B=1, H=32, W=32, C=640, P=1), 2, 3, 1),
    (Config("chain_pair_24px", B=2, H=24, W=20, C=640, P=1), 3, 4, 2),
]


@pytest.mark.parametrize("cfg,K,T,warmup", CHAINS, ids=[c[0].name for c in CHAINS])
def test_component_chain_parity(cfg, K, T, warmup):
    from displaced_patch_parallelism_net_amd.step import ComponentChain
    inp = component_chain_inputs(cfg, K, T)
    bf = cfg.dtype == "bf16"
    xs_v = [values(cfg, x) for x in inp["xs"]]
    params_v = [{"gamma": p["gamma"], "beta": p["beta"], "conv_w": values(cfg, p["conv_w"]), "conv_b": p["conv_b"]}
                for p in inp["params"]]
    want = oracle.async_component_chain(xs_v, params_v, cfg.G, cfg.heads, cfg.gn_eps, bf16=bf,
                                        warmup=warmup) if not bf else None
    tdt = torch.bfloat16 if bf else torch.float32
    chain = ComponentChain(K, cfg.B, cfg.H, cfg.W, cfg.C, cfg.G, cfg.heads, tdt, eps=cfg.gn_eps, head_dim=cfg.D)
    dev_params = [(torch.from_numpy(p["gamma"]).cuda(), torch.from_numpy(p["beta"]).cuda(),
                   to_dev(p["conv_w"], cfg.dtype), torch.from_numpy(p["conv_b"]).cuda()) for p in inp["params"]]
    ref = ComponentChain(K, cfg.B, cfg.H, cfg.W, cfg.C, cfg.G, cfg.heads, tdt, eps=cfg.gn_eps, head_dim=cfg.D)
    for t in range(T):
        sync = t < warmup
        say("component chain", cfg.name, "step", t, "of", T, "sync" if sync else "async")
        x_t = to_dev(inp["xs"][t], cfg.dtype)
        out = chain.step(x_t, dev_params, synchronous=sync)
        torch.cuda.synchronize()
        assert out.data_ptr() == chain.prev[K - 1].data_ptr()
        # data flow: after the step, chain.prev holds this step's outputs and
        # chain.out still holds the previous step's
        for k in range(K):
            src = x_t if k == 0 else (chain.prev[k - 1] if sync else chain.out[k - 1])
            ref.component(k, src, *dev_params[k])
            torch.cuda.synchronize()
            assert torch.equal(ref.out[k].view(torch.int16 if bf else torch.int32),
                               chain.prev[k].view(torch.int16 if bf else torch.int32)), (t, k)
        for k in range(K):
            tag = f"chain {cfg.name} t{t} k{k}"
            p = inp["params"][k]
            # each stage from the device's stored input of that stage
            src = x_t if k == 0 else (chain.prev[k - 1] if sync else chain.out[k - 1])
            y1_in, y2_in = to_host(src), to_host(chain.y1[k])
            gn_want, _ = oracle.groupnorm_stale(y1_in, None, p["gamma"], p["beta"], cfg.H, cfg.G, 0, cfg.gn_eps)
            parity(to_host(chain.y1[k]), gn_want, cfg.dtype, tag + " GN (device input)")
            conv_want = oracle.conv3x3_halo(y2_in, None, params_v[k]["conv_w"], p["conv_b"], 0)
            parity(to_host(chain.y2[k]), conv_want, cfg.dtype, tag + " conv (device input)")
            tok = to_host(chain.y2[k]).reshape(cfg.B, cfg.N, cfg.C)
            attn_want = oracle.self_attn_displaced(tok, tok, tok, cfg.heads).reshape(cfg.B, cfg.H, cfg.W, cfg.C)
            parity(to_host(chain.prev[k]), attn_want, cfg.dtype, tag + " attention (device input)")
            if not bf:
                w = want[t][k]
                parity(to_host(chain.y1[k]), w["y1_exact"], cfg.dtype, tag + " GN (oracle chain)")
                parity(to_host(chain.y2[k]), w["y2_exact"], cfg.dtype, tag + " conv (oracle chain)")
                parity(to_host(chain.prev[k]), w["o_exact"], cfg.dtype, tag + " attention (oracle chain)")


def test_component_chain_first_step_must_be_synchronous():
    from displaced_patch_parallelism_net_amd.step import ComponentChain
    chain = ComponentChain(2, 1, 4, 4, 64, 8, 1, torch.float32)
    with pytest.raises(ValueError):
        chain.step(torch.zeros(1, 4, 4, 64, device="cuda"), [None, None], synchronous=False)
