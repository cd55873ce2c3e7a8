"""GPU parity of the attention block with its projections (DisplacedBlock):
GroupNorm + SiLU with stale statistics -> conv with stale halos -> q
projection and the fused K/V projection into the patch's private K/V buffer ->
attention over the whole buffer -> out projection, chained exactly as the
benchmark runs it, against oracle.displaced_attention_block on the same
seeded inputs (DistriFusion architecture article: DistriGroupNorm,
DistriConv2dPP, DistriSelfAttentionPP around the whole attention module).
With projection weights N(0,1)/sqrt(C) the scores have a spread of about 2
(not one key per query), so the softmax mixing is exercised.  Every stage is
compared with the oracle's value computed from the previous stage's stored
values; the 1024 px workload in full, the 3840 px workload on full
GroupNorm/conv/projection outputs and 256 sampled attention/out rows per
patch.  Each test prints the case it runs before touching the GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import CONFIGS, layer_inputs, projection_inputs, values
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


def _weights(cfg):
    li, pi = layer_inputs(cfg), projection_inputs(cfg)
    v = lambda a: values(cfg, a).astype(np.float64)  # noqa: E731
    host = {"gamma": li["gamma"], "beta": li["beta"], "conv_w": v(li["conv_w"]), "conv_b": li["conv_b"]}
    for n in "qkvo":
        host[f"w_{n}"], host[f"b_{n}"] = v(pi[f"w_{n}"]), pi[f"b_{n}"]
    dev = {"gamma": torch.from_numpy(li["gamma"]).cuda(), "beta": torch.from_numpy(li["beta"]).cuda(),
           "conv_w": to_dev(li["conv_w"], "bf16"), "conv_b": torch.from_numpy(li["conv_b"]).cuda(),
           "w_q": to_dev(pi["w_q"], "bf16"), "b_q": torch.from_numpy(pi["b_q"]).cuda(),
           "w_kv": to_dev(np.concatenate([pi["w_k"], pi["w_v"]], axis=0), "bf16"),
           "b_kv": torch.from_numpy(np.concatenate([pi["b_k"], pi["b_v"]])).cuda(),
           "w_o": to_dev(pi["w_o"], "bf16"), "b_o": torch.from_numpy(pi["b_o"]).cuda()}
    return li, host, dev


def _block_case(cfg, patches, n_sample=None):
    from displaced_patch_parallelism_net_amd.step import DisplacedBlock
    li, h, d = _weights(cfg)
    xs_v, xf_v = values(cfg, li["x_stale"]), values(cfg, li["x_fresh"])
    say("attention block sync step", cfg.name)
    state = oracle.previous_block_state(xs_v, h["gamma"], h["beta"], h["conv_w"], h["conv_b"], h["w_k"], h["b_k"],
                                        h["w_v"], h["b_v"], cfg.P, cfg.G, cfg.gn_eps, bf16=True)
    blk = DisplacedBlock(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, cfg.G, cfg.heads, eps=cfg.gn_eps, head_dim=cfg.D)
    blk.synchronous_step(to_dev(li["x_stale"], "bf16"), d["gamma"], d["beta"], d["conv_w"], d["conv_b"], d["w_kv"],
                         d["b_kv"])
    torch.cuda.synchronize()
    parity(to_host(blk.a1), state["a1_exact"], "bf16", f"block {cfg.name} previous GN+SiLU")
    kv0 = to_host(blk.kv[0])
    parity(kv0[..., :cfg.C], state["k_exact"], "bf16", f"block {cfg.name} previous K")
    parity(kv0[..., cfg.C:], state["v_exact"], "bf16", f"block {cfg.name} previous V")
    # the oracle continues from the device's stored previous-step state
    state = dict(state, a1=to_host(blk.a1), k=kv0[..., :cfg.C], v=kv0[..., cfg.C:])
    xf_d = to_dev(li["x_fresh"], "bf16")
    rng = np.random.default_rng(17)
    for p in patches:
        say("attention block patch step", cfg.name, "patch", p)
        out = blk.patch_step(p, blk.band(xf_d, p), d["gamma"], d["beta"], d["conv_w"], d["conv_b"], d["w_q"],
                             d["b_q"], d["w_kv"], d["b_kv"], d["w_o"], d["b_o"])
        torch.cuda.synchronize()
        rows = None
        if n_sample:
            qi = np.concatenate([[0, cfg.Nq - 1, cfg.W - 1, cfg.Nq // 2], rng.integers(0, cfg.Nq, n_sample - 4)])
            rows = (np.zeros(n_sample, dtype=np.int64), qi)
        want = oracle.displaced_attention_block(xf_v, state, h["gamma"], h["beta"], h["conv_w"], h["conv_b"],
                                                h["w_q"], h["b_q"], h["w_k"], h["b_k"], h["w_v"], h["b_v"], h["w_o"],
                                                h["b_o"], cfg.P, p, cfg.G, cfg.heads, cfg.gn_eps, bf16=True,
                                                attn_rows=rows)
        tag = f"block {cfg.name} p{p}"
        parity(to_host(blk.y1), want["y1_exact"], "bf16", tag + " GN+SiLU")
        parity(to_host(blk.y2), want["y2_exact"], "bf16", tag + " conv")
        parity(to_host(blk.q), want["q_exact"], "bf16", tag + " q")
        t0 = p * cfg.rows * cfg.W
        kvp = to_host(blk.kv[p])
        parity(kvp[:, t0:t0 + cfg.Nq, :cfg.C], want["k_exact"], "bf16", tag + " fresh k in the buffer")
        parity(kvp[:, t0:t0 + cfg.Nq, cfg.C:], want["v_exact"], "bf16", tag + " fresh v in the buffer")
        # the other rows of the private buffer are the previous step's
        keep = np.ones(cfg.N, dtype=bool)
        keep[t0:t0 + cfg.Nq] = False
        np.testing.assert_array_equal(kvp[:, keep, :cfg.C], state["k"][:, keep])
        if rows is None:
            # from the device's stored q and K/V buffer, and along the oracle's own chain
            o_dev = oracle.self_attn_displaced(to_host(blk.q), kvp[..., :cfg.C], kvp[..., cfg.C:], cfg.heads)
            parity(to_host(blk.o), o_dev, "bf16", tag + " attention")
            parity(to_host(out), oracle.linear(to_host(blk.o), h["w_o"], h["b_o"]), "bf16", tag + " out projection")
            parity(to_host(blk.o), want["o_exact"], "bf16", tag + " attention (oracle chain)")
            parity(to_host(out), want["out_exact"], "bf16", tag + " out projection (oracle chain)")
        else:
            # the sampled rows' attention and out projection from the device's
            # stored q and K/V buffer
            q_dev = to_host(blk.q)
            o_rows = oracle.self_attn_displaced(q_dev, kvp[..., :cfg.C], kvp[..., cfg.C:], cfg.heads, rows=rows)
            parity(to_host(blk.o)[rows], o_rows, "bf16", tag + " attention (sampled)")
            out_rows = oracle.linear(to_host(blk.o)[rows], h["w_o"], h["b_o"])
            parity(to_host(out)[rows], out_rows, "bf16", tag + " out projection (sampled)")
            parity(to_host(blk.o)[rows], want["o_rows_exact"], "bf16", tag + " attention (sampled, oracle chain)")


def test_attention_block_parity_1024():
    _block_case(CONFIGS["sdxl_1024"], (0, 3))


def test_attention_block_parity_cfg_pair():
    _block_case(CONFIGS["cfg_pair_1024"], (2,))


def test_attention_block_parity_3840_sampled():
    cfg = CONFIGS["sdxl_3840"]
    _block_case(cfg, (0, cfg.P - 1), n_sample=256)
