"""GPU parity of the projections (dpp_linear), the K/V projection written
straight into the private full-image K/V buffer, GroupNorm + SiLU, and the
displaced self-attention with its projections, against the CPU oracle on the
same seeded inputs.  Each test prints the case it runs before touching the
GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import CONFIGS, Config, f32_to_bf16_bits, layer_inputs, projection_inputs, rows_of, tokens, values
from tests._helpers import bits, parity, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import displaced_patch_parallelism_net_amd as dpp  # fails loudly without libdpp.so
    return dpp


def say(*a):
    print("[case]", *a, flush=True)


def _dpp():
    import displaced_patch_parallelism_net_amd as dpp
    return dpp


def _rand(rng, shape, dtype, scale=1.0):
    a = (scale * rng.standard_normal(shape)).astype(np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


# ======================================================================== linear
# (name, B, M, K, N, ld_x, ld_y, bias, dtype): ragged M/N/K tails, strided rows
LINEAR_CASES = [
    ("tokens_1024", 1, 1024, 640, 640, 640, 640, True, "bf16"),
    ("tokens_7200", 1, 7200, 640, 640, 640, 640, True, "bf16"),      # the 3840 px patch, as timed
    ("kv_7200_k1280", 1, 7200, 1280, 1280, 1280, 1280, True, "bf16"),  # K = 1280: the 20-slice unrolled path
    ("k320", 1, 517, 320, 192, 320, 192, True, "bf16"),                # K = 320: the 5-slice unrolled path
    ("kv_1280", 1, 1000, 640, 1280, 640, 1280, True, "bf16"),
    ("kv_7200", 1, 7200, 640, 1280, 640, 1280, True, "bf16"),          # the fused K/V projection, 256-channel tiles
    ("wide_ragged", 2, 3001, 328, 1152, 336, 1160, True, "bf16"),      # 256-channel tiles, half-empty last tile, generic K
    ("ragged_strided", 2, 301, 200, 84, 208, 96, True, "bf16"),
    ("no_bias", 1, 130, 64, 128, 64, 128, False, "bf16"),
    ("minimal", 1, 1, 8, 4, 8, 4, True, "bf16"),                      # smallest bf16 shape: 1 token, K = 8, N = 4
    ("f32", 2, 37, 24, 20, 30, 22, True, "f32"),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=[c[0] for c in LINEAR_CASES])
def test_linear_parity(case):
    name, B, M, K, N, ldx, ldy, use_bias, dtype = case
    dpp = _dpp()
    rng = np.random.default_rng(21)
    say("linear", name, B, M, K, N)
    x = _rand(rng, (B, M, ldx), dtype)
    w = _rand(rng, (N, K), dtype, 1.0 / np.sqrt(K))
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32) if use_bias else None
    # y: a strided view into a larger buffer with a sentinel fill
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ybuf = torch.full((B, M + 3, ldy), 7.0, dtype=dt, device="cuda")
    y = ybuf[:, 1:M + 1, :N]
    xd = to_dev(x, dtype)[:, :, :K]
    dpp.dpp_linear(y, xd, to_dev(w, dtype), None if bias is None else torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    want = oracle.linear(values(dtype, x)[:, :, :K], values(dtype, w), bias)
    parity(to_host(y), want, dtype, f"linear {name}")
    yb = to_host(ybuf)
    assert np.all(yb[:, 0] == 7.0) and np.all(yb[:, M + 1:] == 7.0), "wrote outside the output rows"
    assert np.all(yb[:, 1:M + 1, N:] == 7.0), "wrote outside the output columns"


def test_kv_projection_written_into_kv_buffer():
    # the fresh patch's K and V (one GEMM with the concatenated weights) land in
    # its token rows of the previous step's K/V buffer; every other row keeps
    # its stale bits
    dpp = _dpp()
    cfg = CONFIGS["sdxl_1024"]
    p = 2
    say("kv projection into buffer", cfg.name, "patch", p)
    li, pi = layer_inputs(cfg), projection_inputs(cfg)
    C, t0, M = cfg.C, p * cfg.rows * cfg.W, cfg.Nq
    x = tokens(rows_of(li["x_fresh"], p * cfg.rows, cfg.rows))
    w_kv = np.concatenate([pi["w_k"], pi["w_v"]], axis=0)
    b_kv = np.concatenate([pi["b_k"], pi["b_v"]])
    kv = to_dev(pi["kv_stale"], "bf16")
    before = bits(kv).copy()
    dpp.dpp_linear(kv[:, t0:t0 + M, :], to_dev(x, "bf16"), to_dev(w_kv, "bf16"), torch.from_numpy(b_kv).cuda())
    torch.cuda.synchronize()
    after = bits(kv)
    assert np.array_equal(after[:, :t0], before[:, :t0]) and np.array_equal(after[:, t0 + M:], before[:, t0 + M:])
    want = oracle.linear(values("bf16", x), values("bf16", w_kv), b_kv)
    parity(to_host(kv[:, t0:t0 + M]), want, "bf16", "kv projection rows")


# ======================================================================== GroupNorm + SiLU
GN_SILU_CASES = [(n, None, p) for n, p in [("tiny_f32", 1), ("sdxl_1024", 2), ("cfg_pair_1024", 0)]] + [
    ("ragged_bf16", Config("gsr", B=2, H=9, W=7, C=96, P=3, G=12, heads=1, D=96), 1),
]


@pytest.mark.parametrize("name,cfg,p", GN_SILU_CASES, ids=[c[0] for c in GN_SILU_CASES])
def test_groupnorm_silu_parity(name, cfg, p):
    dpp = _dpp()
    cfg = cfg or CONFIGS[name]
    say("groupnorm+silu", name, "patch", p)
    inp = layer_inputs(cfg)
    r0 = p * cfg.rows
    xs = values(cfg, inp["x_stale"])
    stale = np.stack([oracle.patch_sums(xs[:, q * cfg.rows:(q + 1) * cfg.rows], cfg.G) for q in range(cfg.P)], axis=1)
    xp = rows_of(inp["x_fresh"], r0, cfg.rows)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    x_d = to_dev(xp, cfg.dtype)
    st_d = torch.from_numpy(stale.astype(np.float32)).cuda()
    g_d, b_d = torch.from_numpy(inp["gamma"]).cuda(), torch.from_numpy(inp["beta"]).cuda()
    ws = torch.empty(dpp.dpp_groupnorm_stale_workspace_bytes(cfg.B, cfg.rows, cfg.W, cfg.C, cfg.G), dtype=torch.uint8,
                     device="cuda")
    y, y0 = torch.empty_like(x_d), torch.empty_like(x_d)
    so, so0 = (torch.zeros(cfg.B, cfg.P, cfg.G, 2, device="cuda") for _ in range(2))
    dpp.dpp_groupnorm_silu_stale(y, so, x_d, st_d, g_d, b_d, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps, ws)
    dpp.dpp_groupnorm_stale(y0, so0, x_d, st_d, g_d, b_d, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps, ws)
    torch.cuda.synchronize()
    want, fresh = oracle.groupnorm_silu_stale(values(cfg, xp), stale.astype(np.float32).astype(np.float64),
                                              inp["gamma"], inp["beta"], cfg.H, cfg.G, p, cfg.gn_eps)
    parity(to_host(y), want, cfg.dtype, f"gn+silu {name}")
    # same statistics as the plain call, bit for bit
    assert np.array_equal(bits(so), bits(so0))


# ======================================================================== projected attention
@pytest.mark.parametrize("name,p", [("sdxl_1024", 1), ("cfg_pair_1024", 3)])
def test_projected_attention_parity(name, p):
    # q = x Wq^T + bq; fresh k, v projected straight into the patch's rows of
    # the previous step's K/V buffer; attention over the buffer; out = o Wo^T + bo
    dpp = _dpp()
    cfg = CONFIGS[name]
    say("projected attention", name, "patch", p)
    li, pi = layer_inputs(cfg), projection_inputs(cfg)
    B, C, heads, M, t0 = cfg.B, cfg.C, cfg.heads, cfg.Nq, p * cfg.rows * cfg.W
    x = tokens(rows_of(li["x_fresh"], p * cfg.rows, cfg.rows))
    w = {n: to_dev(pi[f"w_{n}"], "bf16") for n in "qkvo"}
    b = {n: torch.from_numpy(pi[f"b_{n}"]).cuda() for n in "qkvo"}
    w_kv = to_dev(np.concatenate([pi["w_k"], pi["w_v"]], axis=0), "bf16")
    b_kv = torch.from_numpy(np.concatenate([pi["b_k"], pi["b_v"]])).cuda()
    xd = to_dev(x, "bf16")
    kv = to_dev(pi["kv_stale"], "bf16")
    q = torch.empty(B, M, C, dtype=torch.bfloat16, device="cuda")
    o, out = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(dpp.dpp_self_attn_workspace_bytes(B, M, cfg.N, heads, 64, 0), 1), dtype=torch.uint8,
                     device="cuda")
    dpp.dpp_linear(q, xd, w["q"], b["q"])
    dpp.dpp_linear(kv[:, t0:t0 + M, :], xd, w_kv, b_kv)
    dpp.dpp_self_attn_displaced(o, q, kv[:, :, :C], kv[:, :, C:], heads, 64, 0.0, ws)
    dpp.dpp_linear(out, o, w["o"], b["o"])
    torch.cuda.synchronize()
    kvs = values("bf16", pi["kv_stale"])
    ref = oracle.projected_attention(values("bf16", x), kvs[..., :C], kvs[..., C:], t0,
                                     *(values("bf16", pi[f"w_{n}"]) if i % 2 == 0 else pi[f"b_{n}"]
                                       for n in "qkvo" for i in range(2)), heads, bf16=True)
    parity(to_host(q), ref["q_exact"], "bf16", "q projection")
    parity(to_host(kv[:, t0:t0 + M, :C]), ref["k_exact"], "bf16", "fresh k in buffer")
    parity(to_host(kv[:, t0:t0 + M, C:]), ref["v_exact"], "bf16", "fresh v in buffer")
    parity(to_host(o), ref["o_exact"], "bf16", "attention over projected buffer")
    parity(to_host(out), ref["out_exact"], "bf16", "out projection")
