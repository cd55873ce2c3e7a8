"""GPU pins of the output rounding: every bf16 store rounds to nearest, ties
to even.

Each case is built so that the float32 result before the final store is
exact and known in closed form, and lands on a bf16 tie (exactly half an ulp
between two bf16 values) or a near tie (a few float32 ulps either side of
one).  The stored bits must then equal the round-to-nearest-even bf16 value
of that exact result (oracle.bf16_round, itself pinned to torch's bf16
conversion on the CPU).  Truncation fails the near ties above a tie,
round-half-up fails the ties whose lower neighbour is even, and
round-half-away fails the same ties on the negative side; each test checks
that its data holds every kind.

* conv: one unit weight per output channel (centre tap, input channel =
  output channel), so y = x + bias; unsplit and with the input-channel
  split (float32 partials summed with the bias by the reduction kernel);
* projection: one-hot weight rows, y[m, n] = x[m, perm(n)] + bias[n];
* GroupNorm: balanced +-1 inputs with eps = 0, so the group mean is exactly
  0, the rstd exactly 1, and y = +-gamma_c + beta_c;
* attention: Q = 0 over 2^k keys, so every weight is exactly 1 and o is the
  exact mean of V, unsplit and with the key-range split and merge;
* CFG combine: u + w (c - u) with c - u = +-1 bf16 ulp and w = 0.5, 1.5,
  7.5 and 0.5 +- 2^-10.
Each test prints the case it runs before touching the GPU."""
import numpy as np
import pytest

import oracle
from dpp_synth import bf16_bits_to_f32, f32_to_bf16_bits
from tests._helpers import bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HALF_ULP = 2.0 ** -8   # half a bf16 ulp on [1, 2)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import displaced_patch_parallelism_net_amd as dpp  # fails loudly without libdpp.so
    return dpp


def say(*a):
    print("[case]", *a, flush=True)


def rne_bits(exact) -> np.ndarray:
    """bf16 bits of the round-to-nearest-even value of an exact result."""
    r = oracle.bf16_round(np.asarray(exact, dtype=np.float64))
    return f32_to_bf16_bits(r.astype(np.float32))


def grid_values(rng, shape, sign=None):
    """bf16-exact values +-(1 + j 2^-7), j in [2, 96]: every result below
    (offsets of at most 3/2 ulp) stays inside the binade [1, 2)."""
    j = rng.integers(2, 97, size=shape)
    s = rng.choice([-1.0, 1.0], size=shape) if sign is None else sign
    return s * (1.0 + j * 2.0 ** -7)


# offsets in half ulps of [1, 2): ties, near ties, exact values, quarters
OFFSETS = np.array([1.0, -1.0, 3.0, -3.0, 1.0 + 2.0 ** -12, 1.0 - 2.0 ** -12, -1.0 + 2.0 ** -12,
                    -1.0 - 2.0 ** -12, 0.0, 2.0, 0.5, 1.5, -0.5, -2.0]) * HALF_ULP


def coverage(exact):
    """Counts of the rounding situations in a set of exact results on [1, 2):
    ties rounded up / down in magnitude by RNE, near ties above / below."""
    a = np.abs(np.asarray(exact, dtype=np.float64))
    frac = (a - 1.0) / 2.0 ** -7          # position in ulps
    low = np.floor(frac)
    r = frac - low
    tie = r == 0.5
    tie_up = tie & (low % 2 == 1)         # RNE moves to the even upper neighbour
    tie_down = tie & (low % 2 == 0)
    near_above = (r > 0.5) & (r < 0.5 + 2.0 ** -5)
    near_below = (r < 0.5) & (r > 0.5 - 2.0 ** -5)
    return {"tie_up": int(tie_up.sum()), "tie_down": int(tie_down.sum()),
            "near_above": int(near_above.sum()), "near_below": int(near_below.sum())}


def check(got_bits, exact, what, need_near=True):
    cov = coverage(exact)
    want = rne_bits(exact)
    ndiff = int(np.count_nonzero(got_bits != want))
    print(f"{what}: {exact.size} elements, {cov}, {ndiff} differ from RNE", flush=True)
    assert cov["tie_up"] > 0 and cov["tie_down"] > 0, cov
    if need_near:
        assert cov["near_above"] > 0 and cov["near_below"] > 0, cov
    assert ndiff == 0, f"{what}: {ndiff} stores differ from round-to-nearest-even"


# ======================================================================== conv
@pytest.mark.parametrize("B,H,W,C,row0,rows,split", [
    (1, 6, 40, 64, 2, 2, False),         # patch with both halo rows, one workgroup
    (2, 5, 37, 128, 0, 5, False),        # whole image, ragged width
    (1, 64, 64, 640, 16, 16, True),      # the 1024 px band: input channels split 5 ways
    (1, 18, 240, 128, 6, 6, False),      # six-row x 48-column tiles (the kernel of the 240-wide bands)
])
def test_conv_unit_weight_rounds_to_nearest_even(B, H, W, C, row0, rows, split):
    import displaced_patch_parallelism_net_amd as dpp
    rng = np.random.default_rng(31)
    say("rounding conv", B, H, W, C, row0, rows, "split" if split else "unsplit")
    x = grid_values(rng, (B, rows, W, C))
    stale = rng.standard_normal((B, H, W, C))             # finite; multiplied by zero weights only
    wt = np.zeros((C, 3, 3, C))
    wt[np.arange(C), 1, 1, np.arange(C)] = 1.0
    bias = OFFSETS[np.arange(C) % len(OFFSETS)]
    xb = f32_to_bf16_bits(x.astype(np.float32))
    y = torch.empty(B, rows, W, C, dtype=torch.bfloat16, device="cuda")
    ws = None
    if split:
        wsb = dpp.dpp_conv3x3_halo_workspace_bytes(B, rows, W, C, C)
        assert wsb > 0, "this band is expected to split"
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    whole = row0 == 0 and rows == H
    dpp.dpp_conv3x3_halo(y, to_dev(xb, "bf16"),
                         None if whole else to_dev(f32_to_bf16_bits(stale.astype(np.float32)), "bf16"),
                         to_dev(f32_to_bf16_bits(wt.astype(np.float32)), "bf16"),
                         torch.from_numpy(bias.astype(np.float32)).cuda(), H, row0, workspace=ws)
    torch.cuda.synchronize()
    exact = bf16_bits_to_f32(xb).astype(np.float64) + bias
    check(bits(y), exact, "conv unit weight " + ("split" if split else "unsplit"))


# ======================================================================== projection
@pytest.mark.parametrize("B,M,K,N", [(1, 300, 640, 640), (2, 50, 320, 1280), (1, 33, 72, 64)])
def test_linear_one_hot_rounds_to_nearest_even(B, M, K, N):
    import displaced_patch_parallelism_net_amd as dpp
    rng = np.random.default_rng(32)
    say("rounding linear", B, M, K, N)
    x = grid_values(rng, (B, M, K))
    perm = rng.integers(0, K, size=N)
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    bias = OFFSETS[rng.integers(0, len(OFFSETS), size=N)]
    xb = f32_to_bf16_bits(x.astype(np.float32))
    y = torch.empty(B, M, N, dtype=torch.bfloat16, device="cuda")
    dpp.dpp_linear(y, to_dev(xb, "bf16"), to_dev(f32_to_bf16_bits(w.astype(np.float32)), "bf16"),
                   torch.from_numpy(bias.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    exact = bf16_bits_to_f32(xb).astype(np.float64)[:, :, perm] + bias
    check(bits(y), exact, f"linear one-hot {B}x{M}x{K}x{N}")


# ======================================================================== GroupNorm
def test_groupnorm_exact_statistics_round_to_nearest_even():
    import displaced_patch_parallelism_net_amd as dpp
    B, H, W, C, G, P, p = 2, 8, 10, 640, 32, 4, 1
    R = H // P
    cg = C // G
    rng = np.random.default_rng(33)
    say("rounding groupnorm", B, H, W, C, G, P, p)
    # +-1 alternating over the pixels: every group of the patch sums to 0
    # exactly and its squares to the pixel count; the other patches' stale
    # sums say the same, so with eps = 0 the mean is 0 and the rstd 1.
    sign = np.where((np.arange(R * W) % 2) == 0, 1.0, -1.0).reshape(1, R, W, 1)
    x = np.broadcast_to(sign, (B, R, W, C)).copy()
    stale = np.zeros((B, P, G, 2), dtype=np.float32)
    stale[..., 1] = R * W * cg
    gamma = grid_values(rng, (C,), sign=np.ones(C)) + OFFSETS[rng.integers(0, len(OFFSETS), size=C)]
    beta = np.zeros(C)
    xb = f32_to_bf16_bits(x.astype(np.float32))
    y = torch.empty(B, R, W, C, dtype=torch.bfloat16, device="cuda")
    so = torch.full((B, P, G, 2), 7.0, device="cuda")
    ws = torch.empty(dpp.dpp_groupnorm_stale_workspace_bytes(B, R, W, C, G), dtype=torch.uint8, device="cuda")
    dpp.dpp_groupnorm_stale(y, so, to_dev(xb, "bf16"), torch.from_numpy(stale).cuda(),
                            torch.from_numpy(gamma.astype(np.float32)).cuda(),
                            torch.from_numpy(beta.astype(np.float32)).cuda(), H, G, P, p, 0.0, ws)
    torch.cuda.synchronize()
    exact = x * gamma + beta
    check(bits(y), exact, "groupnorm exact statistics")
    got_s = so.cpu().numpy()[:, p]
    np.testing.assert_array_equal(got_s[..., 0], 0.0)
    np.testing.assert_array_equal(got_s[..., 1], float(R * W * cg))


# ======================================================================== attention
@pytest.mark.parametrize("nkv,heads,use_ws", [(2, 2, False), (64, 1, False), (4096, 2, False), (4096, 2, True),
                                             (8192, 1, True)])
def test_attention_zero_query_mean_rounds_to_nearest_even(nkv, heads, use_ws):
    import displaced_patch_parallelism_net_amd as dpp
    B, nq = 1, 100
    hd = heads * 64
    rng = np.random.default_rng(34)
    say("rounding attention", nkv, "keys", heads, "heads", "split" if use_ws else "unsplit")
    # per channel: values base or base + 1 ulp (sign per channel), with h of
    # the nkv keys high; the mean is base + h/nkv ulp, exactly, and lands on
    # a tie (h = nkv/2), a near tie (nkv/2 +- 1) or a quarter
    base = grid_values(rng, (hd,))
    sgn = np.sign(base)
    kinds = np.array([0.5, 0.5, 0.25, 0.75, 0.0, 1.0])
    frac = kinds[np.arange(hd) % len(kinds)]
    h = np.round(frac * nkv).astype(np.int64)
    if nkv >= 64:
        near = np.arange(hd) % 7
        h = np.where(near == 1, nkv // 2 + 1, np.where(near == 2, nkv // 2 - 1, h))
    v = np.empty((B, nkv, hd))
    for c in range(hd):
        hi = np.zeros(nkv, dtype=bool)
        hi[rng.permutation(nkv)[:h[c]]] = True
        v[0, :, c] = base[c] + sgn[c] * hi * 2.0 ** -7
    k = rng.standard_normal((B, nkv, hd))
    vb = f32_to_bf16_bits(v.astype(np.float32))
    kb = f32_to_bf16_bits(k.astype(np.float32))
    q = torch.zeros(B, nq, hd, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(B, nq, hd, dtype=torch.bfloat16, device="cuda")
    ws = None
    if use_ws:
        wsb = dpp.dpp_self_attn_workspace_bytes(B, nq, nkv, heads, 64, 0)
        assert wsb > 0, "this shape is expected to split the key range"
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    dpp.dpp_self_attn_displaced(o, q, to_dev(kb, "bf16"), to_dev(vb, "bf16"), heads, 64, 0.0, ws)
    torch.cuda.synchronize()
    exact = np.broadcast_to(bf16_bits_to_f32(vb).astype(np.float64).mean(axis=1, keepdims=True), (B, nq, hd))
    check(bits(o), exact, f"attention zero query {nkv} keys {'split' if use_ws else 'unsplit'}",
          need_near=nkv >= 64)


# ======================================================================== CFG
def test_cfg_combine_rounds_to_nearest_even():
    import displaced_patch_parallelism_net_amd as dpp
    n = 4099                           # vector body and a scalar tail
    rng = np.random.default_rng(35)
    say("rounding cfg", n)
    j = rng.integers(16, 81, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    step = rng.choice([-1, 1], size=n)
    u = s * (1.0 + j * 2.0 ** -7)
    c = s * (1.0 + (j + step) * 2.0 ** -7)
    ub, cb = f32_to_bf16_bits(u.astype(np.float32)), f32_to_bf16_bits(c.astype(np.float32))
    ud, cd = to_dev(ub, "bf16"), to_dev(cb, "bf16")
    ws = torch.empty(dpp.dpp_cfg_combine_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    rel = torch.zeros(1, device="cuda")
    allx, allbits = [], []
    for w in (0.5, 1.5, 7.5, 0.5 + 2.0 ** -10, 0.5 - 2.0 ** -10):
        e = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        dpp.dpp_cfg_combine_relmae(e, rel, cd, ud, w, ws)
        torch.cuda.synchronize()
        uv, cv = bf16_bits_to_f32(ub).astype(np.float64), bf16_bits_to_f32(cb).astype(np.float64)
        allx.append(uv + w * (cv - uv))
        allbits.append(bits(e))
    check(np.concatenate(allbits), np.concatenate(allx), "cfg combine")
