"""Pins of the CPU oracle to things other than itself.

Each pin is one of: an independent library routine applied to the plain
definition (torch CPU float64 group_norm / conv2d / scaled_dot_product_attention,
torch's own bf16 conversion), brute force in pure Python loops on tiny inputs,
a closed form worked by hand, or an invariant of the method (stale == fresh
gives the full-image layer; the patch sums add up to the image sums; rows
outside the halo have no influence).  A dropped term, a wrong sign or index,
or a transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from dpp_synth import CONFIGS, Config, layer_inputs, attention_inputs, values

RNG = np.random.default_rng(1234)


def spliced(stale, patch, r0):
    s = stale.copy()
    s[:, r0:r0 + patch.shape[1]] = patch
    return s


def sums_per_patch(x, P, G):
    B, H, W, C = x.shape
    R = H // P
    out = np.zeros((B, P, G, 2))
    cg = C // G
    for q in range(P):
        blk = x[:, q * R:(q + 1) * R]
        for g in range(G):
            v = blk[..., g * cg:(g + 1) * cg]
            out[:, q, g, 0] = v.sum(axis=(1, 2, 3))
            out[:, q, g, 1] = (v * v).sum(axis=(1, 2, 3))
    return out


# ----------------------------------------------------------------- bf16 rounding
def test_bf16_round_hand_ties():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even
    # mantissa (1.0).  1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and
    # 1 + 2^-6 (even): goes up.  Truncation or round-half-up fail one of them.
    a = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20, 0.0, 2.0 ** -130])
    got = oracle.bf16_round(a)
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7, 0.0, 2.0 ** -130])
    np.testing.assert_array_equal(got, want)


def test_bf16_round_matches_torch(torch_cpu):
    torch = torch_cpu
    a = RNG.standard_normal(20000) * np.exp(RNG.uniform(-20, 20, 20000))
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(a), ref)


# ----------------------------------------------------------------- splice
def test_splice_exact():
    full = RNG.standard_normal((2, 6, 5, 3)).astype(np.float32)
    patch = RNG.standard_normal((2, 2, 5, 3)).astype(np.float32)
    out = oracle.splice(full, patch, 3)
    assert out.dtype == np.float32
    np.testing.assert_array_equal(out[:, 3:5], patch)
    np.testing.assert_array_equal(out[:, :3], full[:, :3])
    np.testing.assert_array_equal(out[:, 5:], full[:, 5:])
    assert not np.shares_memory(out, full)


def test_splice_bits_bf16():
    full = RNG.integers(0, 2 ** 16, (1, 4, 3, 8), dtype=np.uint16)
    patch = RNG.integers(0, 2 ** 16, (1, 1, 3, 8), dtype=np.uint16)
    out = oracle.splice(full, patch, 2)
    ref = np.concatenate([full[:, :2], patch, full[:, 3:]], axis=1)
    np.testing.assert_array_equal(out, ref)


# ----------------------------------------------------------------- GroupNorm
def test_gn_hand_example():
    # Image of 2 rows x 1 column x 2 channels, one group: rows [1,3] and [5,7].
    # mean 4, E[x^2] = (1+9+25+49)/4 = 21, var = 21 - 16 = 5.  Patch 0 is row 0
    # (fresh); patch 1's raw sums from the previous step are (12, 74).
    x = np.array([[[[1.0, 3.0]]]])
    stale = np.array([[[[99.0, 99.0]], [[12.0, 74.0]]]])   # slot 0 must be ignored
    gamma = np.array([2.0, 1.0])
    beta = np.array([0.5, 0.0])
    y, fresh = oracle.groupnorm_stale(x, stale, gamma, beta, H=2, G=1, p=0, eps=1e-5)
    r = 1.0 / math.sqrt(5.0 + 1e-5)
    np.testing.assert_allclose(y.reshape(-1), [-3 * r * 2 + 0.5, -1 * r], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(fresh.reshape(-1), [4.0, 10.0])


@pytest.mark.parametrize("P,p", [(1, 0), (2, 0), (2, 1), (4, 2), (3, 2)])
def test_gn_matches_torch_group_norm_on_spliced_image(torch_cpu, P, p):
    torch = torch_cpu
    B, H, W, C, G = 2, 12, 5, 12, 3
    R = H // P
    fresh_full = RNG.standard_normal((B, H, W, C)) * 1.7 + 0.3
    stale_full = fresh_full + 0.05 * RNG.standard_normal((B, H, W, C))
    gamma = 1 + 0.1 * RNG.standard_normal(C)
    beta = 0.1 * RNG.standard_normal(C)
    r0 = p * R
    x_p = fresh_full[:, r0:r0 + R]
    stats = sums_per_patch(stale_full, P, G) if P > 1 else None
    y, fresh = oracle.groupnorm_stale(x_p, stats, gamma, beta, H, G, p, eps=1e-5)
    S = spliced(stale_full, x_p, r0)
    ref = torch.nn.functional.group_norm(torch.from_numpy(S).permute(0, 3, 1, 2), G,
                                         torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-5)
    ref = ref.permute(0, 2, 3, 1).numpy()[:, r0:r0 + R]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(fresh, sums_per_patch(x_p, 1, G)[:, 0], rtol=1e-13, atol=1e-11)


def test_gn_bruteforce_loops():
    # Two-pass mean/variance of the spliced image in plain loops (a different
    # formula than the oracle's raw sums).
    B, H, W, C, G, P, p = 1, 4, 3, 4, 2, 2, 1
    R = H // P
    fresh_full = RNG.standard_normal((B, H, W, C))
    stale_full = RNG.standard_normal((B, H, W, C))
    gamma = RNG.standard_normal(C)
    beta = RNG.standard_normal(C)
    r0 = p * R
    y, _ = oracle.groupnorm_stale(fresh_full[:, r0:r0 + R], sums_per_patch(stale_full, P, G),
                                  gamma, beta, H, G, p, eps=1e-5)
    cg = C // G
    for g in range(G):
        vals = []
        for r in range(H):
            for w in range(W):
                for c in range(g * cg, (g + 1) * cg):
                    src = fresh_full if r0 <= r < r0 + R else stale_full
                    vals.append(src[0, r, w, c])
        mu = sum(vals) / len(vals)
        var = sum((v - mu) ** 2 for v in vals) / len(vals)
        for i in range(R):
            for w in range(W):
                for c in range(g * cg, (g + 1) * cg):
                    want = (fresh_full[0, r0 + i, w, c] - mu) / math.sqrt(var + 1e-5) * gamma[c] + beta[c]
                    assert abs(y[0, i, w, c] - want) < 1e-12


def test_gn_patch_sums_add_to_image_sums_and_own_slot_ignored():
    B, H, W, C, G, P = 1, 8, 4, 6, 3, 4
    x = RNG.standard_normal((B, H, W, C))
    R = H // P
    total = sum(oracle.patch_sums(x[:, q * R:(q + 1) * R], G) for q in range(P))
    np.testing.assert_allclose(total, oracle.patch_sums(x, G), rtol=1e-13, atol=1e-12)
    stats = sums_per_patch(x, P, G)
    gamma, beta = np.ones(C), np.zeros(C)
    y1, _ = oracle.groupnorm_stale(x[:, R:2 * R], stats, gamma, beta, H, G, 1)
    stats2 = stats.copy()
    stats2[:, 1] = 1e6
    y2, _ = oracle.groupnorm_stale(x[:, R:2 * R], stats2, gamma, beta, H, G, 1)
    np.testing.assert_array_equal(y1, y2)
    # and another patch's slot does matter
    stats3 = stats.copy()
    stats3[:, 2, :, 0] += 5.0
    y3, _ = oracle.groupnorm_stale(x[:, R:2 * R], stats3, gamma, beta, H, G, 1)
    assert np.abs(y3 - y1).max() > 1e-3


# ----------------------------------------------------------------- conv
def test_conv_box_filter_hand_example():
    # One channel, all-ones 3x3 kernel, no bias: each output is the sum of its
    # 3x3 neighbourhood with zeros outside the image.  Image 3x3 with values
    # 1..9 (row-major) split in 3 one-row patches; patch 1 (the middle row) is
    # fresh = stale + 100.
    img = np.arange(1.0, 10.0).reshape(1, 3, 3, 1)
    fresh_mid = img[:, 1:2] + 100.0
    w = np.ones((1, 3, 3, 1))
    y = oracle.conv3x3_halo(fresh_mid, img, w, None, row0=1).reshape(-1)
    # column 0: rows 0..2 cols 0..1 -> (1+2) + (104+105) + (7+8) = 227
    # column 1: (1+2+3) + (104+105+106) + (7+8+9) = 345
    # column 2: (2+3) + (105+106) + (8+9) = 233
    np.testing.assert_array_equal(y, [227.0, 345.0, 233.0])
    y0 = oracle.conv3x3_halo(img[:, 0:1], img, w, np.array([0.5]), row0=0).reshape(-1)
    # top row: row -1 is zero padding; (1+2)+(4+5) = 12, 1+2+3+4+5+6 = 21, 2+3+5+6 = 16
    np.testing.assert_array_equal(y0, [12.5, 21.5, 16.5])


@pytest.mark.parametrize("P,p", [(1, 0), (3, 0), (3, 1), (3, 2)])
def test_conv_matches_torch_conv2d_on_spliced_image(torch_cpu, P, p):
    torch = torch_cpu
    B, H, W, Cin, Cout = 2, 9, 7, 5, 4
    R = H // P
    r0 = p * R
    fresh_full = RNG.standard_normal((B, H, W, Cin))
    stale_full = RNG.standard_normal((B, H, W, Cin))
    wt = RNG.standard_normal((Cout, 3, 3, Cin))
    bias = RNG.standard_normal(Cout)
    x_p = fresh_full[:, r0:r0 + R]
    y = oracle.conv3x3_halo(x_p, stale_full if P > 1 else None, wt, bias, r0)
    S = spliced(stale_full, x_p, r0) if P > 1 else x_p
    ref = torch.nn.functional.conv2d(torch.from_numpy(S).permute(0, 3, 1, 2),
                                     torch.from_numpy(wt).permute(0, 3, 1, 2), torch.from_numpy(bias), padding=1)
    ref = ref.permute(0, 2, 3, 1).numpy()[:, r0:r0 + R]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-11)


def test_conv_bruteforce_loops():
    B, H, W, Cin, Cout, P, p = 1, 4, 3, 2, 2, 2, 1
    R = H // P
    r0 = p * R
    fresh_full = RNG.standard_normal((B, H, W, Cin))
    stale_full = RNG.standard_normal((B, H, W, Cin))
    wt = RNG.standard_normal((Cout, 3, 3, Cin))
    bias = RNG.standard_normal(Cout)
    y = oracle.conv3x3_halo(fresh_full[:, r0:r0 + R], stale_full, wt, bias, r0)
    for i in range(R):
        for w in range(W):
            for o in range(Cout):
                acc = bias[o]
                for ky in range(3):
                    for kx in range(3):
                        r, c = r0 + i + ky - 1, w + kx - 1
                        if 0 <= r < H and 0 <= c < W:
                            src = fresh_full if r0 <= r < r0 + R else stale_full
                            for ci in range(Cin):
                                acc += wt[o, ky, kx, ci] * src[0, r, c, ci]
                assert abs(y[0, i, w, o] - acc) < 1e-12


def test_conv_only_halo_rows_of_stale_matter():
    B, H, W, C, P = 1, 12, 5, 3, 4
    R = H // P
    p, r0 = 1, 3
    fresh = RNG.standard_normal((B, R, W, C))
    stale = RNG.standard_normal((B, H, W, C))
    wt = RNG.standard_normal((C, 3, 3, C))
    y = oracle.conv3x3_halo(fresh, stale, wt, None, r0)
    st2 = stale.copy()
    st2[:, :r0 - 1] += 7.0
    st2[:, r0 + R + 1:] -= 3.0
    st2[:, r0:r0 + R] = 1e9          # own rows of the stale image are replaced
    np.testing.assert_array_equal(oracle.conv3x3_halo(fresh, st2, wt, None, r0), y)
    st3 = stale.copy()
    st3[:, r0 - 1] += 1.0            # the top halo row feeds output row 0 only
    d = np.abs(oracle.conv3x3_halo(fresh, st3, wt, None, r0) - y).max(axis=(0, 2, 3))
    assert d[0] > 1e-3 and np.all(d[1:] == 0)


def test_conv_sampled_equals_full():
    B, H, W, C, P = 2, 8, 6, 4, 2
    R = H // P
    fresh = RNG.standard_normal((B, R, W, C))
    stale = RNG.standard_normal((B, H, W, C))
    wt = RNG.standard_normal((3, 3, 3, C))
    bias = RNG.standard_normal(3)
    full = oracle.conv3x3_halo(fresh, stale, wt, bias, R)
    bi, ii, wi = [0, 1, 1, 0], [0, 3, 2, 1], [0, 5, 3, 2]
    got = oracle.conv3x3_halo_sampled(fresh, stale, wt, bias, R, bi, ii, wi)
    np.testing.assert_allclose(got, full[bi, ii, wi], rtol=0, atol=1e-12)


# ----------------------------------------------------------------- attention
def test_attention_hand_example():
    # One head, D = 1 (scale 1): scores [0, ln 3] -> weights [1/4, 3/4];
    # values [1, 5] -> output 1/4 + 15/4 = 4.
    q = np.array([[[math.log(3.0)]]])
    k = np.array([[[0.0], [1.0]]])
    v = np.array([[[1.0], [5.0]]])
    o = oracle.self_attn_displaced(q, k, v, heads=1)
    assert abs(o[0, 0, 0] - 4.0) < 1e-14


def test_attention_matches_torch_sdpa(torch_cpu):
    torch = torch_cpu
    B, Nq, N, heads, D = 2, 7, 23, 3, 8
    q = RNG.standard_normal((B, Nq, heads * D))
    k = RNG.standard_normal((B, N, heads * D))
    v = RNG.standard_normal((B, N, heads * D))
    o = oracle.self_attn_displaced(q, k, v, heads, block=3)

    def split(t):
        return torch.from_numpy(t).reshape(B, -1, heads, D).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(split(q), split(k), split(v))
    ref = ref.permute(0, 2, 1, 3).reshape(B, Nq, heads * D).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    o2 = oracle.self_attn_displaced(q, k, v, heads, scale=0.3)
    ref2 = torch.nn.functional.scaled_dot_product_attention(split(q), split(k), split(v), scale=0.3)
    np.testing.assert_allclose(o2, ref2.permute(0, 2, 1, 3).reshape(B, Nq, heads * D).numpy(), rtol=0, atol=1e-12)


def test_attention_bruteforce_loops():
    B, Nq, N, heads, D = 1, 3, 5, 2, 3
    q = RNG.standard_normal((B, Nq, heads * D))
    k = RNG.standard_normal((B, N, heads * D))
    v = RNG.standard_normal((B, N, heads * D))
    o = oracle.self_attn_displaced(q, k, v, heads)
    for h in range(heads):
        for i in range(Nq):
            s = [sum(q[0, i, h * D + d] * k[0, j, h * D + d] for d in range(D)) / math.sqrt(D) for j in range(N)]
            e = [math.exp(x) for x in s]          # no max subtraction: different route
            z = sum(e)
            for d in range(D):
                want = sum(e[j] * v[0, j, h * D + d] for j in range(N)) / z
                assert abs(o[0, i, h * D + d] - want) < 1e-12


def test_attention_closed_forms():
    B, Nq, N, heads, D = 1, 4, 9, 2, 4
    v = RNG.standard_normal((B, N, heads * D))
    k = RNG.standard_normal((B, N, heads * D))
    # Q = 0: uniform weights -> mean of V
    o = oracle.self_attn_displaced(np.zeros((B, Nq, heads * D)), k, v, heads)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), rtol=0, atol=1e-14)
    # identical key rows: uniform weights whatever Q is
    k_same = np.broadcast_to(k[:, :1], k.shape).copy()
    o = oracle.self_attn_displaced(RNG.standard_normal((B, Nq, heads * D)), k_same, v, heads)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), rtol=0, atol=1e-13)
    # a single key: output = that value
    o = oracle.self_attn_displaced(RNG.standard_normal((B, Nq, heads * D)), k[:, :1], v[:, :1], heads)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :1], o.shape), rtol=0, atol=1e-15)
    # a key that dominates (huge score): output = its value
    k_dom = k.copy()
    qq = RNG.standard_normal((B, Nq, heads * D))
    k_dom[:, 4] = 0
    k_dom[:, 4, :D] = 1e4 * np.sign(qq[:, 0, :D])
    o = oracle.self_attn_displaced(qq[:, :1], k_dom, v, heads)
    np.testing.assert_allclose(o[0, 0, :D], v[0, 4, :D], rtol=0, atol=1e-12)


def test_attention_rows_subset_and_displacement_invariant():
    # stale == fresh: the patch's queries against the full K/V give the rows
    # of full-image attention (synchronous first step).
    B, H, W, heads, D, P = 1, 6, 4, 2, 4, 3
    N = H * W
    x = RNG.standard_normal((B, N, heads * D))
    full = oracle.self_attn_displaced(x, x, x, heads)
    R = H // P
    for p in range(P):
        qs = x[:, p * R * W:(p + 1) * R * W]
        np.testing.assert_allclose(oracle.self_attn_displaced(qs, x, x, heads), full[:, p * R * W:(p + 1) * R * W],
                                   rtol=0, atol=1e-13)
    got = oracle.self_attn_displaced(x, x, x, heads, rows=([0, 0, 0], [5, 0, 23]))
    np.testing.assert_allclose(got, full[0, [5, 0, 23]], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- CFG
def test_cfg_closed_forms():
    u = np.array([1.0, -2.0, 3.0, 0.5])
    c = np.array([2.0, -2.0, 2.5, 1.5])
    eps, rel = oracle.cfg_combine_relmae(c, u, 7.5)
    # u + 7.5 (c - u) = [1+7.5, -2, 3-3.75, 0.5+7.5]; rel = (1+0+0.5+1)/(1+2+3+0.5)
    np.testing.assert_array_equal(eps, [8.5, -2.0, -0.75, 8.0])
    assert rel == pytest.approx(2.5 / 6.5, rel=1e-15)
    x = RNG.standard_normal(1000)
    y = RNG.standard_normal(1000)
    np.testing.assert_array_equal(oracle.cfg_combine_relmae(x, y, 0.0)[0], y)
    np.testing.assert_allclose(oracle.cfg_combine_relmae(x, y, 1.0)[0], x, rtol=0, atol=1e-15)
    # eps_c = (1 + a) eps_u exactly -> rel = |a|
    u = np.array([1.0, -2.0, 4.0, -0.5])
    assert oracle.cfg_combine_relmae(1.25 * u, u, 7.5)[1] == pytest.approx(0.25, rel=1e-15)
    assert oracle.cfg_combine_relmae(0.5 * u, u, 7.5)[1] == pytest.approx(0.5, rel=1e-15)
    assert oracle.cfg_combine_relmae(u, u, 7.5)[1] == 0.0
    assert math.isnan(oracle.cfg_combine_relmae(np.zeros(4), np.zeros(4), 7.5)[1])
    assert math.isinf(oracle.cfg_combine_relmae(np.ones(4), np.zeros(4), 7.5)[1])


# ----------------------------------------------------------------- chained block
def _torch_block_full(torch, x, gamma, beta, wt, bias, G, heads, eps):
    F = torch.nn.functional
    t = torch.from_numpy(x).permute(0, 3, 1, 2)
    a1 = F.group_norm(t, G, torch.from_numpy(gamma), torch.from_numpy(beta), eps=eps)
    a2 = F.conv2d(a1, torch.from_numpy(wt).permute(0, 3, 1, 2), torch.from_numpy(bias), padding=1)
    B, C, H, W = a2.shape
    tok = a2.permute(0, 2, 3, 1).reshape(B, H * W, heads, C // heads).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(tok, tok, tok)
    return (a1.permute(0, 2, 3, 1).numpy(), a2.permute(0, 2, 3, 1).numpy(),
            o.permute(0, 2, 1, 3).reshape(B, H * W, C).numpy())


@pytest.mark.parametrize("P", [1, 2, 4])
def test_block_stale_equals_fresh_is_full_layer(torch_cpu, P):
    # Synchronous first step: with stale == fresh every patch's displaced block
    # equals the unpatched full-image block restricted to its rows.
    torch = torch_cpu
    B, H, W, C, G, heads = 2, 8, 5, 8, 4, 2
    x = RNG.standard_normal((B, H, W, C))
    gamma = 1 + 0.1 * RNG.standard_normal(C)
    beta = 0.1 * RNG.standard_normal(C)
    wt = 0.2 * RNG.standard_normal((C, 3, 3, C))
    bias = 0.1 * RNG.standard_normal(C)
    a1, a2, o_full = _torch_block_full(torch, x, gamma, beta, wt, bias, G, heads, 1e-5)
    st = oracle.previous_step_state(x, gamma, beta, wt, bias, P, G, 1e-5, bf16=False)
    np.testing.assert_allclose(st["a1"], a1, rtol=0, atol=1e-11)
    np.testing.assert_allclose(st["a2"], a2, rtol=0, atol=1e-10)
    R = H // P
    for p in range(P):
        out = oracle.displaced_block(x, st, gamma, beta, wt, bias, P, p, G, heads, 1e-5, bf16=False)
        sl = slice(p * R * W, (p + 1) * R * W)
        np.testing.assert_allclose(out["o"], o_full[:, sl], rtol=0, atol=1e-10)
        np.testing.assert_allclose(out["kv"], a2, rtol=0, atol=1e-10)


def test_block_displaced_differs_only_through_stale_rows(torch_cpu):
    # With stale != fresh, patch p's GN output equals torch group_norm of the
    # spliced image, and its conv output equals torch conv2d of the spliced
    # GN image (fresh own rows, stale halos).
    torch = torch_cpu
    F = torch.nn.functional
    cfg = CONFIGS["tiny_f32"]
    inp = layer_inputs(cfg)
    xf, xs = values(cfg, inp["x_fresh"]).astype(np.float64), values(cfg, inp["x_stale"]).astype(np.float64)
    wt = values(cfg, inp["conv_w"]).astype(np.float64)
    gamma, beta, bias = (inp[k].astype(np.float64) for k in ("gamma", "beta", "conv_b"))
    st = oracle.previous_step_state(xs, gamma, beta, wt, bias, cfg.P, cfg.G, cfg.gn_eps, bf16=False)
    for p in range(cfg.P):
        out = oracle.displaced_block(xf, st, gamma, beta, wt, bias, cfg.P, p, cfg.G, cfg.heads, cfg.gn_eps, bf16=False)
        r0, R = cfg.row0(p), cfg.rows
        S = spliced(xs, xf[:, r0:r0 + R], r0)
        gn = F.group_norm(torch.from_numpy(S).permute(0, 3, 1, 2), cfg.G, torch.from_numpy(gamma),
                          torch.from_numpy(beta), eps=cfg.gn_eps).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(out["y1"], gn[:, r0:r0 + R], rtol=0, atol=1e-11)
        S2 = spliced(st["a1"], out["y1"], r0)
        cv = F.conv2d(torch.from_numpy(S2).permute(0, 3, 1, 2), torch.from_numpy(wt).permute(0, 3, 1, 2),
                      torch.from_numpy(bias), padding=1).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(out["y2"], cv[:, r0:r0 + R], rtol=0, atol=1e-11)


def test_block_bf16_rounds_stored_outputs():
    cfg = Config("t", B=1, H=4, W=4, C=64, P=2, G=8, heads=1, D=64)
    inp = layer_inputs(cfg)
    xf, xs = values(cfg, inp["x_fresh"]), values(cfg, inp["x_stale"])
    wt = values(cfg, inp["conv_w"])
    st = oracle.previous_step_state(xs, inp["gamma"], inp["beta"], wt, inp["conv_b"], cfg.P, cfg.G, 1e-5, bf16=True)
    out = oracle.displaced_block(xf, st, inp["gamma"], inp["beta"], wt, inp["conv_b"], cfg.P, 1, cfg.G, 1, 1e-5, bf16=True)
    for key in ("y1", "y2", "kv"):
        np.testing.assert_array_equal(oracle.bf16_round(out[key]), out[key])
    np.testing.assert_array_equal(oracle.bf16_round(st["a1"]), st["a1"])


def test_oracle_and_synth_are_independent_of_the_gpu_package():
    import pathlib
    root = pathlib.Path(__file__).resolve().parents[1]
    for f in list((root / "oracle").glob("*.py")) + list((root / "dpp_synth").glob("*.py")):
        text = f.read_text()
        assert "displaced_patch_parallelism_net_amd" not in text, f
        assert "ctypes" not in text, f


def test_half_ulp_helper_bounds_bf16_rounding():
    # the parity allowance is exactly the worst rounding distance
    from tests._helpers import half_ulp_bf16
    a = RNG.standard_normal(50000) * np.exp(RNG.uniform(-10, 10, 50000))
    d = np.abs(oracle.bf16_round(a) - a)
    assert np.all(d <= half_ulp_bf16(a) * (1 + 1e-12))
    assert np.max(d / half_ulp_bf16(a)) > 0.99
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([6.0]))[0] == 2.0 ** -6


# ------------------------------------------------------------------ projections and SiLU
def test_silu_closed_forms():
    # z sigmoid(z): 0 -> 0; 1 -> 1/(1+e^-1); odd part: silu(z) - silu(-z) = z;
    # large z -> z, large -z -> 0
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(oracle.silu(np.array([-2.0]))[0] - (-2.0 / (1.0 + math.exp(2.0)))) < 1e-15
    z = RNG.standard_normal(1000) * 4
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-12)
    assert abs(oracle.silu(np.array([60.0]))[0] - 60.0) < 1e-12
    assert abs(oracle.silu(np.array([-60.0]))[0]) < 1e-20
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0


def test_gn_silu_is_silu_of_torch_group_norm(torch_cpu):
    torch = torch_cpu
    x = RNG.standard_normal((1, 6, 5, 8))
    gamma, beta = 1 + 0.1 * RNG.standard_normal(8), 0.1 * RNG.standard_normal(8)
    y, _ = oracle.groupnorm_silu_stale(x, None, gamma, beta, 6, 4, 0, 1e-5)
    t = torch.nn.functional.group_norm(torch.from_numpy(x).permute(0, 3, 1, 2), 4, torch.from_numpy(gamma),
                                       torch.from_numpy(beta), 1e-5)
    want = torch.nn.functional.silu(t).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_linear_bruteforce_and_torch(torch_cpu):
    torch = torch_cpu
    x = RNG.standard_normal((2, 3, 5))
    w = RNG.standard_normal((4, 5))
    b = RNG.standard_normal(4)
    y = oracle.linear(x, w, b)
    for bi in range(2):
        for m in range(3):
            for n in range(4):
                acc = b[n]
                for k in range(5):
                    acc += x[bi, m, k] * w[n, k]
                assert abs(y[bi, m, n] - acc) < 1e-12
    want = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.linear(x, w), y - b, rtol=1e-13, atol=1e-13)


def test_projected_attention_identity_weights_reduce_to_plain():
    # W = I, b = 0: the projections vanish and the result is the identity-
    # projection attention of the spliced buffer (reading R6 as a special case)
    B, N, Nq, C, heads, t0 = 1, 48, 12, 128, 2, 24
    x = RNG.standard_normal((B, Nq, C))
    ks, vs = RNG.standard_normal((B, N, C)), RNG.standard_normal((B, N, C))
    I, z = np.eye(C), np.zeros(C)
    r = oracle.projected_attention(x, ks, vs, t0, I, z, I, z, I, z, I, z, heads, bf16=False)
    K, V = ks.copy(), vs.copy()
    K[:, t0:t0 + Nq] = x
    V[:, t0:t0 + Nq] = x
    np.testing.assert_allclose(r["out"], oracle.self_attn_displaced(x, K, V, heads), rtol=1e-12, atol=1e-12)


def test_projected_attention_splice_commutes_with_projection():
    # projecting the spliced input equals splicing the projections (R11): the
    # stale K/V are the projections of the stale hidden states
    B, N, Nq, C, heads, t0 = 2, 40, 8, 64, 1, 16
    xs = RNG.standard_normal((B, N, C))
    x = RNG.standard_normal((B, Nq, C))
    wq, wk, wv, wo = (RNG.standard_normal((C, C)) / 8 for _ in range(4))
    bq, bk, bv, bo = (RNG.standard_normal(C) / 8 for _ in range(4))
    r = oracle.projected_attention(x, oracle.linear(xs, wk, bk), oracle.linear(xs, wv, bv), t0, wq, bq, wk, bk, wv,
                                   bv, wo, bo, heads, bf16=False)
    xsp = xs.copy()
    xsp[:, t0:t0 + Nq] = x
    K, V = oracle.linear(xsp, wk, bk), oracle.linear(xsp, wv, bv)
    want = oracle.linear(oracle.self_attn_displaced(oracle.linear(x, wq, bq), K, V, heads), wo, bo)
    np.testing.assert_allclose(r["out"], want, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["k"], K, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- stage switching (R13)
U_TRACE = [0.5, 0.3, 0.2, 0.17, 0.16, 0.155, 0.15, 0.16, 0.2, 0.3]


def test_schedule_hand_worked_u_trace():
    # declines 0.2, 0.1, 0.03: the fastest is 0.2, so the first decline at or
    # below 0.05 (step 3) ends the warm-up; the minimum of the parallel stage
    # reaches 0.15 at step 6 and 0.16 > 1.02 * 0.15 at step 7 ends it
    st, t1, t2 = oracle.hybrid_schedule(U_TRACE)
    assert (t1, t2) == (3, 7)
    assert st.tolist() == [0, 0, 0, 1, 1, 1, 1, 2, 2, 2]
    # a longer warm-up floor moves tau1 only
    assert oracle.hybrid_schedule(U_TRACE, min_warmup=5)[1:] == (5, 7)
    # rho = 0.1 needs a decline <= 0.02: step 4 (0.01)
    assert oracle.hybrid_schedule(U_TRACE, rho=0.1)[1:] == (4, 7)
    # eps = 0.1: 0.16 <= 0.165 keeps step 7 parallel; 0.2 > 0.165 ends it at 8
    assert oracle.hybrid_schedule(U_TRACE, eps=0.1)[1:] == (3, 8)


@pytest.mark.parametrize("r,rho", [(0.8, 0.25), (0.9, 0.25), (0.7, 0.1), (0.95, 0.5)])
def test_schedule_geometric_decay_closed_form(r, rho):
    # d_i = r^i: decline_i = r^(i-1) (1 - r), largest at i = 1, so the warm-up
    # ends at the first i with r^(i-1) <= rho: i = 1 + ceil(ln rho / ln r);
    # a strictly falling trace never starts the fully-connecting stage
    x = math.log(rho) / math.log(r)
    assert abs(x - round(x)) > 1e-3
    T = 80
    d = r ** np.arange(T)
    st, t1, t2 = oracle.hybrid_schedule(d, rho=rho)
    assert t1 == 1 + math.ceil(x)
    assert t2 == T
    assert (st[:t1] == 0).all() and (st[t1:] == 1).all()


@pytest.mark.parametrize("g", [1.5, 1.005, 1.0013])
def test_schedule_decay_then_growth_closed_form(g):
    # r^i down to step m, then r^m g^(i-m): the parallel stage's minimum is r^m
    # and it ends at the first i with g^(i-m) > 1 + eps, i.e.
    # i = m + floor(ln(1 + eps) / ln g) + 1
    r, m, T, eps = 0.8, 30, 200, 0.02
    x = math.log(1 + eps) / math.log(g)
    assert abs(x - round(x)) > 1e-2
    i = np.arange(T)
    d = np.where(i <= m, r ** i, r ** m * g ** (i - m))
    st, t1, t2 = oracle.hybrid_schedule(d, eps=eps)
    assert t1 == 8
    assert t2 == m + math.floor(x) + 1
    assert st.tolist() == [0] * t1 + [1] * (t2 - t1) + [2] * (T - t2)


def test_schedule_degenerate_traces():
    T = 12
    # a constant-rate decline never flattens (exact binary steps)
    lin = (T - np.arange(T)) * 0.125
    assert oracle.hybrid_schedule(lin)[1:] == (T, T)
    # ... unless rho = 1: then the first allowed step ends the warm-up
    assert oracle.hybrid_schedule(lin, rho=1.0)[1:] == (1, T)
    assert oracle.hybrid_schedule(lin, rho=1.0, min_warmup=4)[1:] == (4, T)
    # a flat trace has no positive decline: the warm-up never ends
    st, t1, t2 = oracle.hybrid_schedule(np.full(T, 0.3))
    assert (t1, t2) == (T, T) and not st.any()
    # a single step and a rising trace stay in the warm-up
    assert oracle.hybrid_schedule([0.4])[1:] == (1, 1)
    assert oracle.hybrid_schedule(np.arange(1, T + 1) * 0.1)[1:] == (T, T)
    # rho = 0: only a non-falling step ends the warm-up (step 7, 0.16 after
    # 0.15); the parallel stage then starts at 0.16 and 0.2 ends it at step 8
    assert oracle.hybrid_schedule(U_TRACE, rho=0.0)[1:] == (7, 8)


def test_schedule_nan_steps_never_switch():
    # 0/0 discrepancies (NaN) neither end the warm-up nor the parallel stage
    d = list(U_TRACE)
    d[3] = float("nan")          # would have ended the warm-up
    # step 3: NaN decline; step 4: NaN decline; step 5: 0.005 <= 0.05
    assert oracle.hybrid_schedule(d)[1:] == (5, 7)
    d = list(U_TRACE)
    d[7] = float("nan")          # would have ended the parallel stage
    assert oracle.hybrid_schedule(d)[1:] == (3, 8)


def test_schedule_is_causal():
    # the stage of step i depends on steps 0..i only: scheduling a prefix of
    # the trace gives the prefix of the full schedule
    from dpp_synth import relmae_trace
    for seed in range(6):
        d = relmae_trace(seed, 60, noise=0.005)
        full = oracle.hybrid_schedule(d)[0]
        for n in (1, 7, 23, 41, 60):
            assert (oracle.hybrid_schedule(d[:n])[0] == full[:n]).all()
        assert (np.diff(full) >= 0).all()


# ----------------------------------------------------------------- component steps (R14)
def _chain_params(K, C, rng):
    return [{"gamma": 1 + 0.1 * rng.standard_normal(C), "beta": 0.1 * rng.standard_normal(C),
             "conv_w": 0.2 * rng.standard_normal((C, 3, 3, C)), "conv_b": 0.1 * rng.standard_normal(C)}
            for _ in range(K)]


def _torch_seq(torch, x, params, k, G, heads):
    # components 0..k applied in order with torch's own layers, as [B,H,W,C]
    B, H, W, C = x.shape
    for p in params[:k + 1]:
        _, _, o = _torch_block_full(torch, x, p["gamma"], p["beta"], p["conv_w"], p["conv_b"], G, heads, 1e-5)
        x = o.reshape(B, H, W, C)
    return x


def test_component_block_is_torch_block(torch_cpu):
    B, H, W, C, G, heads = 2, 6, 5, 8, 4, 2
    x = RNG.standard_normal((B, H, W, C))
    p = _chain_params(1, C, RNG)[0]
    a1, a2, o = _torch_block_full(torch_cpu, x, p["gamma"], p["beta"], p["conv_w"], p["conv_b"], G, heads, 1e-5)
    r = oracle.component_block(x, p["gamma"], p["beta"], p["conv_w"], p["conv_b"], G, heads, 1e-5, bf16=False)
    np.testing.assert_allclose(r["y1"], a1, rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["y2"], a2, rtol=0, atol=1e-10)
    np.testing.assert_allclose(r["o"], o.reshape(B, H, W, C), rtol=0, atol=1e-10)


@pytest.mark.parametrize("warmup", [1, 2, 5])
def test_async_chain_closed_form(torch_cpu, warmup):
    # Component k at step t sees the input of step s = t while t < warmup and
    # s = max(t - k, warmup - 1) afterwards: the chain's output equals the
    # ordinary model (components 0..k in order, torch layers) applied to x_s.
    # warmup >= T is the synchronous model at every step.
    B, H, W, C, G, heads, K, T = 1, 5, 4, 8, 4, 2, 3, 5
    base = RNG.standard_normal((B, H, W, C))
    xs = [base + 0.3 * t * RNG.standard_normal((B, H, W, C)) for t in range(T)]
    params = _chain_params(K, C, RNG)
    outs = oracle.async_component_chain(xs, params, G, heads, 1e-5, bf16=False, warmup=warmup)
    for t in range(T):
        for k in range(K):
            s = t if t < warmup else max(t - k, warmup - 1)
            want = _torch_seq(torch_cpu, xs[s], params, k, G, heads)
            np.testing.assert_allclose(outs[t][k]["o"], want, rtol=0, atol=1e-9, err_msg=f"t={t} k={k}")
    # the inputs really differ from step to step, so the pin sees the shift
    assert np.abs(_torch_seq(torch_cpu, xs[1], params, 2, G, heads)
                  - _torch_seq(torch_cpu, xs[0], params, 2, G, heads)).max() > 1e-3


def test_async_chain_bf16_rounds_every_stored_output():
    B, H, W, C, G, heads = 1, 4, 4, 64, 8, 1
    xs = [oracle.bf16_round(RNG.standard_normal((B, H, W, C))) for _ in range(2)]
    params = _chain_params(2, C, RNG)
    for p in params:
        p["conv_w"] = p["conv_w"] / 20     # soft attention weights: outputs are not single V rows
    outs = oracle.async_component_chain(xs, params, G, heads, 1e-5, bf16=True)
    for row in outs:
        for r in row:
            for n in ("y1", "y2", "o"):
                assert np.array_equal(r[n], oracle.bf16_round(r[n]))
                assert np.abs(r[n] - r[n + "_exact"]).max() > 0


# ----------------------------------------------------------------- attention block (R15)
def _block_params(C, rng):
    gamma = 1 + 0.1 * rng.standard_normal(C)
    beta = 0.1 * rng.standard_normal(C)
    wt = 0.2 * rng.standard_normal((C, 3, 3, C))
    bias = 0.1 * rng.standard_normal(C)
    proj = [x for _ in range(4) for x in (rng.standard_normal((C, C)) / np.sqrt(C), 0.1 * rng.standard_normal(C))]
    return gamma, beta, wt, bias, proj


def _torch_attention_block(torch, S_gn, S_conv, k_src, gamma, beta, wt, bias, proj, G, heads, eps, r0, R):
    """The block's layers by torch float64 library calls on spliced images:
    group_norm + silu of S_gn, conv2d of S_conv (the spliced GroupNorm+SiLU
    image), the patch's rows projected, attention over K/V = projections of
    k_src (the spliced conv image), out projection."""
    F = torch.nn.functional
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    wq, bq, wk, bk, wv, bv, wo, bo = proj
    gn = F.silu(F.group_norm(T(S_gn).permute(0, 3, 1, 2), G, T(gamma), T(beta), eps=eps))
    cv = F.conv2d(T(S_conv).permute(0, 3, 1, 2), T(wt).permute(0, 3, 1, 2), T(bias), padding=1)
    B, C, H, W = cv.shape
    rows = cv.permute(0, 2, 3, 1)[:, r0:r0 + R].reshape(B, R * W, C)
    q = F.linear(rows, T(wq), T(bq))
    kv_in = T(k_src).reshape(B, H * W, C)
    k, v = F.linear(kv_in, T(wk), T(bk)), F.linear(kv_in, T(wv), T(bv))
    hd = C // heads
    split = lambda t: t.reshape(B, t.shape[1], heads, hd).permute(0, 2, 1, 3)  # noqa: E731
    o = F.scaled_dot_product_attention(split(q), split(k), split(v)).permute(0, 2, 1, 3).reshape(B, R * W, C)
    out = F.linear(o, T(wo), T(bo))
    return gn.permute(0, 2, 3, 1).numpy(), cv.permute(0, 2, 3, 1).numpy(), out.numpy()


@pytest.mark.parametrize("P", [1, 2, 4])
def test_attention_block_stale_equals_fresh_is_full_block(torch_cpu, P):
    # Synchronous first step: with stale == fresh, patch p's block output is
    # the unpatched full-image block's output on its rows.
    torch = torch_cpu
    B, H, W, C, G, heads = 2, 8, 5, 16, 4, 2
    rng = np.random.default_rng(51)
    x = rng.standard_normal((B, H, W, C))
    gamma, beta, wt, bias, proj = _block_params(C, rng)
    wq, bq, wk, bk, wv, bv, wo, bo = proj
    st = oracle.previous_block_state(x, gamma, beta, wt, bias, wk, bk, wv, bv, P, G, 1e-5, bf16=False)
    st1 = oracle.previous_block_state(x, gamma, beta, wt, bias, wk, bk, wv, bv, 1, G, 1e-5, bf16=False)
    full = oracle.displaced_attention_block(x, st1, gamma, beta, wt, bias, *proj, 1, 0, G, heads, 1e-5, bf16=False)
    # the unpatched block is torch's layers on the image itself
    _, _, out_torch = _torch_attention_block(torch, x, full["y1"], full["y2"], gamma, beta, wt, bias, proj, G, heads,
                                             1e-5, 0, H)
    np.testing.assert_allclose(full["out_exact"], out_torch, rtol=0, atol=1e-10)
    R = H // P
    for p in range(P):
        out = oracle.displaced_attention_block(x, st, gamma, beta, wt, bias, *proj, P, p, G, heads, 1e-5, bf16=False)
        np.testing.assert_allclose(out["out_exact"], full["out_exact"][:, p * R * W:(p + 1) * R * W], rtol=0,
                                   atol=1e-11)
        np.testing.assert_allclose(out["k"], full["k"], rtol=0, atol=1e-11)


@pytest.mark.parametrize("P,p", [(2, 0), (4, 1), (4, 3)])
def test_attention_block_matches_torch_layers_on_spliced_images(torch_cpu, P, p):
    # stale != fresh: every stage equals torch's float64 layers on the spliced
    # images the pages' scheme defines (fresh own rows, previous step's rest)
    torch = torch_cpu
    B, H, W, C, G, heads = 1, 8, 6, 16, 4, 2
    rng = np.random.default_rng(52)
    xs = rng.standard_normal((B, H, W, C))
    xf = xs + 0.3 * rng.standard_normal((B, H, W, C))
    gamma, beta, wt, bias, proj = _block_params(C, rng)
    wq, bq, wk, bk, wv, bv, wo, bo = proj
    st = oracle.previous_block_state(xs, gamma, beta, wt, bias, wk, bk, wv, bv, P, G, 1e-5, bf16=False)
    R = H // P
    r0 = p * R
    out = oracle.displaced_attention_block(xf, st, gamma, beta, wt, bias, *proj, P, p, G, heads, 1e-5, bf16=False)
    S_gn = spliced(xs, xf[:, r0:r0 + R], r0)
    S_conv = spliced(st["a1"], out["y1"], r0)
    S_kv = spliced(st["a2"], out["y2"], r0)
    gn, cv, want = _torch_attention_block(torch, S_gn, S_conv, S_kv, gamma, beta, wt, bias, proj, G, heads, 1e-5, r0,
                                          R)
    np.testing.assert_allclose(out["y1"], gn[:, r0:r0 + R], rtol=0, atol=1e-11)
    np.testing.assert_allclose(out["y2"], cv[:, r0:r0 + R], rtol=0, atol=1e-10)
    np.testing.assert_allclose(out["out_exact"], want, rtol=0, atol=1e-10)


def test_attention_block_sampled_rows_equal_full():
    B, H, W, C, G, heads, P, p = 2, 8, 4, 16, 4, 2, 4, 2
    rng = np.random.default_rng(53)
    xs = rng.standard_normal((B, H, W, C))
    xf = xs + 0.3 * rng.standard_normal((B, H, W, C))
    gamma, beta, wt, bias, proj = _block_params(C, rng)
    wq, bq, wk, bk, wv, bv, wo, bo = proj
    for bf in (False, True):
        st = oracle.previous_block_state(xs, gamma, beta, wt, bias, wk, bk, wv, bv, P, G, 1e-5, bf16=bf)
        full = oracle.displaced_attention_block(xf, st, gamma, beta, wt, bias, *proj, P, p, G, heads, 1e-5, bf16=bf)
        bi, qi = np.array([0, 1, 1, 0]), np.array([0, 7, 3, 5])
        part = oracle.displaced_attention_block(xf, st, gamma, beta, wt, bias, *proj, P, p, G, heads, 1e-5, bf16=bf,
                                                attn_rows=(bi, qi))
        np.testing.assert_allclose(part["out_rows_exact"], full["out_exact"][bi, qi], rtol=0, atol=1e-13)
        np.testing.assert_allclose(part["o_rows_exact"], full["o_exact"][bi, qi], rtol=0, atol=1e-13)
