"""Plain float64 oracle functions (test infrastructure only; see package doc).

Layouts are token-major (NHWC): activations [B,H,W,C]; a patch is the row band
[row0, row0+rows) of that, [B,rows,W,C]; token t = row*W + col; head h owns
channels [h*D, (h+1)*D).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------ bf16 storage
def bf16_round(a) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64.

    A bf16 value is a float32 whose low 16 mantissa bits are zero.  The value
    is first rounded to float32 (nearest-even), then its float32 bit pattern u
    is rounded at bit 16: add 0x7FFF plus the lowest kept bit, drop 16 bits.
    Used where a bf16 configuration stores a layer output (reading R6)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return out.reshape(np.shape(a))


# ------------------------------------------------------------------ a1: splice
def splice(full, patch, row0: int) -> np.ndarray:
    """Full-image buffer with rows [row0, row0+rows) replaced by the patch.

    One device's local stand-in for gathering every patch's output and
    concatenating along the height axis into the reused full-image buffer
    (DistriFusion architecture article, communication section).  Exact: the
    result holds the input values unchanged (returned as a new array of the
    input dtype)."""
    full = np.asarray(full)
    patch = np.asarray(patch)
    rows = patch.shape[1]
    out = full.copy()
    out[:, row0:row0 + rows] = patch
    return out


# ------------------------------------------------------------------ a2: GroupNorm
def patch_sums(x_patch, G: int) -> np.ndarray:
    """Raw group sums of a patch: [B,G,2] = (sum x, sum x^2) over the patch's
    rows, all columns and the C/G channels of group g (reading R2)."""
    x = _f64(x_patch)
    B, R, W, C = x.shape
    xg = x.reshape(B, R * W, G, C // G)
    s1 = xg.sum(axis=(1, 3))
    s2 = (xg * xg).sum(axis=(1, 3))
    return np.stack([s1, s2], axis=-1)


def groupnorm_stale(x_patch, stale_stats, gamma, beta, H: int, G: int, p: int, eps: float = 1e-5):
    """GroupNorm of patch p with statistics of the spliced image (reading R2).

    x_patch [B,R,W,C]; stale_stats [B,P,G,2] raw sums of each patch from the
    previous step (slot p is ignored; may be None when P == 1); gamma, beta [C].
    Group statistics: totals T_k = sum_{q != p} stale_stats[:, q, g, k] + the
    fresh sums of x_patch; n = H*W*C/G; mean = T_1/n; var = max(T_2/n - mean^2,
    0).  y = (x - mean)/sqrt(var + eps) * gamma_c + beta_c.
    Returns (y [B,R,W,C] float64, fresh sums [B,G,2] float64).
    Module: DistriGroupNorm (DistriFusion architecture article, normalisation
    section); stale reuse: DistriFusion reading notes, Introduction fourth
    paragraph."""
    x = _f64(x_patch)
    B, R, W, C = x.shape
    cg = C // G
    fresh = patch_sums(x, G)
    total = fresh.copy()
    if stale_stats is not None:
        st = _f64(stale_stats)
        P = st.shape[1]
        for q in range(P):
            if q != p:
                total += st[:, q]
    n = float(H * W * cg)
    mean = total[..., 0] / n                           # [B,G]
    var = np.maximum(total[..., 1] / n - mean * mean, 0.0)
    rstd = 1.0 / np.sqrt(var + eps)
    mean_c = np.repeat(mean, cg, axis=1)[:, None, None, :]   # [B,1,1,C]
    rstd_c = np.repeat(rstd, cg, axis=1)[:, None, None, :]
    y = (x - mean_c) * rstd_c * _f64(gamma) + _f64(beta)
    return y, fresh


def silu(z) -> np.ndarray:
    """SiLU z * sigmoid(z) = z / (1 + exp(-z)), float64 (reading R12)."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def groupnorm_silu_stale(x_patch, stale_stats, gamma, beta, H: int, G: int, p: int, eps: float = 1e-5):
    """SiLU of groupnorm_stale(...): the GroupNorm + SiLU pair that opens an
    SDXL residual block (reading R12).  Returns (silu(y), fresh sums)."""
    y, fresh = groupnorm_stale(x_patch, stale_stats, gamma, beta, H, G, p, eps)
    return silu(y), fresh


# ------------------------------------------------------------------ a3: conv with halos
def _halo_band(x_patch, stale_full, row0: int) -> np.ndarray:
    """Rows [row0-1, row0+rows] of the spliced image, zero-padded by one at
    every image border: [B, rows+2, W+2, Cin].  The interior rows are the fresh
    patch; the two halo rows come from the stale image (reading R3: neighbours'
    fresh rows of this step are never available)."""
    x = _f64(x_patch)
    B, R, W, Cin = x.shape
    if stale_full is None:
        S = x
        H = R
        if row0 != 0:
            raise ValueError("stale image required for a partial band")
    else:
        S = splice(_f64(stale_full), x, row0)   # spliced image S_p (reading R1)
        H = S.shape[1]
    band = np.zeros((B, R + 2, W + 2, Cin))
    for i in range(R + 2):
        r = row0 - 1 + i
        if 0 <= r < H:
            band[:, i, 1:W + 1] = S[:, r]
    return band


def conv3x3_halo(x_patch, stale_full, weight, bias, row0: int) -> np.ndarray:
    """3x3 conv (stride 1, zero pad 1) of the spliced image, output rows of the
    patch only: y[b,i,w,o] = bias[o] + sum_{dy,dx in 0..2} sum_c
    weight[o,dy,dx,c] * Spad[b, row0+i+dy, w+dx, c], where Spad is the spliced
    image padded by one zero row/column on every side.
    x_patch [B,R,W,Cin]; stale_full [B,H,W,Cin] (None when the patch is the
    whole image); weight [Cout,3,3,Cin]; bias [Cout] or None.
    Module: DistriConv2dPP (DistriFusion architecture article, conv section);
    computing only the own region: DistriFusion reading notes, Introduction
    fourth paragraph."""
    band = _halo_band(x_patch, stale_full, row0)
    B, R2, W2, Cin = band.shape
    R, W = R2 - 2, W2 - 2
    wt = _f64(weight)
    Cout = wt.shape[0]
    y = np.zeros((B, R, W, Cout))
    for dy in range(3):
        for dx in range(3):
            tap = band[:, dy:dy + R, dx:dx + W, :]           # [B,R,W,Cin]
            y += tap @ wt[:, dy, dx, :].T
    if bias is not None:
        y += _f64(bias)
    return y


def conv3x3_halo_sampled(x_patch, stale_full, weight, bias, row0: int, b_idx, i_idx, w_idx) -> np.ndarray:
    """conv3x3_halo evaluated only at output positions (b, i, w) of the patch:
    returns [n, Cout].  Same definition, one output pixel at a time."""
    band = _halo_band(x_patch, stale_full, row0)
    wt = _f64(weight)
    Cout = wt.shape[0]
    wflat = wt.reshape(Cout, -1)                               # (dy, dx, c) order
    b_idx, i_idx, w_idx = (np.asarray(v, dtype=np.int64) for v in (b_idx, i_idx, w_idx))
    out = np.empty((len(b_idx), Cout))
    for n, (b, i, w) in enumerate(zip(b_idx, i_idx, w_idx)):
        nb = band[b, i:i + 3, w:w + 3, :].reshape(-1)          # (dy, dx, c) order
        out[n] = wflat @ nb
    if bias is not None:
        out += _f64(bias)
    return out


# ------------------------------------------------------------------ a4: displaced attention
def self_attn_displaced(q, k, v, heads: int, scale: float | None = None, rows=None, block: int = 256) -> np.ndarray:
    """Per batch b and head h: O = softmax(scale Q_h K_h^T) V_h over all keys.

    q [B,Nq,heads*D] (the patch's queries); k, v [B,N,heads*D] (the spliced
    full-image buffer: fresh own rows, stale elsewhere); scale defaults to
    1/sqrt(D) (reading R4).  rows: optional (b_idx, q_idx) to evaluate only
    those query tokens (returns [n, heads*D]); else returns [B,Nq,heads*D].
    Queries are independent, so they are evaluated in groups of `block`.
    Module: DistriSelfAttentionPP (DistriFusion architecture article,
    attention section); global context from stale activations: DistriFusion
    reading notes, Introduction fourth paragraph."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Nq, HD = q.shape
    D = HD // heads
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        b_idx = np.repeat(np.arange(B), Nq)
        q_idx = np.tile(np.arange(Nq), B)
    else:
        b_idx, q_idx = (np.asarray(r, dtype=np.int64) for r in rows)
    out = np.empty((len(b_idx), HD))
    for b in np.unique(b_idx):
        sel = np.nonzero(b_idx == b)[0]
        for s0 in range(0, len(sel), block):
            part = sel[s0:s0 + block]
            qb = q[b, q_idx[part]]                                 # [n, HD]
            for h in range(heads):
                cs = slice(h * D, (h + 1) * D)
                s = scale * (qb[:, cs] @ k[b, :, cs].T)            # [n, N]
                s = s - s.max(axis=1, keepdims=True)
                e = np.exp(s)
                out[part, cs] = (e @ v[b, :, cs]) / e.sum(axis=1, keepdims=True)
    if rows is None:
        return out.reshape(B, Nq, HD)
    return out


# ------------------------------------------------------------------ projections
def linear(x, w, bias=None) -> np.ndarray:
    """y[..., n] = sum_k x[..., k] w[n, k] + bias[n] (float64 matmul).

    The to_q / to_k / to_v / to_out projections of the wrapped attention
    module (DistriSelfAttentionPP, DistriFusion architecture article,
    attention section; reading R11).  w is [N, K] (output-major, as the
    module stores it)."""
    y = _f64(x) @ _f64(w).T
    if bias is not None:
        y = y + _f64(bias)
    return y


def projected_attention(x_patch_tokens, k_stale, v_stale, t0: int, wq, bq, wk, bk, wv, bv, wo, bo, heads: int,
                        bf16: bool, rows=None):
    """Displaced self-attention with its projections (reading R11).

    x_patch_tokens [B,Nq,C]: the patch's input tokens (global tokens
    t0 .. t0+Nq-1); k_stale, v_stale [B,N,C]: the previous step's projected
    K and V of the whole image.  q = x Wq^T + bq; the fresh k, v of the patch
    replace tokens t0 .. t0+Nq-1 of the stale K, V (the splice of the patch's
    rows); o = attention(q, K, V); out = o Wo^T + bo.  bf16 storage rounding
    of q, fresh k and v, and o where the configuration is bf16.  Returns dict
    q, k, v (spliced), o, out as stored, plus q_exact, kv_exact fresh values
    and out_exact (each from the stored previous stage)."""
    x = _f64(x_patch_tokens)
    B, Nq, C = x.shape
    q_exact = linear(x, wq, bq)
    k_exact = linear(x, wk, bk)
    v_exact = linear(x, wv, bv)
    q = _store(q_exact, bf16)
    kf = _store(k_exact, bf16)
    vf = _store(v_exact, bf16)
    K = _f64(k_stale).copy()
    V = _f64(v_stale).copy()
    K[:, t0:t0 + Nq] = kf
    V[:, t0:t0 + Nq] = vf
    o_exact = self_attn_displaced(q, K, V, heads)
    o = _store(o_exact, bf16)
    out_exact = linear(o, wo, bo)
    out = _store(out_exact, bf16)
    res = {"q": q, "k": K, "v": V, "o": o, "out": out, "q_exact": q_exact, "k_exact": k_exact,
           "v_exact": v_exact, "o_exact": o_exact, "out_exact": out_exact}
    if rows is not None:
        b_idx, q_idx = (np.asarray(r, dtype=np.int64) for r in rows)
        res["out_rows_exact"] = out_exact[b_idx, q_idx]
    return res


# ------------------------------------------------------------------ a5: CFG combine
def cfg_combine_relmae(eps_c, eps_u, guidance: float):
    """Classifier-free guidance combine and the denoising discrepancy.

    eps = eps_u + w (eps_c - eps_u);  rel = sum|eps_c - eps_u| / sum|eps_u|
    (reading R5; 0/0 gives NaN, x/0 gives inf).  Branches: Hybridiff technical
    summary section 2A; discrepancy: section 2B."""
    c = _f64(eps_c)
    u = _f64(eps_u)
    d = c - u
    eps = u + guidance * d
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.float64(np.abs(d).sum()) / np.float64(np.abs(u).sum())
    return eps, float(rel)


# ------------------------------------------------------------------ next-2: stage switching
def hybrid_schedule(relmae, rho: float = 0.25, eps: float = 0.02, min_warmup: int = 1):
    """Warm-up / parallel / fully-connecting stages from the discrepancy trace.

    Hybridiff technical summary, section 2B: the denoising steps split into a
    warm-up stage (before tau1), a parallelism stage (tau1 up to tau2) and a
    fully-connecting stage (from tau2); tau1 is where the discrepancy's
    decline flattens and tau2 where it starts to rise, both found from the
    live trace.  Reading R13 makes the two points concrete:
      * the decline at step i is d[i-1] - d[i]; the warm-up ends at the first
        step i >= min_warmup whose decline is at most rho times the largest
        decline so far (which must be positive);
      * the parallel stage ends at the first later step whose discrepancy
        exceeds (1 + eps) times the smallest discrepancy of the parallel stage
        so far.
    Comparisons in float32, the precision the trace is kept in; a NaN step
    (0/0 discrepancy) never ends a stage.  Returns (stage int32 [T], tau1,
    tau2) with T for a boundary that never comes."""
    d = np.asarray(relmae, dtype=np.float32)
    T = d.shape[0]
    rho32 = np.float32(rho)
    grow = np.float32(1) + np.float32(eps)
    stage = np.zeros(T, dtype=np.int32)
    tau1 = tau2 = T
    fastest = np.float32(0)
    with np.errstate(invalid="ignore", over="ignore"):
        # warm-up: look for the flattening point
        for i in range(1, T):
            decline = np.float32(d[i - 1] - d[i])
            if decline > fastest:
                fastest = decline
            if i >= min_warmup and fastest > 0 and decline <= rho32 * fastest:
                tau1 = i
                break
        # parallel stage: look for the rise above its running minimum
        if tau1 < T:
            lowest = d[tau1]
            for i in range(tau1 + 1, T):
                if d[i] > grow * lowest:
                    tau2 = i
                    break
                if d[i] < lowest:
                    lowest = d[i]
    stage[tau1:tau2] = 1
    stage[tau2:] = 2
    return stage, int(tau1), int(tau2)


# ------------------------------------------------------------------ chained block
def _store(a, bf16: bool):
    return bf16_round(a) if bf16 else _f64(a)


def previous_step_state(x_stale, gamma, beta, weight, bias, P: int, G: int, eps: float, bf16: bool):
    """The synchronous first step on the stale input (reading R6): every patch
    sees fresh data, so each layer is the plain full-image layer.

    Returns dict: stale_stats [B,P,G,2] raw sums of each patch of x_stale;
    a1 = GN(x_stale) [B,H,W,C] (stored: bf16-rounded when bf16); a2 =
    conv(a1) [B,H,W,C] (stored); a1_exact, a2_exact: the same layer outputs
    before storage rounding (a2_exact is computed from the stored a1)."""
    xs = _f64(x_stale)
    B, H, W, C = xs.shape
    R = H // P
    stats = np.stack([patch_sums(xs[:, q * R:(q + 1) * R], G) for q in range(P)], axis=1)
    a1_exact, _ = groupnorm_stale(xs, None, gamma, beta, H, G, 0, eps)
    a1 = _store(a1_exact, bf16)
    a2_exact = conv3x3_halo(a1, None, weight, bias, 0)
    a2 = _store(a2_exact, bf16)
    return {"stale_stats": stats, "a1": a1, "a2": a2, "a1_exact": a1_exact, "a2_exact": a2_exact}


def displaced_block(x_fresh, state, gamma, beta, weight, bias, P: int, p: int, G: int, heads: int,
                    eps: float, bf16: bool, attn_rows=None):
    """One device's share (patch p) of GN -> conv -> splice -> attention.

    x_fresh [B,H,W,C]: this step's input (the patch's rows are used); state:
    previous_step_state(...) of the stale input.  Identity projections: the
    conv output of the patch is Q; K = V = the previous step's conv output with
    the patch's rows replaced by the fresh conv output (reading R6).
    Returns dict y1 (GN out), y2 (conv out), kv (spliced buffer) as stored,
    y1_exact, y2_exact, kv_exact (the same before storage rounding; each
    stage computed from the previous stage's stored values), o (attention
    out, unrounded; only attn_rows=(b_idx, q_idx) when given), stats (fresh
    sums)."""
    xf = _f64(x_fresh)
    B, H, W, C = xf.shape
    R = H // P
    r0 = p * R
    x_p = xf[:, r0:r0 + R]
    y1_exact, fresh = groupnorm_stale(x_p, state["stale_stats"], gamma, beta, H, G, p, eps)
    y1 = _store(y1_exact, bf16)
    y2_exact = conv3x3_halo(y1, state["a1"], weight, bias, r0)
    y2 = _store(y2_exact, bf16)
    kv = splice(state["a2"], y2, r0)
    kv_exact = splice(state["a2_exact"], y2_exact, r0)
    q = y2.reshape(B, R * W, C)
    kvt = kv.reshape(B, H * W, C)
    o = self_attn_displaced(q, kvt, kvt, heads, rows=attn_rows)
    return {"y1": y1, "y2": y2, "kv": kv, "y1_exact": y1_exact, "y2_exact": y2_exact, "kv_exact": kv_exact,
            "o": o, "stats": fresh}


# ------------------------------------------------------------------ next-4: component steps
def component_block(x, gamma, beta, weight, bias, G: int, heads: int, eps: float, bf16: bool):
    """One full-image component (one patch, P = 1): GroupNorm -> conv ->
    self-attention with identity projections, Q = K = V = the conv output.

    x [B,H,W,C].  Each stored layer output is rounded to bf16 for bf16
    configurations (reading R6); each stage is computed from the previous
    stage's stored values.  Returns y1, y2, o (stored; o as [B,H,W,C]) and
    y1_exact, y2_exact, o_exact."""
    xv = _f64(x)
    B, H, W, C = xv.shape
    y1_exact, _ = groupnorm_stale(xv, None, gamma, beta, H, G, 0, eps)
    y1 = _store(y1_exact, bf16)
    y2_exact = conv3x3_halo(y1, None, weight, bias, 0)
    y2 = _store(y2_exact, bf16)
    t = y2.reshape(B, H * W, C)
    o_exact = self_attn_displaced(t, t, t, heads).reshape(B, H, W, C)
    o = _store(o_exact, bf16)
    return {"y1": y1, "y2": y2, "o": o, "y1_exact": y1_exact, "y2_exact": y2_exact, "o_exact": o_exact}


def async_component_chain(xs, params, G: int, heads: int, eps: float, bf16: bool, warmup: int = 1):
    """Asynchronous denoising over a chain of components (AsyncDiff abstract):
    the noise-prediction model is cut into K components, one
    per device, and from the end of the warm-up on, component k at step t
    takes the output component k-1 produced at step t-1 (consecutive steps'
    hidden states being close), so all components run at once.  During the
    first `warmup` steps the chain runs in order within the step.

    xs: T inputs of component 0; params: K dicts gamma, beta, conv_w, conv_b.
    Returns outs[t][k] = component_block(...) of component k at step t."""
    T, K = len(xs), len(params)
    outs = []
    for t in range(T):
        row = []
        for k in range(K):
            if k == 0:
                src = xs[t]
            elif t < warmup:
                src = row[k - 1]["o"]
            else:
                src = outs[t - 1][k - 1]["o"]
            p = params[k]
            row.append(component_block(src, p["gamma"], p["beta"], p["conv_w"], p["conv_b"], G, heads, eps, bf16))
        outs.append(row)
    return outs


# ------------------------------------------------------------------ next-1: attention block with projections
def previous_block_state(x_stale, gamma, beta, conv_w, conv_b, wk, bk, wv, bv, P: int, G: int, eps: float,
                         bf16: bool):
    """The synchronous first step of the attention block on the stale input
    (every patch fresh, each layer the plain full-image layer; DistriFusion
    reading notes, Introduction fourth paragraph).

    Returns stale_stats [B,P,G,2] (raw sums of each patch of x_stale), a1 =
    GroupNorm + SiLU of the whole stale image (stored), a2 = its conv
    (stored), and the projected k, v [B,N,C] of a2 (stored): the previous
    step's K/V buffer every patch starts from (readings R11, R12); with
    a1_exact, a2_exact, k_exact, v_exact before storage rounding (each from
    the previous stage's stored values)."""
    xs = _f64(x_stale)
    B, H, W, C = xs.shape
    R = H // P
    stats = np.stack([patch_sums(xs[:, q * R:(q + 1) * R], G) for q in range(P)], axis=1)
    a1_exact = groupnorm_silu_stale(xs, None, gamma, beta, H, G, 0, eps)[0]
    a1 = _store(a1_exact, bf16)
    a2_exact = conv3x3_halo(a1, None, conv_w, conv_b, 0)
    a2 = _store(a2_exact, bf16)
    t = a2.reshape(B, H * W, C)
    k_exact, v_exact = linear(t, wk, bk), linear(t, wv, bv)
    return {"stale_stats": stats, "a1": a1, "a2": a2, "k": _store(k_exact, bf16), "v": _store(v_exact, bf16),
            "a1_exact": a1_exact, "a2_exact": a2_exact, "k_exact": k_exact, "v_exact": v_exact}


def displaced_attention_block(x_fresh, state, gamma, beta, conv_w, conv_b, wq, bq, wk, bk, wv, bv, wo, bo, P: int,
                              p: int, G: int, heads: int, eps: float, bf16: bool, attn_rows=None):
    """One device's share (patch p) of the attention block with its
    projections: GroupNorm + SiLU with stale statistics -> 3x3 conv with stale
    halos -> q projection, and the fresh k, v projections replacing the
    patch's tokens in the previous step's projected K/V -> self-attention over
    all tokens -> out projection (DistriGroupNorm, DistriConv2dPP and
    DistriSelfAttentionPP around the whole attention module: DistriFusion
    architecture article; readings R11, R12).

    x_fresh [B,H,W,C] (the patch's rows are used); state from
    previous_block_state.  Each stored stage is rounded to bf16 when bf16;
    each *_exact value is computed from the previous stage's stored values.
    attn_rows=(b_idx, q_idx) evaluates the attention and the out projection
    only at those query tokens (o_rows_exact, out_rows_exact); otherwise o,
    out and their exact values cover all query tokens."""
    xf = _f64(x_fresh)
    B, H, W, C = xf.shape
    R = H // P
    r0 = p * R
    t0 = r0 * W
    y1_exact, fresh = groupnorm_silu_stale(xf[:, r0:r0 + R], state["stale_stats"], gamma, beta, H, G, p, eps)
    y1 = _store(y1_exact, bf16)
    y2_exact = conv3x3_halo(y1, state["a1"], conv_w, conv_b, r0)
    y2 = _store(y2_exact, bf16)
    tok = y2.reshape(B, R * W, C)
    res = {"y1": y1, "y2": y2, "y1_exact": y1_exact, "y2_exact": y2_exact, "stats": fresh}
    if attn_rows is None:
        res.update(projected_attention(tok, state["k"], state["v"], t0, wq, bq, wk, bk, wv, bv, wo, bo, heads, bf16))
        return res
    q_exact = linear(tok, wq, bq)
    k_exact, v_exact = linear(tok, wk, bk), linear(tok, wv, bv)
    q = _store(q_exact, bf16)
    K, V = _f64(state["k"]).copy(), _f64(state["v"]).copy()
    K[:, t0:t0 + R * W] = _store(k_exact, bf16)
    V[:, t0:t0 + R * W] = _store(v_exact, bf16)
    o_rows_exact = self_attn_displaced(q, K, V, heads, rows=attn_rows)
    res.update({"q_exact": q_exact, "k_exact": k_exact, "v_exact": v_exact, "o_rows_exact": o_rows_exact,
                "out_rows_exact": linear(_store(o_rows_exact, bf16), wo, bo)})
    return res
