"""Seeded synthetic inputs for the displaced-patch-parallel layer step.

This module only draws random numbers and stores them in the storage format the
kernels read (bf16 bit patterns or fp32).  It holds none of the method's
arithmetic: no normalisation, convolution, attention, guidance or statistics.
Both the CPU oracle and the GPU path take their inputs from here, so both see
the same bits.

Workload shapes follow the SDXL U-Net levels that the DistriFusion and Hybridiff
pages evaluate at 1024^2 to 3840^2 output resolution (DistriFusion reading
notes, Introduction fifth paragraph; Hybridiff technical summary, section 4
"Results"): one 640-channel level of the latent, 64x64 at 1024 px, 128x128 at
2048 px, 240x240 at 3840 px.  The pages name no distribution for activations;
the recipe below is a reading: fresh activations ~ N(0,1), the previous step's
(stale) activations = fresh + 0.05 N(0,1), because the premise of displaced
patch parallelism is that adjacent denoising steps see similar inputs
(DistriFusion reading notes, Introduction fourth paragraph).

Streams: every tensor has a fixed stream index; stream i of seed s is
numpy.random.default_rng(SeedSequence(entropy=s, spawn_key=(i,))).  Values are
drawn as float32 and rounded to bf16 with round-to-nearest-even when the
configuration is bf16.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# Fixed stream index per named tensor.  Never renumber: stored fixtures and
# recorded results depend on it.
STREAMS = {
    "x": 0,           # fresh activation, full image [B,H,W,C]
    "x_noise": 1,     # stale = fresh + sigma * this
    "gamma": 2,       # GroupNorm scale: 1 + std * N(0,1)
    "beta": 3,        # GroupNorm shift: std * N(0,1)
    "conv_w": 4,      # conv weight [Cout,3,3,Cin], std * N(0,1)
    "conv_b": 5,      # conv bias [Cout], std * N(0,1)
    "q": 6,           # standalone attention queries, full image [B,N,heads*D]
    "k": 7,           # fresh keys
    "v": 8,           # fresh values
    "k_noise": 9,     # stale keys = fresh + sigma * this
    "v_noise": 10,    # stale values = fresh + sigma * this
    "eps_u": 11,      # unconditional noise prediction
    "eps_c_noise": 12,  # conditional = unconditional + sigma_cfg * this
    "w_q": 13,        # projection weights [C,C], N(0,1)/sqrt(C)
    "w_k": 14,
    "w_v": 15,
    "w_o": 16,
    "b_qkvo": 17,     # projection biases [4,C], weight_std * N(0,1)
    "kv_stale": 18,   # the previous step's projected K and V of the image [B,N,2C]
    "relmae_trace": 19,  # per-step discrepancy trace: shape draws and noise
    "x_steps": 20,    # per-step drift of the component chain's input
}


@dataclass(frozen=True)
class Config:
    """One workload: a latent level [B,H,W,C] split into P equal row bands."""

    name: str
    B: int
    H: int
    W: int
    C: int
    P: int
    G: int = 32
    heads: int = 10
    D: int = 64
    dtype: str = "bf16"             # "bf16" or "f32": storage and I/O type
    latent: Optional[Tuple[int, int, int]] = None  # CFG noise latent (h, w, c)
    guidance: float = 7.5
    stale_sigma: float = 0.05
    cfg_sigma: float = 0.05
    weight_std: float = 0.02
    gn_eps: float = 1e-5
    seed: int = 0

    @property
    def rows(self) -> int:
        """Rows per patch (equal bands; H must divide by P)."""
        return self.H // self.P

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def Nq(self) -> int:
        return self.rows * self.W

    def row0(self, p: int) -> int:
        return p * self.rows

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def __post_init__(self):
        if self.H % self.P:
            raise ValueError(f"{self.name}: H={self.H} not divisible by P={self.P}")
        if self.C % self.G:
            raise ValueError(f"{self.name}: C={self.C} not divisible by G={self.G}")
        if self.heads * self.D != self.C:
            raise ValueError(f"{self.name}: heads*D={self.heads * self.D} != C={self.C}")
        if self.dtype not in ("bf16", "f32"):
            raise ValueError(f"{self.name}: dtype {self.dtype}")


# The five workloads.  Sizes: tiny fp32 (16x16x64, 2 bands of 8 rows, 1 head);
# the 1024 px level (64x64x640, 4 bands of 16 rows); the 2048 px level
# (128x128x640, 8 bands of 16 rows); the 3840 px level (240x240x640, 8 bands of
# 30 rows); a cond/uncond pair at the 1024 px level with the 128x128x4 noise
# latent for classifier-free guidance.
CONFIGS = {
    "tiny_f32": Config("tiny_f32", B=1, H=16, W=16, C=64, P=2, G=32, heads=1, D=64, dtype="f32"),
    "sdxl_1024": Config("sdxl_1024", B=1, H=64, W=64, C=640, P=4),
    "sdxl_2048": Config("sdxl_2048", B=1, H=128, W=128, C=640, P=8),
    "sdxl_3840": Config("sdxl_3840", B=1, H=240, W=240, C=640, P=8, latent=(480, 480, 4)),
    "cfg_pair_1024": Config("cfg_pair_1024", B=2, H=64, W=64, C=640, P=4, latent=(128, 128, 4)),
}
ORDER = ["tiny_f32", "sdxl_1024", "sdxl_2048", "sdxl_3840", "cfg_pair_1024"]


def stream(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(STREAMS[name],)))


def normal(seed: int, name: str, shape) -> np.ndarray:
    return stream(seed, name).standard_normal(size=shape, dtype=np.float32)


# ---------------------------------------------------------------- storage format
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Storage conversion for generated inputs only (finite values)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite synthetic value")
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact float32 values they encode."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(cfg: Config, a: np.ndarray) -> np.ndarray:
    """Activation/weight tensor in the configuration's storage format:
    uint16 bf16 bits for bf16 configurations, float32 otherwise."""
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def values(cfg_or_dtype, a: np.ndarray) -> np.ndarray:
    """Exact float32 values of a stored tensor (bf16 bits widened, fp32 as is)."""
    dtype = cfg_or_dtype if isinstance(cfg_or_dtype, str) else cfg_or_dtype.dtype
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------- generators
def layer_inputs(cfg: Config) -> dict:
    """Inputs of the GroupNorm -> conv -> attention block.

    x_fresh, x_stale: [B,H,W,C] storage format (stale = fresh + sigma N(0,1)).
    gamma, beta: [C] float32 (GroupNorm affine; always fp32).
    conv_w: [C,3,3,C] storage format (output channel, kernel row, kernel col,
            input channel).  conv_b: [C] float32.
    """
    s, B, H, W, C = cfg.seed, cfg.B, cfg.H, cfg.W, cfg.C
    x = normal(s, "x", (B, H, W, C))
    xs = x + np.float32(cfg.stale_sigma) * normal(s, "x_noise", (B, H, W, C))
    gamma = (1.0 + cfg.weight_std * normal(s, "gamma", (C,))).astype(np.float32)
    beta = (cfg.weight_std * normal(s, "beta", (C,))).astype(np.float32)
    w = cfg.weight_std * normal(s, "conv_w", (C, 3, 3, C))
    b = (cfg.weight_std * normal(s, "conv_b", (C,))).astype(np.float32)
    return {
        "x_fresh": store(cfg, x),
        "x_stale": store(cfg, xs),
        "gamma": gamma,
        "beta": beta,
        "conv_w": store(cfg, w),
        "conv_b": b,
    }


def attention_inputs(cfg: Config) -> dict:
    """Standalone displaced-attention inputs, all tokens of the image.

    q: [B,N,heads*D] fresh queries; k, v fresh; k_stale, v_stale = fresh +
    sigma N(0,1).  Storage format."""
    s, B, N, C = cfg.seed, cfg.B, cfg.N, cfg.C
    q = normal(s, "q", (B, N, C))
    k = normal(s, "k", (B, N, C))
    v = normal(s, "v", (B, N, C))
    ks = k + np.float32(cfg.stale_sigma) * normal(s, "k_noise", (B, N, C))
    vs = v + np.float32(cfg.stale_sigma) * normal(s, "v_noise", (B, N, C))
    return {"q": store(cfg, q), "k": store(cfg, k), "v": store(cfg, v),
            "k_stale": store(cfg, ks), "v_stale": store(cfg, vs)}


def projection_inputs(cfg: Config) -> dict:
    """Weights of the attention module's projections and the previous step's
    projected K/V buffer.

    w_q, w_k, w_v, w_o: [C,C] storage format (output-major), N(0,1)/sqrt(C)
    (unit-variance outputs for unit-variance inputs); b_q, b_k, b_v, b_o: [C]
    float32, weight_std N(0,1); kv_stale: [B,N,2C] storage format, K in
    channels [0,C), V in [C,2C), N(0,1)."""
    s, B, N, C = cfg.seed, cfg.B, cfg.N, cfg.C
    sc = np.float32(1.0 / np.sqrt(C))
    out = {f"w_{n}": store(cfg, sc * normal(s, f"w_{n}", (C, C))) for n in "qkvo"}
    b = (cfg.weight_std * normal(s, "b_qkvo", (4, C))).astype(np.float32)
    for i, n in enumerate("qkvo"):
        out[f"b_{n}"] = np.ascontiguousarray(b[i])
    out["kv_stale"] = store(cfg, normal(s, "kv_stale", (B, N, 2 * C)))
    return out


def cfg_inputs(cfg: Config, latent: Optional[Tuple[int, int, int]] = None, n: Optional[int] = None) -> dict:
    """Noise predictions of the two classifier-free-guidance branches.

    eps_u ~ N(0,1); eps_c = eps_u + cfg_sigma N(0,1) (branches close, as in the
    parallel stage of condition-split scheduling).  Flat length n, or the
    configuration's latent (h*w*c) when n is None.  Storage format."""
    if n is None:
        lat = latent or cfg.latent
        if lat is None:
            raise ValueError(f"{cfg.name} has no CFG latent")
        n = int(np.prod(lat))
    u = normal(cfg.seed, "eps_u", (n,))
    c = u + np.float32(cfg.cfg_sigma) * normal(cfg.seed, "eps_c_noise", (n,))
    return {"eps_u": store(cfg, u), "eps_c": store(cfg, c)}


def component_chain_inputs(cfg: Config, K: int, T: int) -> dict:
    """Inputs of a chain of K full-image components over T denoising steps.

    xs: T inputs [B,H,W,C] of the first component, x_t = x + stale_sigma * t *
    N(0,1) (consecutive steps close, as the component scheme assumes); params:
    per component the GroupNorm affine and conv weights of layer_inputs with
    seed cfg.seed + k + 1.  Storage format."""
    B, H, W, C = cfg.B, cfg.H, cfg.W, cfg.C
    x = normal(cfg.seed, "x", (B, H, W, C))
    d = normal(cfg.seed, "x_steps", (B, H, W, C))
    xs = [store(cfg, x + np.float32(cfg.stale_sigma * t) * d) for t in range(T)]
    params = []
    for k in range(K):
        li = layer_inputs(cfg.replace(seed=cfg.seed + k + 1))
        params.append({n: li[n] for n in ("gamma", "beta", "conv_w", "conv_b")})
    return {"xs": xs, "params": params}


def relmae_trace(seed: int, T: int, noise: float = 0.0) -> np.ndarray:
    """Synthetic per-step discrepancy trace [T] float32 in denoising order.

    The shape the condition-split scheduling pages describe: large at the
    start, falling fast, flattening in the middle and rising towards the end.
    d(t) = base + amp exp(-t / decay) + rise max(0, t - t_rise)^2 / T^2, with
    decay, t_rise and the three scales drawn per seed, times (1 + noise N(0,1)).
    """
    g = stream(seed, "relmae_trace")
    base = g.uniform(0.05, 0.2)
    amp = g.uniform(0.5, 2.0)
    decay = g.uniform(0.04, 0.15) * T
    t_rise = g.uniform(0.55, 0.8) * T
    rise = g.uniform(0.5, 3.0)
    t = np.arange(T, dtype=np.float64)
    d = base + amp * np.exp(-t / decay) + rise * np.maximum(0.0, t - t_rise) ** 2 / float(T) ** 2
    if noise:
        d = d * (1.0 + noise * g.standard_normal(T))
    return d.astype(np.float32)


def rows_of(a: np.ndarray, row0: int, rows: int) -> np.ndarray:
    """Row band [row0, row0+rows) of a [B,H,W,C] tensor, contiguous copy."""
    return np.ascontiguousarray(a[:, row0:row0 + rows])


def tokens(a: np.ndarray) -> np.ndarray:
    """[B,H,W,C] -> [B,H*W,C] view (token t = row*W + col)."""
    B, H, W, C = a.shape
    return a.reshape(B, H * W, C)
