"""Benchmark: one displaced-patch-parallel layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:
for every patch p of the workload (P row bands, each the share of one device),
GroupNorm with stale statistics -> 3x3 conv with stale halos -> splice into
the patch's private K/V buffer -> displaced self-attention; then the
classifier-free-guidance combine with the rel-MAE reduction on the noise
latent of that resolution.  All inputs are resident in HBM before timing; the
previous step's state comes from an untimed synchronous step.

value = (conv + attention algorithmic flops of the step) / step time, in
TFLOP/s.  The JSON line also carries the roofline of the dominant kernel
(attention), measured with HIP events recorded on the launch stream around
each attention call inside the timed region, and the CPU oracle's throughput
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Counter-based HBM traffic of one attention call, recorded from rocprofv3
# FETCH_SIZE / WRITE_SIZE passes scaled by a plain-copy calibration.  It is
# reported only while the attention sources still hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_sdxl_3840_traffic.md")
ATTN_SOURCES = ("displaced_patch_parallelism_net_amd/csrc/k_attn.hip",
                "displaced_patch_parallelism_net_amd/csrc/dpp_common.h")
CONV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv_sdxl_3840_traffic.md")
CONV_SOURCES = ("displaced_patch_parallelism_net_amd/csrc/k_conv.hip",
                "displaced_patch_parallelism_net_amd/csrc/dpp_common.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sdxl_3840")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--kernels", action="store_true", help="also time every kernel family separately")
    ap.add_argument("--hbm-sweep", action="store_true",
                    help="also time splice / GroupNorm / CFG over a size sweep, warm and cold last-level cache")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (the splice kernel) 3 times: the known-size "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def source_hash(sources):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def attn_source_hash():
    return source_hash(ATTN_SOURCES)


def conv_source_hash():
    return source_hash(CONV_SOURCES)


def measured_traffic(workload, path=TRAFFIC_FILE, sources=ATTN_SOURCES):
    """HBM bytes per call from a recorded counter summary (the attention's
    by default), or None when there is none for this workload or the
    kernel's sources changed since."""
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != source_hash(sources):
        return None
    return rec.get("traffic_bytes_per_call")


def calib_copy(mib=512, reps=3):
    """A plain copy of known size: one contiguous bf16 slab of `mib` MiB
    spliced into a buffer twice its size, `reps` times."""
    import torch
    import displaced_patch_parallelism_net_amd as dpp
    W, C = 1024, 1024
    R = mib * 2 ** 20 // (W * C * 2)
    full = torch.zeros(1, 2 * R, W, C, dtype=torch.bfloat16, device="cuda")
    patch = torch.ones(1, R, W, C, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        dpp.dpp_splice_patch(full, patch, R)
    torch.cuda.synchronize()
    nbytes = patch.numel() * 2
    print(json.dumps({"calib_copy": "splice_vec_kernel", "bytes_read_per_call": nbytes,
                      "bytes_written_per_call": nbytes, "calls": reps}), flush=True)


def flops(cfg):
    conv = 2.0 * cfg.B * cfg.Nq * cfg.C * 9 * cfg.C
    attn = 4.0 * cfg.B * cfg.heads * cfg.Nq * cfg.N * cfg.D
    return conv, attn


def latent_of(cfg):
    # SD-family VAE: the noise latent is 1/8 of the output resolution, 4 channels.
    if cfg.latent is not None:
        return cfg.latent
    return (2 * cfg.H, 2 * cfg.W, 4)


def cpu_baseline(cfg, budget_s):
    """The oracle (as is) on a bounded sample of the same workload: attention
    for a block of query rows of patch 0 against all keys, and the conv for a
    set of output pixels; throughput in the metric's unit (TFLOP/s)."""
    import oracle
    from dpp_synth import attention_inputs, layer_inputs, rows_of, tokens, values
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = layer_inputs(cfg)
    r0 = 0
    xv = values(cfg, rows_of(inp["x_fresh"], r0, cfg.rows))
    sv = values(cfg, inp["x_stale"])
    wv = values(cfg, inp["conv_w"])
    # calibration run to size the sample to the budget
    rng = np.random.default_rng(0)
    att = attention_inputs(cfg)
    q = values(cfg, att["q"])[:, :cfg.Nq]
    k = values(cfg, att["k_stale"])
    v = values(cfg, att["v_stale"])
    del att
    done_flops = 0.0
    t_total = 0.0
    nq = 16
    npx = 16
    samples = []
    while t_total < budget_s:
        qi = rng.integers(0, cfg.Nq, nq)
        t0 = time.perf_counter()
        oracle.self_attn_displaced(q, k, v, cfg.heads, rows=(np.zeros(nq, dtype=np.int64), qi))
        ii, wi = rng.integers(0, cfg.rows, npx), rng.integers(0, cfg.W, npx)
        oracle.conv3x3_halo_sampled(xv, sv, wv, inp["conv_b"], r0, np.zeros(npx, dtype=np.int64), ii, wi)
        dt = time.perf_counter() - t0
        f = 4.0 * cfg.heads * nq * cfg.N * cfg.D + 2.0 * npx * cfg.C * 9 * cfg.C
        t_total += dt
        done_flops += f
        samples.append((nq, npx))
        if dt < budget_s / 8:
            nq *= 2
            npx *= 2
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    return {
        "value": done_flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: displaced attention of {sum(s[0] for s in samples)} query rows x "
                   f"{cfg.N} keys x {cfg.heads} heads and the halo conv of {sum(s[1] for s in samples)} output "
                   f"pixels x {cfg.C} channels of patch 0 of {cfg.name}; {t_total:.1f} s"),
    }


def release_device_memory():
    """Free every cached device block while the HIP runtime (and a profiler
    attached to it) is still fully up.  Left to the interpreter's exit, the
    caching allocator returns its blocks from static destructors that can run
    after a profiler tool has finalised and torn down its hooks: a host
    SIGSEGV during exit, after the results were written."""
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the step; --gpus must be 1 "
                                   "(the multi-GPU exchange is not implemented)"}))
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
    else:
        out = run(args)
        print(json.dumps(out), flush=True)
    release_device_memory()


def run(args):
    import torch
    import displaced_patch_parallelism_net_amd as dpp
    from displaced_patch_parallelism_net_amd.step import DisplacedLayer
    from dpp_synth import CONFIGS, cfg_inputs, layer_inputs

    cfg = CONFIGS[args.workload]
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = "cuda"

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    inp = layer_inputs(cfg)
    lat = latent_of(cfg)
    cin = cfg_inputs(cfg, latent=lat)
    layer = DisplacedLayer(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, cfg.G, cfg.heads, dt, eps=cfg.gn_eps, head_dim=cfg.D)
    gamma = torch.from_numpy(inp["gamma"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    w = to_dev(inp["conv_w"])
    b = torch.from_numpy(inp["conv_b"]).to(dev)
    x_fresh = to_dev(inp["x_fresh"])
    x_patches = [layer.band(x_fresh, p) for p in range(cfg.P)]
    layer.synchronous_step(to_dev(inp["x_stale"]), gamma, beta, w, b)
    eps_c, eps_u = to_dev(cin["eps_c"]), to_dev(cin["eps_u"])
    eps = torch.empty_like(eps_c)
    rel = torch.zeros(1, dtype=torch.float32, device=dev)
    n_lat = eps_c.numel()
    cfg_ws = torch.empty(dpp.dpp_cfg_combine_workspace_bytes(n_lat), dtype=torch.uint8, device=dev)
    del inp, cin
    torch.cuda.synchronize()

    # Timed steps carry one event pair per patch, around the attention call.
    # Events are created without the system-scope fence (FenceFreeEvent):
    # recording one of torch's events leaves the GPU idle for about 6 us
    # before the next kernel.  Even so each record costs a little, so a pair
    # around every kernel would still slow the very steps it times (+0.5 % at
    # 3840 px, +6 % at 2048 px; the attention pair alone: +0.1 % / +1 %,
    # same-box A/B).  A patch-layer step is timed from one attention's end to
    # the next's; the conv's per-call time comes from back-to-back calls after
    # the timed steps.
    attn_events = []

    def step(record=False):
        for p in range(cfg.P):
            r0 = p * layer.R
            dpp.dpp_groupnorm_stale(layer.y1, layer.stats_next, x_patches[p], layer.stats_prev, gamma, beta, cfg.H,
                                    cfg.G, cfg.P, p, cfg.gn_eps, layer.gn_ws)
            dpp.dpp_conv3x3_halo(layer.y2, layer.y1, layer.a1, w, b, cfg.H, r0, workspace=layer.conv_ws)
            dpp.dpp_splice_patch(layer.kv[p], layer.y2, r0)
            kv = layer.kv[p].view(cfg.B, cfg.N, cfg.C)
            if record:
                e0, e1 = FenceFreeEvent(), FenceFreeEvent()
                e0.record()
            dpp.dpp_self_attn_displaced(layer.o, layer.y2.view(cfg.B, cfg.Nq, cfg.C), kv, kv, cfg.heads, cfg.D, 0.0,
                                        layer.attn_ws)
            if record:
                e1.record()
                attn_events.append((e0, e1))
        dpp.dpp_cfg_combine_relmae(eps, rel, eps_c, eps_u, cfg.guidance, cfg_ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b_) for a, b_ in attn_events]))
    # one patch's GN -> conv -> splice -> attention, by events on the launch
    # stream: from the end of patch p-1's attention to the end of patch p's,
    # for p = 1 .. P-1 of every timed step (patch 0's interval would also hold
    # the previous step's CFG combine)
    patch_ms = np.array([attn_events[s * cfg.P + p - 1][1].elapsed_time(attn_events[s * cfg.P + p][1])
                         for s in range(args.steps) for p in range(1, cfg.P)])

    f_conv, f_attn = flops(cfg)
    step_flops = cfg.P * (f_conv + f_attn)
    value = step_flops / (wall / args.steps) / 1e12
    # The same attention calls back to back between one event pair (the
    # step's last inputs): free of the host's launch gaps that the per-call
    # events inside the step include at small sizes, but run under the
    # sustained load of attention alone, which lowers the clock.
    attn_b2b_ms = time_back_to_back(
        [lambda p=p: dpp.dpp_self_attn_displaced(layer.o, layer.y2.view(cfg.B, cfg.Nq, cfg.C),
                                                  layer.kv[p].view(cfg.B, cfg.N, cfg.C),
                                                  layer.kv[p].view(cfg.B, cfg.N, cfg.C), cfg.heads, cfg.D, 0.0,
                                                  layer.attn_ws) for p in range(cfg.P)], torch)
    attn_tflops = f_attn / (attn_ms * 1e-3) / 1e12
    # the conv's calls back to back, between one event pair (the attention's
    # back-to-back figure above is taken the same way)
    conv_b2b_ms = time_back_to_back(
        [lambda p=p: dpp.dpp_conv3x3_halo(layer.y2, layer.y1, layer.a1, w, b, cfg.H, p * layer.R,
                                           workspace=layer.conv_ws) for p in range(cfg.P)], torch)
    conv_tflops = f_conv / (conv_b2b_ms * 1e-3) / 1e12

    graph = time_graph_step(step, step_flops, torch, args.steps)

    block = time_attention_block(cfg, dpp, torch) if cfg.dtype == "bf16" else None

    kernels = None
    if args.kernels:
        kernels = time_kernels(cfg, layer, x_patches, gamma, beta, w, b, eps, rel, eps_c, eps_u, cfg_ws, dpp, torch)
        if cfg.dtype == "bf16":
            kernels.update(time_projections(cfg, layer, x_patches, gamma, beta, dpp, torch))
            kernels.update(time_component(dpp, torch))
            kernels.update(time_conv_bands(dpp, torch))

    out = {
        "metric": "displaced-attn + halo-conv TFLOP/s (% bf16 MFMA peak); ms per patch-layer step",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, stale = fresh + 0.05 N(0,1), weights 0.02 N(0,1))",
        "config": {
            "workload": (f"{cfg.name}: {cfg.H}x{cfg.W}x{cfg.C} level, {cfg.P} patches x {cfg.rows} rows, "
                         f"GN {cfg.G}, conv3x3 {cfg.C}->{cfg.C}, {cfg.heads}x{cfg.D} attention over {cfg.N} tokens, "
                         f"CFG on {lat[0]}x{lat[1]}x{lat[2]} latent"),
            "batch": cfg.B,
            "patches": cfg.P,
            "tokens": cfg.N,
            "query_tokens_per_patch": cfg.Nq,
        },
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_patch_layer_step": round(ms_step / cfg.P, 4),
        "patch_layer_step_ms": {"median": round(float(np.median(patch_ms)), 4),
                                "p10": round(float(np.percentile(patch_ms, 10)), 4),
                                "p90": round(float(np.percentile(patch_ms, 90)), 4),
                                "sum_over_patches": round(float(np.median(patch_ms)) * cfg.P, 4),
                                "samples": int(patch_ms.size)},
        "roofline": {
            "kernel": "dpp_self_attn_displaced",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(cfg.name),
            "traffic_unit": "bytes per call (attention + split merge), FETCH_SIZE + WRITE_SIZE scaled by a plain copy",
            "avg_launch_ms": round(attn_ms, 5),
            "avg_launch_ms_back_to_back": round(attn_b2b_ms, 5),
            "timing": "HIP events (created without the system-scope fence) on the launch stream around each "
                      "attention call inside the timed steps (avg_launch_ms); around every patch's call launched "
                      "back to back after the timed steps (avg_launch_ms_back_to_back)",
            "flops_per_launch": f_attn,
        },
    }
    out["roofline_conv"] = {
        "kernel": "dpp_conv3x3_halo", "bound": "mfma", "achieved": round(conv_tflops, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(conv_tflops / PEAK_BF16_TFLOPS, 4),
        "avg_launch_ms_back_to_back": round(conv_b2b_ms, 5), "flops_per_launch": f_conv,
        "traffic": measured_traffic(cfg.name, CONV_TRAFFIC_FILE, CONV_SOURCES),
        "traffic_unit": "bytes per call, FETCH_SIZE + WRITE_SIZE scaled by a plain copy",
        "timing": "HIP events (created without the system-scope fence) around every patch's conv call launched "
                  "back to back after the timed steps (no per-call conv events inside the timed steps: their "
                  "records would slow them)"}
    out["graph_replay"] = graph
    if block:
        out["attention_block_step"] = block
    if kernels:
        out["kernels"] = kernels
    if args.hbm_sweep:
        out["hbm_sweep"] = hbm_sweep(cfg, dpp, torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget_s)
    return out


def time_graph_step(step, step_flops, torch, steps):
    """The same step (every patch + CFG) captured once into a HIP graph and
    replayed `steps` times, wall clock with a synchronisation on both sides:
    one host launch per step instead of four binding calls per patch."""
    from displaced_patch_parallelism_net_amd.step import capture_graph
    g = capture_graph(step)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return {"ms_per_step": round(ms, 4), "TFLOP/s": round(step_flops / (ms * 1e-3) / 1e12, 3),
            "steps": steps, "how": "the timed step captured once into a HIP graph, replayed back to back"}


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence, recorded on
    torch's current stream.  Recording one of torch's events ends with a
    system-scope release (cache write-back and invalidate) that leaves the GPU
    idle for about 6 us before the next kernel; this event only takes its
    timestamp.  Uses the HIP runtime the process has already loaded (torch's),
    so the library's launches and these events share one runtime."""
    _hip = None
    _FLAGS = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            with open("/proc/self/maps") as fh:
                paths = sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln and ln.split()[-1].startswith("/")})
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            hip = ctypes.CDLL(paths[0])
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
                getattr(hip, f).restype = ctypes.c_int
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self._FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self):
        import torch
        rc = self._lib().hipEventRecord(self._ev, ctypes_stream(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end):
        """ms from this event to `end`; both must have completed (synchronise first)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "_ev", None) is not None and self._ev.value:
            self._hip.hipEventDestroy(self._ev)


def ctypes_stream(handle):
    import ctypes
    return ctypes.c_void_p(handle)


def host_ahead(torch, n_calls):
    """Hold the stream with a bounded spin kernel (about 100 us of shader
    clock per call that follows, well above the host's cost of one binding
    call) so the host has queued the next `n_calls` calls and their events
    before the GPU reaches them: per-call events then time the kernels, not
    the gaps while the host launches the next one.  (Skipped where torch has
    no such helper: the per-call figures then include launch gaps.)"""
    spin = getattr(torch.cuda, "_sleep", None)  # torch's bounded device spin (a testing helper)
    if spin is not None:
        spin(int(min(n_calls, 4000) * 250000))


def time_back_to_back(calls, torch, min_calls=50):
    """Mean ms per call of `calls` launched round-robin, back to back, for at
    least `min_calls` calls between one pair of events on the current stream
    (after one untimed round, behind a spin that lets the host queue them
    all first)."""
    rounds = -(-min_calls // len(calls))
    for fn in calls:
        fn()
    host_ahead(torch, rounds * len(calls))
    e0, e1 = FenceFreeEvent(), FenceFreeEvent()
    e0.record()
    for _ in range(rounds):
        for fn in calls:
            fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (rounds * len(calls))


def time_attention_block(cfg, dpp, torch, reps=3):
    """The attention block with its projections (GroupNorm + SiLU -> conv ->
    q and fused K/V projections into the private buffer -> attention -> out
    projection) of every patch, after an untimed synchronous step; HIP events
    on the launch stream around each patch step.  Seeded weights
    (layer_inputs, projection_inputs)."""
    from dpp_synth import layer_inputs, projection_inputs
    from displaced_patch_parallelism_net_amd.step import DisplacedBlock

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    li, pi = layer_inputs(cfg), projection_inputs(cfg)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    gamma, beta, cw, cb = f32(li["gamma"]), f32(li["beta"]), bf(li["conv_w"]), f32(li["conv_b"])
    wq, bq, wo, bo = bf(pi["w_q"]), f32(pi["b_q"]), bf(pi["w_o"]), f32(pi["b_o"])
    wkv = bf(np.concatenate([pi["w_k"], pi["w_v"]], axis=0))
    bkv = f32(np.concatenate([pi["b_k"], pi["b_v"]]))
    blk = DisplacedBlock(cfg.B, cfg.H, cfg.W, cfg.C, cfg.P, cfg.G, cfg.heads, eps=cfg.gn_eps, head_dim=cfg.D)
    blk.synchronous_step(bf(li["x_stale"]), gamma, beta, cw, cb, wkv, bkv)
    xf = bf(li["x_fresh"])
    xp = [blk.band(xf, p) for p in range(cfg.P)]
    del li, pi
    for p in range(cfg.P):
        blk.patch_step(p, xp[p], gamma, beta, cw, cb, wq, bq, wkv, bkv, wo, bo)
    torch.cuda.synchronize()
    ev = []
    host_ahead(torch, 8 * reps * cfg.P)
    for _ in range(reps):
        for p in range(cfg.P):
            e0, e1 = FenceFreeEvent(), FenceFreeEvent()
            e0.record()
            blk.patch_step(p, xp[p], gamma, beta, cw, cb, wq, bq, wkv, bkv, wo, bo)
            e1.record()
            ev.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b_) for a, b_ in ev])
    f_conv, f_attn = flops(cfg)
    f_proj = 2.0 * cfg.B * cfg.Nq * cfg.C * cfg.C * 4   # q, k, v, out
    ms = float(np.median(t))
    return {"median_ms": round(ms, 4), "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4), "samples": int(t.size),
            "TFLOP/s": round((f_conv + f_attn + f_proj) / (ms * 1e-3) / 1e12, 2),
            "flops": f_conv + f_attn + f_proj,
            "steps": "GroupNorm+SiLU -> conv -> q and fused K/V projections into the private buffer -> "
                     "attention -> out projection, per patch"}


def time_rounds(families, torch, reps=10, min_calls=16):
    """Per-call time of each call family: `reps` rounds of at least
    `min_calls` calls of the family (its calls round-robin) back to back
    between one pair of HIP events on the launch stream, behind a spin that
    lets the host queue them first.  Returns {name: per-call ms of every
    round}.  (A single call between its own event pair would also time the
    cost of recording the events.)"""
    out = {}
    for name, calls in families.items():
        n = max(min_calls, len(calls))
        for fn in calls:
            fn()
        host_ahead(torch, reps * n)
        pairs = []
        for _ in range(reps):
            e0, e1 = FenceFreeEvent(), FenceFreeEvent()
            e0.record()
            for i in range(n):
                calls[i % len(calls)]()
            e1.record()
            pairs.append((e0, e1, n))
        out[name] = pairs
    torch.cuda.synchronize()
    return {name: np.array([a.elapsed_time(b_) / n for a, b_, n in pairs]) for name, pairs in out.items()}


def time_kernels(cfg, layer, x_patches, gamma, beta, w, b, eps, rel, eps_c, eps_u, cfg_ws, dpp, torch, reps=10):
    """Per-call duration of each call family over all patches (back-to-back
    rounds, time_rounds), with its algorithmic work."""
    P = cfg.P
    fam = {
        "groupnorm": [lambda p=p: dpp.dpp_groupnorm_stale(layer.y1, layer.stats_next, x_patches[p], layer.stats_prev,
                                                          gamma, beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps, layer.gn_ws)
                      for p in range(P)],
        "conv": [lambda p=p: dpp.dpp_conv3x3_halo(layer.y2, layer.y1, layer.a1, w, b, cfg.H, p * layer.R,
                                                  workspace=layer.conv_ws) for p in range(P)],
        "splice": [lambda p=p: dpp.dpp_splice_patch(layer.kv[p], layer.y2, p * layer.R) for p in range(P)],
        "attention": [lambda p=p: dpp.dpp_self_attn_displaced(layer.o, layer.y2.view(cfg.B, cfg.Nq, cfg.C),
                                                              layer.kv[p].view(cfg.B, cfg.N, cfg.C),
                                                              layer.kv[p].view(cfg.B, cfg.N, cfg.C), cfg.heads, cfg.D,
                                                              0.0, layer.attn_ws) for p in range(P)],
        "cfg": [lambda: dpp.dpp_cfg_combine_relmae(eps, rel, eps_c, eps_u, cfg.guidance, cfg_ws)],
    }
    if cfg.dtype == "bf16":
        # a GroupNorm whose input the conv wrote: the conv also emits the
        # group partial sums, and the GroupNorm reads its input once
        nchunk = dpp.dpp_conv3x3_halo_gn_chunks(cfg.rows, cfg.W, cfg.C)
        part = torch.empty(cfg.B, nchunk, cfg.G, 2, dtype=torch.float32, device="cuda")
        h = torch.empty_like(layer.y2)
        fam["conv_with_gn_partials"] = [lambda p=p: dpp.dpp_conv3x3_halo_gn(h, part, layer.y1, layer.a1, w, b, cfg.H,
                                                                            p * layer.R) for p in range(P)]
        fam["groupnorm_presummed"] = [lambda p=p: dpp.dpp_groupnorm_stale_presummed(
            layer.y1, layer.stats_next, h, part, layer.stats_prev, gamma, beta, cfg.H, cfg.G, cfg.P, p, cfg.gn_eps)
            for p in range(P)]
    times = time_rounds(fam, torch, reps)
    es = 2 if cfg.dtype == "bf16" else 4
    f_conv, f_attn = flops(cfg)
    act = cfg.B * cfg.Nq * cfg.C * es
    work = {
        "groupnorm": (2.0 * act + 2 * 4 * cfg.B * cfg.G * (cfg.P + 1), "GB/s", PEAK_HBM_GBS),
        "conv": (f_conv, "TFLOP/s", PEAK_BF16_TFLOPS),
        "splice": (2.0 * act, "GB/s", PEAK_HBM_GBS),
        "attention": (f_attn, "TFLOP/s", PEAK_BF16_TFLOPS),
        "cfg": (3.0 * eps_c.numel() * es, "GB/s", PEAK_HBM_GBS),
        "conv_with_gn_partials": (f_conv, "TFLOP/s", PEAK_BF16_TFLOPS),
        "groupnorm_presummed": (2.0 * act + 2 * 4 * cfg.B * cfg.G * (cfg.P + 1), "GB/s", PEAK_HBM_GBS),
    }
    res = {}
    for k, t in times.items():
        ms = float(np.mean(t))
        amount, unit, peak = work[k]
        rate = amount / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        res[k] = {"avg_ms": round(ms, 5), "median_ms": round(float(np.median(t)), 5),
                  "p10_ms": round(float(np.percentile(t, 10)), 5), "p90_ms": round(float(np.percentile(t, 90)), 5),
                  "rounds": int(t.size), unit: round(rate, 2), "frac_peak": round(rate / peak, 4), "work": amount}
    return res


def time_projections(cfg, layer, x_patches, gamma, beta, dpp, torch, reps=10):
    """The projection calls of the attention module and GroupNorm + SiLU at
    the workload's patch size (not part of the headline step): q = x Wq^T +
    bq, the fresh K/V projection written into the patch's rows of a [B,N,2C]
    K/V buffer, out = o Wo^T + bo.  Seeded weights (projection_inputs).
    For scale, the same two products through PyTorch's own GEMM
    (torch.nn.functional.linear, hipBLASLt; bf16 bias, fresh contiguous
    output): a library reference, not part of this path.  Back-to-back
    rounds (time_rounds)."""
    from dpp_synth import projection_inputs
    pi = projection_inputs(cfg)
    dev = "cuda"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    C, M, P = cfg.C, cfg.Nq, cfg.P
    wq, wo = bf(pi["w_q"]), bf(pi["w_o"])
    wkv = bf(np.concatenate([pi["w_k"], pi["w_v"]], axis=0))
    bq, bo = torch.from_numpy(pi["b_q"]).to(dev), torch.from_numpy(pi["b_o"]).to(dev)
    bkv = torch.from_numpy(np.concatenate([pi["b_k"], pi["b_v"]])).to(dev)
    kv2 = bf(pi["kv_stale"])
    xq = layer.y2.view(cfg.B, M, C)
    q = torch.empty(cfg.B, M, C, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    o = layer.o.view(cfg.B, M, C)
    bq16, bkv16 = bq.to(torch.bfloat16), bkv.to(torch.bfloat16)
    xq2 = xq.reshape(cfg.B * M, C)   # 2-D: a plain GEMM, no batched product
    fam = {
        "groupnorm_silu": [lambda p=p: dpp.dpp_groupnorm_silu_stale(layer.y1, layer.stats_next, x_patches[p],
                                                                    layer.stats_prev, gamma, beta, cfg.H, cfg.G,
                                                                    cfg.P, p, cfg.gn_eps, layer.gn_ws)
                           for p in range(P)],
        "linear_q": [lambda: dpp.dpp_linear(q, xq, wq, bq)],
        "linear_kv_into_buffer": [lambda p=p: dpp.dpp_linear(kv2[:, p * M:(p + 1) * M, :], xq, wkv, bkv)
                                  for p in range(P)],
        "linear_out": [lambda: dpp.dpp_linear(out, o, wo, bo)],
        "library_reference_linear_q": [lambda: torch.nn.functional.linear(xq2, wq, bq16)],
        "library_reference_linear_kv": [lambda: torch.nn.functional.linear(xq2, wkv, bkv16)],
    }
    times = time_rounds(fam, torch, reps)
    act = cfg.B * M * C * 2
    work = {
        "linear_q": (2.0 * cfg.B * M * C * C, "TFLOP/s", PEAK_BF16_TFLOPS),
        "linear_kv_into_buffer": (2.0 * cfg.B * M * C * 2 * C, "TFLOP/s", PEAK_BF16_TFLOPS),
        "linear_out": (2.0 * cfg.B * M * C * C, "TFLOP/s", PEAK_BF16_TFLOPS),
        "groupnorm_silu": (2.0 * act + 2 * 4 * cfg.B * cfg.G * (cfg.P + 1), "GB/s", PEAK_HBM_GBS),
        "library_reference_linear_q": (2.0 * cfg.B * M * C * C, "TFLOP/s", PEAK_BF16_TFLOPS),
        "library_reference_linear_kv": (2.0 * cfg.B * M * C * 2 * C, "TFLOP/s", PEAK_BF16_TFLOPS),
    }
    res = {}
    for k, t in times.items():
        ms = float(np.median(t))
        amount, unit, peak = work[k]
        rate = amount / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        res[k] = {"median_ms": round(ms, 5), unit: round(rate, 2), "frac_peak": round(rate / peak, 4), "work": amount}
    return res


def time_component(dpp, torch, reps=10):
    """One full-image component of the asynchronous component chain (one
    device's work per step when the model is cut into components): GroupNorm
    -> conv -> self-attention over all tokens, at the 2048 px level
    (128 x 128 x 640, 16384 tokens; not part of the headline step)."""
    from dpp_synth import CONFIGS, component_chain_inputs
    from displaced_patch_parallelism_net_amd.step import ComponentChain
    cfg = CONFIGS["sdxl_2048"]
    inp = component_chain_inputs(cfg, 1, 1)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    p = inp["params"][0]
    params = [(dev(p["gamma"]), dev(p["beta"]), dev(p["conv_w"]), dev(p["conv_b"]))]
    x = dev(inp["xs"][0])
    chain = ComponentChain(1, cfg.B, cfg.H, cfg.W, cfg.C, cfg.G, cfg.heads, torch.bfloat16, eps=cfg.gn_eps,
                           head_dim=cfg.D)
    chain.step(x, params, synchronous=True)
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0, e1 = FenceFreeEvent(), FenceFreeEvent()
        e0.record()
        chain.step(x, params, synchronous=True)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b_) for a, b_ in ev]))
    N = cfg.H * cfg.W
    work = 2.0 * cfg.B * N * cfg.C * 9 * cfg.C + 4.0 * cfg.B * cfg.heads * N * N * cfg.D
    rate = work / (ms * 1e-3) / 1e12
    return {"component_step_2048": {"median_ms": round(ms, 5), "TFLOP/s": round(rate, 2),
                                    "frac_peak": round(rate / PEAK_BF16_TFLOPS, 4), "work": work}}


def time_conv_bands(dpp, torch, reps=20):
    """The 640 -> 640 conv of smaller patch bands (not part of the headline
    step), without and with the split-K workspace: the 1024 px level (64 x 64)
    in 4 and 8 patches, the 2048 px level (128 x 128) in 8 patches and the
    3840 px level (240 x 240) in 16 patches.  Back-to-back calls timed as one
    sequence with HIP events; the split count is the library's choice."""
    C = 640
    gen = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for name, H, P in (("1024_p4", 64, 4), ("1024_p8", 64, 8), ("2048_p8", 128, 8), ("3840_p16", 240, 16)):
        R, W = H // P, H
        x = torch.randn(1, R, W, C, device="cuda", generator=gen).to(torch.bfloat16)
        st = torch.randn(1, H, W, C, device="cuda", generator=gen).to(torch.bfloat16)
        w = (0.02 * torch.randn(C, 3, 3, C, device="cuda", generator=gen)).to(torch.bfloat16)
        b = torch.zeros(C, device="cuda")
        y = torch.empty_like(x)
        wsb = dpp.dpp_conv3x3_halo_workspace_bytes(1, R, W, C, C)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
        row = {"rows": R, "W": W, "nsplit": wsb // (R * W * C * 4) if wsb else 1}
        flop = 2.0 * R * W * C * 9 * C
        for mode, wsx in (("unsplit", None), ("split", ws)):
            call = lambda: dpp.dpp_conv3x3_halo(y, x, st, w, b, H, R, workspace=wsx)
            call()
            torch.cuda.synchronize()
            e0, e1 = FenceFreeEvent(), FenceFreeEvent()
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            row[f"{mode}_us"] = round(us, 2)
            row[f"{mode}_TFLOP/s"] = round(flop / (us * 1e-6) / 1e12, 1)
        out[f"conv_band_{name}"] = row
    return out


def hbm_sweep(cfg, dpp, torch, reps=20):
    """Bandwidth of the HBM-bound calls over sizes: the 3840 px patch stacked
    B = 1, 4, 16 times (splice, GroupNorm) and n = 2^16 .. 2^26 (CFG).
    Back-to-back calls timed as one sequence with HIP events (no per-call
    launch latency in the figure).  Warm: every call on the same buffers.
    Cold: the calls rotate over enough independent buffer sets that each
    call's inputs were last touched more than 512 MB earlier (twice the 256 MB
    last-level cache), so they come from HBM.  Algorithmic bytes: one read and
    one write of the patch (plus the tiny statistics) / three n-element
    streams."""
    dev = "cuda"
    LLC_FLUSH = 512 * 2 ** 20

    def n_sets(bytes_per_call, cold):
        return 1 if not cold else int(max(2, -(-LLC_FLUSH // int(bytes_per_call)) + 1))

    def timeit(calls):
        # one untimed call on the last set (reached again only after all others)
        calls[-1]()
        torch.cuda.synchronize()
        e0, e1 = FenceFreeEvent(), FenceFreeEvent()
        e0.record()
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def row(kernel, key, val, nbytes, cold, ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"kernel": kernel, key: val, "bytes": nbytes, "cache": "cold" if cold else "warm",
                "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    res = []
    R, W, C, H, G, P = cfg.rows, cfg.W, cfg.C, cfg.H, cfg.G, cfg.P
    gamma = torch.ones(C, device=dev)
    beta = torch.zeros(C, device=dev)
    for B in (1, 4, 16):
        nbytes = 2.0 * B * R * W * C * 2
        for cold in (False, True):
            k = n_sets(nbytes, cold)
            sets = []
            for _ in range(k):
                full = torch.zeros(B, H, W, C, dtype=torch.bfloat16, device=dev)
                x = torch.randn(B, R, W, C, device=dev).to(torch.bfloat16)
                sets.append((full, x, torch.empty_like(x)))
            st = torch.ones(B, P, G, 2, device=dev)
            so = torch.zeros(B, P, G, 2, device=dev)
            ws = torch.empty(dpp.dpp_groupnorm_stale_workspace_bytes(B, R, W, C, G), dtype=torch.uint8, device=dev)
            sp = [lambda f=f, x=x: dpp.dpp_splice_patch(f, x, 3 * R) for f, x, _ in sets]
            gn = [lambda x=x, y=y: dpp.dpp_groupnorm_stale(y, so, x, st, gamma, beta, H, G, P, 3, 1e-5, ws)
                  for _, x, y in sets]
            res.append(row("splice", "batch", B, nbytes, cold, timeit(sp)))
            res.append(row("groupnorm", "batch", B, nbytes, cold, timeit(gn)))
            # the same GroupNorm with its input's partial sums from the
            # producer (an out projection writing x): x is read once
            M = R * W
            wp = (torch.randn(C, C, device=dev) / C ** 0.5).to(torch.bfloat16)
            nchunk = dpp.dpp_linear_gn_chunks(B, M, C)
            parts = []
            for _, x, _ in sets:
                part = torch.empty(B, nchunk, G, 2, device=dev)
                src = x.clone()
                dpp.dpp_linear_gn(x.view(B, M, C), part, src.view(B, M, C), wp)
                parts.append(part)
                del src
            gnp = [lambda x=x, y=y, pt=pt: dpp.dpp_groupnorm_stale_presummed(y, so, x, pt, st, gamma, beta, H, G, P, 3,
                                                                           1e-5)
                   for (_, x, y), pt in zip(sets, parts)]
            res.append(row("groupnorm_presummed", "batch", B, nbytes, cold, timeit(gnp)))
            del sets, sp, gn, gnp, parts
    for lg in (16, 20, 23, 26):
        n = 2 ** lg
        nbytes = 3.0 * n * 2
        for cold in (False, True):
            k = n_sets(nbytes, cold)
            sets = []
            for _ in range(k):
                c = torch.randn(n, device=dev).to(torch.bfloat16)
                u = torch.randn(n, device=dev).to(torch.bfloat16)
                sets.append((c, u, torch.empty_like(c)))
            rel = torch.zeros(1, device=dev)
            ws = torch.empty(dpp.dpp_cfg_combine_workspace_bytes(n), dtype=torch.uint8, device=dev)
            calls = [lambda c=c, u=u, e=e: dpp.dpp_cfg_combine_relmae(e, rel, c, u, 7.5, ws) for c, u, e in sets]
            res.append(row("cfg", "n", n, nbytes, cold, timeit(calls)))
            del sets, calls
    return res


if __name__ == "__main__":
    main()
