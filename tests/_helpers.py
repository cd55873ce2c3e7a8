"""Shared helpers for the GPU tests: host <-> device transfer of the seeded
inputs and the parity bar.

The bar: float32 paths max-abs-err <= 1e-4; bf16 paths max-abs-err <= 2e-2 x
RMS of the oracle output, measured beyond the output's own storage rounding:
a bf16 result cannot be nearer the exact value than half a bf16 ulp of that
value, so each element's distance is reduced by that half ulp before the
comparison (the raw max-abs-err is printed as well); the rel-MAE scalar
within 1e-3 relative; splices bit-exact."""
import numpy as np

import oracle

F32_TOL = 1e-4
BF16_TOL = 2e-2
REL_TOL = 1e-3


def to_dev(a, dtype: str):
    """Stored numpy tensor (uint16 bf16 bits or float32) -> CUDA tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.cuda()


def to_host(t) -> np.ndarray:
    """CUDA tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy().view(np.uint32)


def half_ulp_bf16(v) -> np.ndarray:
    """Half the spacing of bf16 values at |v| (8 significant bits): the
    largest distance between v and its bf16 rounding."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    h = np.exp2(e - 8.0)
    return np.where(a >= 2.0 ** -126, h, 2.0 ** -134)


def parity(got, want, dtype: str, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - want)
    err = float(diff.max())
    rms = float(np.sqrt(np.mean(want * want)))
    if dtype == "bf16":
        excess = float(np.maximum(diff - half_ulp_bf16(want), 0.0).max())
        ok = excess <= BF16_TOL * rms
        # share of elements that differ from the round-to-nearest-even bf16
        # value of the oracle's result (0 for a correctly rounded exact result)
        not_rne = float(np.mean(got != oracle.bf16_round(want))) if want.size else 0.0
        bar = (f"beyond half an output ulp {excess:.3e} = {excess / max(rms, 1e-30):.3e} x rms <= {BF16_TOL} x rms; "
               f"differs from RNE(oracle) in {100.0 * not_rne:.2f}% of elements")
    else:
        ok = err <= F32_TOL
        bar = f"<= {F32_TOL}"
    msg = f"{what}: max-abs-err {err:.3e}, rms {rms:.3e}, err/rms {err / max(rms, 1e-30):.3e} (bar: {bar})"
    print(msg, flush=True)
    assert ok, msg
    return err, rms


# ------------------------------------------------------------------ guard bands
# Outputs of the GPU parity tests are views into a larger buffer whose head
# and tail hold a sentinel bit pattern; after the call the sentinels must be
# intact, so a write past either end of an output is seen.  The guard length
# keeps the view 16-byte aligned for both storage types.
GUARD = 256
SENTINEL = {2: 0x7FA5, 4: 0x7FA5A5A5}     # quiet-NaN payloads no kernel writes


def guarded_empty(shape, dtype):
    """(base, view): view has `shape` and lies GUARD elements into base; the
    rest of base holds the sentinel."""
    import torch
    n = int(np.prod(shape))
    base = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    es = base.element_size()
    base.view(torch.int16 if es == 2 else torch.int32).fill_(SENTINEL[es])
    return base, base[GUARD:GUARD + n].view(shape)


def guarded_copy(t):
    """A guarded buffer whose view holds a copy of t (in/out operands)."""
    base, view = guarded_empty(tuple(t.shape), t.dtype)
    view.copy_(t)
    return base, view


def check_guards(base, what: str):
    """Asserts that the GUARD elements before and after the view are intact."""
    b = bits(base)
    want = SENTINEL[base.element_size()]
    head, tail = b[:GUARD], b[-GUARD:]
    bad = int(np.count_nonzero(head != want) + np.count_nonzero(tail != want))
    assert bad == 0, f"{what}: {bad} guard elements around the output were overwritten"
