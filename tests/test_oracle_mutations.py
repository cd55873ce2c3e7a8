"""Planted mistakes: each one, applied to a copy of the oracle, must make the
oracle's pins (tests/test_oracle_pins.py) fail.

This is what makes the pins worth trusting: a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle is caught by something
other than the oracle itself.  Each mutation is a one-place text replacement
in oracle/dpp_oracle.py; the pin suite runs on the mutated copy in a separate
process (CPU only).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle/dpp_oracle.py, replacement)
MUTATIONS = [
    ("gn_unbiased_variance", "var = np.maximum(total[..., 1] / n - mean * mean, 0.0)",
     "var = np.maximum(total[..., 1] / n - mean * mean, 0.0) * n / (n - 1)"),
    ("gn_own_stale_slot_used", "            if q != p:\n", "            if True:\n"),
    ("gn_eps_dropped", "rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / np.sqrt(var)"),
    ("gn_beta_dropped", "y = (x - mean_c) * rstd_c * _f64(gamma) + _f64(beta)", "y = (x - mean_c) * rstd_c * _f64(gamma)"),
    ("conv_taps_transposed", "y += tap @ wt[:, dy, dx, :].T", "y += tap @ wt[:, dx, dy, :].T"),
    ("conv_halo_off_by_one", "        r = row0 - 1 + i\n", "        r = row0 + i\n"),
    ("conv_bias_dropped", "    if bias is not None:\n        y += _f64(bias)\n    return y\n",
     "    return y\n"),
    ("attn_scale_dropped", "s = scale * (qb[:, cs] @ k[b, :, cs].T)", "s = (qb[:, cs] @ k[b, :, cs].T)"),
    ("attn_no_normaliser", "out[part, cs] = (e @ v[b, :, cs]) / e.sum(axis=1, keepdims=True)",
     "out[part, cs] = (e @ v[b, :, cs]) / e.sum()"),
    ("cfg_wrong_base", "eps = u + guidance * d", "eps = c + guidance * d"),
    ("relmae_wrong_denominator", "rel = np.float64(np.abs(d).sum()) / np.float64(np.abs(u).sum())",
     "rel = np.float64(np.abs(d).sum()) / np.float64(np.abs(c).sum())"),
    ("bf16_truncates", "r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)",
     "r = (u >> np.uint64(16)) << np.uint64(16)"),
    ("splice_shifted", "out[:, row0:row0 + rows] = patch", "out[:, row0 + 1:row0 + 1 + rows] = patch[:, :-1]"),
    ("linear_weight_not_transposed", "y = _f64(x) @ _f64(w).T", "y = _f64(x) @ _f64(w)"),
    ("silu_sign", "return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    ("schedule_strict_flattening", "decline <= rho32 * fastest", "decline < rho32 * fastest"),
    ("schedule_no_hysteresis", "if d[i] > grow * lowest:", "if d[i] > lowest:"),
    ("chain_reads_this_step", "src = outs[t - 1][k - 1][\"o\"]", "src = row[k - 1][\"o\"]"),
    ("block_kv_not_spliced", "    K[:, t0:t0 + R * W] = _store(k_exact, bf16)\n", "\n"),
    ("block_halo_from_conv_output", "y2_exact = conv3x3_halo(y1, state[\"a1\"], conv_w, conv_b, r0)",
     "y2_exact = conv3x3_halo(y1, state[\"a2\"], conv_w, conv_b, r0)"),
    ("block_previous_kv_from_gn", "    t = a2.reshape(B, H * W, C)\n", "    t = a1.reshape(B, H * W, C)\n"),
]


def _run(mut):
    name, old, new = mut
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        for d in ("oracle", "dpp_synth"):
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("__pycache__"))
        os.makedirs(os.path.join(tmp, "tests"))
        for f in ("conftest.py", "test_oracle_pins.py", "_helpers.py"):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)
        p = os.path.join(tmp, "oracle", "dpp_oracle.py")
        src = open(p).read()
        if src.count(old) != 1:
            return name, None, f"pattern found {src.count(old)} times"
        open(p, "w").write(src.replace(old, new))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "tests/test_oracle_pins.py"], cwd=tmp,
                           capture_output=True, text=True, timeout=600, env=env)
        return name, r.returncode, r.stdout.strip().splitlines()[-1] if r.stdout.strip() else r.stderr[-300:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_unmutated_copy_passes():
    name, rc, tail = _run(("none", "def _f64(a)", "def _f64(a)"))
    assert rc == 0, tail


def test_every_planted_mistake_fails_a_pin():
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run, MUTATIONS))
    survivors = []
    for name, rc, tail in results:
        print(f"{name:32s} rc={rc}  {tail}", flush=True)
        if rc is None:
            pytest.fail(f"mutation {name} no longer applies: {tail}")
        if rc == 0:
            survivors.append(name)
    assert not survivors, f"pins do not catch: {survivors}"
