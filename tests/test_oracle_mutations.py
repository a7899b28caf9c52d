"""The oracle's pins have teeth: each plausible mistake planted in a copy of the
oracle's C source (built on the CPU into a temporary directory) makes the pin
suite fail.  Nothing here touches a GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

DECAY = "for (int64_t j = 0; j < K; ++j) S[i * K + j] *= alpha[j];"
MUTATIONS = {
    "update_sign": ("const double d = b * (v[row * V + i] - pred);",
                    "const double d = b * (v[row * V + i] + pred);"),
    "beta_not_sigmoid": ("const double b = oracle_sigmoid(beta[row]);",
                         "const double b = beta[row];"),
    "update_uses_q": ("S[i * K + j] += d * kh[j];", "S[i * K + j] += d * qh[j];"),
    "gate_drops_dt_bias": ("(g_row[k] + dt_bias_h[k])", "(g_row[k])"),
    "gate_drops_A": ("a_coef * (g_row[k]", "(g_row[k]"),
    "gate_sign": ("lam[k] = lower_bound * oracle_sigmoid", "lam[k] = -lower_bound * oracle_sigmoid"),
    "no_scale": ("out[row * V + i] = scale * acc;", "out[row * V + i] = acc;"),
    "ignores_initial_state": ("S[i] = S0 ? S0[i] : 0.0;", "S[i] = 0.0;"),
    "no_eps": ("return 1.0 / sqrt(s + KDA_ORACLE_EPS);", "return 1.0 / sqrt(s);"),
    "norm_k_with_q": ("const double rk = oracle_inv_norm(k + row * K, K);",
                      "const double rk = oracle_inv_norm(q + row * K, K);"),
    "decay_skipped": (DECAY, ""),
    "state_transposed_read": ("pred += S[i * K + j] * kh[j];",
                              "pred += S[(j % V) * K + (i % K)] * kh[j];"),
}


def _mutate_decay_after_update(src):
    # move the decay loop after the delta-rule loop
    src = src.replace(DECAY, "")
    anchor = "      /* output after the update: o = scale * S qh */"
    return src.replace(anchor, "      for (int64_t i = 0; i < V; ++i)\n        " + DECAY + "\n" + anchor)


def _mutate_output_before_update(src):
    start = src.index("      /* output after the update")
    end = src.index("    }\n\n    if (final_state)")
    out_block = src[start:end]
    src = src[:start] + src[end:]
    anchor = "      /* delta rule"
    return src.replace(anchor, out_block + anchor)


STRUCTURAL = {"decay_after_update": _mutate_decay_after_update,
              "output_before_update": _mutate_output_before_update}


@pytest.mark.parametrize("name", sorted(list(MUTATIONS) + list(STRUCTURAL)))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    if name in MUTATIONS:
        old, new = MUTATIONS[name]
        assert old in src, "mutation anchor missing: " + name
        src = src.replace(old, new)
    else:
        src = STRUCTURAL[name](src)
        assert src != open(SRC).read()
    c_path = tmp_path / "mut.c"
    so_path = tmp_path / "libmut.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB_OVERRIDE=str(so_path), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])


def test_override_refuses_gpu_sessions(tmp_path):
    """With the override set, a session that collects a GPU test fails at collection
    (so no GPU parity run can compare against a planted mistake), while a CPU-only
    session (the pin suite above) runs."""
    env = dict(os.environ, KDA_ORACLE_LIB_OVERRIDE=str(tmp_path / "none.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "--collect-only", "-m", "gpu",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_gpu_sweep.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "KDA_ORACLE_LIB_OVERRIDE" in (r.stdout + r.stderr)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "--collect-only",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-1000:]
