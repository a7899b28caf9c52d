"""Study (CPU, not a test): what storing the recurrent state in bf16 between chunk
updates would cost in accuracy.

FlashKDA keeps its state in bf16 in shared memory and rounds it once per update
cycle ("How FlashKDA Stores On-Chip Recurrent State in BF16 for Memory
Efficiency"; the fp32-FMA update is described in "FlashKDA State Update
Numerical Precision").  This library keeps the state in fp32 registers instead.
The study runs the exact fp64 per-token recurrence three ways on the same seeded
inputs: unrounded (the oracle itself), with the state rounded to fp32 after
every 32-token chunk, and rounded to bf16 (round to nearest even) after every
chunk; it prints the relative L2 error of ``out`` and of the final state of the
rounded runs against the oracle.  Usage: ``python tests/study_state_precision.py``.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from gated_delta_rule_62_amd.workloads import Workload, make_inputs  # noqa: E402

CHUNK = 32


def _round_bf16(x: np.ndarray) -> np.ndarray:
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _round_fp32(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float32).astype(np.float64)


def _recurrence(inp, head, rounding):
    """fp64 per-token recurrence of one head of a batched (B = 1) workload, the
    state passed through ``rounding`` after every CHUNK tokens."""
    f64 = lambda t: t.float().double().numpy()
    q, k, v, g = (f64(inp[n][0, :, head]) for n in ("q", "k", "v", "g"))
    beta = f64(inp["beta"][0, :, head])
    A = np.exp(float(inp["A_log"][head]))
    dt = inp["dt_bias"][head].double().numpy()
    lb, scale = float(inp["lower_bound"]), float(inp["scale"])
    S = f64(inp["initial_state"][0, head]) if inp["initial_state"] is not None else \
        np.zeros((q.shape[1], q.shape[1]))
    out = np.empty_like(q)
    for t in range(q.shape[0]):
        lam = lb / (1.0 + np.exp(-A * (g[t] + dt)))
        kh = k[t] / np.sqrt(k[t] @ k[t] + 1e-6)
        qh = q[t] / np.sqrt(q[t] @ q[t] + 1e-6)
        b = 1.0 / (1.0 + np.exp(-beta[t]))
        S = S * np.exp(lam)[None, :]
        S = S + b * np.outer(v[t] - S @ kh, kh)
        out[t] = scale * (S @ qh)
        if (t + 1) % CHUNK == 0:
            S = rounding(S)
    return out, S


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def main():
    cases = [("T=1024, bf16 N(0, 0.1^2) initial state",
              Workload("study1k", B=1, T=1024, H=4, D=128, seed=31, state_in="bf16"), 4),
             ("T=32768, zero initial state",
              Workload("study32k", B=1, T=32768, H=1, D=128, seed=32, state_in="zero_bf16"), 1)]
    print("| workload | heads | state kept as | out rel-L2 | final state rel-L2 |")
    print("|---|---|---|---|---|")
    for label, w, heads in cases:
        inp = make_inputs(w)
        t0 = time.time()
        ref_out, ref_fin = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                          inp["scale"], inp["A_log"], inp["dt_bias"],
                                          inp["lower_bound"], inp["initial_state"], None)
        for name, rnd in (("fp32 (per chunk)", _round_fp32), ("bf16 (per chunk)", _round_bf16)):
            outs, fins = [], []
            for h in range(heads):
                o, s = _recurrence(inp, h, rnd)
                outs.append(o)
                fins.append(s)
            o = np.stack(outs, axis=1)
            s = np.stack(fins, axis=0)
            print("| %s | %d | %s | %.2e | %.2e |" % (
                label, heads, name, _rel(o, ref_out[0, :, :heads]), _rel(s, ref_fin[0, :heads])),
                flush=True)
        print("<!-- %s: %.1f s -->" % (label, time.time() - t0), flush=True)


if __name__ == "__main__":
    main()
