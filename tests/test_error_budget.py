"""Error budget of the GPU kernel (CPU): where its error against the oracle comes from.

The kernel computes the chunk form of the FlashInfer PR #4262 summary (section 2's
centred operands, section 3's decomposition) with bf16 matrix-core operands and fp32
accumulation.  ``emulate`` follows the same steps in fp64 and rounds to bf16 (round to
nearest even) at each site where the kernel does, one switch per site:

  qc, kc, ki, kr   the centred operands Qc, Kc, Ki and the decayed Kr
  mqk    the stored Mqk (as 2^-Ca Mqk; the power of two is exact)
  sol    the solve operands: the inverses of the diagonal 16x16 blocks of I + L, and -L21
  scopy  the bf16 copy of the state used by the products P = S Kd^T and O0 = S Qd^T
  r      R_top and R_bot - L21 U_top as they enter the blocked solve
  u      U_top inside the solve, and U for the state update and the output
  out    the output tile

The tests hold the relative L2 errors of ``out`` against the fp64 oracle to the values the
design notes quote (every site rounded, which is what the GPU measures; each site alone),
within the slack stated in each test.  ``python tests/test_error_budget.py`` prints the
full table.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from gated_delta_rule_62_amd.workloads import Workload, make_inputs  # noqa: E402

LOG2E = 1.0 / math.log(2.0)
SITES = ("qc", "kc", "ki", "kr", "mqk", "sol", "scopy", "r", "u", "out")
CHUNK = 32


def _bf16(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _np(t):
    return t.to("cpu").double().numpy()


def emulate(inp, rounded):
    """out [T, H, V] and final state [H, V, K] of one batched sequence (B = 1)."""
    r = {s: (_bf16 if s in rounded else (lambda x: x)) for s in SITES}
    q, k, v, beta_l = (_np(inp[n])[0] for n in ("q", "k", "v", "beta"))
    lam = oracle.gate(inp["g"], inp["A_log"], inp["dt_bias"], inp["lower_bound"])[0]
    T, H, K = q.shape
    V = v.shape[-1]
    b = inp["lower_bound"] * LOG2E
    ca = CHUNK * b / 2  # the anchor: the middle of the chunk's decay span
    s0 = inp["initial_state"]
    out = np.zeros((T, H, V))
    fin = np.zeros((H, V, K))
    for h in range(H):
        S = np.zeros((V, K)) if s0 is None else _np(s0)[0, h]
        for c0 in range(0, T, CHUNK):
            rows = slice(c0, min(c0 + CHUNK, T))
            m = rows.stop - rows.start
            qh = q[rows, h] / np.sqrt((q[rows, h] ** 2).sum(-1, keepdims=True) + 1e-6)
            kh = k[rows, h] / np.sqrt((k[rows, h] ** 2).sum(-1, keepdims=True) + 1e-6)
            beta = 1.0 / (1.0 + np.exp(-beta_l[rows, h]))
            G = np.cumsum(lam[rows, h] * LOG2E, axis=0)
            GT = G[-1]
            Qc = r["qc"](qh * np.exp2(G - ca))
            Kc = r["kc"](kh * np.exp2(G - ca))
            Ki = r["ki"](kh * np.exp2(ca - G))
            Kr = r["kr"](kh * np.exp2(GT[None, :] - G))
            A = Kc @ Ki.T
            L = np.where(np.tril(np.ones((m, m), dtype=bool), -1), beta[:, None] * A, 0.0)
            Mqk = r["mqk"](np.where(np.tril(np.ones((m, m), dtype=bool)), Qc @ Ki.T, 0.0))
            t = min(16, m)
            X11 = r["sol"](np.linalg.inv(np.eye(t) + L[:t, :t]))
            Sb = r["scopy"](S)
            P = (Kc * 2.0 ** ca) @ Sb.T          # [m, V]: Kd S^T
            O0 = (Qc * 2.0 ** ca) @ Sb.T         # [m, V]: Qd S^T
            R = beta[:, None] * (v[rows, h] - P)
            U = np.zeros((m, V))
            U[:t] = r["u"](X11 @ r["r"](R[:t]))
            if m > 16:
                X22 = r["sol"](np.linalg.inv(np.eye(m - 16) + L[16:, 16:]))
                L21 = -r["sol"](-L[16:, :16])
                U[16:] = X22 @ r["r"](R[16:] - L21 @ U[:t])
            U = r["u"](U)
            S = S * np.exp2(GT)[None, :] + U.T @ Kr
            S = S.astype(np.float32).astype(np.float64)  # fp32 accumulators
            out[rows, h] = r["out"](inp["scale"] * (O0 + Mqk @ U))
        fin[h] = S
    return out, fin


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


CASES = {"D=128, lb=-5": dict(D=128, lower_bound=-5.0),
         "D=128, lb=-0.01": dict(D=128, lower_bound=-0.01),
         "D=32, lb=-0.01": dict(D=32, lower_bound=-0.01)}


def _case(name):
    w = Workload("budget", B=1, T=512, H=2, seed=41, state_in="fp32", state_out="fp32",
                 **CASES[name])
    inp = make_inputs(w, device="cpu")
    o_ref, f_ref = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                  inp["scale"], inp["A_log"], inp["dt_bias"],
                                  inp["lower_bound"], inp["initial_state"])
    return inp, o_ref[0], f_ref[0]


# out rel-L2 with every site rounded (the GPU measures 3.98e-3, 4.29e-3 and 4.70e-3 on the
# same shapes), and with one site rounded alone at D = 128, lb = -5
ALL_SITES = {"D=128, lb=-5": 3.99e-3, "D=128, lb=-0.01": 4.29e-3, "D=32, lb=-0.01": 4.69e-3}
ONE_SITE = {"qc": 1.75e-3, "kc": 1.6e-5, "ki": 1.70e-3, "kr": 4.5e-5, "mqk": 1.64e-3,
            "sol": 1.8e-5, "scopy": 6.7e-5, "r": 1.67e-3, "u": 1.66e-3, "out": 1.67e-3}


def test_every_site_rounded_reproduces_the_measured_errors():
    """Within 3% of the quoted values, and below the 5e-3 bound with 5% to spare."""
    for name, want in ALL_SITES.items():
        inp, o_ref, _ = _case(name)
        o, _ = emulate(inp, set(SITES))
        got = _rel(o, o_ref)
        assert abs(got - want) <= 0.03 * want, (name, got, want)
        assert got <= 0.95 * 5e-3, (name, got)


def test_single_sites_and_their_quadrature_sum():
    """Each site alone within 10% of the quoted value; the six sites of about one bf16
    rounding each (1.6e-3 to 1.8e-3) add up in quadrature to the every-site error within
    10%; and the site the design notes name as the cheapest to split (Mqk in two bf16
    parts, which removes its rounding) lowers the strong-decay error to 3.69e-3."""
    inp, o_ref, _ = _case("D=128, lb=-5")
    alone = {}
    for site, want in ONE_SITE.items():
        o, _ = emulate(inp, {site})
        alone[site] = _rel(o, o_ref)
        assert abs(alone[site] - want) <= 0.10 * want, (site, alone[site], want)
    big = [v for v in alone.values() if v > 1e-3]
    assert len(big) == 6
    o, _ = emulate(inp, set(SITES))
    total = _rel(o, o_ref)
    assert abs(math.sqrt(sum(v * v for v in alone.values())) - total) <= 0.10 * total
    o, _ = emulate(inp, set(SITES) - {"mqk"})
    assert abs(_rel(o, o_ref) - 3.69e-3) <= 0.03 * 3.69e-3


def main():
    for name in CASES:
        inp, o_ref, f_ref = _case(name)
        print("== %s (T = 512, H = 2)" % name)
        o, f = emulate(inp, set(SITES))
        print("  every site rounded:   out %.2e  state %.2e" % (_rel(o, o_ref), _rel(f, f_ref)))
        for site in SITES:
            o, f = emulate(inp, set(SITES) - {site})
            print("  all but %-6s       out %.2e  state %.2e" % (site, _rel(o, o_ref), _rel(f, f_ref)))
        for site in SITES:
            o, f = emulate(inp, {site})
            print("  only %-6s          out %.2e  state %.2e" % (site, _rel(o, o_ref), _rel(f, f_ref)))


if __name__ == "__main__":
    main()
