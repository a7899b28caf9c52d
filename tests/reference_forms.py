"""Independent fp64 forms of the KDA forward, used only to pin the oracle.

Neither form shares code with the oracle (``oracle/kda_oracle.c``), which runs
the per-token recurrence.  They take the per-token natural-log decay ``lam`` as
an input (the gate has its own closed-form pins), so they check the recurrence
structure: decay order, read-after-update, the delta rule, and state carry.

* ``chunk_form`` writes out the chunk decomposition of the FlashInfer PR #4262
  summary, section 2 (fixed-anchor exponent centring) and section 3
  ("Intra-Chunk and Inter-Chunk Decomposition"): inclusive base-2 prefix G,
  centred operands, L = strictLower(diag(beta) Kc Ki^T),
  Mqk = lowerTri(Qc Ki^T), INV = (I + L)^-1, then S_d, O_0, P, R, U and the
  updates S_new = S_d + U K_r and O = O_0 + U Mqk^T.
* ``brute_force`` composes explicit K x K transition matrices
  M_t = diag(alpha_t) (I - beta_t kh_t kh_t^T), so that
  S_t = S_0 prod M + sum_s beta_s v_s kh_s^T prod_{r>s} M_r, on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
NORM_EPS = 1e-6


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _segments(T_total, B, T, cu):
    if cu is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def chunk_form(q, k, v, lam, beta_logit, scale, chunk, anchor, initial_state=None, cu=None):
    """Chunked forward per the page's equations.

    q, k, lam: [B,T,H,K] fp64 (lam in natural-log units); v: [B,T,H,V];
    beta_logit [B,T,H]; anchor: the scalar exponent centre C (0 disables it).
    Returns (out [B,T,H,V], final [N,H,V,K]).
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf, kf, vf = q.reshape(B * T, H, K), k.reshape(B * T, H, K), v.reshape(B * T, H, V)
    lf, bf = lam.reshape(B * T, H, K), beta_logit.reshape(B * T, H)
    segs = _segments(B * T, B, T, cu)
    out = np.zeros((B * T, H, V))
    fin = np.zeros((len(segs), H, V, K))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S = np.zeros((V, K)) if initial_state is None else initial_state[n, h].copy()
            for c0 in range(s0, s1, chunk):
                rows = slice(c0, min(c0 + chunk, s1))
                qh = _l2n(qf[rows, h])
                kh = _l2n(kf[rows, h])
                beta = _sigmoid(bf[rows, h])
                G = np.cumsum(lf[rows, h] * LOG2E, axis=0)  # inclusive base-2 prefix
                GT = G[-1]
                m = G.shape[0]
                Qc = scale * qh * np.exp2(G - anchor)
                Kc = kh * np.exp2(G - anchor)
                Ki = kh * np.exp2(anchor - G)
                low_strict = np.tril(np.ones((m, m), dtype=bool), -1)
                low_incl = np.tril(np.ones((m, m), dtype=bool), 0)
                L = np.where(low_strict, beta[:, None] * (Kc @ Ki.T), 0.0)
                Mqk = np.where(low_incl, Qc @ Ki.T, 0.0)
                INV = np.linalg.inv(np.eye(m) + L)
                Qd = scale * qh * np.exp2(G)
                Kd = kh * np.exp2(G)
                Kr = kh * np.exp2(GT[None, :] - G)
                a = np.exp2(GT)
                Sd = S * a[None, :]
                O0 = S @ Qd.T
                P = S @ Kd.T
                R = (vf[rows, h].T - P) * beta[None, :]
                U = R @ INV.T
                S = Sd + U @ Kr
                out[rows, h] = (O0 + U @ Mqk.T).T
            fin[n, h] = S
    return out.reshape(B, T, H, V), fin


def chunk_intra(q, k, lam, beta_logit, scale, anchor):
    """(L, Mqk) of one chunk, q/k/lam [m,K] for one head; used by the centring pin."""
    qh, kh = _l2n(q), _l2n(k)
    beta = _sigmoid(beta_logit)
    G = np.cumsum(lam * LOG2E, axis=0)
    m = G.shape[0]
    Qc = scale * qh * np.exp2(G - anchor)
    Kc = kh * np.exp2(G - anchor)
    Ki = kh * np.exp2(anchor - G)
    L = np.where(np.tril(np.ones((m, m), dtype=bool), -1), beta[:, None] * (Kc @ Ki.T), 0.0)
    Mqk = np.where(np.tril(np.ones((m, m), dtype=bool), 0), Qc @ Ki.T, 0.0)
    return L, Mqk


def brute_force(q, k, v, lam, beta_logit, scale, initial_state=None, cu=None):
    """Explicit transition-matrix products; O(T^2) matrix work, tiny inputs only."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf, kf, vf = q.reshape(B * T, H, K), k.reshape(B * T, H, K), v.reshape(B * T, H, V)
    lf, bf = lam.reshape(B * T, H, K), beta_logit.reshape(B * T, H)
    segs = _segments(B * T, B, T, cu)
    out = np.zeros((B * T, H, V))
    fin = np.zeros((len(segs), H, V, K))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S0 = np.zeros((V, K)) if initial_state is None else initial_state[n, h]
            kh = _l2n(kf[s0:s1, h])
            qh = _l2n(qf[s0:s1, h])
            beta = _sigmoid(bf[s0:s1, h])
            Ms = [np.diag(np.exp(lf[s0 + i, h])) @ (np.eye(K) - beta[i] * np.outer(kh[i], kh[i]))
                  for i in range(s1 - s0)]

            def prod(lo, hi):  # M_lo M_{lo+1} ... M_{hi-1}
                P = np.eye(K)
                for i in range(lo, hi):
                    P = P @ Ms[i]
                return P

            def state_after(t):  # state after tokens 0..t of the segment
                S = S0 @ prod(0, t + 1)
                for s in range(t + 1):
                    S = S + beta[s] * np.outer(vf[s0 + s, h], kh[s]) @ prod(s + 1, t + 1)
                return S

            for t in range(s1 - s0):
                out[s0 + t, h] = scale * state_after(t) @ qh[t]
            fin[n, h] = state_after(s1 - s0 - 1) if s1 > s0 else S0
    return out.reshape(B, T, H, V), fin
