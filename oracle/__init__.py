"""CPU oracle for the KDA recurrent prefill forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's ``smoke()`` check and the benchmark's
``cpu_baseline`` leg may import this module.  The product path (the HIP library
and its Python binding) never imports it and never falls back to it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, OpenMP over the
independent (sequence, head) units).  This module only marshals arrays:
it widens inputs to float64, turns batched mode into the equivalent
``cu_seqlens = [0, T, 2T, ...]`` partition of the flattened token axis (the
batched/varlen contract of "How FlashKDA Manages Recurrent State Across
Sequences and Batch Modes"), and calls the C code.

Parity status: the recurrence is pinned by the tests under ``tests/``
(brute-force transition products, the chunk decomposition of the FlashInfer
PR #4262 summary section 3, closed forms and invariants).  The gate formula is
a reading of the pages (they name its inputs and its range, not the formula);
its closed-form values and range are pinned, its agreement with the original
FlashKDA implementation is not (no values for it are printed anywhere).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
# The mutation test points this at a deliberately broken build of the oracle.
_LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIB_OVERRIDE")
_lib = None


def override_active() -> bool:
    """Whether KDA_ORACLE_LIB_OVERRIDE (the mutation test's swapped build) is in force."""
    return bool(_LIB_OVERRIDE)


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``libkda_oracle.so`` with gcc (fp64, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [d, d, d, d, d, ctypes.c_double, d, d, ctypes.c_double,
                                       d, d, d, ctypes.POINTER(ctypes.c_int64), i64, i64, i64,
                                       i64, i64, ctypes.c_int]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_gate.argtypes = [d, d, d, ctypes.c_double, i64, i64, i64, d]
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """float64, C-contiguous copy of a numpy array or a (CPU or device) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only reached when a tensor was passed in
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gate(g, A_log, dt_bias, lower_bound: float) -> np.ndarray:
    """Per-token natural-log decay lam[..., H, K] for g[..., H, K] (the oracle's gate)."""
    g64 = _f64(g)
    shape = g64.shape
    H, K = shape[-2], shape[-1]
    T = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    lam = np.empty((T, H, K), dtype=np.float64)
    a64, d64 = _f64(A_log), _f64(dt_bias)
    assert a64.shape == (H,) and d64.shape == (H, K)
    _load().kda_oracle_gate(_ptr(g64), _ptr(a64), _ptr(d64), float(lower_bound), T, H, K,
                            _ptr(lam))
    return lam.reshape(shape)


def kda_fwd(q, k, v, g, beta, scale: float, A_log, dt_bias, lower_bound: float,
            initial_state=None, cu_seqlens=None, nthreads: int = 0):
    """fp64 KDA forward.

    Shapes follow the ``fwd`` contract of "How FlashKDA Manages Recurrent State
    Across Sequences and Batch Modes": q, k, g ``[B,T,H,K]``, v ``[B,T,H,V]``,
    beta ``[B,T,H]``, A_log ``[H]``, dt_bias ``[H,K]``, state ``[N,H,V,K]`` with
    N = B (batched) or ``len(cu_seqlens) - 1`` (varlen, B must be 1).

    Returns ``(out [B,T,H,V], final_state [N,H,V,K])`` as float64 numpy arrays.
    """
    q64, k64, v64, g64, b64 = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q64.shape
    V = v64.shape[-1]
    assert k64.shape == (B, T, H, K) and g64.shape == (B, T, H, K)
    assert v64.shape == (B, T, H, V) and b64.shape == (B, T, H)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1, "varlen mode packs every sequence into B == 1"
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
    N = len(cu) - 1
    a64, d64 = _f64(A_log), _f64(dt_bias)
    assert a64.shape == (H,) and d64.shape == (H, K)
    s0 = None
    if initial_state is not None:
        s0 = _f64(initial_state)
        assert s0.shape == (N, H, V, K)
    out = np.zeros((B, T, H, V), dtype=np.float64)
    fin = np.zeros((N, H, V, K), dtype=np.float64)
    rc = _load().kda_oracle_fwd(
        _ptr(q64), _ptr(k64), _ptr(v64), _ptr(g64), _ptr(b64), float(scale), _ptr(a64),
        _ptr(d64), float(lower_bound), _ptr(s0) if s0 is not None else None, _ptr(out),
        _ptr(fin), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, B * T, H, K, V,
        int(nthreads))
    if rc != 0:
        raise ValueError("cu_seqlens must be a non-decreasing partition of [0, B*T]")
    return out, fin
