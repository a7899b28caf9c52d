"""MI355X (gfx950) KDA recurrent prefill forward.

A thin ctypes binding over ``libkda.so`` (built from ``csrc/`` with hipcc): it
checks tensor dtypes, devices and contiguity, passes raw device pointers, sizes
and torch's current HIP stream to the C ABI declared in ``include/kda.h``, and
turns status codes into exceptions.  Every step of the computation runs in the
library's kernels; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB_PATH, build  # noqa: F401  (build() is the in-tree compile step)

__all__ = ["kda_fwd", "kda_fwd_sched", "kda_fwd_ordered", "kda_fwd_transposed_state",
           "kda_fwd_bf16_state",
           "kda_fwd_split", "kda_split_workspace_bytes", "kda_fwd_split_noalloc",
           "kda_longest_first", "kda_fwd_check", "c_args",
           "kda_chunk_anchor", "kda_status_string", "KdaError", "library_path", "load_library"]

KDA_OK = 0
KDA_ERR_NULL_ARG = -1
KDA_ERR_BAD_SHAPE = -2
KDA_ERR_BAD_DTYPE = -3
KDA_ERR_BAD_VARLEN = -4
KDA_ERR_BAD_ALIAS = -5
KDA_ERR_BAD_LOWER_BOUND = -6
KDA_ERR_BAD_SCALE = -7
KDA_ERR_BAD_SCHEDULE = -8
KDA_ERR_HIP = -9
KDA_ERR_BAD_WORKSPACE = -10
KDA_ERR_SCRATCH_TOO_SMALL = -11
KDA_DTYPE_BF16 = 0
KDA_DTYPE_FP32 = 1

_lib = None


class KdaError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(kda_status_string(status))


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load ``libkda.so``; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkda.so is not built at %s; run gated_delta_rule_62_amd.build() "
                          "(or __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    common = [vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, vp, i32, vp, i32, vp, i64, i64, i64, i64,
              i64]
    lib.kda_fwd.argtypes = common + [vp]
    lib.kda_fwd.restype = i32
    lib.kda_fwd_sched.argtypes = common + [vp, i32, i32]
    lib.kda_fwd_sched.restype = i32
    lib.kda_fwd_ordered.argtypes = common + [vp, vp]
    lib.kda_fwd_ordered.restype = i32
    lib.kda_fwd_transposed_state.argtypes = common + [vp]
    lib.kda_fwd_transposed_state.restype = i32
    lib.kda_fwd_bf16_state.argtypes = common + [vp, i32, i32]
    lib.kda_fwd_bf16_state.restype = i32
    lib.kda_longest_first.argtypes = [vp, i64, vp, vp]
    lib.kda_longest_first.restype = i32
    lib.kda_split_workspace_bytes.argtypes = [i64, i64, i64, i64, f32, i32]
    lib.kda_split_workspace_bytes.restype = i64
    lib.kda_fwd_split.argtypes = common + [vp, vp, i64, i32, i32]
    lib.kda_fwd_split_noalloc.argtypes = common + [vp, i32, i32]
    lib.kda_fwd_split_noalloc.restype = i32
    lib.kda_split_noalloc_max_bytes.argtypes = []
    lib.kda_split_noalloc_max_bytes.restype = i64
    lib.kda_fwd_split.restype = i32
    lib.kda_fwd_check.argtypes = common + [i32, i32]
    lib.kda_fwd_check.restype = i32
    lib.kda_chunk_anchor.argtypes = [f32, i32]
    lib.kda_chunk_anchor.restype = f32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_chunk_anchor(lower_bound: float, chunk_size: int) -> float:
    return float(load_library().kda_chunk_anchor(float(lower_bound), int(chunk_size)))


def kda_fwd_check(*args) -> int:
    """Host-only validation with raw integer pointers; same arguments as the C function."""
    return int(load_library().kda_fwd_check(*args))


def _state_dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_FP32
    raise TypeError("state tensors must be bfloat16 or float32, got %s" % t.dtype)


def _on_device(t):
    """The library launches on the current HIP device: make t's device current."""
    import torch
    return torch.cuda.device(t.device)


def c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
           final_state, cu_seqlens, stream=None, extra=()):
    """Checks the tensors and returns the C arguments shared by every forward entry point
    (everything up to and including the stream), for callers that launch the C functions
    of ``load_library()`` directly in a tight loop.  Such callers make the tensors' device
    current themselves (``torch.cuda.device``): the library launches on the current one."""
    import torch
    acts = {"q": q, "k": k, "v": v, "g": g, "out": out}
    for name, t in acts.items():
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise TypeError("%s must be a 4-d bfloat16 tensor" % name)
    B, T, H, D = q.shape
    for name, t in acts.items():
        if tuple(t.shape) != (B, T, H, D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (B, T, H, D)))
    if beta.dtype != torch.bfloat16 or tuple(beta.shape) != (B, T, H):
        raise ValueError("beta must be bfloat16 [B,T,H]")
    if A_log.dtype != torch.float32 or tuple(A_log.shape) != (H,):
        raise ValueError("A_log must be float32 [H]")
    if dt_bias.dtype != torch.float32 or tuple(dt_bias.shape) != (H, D):
        raise ValueError("dt_bias must be float32 [H,D]")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-d int64 tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    tensors = [q, k, v, g, beta, out, A_log, dt_bias] + list(extra)
    for t in (initial_state, final_state, cu_seqlens):
        if t is not None:
            tensors.append(t)
    for t in (initial_state, final_state):
        if t is not None and tuple(t.shape) != (N, H, D, D):
            raise ValueError("states must be [N,H,D,D] = %s" % ((N, H, D, D),))
    dev = q.device
    for t in tensors:
        if t.device != dev or dev.type != "cuda":
            raise ValueError("every tensor must live on the same GPU")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    s_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    ptr = lambda t: None if t is None else t.data_ptr()
    return (ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), float(scale), ptr(out), ptr(A_log),
            ptr(dt_bias), float(lower_bound), ptr(initial_state),
            _state_dtype_code(initial_state) if initial_state is not None else 0,
            ptr(final_state), _state_dtype_code(final_state) if final_state is not None else 0,
            ptr(cu_seqlens), N, B, T, H, D, s_ptr)


def kda_fwd_sched(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                  initial_state=None, final_state=None, cu_seqlens=None,
                  chunk_size: int = 0, v_tile: int = 0, stream=None) -> None:
    """Runs the forward on the device tensors given (asynchronous on ``stream``).

    q, k, v, g, out: bf16 ``[B,T,H,D]``; beta bf16 ``[B,T,H]``; A_log fp32 ``[H]``;
    dt_bias fp32 ``[H,D]``; states ``[N,H,D,D]`` bf16 or fp32 (or None);
    cu_seqlens int64 ``[N+1]`` on the device (varlen, B == 1) or None (batched).
    ``chunk_size`` 0 (the longest admissible) or tokens per chunk (32, 16, 8, 4, 2, 1);
    ``v_tile`` 0 (automatic) or the value rows per workgroup.
    ``stream`` defaults to torch's current stream on q's device.
    """
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream)
    with _on_device(q):
        st = load_library().kda_fwd_sched(*args, int(chunk_size), int(v_tile))
    if st != KDA_OK:
        raise KdaError(st)


def kda_fwd_ordered(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, seq_order,
                    initial_state=None, final_state=None, cu_seqlens=None, stream=None) -> None:
    """``kda_fwd`` with the workgroups of sequence ``seq_order[0]`` dispatched first, then
    ``seq_order[1]``, ...  ``seq_order``: int32 ``[N]`` device permutation (see
    ``kda_longest_first``).  The results are bitwise those of ``kda_fwd``."""
    import torch
    if seq_order.dtype != torch.int32 or seq_order.dim() != 1:
        raise ValueError("seq_order must be a 1-d int32 tensor")
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream, extra=(seq_order,))
    if seq_order.numel() != args[15]:
        raise ValueError("seq_order must have one entry per sequence")
    with _on_device(q):
        st = load_library().kda_fwd_ordered(*args, seq_order.data_ptr())
    if st != KDA_OK:
        raise KdaError(st)


def kda_fwd_transposed_state(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                             initial_state=None, final_state=None, cu_seqlens=None,
                             stream=None) -> None:
    """``kda_fwd`` with both states in the key-major layout ``[N,H,D(k),D(v)]``."""
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream)
    with _on_device(q):
        st = load_library().kda_fwd_transposed_state(*args)
    if st != KDA_OK:
        raise KdaError(st)


def kda_fwd_bf16_state(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                       initial_state=None, final_state=None, cu_seqlens=None,
                       chunk_size: int = 0, v_tile: int = 0, stream=None) -> None:
    """``kda_fwd_sched`` with the recurrent state kept in bf16 in LDS (widened to fp32
    for each chunk's update, rounded once back).  D = 128 with 32-token chunks only."""
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream)
    with _on_device(q):
        st = load_library().kda_fwd_bf16_state(*args, int(chunk_size), int(v_tile))
    if st != KDA_OK:
        raise KdaError(st)


def kda_split_workspace_bytes(T_total: int, num_seqs: int, H: int, D: int, lower_bound: float,
                              chunk_size: int = 0) -> int:
    """Bytes of the workspace ``kda_fwd_split`` needs (raises KdaError when the split
    does not run these sizes)."""
    n = load_library().kda_split_workspace_bytes(int(T_total), int(num_seqs), int(H), int(D),
                                                 float(lower_bound), int(chunk_size))
    if n < 0:
        raise KdaError(int(n))
    return int(n)


def kda_fwd_split(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, workspace,
                  initial_state=None, final_state=None, cu_seqlens=None, v_tile: int = 0,
                  stream=None, chunk_size: int = 0) -> None:
    """``kda_fwd`` as two kernels: a token-parallel preparation of every chunk into
    ``workspace`` (a contiguous uint8 device tensor of at least
    ``kda_split_workspace_bytes(..., chunk_size)`` bytes), then the recurrent kernel on
    value tiles of ``v_tile`` rows (0: automatic).  The results are bitwise those of
    ``kda_fwd_sched`` with the same chunk length and value tile."""
    import torch
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-d uint8 tensor")
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream, extra=(workspace,))
    with _on_device(q):
        st = load_library().kda_fwd_split(*args, workspace.data_ptr(), workspace.numel(),
                                          int(chunk_size), int(v_tile))
    if st != KDA_OK:
        raise KdaError(st)


def kda_fwd_split_noalloc(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                          initial_state=None, final_state=None, cu_seqlens=None,
                          v_tile: int = 0, stream=None, chunk_size: int = 0) -> None:
    """``kda_fwd_split`` with the library's per-GPU static scratch as its workspace (for
    callers that cannot allocate); raises ``KdaError(KDA_ERR_SCRATCH_TOO_SMALL)`` when
    the call's workspace would exceed it."""
    args = c_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, stream)
    with _on_device(q):
        st = load_library().kda_fwd_split_noalloc(*args, int(chunk_size), int(v_tile))
    if st != KDA_OK:
        raise KdaError(st)


def kda_longest_first(cu_seqlens, seq_order=None, stream=None):
    """Longest-first order (int32 ``[N]``, on the device) of the sequences of ``cu_seqlens``,
    computed by the library's ordering kernel; written into ``seq_order`` if given."""
    import torch
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be a 1-d int64 GPU tensor")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    N = cu_seqlens.numel() - 1
    if seq_order is None:
        seq_order = torch.empty(max(N, 0), dtype=torch.int32, device=cu_seqlens.device)
    elif (seq_order.dtype != torch.int32 or tuple(seq_order.shape) != (N,)
          or seq_order.device != cu_seqlens.device or not seq_order.is_contiguous()):
        raise ValueError("seq_order must be a contiguous int32 [N] tensor on cu_seqlens' GPU")
    if stream is None:
        stream = torch.cuda.current_stream(cu_seqlens.device)
    s_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with _on_device(cu_seqlens):
        st = load_library().kda_longest_first(cu_seqlens.data_ptr(), N, seq_order.data_ptr()
                                              if N > 0 else None, s_ptr)
    if st != KDA_OK:
        raise KdaError(st)
    return seq_order


def kda_fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None,
            final_state=None, cu_seqlens=None, stream=None) -> None:
    """The FlashKDA ``fwd`` contract with the library's automatic schedule."""
    kda_fwd_sched(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                  final_state, cu_seqlens, 0, 0, stream)
