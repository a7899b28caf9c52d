"""GPU parity with many (sequence, head) units, against the fp64 oracle.

Launches with several times more units than the MI355X has compute units, so that
workgroups start as others finish, formed every way the kernel forms its grid: packed
sequences ranked longest first by the kernel (at most 256 of them), more than 256 in
index order, a caller's order, and batched rows; with empty sequences, short chunks,
both state layouts, state dtype mixes and NULL states.  Tolerances as in the other
parity tests: max-abs 2e-2 and rel-L2 5e-3 over each whole tensor.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_62_amd as kda
import oracle
from gated_delta_rule_62_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 5e-3


def _close(x, ref, what):
    x = x.to("cpu", torch.float64).numpy()
    mx = float(np.abs(x - ref).max())
    rel = float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))
    print("%s: max-abs %.3e rel-L2 %.3e (%.0f%% and %.0f%% of the bounds)"
          % (what, mx, rel, 100 * mx / MAX_ABS, 100 * rel / REL_L2), flush=True)
    assert mx <= MAX_ABS and rel <= REL_L2, "%s: max-abs %.3e rel-L2 %.3e" % (what, mx, rel)


def _lengths(n, hi, seed, p_empty=0.1):
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, hi + 1, (n,), generator=g)
    lens[torch.rand(n, generator=g) < p_empty] = 0
    return lens.tolist()


def _run_and_check(inp, tag, final=True, order=None):
    inp["out"].fill_(float("nan"))
    fin = inp["final_state"] if final else None
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"], inp["out"],
            inp["A_log"], inp["dt_bias"], inp["lower_bound"], inp["initial_state"], fin,
            inp["cu_seqlens"])
    if order is None:
        kda.kda_fwd(*args)
    else:
        kda.kda_fwd_ordered(*args[:10], order, initial_state=inp["initial_state"],
                            final_state=fin, cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    out_ref, fin_ref = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      inp["scale"], inp["A_log"], inp["dt_bias"],
                                      inp["lower_bound"], inp["initial_state"],
                                      inp["cu_seqlens"])
    _close(inp["out"], out_ref, tag + " out")
    if final:
        _close(inp["final_state"], fin_ref, tag + " final_state")


def test_index_order_many_sequences_with_empties():
    # 600 sequences (more than the kernel ranks): index order, 1200 units; empty
    # sequences pass their state through
    w = Workload("p_index", B=1, T=0, H=2, D=128, seed=501, lengths=_lengths(600, 40, 501),
                 state_in="fp32", state_out="fp32")
    inp = make_inputs(w, device="cuda")
    _run_and_check(inp, "600 seqs")
    for n, l in enumerate(w.lengths):
        if l == 0:
            assert torch.equal(inp["final_state"][n], inp["initial_state"][n])


def test_ranked_longest_first_and_caller_order():
    # 200 sequences (ranked by the kernel), H = 4: 800 units; then a caller's order
    w = Workload("p_rank", B=1, T=0, H=4, D=128, seed=502, lengths=_lengths(200, 90, 502),
                 state_in="bf16", state_out="bf16")
    inp = make_inputs(w, device="cuda")
    _run_and_check(inp, "200 seqs ranked")
    order = torch.arange(199, -1, -1, dtype=torch.int32, device="cuda")
    _run_and_check(inp, "200 seqs reversed order", order=order)


def test_batched_rows_and_null_states():
    # batched mode: B = 6, H = 96 gives 576 units; no initial state, then no final state
    w = Workload("p_batch", B=6, T=50, H=96, D=128, seed=503, state_in=None, state_out="fp32")
    inp = make_inputs(w, device="cuda")
    _run_and_check(inp, "batched 576 units")
    _run_and_check(inp, "batched 576 units, no final", final=False)


def test_short_chunks_many_units():
    # lb = -20 takes 8-token chunks in 16-row tiles; 300 sequences x 2 heads
    w = Workload("p_short", B=1, T=0, H=2, D=128, seed=504, lengths=_lengths(300, 64, 504),
                 state_in="fp32", state_out="bf16", lower_bound=-20.0)
    inp = make_inputs(w, device="cuda")
    _run_and_check(inp, "short chunks")


def test_transposed_state_many_units_bitwise():
    w = Workload("p_kv", B=1, T=0, H=4, D=128, seed=505, lengths=_lengths(150, 70, 505),
                 state_in="bf16", state_out="fp32")
    inp = make_inputs(w, device="cuda")
    args = lambda s_in, s_out: (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                                inp["out"], inp["A_log"], inp["dt_bias"], inp["lower_bound"],
                                s_in, s_out, inp["cu_seqlens"])
    kda.kda_fwd(*args(inp["initial_state"], inp["final_state"]))
    torch.cuda.synchronize()
    out_ref, fin_ref = inp["out"].clone(), inp["final_state"].clone()
    s_in_t = inp["initial_state"].transpose(-1, -2).contiguous()
    s_out_t = torch.empty_like(inp["final_state"])
    inp["out"].zero_()
    kda.kda_fwd_transposed_state(*args(s_in_t, s_out_t))
    torch.cuda.synchronize()
    assert torch.equal(inp["out"], out_ref)
    assert torch.equal(s_out_t.transpose(-1, -2), fin_ref)


def test_many_workload_bitwise_deterministic():
    w = WORKLOADS["many"]
    inp = make_inputs(w, device="cuda")
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"], inp["out"],
            inp["A_log"], inp["dt_bias"], inp["lower_bound"], inp["initial_state"],
            inp["final_state"], inp["cu_seqlens"])
    kda.kda_fwd(*args)
    torch.cuda.synchronize()
    ref = (inp["out"].clone(), inp["final_state"].clone())
    for _ in range(3):
        inp["out"].zero_()
        inp["final_state"].zero_()
        kda.kda_fwd(*args)
        torch.cuda.synchronize()
        assert torch.equal(inp["out"], ref[0]) and torch.equal(inp["final_state"], ref[1])
