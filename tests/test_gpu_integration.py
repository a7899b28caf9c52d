"""GPU integration features: a caller-chosen sequence order (and the library's
longest-first ordering kernel), and capture of a forward call in a HIP graph.
Every call goes through the C ABI via the package binding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_62_amd as kda
from gated_delta_rule_62_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _fwd(inp, order=None):
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"], inp["out"],
            inp["A_log"], inp["dt_bias"], inp["lower_bound"])
    if order is None:
        kda.kda_fwd(*args, inp["initial_state"], inp["final_state"], inp["cu_seqlens"])
    else:
        kda.kda_fwd_ordered(*args, order, inp["initial_state"], inp["final_state"],
                            inp["cu_seqlens"])


def _expected_order(lengths):
    return sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))


@pytest.mark.parametrize("lengths", [[7], [0, 0, 3], [5, 9, 9, 1, 0, 9, 2],
                                     "random64", "random1000", "random8192"])
def test_longest_first_order(lengths):
    if isinstance(lengths, str):
        n = int(lengths[6:])
        rng = np.random.default_rng(n)
        lengths = [int(x) for x in rng.integers(0, 40, size=n)]  # many ties
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device=DEV)
    order = kda.kda_longest_first(cu)
    torch.cuda.synchronize()
    assert order.tolist() == _expected_order(lengths)


def test_sequence_order_is_bitwise_neutral():
    lengths = [300, 700, 1024, 33, 0, 512]
    w = Workload("order", B=1, T=0, H=6, D=128, seed=21, lengths=lengths, state_in="fp32",
                 state_out="fp32")
    inp = make_inputs(w, device=DEV)
    _fwd(inp)
    torch.cuda.synchronize()
    ref = (inp["out"].clone(), inp["final_state"].clone())
    n = len(lengths)
    orders = [torch.arange(n, dtype=torch.int32, device=DEV),
              torch.arange(n - 1, -1, -1, dtype=torch.int32, device=DEV),
              kda.kda_longest_first(inp["cu_seqlens"])]
    for order in orders:
        inp["out"].fill_(float("nan"))
        inp["final_state"].fill_(float("nan"))
        _fwd(inp, order)
        torch.cuda.synchronize()
        assert torch.equal(inp["out"], ref[0]), order.tolist()
        assert torch.equal(inp["final_state"], ref[1]), order.tolist()


def test_automatic_longest_first_is_bitwise_neutral():
    """A packed batch whose workgroups outnumber the CUs makes kda_fwd rank the lengths
    in the kernel and dispatch longest first; the results equal those of the identity
    order bitwise (ties in length included)."""
    lengths = [300, 700, 1024, 33, 0, 512, 33, 700]
    w = Workload("auto_order", B=1, T=0, H=48, D=128, seed=27, lengths=lengths,
                 state_in="bf16")
    inp = make_inputs(w, device=DEV)
    assert len(lengths) * 48 > 256  # more workgroups than compute units
    _fwd(inp)
    torch.cuda.synchronize()
    ref = (inp["out"].clone(), inp["final_state"].clone())
    inp["out"].fill_(float("nan"))
    inp["final_state"].fill_(float("nan"))
    _fwd(inp, torch.arange(len(lengths), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(inp["out"], ref[0]) and torch.equal(inp["final_state"], ref[1])


@pytest.mark.parametrize("case", ["small_grid", "ranked_in_kernel", "ordered"])
def test_graph_capture_replays_match_eager(case):
    """The forward records into a HIP graph (no host sync, no allocation, no memset in
    the call); each replay, with eager work and new input values in between, matches an
    eager call on the same inputs bitwise.  Cases: a grid smaller than the GPU; a packed
    batch of 5 sequences x 96 heads (480 workgroups), which the kernel dispatches longest
    first by its own ranking; and the ordering kernel followed by the ordered forward,
    both in the graph."""
    if case == "small_grid":
        w = Workload("graph", B=1, T=0, H=4, D=128, seed=22, lengths=[200, 64, 333],
                     state_in="bf16")
    else:
        w = Workload("graph", B=1, T=0, H=96, D=128, seed=22, lengths=[200, 64, 333, 90, 17],
                     state_in="bf16")
    inp = make_inputs(w, device=DEV)
    order = torch.empty(len(w.lengths), dtype=torch.int32, device=DEV)

    def call():
        if case == "ordered":
            kda.kda_longest_first(inp["cu_seqlens"], order)
            _fwd(inp, order)
        else:
            _fwd(inp)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream's side, as graph capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    if case == "ordered":
        assert order.cpu().tolist() == _expected_order(w.lengths)
    gen = torch.Generator(device=DEV).manual_seed(5)
    for rep in range(3):
        # new values in the captured input buffers (eager work between replays)
        inp["q"].copy_(torch.randn(inp["q"].shape, generator=gen, device=DEV).to(torch.bfloat16))
        inp["v"].mul_(-1)
        inp["out"].fill_(float("nan"))
        inp["final_state"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (inp["out"].clone(), inp["final_state"].clone())
        inp["out"].fill_(float("nan"))
        inp["final_state"].fill_(float("nan"))
        _fwd(inp)
        torch.cuda.synchronize()
        assert torch.equal(got[0], inp["out"]), rep
        assert torch.equal(got[1], inp["final_state"]), rep


@pytest.mark.parametrize("D,state_in,state_out", [(128, "fp32", "fp32"), (128, "bf16", "fp32"),
                                                  (64, "bf16", "bf16"), (32, "fp32", "bf16")])
def test_transposed_state_layout_matches(D, state_in, state_out):
    """States in the key-major [N,H,K,V] layout give bitwise the results of the [N,H,V,K]
    layout on transposed copies, for every state dtype mix and value-tile schedule."""
    w = Workload("kv", B=1, T=0, H=5, D=D, seed=23, lengths=[97, 0, 160, 31],
                 state_in=state_in, state_out=state_out)
    inp = make_inputs(w, device=DEV)
    _fwd(inp)
    torch.cuda.synchronize()
    ref_out, ref_fin = inp["out"].clone(), inp["final_state"].clone()
    s_in_t = inp["initial_state"].transpose(-1, -2).contiguous()
    fin_t = torch.full_like(inp["final_state"], float("nan"))
    inp["out"].fill_(float("nan"))
    kda.kda_fwd_transposed_state(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                 inp["scale"], inp["out"], inp["A_log"], inp["dt_bias"],
                                 inp["lower_bound"], s_in_t, fin_t, inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(inp["out"], ref_out)
    assert torch.equal(fin_t.transpose(-1, -2), ref_fin)
    # exact in-place alias in the transposed layout
    if state_in == state_out:
        st = inp["initial_state"].transpose(-1, -2).contiguous()
        kda.kda_fwd_transposed_state(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["scale"], inp["out"], inp["A_log"], inp["dt_bias"],
                                     inp["lower_bound"], st, st, inp["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(st.transpose(-1, -2), ref_fin)


def test_concurrent_streams_match_sequential():
    """The library keeps no global state, so calls on different streams may overlap: two
    workloads (a batched one and a packed one with an fp32 state) launched on two streams
    at once, three times over, give bitwise the results of running them one after the
    other on the default stream."""
    wa = Workload("streams_a", B=2, T=200, H=8, D=128, seed=601, state_in="bf16")
    wb = Workload("streams_b", B=1, T=0, H=6, D=64, seed=602, lengths=[50, 0, 131, 7],
                  state_in="fp32", state_out="fp32")
    ia, ib = make_inputs(wa, device="cuda"), make_inputs(wb, device="cuda")

    def call(inp, stream=None):
        kda.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"], inp["out"],
                    inp["A_log"], inp["dt_bias"], inp["lower_bound"], inp["initial_state"],
                    inp["final_state"], inp["cu_seqlens"], stream=stream)

    call(ia)
    call(ib)
    torch.cuda.synchronize()
    ref = [(i["out"].clone(), i["final_state"].clone()) for i in (ia, ib)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        for i in (ia, ib):
            i["out"].zero_()
            i["final_state"].zero_()
        torch.cuda.synchronize()
        call(ia, sa)
        call(ib, sb)
        torch.cuda.synchronize()
        for i, (o, f) in zip((ia, ib), ref):
            assert torch.equal(i["out"], o) and torch.equal(i["final_state"], f)
