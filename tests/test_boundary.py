"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side validation returns the documented status codes (no GPU call is made:
kda_fwd_check only compares pointer values and sizes)."""
from __future__ import annotations

import math
import random
import os
import re

import pytest

import gated_delta_rule_62_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        kda.build()
    return kda.load_library()


def _declared_functions():
    names = []
    for hdr in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if hdr.endswith(".h"):
            text = open(os.path.join(ROOT, "include", hdr)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kda_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"kda_fwd", "kda_fwd_sched", "kda_fwd_check", "kda_chunk_anchor",
            "kda_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, -12, -1):
        s = kda.kda_status_string(code)
        assert s.startswith("KDA_")
    assert "UNKNOWN" in kda.kda_status_string(-1234)


def test_anchor_window(lib):
    """The library anchor is the middle of a chunk's decay span, chunk lb log2(e) / 2:
    the pages' 16 lb log2(e) for 32-token chunks, so the centred operands reach at most
    2^118 at the largest span the host admits (236)."""
    log2e = 1.4426950408889634
    for lb in (-0.01, -0.5, -1.0, -3.0, -5.0, -5.1):
        for chunk in (16, 32):
            span = chunk * abs(lb) * log2e
            a = kda.kda_chunk_anchor(lb, chunk)
            assert abs(a + span / 2) < 1e-4, (lb, chunk, a)
            assert -a <= 118.0 + 1e-4
    # lb = -5, 32-token chunks: 16 * -5 * log2(e) = -115.42 (the pages' constant)
    assert abs(kda.kda_chunk_anchor(-5.0, 32) - 16 * -5.0 * log2e) < 1e-4
    assert abs(kda.kda_chunk_anchor(-5.0, 32) + 115.4156) < 1e-3
    assert abs(kda.kda_chunk_anchor(-10.22, 16) + 117.96) < 1e-2
    # one-token chunks: half the token's span, at most half the window (118)
    assert abs(kda.kda_chunk_anchor(-163.5, 1) + 0.5 * 163.5 * log2e) < 1e-3
    assert kda.kda_chunk_anchor(-1e4, 1) == -118.0


# fake device addresses, far apart so that only deliberate overlaps overlap
GB = 1 << 30


def _args(B=2, T=64, H=4, D=128, N=None, has_cu=False, has_s_in=True, has_s_out=True, in_dt=0,
          out_dt=0, lb=-5.0, scale=None, chunk=0, vt=0, **over):
    N = B if N is None else N
    base = dict(q=1 * GB, k=2 * GB, v=3 * GB, g=4 * GB, beta=5 * GB, out=6 * GB, A_log=7 * GB,
                dt_bias=8 * GB, s_in=9 * GB if has_s_in else None,
                s_out=10 * GB if has_s_out else None, cu=11 * GB if has_cu else None)
    base.update(over)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return (base["q"], base["k"], base["v"], base["g"], base["beta"], scale, base["out"],
            base["A_log"], base["dt_bias"], lb, base["s_in"], in_dt, base["s_out"], out_dt,
            base["cu"], N, B, T, H, D, chunk, vt)


def _check(**kw):
    return kda.kda_fwd_check(*_args(**kw))


def test_valid_calls(lib):
    assert _check() == kda.KDA_OK
    assert _check(has_s_in=False, has_s_out=False) == kda.KDA_OK
    assert _check(B=1, T=2024, N=3, has_cu=True, in_dt=1, out_dt=1) == kda.KDA_OK
    assert _check(B=1, T=0, N=3, has_cu=True) == kda.KDA_OK  # every sequence empty
    for D in (32, 64, 128):
        assert _check(D=D) == kda.KDA_OK
    assert _check(chunk=16) == kda.KDA_OK and _check(chunk=32) == kda.KDA_OK
    assert _check(vt=64) == kda.KDA_OK


def test_null_and_shape_errors(lib):
    for name in ("q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"):
        assert _check(**{name: None}) == kda.KDA_ERR_NULL_ARG, name
    # with every sequence empty no activation buffer is touched: NULL is accepted for them
    empty = dict(B=1, T=0, N=3, has_cu=True)
    assert _check(q=None, k=None, v=None, g=None, beta=None, out=None, **empty) == kda.KDA_OK
    assert _check(A_log=None, **empty) == kda.KDA_ERR_NULL_ARG
    assert _check(B=0) == kda.KDA_ERR_BAD_SHAPE
    assert _check(H=0) == kda.KDA_ERR_BAD_SHAPE
    assert _check(T=0) == kda.KDA_ERR_BAD_SHAPE
    assert _check(T=-1) == kda.KDA_ERR_BAD_SHAPE
    for D in (16, 48, 96, 256):
        assert _check(D=D) == kda.KDA_ERR_BAD_SHAPE


def test_size_limits_reject_without_overflow(lib):
    """Sizes whose products would overflow 64 bits are rejected as shapes, never wrapped;
    sizes just inside each limit pass the shape checks."""
    bad = kda.KDA_ERR_BAD_SHAPE
    assert _check(B=1 << 40, T=1 << 40) == bad                  # B T = 2^80
    assert _check(B=1, T=(1 << 40) + 1) == bad
    assert _check(B=1, T=1 << 40) != bad
    assert _check(H=1 << 62) == bad
    assert _check(H=1 << 18, D=128) == bad                      # H D = 2^25
    assert _check(H=(1 << 18) - 1, D=128) != bad
    assert _check(H=1 << 20, D=32) == bad
    assert _check(B=1, T=1 << 40, H=(1 << 20) - 1, D=32) == bad  # ~2^65 activation bytes
    assert _check(B=1, T=(1 << 37) + 1, H=1 << 19, D=32) == bad  # just over 2^62 bytes
    assert _check(B=1, T=1 << 37, H=1 << 19, D=32) != bad        # exactly 2^62 bytes
    assert _check(B=1, T=100, N=1 << 62, has_cu=True) == bad     # num_seqs H overflows
    assert _check(B=1, T=100, N=(1 << 27) + 1, H=4, has_cu=True) == bad
    # num_seqs H = 2^29 passes the unit-count bound but is far beyond the work-item
    # limit of one launch (test_launch_work_item_limit)
    assert _check(B=1, T=100, N=1 << 27, H=4, has_cu=True, has_s_in=False,
                  has_s_out=False) == bad


def test_dtype_and_varlen_errors(lib):
    assert _check(in_dt=2) == kda.KDA_ERR_BAD_DTYPE
    assert _check(out_dt=-1) == kda.KDA_ERR_BAD_DTYPE
    assert _check(has_cu=True, B=2, N=3) == kda.KDA_ERR_BAD_VARLEN
    assert _check(has_cu=True, B=1, N=0) == kda.KDA_ERR_BAD_VARLEN
    assert _check(N=3) == kda.KDA_ERR_BAD_VARLEN  # batched needs N == B


def test_scalar_errors(lib):
    for lb in (0.0, 1.0, float("nan"), float("inf"), float("-inf")):
        assert _check(lb=lb) == kda.KDA_ERR_BAD_LOWER_BOUND, lb
    assert _check(scale=float("nan")) == kda.KDA_ERR_BAD_SCALE
    # decay span chunk |lb| log2(e) <= 236: 32-token chunks to |lb| = 5.1118,
    # 16-token chunks to 10.2236, then 8, 4 and 2 tokens per chunk; one-token chunks
    # take every lower bound whose lb log2(e) is a finite fp32 value (past 163.58 the
    # kernel floors the per-token decay at 2^-236); the automatic schedule takes the
    # longest chunk that fits.
    assert _check(lb=-5.11, chunk=32) == kda.KDA_OK
    assert _check(lb=-5.12, chunk=32) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert _check(lb=-5.12) == kda.KDA_OK
    assert _check(lb=-10.22) == kda.KDA_OK
    assert _check(lb=-10.23, chunk=16) == kda.KDA_ERR_BAD_LOWER_BOUND
    limit = 236.0 / math.log2(math.e)
    for rows in (32, 16, 8, 4, 2):
        inside, outside = -limit / rows * (1 - 1e-4), -limit / rows * (1 + 1e-4)
        assert _check(lb=inside, chunk=rows) == kda.KDA_OK, rows
        assert _check(lb=outside, chunk=rows) == kda.KDA_ERR_BAD_LOWER_BOUND, rows
        assert _check(lb=inside) == kda.KDA_OK, rows
        assert _check(lb=outside) == kda.KDA_OK, rows
    for lb in (-163.5, -163.7, -1e4, -1e30, -2.3e38):
        assert _check(lb=lb) == kda.KDA_OK, lb
        assert _check(lb=lb, chunk=1) == kda.KDA_OK, lb
        assert _check(lb=lb, chunk=2) == kda.KDA_ERR_BAD_LOWER_BOUND, lb
    assert _check(lb=-2.4e38) == kda.KDA_ERR_BAD_LOWER_BOUND  # lb log2(e) overflows fp32
    for rows in (3, 5, 12, 64, -1):
        assert _check(chunk=rows) == kda.KDA_ERR_BAD_SCHEDULE, rows


def test_schedule_errors(lib):
    assert _check(chunk=24) == kda.KDA_ERR_BAD_SCHEDULE
    assert _check(chunk=64) == kda.KDA_ERR_BAD_SCHEDULE
    for rows in (8, 4, 2, 1):  # short chunks run in the 16-row tile's schedules
        assert _check(chunk=rows) == kda.KDA_OK, rows
        assert _check(chunk=rows, vt=64) == kda.KDA_OK, rows
    assert _check(vt=48) == kda.KDA_ERR_BAD_SCHEDULE
    assert _check(vt=16) == kda.KDA_ERR_BAD_SCHEDULE
    assert _check(D=32, vt=64) == kda.KDA_ERR_BAD_SCHEDULE


def test_alias_contract(lib):
    # exact in-place alias: same pointer and dtype
    assert _check(s_out=9 * GB) == kda.KDA_OK
    # same pointer, different dtype: partial overlap of extents
    assert _check(s_out=9 * GB, out_dt=1) == kda.KDA_ERR_BAD_ALIAS
    # partial overlap of the two states
    assert _check(s_out=9 * GB + 256) == kda.KDA_ERR_BAD_ALIAS
    # out overlapping an input, or the final state overlapping an input
    assert _check(out=1 * GB + 2) == kda.KDA_ERR_BAD_ALIAS
    assert _check(out=9 * GB) == kda.KDA_ERR_BAD_ALIAS
    assert _check(s_out=3 * GB) == kda.KDA_ERR_BAD_ALIAS
    assert _check(s_out=6 * GB) == kda.KDA_ERR_BAD_ALIAS
    assert _check(B=1, T=100, N=2, has_cu=True, s_out=11 * GB) == kda.KDA_ERR_BAD_ALIAS
    # adjacent, non-overlapping buffers are fine: q ends where k starts
    act = 2 * 64 * 4 * 128 * 2
    assert _check(k=1 * GB + act) == kda.KDA_OK


def _ordered(seq_order, **kw):
    a = _args(**kw)
    return kda.load_library().kda_fwd_ordered(*a[:-2], None, seq_order)


def test_ordered_and_longest_first_validation(lib):
    """Error paths of kda_fwd_ordered and kda_longest_first return before any launch."""
    assert _ordered(None) == kda.KDA_ERR_NULL_ARG
    # the order array is an input: no output may overlap it
    assert _ordered(12 * GB, out=12 * GB) == kda.KDA_ERR_BAD_ALIAS
    assert _ordered(12 * GB, B=1, T=100, N=2, has_cu=True, s_out=12 * GB) == kda.KDA_ERR_BAD_ALIAS
    # everything kda_fwd rejects is still rejected
    assert _ordered(12 * GB, lb=1.0) == kda.KDA_ERR_BAD_LOWER_BOUND
    lf = lib.kda_longest_first
    assert lf(None, 3, 12 * GB, None) == kda.KDA_ERR_NULL_ARG
    assert lf(11 * GB, 3, None, None) == kda.KDA_ERR_NULL_ARG
    assert lf(11 * GB, 0, 12 * GB, None) == kda.KDA_ERR_BAD_VARLEN
    assert lf(11 * GB, 8193, 12 * GB, None) == kda.KDA_ERR_BAD_VARLEN
    assert lf(11 * GB, 4, 11 * GB + 8, None) == kda.KDA_ERR_BAD_ALIAS


def test_split_workspace_bytes(lib):
    """One record per slot and head: the byte images of Qc, Kc ([C][D+16] bf16), Kr
    ([C][D+16] bf16), the solve operands and Mqk in two parts ([C][C+8] bf16) and the
    decay (D fp32); floor(T_total / chunk) + num_seqs + 1 slots per head."""
    rec32 = 2 * 32 * 144 * 2 + 32 * 144 * 2 + 3 * 32 * 40 * 2 + 128 * 4
    rec16 = 2 * 16 * 144 * 2 + 16 * 144 * 2 + 3 * 16 * 24 * 2 + 128 * 4
    assert rec32 == 35840 and rec16 == 16640
    ws = kda.kda_split_workspace_bytes
    assert ws(32768, 1, 96, 128, -5.0) == 96 * (1024 + 2) * rec32
    assert ws(2024, 3, 96, 128, -5.0) == 96 * (63 + 4) * rec32
    assert ws(2024, 3, 96, 128, -8.0) == 96 * (126 + 4) * rec16       # automatic: 16 tokens
    assert ws(2024, 3, 96, 128, -5.0, 8) == 96 * (253 + 4) * rec16    # 8 tokens in 16 rows
    assert ws(0, 5, 2, 128, -1.0) == 2 * 6 * rec32                   # every sequence empty
    raw = lib.kda_split_workspace_bytes
    assert raw(2024, 3, 96, 64, -5.0, 0) == kda.KDA_ERR_BAD_SCHEDULE  # D = 128 only
    assert raw(2024, 3, 96, 128, 0.0, 0) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert raw(2024, 3, 96, 128, -6.0, 32) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert raw(2024, 3, 96, 128, -5.0, 24) == kda.KDA_ERR_BAD_SCHEDULE
    assert raw(2024, 0, 96, 128, -5.0, 0) == kda.KDA_ERR_BAD_SHAPE
    assert raw(2024, 3, 0, 128, -5.0, 0) == kda.KDA_ERR_BAD_SHAPE
    # a head's records must stay below 2^31 bytes (31-bit offsets)
    assert raw(1 << 22, 1, 1, 128, -5.0, 0) == kda.KDA_ERR_BAD_SHAPE
    assert raw(1 << 20, 1, 1, 128, -5.0, 0) == ((1 << 15) + 2) * rec32
    # the sizing the library computes is floor(T_total / chunk) + N + 1 records per head
    rng = random.Random(11)
    for _ in range(200):
        T, N, H = rng.randint(0, 5000), rng.randint(1, 40), rng.randint(1, 97)
        chunk = rng.choice([32, 16, 8, 4, 2, 1])
        rec = rec32 if chunk == 32 else rec16
        assert raw(T, N, H, 128, -0.5, chunk) == (T // chunk + N + 1) * rec * H


def _split(ws, ws_bytes, vt=0, chunk=0, **kw):
    a = _args(**kw)
    return kda.load_library().kda_fwd_split(*a[:-2], None, ws, ws_bytes, chunk, vt)


def test_split_validation(lib):
    """Error paths of kda_fwd_split return before any launch."""
    need = kda.kda_split_workspace_bytes(2 * 64, 2, 4, 128, -5.0)
    assert _split(None, need) == kda.KDA_ERR_NULL_ARG
    assert _split(12 * GB, need - 1) == kda.KDA_ERR_BAD_WORKSPACE
    assert _split(12 * GB, need, D=64) == kda.KDA_ERR_BAD_SCHEDULE
    assert _split(12 * GB, need, vt=32) == kda.KDA_ERR_BAD_SCHEDULE
    # 16-token chunks run the split at value tile 128 only
    assert _split(12 * GB, 1 << 40, vt=64, lb=-8.0) == kda.KDA_ERR_BAD_SCHEDULE
    # the workspace is written: it may overlap no other buffer
    assert _split(1 * GB, need) == kda.KDA_ERR_BAD_ALIAS
    assert _split(9 * GB + 64, need) == kda.KDA_ERR_BAD_ALIAS
    assert _split(11 * GB - 16, need, B=1, T=128, N=2, has_cu=True) == kda.KDA_ERR_BAD_ALIAS
    # everything kda_fwd rejects is still rejected
    assert _split(12 * GB, need, lb=1.0) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert _split(12 * GB, need, q=None) == kda.KDA_ERR_NULL_ARG
    # a forced chunk length sizes and runs the same split: a workspace sized for
    # 16-token chunks is enough with chunk_size 16 (the call then reaches the alias
    # check, which follows the size check) and too small for the automatic 32
    need16 = kda.kda_split_workspace_bytes(2 * 64, 2, 4, 128, -5.0, 16)
    assert need16 < need
    assert _split(1 * GB, need16, chunk=16) == kda.KDA_ERR_BAD_ALIAS
    assert _split(1 * GB, need16, chunk=0) == kda.KDA_ERR_BAD_WORKSPACE
    assert _split(12 * GB, need, chunk=24) == kda.KDA_ERR_BAD_SCHEDULE
    assert _split(12 * GB, need, chunk=32, lb=-6.0) == kda.KDA_ERR_BAD_LOWER_BOUND


def test_launch_work_item_limit():
    """A launch covers at most 2^32 - 1 work-items: workgroups times their threads.
    D = 32 runs 128-thread workgroups (one per sequence and head); D = 128 with
    32-token chunks and value tile 128 runs 768-thread ones.  The split's prep kernel
    runs one 512-thread workgroup per slot and head."""
    ok = kda.KDA_OK
    packed = dict(B=1, T=8, H=1, has_cu=True, has_s_in=False, has_s_out=False)
    lim32 = ((1 << 32) - 1) // 128
    assert _check(N=lim32, D=32, **packed) == ok
    assert _check(N=lim32 + 1, D=32, **packed) == kda.KDA_ERR_BAD_SHAPE
    lim128 = ((1 << 32) - 1) // 768
    assert _check(N=lim128, D=128, vt=128, **packed) == ok
    assert _check(N=lim128 + 1, D=128, vt=128, **packed) == kda.KDA_ERR_BAD_SHAPE
    ws = kda.load_library().kda_split_workspace_bytes
    limp = ((1 << 32) - 1) // 512
    H = 1 << 10
    slots_ok = limp // H                      # 8191 slots of one sequence
    t_ok = (slots_ok - 2) * 32
    assert ws(t_ok, 1, H, 128, -5.0, 0) > 0
    assert ws(t_ok + 32, 1, H, 128, -5.0, 0) == kda.KDA_ERR_BAD_SHAPE


def test_split_slot_numbering_is_injective_and_fits():
    """The split files chunk c of sequence n under slot floor(start(n) / chunk) + n + c.
    The prep kernel finds a slot's sequence by binary search over first slots, and the
    workspace holds floor(T_total / chunk) + num_seqs + 1 slots per head.  Over random
    packed batches (empty sequences included) and every chunk length:
    * no two chunks share a slot;
    * first slots grow strictly with n;
    * every slot is below the sized count."""
    rng = random.Random(7)
    for _ in range(300):
        lens = [rng.choice([0, 0, 1, rng.randint(1, 9), rng.randint(1, 300)])
                for _ in range(rng.randint(1, 12))]
        cu = [0]
        for length in lens:
            cu.append(cu[-1] + length)
        for chunk in (32, 16, 8, 4, 2, 1):
            slots = cu[-1] // chunk + len(lens) + 1
            seen = set()
            firsts = [cu[n] // chunk + n for n in range(len(lens))]
            assert all(a < b for a, b in zip(firsts, firsts[1:]))
            for n, length in enumerate(lens):
                for c in range((length + chunk - 1) // chunk):
                    j = firsts[n] + c
                    assert j not in seen and 0 <= j < slots
                    seen.add(j)
                    # the binary search's answer: the last sequence whose first slot <= j
                    assert max(m for m in range(len(lens)) if firsts[m] <= j) == n


def test_noalloc_split_rejects_workspaces_beyond_its_scratch(lib):
    """kda_fwd_split_noalloc checks the call's workspace against its 64 MiB static
    scratch on the host and returns before touching the device."""
    cap = lib.kda_split_noalloc_max_bytes()
    assert cap == 64 << 20
    noalloc = lib.kda_fwd_split_noalloc
    # 96 heads of 2 x 1024 tokens need 96 * 67 records of 35,840 bytes: too many
    a = _args(B=2, T=1024, H=96)
    assert kda.kda_split_workspace_bytes(2048, 2, 96, 128, -5.0) > cap
    assert noalloc(*a[:-2], None, 0, 0) == kda.KDA_ERR_SCRATCH_TOO_SMALL
    # validation errors come first, exactly as for kda_fwd_split
    assert noalloc(*_args(B=2, T=1024, H=96, lb=1.0)[:-2], None, 0, 0) == \
        kda.KDA_ERR_BAD_LOWER_BOUND
    assert noalloc(*_args(D=64)[:-2], None, 0, 0) == kda.KDA_ERR_BAD_SCHEDULE
    assert noalloc(*a[:-2], None, 24, 0) == kda.KDA_ERR_BAD_SCHEDULE


def test_bf16_state_mode_schedules(lib):
    """kda_fwd_bf16_state runs D = 128 with 32-token chunks at value tiles 64 and 128
    only; every other schedule returns KDA_ERR_BAD_SCHEDULE on the host, after the
    same argument checks as kda_fwd_sched."""
    f = lib.kda_fwd_bf16_state

    def call(chunk=0, vt=128, **kw):
        a = _args(**kw)
        return f(*a[:-2], None, chunk, vt)

    assert call(D=64, vt=64) == kda.KDA_ERR_BAD_SCHEDULE
    assert call(D=32, vt=32) == kda.KDA_ERR_BAD_SCHEDULE
    assert call(chunk=16) == kda.KDA_ERR_BAD_SCHEDULE
    assert call(chunk=8) == kda.KDA_ERR_BAD_SCHEDULE
    # |lb| = 8 admits 16-token chunks at most: the automatic choice is 16 (no kernel),
    # and forcing 32 breaks the decay window
    assert call(lb=-8.0) == kda.KDA_ERR_BAD_SCHEDULE
    assert call(lb=-8.0, chunk=32) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert call(vt=32) == kda.KDA_ERR_BAD_SCHEDULE
    # the shared checks come first
    assert call(lb=1.0) == kda.KDA_ERR_BAD_LOWER_BOUND
    assert call(s_out=9 * GB + 2) == kda.KDA_ERR_BAD_ALIAS
    assert call(q=None) == kda.KDA_ERR_NULL_ARG
