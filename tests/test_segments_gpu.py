"""GPU: the segment-parallel schedule (long sequences in calls with few
(sequence, head) pairs are cut into segments: each segment's state map
S -> P S + R, the states entering the segments, then every segment from its
state), against the fp64 oracle and against the plain schedule.

The schedule is exact algebra (the recurrence is affine in the state), so the
oracle and its tolerances are unchanged.  The segment table it builds on the
device is integer work and is compared exactly with the plan computed here.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import alloc_outputs, assert_parity, new_workspace, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(autouse=True)
def _reset_hooks():
    import gated_delta_rule_tok_amd as kda
    yield
    kda.kda_debug_set_segment(0)
    kda.kda_debug_set_vsplit(0)
    kda.kda_debug_set_kernel(0)


def _seg_cap(H):
    return (32 + 128) // H


def _align(x):
    return (x + 255) // 256 * 256


def _expected_table(cu, T, L, M):
    """The plan: sequence n is cut into max(1, ceil(len / L)) segments of L
    tokens (the last shorter), in order; unused entries are (-1, 0, 0, 0)."""
    rows = []
    for n in range(len(cu) - 1):
        b = min(max(int(cu[n]), 0), T)
        e = min(max(int(cu[n + 1]), b), T)
        c = max(1, -(-(e - b) // L))
        for j in range(c):
            s = b + j * L
            rows.append((n, s, e if j == c - 1 else s + L, 1 if j == c - 1 else 0))
    assert len(rows) <= M
    rows += [(-1, 0, 0, 0)] * (M - len(rows))
    return np.array(rows, np.int32)


def _run_forced(x, L, ws=None):
    import gated_delta_rule_tok_amd as kda
    d = to_device(x)
    prev = kda.kda_debug_set_segment(L)
    try:
        out, fin, ws0 = alloc_outputs(x, d)
        ws = ws0 if ws is None else ws
        run_gpu(x, d, out=out, fin=fin, ws=ws)
    finally:
        kda.kda_debug_set_segment(prev)
    return d, out, fin, ws


@pytest.mark.parametrize("L", [48, 64, 512])
@pytest.mark.parametrize("state", [None, "fp32", "bf16"])
def test_forced_segments_match_oracle(L, state):
    """A ragged batch (an empty sequence, lengths that are and are not
    multiples of the segment length and of 16) cut into segments of L tokens,
    against the oracle; the table in the workspace is the plan."""
    import torch
    lengths = [700, 0, 333, 1500, 64, 65]
    x = KI.make_inputs(lengths, 2, seed=81, init_state=state)
    print(f"[case] forced segments L={L} state={state} T={x.T}", flush=True)
    d, out, fin, ws = _run_forced(x, L)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"segments of {L}")
    M = x.N + x.T // L
    assert M <= _seg_cap(x.H)
    off = 256 + _align(4 * x.N)
    table = ws[off:off + 16 * M].view(torch.int32).cpu().numpy().reshape(M, 4)
    assert np.array_equal(table, _expected_table(x.cu_seqlens, x.T, L, M)), "segment table"


def test_automatic_segments_on_long_low_parallelism():
    """1 x 8192 tokens, 4 heads: the automatic schedule cuts the sequence
    (128 / 4 = 32 segments of 256 tokens): its table is in the workspace, and
    the result matches the oracle and the plain schedule's.  (With the workloads' decay the plain and the segmented
    results are even bit-identical: a segment's transition underflows to zero
    within a few chunks, and what its entering state still contributes after
    the first chunk lies far below an fp32 unit of the state.)"""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([8192], 4, seed=82, init_state="fp32")
    L = kda.kda_debug_segment_length(x.T, x.H, x.N)   # (automatic)
    assert L == 256
    d = to_device(x)
    out_s, fin_s, ws = alloc_outputs(x, d)
    run_gpu(x, d, out=out_s, fin=fin_s, ws=ws)
    kda.kda_debug_set_segment(1)
    out_p, fin_p = run_gpu(x, d)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out_s, fin_s, oref, fref, label="automatic segments")
    assert_parity(x, out_p, fin_p, oref, fref, label="plain schedule")
    M = 1 + 8192 // L
    off = 256 + _align(4 * x.N)
    table = ws[off:off + 16 * M].view(torch.int32).cpu().numpy().reshape(M, 4)
    assert np.array_equal(table, _expected_table(x.cu_seqlens, x.T, L, M)), "segment table"
    assert (out_s.view(torch.int16) != out_p.view(torch.int16)).float().mean().item() < 1e-3


def test_segments_need_the_area():
    """A workspace with only the status word and the order table: the call
    takes the plain schedule (bit for bit the plain result)."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([4096], 2, seed=83, init_state="fp32")
    d = to_device(x)
    small = torch.zeros(256 + _align(4 * x.N), dtype=torch.uint8, device="cuda")
    out_a, fin_a, _ = alloc_outputs(x, d)
    run_gpu(x, d, out=out_a, fin=fin_a, ws=small)
    kda.kda_debug_set_segment(1)
    out_b, fin_b = run_gpu(x, d)
    torch.cuda.synchronize()
    assert int(small[:4].view(torch.int32).item()) == 0
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(fin_a, fin_b)


def test_segments_in_place_state():
    """final_state aliasing initial_state: the combine reads every initial
    state before the rerun writes any final state."""
    import torch
    x = KI.make_inputs([900, 1200, 17], 3, seed=84, init_state="fp32")
    d = to_device(x)
    import gated_delta_rule_tok_amd as kda
    state = d["s0"].clone()
    out = torch.empty(x.T, x.H, D, dtype=torch.bfloat16, device="cuda")
    ws = new_workspace(x.T, x.H, x.N)
    prev = kda.kda_debug_set_segment(128)
    try:
        kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                  d["dt_bias"], x.lower_bound, x.scale, state, d["cu"], out, state,
                                  ws)
    finally:
        kda.kda_debug_set_segment(prev)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out, state, oref, fref, label="segments, in place")


def test_segments_split_invariant_and_deterministic():
    """Within the schedule, every value split gives the same bits, and a
    repeated call too."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([2000, 1100], 4, seed=85, init_state="fp32")
    d = to_device(x)
    res = []
    kda.kda_debug_set_segment(256)
    for s in (2, 4, 8, 8):
        kda.kda_debug_set_vsplit(s)
        o, f = run_gpu(x, d)
        torch.cuda.synchronize()
        res.append((o.view(torch.int16).cpu(), f.cpu()))
    for o, f in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(f, res[0][1])


def test_segments_graph_replay():
    """The four launches captured in a HIP graph and replayed three times
    (eager work in between), each replay equal to the eager call."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([3000, 500], 2, seed=86, init_state="bf16")
    d = to_device(x)
    kda.kda_debug_set_segment(512)
    out0, fin0 = run_gpu(x, d)
    torch.cuda.synchronize()
    out, fin, ws = alloc_outputs(x, d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run_gpu(x, d, out=out, fin=fin, ws=ws, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out0.view(torch.int16)), f"replay {i}: out"
        assert torch.equal(fin.view(torch.int16), fin0.view(torch.int16)), f"replay {i}: state"
        run_gpu(x, d)


@pytest.mark.parametrize("lb", [0.0, -0.05])
def test_segments_weak_decay(lb):
    """With no or weak decay the transition of a segment is far from zero (the
    state remembers across segments): the combine carries it.  Relative
    bounds, as for the plain schedule at these lower bounds."""
    import torch
    x = KI.make_inputs([1500, 700], 2, seed=87, init_state="fp32", lower_bound=lb)
    d, out, fin, ws = _run_forced(x, 256)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"segments, lower_bound {lb}", relative=True)


def test_segments_on_strided_views():
    """The strided entry point takes the schedule too: q, k, v, g as views of
    one fused projection buffer, beta a strided column slice, out half of a
    wider buffer, bit for bit the dense call's (both segmented), and against
    the oracle."""
    import torch
    import gated_delta_rule_tok_amd as kda
    from test_strided_gpu import SENTINEL, _strided_views
    x = KI.make_inputs([1400, 600], 2, seed=88, init_state="fp32")
    d = to_device(x)
    kda.kda_debug_set_segment(256)
    out_d, fin_d = run_gpu(x, d)
    sd, out_s, obuf = _strided_views(d, "fused_rows")
    _, fin_s, ws = alloc_outputs(x, d)
    run_gpu(x, sd, out=out_s, fin=fin_s, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), out_d.view(torch.int16)), "out differs"
    assert torch.equal(fin_s, fin_d), "final state differs"
    assert bool((obuf[..., :128].view(torch.int16) == SENTINEL).all()), "wrote outside out"
    oref, fref = run_oracle(x)
    assert_parity(x, out_s, fin_s, oref, fref, label="segments, strided views")
