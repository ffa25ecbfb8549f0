"""GPU: the two-workgroup form of the 16-token kernel (a producer workgroup
builds every chunk package of a (sequence, head) pair once, a consumer
workgroup on the same XCD walks the state over all 128 value columns; the
packages go through a ring in the workspace), against the fp64 oracle and
against the single-workgroup kernel.

Both forms run the same arithmetic per value column in the same order, so
their results are compared bit for bit; the oracle tolerances are unchanged.
Whether the two-workgroup form ran is read from the workspace: its loaders
clear the pair's flag words at the end of a call, so flag words filled with
a pattern before the call are zero after it exactly when it ran.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import (alloc_outputs, assert_parity, new_workspace, run_gpu, run_oracle,
                      to_device)

pytestmark = pytest.mark.gpu

D = 128
PATTERN = 0x5A


@pytest.fixture(autouse=True)
def _reset_hooks():
    import gated_delta_rule_tok_amd as kda
    yield
    kda.kda_debug_set_kernel(0)
    kda.kda_debug_set_vsplit(0)
    kda.kda_debug_set_segment(0)


def _align(x):
    return (x + 255) // 256 * 256


def _flags_off(N):
    """Byte offset of the flag words: the status word and order table, then
    the segment area's table, first/count arrays, summaries and entering
    states (160 slots each)."""
    area = 2560 + 768 + 768 + 160 * 3 * D * D * 4
    return 256 + _align(4 * N) + area


def _patterned_workspace(x):
    """A workspace with its second part (sized as for at least 1024 tokens:
    the ring and the flag words live there) holding a pattern; the status
    word stays zero."""
    ws = new_workspace(max(x.T, 1024), x.H, x.N)
    ws[256:].fill_(PATTERN)
    return ws


FLAG_WORDS = 8   # per pair: published counts (2 copy waves), loaded counts (2 loaders), 4 unused
USED_WORDS = 4


def _flag_words(ws, x):
    """The used flag words of every pair, [pairs, 4]."""
    import torch
    off = _flags_off(x.N)
    assert ws.numel() >= off + 8 * FLAG_WORDS * x.N * x.H, "workspace without the flag words"
    w = ws[off:off + 8 * FLAG_WORDS * x.N * x.H].view(torch.int64).cpu().numpy()
    return w.reshape(x.N * x.H, FLAG_WORDS)[:, :USED_WORDS]


def _ran_duo(ws, x) -> bool:
    w = _flag_words(ws, x)
    if (w == 0).all():
        return True
    pat = np.frombuffer(bytes([PATTERN]) * 8, dtype=np.int64)[0]
    assert (w == pat).all(), "flag words neither cleared nor untouched"
    return False


def _plain(x, d):
    """The single-workgroup kernel (a value-split override keeps it)."""
    import torch
    import gated_delta_rule_tok_amd as kda
    prev = kda.kda_debug_set_vsplit(2)
    try:
        o, f = run_gpu(x, d)
        torch.cuda.synchronize()
    finally:
        kda.kda_debug_set_vsplit(prev)
    return o, f


def _same_bits(a, b, what):
    import torch
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b), f"{what} differs from the single-workgroup kernel"


@pytest.mark.parametrize("state", [None, "fp32", "bf16"])
def test_duo_ragged_matches_oracle_and_plain(state):
    """36 pairs (6 sequences x 6 heads: an empty one, lengths that are and are
    not multiples of 16, one of 1500 tokens whose ring of 8 packages wraps many
    times): the automatic choice takes the two-workgroup form; against the
    oracle, and bit for bit against the single-workgroup kernel."""
    import torch
    x = KI.make_inputs([700, 0, 333, 1500, 64, 65], 6, seed=91, init_state=state)
    print(f"[case] duo ragged state={state} T={x.T} pairs={x.N * x.H}", flush=True)
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x), "the two-workgroup form did not run"
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"two workgroups, state {state}")
    o2, f2 = _plain(x, d)
    _same_bits(out, o2, "out")
    _same_bits(fin, f2, "final state")


def test_duo_headline_shape_bit_identical():
    """8 x 2048 tokens, 16 heads (128 pairs, the whole device) in the
    two-workgroup form: bit for bit the single-workgroup kernel."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([2048] * 8, 16, seed=92, init_state="fp32")
    print(f"[case] duo 8x2048 h16", flush=True)
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    kda.kda_debug_set_kernel(6)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    kda.kda_debug_set_kernel(0)
    assert _ran_duo(ws, x)
    o2, f2 = _plain(x, d)
    _same_bits(out, o2, "out")
    _same_bits(fin, f2, "final state")


@pytest.mark.parametrize("lengths,heads", [([300], 2), ([17, 33], 1), ([16], 3), ([5000], 1)])
def test_duo_forced_few_pairs(lengths, heads):
    """Kernel 6 forces the form for few pairs (below the automatic range):
    single chunks, partial chunks, one long sequence; against the oracle and
    the single-workgroup kernel."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs(lengths, heads, seed=93, init_state="fp32")
    print(f"[case] duo forced {lengths} h{heads}", flush=True)
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    kda.kda_debug_set_kernel(6)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    kda.kda_debug_set_kernel(0)
    assert _ran_duo(ws, x)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"two workgroups forced {lengths} h{heads}")
    o2, f2 = _plain(x, d)
    _same_bits(out, o2, "out")
    _same_bits(fin, f2, "final state")


def test_duo_automatic_range():
    """32 pairs stay on the single-workgroup kernel (or the segment schedule),
    33 take the two-workgroup form, 128 pairs of 2048 tokens (above 2^17
    (token, head) pairs) do not; a workspace without its second part keeps the
    single-workgroup kernel."""
    import torch
    for lengths, heads, want in (([2048] * 8, 16, False), ([256] * 8, 4, False),
                                 ([256] * 11, 3, True)):
        x = KI.make_inputs(lengths, heads, seed=94, init_state="fp32")
        d = to_device(x)
        out, fin, _ = alloc_outputs(x, d)
        ws = _patterned_workspace(x)
        run_gpu(x, d, out=out, fin=fin, ws=ws)
        torch.cuda.synchronize()
        assert _ran_duo(ws, x) == want, f"{len(lengths)} x {heads}"
    small = torch.zeros(256 + _align(4 * x.N), dtype=torch.uint8, device="cuda")
    out_s, fin_s, _ = alloc_outputs(x, d)
    run_gpu(x, d, out=out_s, fin=fin_s, ws=small)
    torch.cuda.synchronize()
    assert int(small[:4].view(torch.int32).item()) == 0
    _same_bits(out_s, out, "out without the second part")


def test_duo_repeated_calls_and_graph_replay():
    """Calls with the same workspace in a row, and the call captured in a HIP
    graph (its flag words carry the captured call's nonce) replayed three
    times with eager calls in between: every result equal to the first."""
    import torch
    x = KI.make_inputs([900, 1200, 400, 1000], 10, seed=95, init_state="bf16")
    d = to_device(x)
    out0, fin0, ws = alloc_outputs(x, d)
    run_gpu(x, d, out=out0, fin=fin0, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    for _ in range(2):
        o, f = run_gpu(x, d, out=torch.empty_like(out0), fin=torch.empty_like(fin0), ws=ws)
        torch.cuda.synchronize()
        _same_bits(o, out0, "repeated call out")
        _same_bits(f, fin0, "repeated call state")
    out, fin = torch.empty_like(out0), torch.empty_like(fin0)
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
        run_gpu(x, d, out=torch.empty_like(out0), fin=torch.empty_like(fin0), ws=ws)
    torch.cuda.synchronize()
    assert (_flag_words(ws, x) == 0).all()


def test_duo_random_workspace_contents():
    """Flag words and ring left with arbitrary bytes (another schedule's data,
    an uninitialised buffer): the call's nonce keeps them from being taken for
    its own; the result is the single-workgroup kernel's."""
    import torch
    x = KI.make_inputs([1100, 800, 600], 12, seed=96, init_state="fp32")
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = new_workspace(x.T, x.H, x.N)
    g = torch.Generator(device="cuda").manual_seed(7)
    ws[256:] = torch.randint(0, 256, (ws.numel() - 256,), dtype=torch.uint8, device="cuda",
                             generator=g)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    o2, f2 = _plain(x, d)
    _same_bits(out, o2, "out")
    _same_bits(fin, f2, "final state")


def test_duo_in_place_state():
    """final_state aliasing initial_state."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([500, 900, 33], 12, seed=97, init_state="fp32")
    d = to_device(x)
    state = d["s0"].clone()
    out = torch.empty(x.T, x.H, D, dtype=torch.bfloat16, device="cuda")
    ws = _patterned_workspace(x)
    kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                              d["dt_bias"], x.lower_bound, x.scale, state, d["cu"], out, state, ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    oref, fref = run_oracle(x)
    assert_parity(x, out, state, oref, fref, label="two workgroups, in place")


def test_duo_strided_views():
    """The strided entry point takes the form too: q, k, v, g as views of one
    fused projection buffer, beta a strided column, out half of a wider
    buffer; bit for bit the dense call, and against the oracle."""
    import torch
    from test_strided_gpu import SENTINEL, _strided_views
    x = KI.make_inputs([1000, 700, 300], 12, seed=98, init_state="fp32")
    d = to_device(x)
    out_d, fin_d = run_gpu(x, d)
    sd, out_s, obuf = _strided_views(d, "fused_rows")
    _, fin_s, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    run_gpu(x, sd, out=out_s, fin=fin_s, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    _same_bits(out_s, out_d, "strided out")
    _same_bits(fin_s, fin_d, "strided state")
    assert bool((obuf[..., :128].view(torch.int16) == SENTINEL).all()), "wrote outside out"
    oref, fref = run_oracle(x)
    assert_parity(x, out_s, fin_s, oref, fref, label="two workgroups, strided views")


def test_duo_full_size_against_oracle():
    """4 x 2048 tokens, 16 heads (64 pairs, the automatic choice), fp32 initial
    state: every output and final-state element against the oracle."""
    import torch
    x = KI.make_inputs([2048] * 4, 16, seed=99, init_state="fp32")
    print(f"[case] duo 4x2048 h16 against the oracle", flush=True)
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label="two workgroups, 4x2048 h16")


def test_paths_without_the_form_give_its_bits():
    """40 pairs (5 sequences x 8 heads): the plain forward takes the
    two-workgroup form; the checkpoint entry point (interval 256) and the
    no-allocation entry point never do, and give the same out and final
    state bit for bit."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([1000, 700, 512, 1300, 256], 8, seed=100, init_state="fp32")
    print(f"[case] duo vs checkpoint and no-allocation paths", flush=True)
    d = to_device(x)
    out, fin, _ = alloc_outputs(x, d)
    ws = _patterned_workspace(x)
    run_gpu(x, d, out=out, fin=fin, ws=ws)
    torch.cuda.synchronize()
    assert _ran_duo(ws, x)
    ck = torch.empty(x.T // 256, x.H, D, D, dtype=torch.float32, device="cuda")  # the capacity asked for
    out_c, fin_c, ws_c = alloc_outputs(x, d)
    kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                              x.lower_bound, x.scale, d["s0"], d["cu"], out_c, fin_c, ws_c,
                              checkpoints=ck, checkpoint_interval=256)
    out_n, fin_n, _ = alloc_outputs(x, d)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.kda_chunk_prefill_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                      d["dt_bias"], x.lower_bound, x.scale, d["s0"], d["cu"],
                                      out_n, fin_n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for o, f, what in ((out_c, fin_c, "checkpoint call"), (out_n, fin_n, "no-allocation call")):
        _same_bits(o, out, f"{what} out")
        _same_bits(f, fin, f"{what} final state")
