"""GPU parity: kda_chunk_prefill_fwd (through the C ABI) against the fp64 oracle.

Every output element is compared: out for every token inside a sequence and
the whole final state, at the five workload shapes and at edge cases.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import (alloc_outputs, assert_parity, run_gpu, run_oracle, to_device, to_f64)

pytestmark = pytest.mark.gpu

_cache = {}


def _config(idx):
    if idx not in _cache:
        x = KI.config_inputs(idx)
        print(f"[case] config {idx} {x.meta['config']} T={x.T} H={x.H} N={x.N}", flush=True)
        _cache[idx] = (x, run_oracle(x))
    return _cache[idx]


@pytest.fixture(autouse=True)
def _auto_vsplit():
    import gated_delta_rule_tok_amd as kda
    kda.kda_debug_set_vsplit(0)
    yield
    kda.kda_debug_set_vsplit(0)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_config_parity(idx):
    x, (oref, fref) = _config(idx)
    d = to_device(x)
    out, fin = run_gpu(x, d)
    assert_parity(x, out, fin, oref, fref, label=f"config {idx}")


@pytest.mark.parametrize("kernel,splits", [(5, (1, 2, 4, 8)), (4, (2, 4, 8)), (1, (1, 2, 4, 8)),
                                           (3, (1, 2, 4, 8))])
@pytest.mark.parametrize("idx", [3, 0, 1])
def test_vsplit_bit_identical(idx, kernel, splits):
    """Splitting the value dimension over workgroups changes nothing, bit for
    bit: each value column's arithmetic is the same whatever the split.  The
    16-token kernel (4) takes splits of 2 and more; the 32-token kernel (5),
    the 64-token kernel (1) and the token-serial decode path (3) also run
    unsplit."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x, _ = _config(idx)
    d = to_device(x)
    res = {}
    prev = kda.kda_debug_set_kernel(kernel)
    try:
        for s in splits:
            kda.kda_debug_set_vsplit(s)
            o, f = run_gpu(x, d)
            torch.cuda.synchronize()
            res[s] = (o.view(torch.int16).cpu(), f.cpu())
    finally:
        kda.kda_debug_set_kernel(prev)
    s0 = splits[0]
    for s in splits[1:]:
        assert torch.equal(res[s][0], res[s0][0]), f"out differs with split {s}"
        assert torch.equal(res[s][1], res[s0][1]), f"final state differs with split {s}"


@pytest.mark.parametrize("case", ["config1", "config3", "ragged", "ranked"])
def test_fwd32_kernel_parity(case):
    """The 32-token kernel (the default for lower_bound < -5) matches the
    oracle on the workloads and on ragged batches: lengths that end mid-chunk
    and mid-half, one shorter than a chunk, an empty one, and more sequences
    than the kernel ranks itself (the order table is built by a kernel
    launched first)."""
    import gated_delta_rule_tok_amd as kda
    if case == "ragged":
        x = KI.make_inputs([700, 33, 0, 1, 257, 64, 95, 16], 1, seed=41, init_state="fp32")
        oref, fref = run_oracle(x)
    elif case == "ranked":
        lens = np.random.default_rng(43).integers(100, 600, 24).tolist()
        x = KI.make_inputs(lens, 5, seed=43, init_state="fp32")
        oref, fref = run_oracle(x)
    else:
        x, (oref, fref) = _config(int(case[-1]))
    d = to_device(x)
    prev = kda.kda_debug_set_kernel(5)
    try:
        out, fin = run_gpu(x, d)
    finally:
        kda.kda_debug_set_kernel(prev)
    assert_parity(x, out, fin, oref, fref, label=f"32-token kernel {case}")


@pytest.mark.parametrize("idx", [0, 1, 3])
def test_chunk64_kernel_parity(idx):
    """The 64-token chunk kernel (used for lower_bound < -5 and unsplit
    launches) matches the oracle on the workloads too."""
    import gated_delta_rule_tok_amd as kda
    x, (oref, fref) = _config(idx)
    d = to_device(x)
    prev = kda.kda_debug_set_kernel(1)
    try:
        out, fin = run_gpu(x, d)
    finally:
        kda.kda_debug_set_kernel(prev)
    assert_parity(x, out, fin, oref, fref, label=f"64-token config {idx}")


def test_forced_unsplit_launch():
    """A forced split of 1 runs the 64-token kernel; results stay in parity."""
    import gated_delta_rule_tok_amd as kda
    x, (oref, fref) = _config(3)
    d = to_device(x)
    kda.kda_debug_set_vsplit(1)
    out, fin = run_gpu(x, d)
    assert_parity(x, out, fin, oref, fref, label="forced split 1")


def test_repeat_calls_bit_identical():
    import torch
    x, _ = _config(0)
    d = to_device(x)
    o1, f1 = run_gpu(x, d)
    o2, f2 = run_gpu(x, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)


def test_null_initial_state_equals_zeros():
    import torch
    x = KI.make_inputs([100, 200], 2, seed=31, init_state=None)
    d = to_device(x)
    o1, f1 = run_gpu(x, d)
    z = torch.zeros(2, 2, 128, 128, dtype=torch.float32, device="cuda")
    o2, f2 = run_gpu(x, d, s0=z)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)


@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_in_place_state_update(state):
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([70, 130, 1], 3, seed=32, init_state=state)
    d = to_device(x)
    o1, f1 = run_gpu(x, d)
    s = d["s0"].clone()
    out, _, ws = alloc_outputs(x, d)
    kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                              d["dt_bias"], x.lower_bound, x.scale, s, d["cu"], out, s, ws)
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(s.view(torch.int16) if state == "bf16" else s,
                       f1.view(torch.int16) if state == "bf16" else f1)


def test_ragged_edges_and_untouched_tail():
    import torch
    lengths = [1, 63, 64, 65, 0, 127, 129, 5, 192, 2]
    x = KI.make_inputs(lengths, 3, seed=33, init_state="fp32", extra_tokens=7)
    print(f"[case] ragged {lengths} + 7 tail tokens, H=3", flush=True)
    d = to_device(x)
    out, fin, ws = alloc_outputs(x, d, fill_out=0x7FC1)  # NaN sentinel
    run_gpu(x, d, out, fin, ws)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label="ragged")
    tail = out.view(torch.int16)[int(x.cu_seqlens[-1]):]
    assert bool((tail == 0x7FC1).all()), "rows past the last sequence were written"
    # the empty sequence keeps its initial state exactly
    assert torch.equal(fin[4], d["s0"][4])


@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_zero_tokens_keeps_state(state):
    import torch
    x = KI.make_inputs([0, 0, 0], 2, seed=34, init_state=state)
    d = to_device(x)
    out, fin = run_gpu(x, d)
    torch.cuda.synchronize()
    a = fin.view(torch.int16) if state == "bf16" else fin
    b = d["s0"].view(torch.int16) if state == "bf16" else d["s0"]
    assert torch.equal(a, b)


@pytest.mark.parametrize("lb", [-1.0, -5.0, -5.5])
def test_lower_bound_range(lb):
    x = KI.make_inputs([150, 66], 2, seed=35, init_state="fp32", lower_bound=lb)
    d = to_device(x)
    out, fin = run_gpu(x, d)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"lb={lb}")


@pytest.mark.parametrize("lb", [-5.0, -5.5])
def test_saturated_gate(lb):
    """dt_bias = 8 drives every gate sigmoid to ~1, so each 16-token chunk decays
    by ~16 |lower_bound| log2(e) in log2 units: the widest exponent range the
    kernels' decayed operands see (lower_bound -5 on the pipelined kernel, -5.5
    on the 64-token kernel)."""
    x = KI.make_inputs([150, 66], 2, seed=36, init_state="fp32", lower_bound=lb)
    x.dt_bias[:] = 8.0
    d = to_device(x)
    out, fin = run_gpu(x, d)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"saturated gate lb={lb}")


@pytest.mark.parametrize("lb", [0.0, -0.05])
def test_weak_or_no_decay(lb):
    """Without decay the state keeps growing (|S| ~8x the workloads' scale at
    216 tokens), so the bounds calibrated on the workloads do not apply; every
    bound is scaled by the reference's magnitude (max, mean and RMS)."""
    x = KI.make_inputs([150, 66], 2, seed=35, init_state="fp32", lower_bound=lb)
    d = to_device(x)
    out, fin = run_gpu(x, d)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label=f"lb={lb}", relative=True)


def test_bf16_state_small():
    x = KI.make_inputs([300, 45, 64], 4, seed=36, init_state="bf16")
    d = to_device(x)
    out, fin = run_gpu(x, d)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label="bf16 state")


def test_graph_capture_replay_matches_eager():
    import torch
    x = KI.make_inputs([200, 64, 300], 4, seed=37, init_state="fp32")
    d = to_device(x)
    eo, ef = run_gpu(x, d)
    torch.cuda.synchronize()
    out, fin, ws = alloc_outputs(x, d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run_gpu(x, d, out, fin, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eo.view(torch.int16)), f"replay {rep} out"
        assert torch.equal(fin, ef), f"replay {rep} final state"
        run_gpu(x, d)  # eager work between replays
        torch.cuda.synchronize()


def test_invalid_arguments_raise():
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([10], 1, seed=38, init_state="fp32")
    d = to_device(x)
    out, fin, ws = alloc_outputs(x, d)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                  d["dt_bias"], 0.5, x.scale, d["s0"], d["cu"], out, fin, ws)
    assert e.value.status == 2
    with pytest.raises(TypeError):
        kda.kda_chunk_prefill_fwd(d["q"].float(), d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                  d["dt_bias"], -5.0, x.scale, d["s0"], d["cu"], out, fin, ws)
    small = torch.empty(0, dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                  d["dt_bias"], -5.0, x.scale, d["s0"], d["cu"], out, fin, small)
    assert e.value.status == 3


@pytest.mark.parametrize("idx", [0, 3])
def test_token_serial_kernel_parity(idx):
    """The second, token-serial GPU implementation also matches the oracle."""
    import gated_delta_rule_tok_amd as kda
    x, (oref, fref) = _config(idx)
    d = to_device(x)
    prev = kda.kda_debug_set_kernel(2)
    try:
        out, fin = run_gpu(x, d)
    finally:
        kda.kda_debug_set_kernel(prev)
    assert_parity(x, out, fin, oref, fref, label=f"token-serial config {idx}")


@pytest.mark.parametrize("lengths,state,lb", [
    ([1] * 96, "fp32", -5.0),                 # decode: one token per sequence
    ([2, 3, 0, 2, 1] * 12, "bf16", -5.5),     # speculative-decode-sized, empty ones too
    ([1] * 40 + [30], "fp32", -1.0),          # decode-sized on average, one longer sequence
    ([4, 3, 8, 1] * 10, "fp32", -5.0),        # multi-token decode steps
    ([12, 9, 11] * 10, "fp32", -5.0),         # above the decode threshold: pipelined
])
def test_decode_sized_calls(lengths, state, lb):
    """At most 8 tokens per sequence on average: the automatic choice is the
    decode kernel (token-serial with 16-byte state accesses); both it and the
    pipelined kernel match the oracle from a nonzero initial state, and so does
    the automatic choice above the threshold."""
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs(lengths, 4, seed=43, init_state=state, lower_bound=lb)
    print(f"[case] decode-sized N={x.N} T={x.T} state={state} lb={lb}", flush=True)
    oref, fref = run_oracle(x)
    d = to_device(x)
    for kernel in (0, 4):
        prev = kda.kda_debug_set_kernel(kernel)
        try:
            out, fin = run_gpu(x, d)
        finally:
            kda.kda_debug_set_kernel(prev)
        assert_parity(x, out, fin, oref, fref, label=f"decode-sized kernel {kernel}")


def _bf16_bits(vals):
    return KI.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _degenerate_inputs():
    """A ragged batch with the method's degenerate rows: all-zero q rows, all-zero
    k rows (normalised to zero: the eps under the root keeps them finite), beta
    logits of +inf and -inf (beta exactly 1 and 0) and gate inputs of +-256
    (the sigmoid saturated: decay exactly e^lower_bound or none)."""
    x = KI.make_inputs([150, 1, 47, 0, 96, 33], 3, seed=51, init_state="fp32")
    rng = np.random.default_rng(52)
    T = x.T
    zq = rng.choice(T, 20, replace=False)
    zk = rng.choice(T, 20, replace=False)
    x.q[zq] = 0
    x.k[zk] = 0
    x.k[zq[:3]] = 0                       # some rows with both q and k zero
    binf = rng.choice(T, 30, replace=False)
    x.beta_logits[binf[:15], 0] = _bf16_bits(np.inf)
    x.beta_logits[binf[15:], 1] = _bf16_bits(-np.inf)
    x.beta_logits[binf[:5], 2] = _bf16_bits(-np.inf)
    gt = rng.choice(T, 40, replace=False)
    x.g[gt[:20], :, :64] = _bf16_bits(256.0)
    x.g[gt[20:], :, 64:] = _bf16_bits(-256.0)
    x.g[gt[:10], 1, :] = _bf16_bits(-256.0)
    return x


@pytest.mark.parametrize("kernel", [0, 4, 5, 1, 2, 3])
def test_degenerate_rows(kernel):
    """Zero q / k rows, infinite beta logits and saturated gates, on every
    kernel family, against the oracle."""
    import gated_delta_rule_tok_amd as kda
    x = _degenerate_inputs()
    print(f"[case] degenerate rows kernel={kernel} T={x.T} H={x.H}", flush=True)
    d = to_device(x)
    oref, fref = run_oracle(x)
    assert np.isfinite(oref).all() and np.isfinite(fref).all()
    prev = kda.kda_debug_set_kernel(kernel)
    try:
        out, fin = run_gpu(x, d)
    finally:
        kda.kda_debug_set_kernel(prev)
    assert_parity(x, out, fin, oref, fref, label=f"degenerate rows kernel {kernel}")


@pytest.mark.parametrize("kernel", [0, 5])
@pytest.mark.parametrize("log2_scale", [10, 12, 14])
def test_large_values(log2_scale, kernel):
    """Values and initial state of magnitude 2^10 .. 2^14 (the range the
    header states for the fp16 state update): every bound relative to the
    reference's magnitude."""
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([150, 66, 200], 2, seed=53, init_state="fp32")
    f = np.float32(2.0 ** log2_scale)
    x.v[:] = KI.f32_to_bf16_bits(KI.bf16_bits_to_f32(x.v) * f)
    x.initial_state[:] = x.initial_state * (f / np.float32(0.02 * 4))
    print(f"[case] large values 2^{log2_scale} kernel={kernel}", flush=True)
    d = to_device(x)
    oref, fref = run_oracle(x)
    prev = kda.kda_debug_set_kernel(kernel)
    try:
        out, fin = run_gpu(x, d)
    finally:
        kda.kda_debug_set_kernel(prev)
    assert_parity(x, out, fin, oref, fref, label=f"|v| ~ 2^{log2_scale} kernel {kernel}",
                  relative=True)


def test_kernel_choice_by_batch_average():
    """The automatic choice goes by the batch's average length: the same
    30-token sequence is served by the token-serial decode kernel when it is
    batched with 40 one-token sequences (8 tokens per sequence or fewer on
    average) and by the pipelined kernel when it comes alone.  Both results
    follow the oracle; they need not be the same bits."""
    import torch
    big = KI.make_inputs([30] + [1] * 40, 2, seed=81, init_state="fp32")
    rows = np.arange(0, 30)
    alone = KI.make_inputs([30], 2, seed=81, init_state="fp32")
    # the same 30-token sequence, initial state and parameters in both calls
    for f in ("q", "k", "v", "g", "beta_logits"):
        setattr(alone, f, getattr(big, f)[:30].copy())
    alone.A_log, alone.dt_bias = big.A_log, big.dt_bias
    alone.initial_state = big.initial_state[:1].copy()
    assert big.T <= 8 * big.N and alone.T > 8 * alone.N
    res = {}
    for name, x in (("batched", big), ("alone", alone)):
        d = to_device(x)
        out, fin = run_gpu(x, d)
        torch.cuda.synchronize()
        oref, fref = run_oracle(x)
        assert_parity(x, out, fin, oref, fref, label=f"30-token sequence {name}")
        res[name] = (to_f64(out)[rows], to_f64(fin)[0])
    d = np.abs(res["batched"][0] - res["alone"][0]).max()
    print(f"[kernel choice] max |out batched - out alone| = {d:.3g}", flush=True)
