"""GPU parity of kda_spec_decode_step (the speculative-decode step with
num_accepted_tokens rollback) against the fp64 oracle's reading of it
(oracle.kda_oracle_spec_step).

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import (MAX_ABS_BF16_STATE, MAX_ABS_FP32_STATE, MEAN_ABS, diff_stats, new_workspace,
                      to_device, to_f64)

pytestmark = pytest.mark.gpu

D = 128


def _case(lengths, heads, seed, stride, slots, state):
    x = KI.make_inputs(lengths, heads, seed=seed, init_state=None)
    rng = np.random.default_rng(seed + 1000)
    N = len(lengths)
    # distinct slots per sequence row (as a serving engine's slot table), and
    # some never named
    perm = rng.permutation(slots)[:N * stride].astype(np.int32)
    idx = perm.reshape(N, stride)
    acc = rng.integers(1, stride + 1, size=N).astype(np.int32)
    pool = (0.05 * rng.standard_normal((slots, heads, D, D))).astype(np.float32)
    if state == "bf16":
        pool = KI.f32_to_bf16_bits(pool)
    return x, idx, acc, pool


def _run_gpu(x, d, idx, acc, pool_np, state):
    import torch
    import gated_delta_rule_tok_amd as kda
    dev = d["q"].device
    if state == "bf16":
        pool = torch.from_numpy(pool_np.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        pool = torch.from_numpy(pool_np).to(dev)
    out = torch.empty(x.T, x.H, D, dtype=torch.bfloat16, device=dev)
    ws = new_workspace(x.T, x.H, x.N, dev)
    kda.kda_spec_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                             x.lower_bound, x.scale, pool, d["cu"],
                             torch.from_numpy(idx).to(dev), torch.from_numpy(acc).to(dev), out, ws)
    torch.cuda.synchronize()
    return out, pool


def _check(x, out, pool_gpu, pool_np, o_ref, p_ref, idx, state, label):
    import torch
    tol = MAX_ABS_BF16_STATE if state == "bf16" else MAX_ABS_FP32_STATE
    rows = np.concatenate([np.arange(x.cu_seqlens[i], x.cu_seqlens[i + 1]) for i in range(x.N)])
    so = diff_stats(to_f64(out)[rows], o_ref[rows])
    written = sorted({int(idx[n, i]) for n in range(x.N)
                      for i in range(min(idx.shape[1], int(x.cu_seqlens[n + 1] - x.cu_seqlens[n])))})
    sp = diff_stats(to_f64(pool_gpu)[written], p_ref[written])
    print(f"[parity] {label} out {so} states {sp} ({len(written)} slots)", flush=True)
    assert so["max_abs"] <= tol and so["mean_abs"] <= MEAN_ABS, f"{label} out: {so}"
    assert sp["max_abs"] <= tol and sp["mean_abs"] <= MEAN_ABS, f"{label} states: {sp}"
    # every slot the step does not name keeps its bits
    untouched = [s for s in range(pool_np.shape[0]) if s not in set(written)]
    g = pool_gpu.view(torch.int16 if state == "bf16" else torch.int32).cpu().numpy()
    ref = pool_np.view(np.int16 if state == "bf16" else np.int32)
    assert np.array_equal(g[untouched], ref[untouched]), f"{label}: a slot not named was written"


@pytest.mark.parametrize("state", ["fp32", "bf16"])
@pytest.mark.parametrize("lengths", [[1, 2, 3, 4, 0, 4, 1], [4] * 12])
def test_spec_step_matches_oracle(lengths, state):
    import oracle
    x, idx, acc, pool = _case(lengths, 3, seed=71, stride=4, slots=64, state=state)
    print(f"[case] spec step lengths={lengths} state={state}", flush=True)
    d = to_device(x)
    out, pool_gpu = _run_gpu(x, d, idx, acc, pool, state)
    o_ref, p_ref = oracle.kda_oracle_spec_step(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log,
                                               x.dt_bias, x.lower_bound, x.scale, pool,
                                               x.cu_seqlens, idx, acc)
    _check(x, out, pool_gpu, pool, o_ref, p_ref, idx, state, f"spec step {state}")


def test_spec_steps_roll_back_across_calls():
    """Two steps in a row: the second starts from the states the first stored,
    at the accepted counts it is given (the pool stays on the device)."""
    import torch
    import oracle
    x1, idx, acc0, pool = _case([4, 3, 4, 2], 2, seed=72, stride=4, slots=40, state="fp32")
    d1 = to_device(x1)
    out1, pool_gpu = _run_gpu(x1, d1, idx, acc0, pool, "fp32")
    o1, p1 = oracle.kda_oracle_spec_step(x1.q, x1.k, x1.v, x1.g, x1.beta_logits, x1.A_log,
                                         x1.dt_bias, x1.lower_bound, x1.scale, pool,
                                         x1.cu_seqlens, idx, acc0)
    x2 = KI.make_inputs([3, 4, 1, 2], 2, seed=73, init_state=None)
    x2.A_log, x2.dt_bias = x1.A_log, x1.dt_bias
    acc1 = np.array([2, 3, 1, 2], np.int32)       # accepted prefixes of the first step
    d2 = to_device(x2)
    import gated_delta_rule_tok_amd as kda
    out2 = torch.empty(x2.T, x2.H, D, dtype=torch.bfloat16, device=pool_gpu.device)
    ws = new_workspace(x2.T, x2.H, x2.N, pool_gpu.device)
    kda.kda_spec_decode_step(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["A_log"],
                             d2["dt_bias"], x2.lower_bound, x2.scale, pool_gpu, d2["cu"],
                             torch.from_numpy(idx).to(pool_gpu.device),
                             torch.from_numpy(acc1).to(pool_gpu.device), out2, ws)
    torch.cuda.synchronize()
    o2, p2 = oracle.kda_oracle_spec_step(x2.q, x2.k, x2.v, x2.g, x2.beta_logits, x2.A_log,
                                         x2.dt_bias, x2.lower_bound, x2.scale, p1,
                                         x2.cu_seqlens, idx, acc1)
    rows = np.arange(x2.T)
    so = diff_stats(to_f64(out2)[rows], o2[rows])
    sp = diff_stats(to_f64(pool_gpu), p2)
    print(f"[parity] second step out {so} pool {sp}", flush=True)
    assert so["max_abs"] <= MAX_ABS_FP32_STATE and so["mean_abs"] <= MEAN_ABS, f"out: {so}"
    assert sp["max_abs"] <= MAX_ABS_FP32_STATE and sp["mean_abs"] <= MEAN_ABS, f"pool: {sp}"


@pytest.mark.parametrize("kernel,splits", [(0, (1, 2, 4, 8)), (2, (1, 2, 8))])
def test_spec_step_kernels_and_splits_bit_identical(kernel, splits):
    """The decode kernel at every value split, and the fp32 token-serial kernel,
    give the same bits."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x, idx, acc, pool = _case([2, 4, 3, 1], 2, seed=74, stride=4, slots=24, state="fp32")
    d = to_device(x)
    res = []
    prev = kda.kda_debug_set_kernel(kernel)
    try:
        for s in splits:
            kda.kda_debug_set_vsplit(s)
            out, pg = _run_gpu(x, d, idx, acc, pool, "fp32")
            res.append((out.view(torch.int16).cpu(), pg.cpu()))
    finally:
        kda.kda_debug_set_vsplit(0)
        kda.kda_debug_set_kernel(prev)
    for o, p in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(p, res[0][1])


def test_spec_step_rejects_chunked_kernel_override():
    import torch
    import gated_delta_rule_tok_amd as kda
    x, idx, acc, pool = _case([2, 1], 1, seed=75, stride=2, slots=4, state="fp32")
    d = to_device(x)
    prev = kda.kda_debug_set_kernel(4)
    try:
        with pytest.raises(kda.KdaError):
            _run_gpu(x, d, idx, acc, pool, "fp32")
    finally:
        kda.kda_debug_set_kernel(prev)
