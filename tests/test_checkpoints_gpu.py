"""GPU parity of kda_chunk_prefill_fwd_checkpoints: the state after every
`interval` tokens of each sequence, against the fp64 oracle.

The expected checkpoint (n, j) is the oracle's final state for the first
j * interval tokens of sequence n started from its initial state: the test
gathers those prefixes into one input set (one pseudo-sequence per checkpoint,
in slot order) and runs the plain oracle on it.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import (MAX_ABS_BF16_STATE, MAX_ABS_FP32_STATE, MEAN_ABS, alloc_outputs,
                      assert_parity, diff_stats, host_threads, run_gpu, run_oracle, to_device,
                      to_f64)

pytestmark = pytest.mark.gpu


def _oracle_checkpoints(x: KI.KdaInputs, interval: int) -> np.ndarray:
    """[C, H, 128, 128] fp64: state after each whole interval of each sequence."""
    import oracle
    spans = []  # (sequence, end token)
    for n in range(x.N):
        bos, eos = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        for j in range(1, (eos - bos) // interval + 1):
            spans.append((n, bos + j * interval))
    if not spans:
        return np.zeros((0, x.H, 128, 128))
    idx = np.concatenate([np.arange(int(x.cu_seqlens[n]), e) for n, e in spans])
    cu = np.concatenate([[0], np.cumsum([e - int(x.cu_seqlens[n]) for n, e in spans])]).astype(np.int32)
    s0 = None if x.initial_state is None else x.initial_state[[n for n, _ in spans]]
    _, fin = oracle.kda_oracle_fwd(x.q[idx], x.k[idx], x.v[idx], x.g[idx], x.beta_logits[idx],
                                   x.A_log, x.dt_bias, x.lower_bound, x.scale, s0, cu,
                                   threads=host_threads())
    return fin


def _run_ck(x, d, interval, capacity, sentinel):
    import torch
    import gated_delta_rule_tok_amd as kda
    out, fin, ws = alloc_outputs(x, d)
    ck = torch.empty(capacity, x.H, 128, 128, dtype=d["state_dtype"], device=d["q"].device)
    ck.view(torch.int16 if d["state_dtype"] == torch.bfloat16 else torch.int32).fill_(sentinel)
    kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                              d["dt_bias"], x.lower_bound, x.scale, d["s0"], d["cu"], out, fin,
                              ws, checkpoints=ck, checkpoint_interval=interval)
    torch.cuda.synchronize()
    return out, fin, ck


@pytest.mark.parametrize("lengths, heads, state, interval", [
    ([100, 64, 300, 0, 129, 17], 2, "fp32", 64),
    ([100, 64, 300, 0, 129, 17], 2, "bf16", 64),
    ([96, 250, 33], 3, "fp32", 16),
    ([200, 1, 48, 160], 2, None, 48),
    ([8, 4, 0, 16], 4, "fp32", 16),        # decode-sized: still the pipelined kernel
    ([2048, 1500, 777, 64], 16, "fp32", 256),
])
def test_checkpoints_match_oracle(lengths, heads, state, interval):
    import torch
    x = KI.make_inputs(lengths, heads, seed=7, init_state=state)
    print(f"[case] checkpoints {lengths} H={heads} state={state} interval={interval}", flush=True)
    d = to_device(x)
    count = sum(L // interval for L in lengths)
    capacity = x.T // interval + 2          # more than needed: the tail must stay untouched
    sentinel = 0x3C00 if x.state_bf16 else 0x3F800000   # 1.0 bits, never a checkpoint value here
    out, fin, ck = _run_ck(x, d, interval, capacity, sentinel)
    oref, fref = run_oracle(x)
    assert_parity(x, out, fin, oref, fref, label="checkpoint call")
    cref = _oracle_checkpoints(x, interval)
    assert cref.shape[0] == count
    tol = MAX_ABS_BF16_STATE if x.state_bf16 else MAX_ABS_FP32_STATE
    if count:
        st = diff_stats(to_f64(ck[:count]), cref)
        print(f"[parity] checkpoints {st}", flush=True)
        assert st["max_abs"] <= tol and st["mean_abs"] <= MEAN_ABS, f"checkpoints: {st}"
    tail = ck[count:].view(torch.int16 if x.state_bf16 else torch.int32)
    assert bool((tail == sentinel).all()), "slots past the named checkpoints were written"
    # the same out and final state, bit for bit, as the plain forward call on
    # the pipelined kernel (decode-sized plain calls take the token-serial
    # decode kernel, which agrees with the oracle but not bit for bit)
    import gated_delta_rule_tok_amd as kda
    prev = kda.kda_debug_set_kernel(4)
    try:
        out2, fin2 = run_gpu(x, d)
        torch.cuda.synchronize()
    finally:
        kda.kda_debug_set_kernel(prev)
    rows = np.concatenate([np.arange(x.cu_seqlens[i], x.cu_seqlens[i + 1]) for i in range(x.N)])
    assert torch.equal(out[torch.from_numpy(rows).to(out.device)],
                       out2[torch.from_numpy(rows).to(out.device)])
    assert torch.equal(fin, fin2)
    # a sequence whose length is a multiple of the interval ends on a copy of
    # its final state
    slot = 0
    for n, L in enumerate(lengths):
        slot += L // interval
        if L and L % interval == 0:
            assert torch.equal(ck[slot - 1], fin[n])


def test_checkpoints_split_invariant():
    """Every value split gives the same checkpoints, bit for bit."""
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([300, 129, 64], 2, seed=3, init_state="fp32")
    d = to_device(x)
    res = []
    try:
        for s in (2, 4, 8):
            kda.kda_debug_set_vsplit(s)
            res.append(_run_ck(x, d, 64, x.T // 64, 0)[2])
    finally:
        kda.kda_debug_set_vsplit(0)
    assert all(torch.equal(res[0], r) for r in res[1:])


@pytest.mark.parametrize("layout", ["fused_rows", "per_head"])
def test_checkpoints_strided_match_dense_bitwise(layout):
    """The checkpoint entry point on strided views (its strides argument)
    gives the dense call's checkpoints, output and final state bit for bit."""
    import torch
    import gated_delta_rule_tok_amd as kda
    from test_strided_gpu import _strided_views
    x = KI.make_inputs([150, 66, 33, 1, 128], 3, seed=43, init_state="fp32")
    d = to_device(x)
    print(f"[case] checkpoints strided layout={layout} T={x.T} H={x.H}", flush=True)
    out_d, fin_d, ck_d = _run_ck(x, d, 32, x.T // 32, 0)
    sd, out_s, _ = _strided_views(d, layout)
    _, fin_s, ws = alloc_outputs(x, d)
    ck_s = torch.zeros_like(ck_d)
    kda.kda_chunk_prefill_fwd(sd["q"], sd["k"], sd["v"], sd["g"], sd["beta"], d["A_log"],
                              d["dt_bias"], x.lower_bound, x.scale, d["s0"], d["cu"], out_s,
                              fin_s, ws, checkpoints=ck_s, checkpoint_interval=32)
    torch.cuda.synchronize()
    assert torch.equal(ck_s, ck_d)
    assert torch.equal(fin_s, fin_d)
    rows = torch.from_numpy(np.concatenate([np.arange(x.cu_seqlens[i], x.cu_seqlens[i + 1])
                                            for i in range(x.N)])).to(out_d.device)
    assert torch.equal(out_s[rows], out_d[rows])
