"""GPU: strided q/k/v/g/beta/out views (kda_chunk_prefill_fwd_strided, reached
through the binding) give the dense call's results bit for bit, on every kernel
family, and leave the rest of the output buffer untouched.

The strided entry point is the SURVEY "next" row f1: the pages' wrapper
listing (vLLM PR #55737's report, "Key source snippets") copies q, k, v, g to
dense tensors because FlashKDA fixes their strides, and its "Risks" list counts
the cost of those copies.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import alloc_outputs, assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F  # a bf16 NaN pattern that no kernel writes


def _strided_views(d, layout):
    """q, k, v, g as views into one projection-like buffer, beta as a column
    slice, out as half of a wider buffer."""
    import torch
    q = d["q"]
    T, H, D = q.shape
    if layout == "fused_rows":      # [T, 4 H 128]: q | k | v | g per token
        buf = torch.empty(T, 4 * H * D, dtype=q.dtype, device=q.device)
        views = [buf[:, i * H * D:(i + 1) * H * D].view(T, H, D) for i in range(4)]
    else:                           # [T, H, 4, 128]: q, k, v, g interleaved per head
        buf = torch.empty(T, H, 4, D, dtype=q.dtype, device=q.device)
        views = [buf[:, :, i, :] for i in range(4)]
    for view, name in zip(views, ("q", "k", "v", "g")):
        view.copy_(d[name])
    bbuf = torch.empty(T, 2 * H + 1, dtype=q.dtype, device=q.device)   # odd token stride
    beta = bbuf[:, 1:2 * H + 1:2]                                        # head stride 2
    beta.copy_(d["beta"])
    obuf = torch.empty(T, H, 2 * D, dtype=q.dtype, device=q.device)
    obuf.view(torch.int16).fill_(SENTINEL)
    out = obuf[..., D:]
    sd = dict(d, q=views[0], k=views[1], v=views[2], g=views[3], beta=beta)
    assert not all(t.is_contiguous() for t in (views[0], beta, out))
    return sd, out, obuf


@pytest.mark.parametrize("kernel", [4, 1, 2, 3])
@pytest.mark.parametrize("layout", ["fused_rows", "per_head"])
def test_strided_matches_dense_bitwise(kernel, layout):
    import torch
    import gated_delta_rule_tok_amd as kda
    x = KI.make_inputs([150, 66, 33, 1], 3, seed=41, init_state="fp32")
    d = to_device(x)
    print(f"[case] strided kernel={kernel} layout={layout} T={x.T} H={x.H}", flush=True)
    prev = kda.kda_debug_set_kernel(kernel)
    try:
        out_d, fin_d = run_gpu(x, d)
        sd, out_s, obuf = _strided_views(d, layout)
        _, fin_s, ws = alloc_outputs(x, d)
        run_gpu(x, sd, out=out_s, fin=fin_s, ws=ws)
        torch.cuda.synchronize()
    finally:
        kda.kda_debug_set_kernel(prev)
    assert torch.equal(out_s.view(torch.int16), out_d.view(torch.int16)), "out differs"
    assert torch.equal(fin_s, fin_d), "final state differs"
    untouched = obuf[..., :128].view(torch.int16)
    assert bool((untouched == SENTINEL).all()), "strided out wrote outside its rows"


def test_strided_parity_bf16_state_strong_bound():
    """Strided views on the bf16-state path with lower_bound -5.5 (the 64-token
    kernel), against the oracle."""
    import torch
    x = KI.make_inputs([200, 31], 2, seed=42, init_state="bf16", lower_bound=-5.5)
    d = to_device(x)
    sd, out_s, obuf = _strided_views(d, "per_head")
    _, fin_s, ws = alloc_outputs(x, d)
    run_gpu(x, sd, out=out_s, fin=fin_s, ws=ws)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out_s, fin_s, oref, fref, label="strided bf16 state lb=-5.5")
