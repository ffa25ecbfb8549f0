"""GPU: strided q/k/v/g/beta/out views (kda_chunk_prefill_fwd_strided, reached
through the binding) give the dense call's results bit for bit, on every kernel
family, and leave the rest of the output buffer untouched.

The pages' wrapper listing (vLLM PR #55737's report, "Key source snippets")
copies q, k, v, g to dense tensors because FlashKDA fixes their strides, and
its "Risks" list counts the cost of those copies; the strided entry point
takes the views as they are.

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


@pytest.mark.parametrize("kernel", [4, 5, 1, 2, 3])
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
    """Strided views on the bf16-state path with lower_bound -5.5 (the 32-token
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


def test_strided_headline_workload_matches_oracle():
    """The 8 x 2048, H = 16 workload as a caller holding a fused projection
    output would pass it: q, k, v, g as views into one [T, 4 H 128] buffer,
    beta a strided column slice, out the second half of a wider buffer; the
    default kernel choice, every element against the oracle, and the first
    half of the output buffer untouched."""
    import torch
    x = KI.config_inputs(1)
    print(f"[case] strided headline T={x.T} H={x.H} N={x.N}", flush=True)
    d = to_device(x)
    sd, out_s, obuf = _strided_views(d, "fused_rows")
    _, fin_s, ws = alloc_outputs(x, d)
    run_gpu(x, sd, out=out_s, fin=fin_s, ws=ws)
    torch.cuda.synchronize()
    oref, fref = run_oracle(x)
    assert_parity(x, out_s, fin_s, oref, fref, label="strided 8x2048 H=16")
    untouched = obuf[..., :128].view(torch.int16)
    assert bool((untouched == SENTINEL).all()), "strided out wrote outside its rows"
