"""GPU: kda_chunk_prefill_fwd_noalloc (no workspace: the order table in the
library's static device scratch) gives the results of kda_chunk_prefill_fwd
bit for bit, on two calls in a row, the second with a smaller input, both
with more sequences than the kernels rank themselves (so the scratch is
written and read).

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import pytest

import kda_inputs as KI
from gpu_util import alloc_outputs, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _noalloc(x, d):
    import torch
    import gated_delta_rule_tok_amd as kda
    dev = d["q"].device
    out = torch.empty(x.T, x.H, 128, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(x.N, x.H, 128, 128, dtype=d["state_dtype"], device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kda.kda_chunk_prefill_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                                      d["dt_bias"], x.lower_bound, x.scale, d["s0"], d["cu"], out,
                                      fin, status)
    return out, fin, status


@pytest.mark.parametrize("first,second", [((40, 3, 91), (20, 2, 92)), ((24, 2, 93), (5, 2, 94))])
def test_noalloc_matches_workspace_call(first, second):
    import torch
    for n, h, seed in (first, second):
        x = KI.make_inputs(None, h, seed=seed, init_state="fp32", draw_lengths=(n, 1, 300))
        print(f"[case] no-alloc N={x.N} H={x.H} T={x.T}", flush=True)
        d = to_device(x)
        out_a, fin_a, status = _noalloc(x, d)
        out_b, fin_b = run_gpu(x, d)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a kernel gave up a bounded wait"
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "out differs"
        assert torch.equal(fin_a, fin_b), "final state differs"


def test_noalloc_rejects_too_many_sequences():
    import torch
    import gated_delta_rule_tok_amd as kda
    lib = kda.load_library()
    fake = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = lib.kda_chunk_prefill_fwd_noalloc(*([fake.data_ptr()] * 7), -5.0, 0.088, None,
                                           fake.data_ptr(), fake.data_ptr(), fake.data_ptr(),
                                           fake.data_ptr(), None, 0, 2, 65537, 0)
    assert rc == 1  # KDA_ERR_INVALID_ARG, before any HIP call
