"""Helpers shared by the GPU tests: move seeded inputs to the device, call the
library through its binding, and compare with oracle results."""
from __future__ import annotations

import os

import numpy as np

import kda_inputs as KI

# tolerances of the checkpoint-state test the pages describe (PR #56485's
# report, "Implementation breakdown": 0.01 with fp32 state, 0.03 with bf16
# state), plus a mean-|delta| bound
MAX_ABS_FP32_STATE = 0.01
MAX_ABS_BF16_STATE = 0.03
MEAN_ABS = 1e-4


def host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def to_device(x: KI.KdaInputs, device="cuda"):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    d = dict(q=bf(x.q), k=bf(x.k), v=bf(x.v), g=bf(x.g), beta=bf(x.beta_logits),
             A_log=torch.from_numpy(x.A_log).to(device),
             dt_bias=torch.from_numpy(x.dt_bias).to(device),
             cu=torch.from_numpy(x.cu_seqlens).to(device))
    if x.initial_state is None:
        d["s0"] = None
    elif x.initial_state.dtype == np.uint16:
        d["s0"] = bf(x.initial_state)
    else:
        d["s0"] = torch.from_numpy(x.initial_state).to(device)
    d["state_dtype"] = torch.bfloat16 if x.state_bf16 else torch.float32
    return d


def alloc_outputs(x: KI.KdaInputs, d, fill_out=None):
    import torch
    import gated_delta_rule_tok_amd as kda
    dev = d["q"].device
    out = torch.empty(x.T, x.H, 128, dtype=torch.bfloat16, device=dev)
    if fill_out is not None:
        out.view(torch.int16).fill_(fill_out)
    fin = torch.empty(x.N, x.H, 128, 128, dtype=d["state_dtype"], device=dev)
    ws = new_workspace(x.T, x.H, x.N, dev)
    return out, fin, ws


# Every workspace the GPU tests hand to the library: its status word (the
# first 4 bytes) must still be zero when the test ends (no kernel gave up a
# bounded wait).  Checked by the autouse fixture in conftest.py.
_workspaces = []


def new_workspace(T, H, N, device="cuda"):
    import torch
    import gated_delta_rule_tok_amd as kda
    ws = torch.zeros(max(1, kda.kda_get_workspace_size(T, H, N)), dtype=torch.uint8, device=device)
    _workspaces.append(ws)
    return ws


def check_workspaces():
    """Assert the status word of every workspace used since the last check is 0."""
    import torch
    import gated_delta_rule_tok_amd as kda
    if not _workspaces:
        return
    torch.cuda.synchronize()
    bad = [kda.kda_workspace_status(ws) for ws in _workspaces]
    _workspaces.clear()
    assert not any(bad), f"a kernel gave up a bounded wait (status words {bad})"


def run_gpu(x: KI.KdaInputs, d, out=None, fin=None, ws=None, s0="default", stream=None):
    import gated_delta_rule_tok_amd as kda
    if out is None:
        out, fin, ws = alloc_outputs(x, d)
    kda.kda_chunk_prefill_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                              d["dt_bias"], x.lower_bound, x.scale,
                              d["s0"] if isinstance(s0, str) else s0, d["cu"], out, fin, ws,
                              stream=stream)
    return out, fin


def run_oracle(x: KI.KdaInputs):
    import oracle
    return oracle.kda_oracle_fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                 x.lower_bound, x.scale, x.initial_state, x.cu_seqlens,
                                 threads=host_threads())


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def diff_stats(gpu: np.ndarray, ref: np.ndarray) -> dict:
    if gpu.size == 0:
        return dict(max_abs=0.0, mean_abs=0.0, rel_rms=0.0, ref_max=0.0, ref_mean=0.0)
    d = np.abs(gpu - ref)
    a = np.abs(ref)
    return dict(max_abs=float(d.max()), mean_abs=float(d.mean()),
                rel_rms=float(np.sqrt((d * d).sum() / max((ref * ref).sum(), 1e-300))),
                ref_max=float(a.max()), ref_mean=float(a.mean()))


# Relative bounds for inputs far from the workloads' scale (weak or no decay,
# where the state keeps growing; values of large magnitude).  A bf16 rounding
# adds about 2^-9 / sqrt(3) = 1.1e-3 relative RMS error; an output carries
# three or four of them (its product's two operands and its own rounding),
# about 2-2.5e-3 in all, the fp32 state fewer.  The mean error relative to the
# mean magnitude is of the same size as the RMS ratio.  The bounds leave about
# 2x room:
#   max|d|  <= REL_MAX  * max|ref|
#   mean|d| <= REL_MEAN * mean|ref|
#   RMS(d)  <= REL_RMS  * RMS(ref)
REL_MAX = 1e-2
REL_MEAN = 5e-3
REL_RMS_OUT = 5e-3
REL_RMS_STATE = 3e-3


def assert_parity(x: KI.KdaInputs, out_gpu, fin_gpu, out_ref, fin_ref, label="", rows=None,
                  relative=False):
    """max|d| and mean|d| bounds on out (rows of tokens inside sequences) and on
    the final state.  relative=True scales every bound by the reference's own
    magnitude (REL_MAX, REL_MEAN, REL_RMS_*; the absolute max bound still
    holds where it is the looser one)."""
    tol = MAX_ABS_BF16_STATE if x.state_bf16 else MAX_ABS_FP32_STATE
    if rows is None:
        rows = np.concatenate([np.arange(x.cu_seqlens[i], x.cu_seqlens[i + 1])
                               for i in range(x.N)]) if x.N else np.arange(0)
    so = diff_stats(to_f64(out_gpu)[rows], out_ref[rows])
    sf = diff_stats(to_f64(fin_gpu), fin_ref)
    print(f"[parity] {label} out {so} final {sf}", flush=True)
    if relative:
        for st, rms, what in ((so, REL_RMS_OUT, "out"), (sf, REL_RMS_STATE, "final state")):
            assert st["max_abs"] <= max(tol, REL_MAX * st["ref_max"]), f"{label} {what}: {st}"
            assert st["mean_abs"] <= REL_MEAN * st["ref_mean"] + 1e-12, f"{label} {what}: {st}"
            assert st["rel_rms"] <= rms, f"{label} {what}: {st}"
        return so, sf
    assert so["max_abs"] <= tol and so["mean_abs"] <= MEAN_ABS, f"{label} out: {so}"
    assert sf["max_abs"] <= tol and sf["mean_abs"] <= MEAN_ABS, f"{label} final state: {sf}"
    return so, sf
