"""GPU parity of kda_gate_proj (the gate / beta projections upstream of the
forward) against the fp64 reference oracle.proj.gate_proj.

Bounds, from the arithmetic (per element, from the reference's own values,
u = 2^-24): the GPU sums the K products of P in fp32, 32 per MFMA step, 8
steps per 256-wide quarter, then four quarters per 1024-wide slice, then the
slices, each in order, so no product passes through more than 256 + 3 +
K/1024 <= 256 + K/256 fp32 additions and the sum is off the exact one by at
most (256 + K/256) u sum|h w| (first order).  Two roundings to bf16 of
values that close differ by at most that plus one bf16 unit (taken at the
larger of the two values).  G's inputs are the kernel's own P, already off by
|dP| each: |dG| <= sum_j |dP_j| |w_b| + 128 u sum|P w_b| + one unit.  Nearly
every element is bit-identical to the reference (a flip needs the fp32 error
to straddle a bf16 rounding boundary, about 1 in 10^4 here); the tests also
require that of 99% of them.

PYTEST_DONT_REWRITE: failing asserts must not repr device tensors.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_inputs as KI
from gpu_util import assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

K, NAB, NB = 7168, 144, 1536   # the page's test shapes (12 heads of 128)


def _unit(x):
    """bf16 unit in the last place at |x| (8 significant bits)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def _inputs(M, seed, unit_outputs=False):
    """hidden N(0, 1) [M, K]; weights N(0, 1), or with unit_outputs scaled by
    1/sqrt(depth) so that P and G are N(0, 1) like the forward's g and beta
    logits."""
    rng = np.random.default_rng(seed)
    h = KI.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    sa, sb = (K ** -0.5, 128 ** -0.5) if unit_outputs else (1.0, 1.0)
    wab = KI.f32_to_bf16_bits((sa * rng.standard_normal((NAB, K))).astype(np.float32))
    wb = KI.f32_to_bf16_bits((sb * rng.standard_normal((NB, 128))).astype(np.float32))
    return h, wab, wb


def _dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run(h, wab, wb, ws=None):
    import torch
    import gated_delta_rule_tok_amd as kda
    M = h.shape[0]
    th, twab, twb = _dev(h, torch), _dev(wab, torch), _dev(wb, torch)
    p = torch.empty(M, NAB, dtype=torch.bfloat16, device="cuda")
    g = torch.empty(M, NB, dtype=torch.bfloat16, device="cuda")
    if ws is None:
        ws = torch.zeros(kda.kda_gate_proj_workspace_size(M, K, NAB), dtype=torch.uint8, device="cuda")
    kda.kda_gate_proj(th, twab, twb, p, g, ws)
    torch.cuda.synchronize()
    return p, g, ws, (th, twab, twb)


def _f64(t):
    import torch
    return t.to(torch.float64).cpu().numpy()


def _check(h, wab, wb, p_gpu, g_gpu, label, K_=K):
    from oracle import proj
    p, g, p_exact, _ = proj.gate_proj(h, wab, wb)
    hf, wabf, wbf = proj.bf16_to_f64(h), proj.bf16_to_f64(wab), proj.bf16_to_f64(wb)
    u = 2.0 ** -24
    pg, gg = _f64(p_gpu), _f64(g_gpu)
    dp, dg = np.abs(pg - p), np.abs(gg - g)
    p_bound = ((256 + K_ / 256) * u * (np.abs(hf) @ np.abs(wabf).T)
               + _unit(np.maximum(np.abs(p_exact), np.abs(pg))))
    g_bound = (dp[:, :128] @ np.abs(wbf).T + 128 * u * (np.abs(pg[:, :128]) @ np.abs(wbf).T)
               + _unit(np.maximum(np.abs(g), np.abs(gg))))
    same_p, same_g = float((dp == 0).mean()), float((dg == 0).mean())
    print(f"[parity] {label}: P max |d| {dp.max():.3g} (bound min {p_bound.min():.3g}), identical {same_p:.4f}; "
          f"G max |d| {dg.max():.3g}, identical {same_g:.4f}", flush=True)
    assert np.all(dp <= p_bound), f"{label}: P outside its bound"
    assert np.all(dg <= g_bound), f"{label}: G outside its bound"
    assert same_p >= 0.99 and same_g >= 0.99, f"{label}: too few identical elements"


@pytest.mark.parametrize("M", [1, 2, 8, 14, 16, 37])
def test_proj_matches_reference(M):
    h, wab, wb = _inputs(M, seed=100 + M)
    print(f"[case] projections M={M}", flush=True)
    p, g, ws, _ = _run(h, wab, wb)
    _check(h, wab, wb, p, g, f"M={M}")


@pytest.mark.parametrize("M,k,nab,nb", [(5, 1000, 136, 48), (17, 2056, 128, 16), (3, 8, 144, 1536)])
def test_proj_ragged_shapes(M, k, nab, nb):
    """hidden_dim not a multiple of the 1024-wide slice (nor of 256), n_ab not
    a multiple of 16, n_b not a multiple of 64, two token tiles, one slice of
    8, no beta rows: against the reference, with the same bounds."""
    import torch
    import gated_delta_rule_tok_amd as kda
    from oracle import proj
    rng = np.random.default_rng(130 + M)
    h = KI.f32_to_bf16_bits(rng.standard_normal((M, k), dtype=np.float32))
    wab = KI.f32_to_bf16_bits(rng.standard_normal((nab, k), dtype=np.float32))
    wb = KI.f32_to_bf16_bits(rng.standard_normal((nb, 128), dtype=np.float32))
    th, twab, twb = _dev(h, torch), _dev(wab, torch), _dev(wb, torch)
    p = torch.empty(M, nab, dtype=torch.bfloat16, device="cuda")
    g = torch.empty(M, nb, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.kda_gate_proj_workspace_size(M, k, nab), dtype=torch.uint8, device="cuda")
    kda.kda_gate_proj(th, twab, twb, p, g, ws)
    torch.cuda.synchronize()
    print(f"[case] projections M={M} K={k} n_ab={nab} n_b={nb}", flush=True)
    _check(h, wab, wb, p, g, f"M={M} K={k} n_ab={nab} n_b={nb}", K_=k)


def test_proj_deterministic_and_workspace_reusable():
    """Calls on one workspace give the same bits, also after a call with more
    tokens in between, and on a workspace full of garbage (it needs no
    initialisation)."""
    import torch
    import gated_delta_rule_tok_amd as kda
    ws = torch.zeros(kda.kda_gate_proj_workspace_size(37, K, NAB), dtype=torch.uint8, device="cuda")
    h, wab, wb = _inputs(14, seed=120)
    p1, g1, _, _ = _run(h, wab, wb, ws=ws)
    h2, _, _ = _inputs(37, seed=121)
    _run(h2, wab, wb, ws=ws)
    p2, g2, _, _ = _run(h, wab, wb, ws=ws)
    ws.fill_(0xFF)   # NaN patterns everywhere
    p3, g3, _, _ = _run(h, wab, wb, ws=ws)
    for p_, g_ in ((p2, g2), (p3, g3)):
        assert torch.equal(p1.view(torch.int16), p_.view(torch.int16))
        assert torch.equal(g1.view(torch.int16), g_.view(torch.int16))


def test_proj_graph_capture_replay():
    """Both kernels captured in a HIP graph (no memset nodes) and replayed
    three times, with eager work between the replays, each replay equal to
    the eager call."""
    import torch
    import gated_delta_rule_tok_amd as kda
    h, wab, wb = _inputs(8, seed=122)
    p0, g0, ws, (th, twab, twb) = _run(h, wab, wb)
    p = torch.empty_like(p0)
    g = torch.empty_like(g0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            kda.kda_gate_proj(th, twab, twb, p, g, ws, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        p.zero_()
        g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.view(torch.int16), p0.view(torch.int16)), f"replay {i}: P differs"
        assert torch.equal(g.view(torch.int16), g0.view(torch.int16)), f"replay {i}: G differs"
        _run(h, wab, wb)   # eager work between the replays


def test_proj_feeds_the_forward():
    """The projections' outputs go into the forward as they stand: G as g
    [M, 12, 128], P's columns 128..139 as the beta logits (a strided column
    slice).  Weights scaled so that P and G are of unit size, like the
    workloads' g and beta.  The GPU chain (projections, then the decode-sized
    forward on strided beta) against the oracle chain (reference projections,
    then the fp64 forward) on the same hidden states and weights."""
    import torch
    from oracle import proj
    M, H = 12, NB // 128
    h, wab, wb = _inputs(M, seed=123, unit_outputs=True)
    p_gpu, g_gpu, _, _ = _run(h, wab, wb)
    p_ref, g_ref, _, _ = proj.gate_proj(h, wab, wb)
    x = KI.make_inputs([4, 1, 7], H, seed=124, init_state="fp32")
    assert x.T == M
    # reference inputs of the forward: the oracle chain's g and beta logits
    x.g = proj.f64_to_bf16_bits(g_ref).reshape(M, H, 128)
    x.beta_logits = proj.f64_to_bf16_bits(p_ref[:, 128:128 + H])
    oref, fref = run_oracle(x)
    d = to_device(x)
    d["g"] = g_gpu.view(M, H, 128)
    d["beta"] = p_gpu[:, 128:128 + H]          # token stride 144, head stride 1
    out, fin = run_gpu(x, d)
    torch.cuda.synchronize()
    assert_parity(x, out, fin, oref, fref, label="projections into the forward")
