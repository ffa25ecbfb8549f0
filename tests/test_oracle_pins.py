"""Pins for the fp64 oracle (CPU only).

The oracle (oracle/kda_oracle.c) is the definition of the KDA forward that the
GPU path is held to, so it is itself checked against things other than itself:
hand-worked examples, closed forms, textbook reductions, an independent chunked
derivation, brute force with explicit matrices, and invariants of the
definition.  Each check is a function of the oracle entry point, so the
mutation test at the bottom can run the same checks against deliberately
broken builds of the oracle and show that every planted mistake is caught.

The recurrence is the one vLLM PR #55737's report names ("Features and
motivation"; the FlashKDA wrapper in "Key source snippets"): bounded gate
lower_bound * sigmoid(exp(A_log) * (g + dt_bias)), in-kernel q/k L2 norm, raw
beta logits, scale on q; read as S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
o_t = scale * S_t^T q_t.
"""
from __future__ import annotations

import json
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import kda_inputs as KI
import oracle
from oracle import chunked

D = 128
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
BF16_POS_INF = np.uint16(0x7F80)
BF16_NEG_INF = np.uint16(0xFF80)


def _bf16(x):
    return KI.f32_to_bf16_bits(np.asarray(x, np.float32))


def _w(bits):
    return KI.bf16_bits_to_f32(bits).astype(np.float64)


def _fwd(fwd, x, **kw):
    return fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias, x.lower_bound, x.scale,
               x.initial_state, x.cu_seqlens, **kw)


def _blank(T, H, N_lengths, lb=-5.0, scale=1.0):
    """All-zero input set with the given sequence lengths (fields then edited)."""
    x = KI.make_inputs(N_lengths, H, seed=0, init_state=None, lower_bound=lb, scale=scale)
    assert x.T == T
    for name in ("q", "k", "v", "g"):
        setattr(x, name, np.zeros_like(getattr(x, name)))
    x.beta_logits = np.zeros_like(x.beta_logits)
    x.A_log = np.zeros_like(x.A_log)
    x.dt_bias = np.zeros_like(x.dt_bias)
    return x


def _l2n(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


# ----------------------------------------------------------------------------
# checks: each returns None on success or a message describing the failure
# ----------------------------------------------------------------------------

def _sparse(vec_spec, fill=0.0):
    out = np.full(D, fill, np.float64)
    for c, val in vec_spec.items():
        out[int(c)] = val
    return out


def _logit_bits(v):
    if v == "inf":
        return BF16_POS_INF
    if v == "-inf":
        return BF16_NEG_INF
    return _bf16(np.array([float(v)]))[0]


def check_golden(fwd):
    """Hand-derived worked examples (tests/golden/hand_worked.json)."""
    spec = json.load(open(GOLDEN))
    for case in spec["cases"]:
        toks = case["tokens"]
        T = len(toks)
        q = np.zeros((T, 1, D), np.uint16)
        k, v, g = q.copy(), q.copy(), q.copy()
        bl = np.zeros((T, 1), np.uint16)
        for t, tok in enumerate(toks):
            q[t, 0] = _bf16(_sparse(tok["q"]))
            k[t, 0] = _bf16(_sparse(tok["k"]))
            v[t, 0] = _bf16(_sparse(tok["v"]))
            g[t, 0] = _bf16(_sparse(tok["g"], fill=tok["g_default"]))
            bl[t, 0] = _logit_bits(tok["beta_logit"])
        S0 = None
        if case["initial_state"] is not None:
            S0 = np.zeros((1, 1, D, D), np.float64)
            for r, row in case["initial_state"].items():
                for c, val in row.items():
                    S0[0, 0, int(r), int(c)] = val
        out, fin = fwd(q, k, v, g, bl, np.zeros(1, np.float32), np.zeros((1, D), np.float32),
                       case["lower_bound"], case["scale"], S0, np.array([0, T], np.int32))
        for t, exp in enumerate(case["expected_out"]):
            e = _sparse(exp)
            err = np.abs(out[t, 0] - e).max()
            if err > 1e-9:
                return f"{case['name']}: out[{t}] off by {err:.3e}"
        ef = np.zeros((D, D))
        for r, row in case["expected_final"].items():
            for c, val in row.items():
                ef[int(r), int(c)] = val
        err = np.abs(fin[0, 0] - ef).max()
        if err > 1e-9:
            return f"{case['name']}: final state off by {err:.3e}"
    return None


def check_gate_special_values(fwd):
    """Bounded gate at points where it has a closed value (beta = 0 exposes it).

    With beta = 0 and S0 = ones, one token leaves S[c][:] = a[c], so the decay is
    read straight off the final state.  Head 0: g + dt_bias = 0 -> sigmoid = 1/2;
    g = +256 -> sigmoid = 1; g = -256 -> sigmoid ~ 1e-111 (a = 1).  Head 1 uses
    A_log = log(log 3) and g = 1, so exp(A_log) * g = log 3 and sigmoid = 3/4.
    dt_bias[h][c] is distinct per head and channel, so a wrong index shows.
    """
    lb = -3.0
    x = _blank(1, 2, [1], lb=lb)
    x.beta_logits[:] = BF16_NEG_INF
    x.initial_state = np.ones((1, 2, D, D), np.float64)
    g = np.zeros((2, D), np.float32)
    dtb = np.zeros((2, D), np.float32)
    # head 0: channels 0..31 g=-dt_bias (x=0); 32..63 g=+256; 64..127 g=-256
    vals = np.linspace(-1.5, 1.5, 32).astype(np.float32)
    vals = KI.bf16_bits_to_f32(_bf16(vals))  # exact in bf16 and fp32
    g[0, :32] = vals
    dtb[0, :32] = -vals
    g[0, 32:64] = 256.0
    g[0, 64:] = -256.0
    # head 1: g = 1, dt_bias = 0, A_log = log(log 3)
    g[1, :] = 1.0
    x.g[0] = _bf16(g)
    x.dt_bias = dtb
    x.A_log = np.array([0.0, math.log(math.log(3.0))], np.float32)
    _, fin = _fwd(fwd, x)
    a0 = fin[0, 0, :, 0]
    a1 = fin[0, 1, :, 0]
    if np.abs(fin[0, 0] - a0[:, None]).max() != 0.0:
        return "decay is not constant along each key row"
    want0 = np.concatenate([np.full(32, math.exp(lb / 2)), np.full(32, math.exp(lb)),
                            np.ones(64)])
    if np.abs(a0 - want0).max() > 1e-15:
        return f"head 0 gate special values off by {np.abs(a0 - want0).max():.3e}"
    # A_log rounds to fp32 (rel 6e-8), which moves sigmoid by < 1e-8
    if np.abs(a1 - math.exp(0.75 * lb)).max() > 1e-8:
        return f"head 1 sigmoid(log 3) gate off by {np.abs(a1 - math.exp(0.75 * lb)).max():.3e}"
    return None


def check_pure_decay(fwd):
    """beta = 0 (logit -inf): S_T = Diag(prod_t a_t) S0 and o_t follows it.

    Gate arguments take only the values 0, +256, -256 (A_log = dt_bias = 0), so
    each per-token decay is exactly exp(lb/2), exp(lb) or 1.
    """
    rng = np.random.default_rng(11)
    lb = -0.75
    T, H = 7, 2
    x = _blank(T, H, [3, 4], lb=lb, scale=0.7)
    x.beta_logits[:] = BF16_NEG_INF
    choice = rng.integers(0, 3, size=(T, H, D))
    gvals = np.array([0.0, 256.0, -256.0])[choice]
    avals = np.array([math.exp(lb / 2), math.exp(lb), 1.0])[choice]
    x.g = _bf16(gvals)
    x.q = _bf16(rng.standard_normal((T, H, D)))
    x.k = _bf16(rng.standard_normal((T, H, D)))
    x.v = _bf16(rng.standard_normal((T, H, D)))
    S0 = rng.standard_normal((2, H, D, D))
    x.initial_state = S0
    out, fin = _fwd(fwd, x)
    qn = _l2n(_w(x.q))
    for n, (lo, hi) in enumerate([(0, 3), (3, 7)]):
        for h in range(H):
            P = np.ones(D)
            for t in range(lo, hi):
                P = P * avals[t, h]
                o = x.scale * (P[:, None] * S0[n, h]).T @ qn[t, h]
                if np.abs(out[t, h] - o).max() > 1e-13:
                    return f"pure-decay output off at t={t} h={h}"
            if np.abs(fin[n, h] - P[:, None] * S0[n, h]).max() > 1e-13:
                return f"pure-decay final state off at n={n} h={h}"
    return None


def check_rank1_closed_form(fwd):
    """lower_bound = 0 (no decay), one token: S = S0 - b k (k^T S0) + b k v^T."""
    x = KI.make_inputs([1, 1], 3, seed=21, init_state="fp32", lower_bound=0.0)
    x2 = KI.make_inputs([1, 1], 3, seed=21, init_state=None, lower_bound=0.0)
    out, fin = _fwd(fwd, x)
    out0, fin0 = _fwd(fwd, x2)
    b = 1.0 / (1.0 + np.exp(-_w(x.beta_logits)))
    kn, qn, v = _l2n(_w(x.k)), _l2n(_w(x.q)), _w(x.v)
    S0 = x.initial_state.astype(np.float64)
    for n in range(2):
        for h in range(3):
            t = n
            kk, bb = kn[t, h], b[t, h]
            # zero initial state: rank-1 write and o = scale * b (k.q) v
            if np.abs(fin0[n, h] - bb * np.outer(kk, v[t, h])).max() > 1e-15:
                return "rank-1 write from zero state off"
            o0 = x.scale * bb * (kk @ qn[t, h]) * v[t, h]
            if np.abs(out0[t, h] - o0).max() > 1e-15:
                return "rank-1 output from zero state off"
            S = S0[n, h] - bb * np.outer(kk, kk @ S0[n, h]) + bb * np.outer(kk, v[t, h])
            if np.abs(fin[n, h] - S).max() > 1e-14:
                return "one-token update from nonzero state off"
            if np.abs(out[t, h] - x.scale * S.T @ qn[t, h]).max() > 1e-14:
                return "one-token output from nonzero state off"
    return None


def check_orthonormal_overwrite(fwd):
    """Textbook delta-rule store: with no decay, beta = 1 and k = e_j, row j of
    the state becomes v exactly, the other rows are unchanged, and a query e_j
    reads back scale * v."""
    rng = np.random.default_rng(5)
    T = 4
    x = _blank(T, 1, [T], lb=0.0, scale=0.25)
    x.beta_logits[:] = BF16_POS_INF
    js = [3, 77, 3, 127]
    S = rng.standard_normal((1, 1, D, D)).astype(np.float32)
    x.initial_state = S
    Sref = S[0, 0].astype(np.float64).copy()
    for t, j in enumerate(js):
        kv = np.zeros(D)
        kv[j] = 64.0
        x.k[t, 0] = _bf16(kv)
        x.q[t, 0] = _bf16(kv)
        x.v[t, 0] = _bf16(rng.standard_normal(D))
    out, fin = _fwd(fwd, x)
    for t, j in enumerate(js):
        Sref[j] = _w(x.v[t, 0])
        # the 1e-6 inside the norm makes k_hat = 1 - 1.2e-10, not exactly 1
        if np.abs(out[t, 0] - 0.25 * _w(x.v[t, 0])).max() > 1e-9:
            return f"read-back after store {t} off"
    if np.abs(fin[0, 0] - Sref).max() > 1e-9:
        return "overwrite touched other rows or stored the wrong row"
    return None


def check_dense_bruteforce(fwd):
    """Explicit 128x128 matrices: S <- (I - b k k^T) @ Diag(a) @ S + b k v^T."""
    x = KI.make_inputs([5, 3], 2, seed=3, init_state="fp32")
    out, fin = _fwd(fwd, x)
    q, k, v, g = (_w(a) for a in (x.q, x.k, x.v, x.g))
    b = 1.0 / (1.0 + np.exp(-_w(x.beta_logits)))
    I = np.eye(D)
    for n in range(2):
        for h in range(2):
            S = x.initial_state[n, h].astype(np.float64)
            for t in range(x.cu_seqlens[n], x.cu_seqlens[n + 1]):
                lam = x.lower_bound / (1.0 + np.exp(-np.exp(np.float64(x.A_log[h]))
                                                    * (g[t, h] + x.dt_bias[h])))
                kn, qn = _l2n(k[t, h]), _l2n(q[t, h])
                S = (I - b[t, h] * np.outer(kn, kn)) @ np.diag(np.exp(lam)) @ S \
                    + b[t, h] * np.outer(kn, v[t, h])
                if np.abs(out[t, h] - x.scale * S.T @ qn).max() > 1e-13:
                    return f"dense brute force: output off at t={t} h={h}"
            if np.abs(fin[n, h] - S).max() > 1e-13:
                return f"dense brute force: final state off at n={n} h={h}"
    return None


def check_chunked_equals_recurrent(fwd):
    """Independent chunked (WY/UT) derivation agrees with the token recurrence."""
    for lengths, C in (([1, 63], 16), ([64, 65], 64), ([200], 3), ([17, 0, 40], 1),
                       ([130], 64)):
        x = KI.make_inputs(lengths, 2, seed=len(lengths) * 7 + C, init_state="fp32")
        out, fin = _fwd(fwd, x)
        o2, f2 = chunked.kda_chunked_fwd(_w(x.q), _w(x.k), _w(x.v), _w(x.g), _w(x.beta_logits),
                                         x.A_log.astype(np.float64),
                                         x.dt_bias.astype(np.float64), x.lower_bound, x.scale,
                                         x.initial_state.astype(np.float64), x.cu_seqlens,
                                         chunk=C)
        eo = np.abs(out - o2).max() / max(np.abs(out).max(), 1e-30)
        ef = np.abs(fin - f2).max() / max(np.abs(fin).max(), 1e-30)
        if eo > 1e-12 or ef > 1e-12:
            return f"chunked vs recurrent differ (lengths={lengths}, C={C}): {eo:.2e} {ef:.2e}"
    return None


def check_segment_split(fwd):
    """Checkpoint/resume: [0, m) then [m, T) from the handed-over state equals
    one pass, for chunk-aligned and unaligned m."""
    x = KI.make_inputs([300], 2, seed=9, init_state="fp32")
    out, fin = _fwd(fwd, x)
    for m in (64, 100, 1, 299):
        a = KI.make_inputs([300], 2, seed=9, init_state="fp32")
        a.cu_seqlens = np.array([0, m], np.int32)
        o1, f1 = _fwd(fwd, a)
        b = KI.make_inputs([300], 2, seed=9, init_state="fp32")
        b.initial_state = f1
        b.cu_seqlens = np.array([m, 300], np.int32)
        o2, f2 = _fwd(fwd, b)
        if not (np.array_equal(o1[:m], out[:m]) and np.array_equal(o2[m:], out[m:])
                and np.array_equal(f2, fin)):
            return f"segment split at {m} differs from one pass"
    return None


def check_linearity(fwd):
    """For fixed q, k, g, beta the map (V, S0) -> (out, final) is linear."""
    rng = np.random.default_rng(2)
    x = KI.make_inputs([40, 25], 2, seed=4, init_state=None)
    v = _w(x.v)
    mask = np.zeros(D, bool)
    mask[rng.permutation(D)[:64]] = True
    v1 = np.where(mask, v, 0.0)
    v2 = np.where(mask, 0.0, v)
    S1 = rng.standard_normal((2, 2, D, D))
    S2 = rng.standard_normal((2, 2, D, D))
    res = []
    for vv, SS in ((v1, S1), (v2, S2), (v1 + v2, S1 + S2), (2 * v1, 2 * S1)):
        x.v = _bf16(vv)
        x.initial_state = SS
        res.append(_fwd(fwd, x))
    (oa, fa), (ob, fb), (oc, fc), (od, fd) = res
    tol = 1e-13 * max(np.abs(fc).max(), 1.0)
    if np.abs(oc - oa - ob).max() > tol or np.abs(fc - fa - fb).max() > tol:
        return "not additive in (V, S0)"
    if np.abs(od - 2 * oa).max() > tol or np.abs(fd - 2 * fa).max() > tol:
        return "not homogeneous in (V, S0)"
    return None


def check_invariances(fwd):
    """Positive rescaling of q or k leaves results unchanged (L2 norm present);
    permuting heads or sequences permutes the results."""
    x = KI.make_inputs([30, 45, 20], 3, seed=8, init_state="fp32")
    out, fin = _fwd(fwd, x)
    y = KI.make_inputs([30, 45, 20], 3, seed=8, init_state="fp32")
    y.q = _bf16(4.0 * _w(y.q))
    y.k = _bf16(0.5 * _w(y.k))
    o2, f2 = _fwd(fwd, y)
    # only the 1e-6 inside the norm distinguishes the two (relative < 1e-7)
    if np.abs(o2 - out).max() > 1e-6 * np.abs(out).max() or \
            np.abs(f2 - fin).max() > 1e-6 * np.abs(fin).max():
        return "rescaling q/k changed the result (norm missing or wrong)"
    ph = np.array([2, 0, 1])
    z = KI.make_inputs([30, 45, 20], 3, seed=8, init_state="fp32")
    for name in ("q", "k", "v", "g"):
        setattr(z, name, np.ascontiguousarray(getattr(z, name)[:, ph]))
    z.beta_logits = np.ascontiguousarray(z.beta_logits[:, ph])
    z.A_log = np.ascontiguousarray(z.A_log[ph])
    z.dt_bias = np.ascontiguousarray(z.dt_bias[ph])
    z.initial_state = np.ascontiguousarray(z.initial_state[:, ph])
    o3, f3 = _fwd(fwd, z)
    if not (np.array_equal(o3, out[:, ph]) and np.array_equal(f3, fin[:, ph])):
        return "permuting heads does not permute results"
    # sequences in reverse order
    w = KI.make_inputs([30, 45, 20], 3, seed=8, init_state="fp32")
    segs = [(0, 30), (30, 75), (75, 95)][::-1]
    idx = np.concatenate([np.arange(a, b) for a, b in segs])
    for name in ("q", "k", "v", "g", "beta_logits"):
        setattr(w, name, np.ascontiguousarray(getattr(w, name)[idx]))
    w.initial_state = np.ascontiguousarray(w.initial_state[::-1])
    w.cu_seqlens = np.array([0, 20, 65, 95], np.int32)
    o4, f4 = _fwd(fwd, w)
    if not (np.array_equal(o4, out[idx]) and np.array_equal(f4, fin[::-1])):
        return "permuting sequences does not permute results"
    return None


CHECKS = [check_golden, check_gate_special_values, check_pure_decay, check_rank1_closed_form,
          check_orthonormal_overwrite, check_dense_bruteforce, check_chunked_equals_recurrent,
          check_segment_split, check_linearity, check_invariances]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check, oracle_mod):
    msg = check(oracle_mod.kda_oracle_fwd)
    assert msg is None, msg


# ----------------------------------------------------------------------------
# edge cases of the contract
# ----------------------------------------------------------------------------

def test_empty_sequences_keep_state(oracle_mod):
    x = KI.make_inputs([0, 5, 0], 2, seed=1, init_state="fp32", extra_tokens=3)
    out, fin = _fwd(oracle_mod.kda_oracle_fwd, x)
    assert np.array_equal(fin[0], x.initial_state[0].astype(np.float64))
    assert np.array_equal(fin[2], x.initial_state[2].astype(np.float64))
    assert not np.array_equal(fin[1], x.initial_state[1].astype(np.float64))
    assert np.all(out[5:] == 0.0)  # rows past the last sequence untouched


def test_zero_tokens(oracle_mod):
    x = KI.make_inputs([0, 0], 1, seed=1, init_state="bf16")
    out, fin = _fwd(oracle_mod.kda_oracle_fwd, x)
    assert out.shape == (0, 1, D)
    assert np.array_equal(fin, _w(x.initial_state))


def test_null_initial_state_is_zero(oracle_mod):
    x = KI.make_inputs([50, 14], 2, seed=6, init_state=None)
    o1, f1 = _fwd(oracle_mod.kda_oracle_fwd, x)
    x.initial_state = np.zeros((2, 2, D, D), np.float32)
    o2, f2 = _fwd(oracle_mod.kda_oracle_fwd, x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_threads_do_not_change_results(oracle_mod):
    x = KI.make_inputs([33, 70, 12, 1], 3, seed=2, init_state="fp32")
    a = oracle_mod.kda_oracle_fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                  x.lower_bound, x.scale, x.initial_state, x.cu_seqlens,
                                  threads=1)
    b = oracle_mod.kda_oracle_fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                  x.lower_bound, x.scale, x.initial_state, x.cu_seqlens,
                                  threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bf16_state_widens_exactly(oracle_mod):
    x = KI.make_inputs([10], 1, seed=3, init_state="bf16")
    o1, f1 = _fwd(oracle_mod.kda_oracle_fwd, x)
    x.initial_state = _w(x.initial_state)
    o2, f2 = _fwd(oracle_mod.kda_oracle_fwd, x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


# ----------------------------------------------------------------------------
# mutation test: plant plausible mistakes in a copy of the oracle (CPU only)
# ----------------------------------------------------------------------------

MUTANTS = {
    "decay_on_value_columns": ("S[c * D + j] *= a[c];", "S[c * D + j] *= a[j];"),
    "beta_dropped_from_write": ("+= b * k[c] * (v[j] - p[j]);", "+= k[c] * (v[j] - p[j]);"),
    "erase_sign_flipped": ("(v[j] - p[j])", "(v[j] + p[j])"),
    "sigmoid_sign_flipped": ("J->lower_bound / (1.0 + exp(-x))", "J->lower_bound / (1.0 + exp(x))"),
    "A_log_not_exponentiated": ("exp((double)J->A_log[h])", "((double)J->A_log[h])"),
    "dt_bias_head_ignored": ("J->dt_bias + (size_t)h * D", "J->dt_bias"),
    "k_not_normalised": ("k[c] *= rk;", "k[c] *= 1.0;"),
    "q_not_normalised": ("q[c] *= rq;", "q[c] *= 1.0;"),
    "output_transposed": ("o[j] += S[c * D + j] * q[c];", "o[j] += S[j * D + c] * q[c];"),
    "scale_dropped": ("o[j] *= J->scale;", "o[j] *= 1.0;"),
    "beta_logit_not_squashed": (
        "const double b = 1.0 / (1.0 + exp(-bf16_bits_to_double(J->beta_logits[(size_t)t * H + h])));",
        "const double b = bf16_bits_to_double(J->beta_logits[(size_t)t * H + h]);"),
    "gate_bound_dropped": ("const double lam = J->lower_bound / (1.0 + exp(-x));",
                           "const double lam = -1.0 / (1.0 + exp(-x));"),
    "erase_uses_undecayed_key_row": ("p[j] += S[c * D + j] * k[c];",
                                     "p[j] += S[c * D + j] * k[c] / a[c];"),
    "eps_too_large": ("#define KDA_ORACLE_EPS 1e-6", "#define KDA_ORACLE_EPS 1e-2"),
}


@pytest.mark.slow
def test_pins_catch_planted_mistakes(oracle_mod):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "kda_oracle.c")).read()
    tmp = tempfile.mkdtemp(prefix="kda_mutants_")
    try:
        survivors = []
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) >= 1, f"mutation site for {name} not found"
            c = os.path.join(tmp, f"{name}.c")
            so = os.path.join(tmp, f"{name}.so")
            open(c, "w").write(src.replace(old, new))
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                                   c, "-o", so, "-lm"])

            def fwd(*a, _so=so, **kw):
                return oracle_mod.kda_oracle_fwd(*a, library=_so, **kw)

            caught = []
            for chk in CHECKS:
                try:
                    m = chk(fwd)
                except Exception as e:  # a crash also counts as caught
                    m = repr(e)
                if m is not None:
                    caught.append(chk.__name__)
            if not caught:
                survivors.append(name)
        assert not survivors, f"mutants not caught by any pin: {survivors}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


# ---- the speculative-decode step (kda_oracle_spec_step) --------------------------

def _spec_inputs(lengths, heads, seed, slots):
    x = KI.make_inputs(lengths, heads, seed=seed, init_state=None)
    pool = (0.05 * np.random.default_rng(seed).standard_normal((slots, heads, D, D))).astype(np.float32)
    return x, pool


def test_spec_step_rollback_resumes_the_accepted_prefix():
    """Rollback: a step verifying 4 draft tokens stores the state after each;
    the next step, told that 2 were accepted, continues from the state after
    the second.  Its output and states must equal the plain forward over the
    accepted history (2 tokens of the first step, then the second step's)."""
    x1, pool = _spec_inputs([4, 3], 2, seed=61, slots=10)
    idx = np.array([[0, 1, 2, 3, 8], [4, 5, 6, 7, 9]], np.int32)
    acc0 = np.array([5, 5], np.int32)       # both start from their last slot (8, 9)
    o1, pool1 = oracle.kda_oracle_spec_step(x1.q, x1.k, x1.v, x1.g, x1.beta_logits, x1.A_log,
                                            x1.dt_bias, x1.lower_bound, x1.scale, pool,
                                            x1.cu_seqlens, idx, acc0)
    x2 = KI.make_inputs([3, 2], 2, seed=62, init_state=None)
    acc1 = np.array([2, 3], np.int32)       # 2 of the first sequence's, 3 of the second's
    o2, pool2 = oracle.kda_oracle_spec_step(x2.q, x2.k, x2.v, x2.g, x2.beta_logits, x1.A_log,
                                            x1.dt_bias, x1.lower_bound, x1.scale, pool1,
                                            x2.cu_seqlens, idx, acc1)
    for n, (a, start_slot) in enumerate(((2, 8), (3, 9))):
        b1, b2 = int(x1.cu_seqlens[n]), int(x2.cu_seqlens[n])
        L2 = int(x2.cu_seqlens[n + 1]) - b2
        hist = lambda f1, f2: np.concatenate([f1[b1:b1 + a], f2[b2:b2 + L2]])
        cu = np.array([0, a + L2], np.int32)
        o, fin = oracle.kda_oracle_fwd(hist(x1.q, x2.q), hist(x1.k, x2.k), hist(x1.v, x2.v),
                                       hist(x1.g, x2.g), hist(x1.beta_logits, x2.beta_logits),
                                       x1.A_log, x1.dt_bias, x1.lower_bound, x1.scale,
                                       pool[start_slot][None].astype(np.float64), cu)
        np.testing.assert_allclose(o[:a], o1[b1:b1 + a], rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[a:], o2[b2:b2 + L2], rtol=0, atol=1e-12)
        np.testing.assert_allclose(pool2[idx[n, L2 - 1]], fin[0], rtol=0, atol=1e-12)


def test_spec_step_out_of_range_slots_and_counts():
    """An accepted count outside [1, S] or an out-of-range slot gives the zero
    start state; out-of-range destination slots and tokens past the row store
    nothing; a start slot among the sequence's own slots is read before the
    step writes it."""
    x, pool = _spec_inputs([3, 2, 3], 1, seed=63, slots=6)
    idx = np.array([[0, 1, -1], [2, 99, 3], [4, 5, 0]], np.int32)[:, :2]   # S = 2
    idx = np.ascontiguousarray(idx)
    acc = np.array([1, 0, 2], np.int32)     # seq 0 starts from slot 0 (its own first slot)
    o, p = oracle.kda_oracle_spec_step(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                       x.lower_bound, x.scale, pool, x.cu_seqlens, idx, acc)

    def run(n, start):
        b, e = int(x.cu_seqlens[n]), int(x.cu_seqlens[n + 1])
        outs, fins = [], []
        for i in range(e - b):
            oo, ff = oracle.kda_oracle_fwd(x.q[b:b + i + 1], x.k[b:b + i + 1], x.v[b:b + i + 1],
                                           x.g[b:b + i + 1], x.beta_logits[b:b + i + 1],
                                           x.A_log, x.dt_bias, x.lower_bound, x.scale,
                                           start[None], np.array([0, i + 1], np.int32))
            outs.append(oo[i])
            fins.append(ff[0])
        return outs, fins

    zero = np.zeros((1, D, D))
    o0, f0 = run(0, pool[0].astype(np.float64))       # slot 0 read before being overwritten
    o1, f1 = run(1, zero)                             # accepted count 0: zero state
    o2, f2 = run(2, pool[5].astype(np.float64))       # idx[2][1] = 5
    np.testing.assert_allclose(o[0:3], np.stack(o0), atol=1e-12, rtol=0)
    np.testing.assert_allclose(o[3:5], np.stack(o1), atol=1e-12, rtol=0)
    np.testing.assert_allclose(o[5:8], np.stack(o2), atol=1e-12, rtol=0)
    np.testing.assert_allclose(p[0], f0[0], atol=1e-12, rtol=0)   # seq 0, token 0
    np.testing.assert_allclose(p[1], f0[1], atol=1e-12, rtol=0)   # token 1; token 2 has no slot
    np.testing.assert_allclose(p[2], f1[0], atol=1e-12, rtol=0)   # seq 1 token 0; slot 99 ignored
    np.testing.assert_allclose(p[4], f2[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(p[5], f2[1], atol=1e-12, rtol=0)
    np.testing.assert_array_equal(p[3], pool[3].astype(np.float64))  # never named: untouched


# ---- the gate / beta projections (oracle.proj) --------------------------------------

def _bits(x):
    from oracle import proj
    return proj.f64_to_bf16_bits(np.asarray(x, np.float64))


def test_proj_round_bf16_against_brute_force():
    """round_bf16 is the nearest bf16 value (ties to even), checked against a
    search over every finite bf16 value near each input."""
    from oracle import proj
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-3, 4, 300),
                         [257.0, 259.0, 1444.0, -257.0, 0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]])
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    allbits = allbits[(allbits & 0x7F80) != 0x7F80]   # drop infinities and NaNs
    vals = proj.bf16_to_f64(allbits)
    for x in xs:
        d = np.abs(vals - x)
        best = d.min()
        cands = vals[d == best]
        if len(cands) > 1:   # a tie: the candidate with an even last significand bit
            cb = allbits[d == best]
            cands = cands[(cb & 1) == 0]
        assert proj.round_bf16(np.array([x]))[0] == cands[0], x


def test_proj_hand_worked():
    """One token, K = 8, hidden = 1..8; rows of w_ab and w_b chosen so every
    value is worked out by hand:
      P[0] = sum 1..8 = 36;  P[1] = 32 * 36 = 1152 (exact in bf16);
      P[2] = 255 * 1 + 1 * 2 = 257 -> 256 (halfway between 256 and 258: even);
      P[3] = 255 * 1 + 2 * 2 = 259 -> 260 (halfway between 258 and 260: even);
      P[128] = 8 (last channel), P[129] = 1-2+3-4+5-6+7-8 = -4; other rows 0.
      G[j] = P[j] for j < 4 (unit rows of w_b);
      G[14] = P[3] - P[2] = 260 - 256 = 4;
      G[15] = P[0] + P[1] + P[2] = 36 + 1152 + 256 = 1444 -> 1440 (bf16 spacing
      8 at 2^10; 1444 is halfway between 1440 and 1448: even)."""
    from oracle import proj
    K = 8
    hidden = np.arange(1, K + 1, dtype=np.float64)[None]
    wab = np.zeros((130, K))
    wab[0] = 1.0
    wab[1] = 32.0
    wab[2, 0], wab[2, 1] = 255.0, 1.0            # 257 is not a bf16 value: two terms
    wab[3, 0], wab[3, 1] = 255.0, 2.0            # 255 + 4 = 259
    wab[128, K - 1] = 1.0
    wab[129] = [1, -1, 1, -1, 1, -1, 1, -1]
    wb = np.zeros((16, 128))
    for j in range(4):
        wb[j, j] = 1.0
    wb[14, 3], wb[14, 2] = 1.0, -1.0
    wb[15, 0] = wb[15, 1] = wb[15, 2] = 1.0
    p, g, p_exact, g_exact = proj.gate_proj(_bits(hidden), _bits(wab), _bits(wb))
    want_p = np.zeros(130)
    want_p[[0, 1, 2, 3, 128, 129]] = [36, 1152, 256, 260, 8, -4]
    np.testing.assert_array_equal(p[0], want_p)
    assert p_exact[0, 2] == 257 and p_exact[0, 3] == 259
    want_g = np.zeros(16)
    want_g[[0, 1, 2, 3, 14, 15]] = [36, 1152, 256, 260, 4, 1440]
    np.testing.assert_array_equal(g[0], want_g)
    assert g_exact[0, 15] == 1444


def test_proj_brute_force_small_integers():
    """Small integers (every sum exact in bf16) against plain Python loops."""
    from oracle import proj
    rng = np.random.default_rng(5)
    M, K, nab, nb = 3, 16, 136, 32
    h = rng.integers(-3, 4, (M, K)).astype(np.float64)
    wab = rng.integers(-2, 3, (nab, K)).astype(np.float64)
    wb = np.zeros((nb, 128))
    wb[:, :6] = rng.integers(-1, 2, (nb, 6))
    p, g, _, _ = proj.gate_proj(_bits(h), _bits(wab), _bits(wb))
    for m in range(M):
        for n in range(nab):
            assert p[m, n] == sum(h[m, k] * wab[n, k] for k in range(K))
        for n in range(nb):
            assert g[m, n] == sum(p[m, j] * wb[n, j] for j in range(128))


def test_segment_maps_compose_to_the_one_pass_result(oracle_mod):
    """The algebra of the segment-parallel schedule, in the oracle's fp64: the
    recurrence is affine in the state, so a segment maps its entering state S
    to P S + R, with P the segment run from the identity with zero values and
    R the segment run from zero with its values.  Chaining S_{j+1} = P_j S_j +
    R_j over the segments gives each segment's end state as a rerun from S_j
    computes it, and the one-pass final state; the reruns' outputs are the
    one-pass outputs.  Weak decay (lower_bound -0.3) keeps P far from zero, and
    the segment bounds are not multiples of 16."""
    x = KI.make_inputs([97], 2, seed=90, init_state="fp32", lower_bound=-0.3)
    H = x.H
    run = lambda sl, v, s0: oracle.kda_oracle_fwd(
        x.q[sl], x.k[sl], v[sl], x.g[sl], x.beta_logits[sl], x.A_log, x.dt_bias,
        x.lower_bound, x.scale, s0, np.array([0, sl.stop - sl.start], np.int32))
    out1, fin1 = oracle.kda_oracle_fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                       x.lower_bound, x.scale, x.initial_state, x.cu_seqlens)
    zeros_v = np.zeros_like(x.v)
    eye = np.broadcast_to(np.eye(128), (1, H, 128, 128)).copy()
    S = x.initial_state.astype(np.float64)[0]
    outs = np.zeros_like(out1)
    for a, b in ((0, 30), (30, 64), (64, 97)):
        sl = slice(a, b)
        _, P = run(sl, zeros_v, eye)
        _, R = run(sl, x.v, None)
        o_seg, S_end = run(sl, x.v, S[None])
        outs[sl] = o_seg
        S = np.einsum("hij,hjk->hik", P[0], S) + R[0]
        assert np.abs(P[0]).max() > 1e-3                      # the map carries the state
        np.testing.assert_allclose(S, S_end[0], rtol=0, atol=1e-12 * max(1.0, np.abs(S).max()))
    np.testing.assert_allclose(S, fin1[0], rtol=0, atol=1e-12 * max(1.0, np.abs(S).max()))
    np.testing.assert_allclose(outs, out1, rtol=0, atol=1e-12 * max(1.0, np.abs(out1).max()))
