"""fp64 CPU oracle for the KDA chunked-prefill forward -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and the GPU
library never calls it.

Contents
  kda_oracle.c   the token-by-token fp64 recurrence (the definition), built
                 with gcc into liboracle_kda.so and called through ctypes
  chunked.py     an independent fp64 numpy derivation of the same function in
                 the chunked (WY / UT) form; used to cross-check the recurrence

See kda_oracle.c for the equations and the passages of the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kda.so")

HEAD_DIM = 128


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_libs = {}


def load_library(path: str | None = None):
    """ctypes handle of a built oracle library (default: the one built here)."""
    if path is None:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
    if path not in _libs:
        lib = ctypes.CDLL(path)
        fn = lib.kda_oracle_fwd
        P = ctypes.c_void_p
        fn.argtypes = [P, P, P, P, P, P, P, ctypes.c_double, ctypes.c_double, P, ctypes.c_int,
                       P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
        fn.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def kda_oracle_fwd(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale,
                   initial_state, cu_seqlens, *, threads=None, library=None):
    """Run the fp64 recurrence.

    q, k, v, g      uint16 bf16 bit patterns, shape [T, H, 128]
    beta_logits     uint16 bf16 bit patterns, shape [T, H]
    A_log           float32 [H];  dt_bias float32 [H, 128]
    initial_state   None (zeros) or [N, H, 128, 128]: float32, uint16 bf16 bit
                    patterns, or float64
    cu_seqlens      int32 [N + 1]
    library         path of an alternative build of kda_oracle.c (tests only)
    Returns (out float64 [T, H, 128], final_state float64 [N, H, 128, 128]).
    """
    q, k, v, g = (_as(x, np.uint16) for x in (q, k, v, g))
    beta_logits = _as(beta_logits, np.uint16)
    A_log = _as(A_log, np.float32)
    dt_bias = _as(dt_bias, np.float32)
    cu = _as(cu_seqlens, np.int32)
    T, H, D = q.shape
    assert D == HEAD_DIM and k.shape == q.shape and v.shape == q.shape and g.shape == q.shape
    assert beta_logits.shape == (T, H) and A_log.shape == (H,) and dt_bias.shape == (H, D)
    N = cu.shape[0] - 1
    assert N >= 0 and (N == 0 or (cu[0] >= 0 and cu[-1] <= T and np.all(np.diff(cu) >= 0)))
    kind = 0
    if initial_state is not None:
        initial_state = np.ascontiguousarray(initial_state)
        kinds = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}
        if initial_state.dtype not in kinds:
            raise TypeError(f"initial_state dtype {initial_state.dtype} not supported")
        kind = kinds[initial_state.dtype]
        assert initial_state.shape == (N, H, D, D)
    out = np.zeros((T, H, D), np.float64)
    fin = np.zeros((N, H, D, D), np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = load_library(library).kda_oracle_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta_logits), _ptr(A_log), _ptr(dt_bias),
        float(lower_bound), float(scale), _ptr(initial_state), kind,
        _ptr(cu), H, N, _ptr(out), _ptr(fin), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    return out, fin


def kda_oracle_spec_step(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale,
                         state_pool, cu_seqlens, state_indices, num_accepted_tokens, *,
                         threads=None):
    """One speculative-decode step with num_accepted_tokens rollback, in fp64.

    The reading (vLLM PR #55737's report, "Implementation breakdown" item 4
    and the spec-decode discussion: the speculative tokens keep the per-token
    recurrent kernel with its num_accepted_tokens rollback): sequence n starts
    from pool slot state_indices[n][num_accepted_tokens[n] - 1] (the zero
    state if that count or slot is out of range), runs the recurrence over its
    tokens, and the state after its i-th token goes to slot
    state_indices[n][i] (nothing for a slot out of range or i past the row).

    Written as the definition: every state after token i is the final state
    of kda_oracle_fwd over the sequence's first i + 1 tokens from the start
    state; all start states are taken from the pool as it was before the
    step.  state_pool: [S, H, 128, 128] float32, float64 or uint16 bf16 bits.
    Returns (out float64 [T, H, 128], the pool after the step as float64).
    """
    q, k, v, g = (np.ascontiguousarray(x) for x in (q, k, v, g))
    beta_logits = np.ascontiguousarray(beta_logits)
    cu = np.asarray(cu_seqlens, np.int64)
    idx = np.asarray(state_indices, np.int64)
    acc = np.asarray(num_accepted_tokens, np.int64)
    N, stride = idx.shape
    pool = np.asarray(state_pool)
    if pool.dtype == np.uint16:
        pool = (pool.astype(np.uint32) << 16).view(np.float32)
    pool = pool.astype(np.float64)
    S, H = pool.shape[0], pool.shape[1]
    T = q.shape[0]
    out = np.zeros((T, H, HEAD_DIM), np.float64)
    new_pool = pool.copy()
    # one pseudo-sequence per (sequence, prefix length): the prefix's tokens,
    # started from the sequence's start state
    rows, lens, starts, dest = [], [], [], []
    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        a = int(acc[n])
        slot = int(idx[n, a - 1]) if 1 <= a <= stride else -1
        start = pool[slot] if 0 <= slot < S else np.zeros((H, HEAD_DIM, HEAD_DIM))
        for i in range(eos - bos):
            rows.append(np.arange(bos, bos + i + 1))
            lens.append(i + 1)
            starts.append(start)
            dest.append((n, i, bos))
    if not rows:
        return out, new_pool
    sel = np.concatenate(rows)
    pcu = np.zeros(len(lens) + 1, np.int32)
    pcu[1:] = np.cumsum(lens)
    o, fin = kda_oracle_fwd(q[sel], k[sel], v[sel], g[sel], beta_logits[sel], A_log, dt_bias,
                            lower_bound, scale, np.stack(starts), pcu, threads=threads)
    for m, (n, i, bos) in enumerate(dest):
        out[bos + i] = o[pcu[m + 1] - 1]       # the prefix's last token is token i
        if i < stride:
            slot = int(idx[n, i])
            if 0 <= slot < S:
                new_pool[slot] = fin[m]
    return out, new_pool
