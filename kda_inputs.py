"""Seeded synthetic inputs for the KDA chunked-prefill forward.

This module only draws random numbers and stores them in the dtypes the
operation takes (bf16 as 16-bit patterns, round-to-nearest-even from fp32).
It holds none of the method's arithmetic, and it is the one thing the oracle
side and the GPU side of the test suite share.

Workloads follow the shapes the pages measure: 8 sequences x 2048 tokens and
1 x 16384 tokens (vLLM PR #55737's report, "Features and motivation"), the
low-parallelism regime that triggers the value-dimension split (PR #52458's
report, "Features and motivation"), and fp32 / bf16 checkpoint state (PR
#56485's report, "Implementation breakdown").  head_dim is 128 throughout.

Recipe (numpy Generator(PCG64(seed)); seed = config index for the named
configurations).  Draw order is fixed:
    lengths (ragged configs only) -> q -> k -> v -> g -> beta_logits
    -> A_log -> dt_bias -> initial_state
    q, k, v, g       N(0, 1) fp32 -> bf16, shape [T, H, 128]
    beta_logits      N(0, 1) fp32 -> bf16, shape [T, H]
    A_log            log(U(1, 16)) fp32, shape [H]
    dt_bias          N(0, sd 0.1) fp32, shape [H, 128]
    initial_state    N(0, sd 0.02), fp32 or bf16, shape [N, H, 128, 128]
    lower_bound      -5.0;  scale = 128 ** -0.5
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
LOWER_BOUND = -5.0
SCALE = HEAD_DIM ** -0.5


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class KdaInputs:
    q: np.ndarray            # uint16 bf16 bits [T, H, 128]
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta_logits: np.ndarray  # uint16 bf16 bits [T, H]
    A_log: np.ndarray        # float32 [H]
    dt_bias: np.ndarray      # float32 [H, 128]
    initial_state: np.ndarray | None  # float32 or uint16 [N, H, 128, 128]
    cu_seqlens: np.ndarray   # int32 [N + 1]
    state_bf16: bool
    lower_bound: float = LOWER_BOUND
    scale: float = SCALE
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)


def make_inputs(lengths, heads, seed, *, init_state="fp32", state_bf16=None,
                lower_bound=LOWER_BOUND, scale=SCALE, extra_tokens=0,
                draw_lengths=None) -> KdaInputs:
    """Draw one input set.

    lengths        sequence lengths (ignored when draw_lengths is given)
    init_state     None (zero state, passed as NULL), "fp32" or "bf16"
    state_bf16     dtype of the final state; defaults to init_state == "bf16"
    extra_tokens   rows appended after the last sequence (not covered by any
                   sequence; the output there must stay untouched)
    draw_lengths   (count, lo, hi): draw lengths uniform in [lo, hi] first
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if draw_lengths is not None:
        cnt, lo, hi = draw_lengths
        lengths = rng.integers(lo, hi + 1, size=cnt)
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1]) + int(extra_tokens)
    H, D = int(heads), HEAD_DIM

    def bf16_normal(shape):
        return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))

    q = bf16_normal((T, H, D))
    k = bf16_normal((T, H, D))
    v = bf16_normal((T, H, D))
    g = bf16_normal((T, H, D))
    beta_logits = bf16_normal((T, H))
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal((H, D))).astype(np.float32)
    N = len(lengths)
    if init_state is None:
        init = None
    else:
        s = (0.02 * rng.standard_normal((N, H, D, D), dtype=np.float32)).astype(np.float32)
        init = f32_to_bf16_bits(s) if init_state == "bf16" else s
    if state_bf16 is None:
        state_bf16 = init_state == "bf16"
    if init is not None and (init.dtype == np.uint16) != bool(state_bf16):
        raise ValueError("initial and final state share one dtype")
    return KdaInputs(q, k, v, g, beta_logits, A_log, dt_bias, init, cu.astype(np.int32),
                     bool(state_bf16), float(lower_bound), float(scale),
                     meta={"seed": seed, "lengths": lengths.tolist() if N <= 64 else None})


# The five workloads.  Index 1 is the headline one (8 x 2048 tokens, 16 heads).
CONFIGS = {
    0: dict(name="tiny_1x256_h2", lengths=[256], heads=2, init_state=None, state_bf16=False),
    1: dict(name="varlen_8x2048_h16", lengths=[2048] * 8, heads=16, init_state="fp32",
            state_bf16=False),
    2: dict(name="long_1x16384_h16", lengths=[16384], heads=16, init_state=None,
            state_bf16=False),
    3: dict(name="vsplit_2x8192_h4", lengths=[8192] * 2, heads=4, init_state="fp32",
            state_bf16=False),
    4: dict(name="ragged_32x1to4096_h32_bf16state", lengths=None, heads=32,
            init_state="bf16", state_bf16=True, draw_lengths=(32, 1, 4096)),
}


def config_inputs(idx: int) -> KdaInputs:
    c = CONFIGS[idx]
    x = make_inputs(c["lengths"], c["heads"], seed=idx, init_state=c["init_state"],
                    state_bf16=c["state_bf16"], draw_lengths=c.get("draw_lengths"))
    x.meta["config"] = c["name"]
    return x
