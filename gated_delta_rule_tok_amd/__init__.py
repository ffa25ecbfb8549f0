"""Python binding of libkda.so, the MI355X (gfx950) KDA chunked-prefill forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kda.h.  Tensors are torch tensors
used as device memory; the stream defaults to torch's current stream.  There
is no CPU fallback: if libkda.so is missing, every call raises.

    ws = torch.zeros(kda_get_workspace_size(T, H, N), dtype=torch.uint8, device="cuda")
    kda_chunk_prefill_fwd(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, scale,
                          initial_state, cu_seqlens, out, final_state, ws)

q, k, v, g, out and beta_logits may be strided views (channels contiguous, for
[T, H, 128] both strides multiples of 8 elements): they then go through
kda_chunk_prefill_fwd_strided, with no copy.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["kda_get_workspace_size", "kda_chunk_prefill_fwd", "kda_status_string",
           "kda_workspace_status",
           "kda_last_hip_error", "kda_debug_set_vsplit", "kda_debug_set_kernel", "kda_debug_set_segment", "kda_debug_segment_length", "kda_debug_two_workgroups", "kda_spec_decode_step", "kda_chunk_prefill_fwd_noalloc", "kda_gate_proj",
           "kda_gate_proj_workspace_size", "KdaError", "library_path", "load_library"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

HEAD_DIM = 128
KDA_OK = 0
KDA_STATE_FP32 = 0
KDA_STATE_BF16 = 1

_lib = None


class _Strides(ctypes.Structure):
    """kda_strides_t of include/kda.h (element strides)."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_token", "q_head", "k_token", "k_head", "v_token", "v_head", "g_token", "g_head",
        "beta_token", "beta_head", "out_token", "out_head")]


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so once; raises if it has not been built.

    torch's wheel carries its own HIP runtime (libamdhip64, SONAME
    libamdhip64.so.7, the same SONAME as the system ROCm copy).  torch is
    imported first so that its runtime is in the process before libkda.so is
    mapped: the dynamic loader then resolves libkda.so's libamdhip64.so.7 to
    that same copy.  Loading libkda.so first would bring in the system copy, and
    torch would then load a second HIP runtime that sees no device.
    """
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401  (see above: one HIP runtime per process)
        except ImportError:
            pass
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m gated_delta_rule_tok_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float)
        lib.kda_get_workspace_size.argtypes = [I64, I32, I32]
        lib.kda_get_workspace_size.restype = SZ
        lib.kda_chunk_prefill_fwd.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, P, P,
                                              I64, I32, I32, ctypes.c_int, SZ]
        lib.kda_chunk_prefill_fwd.restype = ctypes.c_int
        lib.kda_chunk_prefill_fwd_strided.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, P,
                                                      P, I64, I32, I32, ctypes.c_int, SZ,
                                                      ctypes.POINTER(_Strides)]
        lib.kda_chunk_prefill_fwd_strided.restype = ctypes.c_int
        lib.kda_chunk_prefill_fwd_checkpoints.argtypes = [
            P, P, P, P, P, P, P, F, F, P, P, P, P, P, P, I64, I32, I32, ctypes.c_int, SZ,
            ctypes.POINTER(_Strides), P, I32, I64]
        lib.kda_chunk_prefill_fwd_checkpoints.restype = ctypes.c_int
        lib.kda_chunk_prefill_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, P, P,
                                                      I64, I32, I32, ctypes.c_int]
        lib.kda_chunk_prefill_fwd_noalloc.restype = ctypes.c_int
        lib.kda_gate_proj_workspace_size.argtypes = [I32, I32, I32]
        lib.kda_gate_proj_workspace_size.restype = SZ
        lib.kda_gate_proj.argtypes = [P, P, P, P, P, P, SZ, P, I32, I32, I32, I32]
        lib.kda_gate_proj.restype = ctypes.c_int
        lib.kda_spec_decode_step.argtypes = [P, P, P, P, P, P, P, F, F, P, I64, P, P, I32, P, P,
                                             P, P, I64, I32, I32, ctypes.c_int, SZ]
        lib.kda_spec_decode_step.restype = ctypes.c_int
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_last_hip_error.argtypes = []
        lib.kda_last_hip_error.restype = ctypes.c_char_p
        lib.kda_debug_set_kernel.argtypes = [ctypes.c_int]
        lib.kda_debug_set_kernel.restype = ctypes.c_int
        lib.kda_debug_set_vsplit.argtypes = [ctypes.c_int]
        lib.kda_debug_set_vsplit.restype = ctypes.c_int
        lib.kda_debug_set_segment.argtypes = [ctypes.c_int]
        lib.kda_debug_set_segment.restype = ctypes.c_int
        lib.kda_debug_segment_length.argtypes = [I64, I32, I32]
        lib.kda_debug_segment_length.restype = I32
        lib.kda_debug_two_workgroups.argtypes = [I64, I32, I32, I32]
        lib.kda_debug_two_workgroups.restype = I32
        _lib = lib
    return _lib


def kda_get_workspace_size(max_tokens: int, heads: int, max_seqs: int) -> int:
    return int(load_library().kda_get_workspace_size(int(max_tokens), int(heads), int(max_seqs)))


def kda_workspace_status(workspace) -> int:
    """The workspace's status word (its first 4 bytes, see include/kda.h): 0 while
    every call that used it ran to completion normally; nonzero (the kind of
    wait, 1: LDS counters) once a kernel gave up a bounded wait (the outputs of
    that call are void).  Synchronises the device."""
    import torch
    return int(workspace[:4].view(torch.int32)[0].item())


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_last_hip_error() -> str:
    return load_library().kda_last_hip_error().decode()


def kda_debug_set_kernel(k: int) -> int:
    """Test hook: 0 automatic (default), 1 64-token kernel, 2 token-serial
    kernel, 3 token-serial kernel with decode staging, 4 pipelined 16-token
    kernel (where it applies), 5 pipelined 32-token kernel."""
    prev = load_library().kda_debug_set_kernel(int(k))
    if prev < 0:
        raise ValueError(f"invalid kernel selector {k}")
    return prev


def kda_debug_set_vsplit(s: int) -> int:
    """Test hook: force the value split (1, 2, 4, 8) or 0 for automatic."""
    prev = load_library().kda_debug_set_vsplit(int(s))
    if prev < 0:
        raise ValueError(f"invalid value split {s}")
    return prev


def kda_debug_set_segment(length: int) -> int:
    """Test hook: the segment-parallel schedule -- 0 automatic, 1 never, or
    segments of `length` tokens (a multiple of 16) where the call allows it."""
    prev = load_library().kda_debug_set_segment(int(length))
    if prev < 0:
        raise ValueError(f"invalid segment length {length}")
    return prev


def kda_debug_segment_length(num_tokens: int, heads: int, num_seqs: int) -> int:
    """The segment length a call of these sizes would use (0: one piece)."""
    return int(load_library().kda_debug_segment_length(int(num_tokens), int(heads), int(num_seqs)))


def kda_debug_two_workgroups(num_tokens: int, heads: int, num_seqs: int, cus: int = 256) -> bool:
    """Whether a call of these sizes (with the workspace's second part) runs
    the 16-token kernel in two workgroups per (sequence, head) on a device of
    cus compute units."""
    return bool(load_library().kda_debug_two_workgroups(int(num_tokens), int(heads), int(num_seqs),
                                                        int(cus)))


def _check(t, name, dtype, shape=None, strided=False):
    """Device pointer of t after the dtype/shape checks.  strided: the leading
    two strides may be anything non-negative (the last dim must be dense)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if strided:
        if t.numel() and (any(st < 0 for st in t.stride())
                          or (t.dim() == 3 and t.stride(2) != 1 and t.shape[2] > 1)):
            raise ValueError(f"{name} must have non-negative strides and contiguous channels")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")
    return t.data_ptr()


def _flat(t, name, shape):
    """t seen with `shape` without a copy: the library keeps only the data
    pointer, and a temporary copy would go back to torch's allocator before
    the queued kernel reads it."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (its data is read in place)")
    if t.numel() != math.prod(shape):
        raise ValueError(f"{name} has {t.numel()} elements, expected {math.prod(shape)}")
    return t.view(shape)


def kda_chunk_prefill_fwd(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound: float,
                          scale: float, initial_state, cu_seqlens, out, final_state, workspace,
                          stream=None, checkpoints=None, checkpoint_interval: int = 0) -> None:
    """Queue one KDA chunked-prefill forward (see include/kda.h for the contract).

    q, k, v, g, out [T, H, 128] bf16; beta_logits [T, H] bf16; A_log [H] fp32;
    dt_bias [H, 128] fp32; initial_state None or [N, H, 128, 128]; final_state
    [N, H, 128, 128] (fp32 or bf16, the same dtype as initial_state);
    cu_seqlens [N + 1] int32; workspace uint8 (or None if no workspace is
    needed); stream: a torch.cuda.Stream, a raw hipStream_t int, or None for
    torch's current stream.  Leading singleton batch dims ([1, T, H, 128]) are
    accepted.  checkpoints: None, or [C, H, 128, 128] in the state dtype to
    receive the state after every checkpoint_interval tokens of each sequence
    (kda_chunk_prefill_fwd_checkpoints; C >= T // checkpoint_interval).
    """
    import torch
    lib = load_library()

    def squeeze_batch(t):
        return t[0] if (t is not None and t.dim() == 4 and t.shape[0] == 1
                        and t.shape[-1] == HEAD_DIM and t.shape[-2] != HEAD_DIM) else t

    q, k, v, g, out = (squeeze_batch(t) for t in (q, k, v, g, out))
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    T, H, D = q.shape
    if D != HEAD_DIM:
        raise ValueError(f"head_dim must be {HEAD_DIM}, got {D}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    bf = torch.bfloat16
    if final_state.dtype == torch.float32:
        sdt = KDA_STATE_FP32
    elif final_state.dtype == torch.bfloat16:
        sdt = KDA_STATE_BF16
    else:
        raise TypeError(f"state dtype must be float32 or bfloat16, got {final_state.dtype}")
    sshape = (N, H, HEAD_DIM, HEAD_DIM)
    if beta_logits.dim() == 3 and beta_logits.shape[0] == 1:
        beta_logits = beta_logits[0]
    if beta_logits.dim() == 3 and beta_logits.shape[-1] == 1:
        beta_logits = beta_logits[..., 0]
    views = {"q": q, "k": k, "v": v, "g": g, "beta": beta_logits, "out": out}
    ptrs = [
        _check(q, "q", bf, (T, H, D), strided=True), _check(k, "k", bf, (T, H, D), strided=True),
        _check(v, "v", bf, (T, H, D), strided=True), _check(g, "g", bf, (T, H, D), strided=True),
        _check(beta_logits, "beta_logits", bf, (T, H), strided=True),
        _check(_flat(A_log, "A_log", (H,)), "A_log", torch.float32, (H,)),
        _check(_flat(dt_bias, "dt_bias", (H, D)), "dt_bias", torch.float32, (H, D)),
    ]
    s0 = None if initial_state is None else _check(initial_state, "initial_state",
                                                   final_state.dtype, sshape)
    cu = _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    o = _check(out, "out", bf, (T, H, D), strided=True)
    fs = _check(final_state, "final_state", final_state.dtype, sshape)
    if workspace is None:
        ws, wsb = None, 0
    else:
        ws = _check(workspace, "workspace", torch.uint8)
        wsb = workspace.numel()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    args = (*ptrs, float(lower_bound), float(scale), s0, cu, o, fs, ws,
            ctypes.c_void_p(int(stream)), T, H, N, sdt, wsb)
    st = None
    if not all(t.is_contiguous() for t in views.values()):
        st = _Strides()
        for name in ("q", "k", "v", "g", "out"):
            setattr(st, f"{name}_token", views[name].stride(0))
            setattr(st, f"{name}_head", views[name].stride(1))
        st.beta_token, st.beta_head = views["beta"].stride(0), views["beta"].stride(1)
    if checkpoints is not None:
        if checkpoints.dim() != 4:
            raise ValueError("checkpoints must be [C, H, 128, 128]")
        ck = _check(checkpoints, "checkpoints", final_state.dtype,
                    (checkpoints.shape[0], H, HEAD_DIM, HEAD_DIM))
        rc = lib.kda_chunk_prefill_fwd_checkpoints(
            *args, None if st is None else ctypes.byref(st), ck, int(checkpoint_interval),
            int(checkpoints.shape[0]))
    elif st is None:
        rc = lib.kda_chunk_prefill_fwd(*args)
    else:
        rc = lib.kda_chunk_prefill_fwd_strided(*args, ctypes.byref(st))
    if rc != KDA_OK:
        detail = lib.kda_last_hip_error().decode() if rc == 4 else ""
        raise KdaError(rc, f"kda_chunk_prefill_fwd: {kda_status_string(rc)} {detail}".strip())


def kda_spec_decode_step(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound: float, scale: float,
                         state_pool, cu_seqlens, state_indices, num_accepted_tokens, out, workspace,
                         stream=None) -> None:
    """Queue one speculative-decode step with num_accepted_tokens rollback (see
    include/kda.h, kda_spec_decode_step).

    q, k, v, g, out [T, H, 128] bf16 (dense); beta_logits [T, H] bf16;
    state_pool [num_slots, H, 128, 128] fp32 or bf16 (read and written in
    place); cu_seqlens [N + 1] int32; state_indices [N, S] int32;
    num_accepted_tokens [N] int32; workspace uint8.
    """
    import torch
    lib = load_library()
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    T, H, D = q.shape
    if D != HEAD_DIM:
        raise ValueError(f"head_dim must be {HEAD_DIM}, got {D}")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    N = cu_seqlens.numel() - 1
    bf = torch.bfloat16
    if state_pool.dtype == torch.float32:
        sdt = KDA_STATE_FP32
    elif state_pool.dtype == torch.bfloat16:
        sdt = KDA_STATE_BF16
    else:
        raise TypeError(f"state dtype must be float32 or bfloat16, got {state_pool.dtype}")
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots, H, 128, 128]")
    if state_indices.dim() != 2 or state_indices.shape[0] != N:
        raise ValueError(f"state_indices must be [N, S] with N = {N}")
    ptrs = [_check(t, n, bf, (T, H, D)) for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"))]
    ptrs += [_check(beta_logits, "beta_logits", bf, (T, H)),
             _check(_flat(A_log, "A_log", (H,)), "A_log", torch.float32, (H,)),
             _check(_flat(dt_bias, "dt_bias", (H, D)), "dt_bias", torch.float32, (H, D))]
    pool = _check(state_pool, "state_pool", state_pool.dtype,
                  (state_pool.shape[0], H, HEAD_DIM, HEAD_DIM))
    cu = _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    idx = _check(state_indices, "state_indices", torch.int32, tuple(state_indices.shape))
    acc = _check(num_accepted_tokens, "num_accepted_tokens", torch.int32, (N,))
    o = _check(out, "out", bf, (T, H, D))
    ws = _check(workspace, "workspace", torch.uint8)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    rc = lib.kda_spec_decode_step(*ptrs, float(lower_bound), float(scale), pool,
                                  int(state_pool.shape[0]), cu, idx, int(state_indices.shape[1]),
                                  acc, o, ws, ctypes.c_void_p(int(stream)), T, H, N, sdt,
                                  workspace.numel())
    if rc != KDA_OK:
        detail = lib.kda_last_hip_error().decode() if rc == 4 else ""
        raise KdaError(rc, f"kda_spec_decode_step: {kda_status_string(rc)} {detail}".strip())


def kda_chunk_prefill_fwd_noalloc(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound: float,
                                  scale: float, initial_state, cu_seqlens, out, final_state, status,
                                  stream=None) -> None:
    """kda_chunk_prefill_fwd without a workspace (see include/kda.h,
    kda_chunk_prefill_fwd_noalloc): dense tensors as for the forward call;
    status a device int32 tensor of one element (the status word)."""
    import torch
    lib = load_library()
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    T, H, D = q.shape
    if D != HEAD_DIM:
        raise ValueError(f"head_dim must be {HEAD_DIM}, got {D}")
    N = cu_seqlens.numel() - 1
    if N < 1:
        raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
    bf = torch.bfloat16
    if final_state.dtype == torch.float32:
        sdt = KDA_STATE_FP32
    elif final_state.dtype == torch.bfloat16:
        sdt = KDA_STATE_BF16
    else:
        raise TypeError(f"state dtype must be float32 or bfloat16, got {final_state.dtype}")
    sshape = (N, H, HEAD_DIM, HEAD_DIM)
    ptrs = [_check(t, n, bf, (T, H, D)) for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"))]
    ptrs += [_check(beta_logits, "beta_logits", bf, (T, H)),
             _check(_flat(A_log, "A_log", (H,)), "A_log", torch.float32, (H,)),
             _check(_flat(dt_bias, "dt_bias", (H, D)), "dt_bias", torch.float32, (H, D))]
    s0 = None if initial_state is None else _check(initial_state, "initial_state",
                                                   final_state.dtype, sshape)
    cu = _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    o = _check(out, "out", bf, (T, H, D))
    fs = _check(final_state, "final_state", final_state.dtype, sshape)
    st = _check(status, "status", torch.int32, (1,))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    rc = lib.kda_chunk_prefill_fwd_noalloc(*ptrs, float(lower_bound), float(scale), s0, cu, o, fs, st,
                                           ctypes.c_void_p(int(stream)), T, H, N, sdt)
    if rc != KDA_OK:
        detail = lib.kda_last_hip_error().decode() if rc == 4 else ""
        raise KdaError(rc, f"kda_chunk_prefill_fwd_noalloc: {kda_status_string(rc)} {detail}".strip())


def kda_gate_proj_workspace_size(num_tokens: int, hidden_dim: int, n_ab: int) -> int:
    return int(load_library().kda_gate_proj_workspace_size(int(num_tokens), int(hidden_dim),
                                                             int(n_ab)))


def kda_gate_proj(hidden, w_ab, w_b, p_ab, g, workspace, stream=None) -> None:
    """Queue the gate / beta projections (see include/kda.h, kda_gate_proj):
    P = bf16(hidden w_ab^T) into p_ab [M, n_ab], G = bf16(P[:, :128] w_b^T)
    into g [M, n_b] (or a [M, n_b / 128, 128] view).  bf16 tensors, dense;
    workspace uint8 of kda_gate_proj_workspace_size bytes (no initialisation
    needed)."""
    import torch
    lib = load_library()
    bf = torch.bfloat16
    if hidden.dim() != 2 or w_ab.dim() != 2 or w_b.dim() != 2:
        raise ValueError("hidden, w_ab and w_b must be 2-D")
    M, K = hidden.shape
    n_ab, n_b = w_ab.shape[0], w_b.shape[0]
    ptrs = [_check(hidden, "hidden", bf, (M, K)), _check(w_ab, "w_ab", bf, (n_ab, K)),
            _check(w_b, "w_b", bf, (n_b, 128)), _check(p_ab, "p_ab", bf, (M, n_ab)),
            _check(g.reshape(M, n_b) if g.is_contiguous() else g, "g", bf, (M, n_b))]
    ws = _check(workspace, "workspace", torch.uint8)
    if stream is None:
        stream = torch.cuda.current_stream(hidden.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    rc = lib.kda_gate_proj(*ptrs, ws, workspace.numel(), ctypes.c_void_p(int(stream)), M, K, n_ab,
                           n_b)
    if rc != KDA_OK:
        detail = lib.kda_last_hip_error().decode() if rc == 4 else ""
        raise KdaError(rc, f"kda_gate_proj: {kda_status_string(rc)} {detail}".strip())
