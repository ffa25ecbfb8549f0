"""Host-side tests of the C ABI (no GPU needed).

Every call here fails its argument checks before the library makes any HIP
call, so it runs on a machine without a GPU.  Fake pointers are only ever
passed together with an argument that is invalid.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import gated_delta_rule_tok_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: each call below is rejected first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = kda.load_library()
    names = _declared_functions()
    assert set(names) == {"kda_get_workspace_size", "kda_chunk_prefill_fwd",
                          "kda_chunk_prefill_fwd_strided", "kda_chunk_prefill_fwd_checkpoints",
                          "kda_status_string",
                          "kda_last_hip_error", "kda_debug_set_vsplit", "kda_debug_set_kernel",
                          "kda_debug_set_segment", "kda_debug_segment_length",
                          "kda_debug_two_workgroups",
                          "kda_spec_decode_step", "kda_chunk_prefill_fwd_noalloc",
                          "kda_gate_proj", "kda_gate_proj_workspace_size"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/kda.h but not exported"


def test_workspace_size_is_pure_and_monotone():
    f = kda.kda_get_workspace_size
    assert f(16384, 16, 8) == f(16384, 16, 8)
    assert f(-1, 16, 8) == 0 and f(10, 0, 8) == 0 and f(10, 4, 0) == 0
    prev = 0
    for n in (1, 2, 8, 64, 1000):
        cur = f(65536, 32, n)
        assert cur >= prev
        prev = cur
    for t in (0, 1, 64, 65, 16384):
        assert f(t + 1, 16, 8) >= f(t, 16, 8)
    for h in (1, 2, 16, 32):
        assert f(16384, h + 1, 8) >= f(16384, h, 8)
    assert f(16384, 16, 8) % 256 == 0


def test_status_strings():
    for code in range(5):
        assert kda.kda_status_string(code).startswith("KDA_")
    assert kda.kda_status_string(0) == "KDA_OK"
    assert kda.kda_status_string(99) == "KDA_ERR_UNKNOWN"


def test_last_hip_error_empty_without_failures():
    assert kda.kda_last_hip_error() == ""


def test_debug_vsplit_hook():
    lib = kda.load_library()
    assert lib.kda_debug_set_vsplit(3) == -1
    assert lib.kda_debug_set_vsplit(16) == -1
    prev = lib.kda_debug_set_vsplit(4)
    assert prev in (0, 1, 2, 4, 8)
    assert lib.kda_debug_set_vsplit(0) == 4
    with pytest.raises(ValueError):
        kda.kda_debug_set_vsplit(5)


def _call(**over):
    """kda_chunk_prefill_fwd through ctypes with valid-looking defaults."""
    lib = kda.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, scale=128 ** -0.5, s0=None, cu=FAKE, out=FAKE, sT=FAKE, ws=FAKE,
             stream=None, T=16384, H=16, N=8, sdt=0, wsb=1 << 20)
    a.update(over)
    return lib.kda_chunk_prefill_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                     a["dt_bias"], a["lb"], a["scale"], a["s0"], a["cu"],
                                     a["out"], a["sT"], a["ws"], a["stream"], a["T"], a["H"],
                                     a["N"], a["sdt"], a["wsb"])


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "cu", "out",
                                  "sT"])
def test_null_required_pointer_rejected(name):
    assert _call(**{name: None}) == INVALID


@pytest.mark.parametrize("over", [
    dict(T=-1), dict(T=2 ** 31), dict(H=0), dict(H=-3), dict(N=0), dict(N=-1),
    dict(sdt=2), dict(sdt=-1), dict(lb=float("nan")), dict(lb=float("-inf")),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(N=2 ** 28, H=16),
    dict(T=2 ** 20, H=16), dict(T=2 ** 24, H=1),
    # rows up to 256 past the end must stay addressable: (T + 256) H 128 < 2^31
    dict(T=2 ** 24 - 100, H=1),
])
def test_bad_sizes_and_scalars_rejected(over):
    assert _call(**over) == INVALID


@pytest.mark.parametrize("lb", [0.5, 1e-3, -5.6, -100.0])
def test_lower_bound_outside_range_unsupported(lb):
    assert _call(lb=lb) == UNSUPPORTED


def test_workspace_too_small():
    need = kda.kda_get_workspace_size(16384, 16, 8)
    assert need > 0
    # a call needs the status word and the order table; the segment area is optional
    base = 256 + 256
    assert _call(wsb=base - 1) == WS_SMALL
    assert _call(wsb=0) == WS_SMALL
    # enough bytes claimed but no pointer
    assert _call(ws=None, wsb=need) == INVALID
    assert _call(ws=None, wsb=base) == INVALID


# The segment area: 160 table entries (16 bytes), first/count ints, and 160
# (pseudo-sequence, head) slots of a summary (local state and transition) and
# an entering state, fp32 128 x 128 each; the same for every head count.
SEG_AREA = 2560 + 768 + 768 + 160 * 3 * 128 * 128 * 4 + 128 * 8 * 8  # + the two-workgroup flag words


@pytest.mark.parametrize("heads", [1, 2, 3, 4, 16, 32, 33, 64])
def test_workspace_segment_area(heads):
    f = kda.kda_get_workspace_size
    base = 256 + 256
    assert f(1023, heads, 8) == base                    # no call this small segments
    assert f(1024, heads, 8) == base + SEG_AREA
    assert f(1 << 20, heads, 1) == 256 + 256 + SEG_AREA  # independent of the token count
    assert SEG_AREA < 32 << 20


@pytest.mark.parametrize("T,H,N,L", [
    (16384, 16, 1, 2048),    # 1 x 16384, 16 heads: 128 / 16 = 8 segments
    (16384, 4, 2, 512),      # 2 x 8192, 4 heads: 32 segments of 512
    (8192, 4, 1, 256),       # 8192 / 32, at least 256 tokens
    (1024, 4, 1, 256),       # at least 1024 tokens per sequence on average
    (1023, 4, 1, 0),
    (4096, 4, 8, 0),         # 512 tokens per sequence
    (4096, 8, 4, 0),         # 32 pairs need 2048 tokens per sequence
    (2048, 8, 2, 256),       # 16 pairs, 1024 tokens per sequence
    (4096, 16, 2, 512),      # 32 pairs, 2048 tokens per sequence
    (16384, 16, 8, 0),       # 128 (sequence, head) pairs: one piece
    (256, 2, 1, 0),          # fewer than 1024 tokens per sequence
    (65536, 32, 1, 16384),   # 128 / 32 = 4 segments; 1 + 4 pseudo-sequences x 32 <= 160
    (4096, 32, 1, 1024),     # the same cut at 4096 tokens
    (65536, 32, 2, 0),       # 64 (sequence, head) pairs: one piece
    (0, 4, 1, 0),
])
def test_segment_plan(T, H, N, L):
    assert kda.kda_debug_segment_length(T, H, N) == L


def test_segment_plan_follows_the_hook():
    prev = kda.kda_debug_set_segment(1)
    try:
        assert kda.kda_debug_segment_length(16384, 16, 1) == 0
        kda.kda_debug_set_segment(64)
        assert kda.kda_debug_segment_length(2000, 2, 3) == 64    # 3 + 31 = 34 <= 80
        assert kda.kda_debug_segment_length(6000, 2, 3) == 0     # 3 + 93 > 80
        assert kda.kda_debug_segment_length(16384, 16, 8) == 0   # 8 + 256 > 10
    finally:
        kda.kda_debug_set_segment(prev)


def test_debug_segment_hook():
    lib = kda.load_library()
    for bad in (-1, 2, 15, 24, 1 << 25):
        assert lib.kda_debug_set_segment(bad) == -1
    prev = lib.kda_debug_set_segment(64)
    assert lib.kda_debug_set_segment(1) == 64
    assert lib.kda_debug_set_segment(prev) == 1
    with pytest.raises(ValueError):
        kda.kda_debug_set_segment(17)


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    T, H = 4, 1
    bf = torch.bfloat16
    q = torch.zeros(T, H, 128, dtype=bf)
    with pytest.raises((ValueError, TypeError)):
        kda.kda_chunk_prefill_fwd(q, q, q, q, torch.zeros(T, H, dtype=bf),
                                  torch.zeros(H), torch.zeros(H, 128), -5.0, 0.1, None,
                                  torch.tensor([0, T], dtype=torch.int32), q,
                                  torch.zeros(1, H, 128, 128), None)


def test_one_hip_runtime_in_the_process():
    """libkda.so must bind to the HIP runtime torch already loaded (same SONAME);
    a second libamdhip64 in the process sees no device."""
    kda.load_library()
    maps = open("/proc/self/maps").read().splitlines()
    libs = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(libs) == 1, f"more than one HIP runtime mapped: {sorted(libs)}"


def test_misaligned_dense_tensor_rejected():
    # q, k, v, g and out are read and written with 8- and 16-byte accesses
    for name in ("q", "k", "v", "g", "out"):
        assert _call(**{name: ctypes.c_void_p(0x1008)}) == INVALID
    assert _call(beta=ctypes.c_void_p(0x1001)) == INVALID


def _dense_strides(H):
    row = H * 128
    return kda._Strides(row, 128, row, 128, row, 128, row, 128, H, 1, row, 128)


def _call_strided(strides, **over):
    """kda_chunk_prefill_fwd_strided through ctypes; defaults as _call."""
    lib = kda.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, scale=128 ** -0.5, s0=None, cu=FAKE, out=FAKE, sT=FAKE, ws=FAKE,
             stream=None, T=16384, H=16, N=8, sdt=0, wsb=1 << 20)
    a.update(over)
    return lib.kda_chunk_prefill_fwd_strided(
        a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"], a["lb"],
        a["scale"], a["s0"], a["cu"], a["out"], a["sT"], a["ws"], a["stream"], a["T"], a["H"],
        a["N"], a["sdt"], a["wsb"], None if strides is None else ctypes.byref(strides))


def test_strided_entry_checks():
    assert _call_strided(None) == INVALID
    # the checks run in the dense call's order: a bad lower_bound with good
    # strides is UNSUPPORTED, exactly as for the dense entry
    assert _call_strided(_dense_strides(16), lb=-7.0) == UNSUPPORTED
    assert _call_strided(_dense_strides(16), wsb=0) == WS_SMALL
    for field, value in [("q_token", 16 * 128 + 4), ("k_head", 132), ("v_token", -8),
                         ("g_head", 3), ("out_token", 2 ** 20), ("beta_token", -1),
                         ("beta_head", 2 ** 30)]:
        st = _dense_strides(16)
        setattr(st, field, value)
        assert _call_strided(st) == INVALID, field
    # (T + 256) * token + (H - 1) * head + 128 must stay below 2^31 elements
    st = _dense_strides(16)
    st.q_token = 16 * 128 * 128
    assert _call_strided(st, T=16384) == INVALID
    st.q_token = 16 * 128 * 4
    assert _call_strided(st, T=16384, lb=-7.0) == UNSUPPORTED  # strides accepted
    # strides whose products would wrap a 64-bit integer are rejected, not wrapped
    for field in ("q_token", "k_head", "g_token", "beta_head"):
        for value in (2 ** 55, 2 ** 62, 2 ** 63 - 8):
            st = _dense_strides(16)
            setattr(st, field, value)
            assert _call_strided(st) == INVALID, (field, value)


def test_python_binding_strided_views_keep_channel_contiguity():
    torch = pytest.importorskip("torch")
    T, H = 4, 2
    bf = torch.bfloat16
    big = torch.zeros(T, H, 256, dtype=bf)
    with pytest.raises((ValueError, TypeError)):
        # channels not contiguous (stride 2): rejected before anything else
        kda._check(big[..., ::2], "q", bf, (T, H, 128), strided=True)


def test_python_binding_never_copies_parameters():
    """A_log and dt_bias are passed by data pointer: a non-contiguous tensor
    is rejected instead of copied into a temporary that torch could recycle
    before the queued kernel reads it."""
    torch = pytest.importorskip("torch")
    H = 4
    a = torch.zeros(2 * H)
    with pytest.raises(ValueError):
        kda._flat(a[::2], "A_log", (H,))
    d = torch.zeros(128, H).t()
    with pytest.raises(ValueError):
        kda._flat(d, "dt_bias", (H, 128))
    with pytest.raises(ValueError):
        kda._flat(torch.zeros(H + 1), "A_log", (H,))
    flat = torch.zeros(H, 1)
    v = kda._flat(flat, "A_log", (H,))
    assert v.data_ptr() == flat.data_ptr() and tuple(v.shape) == (H,)


def test_debug_kernel_hook():
    lib = kda.load_library()
    for k in (1, 2, 3, 4, 5, 6, 0):
        assert lib.kda_debug_set_kernel(k) >= 0
    assert lib.kda_debug_set_kernel(7) == -1
    assert lib.kda_debug_set_kernel(-1) == -1
    assert lib.kda_debug_set_kernel(0) == 0


def _call_ck(ck=FAKE, interval=64, cap=256, **over):
    """kda_chunk_prefill_fwd_checkpoints through ctypes (dense), valid-looking
    defaults; every call below is rejected before any device access."""
    lib = kda.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, scale=128 ** -0.5, s0=None, cu=FAKE, out=FAKE, sT=FAKE, ws=FAKE,
             stream=None, T=16384, H=16, N=8, sdt=0, wsb=1 << 20)
    a.update(over)
    return lib.kda_chunk_prefill_fwd_checkpoints(
        a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"], a["lb"],
        a["scale"], a["s0"], a["cu"], a["out"], a["sT"], a["ws"], a["stream"], a["T"], a["H"],
        a["N"], a["sdt"], a["wsb"], None, ck, interval, cap)


@pytest.mark.parametrize("ck, interval, cap", [
    (None, 64, 256),     # no checkpoint buffer
    (FAKE, 0, 256), (FAKE, -64, 256), (FAKE, 40, 2 ** 20), (FAKE, 8, 2 ** 20),  # interval
    (FAKE, 64, 255), (FAKE, 16, 1023),  # capacity below T / interval (16384 tokens)
])
def test_checkpoint_arguments_rejected(ck, interval, cap):
    assert _call_ck(ck, interval, cap) == INVALID


def test_checkpoints_below_lower_bound_min_unsupported():
    # the checkpoint call keeps the forward's lower_bound range [-5.5, 0]
    assert _call_ck(lb=-5.75) == UNSUPPORTED
    assert _call_ck(lb=0.5) == UNSUPPORTED


def test_checkpoints_keep_the_forward_checks():
    assert _call_ck(q=None) == INVALID
    assert _call_ck(wsb=0) == WS_SMALL


def _call_spec(**over):
    """kda_spec_decode_step through ctypes (every call below is rejected before
    any HIP call, so the fake pointers are never dereferenced)."""
    lib = kda.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0,
             scale=128 ** -0.5, pool=FAKE, slots=16, cu=FAKE, idx=FAKE, stride=4, acc=FAKE,
             out=FAKE, ws=FAKE, stream=None, T=8, H=2, N=2, sdt=0, wsb=1 << 20)
    a.update(over)
    return lib.kda_spec_decode_step(
        a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"], a["lb"], a["scale"],
        a["pool"], a["slots"], a["cu"], a["idx"], a["stride"], a["acc"], a["out"], a["ws"],
        a["stream"], a["T"], a["H"], a["N"], a["sdt"], a["wsb"])


@pytest.mark.parametrize("over", [dict(pool=None), dict(idx=None), dict(acc=None), dict(slots=0),
                                  dict(slots=-3), dict(stride=0), dict(cu=None), dict(N=0),
                                  dict(slots=2 ** 62)])
def test_spec_step_argument_checks(over):
    assert _call_spec(**over) == 1  # KDA_ERR_INVALID_ARG


def test_spec_step_range_and_workspace_checks():
    assert _call_spec(lb=-7.0) == 2        # KDA_ERR_UNSUPPORTED
    assert _call_spec(wsb=0) == 3          # KDA_ERR_WORKSPACE_TOO_SMALL



def _call_proj(**over):
    lib = kda.load_library()
    a = dict(hidden=FAKE, w_ab=FAKE, w_b=FAKE, p_ab=FAKE, g=FAKE, ws=FAKE, wsb=1 << 22, stream=None,
             M=8, K=7168, n_ab=144, n_b=1536)
    a.update(over)
    return lib.kda_gate_proj(a["hidden"], a["w_ab"], a["w_b"], a["p_ab"], a["g"], a["ws"], a["wsb"],
                             a["stream"], a["M"], a["K"], a["n_ab"], a["n_b"])


@pytest.mark.parametrize("over", [dict(hidden=None), dict(w_ab=None), dict(w_b=None), dict(g=None),
                                  dict(p_ab=None), dict(ws=None), dict(M=-1), dict(M=65537), dict(K=0), dict(K=7170),
                                  dict(n_ab=120), dict(n_ab=146), dict(n_b=1544), dict(n_b=0),
                                  dict(hidden=ctypes.c_void_p(0x1008))])
def test_proj_argument_checks(over):
    assert _call_proj(**over) == INVALID


def test_proj_workspace_checks():
    need = kda.kda_gate_proj_workspace_size(8, 7168, 144)
    # one fp32 16 x 16 partial tile per (1024-wide K slice, 16 rows of w_ab, 16 tokens)
    assert need == 7 * 9 * 256 * 4
    assert _call_proj(wsb=need - 1) == WS_SMALL
    assert kda.kda_gate_proj_workspace_size(-1, 7168, 144) == 0
    assert kda.kda_gate_proj_workspace_size(17, 7168, 144) == 2 * 7 * 9 * 256 * 4  # two token tiles
    assert kda.kda_gate_proj_workspace_size(5, 1000, 136) == 1 * 9 * 256 * 4       # ragged K and n_ab


def test_two_workgroup_rule():
    """The two-workgroup form: 33-96 pairs, or 97-128 pairs and at most 2^17
    (token, head) pairs, that fit twice on the device, after the decode and
    segment rules; kernel 6 forces it wherever it fits; a value-split
    override keeps the single-workgroup kernel."""
    f = kda.kda_debug_two_workgroups
    assert not f(16384, 16, 8)               # 128 pairs x 2048 tokens: 2^18 token-heads
    assert not f(14336, 16, 7)               # 112 pairs x 2048
    assert f(12288, 16, 6)                   # 96 pairs x 2048: any length up to 96 pairs
    assert f(32768, 8, 8)                    # 64 pairs x 4096
    assert f(16384, 8, 16)                   # 128 pairs x 1024: 2^17 token-heads
    assert f(8192, 16, 4)                    # 64 pairs x 2048
    assert f(16384, 4, 32)                   # 128 pairs x 512
    assert not f(8192, 16, 2)                # 32 pairs (the segment schedule takes it)
    assert not f(2048, 4, 8)                 # 32 pairs
    assert f(2816, 3, 11)                    # 33 pairs
    assert not f(20000, 3, 50)               # 150 pairs: more than 128
    assert not f(16384, 4, 32, cus=200)      # 2 x 128 pairs do not fit on 200 CUs
    assert not f(256, 16, 40)                # decode-sized (6.4 tokens per sequence)
    assert not f(0, 0, 1) and not f(-1, 1, 1)
    lib = kda.load_library()
    try:
        lib.kda_debug_set_kernel(6)
        assert f(300, 2, 1) and f(16384, 16, 8) and not f(16384, 16, 9)
        lib.kda_debug_set_kernel(5)
        assert not f(8192, 16, 4)
        lib.kda_debug_set_kernel(0)
        lib.kda_debug_set_vsplit(2)
        assert not f(8192, 16, 4)
    finally:
        lib.kda_debug_set_kernel(0)
        lib.kda_debug_set_vsplit(0)
