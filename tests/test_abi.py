"""CPU checks of the C ABI: the library loads, exports every declared symbol, and its
host-side validation returns the documented status codes without launching."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "gated_delta_rule_31_amd", "libkda.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libkda.so is not built; run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kda_bounded_decay", "kda_chunk_fwd", "kda_recurrent_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "missing export %s" % n


def test_status_strings_and_version(lib):
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    assert lib.kda_status_string(0) == b"ok"
    for s in range(1, 8):
        assert lib.kda_status_string(s) not in (b"", b"unknown status")
    assert lib.kda_abi_version() == 4


def _chunk(lib, **kw):
    vp = ctypes.c_void_p
    args = dict(q=1, k=2, v=3, in_dtype=1, gate=4, gate_kind=1, beta=5, s0=None, sf=None, cu=None,
                num_seqs=0, B=1, T=64, H=2, K=16, V=16, C=16, scale=1.0, out=0x1000, out_dtype=1, ws=None,
                ws_bytes=0)
    args.update(kw)
    f = lib.kda_chunk_fwd
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                  vp, ctypes.c_int, vp, ctypes.c_size_t, vp]
    a = args
    return f(a["q"], a["k"], a["v"], a["in_dtype"], a["gate"], a["gate_kind"], a["beta"], a["s0"], a["sf"],
             a["cu"], a["num_seqs"], a["B"], a["T"], a["H"], a["K"], a["V"], a["C"], a["scale"], a["out"],
             a["out_dtype"], a["ws"], a["ws_bytes"], None)


# Each case is rejected on the host before any HIP call (the pointers are fake); the same
# holds for every call in the backward validation tests below.
@pytest.mark.parametrize("kw,status", [
    (dict(K=17), 4), (dict(V=256), 4), (dict(C=48), 4), (dict(H=0), 2), (dict(T=-1), 2),
    (dict(in_dtype=7), 3), (dict(gate_kind=5), 3), (dict(q=None), 1), (dict(out=None), 1),
    (dict(cu=9, B=2, num_seqs=1), 5), (dict(out=3), 6), (dict(sf=4), 6), (dict(sf=0x1000), 6),
    # the output must be 8-byte aligned (bf16) or 16-byte aligned (float32)
    (dict(out=0x1004), 5), (dict(out=0x1008, out_dtype=0), 5),
])
def test_chunk_validation(lib, kw, status):
    assert _chunk(lib, **kw) == status


def _ws_size(lib, in_dtype=1, B=1, T=64, num_seqs=0, varlen=0, H=2, K=16, V=16, C=16):
    f = lib.kda_chunk_fwd_workspace_size
    f.restype = ctypes.c_size_t
    i32 = ctypes.c_int
    f.argtypes = [i32, i32, ctypes.c_int64, i32, i32, i32, i32, i32, i32]
    return f(in_dtype, B, T, num_seqs, varlen, H, K, V, C)


def test_chunk_workspace_size(lib):
    # bf16 path, K = V = 128, C = 32: (3 C K + 3 C^2) fp16 operands (Qt, Bw, Kt; T, A_qk
    # hi and lo) + (K + C) floats per (chunk, head), T = 8192 being 256 chunks per head;
    # then one float32 K x V state per (sequence, head)
    per = 2 * (3 * 32 * 128 + 3 * 32 * 32) + 4 * (128 + 32)
    st = 4 * 128 * 128
    assert _ws_size(lib, T=8192, H=96, K=128, V=128, C=32) == 256 * 96 * per + 96 * st
    # a ragged length rounds up; packed sequences get T / C + N slots
    assert _ws_size(lib, T=8193, H=96, K=128, V=128, C=32) == 257 * 96 * per + 96 * st
    assert _ws_size(lib, T=8192, num_seqs=8, varlen=1, H=96, K=128, V=128, C=32) == (256 + 8) * 96 * per + 8 * 96 * st
    assert _ws_size(lib, B=2, T=64, K=16, V=16, C=16, in_dtype=0) == \
        2 * 4 * 2 * (4 * (3 * 16 * 16 + 2 * 256) + 4 * 32) + 2 * 2 * 4 * 16 * 16
    assert _ws_size(lib, K=24) == 0 and _ws_size(lib, C=48) == 0 and _ws_size(lib, H=0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=64, ws_bytes=16), 5),                  # too small
    (dict(ws=72, ws_bytes=1 << 20), 5),             # not 16-byte aligned
    (dict(q=64, ws=64, ws_bytes=1 << 20), 6),       # the workspace is q
    (dict(out=0x2000, ws=0x2000, ws_bytes=1 << 20), 6),  # the workspace is out
    (dict(ws=64, ws_bytes=1 << 20, K=24), 4),       # unsupported width
])
def test_chunk_workspace_validation(lib, kw, status):
    assert _chunk(lib, **kw) == status


def test_gate_validation(lib):
    vp = ctypes.c_void_p
    f = lib.kda_bounded_decay
    f.restype = ctypes.c_int
    f.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_float, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, vp, vp]
    assert f(1, 1, 2, None, 0.0, 4, 2, 8, 0, 3, None) == 5      # lower_bound must be < 0
    assert f(1, 1, 2, None, -5.0, 4, 0, 8, 0, 3, None) == 2     # H = 0
    assert f(1, 9, 2, None, -5.0, 4, 2, 8, 0, 3, None) == 3     # bad dtype
    assert f(None, 1, 2, None, -5.0, 4, 2, 8, 0, 3, None) == 1  # NULL logits
    assert f(1, 1, 2, None, -5.0, 4, 2, 8, 0, 1, None) == 6     # out aliases logits
    assert f(None, 1, None, None, -5.0, 0, 2, 8, 0, None, None) == 0  # rows = 0: nothing to do


def test_step_validation(lib):
    vp = ctypes.c_void_p
    f = lib.kda_recurrent_step
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, ctypes.c_int, vp]
    assert f(1, 2, 3, 1, 4, 0, 5, 16, 2, 2, 24, 16, 1.0, 7, 1, None) == 4     # K = 24
    assert f(1, 2, 3, 1, 4, 0, 5, None, 2, 2, 16, 16, 1.0, 7, 1, None) == 1   # NULL state
    assert f(1, 2, 3, 1, 4, 0, 5, 16, 2, 2, 16, 16, 1.0, 3, 1, None) == 6     # out aliases v
    assert f(1, 2, 3, 1, 4, 0, 5, 18, 2, 2, 16, 16, 1.0, 7, 1, None) == 5     # misaligned state
    assert f(None, None, None, 1, None, 0, None, None, 0, 2, 16, 16, 1.0, None, 1, None) == 0  # B = 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    import gated_delta_rule_31_amd as kda
    z = torch.zeros(2, 3, 16)
    with pytest.raises(ValueError):
        kda.bounded_decay(z, torch.zeros(3))


def test_fused_gate_validation(lib):
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    f = lib.kda_chunk_fwd_fused_gate
    f.restype = i32
    u32 = ctypes.c_uint
    f.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, vp, vp, i32, i32, ctypes.c_int64, i32, i32, i32,
                  i32, f32, vp, i32, vp, ctypes.c_size_t, vp]

    def chunk(z=4, ls=8, bias=None, lb=-5.0, out=0x1000, K=16, flags=0, ws=None, nws=0):
        return f(1, 2, 3, 1, z, ls, bias, lb, flags, 5, None, None, None, 0, 1, 64, 2, K, 16, 16, 1.0, out, 1,
                 ws, nws, None)
    assert chunk(lb=0.0) == 5        # lower bound must be negative
    assert chunk(lb=-6.0) == 5       # and >= -5 on the chunk path (the tile rescale bound)
    assert chunk(z=None) == 1        # NULL logits
    assert chunk(ls=None) == 1       # NULL log_scale
    assert chunk(out=4) == 6         # out aliases the logits
    assert chunk(out=8) == 6         # out aliases log_scale
    assert chunk(K=24) == 4          # unsupported width
    assert chunk(flags=8) == 5       # unknown preparation flag
    assert chunk(z=64, ws=64, nws=1 << 20) == 6   # the workspace is the logits
    assert chunk(ws=64, nws=8) == 5        # workspace too small
    g = lib.kda_recurrent_step_fused_gate
    g.restype = i32
    g.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, u32, vp, vp, i32, i32, i32, i32, f32, vp, i32, vp]
    assert g(1, 2, 3, 1, 4, 8, None, 0.0, 0, 5, 16, 2, 2, 16, 16, 1.0, 7, 1, None) == 5   # lower bound >= 0
    assert g(1, 2, 3, 1, 4, 8, None, -9.0, 0, 5, None, 2, 2, 16, 16, 1.0, 7, 1, None) == 1  # any bound; NULL state
    assert g(1, 2, 3, 1, None, 8, None, -5.0, 0, 5, 16, 2, 2, 16, 16, 1.0, 7, 1, None) == 1  # NULL logits
    assert g(1, 2, 3, 1, 4, 8, None, -5.0, 0, 5, 16, 2, 2, 16, 16, 1.0, 4, 1, None) == 6   # out aliases logits
    assert g(1, 2, 3, 1, 4, 8, None, -5.0, 16, 5, 16, 2, 2, 16, 16, 1.0, 7, 1, None) == 5  # unknown flag


def test_recurrent_fwd_validation(lib):
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    f = lib.kda_recurrent_fwd
    f.restype = i32
    f.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, ctypes.c_int64, i32, i32, i32, f32, vp,
                  i32, vp]

    def call(q=1, gk=0, K=16, T=8, B=1, cu=None, out=6, sf=None):
        return f(q, 2, 3, 1, 4, gk, 5, None, sf, cu, 0, B, T, 2, K, 16, 1.0, out, 1, None)
    assert call(K=24) == 4
    assert call(gk=3) == 3
    assert call(T=-1) == 2
    assert call(q=None) == 1
    assert call(out=2) == 6
    assert call(sf=3) == 6
    assert call(cu=9, B=2) == 5
    assert call(T=0, q=None, out=None) == 0   # empty: nothing to do without a final state
    assert call(out=66) == 5                  # bf16 output not 8-byte aligned
    assert call(out=64, sf=72) == 5           # final state not 16-byte aligned
    g = lib.kda_recurrent_fwd_fused_gate
    g.restype = i32
    g.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, ctypes.c_uint, vp, vp, vp, vp, i32, i32, ctypes.c_int64, i32,
                  i32, i32, f32, vp, i32, vp]
    assert g(1, 2, 3, 1, 4, 8, None, 0.0, 0, 5, None, None, None, 0, 1, 8, 2, 16, 16, 1.0, 6, 1, None) == 5
    assert g(1, 2, 3, 1, 4, None, None, -9.0, 0, 5, None, None, None, 0, 1, 8, 2, 16, 16, 1.0, 6, 1, None) == 1


def test_chunk_bwd_validation(lib):
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    ws = lib.kda_chunk_bwd_workspace_size
    ws.restype = sz
    ws.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    need = ws(1, 64, 2, 16, 16, 0, 0)
    assert need > 0 and ws(1, 64, 2, 24, 16, 0, 0) == 0
    assert ws(2, 130, 3, 32, 64, 0, 0) == 6 * ws(1, 64, 3, 32, 64, 0, 0)  # 3 chunks per batch row
    assert ws(1, 130, 3, 32, 64, 4, 1) == 6 * ws(1, 64, 3, 32, 64, 0, 0)  # varlen: T // 64 + N slots
    f = lib.kda_chunk_bwd
    f.restype = i32
    f.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp, i32, vp, vp, vp,
                  vp, i32, vp, vp, vp, vp, sz, vp]

    def call(q=1, K=16, T=64, B=1, cu=None, ns=0, dq=11, dgate=14, gk=0, dt=1, wsz=need, work=20, ds0=None):
        return f(q, 2, 3, dt, 4, gk, 5, None, cu, ns, B, T, 2, K, 16, 1.0, 6, 1, None, dq, 12, 13, 1, dgate, 15,
                 ds0, work, wsz, None)
    assert call(K=24) == 4
    assert call(T=-1) == 2
    assert call(dt=5) == 3
    assert call(gk=4) == 3
    assert call(q=None) == 1
    assert call(work=None) == 1
    assert call(wsz=need - 1) == 5           # workspace too small
    assert call(dq=2) == 6                   # dq aliases k
    assert call(dgate=11) == 6               # two outputs share a buffer
    assert call(ds0=6) == 6                  # d_initial_state aliases d_out
    assert call(cu=9, B=2, ns=1) == 5
    assert call(T=0, q=None, work=None) == 0  # empty: no token gradients, no d_initial_state asked


def test_bounded_decay_bwd_validation(lib):
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    f = lib.kda_bounded_decay_bwd
    f.restype = i32
    f.argtypes = [vp, i32, vp, vp, f32, i64, i32, i32, vp, i32, vp, i32, vp, vp, vp]

    def call(z=1, ls=2, lb=-5.0, rows=4, H=2, K=8, g=3, gk=0, dz=4, dt=0, dls=5, db=6):
        return f(z, 1, ls, None, lb, rows, H, K, g, gk, dz, dt, dls, db, None)
    assert call(lb=0.0) == 5
    assert call(H=0) == 2
    assert call(gk=3) == 3
    assert call(dt=7) == 3
    assert call(ls=None) == 1
    assert call(g=None) == 1
    assert call(dz=3) == 6                   # d_logits aliases grad
    assert call(db=5) == 6                   # d_bias and d_log_scale share a buffer
    assert call(rows=0, z=None, g=None, dz=None, dls=None, db=None) == 0


def test_python_prefill_form_selection():
    """The binding picks the prefill form from two_pass / TWO_PASS and the shape: a
    workspace of the size the library asks for, none for two_pass=False or a shape the
    two-kernel form lacks (by default), and an error when that form is asked for by name."""
    import torch
    import gated_delta_rule_31_amd as kda
    q = torch.zeros(1, 100, 2, 64, dtype=torch.bfloat16)  # a host tensor: no device work happens here
    ws, n = kda._chunk_workspace(None, None, q, 1, 64, 32, False)
    assert n == kda.chunk_fwd_workspace_size(torch.bfloat16, 1, 100, 2, 64, 64, 32) > 0 and ws.numel() == n
    assert kda._chunk_workspace(False, None, q, 1, 64, 32, False) == (None, 0)
    # float32 K = V = 128 at chunk 64 has no two-kernel form (two packages exceed the LDS);
    # bf16 has one (the pre-pass stages the key columns in two halves)
    assert kda.chunk_fwd_workspace_size(torch.bfloat16, 1, 100, 2, 128, 128, 64) > 0
    q128 = torch.zeros(1, 100, 2, 128, dtype=torch.float32)
    assert kda.chunk_fwd_workspace_size(torch.float32, 1, 100, 2, 128, 128, 64) == 0
    assert kda._chunk_workspace(None, None, q128, 1, 128, 64, False) == (None, 0)
    with pytest.raises(kda.KDAError):
        kda._chunk_workspace(True, None, q128, 1, 128, 64, False)
    given = torch.empty(n, dtype=torch.uint8)
    assert kda._chunk_workspace(None, given, q, 1, 64, 32, False) == (given, n)
    with pytest.raises(ValueError):
        kda._chunk_workspace(None, torch.empty(n, dtype=torch.float32), q, 1, 64, 32, False)
